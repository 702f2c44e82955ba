"""wq_linear_noalloc: the dispatch of wq_linear with the GEMM's scratch in the
library's static device array instead of a caller workspace.

Through the C ABI, its output must equal wq_linear's bit for bit when
wq_linear gets a workspace of the static array's size (the same split plan,
so the same kernels and summation order), and meet the oracle's tolerance.
Two calls in a row, the second smaller, check that the array's leftover
contents from the first call do not leak into the second."""

import ctypes

import numpy as np
import pytest

import oracle as O
import wq_inputs as I

torch = pytest.importorskip("torch")
import weight_only_int4_wq_amd as wq  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wq.lib()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def layer(seed, N, K, bits, gs, act):
    w = I.weights(seed, N, K, 0.02)
    g_idx = I.act_order_gidx(seed, K, gs) if act else None
    ref = O.quantize_linear_layer(w, bits, gs, g_idx=g_idx)
    perm = None if g_idx is None else wq.act_order_perm(dev(g_idx), gs)
    codes, scales, zeros = wq.quantize_rtn(dev(w), bits, gs, perm=perm)
    packed, perm2 = wq.pack(codes, bits, gs, g_idx=None if g_idx is None else dev(g_idx))
    return dict(packed=packed, scales=scales, zeros=zeros, perm=perm2, ref=ref)


def ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def call_noalloc(x, L, bits, gs):
    M, K = x.shape
    N = L["packed"].shape[0]
    y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    st = wq.lib().wq_linear_noalloc(ptr(x), ptr(L["packed"]), ptr(L["scales"]), ptr(L["zeros"]), ptr(L["perm"]),
                                    ptr(y), M, N, K, bits, gs, None)
    return st, y


def call_linear(x, L, bits, gs, ws):
    M, K = x.shape
    N = L["packed"].shape[0]
    y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    st = wq.lib().wq_linear(ptr(x), ptr(L["packed"]), ptr(L["scales"]), ptr(L["zeros"]), ptr(L["perm"]), ptr(y),
                            M, N, K, bits, gs, ptr(ws), ws.numel(), None)
    return st, y


def check(y, x, ref):
    yr = O.linear_ref(x, ref["w_hat"])
    yg = y.cpu().numpy().astype(np.float64)
    rel = np.linalg.norm(yg - yr) / np.linalg.norm(yr)
    assert rel <= 1e-3 and np.abs(yg - yr).max() <= 5e-2, rel


@pytest.mark.parametrize("first,second", [
    # (M, N, K, bits, gs, act-order): the first call leaves gathered
    # activations and split-K partials behind, the second is smaller
    ((256, 4096, 4096, 4, 128, True), (64, 1000, 1024, 4, 128, True)),
    ((32, 8192, 8192, 4, 128, False), (8, 520, 2048, 3, 32, False)),
    ((300, 1000, 4128, 8, 32, True), (3, 256, 512, 4, 128, True)),
    # decode batches whose activations exceed LDS: K-slab partials
    ((16, 4104, 11008, 4, 128, False), (7, 100, 16384, 2, 64, False)),
])
def test_noalloc_matches_linear_on_two_calls(first, second):
    ws = torch.empty((wq.noalloc_scratch_bytes(),), dtype=torch.uint8, device="cuda")
    for i, (M, N, K, bits, gs, act) in enumerate((first, second)):
        L = layer((300, i, M, N), N, K, bits, gs, act)
        x = I.activations((301, i, M), M, K)
        xd = dev(x)
        st, y = call_noalloc(xd, L, bits, gs)
        assert st == 0, wq.status_str(st)
        st, y_ref = call_linear(xd, L, bits, gs, ws)
        assert st == 0, wq.status_str(st)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), (M, N, K)
        check(y, x, L["ref"])


def test_noalloc_rejects_gather_beyond_the_static_array():
    cap = wq.noalloc_scratch_bytes()
    K = 4096
    M = cap // (2 * K) + 1                       # M*K*2 bytes just over the array
    L = layer((302,), 64, K, 4, 128, True)
    x = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    st, _ = call_noalloc(x, L, 4, 128)
    assert st == wq.WQ_ERR_TOO_LARGE
    assert "static" in wq.status_str(st)
    # without act-order nothing has to fit: the GEMM runs unsplit if need be
    L2 = layer((303,), 64, K, 4, 128, False)
    st, y = call_noalloc(x, L2, 4, 128)
    assert st == 0 and torch.count_nonzero(y).item() == 0
