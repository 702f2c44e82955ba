"""The Python binding's argument checks, on the CPU.

The C ABI receives bare pointers and cannot tell a short buffer from a long
one, so the binding checks every shape and device before it takes a
pointer.  These tests use storage-less "meta" tensors: every shape error
must surface as ValueError, and a call whose shapes are all consistent must
still refuse to pass non-GPU memory to the library."""

import pytest

torch = pytest.importorskip("torch")
import weight_only_int4_wq_amd as wq  # noqa: E402

M, N, K, BITS, GS = 2, 64, 256, 4, 128
G = K // GS


def meta(*shape, dtype=torch.float16):
    return torch.empty(shape, dtype=dtype, device="meta")


def layer():
    return dict(packed=meta(N, K * BITS // 32, dtype=torch.int32), scales=meta(N, G),
                zeros=meta(N, G, dtype=torch.uint8))


def test_consistent_meta_call_refuses_non_gpu_memory():
    L = layer()
    with pytest.raises(ValueError, match="GPU tensors"):
        wq.gemv(meta(M, K), L["packed"], L["scales"], L["zeros"], BITS, GS)


@pytest.mark.parametrize("fn", [wq.gemv, wq.gemm, wq.linear])
def test_product_out_shape_is_checked(fn):
    L = layer()
    for bad in ((M, N - 1), (M + 1, N), (N, M)):
        with pytest.raises(ValueError, match="out must have shape"):
            fn(meta(M, K), L["packed"], L["scales"], L["zeros"], BITS, GS, out=meta(*bad))


def test_product_operand_shapes_are_checked():
    L = layer()
    with pytest.raises(ValueError, match="scales"):
        wq.gemv(meta(M, K), L["packed"], meta(N, G + 1), L["zeros"], BITS, GS)
    with pytest.raises(ValueError, match="zeros"):
        wq.gemv(meta(M, K), L["packed"], L["scales"], meta(N - 1, G, dtype=torch.uint8), BITS, GS)
    with pytest.raises(ValueError, match="packed"):
        wq.gemv(meta(M, K + 32), L["packed"], L["scales"], L["zeros"], BITS, GS)
    with pytest.raises(ValueError, match="perm"):
        wq.gemv(meta(M, K), L["packed"], L["scales"], L["zeros"], BITS, GS, perm=meta(K - 1, dtype=torch.int32))


def test_operands_must_share_the_activation_device():
    L = layer()
    with pytest.raises(ValueError, match="is on cpu"):
        wq.gemv(meta(M, K), torch.empty(L["packed"].shape, dtype=torch.int32), L["scales"], L["zeros"], BITS, GS)
    with pytest.raises(ValueError, match="is on cpu"):
        wq.gemv(meta(M, K), L["packed"], L["scales"], L["zeros"], BITS, GS, out=torch.empty((M, N), dtype=torch.float16))


def test_fused_entry_points_check_out_scale_and_bias():
    L = layer()
    x = meta(M, K)
    with pytest.raises(ValueError, match="out must have shape"):
        wq.gemv_silu_mul(x, L["packed"], L["scales"], L["zeros"], BITS, GS, out=meta(M, N))
    with pytest.raises(ValueError, match="act_scale"):
        wq.gemv_ex(x, L["packed"], L["scales"], L["zeros"], BITS, GS, act_scale=meta(K - 8))
    with pytest.raises(ValueError, match="bias"):
        wq.gemv_ex(x, L["packed"], L["scales"], L["zeros"], BITS, GS, bias=meta(N // 2))
    with pytest.raises(ValueError, match="out must have shape"):
        wq.gemv_ex(x, L["packed"], L["scales"], L["zeros"], BITS, GS, silu=True, out=meta(M, N))


def test_activation_scaling_and_fold_check_s_and_out():
    x = meta(M, K)
    with pytest.raises(ValueError, match="s must have shape"):
        wq.scale_act(x, meta(K - 1))
    with pytest.raises(ValueError, match="out must have shape"):
        wq.scale_act(x, meta(K), out=meta(M, K - 8))
    w = meta(N, K)
    with pytest.raises(ValueError, match="s must have shape"):
        wq.awq_fold(w, meta(N))
    with pytest.raises(ValueError, match="out must have shape"):
        wq.awq_fold(w, meta(K), out=meta(N - 1, K))
    with pytest.raises(ValueError, match="out must have shape"):
        wq.awq_clip(meta(16, K), w, out=meta(N, K // 2))


def test_quantized_linear_falls_back_when_the_fused_kernel_declines(monkeypatch):
    # the library's fused decode entry point reports shapes it does not
    # take as WQ_ERR_UNSUPPORTED; the layer then scales x and runs the
    # plain product (no size rule of its own)
    calls = []

    def gemv_ex(*a, **k):
        calls.append("gemv_ex")
        raise wq.WQError("unsupported", wq.WQ_ERR_UNSUPPORTED)

    def scale_act(x, s):
        calls.append("scale_act")
        return x

    def linear(x, *a, **k):
        calls.append("linear")
        return "y"

    monkeypatch.setattr(wq, "gemv_ex", gemv_ex)
    monkeypatch.setattr(wq, "scale_act", scale_act)
    monkeypatch.setattr(wq, "linear", linear)
    monkeypatch.setattr(wq, "gemv_max_m", lambda: 4)
    L = layer()
    q = wq.QuantizedLinear(L["packed"], L["scales"], L["zeros"], BITS, GS, K, act_scale=meta(K))
    assert q(meta(1, K)) == "y"
    assert calls == ["gemv_ex", "scale_act", "linear"]

    def gemv_ex_bad(*a, **k):
        raise wq.WQError("bad argument", wq.WQ_ERR_ARG)

    monkeypatch.setattr(wq, "gemv_ex", gemv_ex_bad)
    with pytest.raises(wq.WQError):
        q(meta(1, K))
