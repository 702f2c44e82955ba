"""The C-ABI library loads on the CPU, exports every declared symbol and
rejects bad arguments on the host before any device work.  No kernel is
launched here: every call below fails argument validation."""

import ctypes

import pytest

import weight_only_int4_wq_amd as wq

WQ_OK, WQ_ERR_ARG, WQ_ERR_UNSUPPORTED, WQ_ERR_HIP = 0, 1, 2, 3
FAKE = ctypes.c_void_p(0x10000)       # 16-byte aligned, never dereferenced
FAKE_MIS = ctypes.c_void_p(0x10008)   # misaligned


def _gpu_visible():
    try:
        import torch
    except ImportError:
        return False
    return torch.cuda.device_count() > 0


# The calls below pass made-up device addresses and rely on host-side
# validation rejecting them.  Where a GPU is visible a validation regression
# would launch a kernel on such an address, so they run only without one.
fake_pointers = pytest.mark.skipif(_gpu_visible(), reason="passes made-up device addresses")


def test_library_exports_every_declared_symbol():
    names = wq.exported_names()
    expected = {"wq_status_str", "wq_version", "wq_quantize_rtn", "wq_awq_scales", "wq_awq_fold",
                "wq_act_order_perm", "wq_pack", "wq_unpack", "wq_dequant", "wq_scale_act",
                "wq_workspace_size", "wq_gemv", "wq_gemm", "wq_linear", "wq_gemv_max_m",
                "wq_awq_search", "wq_awq_search_workspace_size", "wq_gemv_silu_mul",
                "wq_gptq_quantize", "wq_gptq_workspace_size", "wq_awq_clip", "wq_gemv_ex", "wq_linear_noalloc", "wq_stream_read"}
    assert set(names) == expected
    handle = wq.lib()
    for name in names:
        assert hasattr(handle, name), name


def test_status_strings_and_version():
    assert wq.status_str(WQ_OK) == "ok"
    for code in (WQ_ERR_ARG, WQ_ERR_UNSUPPORTED, WQ_ERR_HIP):
        assert len(wq.status_str(code)) > 5
    assert wq.status_str(99) == "unknown status"
    assert wq.version().count(".") == 2
    assert 1 <= wq.gemv_max_m() <= 16


def test_workspace_size():
    # enough output tiles to fill the GPU: no split, no workspace
    assert wq.workspace_size(2048, 11008, 4096, 4, False) == 0
    # act-order gather (M*K fp16) plus, with few tiles, whole fp32 copies of y
    ws = wq.workspace_size(256, 4096, 4096, 4, True)
    gather = 256 * 4096 * 2
    assert ws > gather and (ws - gather) % (256 * 4096 * 4) == 0
    assert 2 <= (ws - gather) // (256 * 4096 * 4) <= 16
    # few tiles along a long K: split partials only
    ws = wq.workspace_size(32, 8192, 28672, 4, False)
    assert ws > 0 and ws % (32 * 8192 * 4) == 0
    # decode batch whose activations exceed LDS: fp32 partials of the K-slabs
    # (or of the GEMM's split, whichever is larger), whole copies of y
    ws = wq.workspace_size(16, 4096, 11008, 4, False)
    assert ws > 0 and ws % (16 * 4096 * 4) == 0
    # invalid arguments
    assert wq.workspace_size(0, 4096, 4096, 4, False) == 0
    assert wq.workspace_size(256, 4096, 4096, 5, False) == 0


def _mm(name, x=FAKE, packed=FAKE, scales=FAKE, zeros=None, perm=None, y=FAKE, M=1, N=64, K=128, bits=4,
        gs=128, ws=None, wsb=0):
    fn = getattr(wq.lib(), name)
    return fn(x, packed, scales, zeros, perm, y, M, N, K, bits, gs, ws, wsb, None)


@fake_pointers
@pytest.mark.parametrize("name", ["wq_gemv", "wq_gemm", "wq_linear"])
def test_matmul_argument_checks(name):
    assert _mm(name, x=None) == WQ_ERR_ARG
    assert _mm(name, scales=None) == WQ_ERR_ARG
    assert _mm(name, y=None) == WQ_ERR_ARG
    assert _mm(name, K=100) == WQ_ERR_ARG            # K not a multiple of 32
    assert _mm(name, K=0) == WQ_ERR_ARG
    assert _mm(name, M=-1) == WQ_ERR_ARG
    assert _mm(name, gs=100) == WQ_ERR_ARG           # not a multiple of 32
    assert _mm(name, gs=96, K=128) == WQ_ERR_ARG     # does not divide K
    assert _mm(name, gs=0) == WQ_ERR_ARG
    assert _mm(name, bits=5) == WQ_ERR_UNSUPPORTED
    assert _mm(name, bits=16) == WQ_ERR_UNSUPPORTED
    assert _mm(name, x=FAKE_MIS) == WQ_ERR_ARG
    assert _mm(name, y=FAKE_MIS) == WQ_ERR_ARG
    assert _mm(name, packed=FAKE_MIS) == WQ_ERR_ARG
    assert _mm(name, M=2, perm=FAKE_MIS, ws=FAKE, wsb=1 << 20) == WQ_ERR_ARG
    # empty problems are valid and enqueue nothing
    assert _mm(name, M=0) == WQ_OK
    assert _mm(name, N=0) == WQ_OK
    assert _mm(name, M=0, x=None, y=None) == WQ_OK   # an empty tensor may have no storage


@fake_pointers
def test_awq_search_argument_checks():
    L = wq.lib()
    size = L.wq_awq_search_workspace_size
    assert size(64, 32, 256, 4, 128, 20) > 0
    assert size(64, 32, 256, 4, 128, 1) == 0       # a grid needs two points
    assert size(64, 32, 250, 4, 128, 20) == 0      # K not a multiple of 32
    assert size(64, 32, 256, 5, 128, 20) == 0      # unsupported width
    assert size(64, 32, 256, 4, 96, 20) == 0       # group does not divide K
    losses = (ctypes.c_double * 20)()
    lp = ctypes.cast(losses, ctypes.c_void_p)
    assert L.wq_awq_search(None, FAKE, 64, 32, 256, 4, 128, 0, 20, lp, None, FAKE, 1 << 30, None) == WQ_ERR_ARG
    assert L.wq_awq_search(FAKE, FAKE, 64, 32, 256, 4, 128, 0, 20, None, None, FAKE, 1 << 30, None) == WQ_ERR_ARG
    assert L.wq_awq_search(FAKE_MIS, FAKE, 64, 32, 256, 4, 128, 0, 20, lp, None, FAKE, 1 << 30, None) == WQ_ERR_ARG
    assert L.wq_awq_search(FAKE, FAKE, 64, 32, 256, 5, 128, 0, 20, lp, None, FAKE, 1 << 30, None) == WQ_ERR_UNSUPPORTED
    need = size(64, 32, 256, 4, 128, 20)
    assert L.wq_awq_search(FAKE, FAKE, 64, 32, 256, 4, 128, 0, 20, lp, None, FAKE, need - 1, None) == WQ_ERR_ARG


@fake_pointers
def test_gemv_silu_mul_argument_checks():
    L = wq.lib()
    f = L.wq_gemv_silu_mul
    assert f(FAKE, FAKE, FAKE, None, None, FAKE, 1, 63, 128, 4, 128, None) == WQ_ERR_ARG       # odd N
    assert f(FAKE, FAKE, FAKE, None, None, FAKE, 5, 64, 128, 4, 128, None) == WQ_ERR_UNSUPPORTED
    assert f(None, FAKE, FAKE, None, None, FAKE, 1, 64, 128, 4, 128, None) == WQ_ERR_ARG
    assert f(FAKE, FAKE, FAKE, None, None, FAKE, 1, 64, 128, 5, 128, None) == WQ_ERR_UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, None, None, FAKE, 0, 64, 128, 4, 128, None) == WQ_OK


@fake_pointers
def test_gemv_rejects_large_m():
    assert _mm("wq_gemv", M=17) == WQ_ERR_UNSUPPORTED


@fake_pointers
def test_gemm_act_order_needs_workspace():
    assert _mm("wq_gemm", M=64, perm=FAKE) == WQ_ERR_ARG
    assert _mm("wq_gemm", M=64, perm=FAKE, ws=FAKE, wsb=64 * 128 * 2 - 1) == WQ_ERR_ARG


@fake_pointers
def test_setup_entry_points_check_arguments():
    L = wq.lib()
    assert L.wq_quantize_rtn(None, None, 4, 128, 4, 128, 0, FAKE, FAKE, FAKE, None) == WQ_ERR_ARG
    assert L.wq_quantize_rtn(FAKE, None, 4, 128, 4, 128, 0, FAKE, FAKE, None, None) == WQ_ERR_ARG  # zeros needed
    assert L.wq_quantize_rtn(FAKE, None, 4, 128, 4, 128, 1, FAKE, FAKE, FAKE, None) == WQ_ERR_ARG  # no zeros if sym
    assert L.wq_quantize_rtn(FAKE, None, 4, 128, 6, 128, 0, FAKE, FAKE, FAKE, None) == WQ_ERR_UNSUPPORTED
    assert L.wq_awq_scales(FAKE, 4, 128, 1.5, FAKE, None) == WQ_ERR_ARG
    assert L.wq_awq_scales(FAKE, 4, 128, -0.1, FAKE, None) == WQ_ERR_ARG
    assert L.wq_awq_fold(None, FAKE, 4, 128, FAKE, None) == WQ_ERR_ARG
    assert L.wq_act_order_perm(FAKE, 128, 96, FAKE, None) == WQ_ERR_ARG
    assert L.wq_act_order_perm(FAKE, 100, 32, FAKE, None) == WQ_ERR_ARG
    assert L.wq_pack(FAKE, None, 100, 4, 4, 128, FAKE, None, None) == WQ_ERR_ARG
    assert L.wq_pack(FAKE, FAKE, 128, 4, 4, 128, FAKE, None, None) == WQ_ERR_ARG   # perm required
    assert L.wq_pack(FAKE, None, 128, 4, 7, 128, FAKE, None, None) == WQ_ERR_UNSUPPORTED
    assert L.wq_unpack(FAKE_MIS, None, 128, 4, 4, FAKE, None) == WQ_ERR_ARG
    assert L.wq_dequant(FAKE, None, None, None, 128, 4, 4, 128, FAKE, None) == WQ_ERR_ARG
    assert L.wq_scale_act(FAKE, FAKE, 4, 100, FAKE, None) == WQ_ERR_ARG
    assert L.wq_scale_act(FAKE, FAKE_MIS, 4, 128, FAKE, None) == WQ_ERR_ARG
    assert L.wq_scale_act(FAKE, FAKE, 0, 128, FAKE, None) == WQ_OK


def test_binding_raises_on_status():
    with pytest.raises(wq.WQError):
        wq._check(WQ_ERR_ARG, "wq_gemv")


@fake_pointers
def test_gptq_argument_checks():
    L = wq.lib()
    size = L.wq_gptq_workspace_size
    assert size(64, 32, 256) > 5 * 256 * 256 * 4
    assert size(0, 32, 256) == 0

    def call(x=FAKE, w=FAKE, M=64, N=32, K=256, bits=4, gs=128, sym=0, damp=0.01, zeros=FAKE, ws=FAKE,
             wsb=1 << 30, act=0, g_idx=None):
        return L.wq_gptq_quantize(x, w, M, N, K, bits, gs, sym, damp, act, FAKE, FAKE, zeros, g_idx, ws, wsb, None)

    assert call(x=None) == WQ_ERR_ARG
    assert call(ws=None) == WQ_ERR_ARG
    assert call(M=48) == WQ_ERR_ARG                # M not a multiple of 32
    assert call(K=250) == WQ_ERR_ARG
    assert call(gs=96, K=384) == WQ_ERR_ARG        # neither divides nor is a multiple of the 64-column block
    assert call(bits=5) == WQ_ERR_UNSUPPORTED
    assert call(sym=1) == WQ_ERR_ARG               # symmetric takes no zeros
    assert call(zeros=None) == WQ_ERR_ARG          # asymmetric needs zeros
    assert call(damp=-0.1) == WQ_ERR_ARG
    assert call(damp=1.0) == WQ_ERR_ARG
    assert call(x=FAKE_MIS) == WQ_ERR_ARG
    assert call(wsb=size(64, 32, 256) - 1) == WQ_ERR_ARG
    assert call(act=1) == WQ_ERR_ARG               # act-order needs the g_idx output


@fake_pointers
def test_awq_clip_argument_checks():
    f = wq.lib().wq_awq_clip

    def call(x=FAKE, w=FAKE, M=64, N=32, K=256, bits=4, gs=128, sym=0, n_grid=20, n_ratios=10, out=FAKE):
        return f(x, w, M, N, K, bits, gs, sym, n_grid, n_ratios, out, None, None, None)

    assert call(x=None) == WQ_ERR_ARG
    assert call(out=None) == WQ_ERR_ARG
    assert call(M=0) == WQ_ERR_ARG
    assert call(K=250) == WQ_ERR_ARG
    assert call(gs=96, K=192) == WQ_ERR_UNSUPPORTED     # only 32, 64, 128, 256
    assert call(gs=-1, K=512) == WQ_ERR_UNSUPPORTED
    assert call(gs=100) == WQ_ERR_ARG
    assert call(bits=5) == WQ_ERR_UNSUPPORTED
    assert call(n_ratios=0) == WQ_ERR_ARG
    assert call(n_ratios=21) == WQ_ERR_ARG              # more ratios than grid steps
    assert call(out=FAKE_MIS) == WQ_ERR_ARG


@fake_pointers
def test_gemv_ex_argument_checks():
    f = wq.lib().wq_gemv_ex

    def call(x=FAKE, s=None, b=None, y=FAKE, M=1, N=64, K=128, bits=4, gs=128, silu=0):
        return f(x, FAKE, FAKE, None, None, s, b, y, M, N, K, bits, gs, silu, None)

    assert call(x=None) == WQ_ERR_ARG
    assert call(s=FAKE_MIS) == WQ_ERR_ARG          # act_scale must be 16-byte aligned
    assert call(silu=1, N=63) == WQ_ERR_ARG
    assert call(M=5) == WQ_ERR_UNSUPPORTED
    assert call(bits=5) == WQ_ERR_UNSUPPORTED
    assert call(M=0) == WQ_OK


def _declared_names():
    import os
    import re
    src = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "wq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(wq_[a-z_0-9]+)\s*\(", src, flags=re.M))


def test_header_declares_exactly_the_exports():
    declared = _declared_names()
    assert len(declared) >= 20
    assert declared == set(wq.exported_names())


def test_header_is_plain_c(tmp_path):
    import os
    import shutil
    import subprocess
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("no C compiler")
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    src = tmp_path / "use_wq.c"
    names = sorted(_declared_names())
    src.write_text("#include <wq.h>\n#include <stdio.h>\ntypedef void (*fn_t)(void);\nint main(void) {\n"
                   "    const fn_t fns[] = {\n" + "".join(f"        (fn_t)&{n},\n" for n in names) + "    };\n"
                   "    printf(\"%d\\n\", (int)(sizeof fns / sizeof fns[0]));\n    return 0;\n}\n")
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", inc, "-c", str(src), "-o",
                        str(tmp_path / "use_wq.o")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
