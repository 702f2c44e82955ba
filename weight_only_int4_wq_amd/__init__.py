"""Weight-only quantized linear layers on AMD gfx950 (MI355X).

Thin Python binding over libwq.so, the HIP library whose C ABI is declared in
include/wq.h.  Every function here only checks and marshals arguments (torch
tensors for device memory, torch's current HIP stream) and calls the entry
point of the same name; all computation runs in the library's kernels.
There is no fallback: if libwq.so is missing or cannot be loaded, every call
raises.
"""

from __future__ import annotations

import ctypes
import os
import re

__all__ = [
    "lib", "lib_path", "header_path", "exported_names", "WQError",
    "quantize_rtn", "awq_scales", "awq_fold", "awq_search", "awq_clip", "gptq_quantize", "act_order_perm", "pack", "unpack",
    "dequant", "scale_act", "workspace_size", "gemv", "gemm", "linear", "gemv_silu_mul", "gemv_ex", "gemv_max_m",
    "linear_noalloc", "noalloc_scratch_bytes", "stream_read",
    "status_str", "version", "QuantizedLinear",
]

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_PKG_DIR, "libwq.so")
header_path = os.path.join(os.path.dirname(_PKG_DIR), "include", "wq.h")

_lib = None

_VP = ctypes.c_void_p
_I32 = ctypes.c_int32
_SIG = {
    "wq_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "wq_version": (ctypes.c_char_p, []),
    "wq_quantize_rtn": (ctypes.c_int, [_VP, _VP, _I32, _I32, _I32, _I32, _I32, _VP, _VP, _VP, _VP]),
    "wq_awq_scales": (ctypes.c_int, [_VP, _I32, _I32, ctypes.c_double, _VP, _VP]),
    "wq_awq_fold": (ctypes.c_int, [_VP, _VP, _I32, _I32, _VP, _VP]),
    "wq_act_order_perm": (ctypes.c_int, [_VP, _I32, _I32, _VP, _VP]),
    "wq_pack": (ctypes.c_int, [_VP, _VP, _I32, _I32, _I32, _I32, _VP, _VP, _VP]),
    "wq_unpack": (ctypes.c_int, [_VP, _VP, _I32, _I32, _I32, _VP, _VP]),
    "wq_dequant": (ctypes.c_int, [_VP, _VP, _VP, _VP, _I32, _I32, _I32, _I32, _VP, _VP]),
    "wq_scale_act": (ctypes.c_int, [_VP, _VP, _I32, _I32, _VP, _VP]),
    "wq_workspace_size": (ctypes.c_size_t, [_I32, _I32, _I32, _I32, _I32]),
    "wq_gemv_max_m": (_I32, []),
    "wq_awq_search": (ctypes.c_int, [_VP, _VP, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _VP, _VP, _VP,
                                     ctypes.c_size_t, _VP]),
    "wq_awq_search_workspace_size": (ctypes.c_size_t, [_I32, _I32, _I32, _I32, _I32, _I32]),
    "wq_gptq_quantize": (ctypes.c_int, [_VP, _VP, _I32, _I32, _I32, _I32, _I32, _I32, ctypes.c_double, _I32, _VP,
                                        _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP]),
    "wq_gptq_workspace_size": (ctypes.c_size_t, [_I32, _I32, _I32]),
    "wq_awq_clip": (ctypes.c_int, [_VP, _VP, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _VP, _VP, _VP, _VP]),
}
_SIG["wq_gemv_silu_mul"] = (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _I32, _I32, _I32, _I32, _I32, _VP])
_SIG["wq_stream_read"] = (ctypes.c_int, [_VP, ctypes.c_size_t, _VP, _VP])
_SIG["wq_linear_noalloc"] = (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _I32, _I32, _I32, _I32, _I32, _VP])
_SIG["wq_gemv_ex"] = (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _I32, _I32, _I32, _I32, _I32, _VP])
for _name in ("wq_gemv", "wq_gemm", "wq_linear"):
    _SIG[_name] = (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _I32, _I32, _I32, _I32, _I32,
                                  _VP, ctypes.c_size_t, _VP])


WQ_ERR_ARG, WQ_ERR_UNSUPPORTED, WQ_ERR_HIP, WQ_ERR_TOO_LARGE = 1, 2, 3, 4


class WQError(RuntimeError):
    """A libwq entry point returned a non-zero status (kept in `status`)."""

    def __init__(self, msg, status=0):
        super().__init__(msg)
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libwq.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise RuntimeError(
                f"{lib_path} is missing: build it with `python -m weight_only_int4_wq_amd.build` "
                "(there is no non-HIP fallback)")
        handle = ctypes.CDLL(lib_path)
        for name, (res, args) in _SIG.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def exported_names() -> list:
    """Function names declared in include/wq.h."""
    with open(header_path) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(wq_[a-z0-9_]+)\s*\(", text)) - {"wq_status"})


def status_str(code: int) -> str:
    return lib().wq_status_str(code).decode()


def version() -> str:
    return lib().wq_version().decode()


def gemv_max_m() -> int:
    return int(lib().wq_gemv_max_m())


def _check(code: int, what: str) -> None:
    if code != 0:
        raise WQError(f"{what}: {status_str(code)} (status {code})", code)


# ----------------------------------------------------------- marshalling --

def _torch():
    import torch
    return torch


def _dev(t, dtype, name, ndim=None, allow_none=False, shape=None, device=None):
    """Check a tensor argument: dtype, contiguity, rank, and when given its
    exact shape and device (the C ABI sees only pointers, so a short or
    misplaced buffer must be caught here).  That it is a GPU tensor is
    checked when its pointer is taken, after every shape check."""
    torch = _torch()
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _ptr(t):
    if t is None:
        return None
    if t.device.type != "cuda":
        raise ValueError(f"tensor arguments must be GPU tensors, got one on {t.device}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device=None):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _groups(K: int, group_size: int) -> int:
    return 1 if group_size == -1 else K // group_size


# ------------------------------------------------------------ set-up ops --

def quantize_rtn(w, bits: int, group_size: int, perm=None, symmetric: bool = False):
    """RTN group quantization of fp16 w [N][K] -> (codes u8 [N][K], scales fp16
    [N][G], zeros u8 [N][G] or None)."""
    torch = _torch()
    w = _dev(w, torch.float16, "w", 2)
    N, K = w.shape
    perm = _dev(perm, torch.int32, "perm", 1, allow_none=True, shape=(K,), device=w.device)
    G = _groups(K, group_size)
    codes = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    scales = torch.empty((N, G), dtype=torch.float16, device=w.device)
    zeros = None if symmetric else torch.empty((N, G), dtype=torch.uint8, device=w.device)
    _check(lib().wq_quantize_rtn(_ptr(w), _ptr(perm), N, K, bits, group_size, int(symmetric),
                                 _ptr(codes), _ptr(scales), _ptr(zeros), _stream(w.device)),
           "wq_quantize_rtn")
    return codes, scales, zeros


def awq_scales(x, alpha: float = 0.5):
    """AWQ per-input-channel scale fp16 [K] from activations x fp16 [M][K]."""
    torch = _torch()
    x = _dev(x, torch.float16, "x", 2)
    M, K = x.shape
    s = torch.empty((K,), dtype=torch.float16, device=x.device)
    _check(lib().wq_awq_scales(_ptr(x), M, K, float(alpha), _ptr(s), _stream(x.device)), "wq_awq_scales")
    return s


def awq_fold(w, s, out=None):
    """fp16(W[n][k] * s[k])."""
    torch = _torch()
    w = _dev(w, torch.float16, "w", 2)
    N, K = w.shape
    s = _dev(s, torch.float16, "s", 1, shape=(K,), device=w.device)
    out = torch.empty_like(w) if out is None else _dev(out, torch.float16, "out", 2, shape=(N, K), device=w.device)
    _check(lib().wq_awq_fold(_ptr(w), _ptr(s), N, K, _ptr(out), _stream(w.device)), "wq_awq_fold")
    return out


def awq_search(x, w, bits: int = 4, group_size: int = 128, n_grid: int = 20, symmetric: bool = False):
    """AWQ's grid search for alpha on calibration activations x fp16 [M][K]
    and weights w fp16 [N][K].  Returns (alphas list, losses list, best
    index); alpha_i = i / (n_grid - 1).  Synchronizes the stream."""
    torch = _torch()
    x = _dev(x, torch.float16, "x", 2)
    w = _dev(w, torch.float16, "w", 2, device=x.device)
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError("w must be [N][K] with the K of x")
    need = int(lib().wq_awq_search_workspace_size(M, N, K, bits, group_size, n_grid))
    if need == 0:
        raise ValueError("invalid AWQ search arguments")
    ws = torch.empty((need,), dtype=torch.uint8, device=x.device)
    losses = (ctypes.c_double * n_grid)()
    best = ctypes.c_int32(-1)
    _check(lib().wq_awq_search(_ptr(x), _ptr(w), M, N, K, bits, group_size, int(bool(symmetric)), n_grid,
                               ctypes.cast(losses, _VP), ctypes.cast(ctypes.byref(best), _VP), _ptr(ws), need,
                               _stream(x.device)), "wq_awq_search")
    alphas = [i / (n_grid - 1) for i in range(n_grid)]
    return alphas, list(losses), int(best.value)


def awq_clip(x, w, bits: int = 4, group_size: int = 128, n_grid: int = 20, n_ratios: int = 10,
             symmetric: bool = False, out=None, with_losses: bool = False):
    """AWQ's clipping-threshold search on calibration activations x fp16
    [M][K] for weights w fp16 [N][K] -> (w_clip fp16 [N][K], best int32
    [N][G], losses fp32 [N][G][n_ratios] or None).  out may be w (in place)."""
    torch = _torch()
    x = _dev(x, torch.float16, "x", 2)
    w = _dev(w, torch.float16, "w", 2, device=x.device)
    N, K = w.shape
    if x.shape[1] != K:
        raise ValueError("x must be [M][K] with the K of w")
    G = _groups(K, group_size)
    out = torch.empty_like(w) if out is None else _dev(out, torch.float16, "out", 2, shape=(N, K), device=w.device)
    best = torch.empty((N, G), dtype=torch.int32, device=w.device)
    losses = torch.empty((N, G, n_ratios), dtype=torch.float32, device=w.device) if with_losses else None
    _check(lib().wq_awq_clip(_ptr(x), _ptr(w), x.shape[0], N, K, bits, group_size, int(bool(symmetric)), n_grid,
                             n_ratios, _ptr(out), _ptr(best), _ptr(losses), _stream(w.device)), "wq_awq_clip")
    return out, best, losses


def gptq_quantize(w, x, bits: int = 4, group_size: int = 128, symmetric: bool = False, damp: float = 0.01,
                  act_order: bool = False):
    """GPTQ of fp16 w [N][K] on calibration activations x fp16 [M][K] ->
    (codes u8 [N][K], scales fp16 [N][G], zeros u8 [N][G] or None, g_idx
    int32 [K] or None), the layout quantize_rtn returns plus the act-order
    group map."""
    torch = _torch()
    w = _dev(w, torch.float16, "w", 2)
    x = _dev(x, torch.float16, "x", 2, device=w.device)
    N, K = w.shape
    M = x.shape[0]
    if x.shape[1] != K:
        raise ValueError("x must be [M][K] with the K of w")
    need = int(lib().wq_gptq_workspace_size(M, N, K))
    if need == 0:
        raise ValueError("invalid GPTQ sizes")
    G = _groups(K, group_size)
    ws = torch.empty((need,), dtype=torch.uint8, device=w.device)
    codes = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    scales = torch.empty((N, G), dtype=torch.float16, device=w.device)
    zeros = None if symmetric else torch.empty((N, G), dtype=torch.uint8, device=w.device)
    g_idx = torch.empty((K,), dtype=torch.int32, device=w.device) if act_order else None
    _check(lib().wq_gptq_quantize(_ptr(x), _ptr(w), M, N, K, bits, group_size, int(bool(symmetric)), float(damp),
                                  int(bool(act_order)), _ptr(codes), _ptr(scales), _ptr(zeros), _ptr(g_idx), _ptr(ws),
                                  need, _stream(w.device)), "wq_gptq_quantize")
    return codes, scales, zeros, g_idx


def act_order_perm(g_idx, group_size: int):
    """Stable packing order of the act-order group map (synchronizes)."""
    torch = _torch()
    g_idx = _dev(g_idx, torch.int32, "g_idx", 1)
    K = g_idx.shape[0]
    perm = torch.empty((K,), dtype=torch.int32, device=g_idx.device)
    _check(lib().wq_act_order_perm(_ptr(g_idx), K, group_size, _ptr(perm), _stream(g_idx.device)),
           "wq_act_order_perm")
    return perm


def pack(codes, bits: int, group_size: int = -1, g_idx=None):
    """Pack codes u8 [N][K] -> (packed int32 [N][K*bits/32] holding uint32
    words, perm int32 [K] or None)."""
    torch = _torch()
    codes = _dev(codes, torch.uint8, "codes", 2)
    N, K = codes.shape
    g_idx = _dev(g_idx, torch.int32, "g_idx", 1, allow_none=True, shape=(K,), device=codes.device)
    if (K * bits) % 32:
        raise ValueError("K * bits must be a multiple of 32")
    packed = torch.empty((N, K * bits // 32), dtype=torch.int32, device=codes.device)
    perm = None if g_idx is None else torch.empty((K,), dtype=torch.int32, device=codes.device)
    _check(lib().wq_pack(_ptr(codes), _ptr(g_idx), K, N, bits, group_size, _ptr(packed), _ptr(perm),
                         _stream(codes.device)), "wq_pack")
    return packed, perm


def unpack(packed, bits: int, K: int, perm=None):
    torch = _torch()
    packed = _dev(packed, torch.int32, "packed", 2)
    perm = _dev(perm, torch.int32, "perm", 1, allow_none=True, shape=(K,), device=packed.device)
    N = packed.shape[0]
    if packed.shape[1] * 32 != K * bits:
        raise ValueError("packed width does not match K * bits / 32")
    codes = torch.empty((N, K), dtype=torch.uint8, device=packed.device)
    _check(lib().wq_unpack(_ptr(packed), _ptr(perm), K, N, bits, _ptr(codes), _stream(packed.device)),
           "wq_unpack")
    return codes


def dequant(packed, scales, zeros, bits: int, group_size: int, K: int, perm=None):
    """fp16 dequantized weights [N][K] in original channel order."""
    torch = _torch()
    packed = _dev(packed, torch.int32, "packed", 2)
    d = packed.device
    scales = _dev(scales, torch.float16, "scales", 2, device=d)
    zeros = _dev(zeros, torch.uint8, "zeros", 2, allow_none=True, device=d)
    perm = _dev(perm, torch.int32, "perm", 1, allow_none=True, device=d)
    N = packed.shape[0]
    _check_meta(N, K, bits, group_size, packed, scales, zeros, perm)
    w = torch.empty((N, K), dtype=torch.float16, device=packed.device)
    _check(lib().wq_dequant(_ptr(packed), _ptr(scales), _ptr(zeros), _ptr(perm), K, N, bits, group_size,
                            _ptr(w), _stream(packed.device)), "wq_dequant")
    return w


def _check_meta(N, K, bits, group_size, packed, scales, zeros, perm):
    G = _groups(K, group_size) if group_size == -1 or (group_size > 0 and K % group_size == 0) else None
    if packed.shape != (N, K * bits // 32):
        raise ValueError("packed must be [N][K*bits/32]")
    if G is not None and tuple(scales.shape) != (N, G):
        raise ValueError("scales must be [N][G]")
    if zeros is not None and G is not None and tuple(zeros.shape) != (N, G):
        raise ValueError("zeros must be [N][G]")
    if perm is not None and tuple(perm.shape) != (K,):
        raise ValueError("perm must be [K]")


def _layer_args(x, packed, scales, zeros, perm, bits, group_size):
    """Check the operands of a product call: types, shapes against x's K and
    packed's N, and that every one lives on x's device."""
    torch = _torch()
    x = _dev(x, torch.float16, "x", 2)
    d = x.device
    packed = _dev(packed, torch.int32, "packed", 2, device=d)
    scales = _dev(scales, torch.float16, "scales", 2, device=d)
    zeros = _dev(zeros, torch.uint8, "zeros", 2, allow_none=True, device=d)
    perm = _dev(perm, torch.int32, "perm", 1, allow_none=True, device=d)
    _check_meta(packed.shape[0], x.shape[1], bits, group_size, packed, scales, zeros, perm)
    return x, packed, scales, zeros, perm


# ----------------------------------------------------------- hot path ----

def scale_act(x, s, out=None):
    """fp16(x / s) per input channel (AWQ activation side)."""
    torch = _torch()
    x = _dev(x, torch.float16, "x", 2)
    M, K = x.shape
    s = _dev(s, torch.float16, "s", 1, shape=(K,), device=x.device)
    out = torch.empty_like(x) if out is None else _dev(out, torch.float16, "out", 2, shape=(M, K), device=x.device)
    _check(lib().wq_scale_act(_ptr(x), _ptr(s), M, K, _ptr(out), _stream(x.device)), "wq_scale_act")
    return out


def workspace_size(M: int, N: int, K: int, bits: int, has_perm: bool) -> int:
    """Bytes of workspace wq_gemv, wq_gemm and wq_linear use for these
    arguments (act-order gather, split-K partials); 0 when none."""
    return int(lib().wq_workspace_size(M, N, K, bits, int(bool(has_perm))))


def _matmul(entry: str, x, packed, scales, zeros, bits, group_size, perm=None, out=None, workspace=None):
    torch = _torch()
    x, packed, scales, zeros, perm = _layer_args(x, packed, scales, zeros, perm, bits, group_size)
    M, K = x.shape
    N = packed.shape[0]
    y = torch.empty((M, N), dtype=torch.float16, device=x.device) if out is None else \
        _dev(out, torch.float16, "out", 2, shape=(M, N), device=x.device)
    # one query sizes the GEMM's act-order gather and split-K partials and the
    # decode kernel's K split (M <= 32, no act-order); the act-order GEMV
    # uses no workspace
    need = 0 if (entry == "wq_gemv" and perm is not None) else workspace_size(M, N, K, bits, perm is not None)
    ws_bytes = 0
    if need:
        if workspace is None:
            workspace = torch.empty((need,), dtype=torch.uint8, device=x.device)
        workspace = _dev(workspace, torch.uint8, "workspace", 1, device=x.device)
        ws_bytes = workspace.numel()
    else:
        workspace = None
    fn = getattr(lib(), entry)
    _check(fn(_ptr(x), _ptr(packed), _ptr(scales), _ptr(zeros), _ptr(perm), _ptr(y), M, N, K, bits,
              group_size, _ptr(workspace), ws_bytes, _stream(x.device)), entry)
    return y


def gemv(x, packed, scales, zeros, bits: int, group_size: int, perm=None, out=None, workspace=None):
    """Decode kernel, 1 <= M <= 16; up to 32 without act-order for K >= 256."""
    return _matmul("wq_gemv", x, packed, scales, zeros, bits, group_size, perm, out, workspace)


def gemm(x, packed, scales, zeros, bits: int, group_size: int, perm=None, out=None, workspace=None):
    """Matrix-core kernel, any M."""
    return _matmul("wq_gemm", x, packed, scales, zeros, bits, group_size, perm, out, workspace)


def linear(x, packed, scales, zeros, bits: int, group_size: int, perm=None, out=None, workspace=None):
    """Batch-size dispatch between gemv and gemm."""
    return _matmul("wq_linear", x, packed, scales, zeros, bits, group_size, perm, out, workspace)


def stream_read(src, nbytes: int, sink):
    """Measurement reference: read nbytes of src (a device tensor) with the
    plain streaming-read kernel; sink is an int32 device tensor of >= 1 entry."""
    torch = _torch()
    src = _dev(src, src.dtype if src is not None else torch.uint8, "src")
    sink = _dev(sink, torch.int32, "sink", 1)
    if nbytes > src.numel() * src.element_size():
        raise ValueError("nbytes exceeds src")
    _check(lib().wq_stream_read(_ptr(src), int(nbytes), _ptr(sink), _stream(src.device)), "wq_stream_read")


def noalloc_scratch_bytes() -> int:
    """Size of linear_noalloc's static scratch array (WQ_NOALLOC_SCRATCH_BYTES
    in include/wq.h)."""
    with open(header_path) as f:
        m = re.search(r"#define\s+WQ_NOALLOC_SCRATCH_BYTES\s+\((\d+)u \* (\d+)u \* (\d+)u\)", f.read())
    return int(m.group(1)) * int(m.group(2)) * int(m.group(3))


def linear_noalloc(x, packed, scales, zeros, bits: int, group_size: int, perm=None, out=None):
    """linear without a workspace: the library's static scratch array holds
    the GEMM's intermediates.  Calls on one GPU must be ordered."""
    torch = _torch()
    x, packed, scales, zeros, perm = _layer_args(x, packed, scales, zeros, perm, bits, group_size)
    M, K = x.shape
    N = packed.shape[0]
    y = torch.empty((M, N), dtype=torch.float16, device=x.device) if out is None else \
        _dev(out, torch.float16, "out", 2, shape=(M, N), device=x.device)
    _check(lib().wq_linear_noalloc(_ptr(x), _ptr(packed), _ptr(scales), _ptr(zeros), _ptr(perm), _ptr(y), M, N, K,
                                   bits, group_size, _stream(x.device)), "wq_linear_noalloc")
    return y


def gemv_silu_mul(x, packed, scales, zeros, bits: int, group_size: int, perm=None, out=None):
    """Fused gate/up decode projection: packed holds the gate rows stacked
    over the up rows (N = 2I); returns fp16 [M][I] = silu(gate) * up."""
    torch = _torch()
    x, packed, scales, zeros, perm = _layer_args(x, packed, scales, zeros, perm, bits, group_size)
    M, K = x.shape
    N = packed.shape[0]
    if N % 2:
        raise ValueError("the stacked gate/up weight needs an even row count")
    y = torch.empty((M, N // 2), dtype=torch.float16, device=x.device) if out is None else \
        _dev(out, torch.float16, "out", 2, shape=(M, N // 2), device=x.device)
    _check(lib().wq_gemv_silu_mul(_ptr(x), _ptr(packed), _ptr(scales), _ptr(zeros), _ptr(perm), _ptr(y), M, N, K,
                                  bits, group_size, _stream(x.device)), "wq_gemv_silu_mul")
    return y


def gemv_ex(x, packed, scales, zeros, bits: int, group_size: int, perm=None, act_scale=None, bias=None,
            silu: bool = False, out=None):
    """Decode GEMV (M <= 4) with the AWQ activation scaling x' = fp16(x / s)
    done while the activations are staged (act_scale fp16 [K]) and a bias
    (fp16 [N]) added before the output rounding; with silu the stacked
    gate/up epilogue of gemv_silu_mul (bias on both halves first)."""
    torch = _torch()
    x, packed, scales, zeros, perm = _layer_args(x, packed, scales, zeros, perm, bits, group_size)
    M, K = x.shape
    N = packed.shape[0]
    act_scale = _dev(act_scale, torch.float16, "act_scale", 1, allow_none=True, shape=(K,), device=x.device)
    bias = _dev(bias, torch.float16, "bias", 1, allow_none=True, shape=(N,), device=x.device)
    if silu and N % 2:
        raise ValueError("the stacked gate/up weight needs an even row count")
    cols = N // 2 if silu else N
    y = torch.empty((M, cols), dtype=torch.float16, device=x.device) if out is None else \
        _dev(out, torch.float16, "out", 2, shape=(M, cols), device=x.device)
    _check(lib().wq_gemv_ex(_ptr(x), _ptr(packed), _ptr(scales), _ptr(zeros), _ptr(perm), _ptr(act_scale),
                            _ptr(bias), _ptr(y), M, N, K, bits, group_size, int(bool(silu)), _stream(x.device)),
           "wq_gemv_ex")
    return y


class QuantizedLinear:
    """A quantized linear layer held in device memory: packed weights, group
    scales and zero-points, optional act-order perm and AWQ input scale.

    `from_float` quantizes fp16 weights on the GPU (optionally folding an AWQ
    scale first); calling the object runs y = x . dequant(Wq)^T.
    """

    def __init__(self, packed, scales, zeros, bits, group_size, K, perm=None, act_scale=None):
        self.packed, self.scales, self.zeros = packed, scales, zeros
        self.bits, self.group_size, self.K = bits, group_size, K
        self.N = packed.shape[0]
        self.perm, self.act_scale = perm, act_scale

    @classmethod
    def from_float(cls, w, bits: int = 4, group_size: int = 128, g_idx=None, symmetric: bool = False,
                   act_scale=None):
        if act_scale is not None:
            w = awq_fold(w, act_scale)
        N, K = w.shape
        perm = None
        if g_idx is not None:
            perm = act_order_perm(g_idx, group_size)
        codes, scales, zeros = quantize_rtn(w, bits, group_size, perm=perm, symmetric=symmetric)
        packed, perm2 = pack(codes, bits, group_size, g_idx=g_idx)
        return cls(packed, scales, zeros, bits, group_size, K, perm2, act_scale)

    def __call__(self, x, out=None, workspace=None, kernel: str = "linear"):
        if self.act_scale is not None:
            if kernel in ("linear", "gemv") and 1 <= x.shape[0] <= gemv_max_m():
                # decode: the division happens while the GEMV stages x; the
                # library reports the shapes its fused kernel does not take
                try:
                    return gemv_ex(x, self.packed, self.scales, self.zeros, self.bits, self.group_size,
                                   perm=self.perm, act_scale=self.act_scale, out=out)
                except WQError as e:
                    if e.status != WQ_ERR_UNSUPPORTED:
                        raise
            x = scale_act(x, self.act_scale)
        fn = {"linear": linear, "gemv": gemv, "gemm": gemm}[kernel]
        return fn(x, self.packed, self.scales, self.zeros, self.bits, self.group_size, self.perm, out, workspace)
