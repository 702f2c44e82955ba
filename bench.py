"""Throughput of the weight-only quantized linear layer on one MI355X.

One step = one decode token (M = 1) through the four 4-bit, group-128
quantized linears of a Llama-7B-shaped layer: fused qkv (4096 -> 12288),
o_proj (4096 -> 4096), fused gate+up (4096 -> 22016) and down
(11008 -> 4096), each dispatched by batch size (M = 1 -> the GEMV kernel).
`value` is packed-weight bytes streamed per second (GB/s).  The same JSON line
also carries the prefill figure: M = 2048, K = 4096, N = 11008 with AWQ input
scaling, in TFLOP/s on the matrix-core GEMM.

Weights are random-init (seeded Gaussian) and quantized on the GPU by the
library itself; activations are seeded Gaussian.  A rotating pool of more
than 1 GiB of distinct weight copies keeps every step reading from HBM rather
than from the 256 MB Infinity Cache.  The steps over the pool are captured
in one HIP graph (plus one for a remainder, so exactly --steps steps run)
and timed with HIP events on the stream the graphs replay on.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       python bench.py --only decode|prefill|copy|configs|silu|fused|awq|gptq
(one leg, one JSON line: the profiler runs, every synthetic workload, the
fused decode epilogues, AWQ's alpha and clipping searches, GPTQ)
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import wq_inputs as I  # noqa: E402

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, 8 TB/s
FP16_MFMA_PEAK_TFLOPS = 2516.6   # MI355X dense fp16 matrix cores (2.5 PFLOP/s)
POOL_BYTES = 1 << 30             # rotate at least 1 GiB of distinct copies

DECODE_SHAPES = [("qkv", 4096, 12288), ("o_proj", 4096, 4096), ("gate_up", 4096, 22016), ("down", 11008, 4096)]
PREFILL = dict(M=2048, K=4096, N=11008)
BITS, GROUP = 4, 128


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=1000)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--gemm-steps", type=int, default=0, help="prefill iterations (default: steps // 5)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cfg", default=None, help="with --only configs: comma-separated workload names to run "
                   "(single-gemv, llama7b-decode, prefill-awq, 70b-layer, gptq-variant)")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    p.add_argument("--only", choices=["decode", "prefill", "copy", "configs", "awq", "silu", "gptq", "fused"], default=None,
                   help="run one leg only (for profiler runs); 'copy' runs plain device-to-device "
                        "copies of a known size, the reference for scaling HBM byte counters; "
                        "'configs' times every case of the five synthetic workloads; 'awq' times "
                        "AWQ's alpha and clipping searches on the prefill layer; 'silu' the fused gate/up "
                        "decode projection; 'fused' the GEMV with x/s and bias fused; 'gptq' GPTQ of the "
                        "prefill layer")
    return p.parse_args()


def layer_bytes(M, K, N, bits=BITS, group=GROUP):
    G = K // group
    packed = N * K * bits // 8
    meta = N * G * 2 + N * G       # fp16 scales + uint8 zeros
    act = M * K * 2 + M * N * 2    # x in, y out
    return packed, packed + meta + act


# Device sources each timed kernel is built from (kernel file + shared headers).
GEMV_SOURCES = ("wq_gemv.hip", "wq_common.h")
GEMM_SOURCES = ("wq_gemm_large.hip", "wq_gemm_common.h", "wq_common.h")
# the decode projections' M = 1 kernels: K = 4096 layers refill one slot
# before its sums (4 blocks per CU), the K = 11008 layer keeps two slots
GEMV_KERNEL = ("gemv_stream_kernel<4,1,2,1,1,true,false,false,false,4,true> (qkv, o_proj, gate+up); "
               "gemv_stream_kernel<4,1,2,2,1,true,false,false,false,4,false> (down)")
GEMM_KERNEL = "gemm_large_kernel<4,true,true,false,128>"


def src_sha(parts):
    """Hash of the device sources a kernel is compiled from."""
    h = hashlib.sha256()
    for part in parts:
        with open(os.path.join(ROOT, "weight_only_int4_wq_amd", "csrc", part), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(parts, key):
    """HBM bytes per launch measured by rocprofv3 counters, if the committed
    summary was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
        entry = data[key]
        if entry.get("kernel_source_sha") != src_sha(parts):
            return None
        return entry.get("hbm_bytes_per_launch")
    except (OSError, KeyError, ValueError):
        return None


# ------------------------------------------------------------ GPU legs ----

def build_decode_pool(wq, torch):
    """One quantized copy of each decode projection, replicated into a pool."""
    base = []
    for i, (name, K, N) in enumerate(DECODE_SHAPES):
        w = torch.from_numpy(I.weights((2, K, N), N, K, 0.02)).cuda()
        layer = wq.QuantizedLinear.from_float(w, bits=BITS, group_size=GROUP)
        del w
        x = torch.from_numpy(I.activations((2, K, N), 1, K)).cuda()
        y = torch.empty((1, N), dtype=torch.float16, device="cuda")
        base.append(dict(name=name, K=K, N=N, layer=layer, x=x, y=y))
    per_copy = sum(b["layer"].packed.numel() * 4 + b["layer"].scales.numel() * 2 + b["layer"].zeros.numel()
                   for b in base)
    copies = max(2, -(-POOL_BYTES // per_copy))
    pool = [base]
    for _ in range(copies - 1):
        entry = []
        for b in base:
            L = b["layer"]
            clone = wq.QuantizedLinear(L.packed.clone(), L.scales.clone(), L.zeros.clone(), BITS, GROUP, b["K"])
            entry.append(dict(b, layer=clone))
        pool.append(entry)
    return pool, per_copy


def capture(torch, fn, n):
    """One HIP graph that runs fn(0), fn(1), ..., fn(n-1) back to back."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(n):              # eager warm-up of every pool entry
            fn(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    torch.cuda.synchronize()
    return g


def timed(torch, fn, n_pool, steps, warmup):
    """Time exactly `steps` calls fn(i % n_pool) (after `warmup` untimed ones)
    with HIP events on the stream the graphs replay on.  The calls run as
    replays of a graph of n_pool calls plus one graph for the remainder."""
    full = capture(torch, fn, n_pool)
    rem = steps % n_pool
    part = capture(torch, fn, rem) if rem else None
    stream = torch.cuda.current_stream()
    for _ in range(max(1, -(-warmup // n_pool))):
        full.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps // n_pool):
        full.replay()
    if part is not None:
        part.replay()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps  # ms per call


def decode_leg(wq, torch, steps, warmup):
    pool, per_copy = build_decode_pool(wq, torch)

    def step(i):
        for b in pool[i]:
            wq.linear(b["x"], b["layer"].packed, b["layer"].scales, b["layer"].zeros, BITS, GROUP, out=b["y"])

    ms = timed(torch, step, len(pool), steps, warmup)
    packed_b = sum(layer_bytes(1, K, N)[0] for _, K, N in DECODE_SHAPES)
    all_b = sum(layer_bytes(1, K, N)[1] for _, K, N in DECODE_SHAPES)
    # Kernel view: every launch in a step is the same GEMV kernel; the event
    # time of a step spread over its launches is the average launch duration.
    n_launch = len(DECODE_SHAPES)
    per_layer = {}
    for li, (name, K, N) in enumerate(DECODE_SHAPES):
        def one(i, li=li):
            b = pool[i][li]
            wq.linear(b["x"], b["layer"].packed, b["layer"].scales, b["layer"].zeros, BITS, GROUP, out=b["y"])
        ms1 = timed(torch, one, len(pool), steps, warmup)
        pk, al = layer_bytes(1, K, N)
        per_layer[name] = dict(K=K, N=N, us=round(ms1 * 1e3, 3), packed_GBs=round(pk / (ms1 * 1e6), 1),
                               all_GBs=round(al / (ms1 * 1e6), 1))
    # Achievable: the plain streaming-read kernel (wq_stream_read) over the
    # same packed bytes of each projection, launched and timed the same way
    # (graph replays over the rotating pool).
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    floor_us = 0.0
    for li, (name, K, N) in enumerate(DECODE_SHAPES):
        def rd(i, li=li):
            p = pool[i][li]["layer"].packed
            wq.stream_read(p, p.numel() * 4, sink)
        ms1 = timed(torch, rd, len(pool), steps, warmup)
        pk = layer_bytes(1, K, N)[0]
        per_layer[name]["stream_read_us"] = round(ms1 * 1e3, 3)
        per_layer[name]["frac_of_stream_read"] = round(ms1 * 1e3 / per_layer[name]["us"], 4)
        floor_us += ms1 * 1e3
    torch.cuda.synchronize()
    return dict(ms=ms, packed_b=packed_b, all_b=all_b, n_launch=n_launch, copies=len(pool),
                pool_bytes=per_copy * len(pool), per_layer=per_layer, stream_read_step_us=floor_us)


def prefill_leg(wq, torch, steps, warmup, sclk_probe=False):
    M, K, N = PREFILL["M"], PREFILL["K"], PREFILL["N"]
    seed = (3, 1)
    x_np = I.with_outliers(I.activations(seed, M, K), I.outlier_channels(seed, K))
    x = torch.from_numpy(x_np).cuda()
    s = wq.awq_scales(x, 0.5)
    w = torch.from_numpy(I.weights(seed, N, K, 0.02)).cuda()
    layer = wq.QuantizedLinear.from_float(w, bits=BITS, group_size=GROUP, act_scale=s)
    del w
    per_copy = layer.packed.numel() * 4 + layer.scales.numel() * 3 + M * K * 2 * 2 + M * N * 2
    copies = max(2, -(-POOL_BYTES // per_copy))
    pool = []
    for c in range(copies):
        L = layer if c == 0 else wq.QuantizedLinear(layer.packed.clone(), layer.scales.clone(),
                                                    layer.zeros.clone(), BITS, GROUP, K, act_scale=s)
        pool.append(dict(L=L, x=x.clone(), xs=torch.empty_like(x),
                         y=torch.empty((M, N), dtype=torch.float16, device="cuda")))

    def full(i):
        p = pool[i]
        wq.scale_act(p["x"], s, out=p["xs"])
        wq.linear(p["xs"], p["L"].packed, p["L"].scales, p["L"].zeros, BITS, GROUP, out=p["y"])

    def gemm_only(i):
        p = pool[i]
        wq.linear(p["xs"], p["L"].packed, p["L"].scales, p["L"].zeros, BITS, GROUP, out=p["y"])

    def act_only(i):
        p = pool[i]
        wq.scale_act(p["x"], s, out=p["xs"])

    # Context: the vendor dense fp16 GEMM (torch.matmul -> hipBLASLt) at the
    # same M, N, K with dense fp16 weights, timed eagerly (launch gaps are
    # negligible at this size) over four distinct operand copies.
    dense = [(torch.randn(M, K, dtype=torch.float16, device="cuda"),
              torch.randn(N, K, dtype=torch.float16, device="cuda"),
              torch.empty(M, N, dtype=torch.float16, device="cuda")) for _ in range(4)]
    for i in range(8):
        a, b, c = dense[i % 4]
        torch.matmul(a, b.t(), out=c)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for i in range(steps):
        a, b, c = dense[i % 4]
        torch.matmul(a, b.t(), out=c)
    ev1.record()
    torch.cuda.synchronize()
    ms_dense = ev0.elapsed_time(ev1) / steps
    del dense

    ms_full = timed(torch, full, copies, steps, warmup)
    ms_gemm = timed(torch, gemm_only, copies, steps, warmup)
    ms_act = timed(torch, act_only, copies, steps, warmup)
    torch.cuda.synchronize()
    # shader clock under this load (the matrix-core peak assumes 2.4 GHz)
    g = capture(torch, gemm_only, copies)

    def busy():
        for _ in range(20):
            g.replay()
        torch.cuda.synchronize()

    sclk = sample_sclk(busy, 3.0) if sclk_probe else None
    return dict(ms_full=ms_full, ms_gemm=ms_gemm, ms_act=ms_act, copies=copies, ms_dense=ms_dense, sclk=sclk)


def config_cases():
    """Every (shape, M, format) case of the five synthetic workloads."""
    cases = [dict(cfg="single-gemv", K=4096, N=4096, M=1, bits=4, group=128, sigma=0.02)]
    for _, K, N in DECODE_SHAPES:
        for M in (1, 4, 16):
            cases.append(dict(cfg="llama7b-decode", K=K, N=N, M=M, bits=4, group=128, sigma=0.02))
    cases.append(dict(cfg="prefill-awq", K=4096, N=11008, M=2048, bits=4, group=128, sigma=0.02, awq=True))
    for K, N in ((8192, 28672), (28672, 8192), (8192, 10240)):
        for M in (1, 8, 32, 512):
            cases.append(dict(cfg="70b-layer", K=K, N=N, M=M, bits=4, group=128, sigma=0.015))
    for bits in (2, 3, 8):
        for group in (32, 128, -1):
            for act in ((False, True) if group != -1 else (False,)):
                for M in (1, 256):
                    cases.append(dict(cfg="gptq-variant", K=4096, N=4096, M=M, bits=bits, group=group,
                                      sigma=0.02, sym=True, act_order=act))
    return cases


def kernel_name(M, act_order, gemv_max_m):
    """Which kernel wq_linear runs for this case (a label for the record)."""
    if M == 1:
        return "gemv-stream"
    if M <= gemv_max_m and not act_order:
        return "gemv-skinny-mfma"
    if M <= 4:
        return "gemv-stream"
    return "gemm"


def configs_leg(wq, torch, launches, only=None):
    """Time wq_linear on every config case (rotating weight pools of at least
    1 GiB, graph replays, HIP events); one JSON line per case.  only: names
    of the workloads to run (all when None)."""
    rows = []
    for ci, c in enumerate(config_cases()):
        if only and c["cfg"] not in only:
            continue
        K, N, M, bits, group = c["K"], c["N"], c["M"], c["bits"], c["group"]
        seed = (7, ci)
        x = torch.from_numpy(I.activations(seed, M, K)).cuda()
        act_scale = None
        if c.get("awq"):
            xo = I.with_outliers(I.activations(seed, M, K), I.outlier_channels(seed, K))
            act_scale = wq.awq_scales(torch.from_numpy(xo).cuda(), 0.5)
            x = wq.scale_act(torch.from_numpy(xo).cuda(), act_scale)
        w = torch.from_numpy(I.weights(seed, N, K, c["sigma"])).cuda()
        g_idx = None
        if c.get("act_order"):
            g_idx = torch.from_numpy(I.act_order_gidx(seed, K, group)).cuda()
        layer = wq.QuantizedLinear.from_float(w, bits=bits, group_size=group, g_idx=g_idx,
                                              symmetric=bool(c.get("sym")), act_scale=act_scale)
        del w
        zeros = layer.zeros if not c.get("sym") else None
        G = 1 if group == -1 else K // group
        packed_b = N * K * bits // 8
        all_b = packed_b + N * G * 2 + (N * G if zeros is not None else 0) + M * K * 2 + M * N * 2 + \
            (4 * K if layer.perm is not None else 0)
        per_copy = packed_b + N * G * 3
        copies = max(2, -(-POOL_BYTES // per_copy))
        pool = [(layer.packed, layer.scales, zeros)] + [
            (layer.packed.clone(), layer.scales.clone(), None if zeros is None else zeros.clone())
            for _ in range(copies - 1)]
        y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        need = wq.workspace_size(M, N, K, bits, layer.perm is not None)
        ws = torch.empty((max(need, 1),), dtype=torch.uint8, device="cuda")

        def call(i):
            p, sc, z = pool[i]
            wq.linear(x, p, sc, z, bits, group, perm=layer.perm, out=y, workspace=ws if need else None)

        n = max(copies, launches)
        ms = timed(torch, call, copies, n, copies)
        flops = 2.0 * M * N * K
        t = ms * 1e-3
        bound = "hbm" if all_b / (HBM_PEAK_GBS * 1e9) > flops / (FP16_MFMA_PEAK_TFLOPS * 1e12) else "mfma"
        row = dict(cfg=c["cfg"], K=K, N=N, M=M, bits=bits, group=group, sym=bool(c.get("sym")),
                   act_order=bool(c.get("act_order")), awq=bool(c.get("awq")),
                   kernel=kernel_name(M, layer.perm is not None, wq.gemv_max_m()), us=round(ms * 1e3, 2),
                   packed_GBs=round(packed_b / t / 1e9, 1), all_GBs=round(all_b / t / 1e9, 1),
                   TFLOPs=round(flops / t / 1e12, 2), bound=bound,
                   frac=round(all_b / t / 1e9 / HBM_PEAK_GBS if bound == "hbm" else
                              flops / t / 1e12 / FP16_MFMA_PEAK_TFLOPS, 4),
                   pool_copies=copies)
        rows.append(row)
        print(json.dumps(row), flush=True)
        del pool, layer, x, y, ws
        torch.cuda.empty_cache()
    return rows


def silu_leg(wq, torch, steps):
    """Fused gate/up + SiLU decode projection (K = 4096, 2 x 11008 rows,
    M = 1, 4-bit, group 128): one wq_gemv_silu_mul launch against the plain
    GEMV of the stacked weight followed by torch's silu(g) * u, both over a
    rotating pool of weight copies in graph replays."""
    K, N = 4096, 22016
    w = torch.from_numpy(I.weights((2, K, N), N, K, 0.02)).cuda()
    L = wq.QuantizedLinear.from_float(w, bits=BITS, group_size=GROUP)
    del w
    x = torch.from_numpy(I.activations((2, K, N), 1, K)).cuda()
    per_copy = L.packed.numel() * 4 + L.scales.numel() * 3
    copies = max(2, -(-POOL_BYTES // per_copy))
    pool = [(L.packed, L.scales, L.zeros)] + [(L.packed.clone(), L.scales.clone(), L.zeros.clone())
                                              for _ in range(copies - 1)]
    y_full = torch.empty((1, N), dtype=torch.float16, device="cuda")
    y_half = torch.empty((1, N // 2), dtype=torch.float16, device="cuda")

    def fused(i):
        p, sc, z = pool[i]
        wq.gemv_silu_mul(x, p, sc, z, BITS, GROUP, out=y_half)

    def plain(i):
        p, sc, z = pool[i]
        wq.gemv(x, p, sc, z, BITS, GROUP, out=y_full)

    def unfused(i):
        plain(i)
        g, u = y_full[:, :N // 2], y_full[:, N // 2:]
        torch.mul(torch.nn.functional.silu(g), u, out=y_half)

    res = {}
    for name, fn in (("fused_us", fused), ("gemv_only_us", plain), ("gemv_then_torch_silu_mul_us", unfused)):
        res[name] = round(timed(torch, fn, copies, max(steps, copies), copies) * 1e3, 3)
    packed_b = N * K * BITS // 8
    res["fused_packed_GBs"] = round(packed_b / (res["fused_us"] * 1e-6) / 1e9, 1)
    return dict(leg="gate_up_silu", workload="llama7b gate+up 4096x(2x11008), M=1, 4-bit g128", **res)


def fused_leg(wq, torch, steps):
    """AWQ decode with the activation scaling and a bias fused into the GEMV
    (wq_gemv_ex) against wq_scale_act + wq_gemv + a torch bias add, on the
    4096 x 4096 projection and the 4096 x 22016 gate/up projection (M = 1,
    4-bit, group 128), over a rotating pool of weight copies in graph
    replays."""
    res = {}
    K = 4096
    x = torch.from_numpy(I.activations((5, K), 1, K)).cuda()
    s_h = wq.awq_scales(torch.from_numpy(I.activations((5, K), 64, K)).cuda(), 0.5)
    for name, N in (("o_proj_4096x4096", 4096), ("gate_up_4096x22016", 22016)):
        w = torch.from_numpy(I.weights((5, K, N), N, K, 0.02)).cuda()
        L = wq.QuantizedLinear.from_float(w, bits=BITS, group_size=GROUP)
        del w
        b = torch.from_numpy((np.random.default_rng([5, N]).standard_normal(N) * 0.1).astype(np.float16)).cuda()
        per_copy = L.packed.numel() * 4 + L.scales.numel() * 3
        copies = max(2, -(-POOL_BYTES // per_copy))
        pool = [(L.packed, L.scales, L.zeros)] + [(L.packed.clone(), L.scales.clone(), L.zeros.clone())
                                                  for _ in range(copies - 1)]
        y = torch.empty((1, N), dtype=torch.float16, device="cuda")
        xs = torch.empty_like(x)

        def fused(i):
            p, sc, z = pool[i]
            wq.gemv_ex(x, p, sc, z, BITS, GROUP, act_scale=s_h, bias=b, out=y)

        def unfused(i):
            p, sc, z = pool[i]
            wq.scale_act(x, s_h, out=xs)
            wq.gemv(xs, p, sc, z, BITS, GROUP, out=y)
            y.add_(b)

        def plain(i):
            p, sc, z = pool[i]
            wq.gemv(x, p, sc, z, BITS, GROUP, out=y)

        r = {}
        for key, fn in (("fused_us", fused), ("scale_gemv_bias_us", unfused), ("gemv_only_us", plain)):
            r[key] = round(timed(torch, fn, copies, max(steps, copies), copies) * 1e3, 3)
        res[name] = r
        del pool, L
    return dict(leg="fused_scale_bias", workload="llama7b decode projections, M=1, 4-bit g128, AWQ x/s + bias",
                **res)


def awq_leg(wq, torch, repeats, cpu):
    """AWQ's alpha search (20 grid points) on the prefill layer's calibration
    batch: M = 2048, K = 4096, N = 11008, 1% outlier channels x20, 4-bit,
    group 128.  The search synchronizes, so it is timed by the wall clock
    around whole searches.  With cpu, the oracle's search on a sample of the
    layer's output columns, timed the same way."""
    M, K, N = PREFILL["M"], PREFILL["K"], PREFILL["N"]
    seed = (3, 1)
    x_np = I.with_outliers(I.activations(seed, M, K), I.outlier_channels(seed, K))
    w_np = I.weights(seed, N, K, 0.02)
    x, w = torch.from_numpy(x_np).cuda(), torch.from_numpy(w_np).cuda()
    alphas, losses, best = wq.awq_search(x, w, BITS, GROUP)  # warm-up
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(repeats):
        alphas, losses, best = wq.awq_search(x, w, BITS, GROUP)
    gpu_s = (time.perf_counter() - t0) / repeats
    out = dict(leg="awq_search", workload="prefill-awq-w4g128 calibration: M=2048 K=4096 N=11008, 20 alphas",
               gpu_ms_per_search=round(gpu_s * 1e3, 2), gpu_ms_per_alpha=round(gpu_s * 1e3 / len(alphas), 3),
               gpu_columns_per_s=round(N / gpu_s, 1), best_alpha=round(alphas[best], 4),
               loss_best_over_rtn=round(losses[best] / losses[0], 4))
    # clipping search on the rescaled layer, 512 calibration rows, 10 ratios
    s_h = wq.awq_scales(x, alphas[best])
    w_f = wq.awq_fold(w, s_h)
    x_c = wq.scale_act(x[:512].contiguous(), s_h)
    w_c, best_c, _ = wq.awq_clip(x_c, w_f, BITS, GROUP)  # warm-up
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(repeats):
        w_c, best_c, _ = wq.awq_clip(x_c, w_f, BITS, GROUP)
    torch.cuda.synchronize()
    clip_s = (time.perf_counter() - t0) / repeats
    out["clip"] = dict(workload="clip search after the chosen alpha: M=512 K=4096 N=11008, 10 ratios",
                       gpu_ms=round(clip_s * 1e3, 3), frac_groups_clipped=round(float((best_c > 0).float().mean()), 4))
    if cpu:
        import oracle as O
        cols = 32
        t0 = time.perf_counter()
        a_o, l_o, b_o = O.awq_search(x_np, w_np[:cols], BITS, GROUP)
        cpu_s = time.perf_counter() - t0
        out["cpu_baseline"] = dict(kind="oracle", sample=f"{cols} output columns of the same layer, full M and K, "
                                                          f"20 alphas", seconds=round(cpu_s, 2),
                                   columns_per_s=round(cols / cpu_s, 2), best_alpha=round(float(a_o[b_o]), 4))
        rows = 64
        xc_np, wf_np = x_c.cpu().numpy(), w_f.cpu().numpy()
        t0 = time.perf_counter()
        O.awq_clip_search(xc_np, wf_np[:rows], BITS, GROUP)
        cpu_c = time.perf_counter() - t0
        out["clip"]["cpu_baseline"] = dict(kind="oracle", sample=f"{rows} weight rows, same M, K and ratios",
                                           seconds=round(cpu_c, 2), rows_per_s=round(rows / cpu_c, 2),
                                           gpu_rows_per_s=round(N / clip_s, 1))
    return out


def gptq_leg(wq, torch, repeats, cpu):
    """GPTQ of the prefill layer (K = 4096, N = 11008, 4-bit, group 128) on
    M = 2048 calibration tokens with correlated input channels, timed by the
    wall clock around whole calls (synchronized).  Reports the layer's output
    error relative to plain RTN's on the same tokens.  With cpu, the oracle on
    a sample of weight rows (its Hessian, inverse and Cholesky factor are
    computed in full), timed the same way."""
    M, K, N = PREFILL["M"], PREFILL["K"], PREFILL["N"]
    seed = (3, 2)
    x_np = I.correlated_activations(seed, M, K)
    w_np = I.weights(seed, N, K, 0.02)
    x, w = torch.from_numpy(x_np).cuda(), torch.from_numpy(w_np).cuda()
    codes, scales, zeros, _ = wq.gptq_quantize(w, x, BITS, GROUP)  # warm-up
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(repeats):
        codes, scales, zeros, _ = wq.gptq_quantize(w, x, BITS, GROUP)
    torch.cuda.synchronize()
    gpu_s = (time.perf_counter() - t0) / repeats

    def out_err(c, sc, z):
        # || x . (w_hat - w)^T || in fp32 (measurement only)
        g = K // GROUP
        wh = (c.float().view(N, g, GROUP) - z.float().view(N, g, 1)) * sc.float().view(N, g, 1)
        d = wh.view(N, K).half().float() - w.float()
        return float(torch.linalg.norm(x.float() @ d.t()))

    rc, rs, rz = wq.quantize_rtn(w, BITS, GROUP)
    ratio = out_err(codes, scales, zeros) / out_err(rc, rs, rz)
    out = dict(leg="gptq", workload="prefill-gptq-w4g128 calibration: M=2048 K=4096 N=11008, correlated channels",
               gpu_ms_per_layer=round(gpu_s * 1e3, 2), gpu_rows_per_s=round(N / gpu_s, 1),
               out_err_gptq_over_rtn=round(ratio, 4))
    if cpu:
        import oracle as O
        rows = 64
        t0 = time.perf_counter()
        O.gptq_quantize(w_np[:rows], x_np, BITS, GROUP)
        cpu_s = time.perf_counter() - t0
        out["cpu_baseline"] = dict(kind="oracle", sample=f"{rows} weight rows of the same layer, full M and K "
                                                          f"(Hessian, inverse and factor in full)",
                                   seconds=round(cpu_s, 2), rows_per_s=round(rows / cpu_s, 2))
    return out


# -------------------------------------------------------- CPU baseline ----

def host_info():
    """Cores the process may run on, the CPU model and the BLAS NumPy uses."""
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        cfg = np.__config__.CONFIG  # numpy >= 1.25
        b = cfg.get("Build Dependencies", {}).get("blas", {})
        blas = " ".join(str(b.get(k)) for k in ("name", "version") if b.get(k))
    except Exception:
        pass
    return dict(cores=cores, cpu_model=model, blas=blas)


def _blas_limit(cores):
    """Run the oracle's BLAS calls on `cores` threads (all the process may
    use); returns a context manager."""
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=cores)
    except Exception:  # pragma: no cover
        import contextlib
        return contextlib.nullcontext()


def cpu_baseline(target_s):
    """The CPU oracle (unpack -> dequant -> float64 product) on a bounded
    sample of output columns of each decode projection, M = 1, on every core
    the process may use."""
    import oracle as O
    info = host_info()

    def run(rows_per_layer):
        t_total, packed_total = 0.0, 0
        for name, K, N in DECODE_SHAPES:
            r = min(rows_per_layer, N)
            w = I.weights((2, K, N), r, K, 0.02)  # same distribution as the GPU layer
            q = O.quantize_linear_layer(w, BITS, GROUP)
            x = I.activations((2, K, N), 1, K)
            t0 = time.perf_counter()
            codes = O.unpack(q["packed"], BITS, K)
            w_hat = O.dequant(codes, q["scales"], q["zeros"], BITS, GROUP)
            O.linear_ref(x, w_hat)
            t_total += time.perf_counter() - t0
            packed_total += r * K * BITS // 8
        return t_total, packed_total

    with _blas_limit(info["cores"]):
        t, b = run(64)
        rows = int(64 * max(1.0, target_s / max(t, 1e-3)))
        rows = min(rows, max(N for _, _, N in DECODE_SHAPES))
        t, b = run(rows)
    return dict(value=round(b / t / 1e9, 4), unit="GB/s (packed weights, M=1)", cores=info["cores"],
                kind="oracle",
                sample=f"{rows} output columns (capped at N) of each of the 4 decode projections, M=1; "
                       f"unpack + dequant + float64 product; {t:.1f} s",
                seconds=round(t, 2), cpu_model=info["cpu_model"], blas=info["blas"])


def cpu_gemm_baseline(target_s):
    """The CPU oracle on the prefill product (M = 2048, K = 4096, 4-bit,
    group 128): unpack, dequant and the float64 product for a sample of
    output columns, reported in GFLOP/s of the sampled product."""
    import oracle as O
    info = host_info()
    M, K, N = PREFILL["M"], PREFILL["K"], PREFILL["N"]
    x = I.activations((3, 1), M, K)

    def run(cols):
        w = I.weights((3, 1), cols, K, 0.02)
        q = O.quantize_linear_layer(w, BITS, GROUP)
        t0 = time.perf_counter()
        codes = O.unpack(q["packed"], BITS, K)
        w_hat = O.dequant(codes, q["scales"], q["zeros"], BITS, GROUP)
        O.linear_ref(x, w_hat)
        return time.perf_counter() - t0

    with _blas_limit(info["cores"]):
        t = run(64)
        cols = int(64 * max(1.0, target_s / max(t, 1e-3)))
        cols = min(cols, N)
        t = run(cols)
    return dict(value=round(2.0 * M * cols * K / t / 1e9, 2), unit="GFLOP/s (M=2048 prefill product)",
                cores=info["cores"], kind="oracle",
                sample=f"{cols} of the {N} output columns, all M={M} rows and K={K}; unpack + dequant + "
                       f"float64 product; {t:.1f} s",
                seconds=round(t, 2), cpu_model=info["cpu_model"], blas=info["blas"])


def sample_sclk(busy, seconds):
    """Shader clock while `busy()` keeps the GPU loaded: amd-smi (or
    rocm-smi) is polled from a second thread.  Returns {"MHz": [...],
    "source": tool} or None when no tool answers."""
    import re
    import subprocess
    import threading
    seen, src = [], [None]

    def poll():
        t_end = time.time() + seconds
        while time.time() < t_end:
            for cmd in (["amd-smi", "metric", "--clock", "--json"], ["rocm-smi", "--showclocks", "--json"]):
                try:
                    out = subprocess.run(cmd, capture_output=True, text=True, timeout=10).stdout
                except Exception:
                    continue
                vals = []
                if cmd[0] == "amd-smi":
                    try:
                        data = json.loads(out)
                        def walk(o, path=""):
                            if isinstance(o, dict):
                                for k, v in o.items():
                                    walk(v, path + "/" + str(k).lower())
                            elif isinstance(o, list):
                                for v in o:
                                    walk(v, path)
                            elif ("gfx" in path or "sclk" in path) and path.endswith("clk") is False and \
                                    ("cur" in path or path.endswith("value")) and isinstance(o, (int, float)):
                                vals.append(float(o))
                        walk(data)
                    except Exception:
                        vals = []
                else:
                    vals = [float(v) for v in re.findall(r"sclk[^\"]*\"\s*:\s*\"\((\d+)Mhz\)", out)]
                if vals:
                    seen.append(max(vals))
                    src[0] = cmd[0]
                    break
            time.sleep(0.2)

    th = threading.Thread(target=poll)
    th.start()
    t_end = time.time() + seconds
    while time.time() < t_end:
        busy()
    th.join()
    if not seen:
        return None
    return {"MHz": sorted(seen), "source": src[0], "load": "prefill GEMM graph replays"}


# ----------------------------------------------------------------- main ----

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures a single GPU; --gpus {args.gpus} is not implemented (the layer shards across GPUs but this path runs on one)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import weight_only_int4_wq_amd as wq
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    wq.lib()
    gemm_steps = args.gemm_steps or max(10, args.steps // 5)

    if args.only == "copy":
        nbytes = 512 << 20
        src = torch.empty(nbytes // 2, dtype=torch.float16, device="cuda").normal_()
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"leg": "copy", "bytes_read_per_copy": nbytes, "bytes_written_per_copy": nbytes,
                          "copies": args.steps}), flush=True)
        return
    if args.only == "decode":
        dec = decode_leg(wq, torch, args.steps, args.warmup)
        print(json.dumps({"leg": "decode", "ms_per_step": dec["ms"], "per_layer": dec["per_layer"]}), flush=True)
        return
    if args.only == "silu":
        print(json.dumps(silu_leg(wq, torch, max(args.steps, 200))), flush=True)
        return
    if args.only == "awq":
        print(json.dumps(awq_leg(wq, torch, 3, not args.no_cpu_baseline)), flush=True)
        return
    if args.only == "fused":
        print(json.dumps(fused_leg(wq, torch, max(args.steps, 200))), flush=True)
        return
    if args.only == "gptq":
        print(json.dumps(gptq_leg(wq, torch, 3, not args.no_cpu_baseline)), flush=True)
        return
    if args.only == "configs":
        configs_leg(wq, torch, max(args.steps, 1), args.cfg.split(",") if args.cfg else None)
        return
    if args.only == "prefill":
        pre = prefill_leg(wq, torch, gemm_steps, max(5, args.warmup // 5))
        print(json.dumps({"leg": "prefill", **pre}), flush=True)
        return
    t0 = time.time()
    dec = decode_leg(wq, torch, args.steps, args.warmup)
    print(f"[bench] decode leg done in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    t0 = time.time()
    pre = prefill_leg(wq, torch, gemm_steps, max(5, args.warmup // 5), sclk_probe=True)
    print(f"[bench] prefill leg done in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    ms = dec["ms"]
    value = dec["packed_b"] / (ms * 1e-3) / 1e9
    launch_us = ms * 1e3 / dec["n_launch"]
    achieved = dec["all_b"] / dec["n_launch"] / (launch_us * 1e-6) / 1e9
    tr = traffic_from_profile(GEMV_SOURCES, "gemv_decode_step")

    M, K, N = PREFILL["M"], PREFILL["K"], PREFILL["N"]
    flops = 2.0 * M * N * K
    gemm_tflops = flops / (pre["ms_gemm"] * 1e-3) / 1e12
    step_tflops = flops / (pre["ms_full"] * 1e-3) / 1e12
    gtr = traffic_from_profile(GEMM_SOURCES, "gemm_prefill")

    cpu = cpu_gemm = None
    if not args.no_cpu_baseline:
        t0 = time.time()
        cpu = cpu_baseline(args.cpu_seconds)
        cpu_gemm = cpu_gemm_baseline(args.cpu_seconds / 2)
        print(f"[bench] cpu baselines done in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    line = {
        "metric": "W4A16 GEMV HBM GB/s (M=1) & GEMM TFLOP/s (M=2048), % of roofline",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {
            "workload": "llama7b-decode-layer-w4g128-M1: qkv 4096x12288, o_proj 4096x4096, "
                        "gate_up 4096x22016, down 11008x4096; 4-bit asymmetric RTN, group 128, fp16 x",
            "M": 1, "bits": BITS, "group_size": GROUP,
            "value_bytes": "packed 4-bit weight bytes per step (%d)" % dec["packed_b"],
            "rotating_pool_bytes": dec["pool_bytes"], "pool_copies": dec["copies"],
            "per_layer": dec["per_layer"],
        },
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": tr,
            "kernel": GEMV_KERNEL + " (every decode projection)", "avg_launch_us": round(launch_us, 3),
            "bytes_per_launch": dec["all_b"] / dec["n_launch"],
            "achievable": {
                "what": "plain streaming-read kernel (wq_stream_read) over the same packed bytes, launched and "
                        "timed the same way: the measured floor of a kernel that only reads the weights",
                "step_us": round(dec["stream_read_step_us"], 3),
                "packed_GBs": round(dec["packed_b"] / (dec["stream_read_step_us"] * 1e-6) / 1e9, 1),
                "frac_of_achievable": round(dec["stream_read_step_us"] / (ms * 1e3), 4),
            },
        },
        "gemm": {
            "workload": "prefill-awq-w4g128: M=2048 K=4096 N=11008, 1% outlier channels x20, "
                        "s=mean|x|^0.5 folded into W, x/s at input",
            "value": round(gemm_tflops, 1), "unit": "TFLOP/s",
            "step_tflops_incl_act_scaling": round(step_tflops, 1),
            "ms_gemm": round(pre["ms_gemm"], 5), "ms_scale_act": round(pre["ms_act"], 5),
            "ms_step": round(pre["ms_full"], 5), "pool_copies": pre["copies"],
            "context_dense_fp16": {
                "what": "torch.matmul fp16 (hipBLASLt) at the same M, N, K on dense fp16 weights",
                "us": round(pre["ms_dense"] * 1e3, 2),
                "tflops": round(flops / (pre["ms_dense"] * 1e-3) / 1e12, 1)},
            "roofline": {
                "bound": "mfma", "achieved": round(gemm_tflops, 1), "peak": FP16_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(gemm_tflops / FP16_MFMA_PEAK_TFLOPS, 4), "traffic": gtr,
                "kernel": GEMM_KERNEL, "avg_launch_us": round(pre["ms_gemm"] * 1e3, 3),
                "flops_per_launch": flops,
            },
            "sclk_under_load": pre.get("sclk"),
            "cpu_baseline": cpu_gemm,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
