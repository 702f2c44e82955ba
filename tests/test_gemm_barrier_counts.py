"""Static check of the GEMM kernels' copy barriers (no GPU needed).

The GEMM kernels keep activation copies (global -> LDS by DMA) and weight
loads in flight across stages and end a stage with `s_waitcnt vmcnt(N)` +
`s_barrier`, where N counts the loads issued after the ones the next stage
needs.  That count is only right if every stage really issues those loads:
register loads whose results are never read are dropped by the compiler,
and a barrier that still counts them lets the next stage read an activation
tile whose copy has not landed.  This test compiles the GEMM sources for
gfx950 and checks, in the generated code of every GEMM kernel, that each
barrier's wait count N is 0 or at most the number of vector-memory loads
issued since the previous barrier (in code order, which is program order
for these kernels: straight-line stages inside one unrolled loop).
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "weight_only_int4_wq_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")


def _assembly(src, tmp_path):
    out = tmp_path / (os.path.basename(src) + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", f"-I{os.path.join(ROOT, 'include')}", "--cuda-device-only", "-S", src, "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text()


def _barrier_counts(asm, kernel_pattern):
    """{kernel symbol: [(loads possibly in flight at the barrier, loads issued
    since the previous barrier)]}, walking the code in order: every load adds
    one to the in-flight bound, every s_waitcnt vmcnt(N) caps it at N."""
    out = {}
    for name in re.findall(r"^(_ZN\S*" + kernel_pattern + r"\S*):", asm, re.M):
        body = asm.split(name + ":", 1)[1].split(".Lfunc_end", 1)[0]
        lines = [l.split(";")[0].strip() for l in body.splitlines()]
        inflight, since, rows = 0, 0, []
        for l in lines:
            if re.match(r"(global_load|buffer_load)", l):
                inflight += 1
                since += 1
                continue
            m = re.match(r"s_waitcnt\s.*vmcnt\((\d+)\)", l)
            if m:
                inflight = min(inflight, int(m.group(1)))
            elif l.startswith("s_barrier"):
                rows.append((inflight, since))
                since = 0
        out[name] = rows
    return out


@pytest.mark.parametrize("src,pattern", [("wq_gemm_large.hip", "17gemm_large_kernel"), ("wq_gemm.hip", "11gemm_kernel")])
def test_copy_barriers_wait_for_loads_actually_issued(src, pattern, tmp_path):
    asm = _assembly(os.path.join(CSRC, src), tmp_path)
    counts = _barrier_counts(asm, pattern)
    assert counts, f"no {pattern} instantiations found"
    # loads still in flight at a barrier must all have been issued after the
    # previous barrier (the copies the next stage reads were issued before it)
    bad = {k: v for k, v in counts.items() if any(n > loads for n, loads in v)}
    assert not bad, "barrier passes with earlier loads in flight:\n" + "\n".join(f"{k}: {v}" for k, v in bad.items())
    assert all(len(v) >= 2 for v in counts.values())
