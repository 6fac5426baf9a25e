"""Lint: no floating-point atomic instruction anywhere in the library's device code.

Bitwise reproducibility rests on every floating-point sum running in a fixed
order ("Mixture-of-Kittens(MoK)란?" explainer, section 1: the same input gives
the same output); a floating-point atomic add would make the order depend on
timing. The check compiles each HIP source of the library for gfx950 to
device assembly (compile only, nothing runs) and scans every atomic
instruction: integer atomics (claim counters, status bits) are allowed,
any atomic on f16 / bf16 / f32 / f64 data fails. A planted control proves the
scan sees a float atomic when one is there."""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_layer_table_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# vector-memory and LDS atomics (global_atomic_*, buffer_atomic_*, flat_atomic_*,
# ds_add_*, ds_min_*, ...); a float type shows in the mnemonic's suffix
ATOMIC = re.compile(r"^\s*((?:global|buffer|flat)_atomic_\w+|ds_(?:add|sub|rsub|min|max|pk_add|cmpst|cmpswap|"
                    r"wrxchg|inc|dec|and|or|xor|mskor)\w*)\b", re.M)
FLOAT = re.compile(r"(_f16|_bf16|_f32|_f64|fadd|fmin|fmax)\b")


def device_asm(src: str, out: str, extra=()):
    subprocess.run([HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
                    "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), *extra, "--cuda-device-only", "-S",
                    "-x", "hip", src, "-o", out], check=True, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    return open(out).read()


def float_atomics(asm: str):
    return sorted({m for m in ATOMIC.findall(asm) if FLOAT.search(m)})


def test_scan_sees_a_planted_float_atomic(tmp_path):
    src = tmp_path / "planted.hip"
    src.write_text("#include <hip/hip_runtime.h>\n"
                   "__global__ void k(float *p, float v, int *q) { atomicAdd(p, v); atomicAdd(q, 1); }\n")
    asm = device_asm(str(src), str(tmp_path / "planted.s"))
    assert float_atomics(asm), "the planted fp32 atomic add was not recognised"
    ints = [m for m in ATOMIC.findall(asm) if not FLOAT.search(m)]
    assert ints, "the integer atomic add was not recognised"


def test_library_has_no_float_atomics(tmp_path):
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    assert "layer.hip" in srcs and "schedule.hip" in srcs

    def one(f):
        return f, device_asm(os.path.join(CSRC, f), str(tmp_path / (f + ".s")))

    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        results = list(ex.map(one, srcs))
    seen = 0
    for f, asm in results:
        seen += len(ATOMIC.findall(asm))
        assert not float_atomics(asm), f"{f}: floating-point atomics {float_atomics(asm)}"
    assert seen > 0    # the library does use integer atomics (queues, status bits): the scan reached them
