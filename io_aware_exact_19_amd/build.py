"""Build libfa.so (the C-ABI attention library) for gfx950 with hipcc, in-tree.

Usage: ``python -m io_aware_exact_19_amd.build`` (or ``build_library()``).
The library lands next to this file so that it travels with the source tree.
"""

from __future__ import annotations

import os
import re
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfa.so")
SOURCES = ["fa_api.cpp", "fa_prefill.hip", "fa_decode.hip", "fa_backward.hip",
           "fa_backward_dq.hip", "fa_fp8.hip"]
ARCH = "gfx950"
# flags for one source only: the dQ kernel's working set fits in the
# architectural VGPRs, and with its matrix results there the score
# accumulators reach the softmax without a copy out of the accumulation
# registers (the dK, dV kernel's does not fit, so it keeps the default)
SOURCE_FLAGS = {"fa_backward_dq.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # keep the compiler from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


_MFMA8 = re.compile(r"v_mfma_scale_f32_32x32x64_f8f6f4 v\[(\d+):(\d+)\], v\[(\d+):(\d+)\], "
                    r"v\[(\d+):(\d+)\]")


def check_fp8_operand_overlap(extra_flags=None, csrc=CSRC) -> int:
    """Compile the fp8 kernels to assembly and fail if the result registers of
    any fp8 matrix instruction overlap its operand registers: this compiler
    allows such an allocation when the accumulator input is not tied to the
    result, and the instruction then reads back garbage.  Returns the number
    of instructions checked."""
    src = os.path.join(csrc, "fa_fp8.hip")
    with tempfile.TemporaryDirectory() as tmp:
        out = os.path.join(tmp, "fa_fp8.s")
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "--cuda-device-only", "-S",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *(extra_flags or []),
               "-o", out, src]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"hipcc -S failed with exit code {res.returncode}")
        n = 0
        for line in open(out):
            m = _MFMA8.search(line)
            if not m:
                continue
            n += 1
            d0, d1, a0, a1, b0, b1 = (int(x) for x in m.groups())
            if not (d1 < a0 or a1 < d0) or not (d1 < b0 or b1 < d0):
                raise RuntimeError(f"fp8 matrix instruction with overlapping registers: {line.strip()}")
    if n == 0:
        raise RuntimeError("no fp8 matrix instruction found in fa_fp8.hip's assembly")
    return n


def build_library(verbose: bool = False, extra_flags=None, csrc=CSRC, out=LIB) -> str:
    """Compile every HIP source (each with its own flags, in parallel) and
    link them into ``out`` (libfa.so beside this file); returns its path."""
    from concurrent.futures import ThreadPoolExecutor

    with tempfile.TemporaryDirectory() as tmp:
        def compile_one(name):
            obj = os.path.join(tmp, name + ".o")
            cmd = [hipcc(), *HIPCC_FLAGS, *SOURCE_FLAGS.get(name, []), *(extra_flags or []),
                   "-c", "-o", obj, os.path.join(csrc, name)]
            return cmd, obj, subprocess.run(cmd, capture_output=True, text=True)

        with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as pool:
            results = list(pool.map(compile_one, SOURCES))
        for cmd, _, res in results:
            if verbose:
                print(" ".join(cmd), flush=True)
            if res.returncode != 0:
                sys.stderr.write(res.stdout + res.stderr)
                raise RuntimeError(f"hipcc failed with exit code {res.returncode}: {cmd[-1]}")
        tmp_lib = out + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-fPIC", "-shared", "-o", tmp_lib,
               *(obj for _, obj, _ in results)]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"hipcc link failed with exit code {res.returncode}")
    n = check_fp8_operand_overlap(extra_flags, csrc)
    if verbose:
        print(f"fp8 matrix instructions checked for register overlap: {n}", flush=True)
    os.replace(tmp_lib, out)
    return out


if __name__ == "__main__":
    print(build_library(verbose=True))
