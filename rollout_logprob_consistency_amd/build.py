"""Build liblp.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m rollout_logprob_consistency_amd.build [--verbose]

Compiles every .hip file under csrc/ into one shared library next to this
file, with hipcc for gfx950. Packed-fp32 instructions are disabled for all
device code. The device assembly of score.hip is then checked for wait-state
hazards around its inline-assembly MFMAs (isa_check.py); a violation fails
the build. The comparison kernel's assembly is checked for ds_bpermute (its
reductions use DPP, ds_swizzle and readlane). Both files' buffer -> LDS copies
(inline assembly) are checked for VALU writes of their SGPR operands fewer than
5 wait states before them.
"""

from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "liblp.so")
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"),
              shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build liblp)")


def compile_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        f"-I{INCLUDE}", f"-I{CSRC}",
    ]


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compile csrc/*.hip into liblp.so; returns the library path."""
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources under " + CSRC)
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.basename(s) + ".o") for s in srcs]

    def compile_one(src_obj):
        s, o = src_obj
        cmd = [hipcc(), *compile_flags(), *(extra or []), "-c", s, "-o", o]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {s}:\n{r.stdout}\n{r.stderr}")
        if verbose and (r.stdout or r.stderr):
            print(r.stdout + r.stderr, flush=True)

    # The translation units and the two assembly checks are independent:
    # run them side by side (hipcc is single-threaded per file).
    jobs = max(1, min(8, os.cpu_count() or 1))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        futs = [ex.submit(compile_one, so) for so in zip(srcs, objs)]
        futs.append(ex.submit(check_score_isa, objdir, extra, verbose))
        futs.append(ex.submit(check_compare_isa, objdir, extra, verbose))
        for f in futs:
            f.result()
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def check_score_isa(objdir: str, extra: list[str] | None = None, verbose: bool = False) -> None:
    """Compile score.hip to device assembly with the same flags and run the
    inline-assembly MFMA hazard check on it."""
    from rollout_logprob_consistency_amd import isa_check
    src = os.path.join(CSRC, "score.hip")
    out = os.path.join(objdir, "score.device.s")
    cmd = [hipcc(), *compile_flags(), *(extra or []), "--cuda-device-only", "-S", src, "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{r.stdout}\n{r.stderr}")
    text = open(out).read()
    problems = isa_check.check_asm(text)
    if problems:
        raise RuntimeError("inline-assembly MFMA hazard check failed:\n" + "\n".join(problems[:20]))
    problems = isa_check.check_lds_dma_sgpr(text)
    if problems:
        raise RuntimeError("buffer -> LDS copy SGPR hazard check failed:\n" + "\n".join(problems[:20]))


def check_compare_isa(objdir: str, extra: list[str] | None = None, verbose: bool = False) -> None:
    """Compile compare.hip to device assembly and check that the comparison
    kernel's reductions use no ds_bpermute (DPP, ds_swizzle and readlane only)."""
    from rollout_logprob_consistency_amd import isa_check
    src = os.path.join(CSRC, "compare.hip")
    out = os.path.join(objdir, "compare.device.s")
    cmd = [hipcc(), *compile_flags(), *(extra or []), "--cuda-device-only", "-S", src, "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{r.stdout}\n{r.stderr}")
    text = open(out).read()
    problems = isa_check.check_no_bpermute(text, "compare_kernel")
    if problems:
        raise RuntimeError("compare_kernel cross-lane check failed:\n" + "\n".join(problems))
    problems = isa_check.check_lds_dma_sgpr(text, "compare_kernel")
    if problems:
        raise RuntimeError("buffer -> LDS copy SGPR hazard check failed:\n" + "\n".join(problems[:20]))


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
