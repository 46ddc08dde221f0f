"""Builds libfa.so (the C-ABI library) in-tree with hipcc for gfx950.

Usage:  python -m exact_attention_41_amd.build [-v]
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libfa.so")
SOURCES = ["fa_api.hip", "fa_fwd.hip", "fa_fwd256.hip", "fa_fwd_fp8.hip", "fa_bwd.hip",
           "fa_decode.hip", "fa_clock.hip"]
# Per-source flags. The backward kernels and the d = 256 forward keep their
# accumulators in AGPRs through inline assembly; every other matrix product
# there should write VGPRs, where the VALU reads its results, rather than the
# compiler's AGPR form for kernels that own a whole SIMD. Their per-tile
# software pipeline is one fully unrolled loop, larger than the default size
# limit for an unroll pragma.
_ONE_WAVE_PER_SIMD = ["-mllvm", "-amdgpu-mfma-vgpr-form=1",
                      "-mllvm", "-pragma-unroll-threshold=100000"]
SOURCE_FLAGS = {"fa_bwd.hip": _ONE_WAVE_PER_SIMD, "fa_fwd256.hip": _ONE_WAVE_PER_SIMD}
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libfa.so")


def compile_flags(extra=()):
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # No packed-fp32 VALU instructions in device code.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC, *extra,
    ]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = (res.stdout or "") + (res.stderr or "")
    # The host pass does not know the device-only feature; that warning is noise.
    lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l]
    if res.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines), flush=True)
    return "\n".join(lines)


def build(verbose: bool = False, extra_flags=(), out_path: str = LIB_PATH) -> str:
    """Compile every source for gfx950 and link libfa.so; returns its path."""
    cc = hipcc()
    tmp = tempfile.mkdtemp(prefix="fa_build_")
    try:
        objs = []
        cmds = []
        for src in SOURCES:
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            objs.append(obj)
            flags = compile_flags([*SOURCE_FLAGS.get(src, []), *extra_flags])
            cmds.append([cc, *flags, "-c", os.path.join(CSRC, src), "-o", obj])
        with cf.ThreadPoolExecutor(max_workers=len(cmds)) as ex:
            list(ex.map(lambda c: _run(c, verbose), cmds))
        tmp_out = out_path + ".tmp"
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_out, *objs], verbose)
        os.replace(tmp_out, out_path)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return out_path


def resource_report(src: str = "fa_fwd.hip") -> str:
    """Per-kernel register/LDS/scratch report of one source (device pass only)."""
    cc = hipcc()
    with tempfile.TemporaryDirectory() as tmp:
        cmd = [cc, *compile_flags([*SOURCE_FLAGS.get(src, []), "-Rpass-analysis=kernel-resource-usage"]),
               "--cuda-device-only", "-c", os.path.join(CSRC, src), "-o", os.path.join(tmp, "x.o")]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(res.stderr)
        return res.stderr


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
