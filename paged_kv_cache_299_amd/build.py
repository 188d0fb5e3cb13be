"""Build libpa.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: python -m paged_kv_cache_299_amd.build   (always recompiles)
"""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpa.so")
SOURCES = ["pa_api.hip", "pa_decode.hip", "pa_prefill.hip", "pa_cascade.hip", "pa_cache.hip",
           "pa_vkv.hip", "pa_debug.hip"]
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # no packed-fp32 VALU forms (v_pk_add/mul/fma_f32) in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpa)")


def build(verbose: bool = False, extra_flags=(), out: str = LIB) -> str:
    """Compile every source into one shared library at `out` (always recompiles)."""
    tmp = out + ".tmp"
    cmd = [hipcc(), *FLAGS, *extra_flags, "-o", tmp, *[os.path.join(CSRC, s) for s in SOURCES]]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(ln for ln in res.stderr.splitlines() if noise not in ln and ln.strip())
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err:
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
