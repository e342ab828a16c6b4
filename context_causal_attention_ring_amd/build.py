"""Build libringattn.so in-tree with hipcc for gfx950.

Usage: python -m context_causal_attention_ring_amd.build [-v]
"""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libringattn.so")
# The same library with a wait and a barrier around every tile of the fused
# kernel: race-free by construction, so a test can require the product
# library to match it bit for bit.
SYNC_LIB = os.path.join(PKG, "libringattn_sync.so")
SOURCES = ["ringattn_api.hip", "ring_attn_fused.hip", "kv_cache_write.hip",
           "merge_attn_states.hip"]
ARCH = os.environ.get("RINGATTN_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 math stays off: the compiler must not emit v_pk_*_f32
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; libringattn needs ROCm's hipcc to build")


def _compile(out, extra, verbose):
    tmp = out + f".tmp{os.getpid()}"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-o", tmp] + [os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l)
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


def build(verbose=False):
    """Compile every source into libringattn.so and the checking build
    libringattn_sync.so (always recompiles)."""
    _compile(SYNC_LIB, ["-DRA_SYNC_EVERY_TILE"], verbose)
    return _compile(LIB, [], verbose)


def assemble(source="ring_attn_fused.hip", out=None, extra=()):
    """Device assembly of one source (for reading register use and spills)."""
    out = out or os.path.join(PKG, os.path.splitext(source)[0] + ".s")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "--cuda-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument", *extra, "-o", out, os.path.join(CSRC, source)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
