"""Build libbkv.so (HIP, gfx950) in-tree with hipcc.

All device code is compiled with floating-point contraction off (the RoPE
rotation and FPS arithmetic follow a fixed operation order) and without
packed-fp32 instruction selection.  Each source compiles to its own object
(in parallel), then the objects link into the shared library.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbkv.so")
OBJ = os.path.join(HERE, "_build")
SOURCES = ["bkv_api.hip", "bkv_fps.hip", "bkv_score.hip", "bkv_select.hip", "bkv_compact.hip", "bkv_stream.hip",
           "bkv_evict.hip", "bkv_prefill.hip", "bkv_sources.hip", "bkv_attention.hip"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd: list, verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature; that warning is expected
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l]
    if msgs and (verbose or r.returncode):
        print("\n".join(msgs), file=sys.stderr)
    if r.returncode:
        raise RuntimeError("hipcc failed: " + " ".join(cmd[-3:]))


def device_flags(arch: str = "gfx950") -> list:
    """The compile flags every source is built with (besides the include paths)."""
    return [f"--offload-arch={arch}", "-O3", "-std=c++17", "-fPIC",
            "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall"]


def build(verbose: bool = False, arch: str = "gfx950") -> str:
    os.makedirs(OBJ, exist_ok=True)
    flags = device_flags(arch) + ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = [os.path.join(OBJ, s.replace(".hip", ".o")) for s in SOURCES]
    jobs = max(1, min(len(SOURCES), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda so: _run([hipcc()] + flags + ["-c", os.path.join(CSRC, so[0]), "-o", so[1]], verbose),
                    zip(SOURCES, objs)))
    _run([hipcc(), f"--offload-arch={arch}", "-shared", "-fPIC", "-o", LIB + ".tmp"] + objs, verbose)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
