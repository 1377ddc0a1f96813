"""Build libmhc.so (the gfx950 HIP library) in-tree with hipcc."""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmhc.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # packed fp32 VALU instructions stay off in every kernel of this library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
OBJ_DIR = os.path.join(ROOT, "_build", "obj")
# hipcc's host pass warns once per source that it does not know the packed-fp32
# feature; that line is expected.  Anything else is shown.
_NOISE = "'-packed-fp32-ops' is not a recognized feature"


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if ln.strip() and _NOISE not in ln]
    return r.returncode, msgs


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every csrc/*.hip to an object (in parallel), then link libmhc.so."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(OBJ_DIR, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]
    srcs = sources()
    objs = [os.path.join(OBJ_DIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    cmds = [[hipcc, *HIPCC_FLAGS, *inc, "-c", "-o", o, s] for s, o in zip(srcs, objs)]
    jobs = jobs or min(len(cmds), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_run, cmds))
    msgs = [m for _, ms in results for m in ms]
    if any(rc != 0 for rc, _ in results):
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs[:60]))
    tmp = LIB + ".tmp"
    rc, lmsgs = _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    if rc != 0:
        raise RuntimeError("hipcc link failed:\n" + "\n".join(lmsgs[:60]))
    if verbose and (msgs or lmsgs):
        print("\n".join(msgs + lmsgs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
