"""Build libkda.so (the C-ABI HIP library) in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libkda.so")
SOURCES = ["kda_api.hip", "kda_prefill.hip", "kda_prefill_f32.hip", "kda_decode.hip", "kda_layer.hip"]

# The packed-fp32 feature is disabled for all device code: the compiler must not
# form packed fp32 add/mul/fma instructions from ordinary float code.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Werror",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(out: str = LIB, verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), then link the library."""
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(CSRC, src.replace(".hip", ".o"))
        cmd = [hipcc(), *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd, stderr=subprocess.PIPE, text=True), src))
        objs.append(obj)
    errors = []
    for p, src in procs:
        _, err = p.communicate()
        # hipcc's host pass does not know the packed-fp32 feature and says so.
        err = "\n".join(l for l in err.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            errors.append("%s:\n%s" % (src, err))
        elif err.strip() and verbose:
            print(err)
    if errors:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errors))
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                   check=True)
    os.replace(tmp, out)
    for obj in objs:
        os.remove(obj)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
