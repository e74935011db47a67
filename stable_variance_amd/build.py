"""Build libstable_variance.so for gfx950 with hipcc (in-tree, no JIT cache)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "sv_lib.hip")
SRCS = [SRC, os.path.join(HERE, "csrc", "sv_adn.hip"), os.path.join(HERE, "csrc", "sv_adn_folds_9_14.hip"),
        os.path.join(HERE, "csrc", "sv_adn_folds_15_21.hip"), os.path.join(HERE, "csrc", "sv_f64.hip")]
DEPS = SRCS + [os.path.join(HERE, "csrc", "sv_device.hpp"), os.path.join(HERE, "csrc", "sv_host.hpp"),
               os.path.join(HERE, "csrc", "sv_index.hpp"), os.path.join(HERE, "csrc", "sv_adn_kernel.hpp"),
               os.path.join(ROOT, "include", "stable_variance.h")]
OUT_DIR = os.path.join(HERE, "_lib")
LIB = os.path.join(OUT_DIR, "libstable_variance.so")

# -ffp-contract=off and no fast-math keep every TwoSum operation rounded on
# its own; packed FP32 instructions are disabled for the device code.
HIPCC_FLAGS = [
    "-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wextra",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    return "hipcc"


def build(verbose: bool = False) -> str:
    """Compile the HIP sources (in parallel) and link the shared object; returns its path."""
    os.makedirs(OUT_DIR, exist_ok=True)
    flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    objs, procs = [], []
    for src in SRCS:
        obj = os.path.join(OUT_DIR, os.path.splitext(os.path.basename(src))[0] + ".o")
        cmd = [hipcc(), *flags, "-c", src, "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        objs.append(obj)
    errors = []
    for cmd, pr in procs:
        out, err = pr.communicate()
        if pr.returncode != 0:
            errors.append(" ".join(cmd) + "\n" + out + err)
        elif verbose:
            print(" ".join(cmd))
    if errors:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errors))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    if verbose:
        print(" ".join(cmd))
    os.replace(tmp, LIB)
    for obj in objs:
        os.remove(obj)
    return LIB


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(d) > t for d in DEPS)


if __name__ == "__main__":
    print(build(verbose=True))
