"""Build libfp8q.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import glob
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libfp8q.so")
# measurement probes for the benchmark (same memory traffic without the method's
# arithmetic); a library of their own, outside the interface of libfp8q.so
PROBE_LIB_PATH = os.path.join(PKG, "libfp8q_probe.so")
ARCH = "gfx950"

# -ffp-contract=off: every binary32 step is the one written (the kernels spell out
#   their FMAs); -fhip-fp32-correctly-rounded-divide-sqrt: '/' is the IEEE division;
# -packed-fp32-ops off: no v_pk_{add,mul,fma}_f32 in the generated code;
# -instcombine-max-copied-from-constant-users: the kernels read their argument table in
#   place only if the optimiser follows every use of it; the largest instance (mixed
#   sources with the appended update) has more uses than it follows by default (300 is
#   also too few), which leaves a 3.2 KB copy of the table on the stack.
HIP_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-instcombine-max-copied-from-constant-users=4096",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libfp8q.so)")


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _link(out: str, srcs: list[str], verbose: bool) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIP_FLAGS, "-shared", "-I", INCLUDE, "-I", CSRC, "-o", tmp, *srcs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = ("packed-fp32-ops", "--hip-link")
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if not any(n in ln for n in noise)]
    if res.returncode != 0:
        raise RuntimeError("%s build failed:\n" % os.path.basename(out) + " ".join(cmd) + "\n"
                           + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    _link(LIB_PATH, sources(), verbose)
    _link(PROBE_LIB_PATH, sorted(glob.glob(os.path.join(CSRC, "probe", "*.hip"))), verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
