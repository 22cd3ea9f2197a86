"""Build step: compile the HIP sources into ``libwa.so`` for gfx950, in the package folder.

    python -m sliding_window_gqa_amd.build

Always recompiles. Packed fp32 VALU instructions are disabled for the device code
(``-packed-fp32-ops``); the host pass warns that it does not know that feature. MFMA
accumulators are kept in VGPRs (``-amdgpu-mfma-vgpr-form``): with the compiler's default
AGPR form the d = 256 prompt kernel copied its 128 output accumulators between AGPRs and
VGPRs on every key tile, for the rarely taken rescale of O.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libwa.so")
SOURCES = ["decode.hip", "prompt.hip", "prepare.hip", "wa_abi.hip"]
ARCH = "gfx950"


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def compile_flags(extra=()):
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        "-Wno-unused-command-line-argument",
        *extra,
    ]


def build(out=LIB, extra=(), verbose=False):
    tmp = out + ".tmp"
    cmd = [hipcc(), *compile_flags(extra), "-shared", "-o", tmp,
           *[os.path.join(CSRC, s) for s in SOURCES]]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed with status {r.returncode}")
    # a kernel whose host stub the host pass dropped leaves an undefined symbol that only
    # fails at load time: refuse such a library here
    nm = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [l.split()[-1] for l in nm.stdout.splitlines() if "__device_stub__" in l]
    if nm.returncode != 0 or missing:
        os.remove(tmp)
        raise RuntimeError("kernel stubs missing from the host code: " + ", ".join(missing or [nm.stderr]))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
