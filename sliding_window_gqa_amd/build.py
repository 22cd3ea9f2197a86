"""Build step: compile the HIP sources into ``libwa.so`` for gfx950, in the package folder.

    python -m sliding_window_gqa_amd.build

Always recompiles. Packed fp32 VALU instructions are disabled for the device code
(``-packed-fp32-ops``); the host pass warns that it does not know that feature. MFMA
accumulators are kept in VGPRs (``-amdgpu-mfma-vgpr-form``): with the compiler's default
AGPR form the d = 256 prompt kernel copied its 128 output accumulators between AGPRs and
VGPRs on every key tile, for the rarely taken rescale of O.
"""

import concurrent.futures
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libwa.so")
# Compilation units: (source, preprocessor defines). The kernel templates are instantiated by
# compiling one file once per variant the launchers call, so that they compile in parallel.
UNITS = [("decode.hip", ()), ("prompt.hip", ()), ("prepare.hip", ()), ("wa_abi.hip", ()),
         *[("decode_inst.hip", (f"WA_INST_D={d}", f"WA_INST_G={g}", "WA_INST_WHOLE=0"))
           for d in (128, 256) for g in (1, 2, 4, 8, 16)],
         *[("decode_inst.hip", ("WA_INST_D=256", f"WA_INST_G={g}", "WA_INST_WHOLE=1")) for g in (1, 2)],
         *[("prompt_inst.hip", (f"WA_INST_D={d}", f"WA_INST_NP={p}", f"WA_INST_POST={int(p == 1)}"))
           for d in (128, 256) for p in (1, 2, 3)]]
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


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed with status {r.returncode}: {' '.join(cmd)}")


def build(out=LIB, extra=(), verbose=False):
    """Compile every source to an object in parallel (each carries its own device code),
    then link the shared library; ``extra`` adds compiler flags (e.g. -D defines)."""
    tmp = out + ".tmp"
    with tempfile.TemporaryDirectory(prefix="wa_build_") as objdir:
        objs, cmds = [], []
        for i, (src, defs) in enumerate(UNITS):
            o = os.path.join(objdir, f"{i:02d}_{os.path.splitext(src)[0]}.o")
            objs.append(o)
            cmds.append([hipcc(), *compile_flags(extra), *[f"-D{d}" for d in defs], "-c", "-o", o,
                         os.path.join(CSRC, src)])
        workers = min(len(cmds), max(1, os.cpu_count() or 1))
        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
            for f in [ex.submit(_run, c, verbose) for c in cmds]:
                f.result()
        _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    # a kernel whose host stub the host pass dropped leaves an undefined symbol that only
    # fails at load time: refuse such a library here
    nm = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    # (and a launcher declared in one file but defined nowhere, e.g. a variant left out of UNITS)
    missing = [l.split()[-1] for l in nm.stdout.splitlines()
               if "__device_stub__" in l or "_ZN2wa" in l]
    if nm.returncode != 0 or missing:
        os.remove(tmp)
        raise RuntimeError("undefined library symbols: " + ", ".join(missing or [nm.stderr]))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
