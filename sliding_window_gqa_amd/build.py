"""Build step: compile the HIP sources into ``libwa.so`` for gfx950, in the package folder,
and the control builds ``libwa_control<k>.so`` used by the GPU control tests: the same
library with one planted mistake each (``-DWA_CONTROL=k``, the list in csrc/wa_common.h),
which recompile only the units the mistake touches and share every other object.

    python -m sliding_window_gqa_amd.build [--no-controls]

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


def _decode_unit(src, defs):
    return src in ("decode.hip", "decode_inst.hip")


def _decode_merge_unit(src, defs):
    return src == "decode.hip" or (src == "decode_inst.hip" and "WA_INST_WHOLE=1" in defs)


def _prompt_unit(src, defs):
    return src == "prompt_inst.hip"


# control k -> the units its planted mistake touches (recompiled with -DWA_CONTROL=k)
CONTROLS = {1: _decode_unit, 2: _prompt_unit, 3: _decode_merge_unit, 4: _decode_merge_unit,
            5: _prompt_unit, 6: _prompt_unit}


def control_lib(k):
    return os.path.join(HERE, f"libwa_control{k}.so")


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


def _link(out, objs, verbose):
    tmp = out + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    # a kernel whose host stub the host pass dropped leaves an undefined symbol that only
    # fails at load time: refuse such a library here
    # (and a launcher declared in one file but defined nowhere, e.g. a variant left out of UNITS)
    nm = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [l.split()[-1] for l in nm.stdout.splitlines()
               if "__device_stub__" in l or "_ZN2wa" in l]
    if nm.returncode != 0 or missing:
        os.remove(tmp)
        raise RuntimeError("undefined library symbols: " + ", ".join(missing or [nm.stderr]))
    os.replace(tmp, out)


def build(out=LIB, extra=(), verbose=False, controls=True):
    """Compile every unit to an object in parallel (each carries its own device code), link
    the library; with ``controls`` also the control builds. ``extra`` adds compiler flags."""
    with tempfile.TemporaryDirectory(prefix="wa_build_") as objdir:
        jobs = []          # (object, command)
        product = []
        for i, (src, defs) in enumerate(UNITS):
            o = os.path.join(objdir, f"{i:02d}_{os.path.splitext(src)[0]}.o")
            product.append(o)
            jobs.append((o, [hipcc(), *compile_flags(extra), *[f"-D{d}" for d in defs], "-c", "-o", o,
                             os.path.join(CSRC, src)]))
        variants = {}
        if controls:
            for k, touches in CONTROLS.items():
                objs = []
                for i, (src, defs) in enumerate(UNITS):
                    if touches(src, defs):
                        o = os.path.join(objdir, f"c{k}_{i:02d}_{os.path.splitext(src)[0]}.o")
                        jobs.append((o, [hipcc(), *compile_flags(extra), *[f"-D{d}" for d in defs],
                                         f"-DWA_CONTROL={k}", "-c", "-o", o, os.path.join(CSRC, src)]))
                        objs.append(o)
                    else:
                        objs.append(product[i])
                variants[k] = objs
        workers = min(len(jobs), max(1, os.cpu_count() or 1))
        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
            for f in [ex.submit(_run, cmd, verbose) for _, cmd in jobs]:
                f.result()
        _link(out, product, verbose)
        for k, objs in variants.items():
            _link(control_lib(k), objs, verbose)
    return out


if __name__ == "__main__":
    print(build(verbose=True, controls="--no-controls" not in sys.argv))
