"""Build ``lib/libq4w.so`` from ``csrc/`` with hipcc for gfx950.

Run ``python -m bit_quantized_weight_amd.build`` (or ``__graft_entry__.build()``).
Always recompiles.  Flags: no fast-math; fp32 division and sqrt correctly
rounded and fp32 denormals kept (the quantizers must be bit-exact); packed
fp32 instructions disabled in device code.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "lib")
OUT = os.path.join(OUT_DIR, "libq4w.so")

SOURCES = ["q4w_api.cpp", "q4_pack.hip", "q4_gemv.hip", "q4_gemv_mfma.hip", "q4_gemv_mfma4.hip", "a8w4.hip",
           "q4_attn.hip", "stream_read.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

DEVICE_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fno-fast-math",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]

# Per-source extra flags.  The matrix-core skinny kernel consumes every MFMA
# result in VALU right away; the VGPR form of MFMA avoids copying each result
# out of the accumulation registers (4 extra VALU ops per MFMA).
EXTRA_FLAGS = {
    "q4_gemv_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose=True, jobs=8):
    """Compile every source to an object in parallel, then link the shared library."""
    os.makedirs(OUT_DIR, exist_ok=True)
    objdir = os.path.join(OUT_DIR, "_obj")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [HIPCC, *DEVICE_FLAGS, *EXTRA_FLAGS.get(src, []), *inc, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    errors = []
    for cmd, p in procs:
        out, _ = p.communicate()
        out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            errors.append(f"{' '.join(cmd)}\n{out}")
        elif verbose and out.strip():
            print(out)
    if errors:
        raise RuntimeError("hipcc failed:\n" + "\n\n".join(errors))
    tmp = OUT + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
