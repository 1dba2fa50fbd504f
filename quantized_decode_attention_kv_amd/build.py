"""Build libkvq.so (the C-ABI library) for gfx950 with hipcc, in-tree.

    python -m quantized_decode_attention_kv_amd.build

Compiles every source under csrc/ to an object with hipcc and links one shared
library next to this file.  No GPU is needed (hipcc cross-compiles).
"""

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvq.so")
ARCH = os.environ.get("KVQ_OFFLOAD_ARCH", "gfx950")

SOURCES = ["kvq_api.cpp", "kvq_stream.cpp", "kvq_pack.hip", "kvq_append.hip", "kvq_decode_generic.hip",
           "kvq_decode_mfma.hip", "kvq_decode_merge.hip",
           "kvq_probe.hip", "kvq_scratch.hip"]

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-x", "hip",
    "--offload-arch=" + ARCH,
    # packed fp32 VALU forms stay off; the compiler emits scalar fp32 instead
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the quantizer contract needs the correctly rounded fp32 divide
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # matrix-core results stay in ordinary VGPRs: the decode loop scales its
    # accumulators on the VALU, which would otherwise copy them out of AGPRs
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
]


# Per-source additions.  The pack kernels take finite inputs (NaN and infinity are
# outside the quantizer's contract): without NaNs to honour, min / max need no
# quieting of their operands, which was one VALU instruction in ten of the
# VALU-bound pack kernel.  Results for finite inputs are unchanged.
SOURCE_FLAGS = {"kvq_pack.hip": ["-fno-honor-nans"]}


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; ROCm is required to build libkvq.so")
    return exe


def build(verbose: bool = False) -> str:
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="kvq_build_") as tmp:
        objs = []
        procs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            cmd = [cc, *FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
        failed = []
        for src, p in procs:
            out, _ = p.communicate()
            text = out.decode(errors="replace")
            # the host pass does not know the packed-fp32 feature flag; that warning is expected
            lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l and l.strip()]
            if p.returncode != 0:
                failed.append((src, text))
            elif verbose and lines:
                print("\n".join(lines))
        if failed:
            raise RuntimeError("hipcc failed:\n" + "\n".join("== %s ==\n%s" % f for f in failed))
        tmp_lib = LIB + ".tmp"
        cmd = [cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp_lib]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + r.stdout.decode(errors="replace"))
        os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
