"""Build libfairy.so for gfx950 (in-tree).

    python -m bit_complex_weight_amd.build

Each HIP source is compiled by hipcc into _build/ (in parallel), then linked
into bit_complex_weight_amd/libfairy.so.  Packed-fp32 VALU instructions are
disabled for all device code.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfairy.so")
SOURCES = ["fairy_api.hip", "fairy_quant.hip", "fairy_gemv.hip", "fairy_gemv_bf16.hip",
           "fairy_gemv_f32.hip", "fairy_gemv_i8.hip", "fairy_gemm.hip", "fairy_gemm_mfma.hip", "fairy_gemm_valu.hip",
           "fairy_layer.hip", "fairy_attention.hip", "fairy_gemv_lut.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-flush-denormals-to-zero", "-ffp-contract=off",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


# Per-source code-generation options.  The attention kernel runs softmax
# arithmetic on its MFMA results every key chunk; with the accumulators in
# ordinary VGPRs (the MFMA "VGPR form") no accumulator-register moves are
# needed around that arithmetic.
SOURCE_FLAGS = {
    "fairy_attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
