"""Build libfade.so in-tree with hipcc for gfx950.

Each kernel translation unit is compiled to an object under _build/ and the
objects are linked into tiered_quantized_kv_amd/libfade.so. Always compiles
(no staleness check): callers that want the existing library simply load it.
"""
import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfade.so")
SOURCES = ["k_quant.hip", "k_decode.hip", "k_h2o.hip", "k_evict.hip", "k_pq.hip", "k_pq_tier.hip", "fade_api.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # never emit packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE division and square root in fp32 (the quantizer's exact quotient)
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
    "-I", os.path.join(ROOT, "include"),
]


# Per-source flags. The H2O prefill kernels take their MFMA results into
# VGPRs: the fp32 score tiles feed VALU exp / sum work at once, and the
# accumulator-to-VGPR copy per score is then not needed.
EXTRA = {"k_h2o.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    return obj, err


def build(verbose=False, jobs=4):
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in results]
    if verbose:
        for _, e in results:
            if e.strip():
                print(e, file=sys.stderr)
    tmp = LIB + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
