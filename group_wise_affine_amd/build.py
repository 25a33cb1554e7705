"""Build libqmm.so (HIP, gfx950) in-tree with hipcc.

Sources are compiled to objects in parallel under _build/ and linked into
group_wise_affine_amd/libqmm.so. Flags:
  --offload-arch=gfx950                  CDNA4 only
  -fhip-fp32-correctly-rounded-divide-sqrt  IEEE division (the quantizer's
                                         codes depend on it)
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                         no packed fp32 VALU instructions
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libqmm.so")
CEILING_LIB = os.path.join(HERE, "libqmm_ceiling.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.cpp", "quantize.hip", "qmv.hip", "qmn.hip", "qmn_tile.hip", "fpq.hip", "apk.hip", "qmv_mfma_f16.hip", "qmv_mfma_bf16.hip", "qmm.hip",
           "tile_gemm_f16.hip", "tile_gemm_bf16.hip", "tile_conv_f16.hip", "tile_conv_bf16.hip",
           "tile_fp.hip", "tile_apk.hip"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-warning-option",
    "-I" + os.path.join(ROOT, "include"),
]


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stderr}")
    # the host pass warns about the device-only target feature; drop that noise
    msgs = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l
            and "not a recognized feature" not in l]
    return obj, "\n".join(msgs)


def build(verbose=False, jobs=None):
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = []
    for obj, msg in results:
        objs.append(obj)
        if verbose and msg.strip():
            print(msg)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, LIB)
    build_ceiling()
    return LIB


def build_ceiling():
    """libqmm_ceiling.so: the benchmark's single-launch floor kernels
    (csrc/ceiling.hip, include/qmm_ceiling.h), separate from libqmm."""
    tmp = CEILING_LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-shared", os.path.join(CSRC, "ceiling.hip"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for ceiling.hip:\n{' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, CEILING_LIB)
    return CEILING_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
