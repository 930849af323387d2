"""Build libnq.so (gfx950) in-tree with hipcc.

Each kernel family compiles as its own translation unit (in parallel), then
everything links into one shared library exporting the C ABI of
include/nq.h.  Flags that matter for exactness:

* ``-ffp-contract=off``: no fused multiply-add; every page operation is its
  own binary32 rounding;
* fp32 / fp16 denormals stay enabled (HIP's default; the kernel descriptors
  carry denorm mode 3);
* ``-fhip-fp32-correctly-rounded-divide-sqrt``: the "nvfp4" quotient is a
  correctly rounded division;
* ``-Xclang -target-feature -Xclang -packed-fp32-ops`` is passed as given (the
  build never emits packed-fp32 VALU instructions).

The matrix-core product units (k_gemm_*.hip) also take
``-mllvm -amdgpu-mfma-vgpr-form=1``: MFMA results land in VGPRs, so the
binary32 scaling reads them without an AGPR copy per value.
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libnq.so")
ARCH = os.environ.get("NQ_OFFLOAD_ARCH", "gfx950")

KERNEL_SOURCES = ["k_simple.hip", "k_kquant.hip", "k_iq.hip", "k_fp4.hip", "k_ternary.hip", "k_fp8row.hip",
                  "k_gqenc.hip", "k_q8_1.hip", "k_gemv_simple.hip", "k_gemv_kquant.hip", "k_gemv_iq.hip",
                  "k_gemv_fp4t.hip", "k_gemm_simple.hip", "k_gemm_kquant.hip", "k_gemm_iq.hip",
                  "k_gemm_fp4t.hip", "k_many_simple.hip", "k_many_kquant.hip", "k_many_iq.hip", "k_many_fp4.hip",
                  "k_many_ternary.hip", "k_measure.hip"]
HOST_SOURCES = ["nq_abi.cpp", "nq_noalloc.hip"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wno-unused-function"]
DEVICE = [f"--offload-arch={ARCH}", "-fhip-fp32-correctly-rounded-divide-sqrt",
          "-fno-gpu-flush-denormals-to-zero",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.exists(c) or c == "hipcc":
            return c
    raise RuntimeError("hipcc not found")


MFMA_UNITS = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer for the host
# sources (the C ABI's validators and launchers); device code is built as
# always.  Used by tests/run_sanitized.py for libnq_san.so.
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _compile(src, is_kernel, build_dir=BUILD, defines=(), sanitize=False):
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    extra = MFMA_UNITS if src.startswith("k_gemm_") else []
    if sanitize and src in HOST_SOURCES:
        extra = extra + SAN_HOST
    cmd = [_hipcc(), *COMMON, *DEVICE, *extra, *[f"-D{d}" for d in defines], "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs=None, verbose=False, out=LIB, defines=(), sanitize=False):
    """Compile every source and link the library (default: libnq.so in-tree).

    `defines` are extra -D macros (the tuning knobs NQ_UPT, NQ_RESIDENT_PER_CU,
    NQ_NT_STORE, NQ_NTL of csrc/nq_kernel.h, NQ_F8_NB of csrc/nq_fp8row.h and
    NQ_GM_REWRITE_M of csrc/nq_gemm.h);
    a non-default `out` builds elsewhere; `sanitize` builds the host sources
    with AddressSanitizer and UndefinedBehaviorSanitizer.
    """
    build_dir = BUILD if out == LIB else out + ".build"
    os.makedirs(build_dir, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 4)
    work = [(s, True, build_dir, tuple(defines), sanitize) for s in KERNEL_SOURCES + HOST_SOURCES]
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda a: _compile(*a), work))
    tmp = out + ".tmp"
    # (sanitized objects resolve their runtime against the one the test run preloads)
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}", file=sys.stderr)
    return out


if __name__ == "__main__":
    build(verbose=True)
