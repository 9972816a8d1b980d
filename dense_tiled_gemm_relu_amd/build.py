"""Build the HIP libraries of the package for gfx950.

* ``libgemm_relu.so``       — the product: C-ABI gemm_relu / gemm_relu_strerror /
                              gemm_relu_plan (include/gemm_relu.h);
* ``libgemm_relu_probe.so`` — test-only lane-layout probes and the MFMA-rate
  diagnostic (MFMA-only throughput on random operands).

Objects go to ``_build/`` at the repository root; the libraries are written
next to this file, where the Python binding loads them.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

LIB = os.path.join(PKG, "libgemm_relu.so")
PROBE_LIB = os.path.join(PKG, "libgemm_relu_probe.so")

LIB_SOURCES = ["gemm_relu_api.hip", "inst_f16_nn.hip", "inst_f16_nt.hip",
               "inst_bf16_nn.hip", "inst_bf16_nt.hip", "inst_f8e4m3_nn.hip",
               "inst_f8e4m3_nt.hip", "inst_f8e5m2_nn.hip", "inst_f8e5m2_nt.hip",
               "inst_mx_e4m3.hip", "inst_mx_e5m2.hip", "inst_mx_e2m1.hip", "inst_sp.hip",
               "inst_i16.hip"]
PROBE_SOURCES = ["probe_layouts.hip", "probe_mfma_rate.hip", "probe_mfma16.hip", "probe_fp8.hip",
                 "probe_sparse.hip"]
HEADERS = ["gemm_relu_kernel.hpp", "configs.hpp", "gemm_sp_relu_kernel.hpp"]

# gfx950 only.  Packed fp32 ALU ops are switched off: the compiler otherwise
# forms v_pk_* fp32 instructions from ordinary float code.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]


# Per-source extra flags.  The sparse kernel's accumulators: by default the
# compiler splits them between VGPRs and AGPRs for v_smfmac and spills the
# copy offsets, whose reloads drain the copy pipeline every step; the VGPR
# form of the matrix instructions leaves the main loop spill-free.
EXTRA_FLAGS = {"inst_sp.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
               "inst_i16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
               "probe_mfma16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _newer(target, deps):
    if not os.path.exists(target):
        return True
    t = os.path.getmtime(target)
    return any(os.path.getmtime(d) > t for d in deps)


# GEMM_RELU_COMPARISON_CONFIGS=1 in the environment at build time also
# compiles the comparison configurations (never chosen by plan selection;
# selectable by name with GEMM_RELU_FORCE_CONFIG).  The default build leaves
# them out.
def _config_flags():
    on = os.environ.get("GEMM_RELU_COMPARISON_CONFIGS", "") not in ("", "0")
    return ["-DGEMM_RELU_COMPARISON_CONFIGS"] if on else []


def _compile(src, force, verbose):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    deps = [os.path.join(CSRC, src)] + [os.path.join(CSRC, h) for h in HEADERS] + \
        [os.path.join(INCLUDE, "gemm_relu.h")]
    if force or _newer(obj, deps):
        cmd = [HIPCC] + HIP_FLAGS + _config_flags() + EXTRA_FLAGS.get(src, []) + \
            ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr[-4000:]))
    return obj


def _link(objs, out, verbose):
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build(force=True, verbose=False, jobs=None):
    """Compile and link both libraries.  force=False skips up-to-date objects."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 1)
    srcs = LIB_SOURCES + PROBE_SOURCES
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, force, verbose), srcs)))
    _link([objs[s] for s in LIB_SOURCES], LIB, verbose)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB, verbose)
    return LIB, PROBE_LIB


if __name__ == "__main__":
    print(build(force="--force" in sys.argv, verbose=True))
