"""Builds libattn.so (the HIP library behind include/attn.h) in-tree for gfx950.

Every source under csrc/ is compiled with hipcc into _build/ and linked into
forward_backward_amd/libattn.so. Run ``python -m forward_backward_amd.build``;
``--debug`` builds libattn_debug.so instead (the same sources with -DATTN_DEBUG,
objects in _build_debug/): every global load and global->LDS copy of its
kernels checks its address against the call's buffers (attn_debug_take).
"""

from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libattn.so")
BUILD_DEBUG = os.path.join(HERE, "_build_debug")
LIB_DEBUG = os.path.join(HERE, "libattn_debug.so")
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # Keep the compiler from forming packed fp32 ops (v_pk_*_f32).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]

# Per-source options. The dQ kernels and the head_dim 32-128 forward are
# scheduled with LLVM's max-ILP strategy: dQ 2.7% faster at B4 H8 d128 T8192
# (1.453 -> 1.414 ms, ten rounds each) with the same registers; the forward 1%
# at head_dim 128 and 4% at 64, with one 8-byte spill outside its loop. The
# other sources keep the default: there it measured the same or slower (the
# head_dim 256 forward 7%), or made kernels spill or lose occupancy.
# The head_dim 32/64 dK/dV kernel keeps its MFMA results in ordinary vector
# registers (LLVM's choice was accumulation registers, read back with 32
# v_accvgpr_read per step for the softmax): 13% faster at 32 and 9% at 64, same
# occupancy. On the head_dim 256 kernels the same option measured 18% slower.
# The decode kernels too: the split kernel at C5 45.3 -> 44.8 us per call.
# The persistent head_dim 128 dK/dV kernel is scheduled with the iterative
# max-occupancy strategy: under the default and max-ILP strategies its step
# loops waited for each LDS read before the product that uses it (18 and 15
# full LDS drains per S-wave step against 11), and the kernel ran 3-5% slower
# than with one workgroup per item; with it, 0.9% faster than that at B4 H8
# d128 T8192, 2% causal, 7.5% with a 1024-key window, 15% with KV lengths.
PER_FILE = {
    "attn_dq.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
    "attn_dkdv_queue.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-maxocc"],
    "attn_fwd.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
    "attn_dkdv_small.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "attn_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, extra, build_dir: str = BUILD) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON, *PER_FILE.get(os.path.basename(src), []), *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{out}")
    return obj


def build(verbose: bool = False, extra=(), debug: bool = False) -> str:
    build_dir, lib = (BUILD_DEBUG, LIB_DEBUG) if debug else (BUILD, LIB)
    extra = [*extra, "-DATTN_DEBUG"] if debug else list(extra)
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, build_dir), srcs))
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    args = sys.argv[1:]
    build(verbose=True, extra=[a for a in args if a != "--debug"], debug="--debug" in args)
