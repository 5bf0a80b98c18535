"""Build the HIP library in-tree: libpaged_prefill.so next to this file.

hipcc cross-compiles for gfx950 without a GPU.  Packed fp32 instructions are
disabled for the device code (they are emitted by the compiler on its own
from plain float code otherwise).

MFMA instructions are selected in their VGPR form (accumulator and result in
the unified register file, moved to AGPRs only where the register allocator
wants): in the default AGPR form every score tile the softmax reads is
copied out of AGPRs, and the allocator parks output accumulators in VGPRs
around the score tiles, some 60-130 extra moves per key tile.  Each head
dimension has its own translation unit so the choice can differ per head
dimension; PPA_MFMA_VGPR_FORM=0 selects the AGPR form for comparison.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpaged_prefill.so")
BUILD_DIR = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# device sources and their MFMA register form
KERNEL_SOURCES = (
    ("attention.hip", "0"),
    # head dims 64/128 with two query blocks per wave: only the AGPR form fits
    ("attention_d64_d128.hip", os.environ.get("PPA_MFMA_VGPR_FORM_D128", "0")),
    ("attention_d64_d128_qb1.hip", os.environ.get("PPA_MFMA_VGPR_FORM", "1")),
    ("attention_d256.hip", os.environ.get("PPA_MFMA_VGPR_FORM", "1")),
    # the VGPR form's AGPR-rewrite pass crashes the compiler on these
    ("attention_d256_small_pages.hip", "0"),
    # 8-bit pages: the widening step needs registers the VGPR form does not
    # leave at head dimension 256 (it spills there); the AGPR form does not spill
    ("attention_q8_d64_d128.hip", os.environ.get("PPA_MFMA_VGPR_FORM_Q8", "0")),
    ("attention_q8_d256.hip", os.environ.get("PPA_MFMA_VGPR_FORM_Q8", "0")),
    # the narrow (decode) kernel
    ("decode.hip", os.environ.get("PPA_MFMA_VGPR_FORM_DEC", "1")),
    ("decode16.hip", os.environ.get("PPA_MFMA_VGPR_FORM_DEC", "1")),
    ("kv_append.hip", "0"),
    ("noalloc.hip", "0"),
)
HOST_SOURCES = ("api.cpp", "plan.cpp")
COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"build step failed ({res.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose=False, resource_usage=False, jobs=None):
    """Compile every translation unit (in parallel, `jobs` at a time; default
    MAX_JOBS or the CPU count, at most 16) and link the library."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    extra = ["-Rpass-analysis=kernel-resource-usage"] if resource_usage else []
    steps = []
    for src, vgpr_form in KERNEL_SOURCES:
        kern_obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        steps.append(([HIPCC, f"--offload-arch={ARCH}", *COMMON, *DEVICE_FLAGS, "-mllvm",
                       "-amdgpu-mfma-vgpr-form=" + vgpr_form, f"-DPPA_MFMA_AGPR_FORM={1 - int(vgpr_form)}",
                       *extra, "-c", os.path.join(CSRC, src), "-o", kern_obj],
                      kern_obj))
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".cpp", ".o"))
        steps.append(([HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj], obj))
    if jobs is None:
        jobs = int(os.environ.get("MAX_JOBS", "0") or 0) or (os.cpu_count() or 1)
    jobs = max(1, min(16, jobs))
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        futures = [pool.submit(_run, cmd, verbose or resource_usage) for cmd, _ in steps]
        for f in futures:
            f.result()
    objs = [obj for _, obj in steps]
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, resource_usage="--usage" in sys.argv)
