"""Build libattn_fwd.so (the gfx950 HIP kernels and the C ABI) in-tree.

The library holds the forward (csrc/attn_fwd.hip), the backward
(csrc/attn_bwd.hip), the general-layout forward (csrc/attn_general.hip) and
the row softmax (csrc/softmax.hip); csrc/mfma_pipe.h is shared by the
backward and the general forward.

    python -m io_aware_attention_flash_amd.build

hipcc cross-compiles for gfx950 on a machine without a GPU. Packed-fp32
instructions are disabled for all device code. The kernels' per-step loops
are fully unrolled (their register arrays are indexed by compile-time step
numbers); the unroll budget is raised so they stay so, and the build fails
if any kernel ends up using scratch memory.
"""
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", n)
        for n in ("attn_fwd.hip", "attn_bwd.hip", "attn_general.hip", "softmax.hip")]
LIB = os.path.join(PKG, "libattn_fwd.so")
INCLUDE = os.path.join(ROOT, "include")
ARCH = os.environ.get("ATTN_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-shared", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-pragma-unroll-threshold=65536",
    "-Rpass-analysis=kernel-resource-usage",
    "-Wall", "-Wno-unused-function",
]


def scratch_users(remarks):
    """Kernels whose resource-usage remarks report scratch (private) memory."""
    bad, name = [], None
    for line in remarks.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name and int(m.group(1)) > 0:
            bad.append((name, int(m.group(1))))
    return bad


def build(verbose=False, extra=()):
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc] + HIPCC_FLAGS + list(extra) + ["-I", INCLUDE] + SRCS + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building %s" % LIB)
    bad = scratch_users(res.stderr)
    if bad:
        os.remove(tmp)
        raise RuntimeError("kernels use scratch memory (a step loop was not unrolled or "
                           "registers spilled): %s" % ", ".join("%s (%d B/lane)" % b for b in bad))
    os.replace(tmp, LIB)
    return LIB


def is_stale():
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    srcs = SRCS + [os.path.join(INCLUDE, "attn.h"), os.path.join(PKG, "csrc", "mfma_pipe.h")]
    return any(os.path.getmtime(s) > t for s in srcs)


if __name__ == "__main__":
    print(build(verbose=True))
