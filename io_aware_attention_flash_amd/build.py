"""Build libattn_fwd.so (the gfx950 HIP kernels and the C ABI) in-tree.

The library holds the forward (csrc/attn_fwd.hip), the backward
(csrc/attn_bwd.hip), the general-layout forward (csrc/attn_general.hip) and
the row softmax (csrc/softmax.hip); csrc/mfma_pipe.h is shared by the
backward and the general forward.

    python -m io_aware_attention_flash_amd.build

hipcc cross-compiles for gfx950 on a machine without a GPU. Each source is
compiled to an object in its own process (in parallel), then the objects are
linked into the shared library. Packed-fp32 instructions are disabled for all
device code. The kernels' per-step loops are fully unrolled (their register
arrays are indexed by compile-time step numbers); the unroll budget is raised
so they stay so, and the build fails if any kernel ends up using scratch
memory.

Next to the library, ``libattn_fwd.so.digest`` records a digest of the
sources, the header and the flags it was built from; ``is_stale()`` compares
it with the current sources, so a library copied along with a changed source
tree is rebuilt rather than used (file times are not trusted: copies of the
tree may not keep them).
"""
import concurrent.futures
import hashlib
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", n)
        for n in ("attn_fwd.hip", "attn_bwd.hip", "attn_general.hip", "softmax.hip")]
HEADERS = [os.path.join(ROOT, "include", "attn.h"), os.path.join(PKG, "csrc", "mfma_pipe.h")]
LIB = os.path.join(PKG, "libattn_fwd.so")
DIGEST = LIB + ".digest"
INCLUDE = os.path.join(ROOT, "include")
ARCH = os.environ.get("ATTN_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-pragma-unroll-threshold=65536",
    "-Rpass-analysis=kernel-resource-usage",
    "-Wall", "-Wno-unused-function",
]


def hipcc_path():
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


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


def source_digest(extra=()):
    """sha256 over the sources, headers and compiler flags of a build."""
    h = hashlib.sha256()
    for path in SRCS + HEADERS:
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    h.update(" ".join(HIPCC_FLAGS + list(extra)).encode())
    return h.hexdigest()


def compile_objects(out_dir, extra=(), verbose=False, jobs=4):
    """Compile every source to out_dir/<name>.o in parallel. Raises on a
    compiler error or when a kernel uses scratch memory."""
    os.makedirs(out_dir, exist_ok=True)

    def one(src):
        obj = os.path.join(out_dir, os.path.basename(src) + ".o")
        cmd = [hipcc_path()] + HIPCC_FLAGS + list(extra) + ["-I", INCLUDE, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        return src, obj, res

    objs = []
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        for src, obj, res in ex.map(one, SRCS):
            if res.returncode != 0:
                sys.stderr.write(res.stdout + res.stderr)
                raise RuntimeError("hipcc failed on %s" % src)
            bad = scratch_users(res.stderr)
            if bad:
                raise RuntimeError("%s: kernels use scratch memory (a step loop was not unrolled "
                                   "or registers spilled): %s" % (
                                       os.path.basename(src),
                                       ", ".join("%s (%d B/lane)" % b for b in bad)))
            objs.append(obj)
    return objs


def link(objs, out):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc_path(), "--offload-arch=" + ARCH, "-shared", "-fPIC"] + objs + ["-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("linking %s failed" % out)
    os.replace(tmp, out)
    return out


def build(verbose=False, extra=(), out=LIB, jobs=4):
    """Compile and link the library (always; see ensure_built for the
    build-if-stale form). `extra` holds additional compiler flags such as
    -D overrides of the compile-time configuration."""
    obj_dir = os.path.join(ROOT, "build", "obj_%s_%d" % (
        hashlib.sha256(("%s|%s" % (out, " ".join(extra))).encode()).hexdigest()[:8], os.getpid()))
    try:
        objs = compile_objects(obj_dir, extra, verbose, jobs)
        link(objs, out)
    finally:
        shutil.rmtree(obj_dir, ignore_errors=True)
    if out == LIB:
        with open(DIGEST, "w") as f:
            f.write(source_digest(extra) + "\n")
    return out


def is_stale():
    """True when the library is missing or was built from other sources or
    flags than the current ones."""
    if not os.path.exists(LIB) or not os.path.exists(DIGEST):
        return True
    with open(DIGEST) as f:
        return f.read().strip() != source_digest()


def ensure_built(verbose=False):
    """Build the library when it is missing or stale; return its path. When
    ATTN_LIB_PATH names another build (a sweep variant), that one must exist
    and nothing is built."""
    other = os.environ.get("ATTN_LIB_PATH")
    if other:
        if not os.path.exists(other):
            raise RuntimeError("ATTN_LIB_PATH=%s does not exist" % other)
        return other
    if is_stale():
        build(verbose=verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
