"""Build libpmx.so (HIP for gfx950) in-tree with hipcc.

    python -m preconditioned_optimizer_matrix_amd.build

Compiles every csrc/*.hip translation unit to an object in parallel and links
the shared library next to this file.  Packed fp32 vector instructions are
disabled for all device code (-packed-fp32-ops).
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpmx.so")
ARCH = "gfx950"

COMMON = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(os.path.dirname(HERE), "include"),
]


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc()] + COMMON + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, errs))
    return obj, errs


def build(verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(_compile, srcs))
    objs = []
    for obj, errs in results:
        objs.append(obj)
        if verbose and errs.strip():
            print(errs, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


# Host sanitizers for the C++ runtime: the translation units that carry the
# host logic (argument checks, workspace carving, alias checks, descriptor
# tables) are rebuilt with AddressSanitizer and UndefinedBehaviorSanitizer on
# their host pass only (-Xarch_host before every -fsanitize=; the GPU code is
# compiled as usual) and linked with the other objects into libpmx_san.so.
# Load it with the clang ASan runtime preloaded (asan_runtime()).
SAN_LIB = os.path.join(HERE, "libpmx_san.so")
SAN_SOURCES = ("pmx_api.hip", "pmx_shampoo.hip")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def asan_runtime():
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("clang ASan runtime not found")
    return hits[-1]


def build_sanitized(verbose=True):
    san = os.path.join(BUILD, "san")
    os.makedirs(san, exist_ok=True)
    objs = []
    for src in sources():
        base = os.path.basename(src)
        if base in SAN_SOURCES:
            obj = os.path.join(san, base + ".o")
            cmd = [hipcc()] + COMMON + SAN_FLAGS + ["-c", src, "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr))
        else:
            obj = os.path.join(BUILD, base + ".o")
            if not os.path.exists(obj):
                obj, _ = _compile(src)
        objs.append(obj)
    tmp = SAN_LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-Xarch_host",
           "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libsan",
           "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, SAN_LIB)
    if verbose:
        print("built", SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "--sanitize":
        build_sanitized()
    else:
        build()
