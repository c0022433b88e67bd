"""Build the HIP library of the MoE FFN layer for gfx950, in-tree.

    python -m expert_ffn_dispatch_amd.build              # libmoe_ffn.so
    python -m expert_ffn_dispatch_amd.build --sanitize   # libmoe_ffn_san.so

compiles csrc/*.hip with hipcc (one object per file, in parallel) and links
expert_ffn_dispatch_amd/libmoe_ffn.so.  Always recompiles.

--sanitize builds the same sources with the host code under AddressSanitizer
and UndefinedBehaviorSanitizer (device code as in the normal build) into
libmoe_ffn_san.so, for running the host-side argument checks of the C ABI on
the CPU.  The library leaves the sanitizer runtime unresolved: the process
that loads it preloads the ASan runtime (asan_runtime()), which also holds
the UBSan handlers, and points MOE_FFN_LIB at it.
"""
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe_ffn.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}",
]


# host code only: each sanitizer flag sits behind -Xarch_host
SAN_FLAGS = [
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g",
]
SAN_BUILD = os.path.join(ROOT, "_build_san")
SAN_LIB = os.path.join(PKG, "libmoe_ffn_san.so")


def _compile(src: str, build_dir: str, extra: list) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def _build(lib: str, build_dir: str, extra: list, link_extra: list, verbose: bool) -> str:
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, extra), srcs))
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_extra, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


def build(verbose: bool = False) -> str:
    return _build(LIB, BUILD, [], [], verbose)


def build_sanitized(verbose: bool = False) -> str:
    return _build(SAN_LIB, SAN_BUILD, SAN_FLAGS, ["-shared-libsan", *SAN_FLAGS[:4]], verbose)


def sanitized_is_current() -> bool:
    """True when libmoe_ffn_san.so is newer than every source and header."""
    if not os.path.exists(SAN_LIB):
        return False
    srcs = glob.glob(os.path.join(CSRC, "*")) + glob.glob(os.path.join(ROOT, "include", "*.h"))
    return os.path.getmtime(SAN_LIB) > max(os.path.getmtime(f) for f in srcs)


def asan_runtime() -> str:
    """Path of the compiler's shared ASan runtime, or "" if it is absent."""
    r = subprocess.run([HIPCC, "--print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
        return path
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else ""


if __name__ == "__main__":
    if "--sanitize" in sys.argv[1:]:
        build_sanitized(verbose=True)
    else:
        build(verbose=True)
    sys.exit(0)
