"""Build libpagedattn.so in-tree with hipcc for gfx950.

Every HIP source under ``csrc/`` is compiled to an object with hipcc, every
host-only C++ source (``*.cpp``: the block manager) with the host C++
compiler, all in parallel; the objects are linked into
``paged_kv_cache_93_amd/libpagedattn.so``.  Run as a module
(``python -m paged_kv_cache_93_amd.build``) or call :func:`build`.
"""

from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libpagedattn.so")
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-Wall",
    "-Wno-unused-parameter",
    # no compiler-generated packed-FP32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


# Per-source additions.  The prefill attention kernels' arithmetic never meets
# a NaN (masked scores are set to -inf before any maximum, and V rows that may
# hold anything are zeroed), so their units are compiled without NaN
# semantics: a maximum is then one instruction, where IEEE NaN handling makes
# the compiler quiet both inputs first.  Infinities keep their meaning.
SOURCE_FLAGS = {
    "pa_prefill_bf16.hip": ["-fno-honor-nans"],
    "pa_prefill_fp8.hip": ["-fno-honor-nans"],
}


HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-Wextra",
              "-Wno-unused-parameter", f"-I{INCLUDE}", f"-I{CSRC}"]


def host_cxx() -> str:
    for name in ("g++", "c++", "clang++"):
        path = shutil.which(name)
        if path:
            return path
    raise RuntimeError("no host C++ compiler found")


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; libpagedattn needs the ROCm toolchain")
    return path


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    noise = "is not a recognized feature for this target"
    text = "\n".join(ln for ln in proc.stdout.splitlines() if noise not in ln)
    if proc.returncode != 0:
        raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(cmd)}\n{text}")
    return text


# Host-side sanitizers for the CPU test build (build(sanitize=True)).  On a
# hipcc line every -fsanitize= sits behind -Xarch_host: the device code is
# built as usual, only its host side is instrumented.
SAN_FLAGS = ["-fsanitize=address", "-fsanitize=undefined", "-fno-omit-frame-pointer",
             "-fno-sanitize-recover=undefined", "-g"]
SAN_LIB_PATH = os.path.join(BUILD_DIR, "san", "libpagedattn_san.so")


def sanitizer_runtime() -> str:
    """The clang address-sanitizer runtime (it carries the UBSan handlers too),
    to LD_PRELOAD into a process that loads the sanitized library."""
    paths = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(
        hipcc()))), "lib", "llvm", "lib", "clang", "*", "lib", "linux",
        "libclang_rt.asan-x86_64.so")))
    if not paths:
        raise RuntimeError("clang's address-sanitizer runtime was not found")
    return paths[-1]


def build(verbose: bool = False, jobs: int | None = None, defines=(), out: str | None = None,
          build_dir: str | None = None, sanitize: bool = False) -> str:
    """Compile every csrc/*.hip and csrc/*.cpp and link a shared library; returns its path.

    ``defines`` are extra ``NAME=VALUE`` preprocessor definitions (tuning
    knobs); ``out`` is the library path (default: the in-tree libpagedattn.so).
    ``sanitize`` builds the host code - the block manager, argument checks and
    launch code - with AddressSanitizer and UndefinedBehaviorSanitizer into a
    separate CPU test library (default ``_build/san/libpagedattn_san.so``), for
    processes started with ``LD_PRELOAD`` of :func:`sanitizer_runtime`; the
    device code is the same as in the product library.
    """
    if out is None:
        out = SAN_LIB_PATH if sanitize else LIB_PATH
    if build_dir is None:
        build_dir = os.path.join(BUILD_DIR, "san") if sanitize else BUILD_DIR
    os.makedirs(build_dir, exist_ok=True)
    os.makedirs(os.path.dirname(out), exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not sources:
        raise RuntimeError("no HIP sources found")
    cc = hipcc()
    flags = [*COMMON_FLAGS, *(f"-D{d}" for d in defines)]
    host_cc, host_flags = host_cxx(), HOST_FLAGS
    if sanitize:
        for f in SAN_FLAGS:
            flags += ["-Xarch_host", f]
        # the same compiler family as hipcc's host pass, so one runtime serves both
        host_cc = os.path.join(os.path.dirname(os.path.realpath(cc)), "..", "lib", "llvm", "bin",
                               "clang++")
        host_flags = [*HOST_FLAGS, *SAN_FLAGS]
    objects = [os.path.join(build_dir, os.path.basename(s) + ".o") for s in sources]
    cmds = [[cc, *flags, *SOURCE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
            for src, obj in zip(sources, objects)]
    for src in sorted(glob.glob(os.path.join(CSRC, "*.cpp"))):
        obj = os.path.join(build_dir, os.path.basename(src) + ".o")
        objects.append(obj)
        cmds.append([host_cc, *host_flags, *(f"-D{d}" for d in defines), "-c", src, "-o", obj])
    jobs = jobs or min(len(cmds), os.cpu_count() or 4, 16)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        for log in ex.map(_run, cmds):
            if verbose and log.strip():
                print(log)
    tmp = out + ".tmp"
    log = _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objects])
    if verbose and log.strip():
        print(log)
    os.replace(tmp, out)
    return out


def link_c_program(source: str, out: str, lib: str = LIB_PATH) -> str:
    """Compile a plain C99 program against include/ and link it to libpagedattn.

    This is how a C caller uses the library: the header, the HIP runtime's C
    API for memory and streams, and ``-lpagedattn`` with an rpath to the
    library's directory.  Returns ``out``.
    """
    cc = shutil.which("gcc") or shutil.which("cc")
    if not cc:
        raise RuntimeError("no C compiler found")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    lib_dir = os.path.dirname(os.path.abspath(lib))
    # relative to the program, so the pair can move together
    rel = os.path.relpath(lib_dir, os.path.dirname(os.path.abspath(out)))
    _run([cc, "-std=c99", "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
          f"-I{INCLUDE}", f"-I{rocm}/include", source, "-o", out,
          f"-L{lib_dir}", "-lpagedattn", f"-L{rocm}/lib", "-lamdhip64", "-lm",
          f"-Wl,-rpath,$ORIGIN/{rel}", f"-Wl,-rpath,{rocm}/lib"])
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
