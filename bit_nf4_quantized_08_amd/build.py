"""Build libqlora_nf4.so in-tree with hipcc for gfx950.

Run ``python -m bit_nf4_quantized_08_amd.build`` (or call :func:`build`).  Each
translation unit is compiled to an object under ``_build/`` in parallel, then
linked into ``bit_nf4_quantized_08_amd/libqlora_nf4.so``.
"""

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libqlora_nf4.so")
BUILD = os.path.join(ROOT, "_build")
SOURCES = ["api.cpp", "codebook.cpp", "trace.cpp", "device.cpp", "k_codec.hip", "k_linear.hip", "k_qgemm.hip", "k_lowrank.hip", "k_merge.hip", "k_adamw8.hip"]
ARCH = "gfx950"

# Packed fp32 instructions are kept out of all device code.
HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


# Host-side sanitizer build of the C-ABI layer (argument checking, the codebook,
# the trace log, the device cache): those translation units are compiled with
# AddressSanitizer and UndefinedBehaviorSanitizer on the host side only (device
# code is never instrumented), then linked with the ordinary kernel objects.
# The library loads only into a process that preloads the clang ASan runtime
# (sanitizer_runtime()); the CPU ABI tests run against it in a child process.
HOST_SOURCES = ["api.cpp", "codebook.cpp", "trace.cpp", "device.cpp"]
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_OUT = os.path.join(BUILD, "asan", "libqlora_nf4_asan.so")


def sanitizer_runtime():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    r = subprocess.run([os.path.join(rocm, "llvm", "bin", "clang"), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isfile(path) else None


def build_sanitized(verbose=False):
    d = os.path.dirname(SAN_OUT)
    os.makedirs(d, exist_ok=True)

    def host_obj(src):
        obj = os.path.join(d, src + ".o")
        cmd = [hipcc(), *HIPCC_FLAGS, "-O1", "-g", *SAN_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        return obj

    kernels = [s for s in SOURCES if s not in HOST_SOURCES]
    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        hobjs = list(ex.map(host_obj, HOST_SOURCES))
        kobjs = [os.path.join(BUILD, s + ".o") for s in kernels]
        missing = [s for s, o in zip(kernels, kobjs) if not os.path.isfile(o)]
        list(ex.map(_compile, missing))
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *SAN_FLAGS, "-shared-libsan", *hobjs, *kobjs,
           "-o", SAN_OUT]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("sanitized link failed:\n" + r.stderr)
    if verbose:
        print("built", SAN_OUT)
    return SAN_OUT


if __name__ == "__main__":
    build(verbose=True)
