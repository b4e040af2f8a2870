"""Build libtp.so (the HIP kernels and the C ABI) in-tree for gfx950.

Every translation unit is compiled with hipcc for --offload-arch=gfx950 only,
with packed-fp32 instruction selection disabled on the device side, then linked
into int4_quantized_gemm_amd/libtp.so.
"""

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtp.so")
SOURCES = ["api.cpp", "rotate.hip", "gemm.hip", "lora.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function",
]


def _compile(src, verbose):
    out = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC] + COMMON + lang + ["-c", os.path.join(CSRC, src), "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # The host pass does not know the device-only feature and says so; keep
    # every other diagnostic visible.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if noise not in l]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    return out


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


def build_sanitized_api(outdir, verbose=False):
    """A host-sanitized copy of the library for the CPU tests of the C ABI:
    api.cpp (host code only) built with g++ under AddressSanitizer and
    UndefinedBehaviorSanitizer, linked with the HIP objects of the last build()
    (no GPU code is built with a sanitizer). Returns the .so path; a Python
    process loads it with the sanitizer runtime preloaded."""
    objs = [os.path.join(BUILD, s + ".o") for s in SOURCES if s.endswith(".hip")]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        raise FileNotFoundError("run build() first; missing " + ", ".join(missing))
    os.makedirs(outdir, exist_ok=True)
    api_o = os.path.join(outdir, "api_sanitized.o")
    lib = os.path.join(outdir, "libtp_sanitized.so")
    san = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined"]
    steps = [
        ["g++", "-O1", "-g", "-std=c++17", "-fPIC"] + san + ["-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
                                                             "-I", os.path.join(ROOT, "include"), "-c",
                                                             os.path.join(CSRC, "api.cpp"), "-o", api_o],
        ["g++", "-shared"] + san + ["-o", lib, api_o] + objs + ["-L/opt/rocm/lib", "-lamdhip64",
                                                                "-Wl,-rpath,/opt/rocm/lib"],
    ]
    for cmd in steps:
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(" ".join(cmd[:2]) + " failed:\n" + r.stdout + r.stderr)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
