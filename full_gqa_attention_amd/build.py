"""Build libmuse_attn.so for gfx950 in-tree with hipcc.

Every HIP source is compiled with packed-f32 instruction generation switched
off (``-Xclang -target-feature -Xclang -packed-fp32-ops``) and without fast
math: RoPE needs the accurate sin/cos.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "libmuse_attn.so")
SOURCES = ["muse_attn.cpp", "prep.hip", "prefill.hip", "decode.hip", "relocate.hip", "verify.hip",
           "outproj.hip"]
ARCH = "gfx950"
# The prefill kernels keep their Q.K and P.V accumulators in VGPRs: the scores
# feed the VALU softmax directly, and the AGPRs serve as spill space.
EXTRA_FLAGS = {"prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
# hipBLASLt computes the o_proj GEMM for more than a few tokens
LINK_LIBS = ["-lhipblaslt"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def common_flags():
    return ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def build(verbose: bool = False) -> str:
    """Compile every source (in parallel) and link the shared library."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmd = [hipcc()] + common_flags() + EXTRA_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass warns that it does not know the packed-fp32 feature
        text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append(src)
            sys.stderr.write(text + "\n")
        elif verbose and text.strip():
            print(text)
    if failed:
        raise RuntimeError(f"hipcc failed on {failed}")
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, *LINK_LIBS, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


SAN_LIB_PATH = os.path.join(PKG, "libmuse_attn_san.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def build_sanitized() -> str:
    """libmuse_attn_san.so: the host code (argument checks, workspace layout,
    launch set-up) built with AddressSanitizer and UndefinedBehaviorSanitizer,
    linked with the kernels of the regular build (GPU code is not
    instrumented).  A process that loads it must preload clang's ASan runtime
    (``asan_runtime()``)."""
    if not all(os.path.exists(os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")) for src in SOURCES):
        build()
    san_dir = os.path.join(BUILD_DIR, "san")
    os.makedirs(san_dir, exist_ok=True)
    host_obj = os.path.join(san_dir, "muse_attn.o")
    cmd = [hipcc()] + common_flags() + SAN_FLAGS + ["-c", os.path.join(CSRC, "muse_attn.cpp"), "-o", host_obj]
    out = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if out.returncode != 0:
        sys.stderr.write(out.stdout.decode(errors="replace"))
        raise RuntimeError("hipcc failed on the sanitized muse_attn.cpp")
    objs = [host_obj] + [os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o") for src in SOURCES
                         if src != "muse_attn.cpp"]
    tmp = SAN_LIB_PATH + ".tmp"
    subprocess.run([hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-fsanitize=address,undefined",
                    "-shared-libasan", *objs, *LINK_LIBS, "-o", tmp], check=True)
    os.replace(tmp, SAN_LIB_PATH)
    return SAN_LIB_PATH


TIMELINE_LIB_PATH = os.path.join(PKG, "libmuse_attn_timeline.so")


def build_timeline() -> str:
    """libmuse_attn_timeline.so: the regular library with decode.hip built
    with MUSE_DECODE_TIMELINE, whose decode kernels record per-workgroup
    phase times (include/muse_attn_timeline.h).  For profiling only."""
    if not all(os.path.exists(os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")) for src in SOURCES):
        build()
    tl_dir = os.path.join(BUILD_DIR, "timeline")
    os.makedirs(tl_dir, exist_ok=True)
    obj = os.path.join(tl_dir, "decode.o")
    cmd = [hipcc()] + common_flags() + ["-DMUSE_DECODE_TIMELINE", "-c", os.path.join(CSRC, "decode.hip"), "-o", obj]
    out = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if out.returncode != 0:
        sys.stderr.write(out.stdout.decode(errors="replace"))
        raise RuntimeError("hipcc failed on the timeline decode.hip")
    objs = [obj] + [os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o") for src in SOURCES
                    if src != "decode.hip"]
    tmp = TIMELINE_LIB_PATH + ".tmp"
    subprocess.run([hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, *LINK_LIBS, "-o", tmp], check=True)
    os.replace(tmp, TIMELINE_LIB_PATH)
    return TIMELINE_LIB_PATH


def asan_runtime() -> str:
    """clang's shared ASan runtime (it carries the UBSan handlers too)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    out = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], stdout=subprocess.PIPE, check=True)
    path = out.stdout.decode().strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("clang's shared ASan runtime was not found")
    return path


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_sanitized())
    elif "--timeline" in sys.argv:
        print(build_timeline())
    else:
        print(build(verbose="-v" in sys.argv))
