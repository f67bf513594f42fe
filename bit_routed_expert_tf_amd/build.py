"""Build ``libtf.so`` (the gfx950 HIP kernels and the C ABI) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libtf.so")
BUILD = os.path.join(HERE, "_build")
SOURCES = ["tf_api.cpp", "tf_decode.hip", "tf_slot.hip", "tf_grouped.hip", "tf_prefill.hip", "tf_sample.hip", "tf_attn.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 ops are switched off for every device pass.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


# Host code instrumented by AddressSanitizer and UndefinedBehaviorSanitizer
# (each flag for the host pass only; the device code is built as usual).  The
# sanitizer runtime is not linked: the process that loads such a build
# preloads clang's shared ASan runtime, which also carries UBSan's handlers.
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def _compile(src, build_dir=None, extra=()):
    obj = os.path.join(build_dir or BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, f"--offload-arch={ARCH}", *COMMON, *DEVICE_FLAGS, *extra, "-c",
           os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose=False):
    """Compile every source for gfx950 and link ``libtf.so`` (always rebuilds)."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with ThreadPoolExecutor(len(srcs)) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


def build_host_sanitized(out_dir):
    """The same library with ASan/UBSan-instrumented host code, as
    out_dir/libtf_san.so (rebuilt when a source is newer)."""
    os.makedirs(out_dir, exist_ok=True)
    out = os.path.join(out_dir, "libtf_san.so")
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    deps = [os.path.join(CSRC, f) for f in os.listdir(CSRC)] + [os.path.join(ROOT, "include", "tf.h")]
    if os.path.exists(out) and os.path.getmtime(out) > max(os.path.getmtime(p) for p in deps):
        return out
    with ThreadPoolExecutor(len(srcs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, out_dir, HOST_SANITIZE), srcs))
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    return out


if __name__ == "__main__":
    build(verbose=True)
