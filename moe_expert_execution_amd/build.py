"""Build libftmoe.so (HIP for gfx950 + host C++) in the package directory.

    python -m moe_expert_execution_amd.build

Every HIP source is compiled with hipcc for gfx950 only, with packed-fp32
instruction selection disabled; host-only sources get the same compiler with
AVX-512 enabled for the host expert executor.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(HERE, "libftmoe.so")
BUILD = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_SOURCES = ["control.hip", "route.hip", "plan.hip", "gemv.hip", "gemm.hip", "combine.hip", "scratch.hip", "decode.hip"]
HOST_SOURCES = ["api.cpp", "host_exec.cpp"]
COMMON = ["-O3", "-fPIC", "-std=c++17", "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function",
          "-Wno-unused-variable"]
HIP_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-munsafe-fp-atomics"]
HOST_FLAGS = ["-I", "/opt/rocm/include", "-Wno-c++20-extensions", "-mavx512f", "-mavx512bw", "-mavx512vl", "-mavx512dq", "-mavx512bf16", "-mfma", "-pthread", "-D__HIP_PLATFORM_AMD__"]


def _obj(src):
    return os.path.join(BUILD, src.rsplit(".", 1)[0] + ".o")


def _compile(src):
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [HIPCC] + COMMON + HIP_FLAGS + ["-x", "hip", "-c", path, "-o", _obj(src)]
    else:
        cmd = [HIPCC] + COMMON + HOST_FLAGS + ["-x", "c++", "-c", path, "-o", _obj(src)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    return src, r.returncode, msgs


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = HIP_SOURCES + HOST_SOURCES
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(_compile, srcs))
    failed = False
    for src, rc, msgs in results:
        if msgs and (verbose or rc):
            print(f"[{src}]\n{msgs}", file=sys.stderr)
        failed |= rc != 0
    if failed:
        raise RuntimeError("libftmoe build failed")
    tmp = OUT + f".tmp{os.getpid()}"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + [_obj(s) for s in srcs] + ["-pthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        print(r.stdout + r.stderr, file=sys.stderr)
        raise RuntimeError("libftmoe link failed")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build())
