"""Build the HIP library libbgtq.so in-tree for gfx950.

Steps: compile and run the codebook table generator (host C++), then compile the kernels and the
host C ABI with hipcc and link one shared library next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libbgtq.so")
ARCH = os.environ.get("BGTQ_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument"]
KERNEL_UNITS = ["bgtq_kernels.hip", "bgtq_decode_gtq.hip", "bgtq_quant_rows.hip", "bgtq_logquant.hip",
                "bgtq_noalloc.hip"]
HOST_UNITS = ["bgtq_host.cpp"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    gen_dir = os.path.join(CSRC, "generated")
    os.makedirs(gen_dir, exist_ok=True)
    gen_exe = os.path.join(BUILD, "gen_codebook")
    _run(["g++", "-O2", "-std=c++17", "-o", gen_exe, os.path.join(CSRC, "gen_codebook.cpp")])
    _run([gen_exe, os.path.join(gen_dir, "bgtq_codebook_data.h")])
    objs, jobs = [], []
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        for u in KERNEL_UNITS + HOST_UNITS:
            obj = os.path.join(BUILD, u + ".o")
            objs.append(obj)
            lang = [] if u.endswith(".hip") else ["-x", "hip"]
            jobs.append(ex.submit(_run, [HIPCC, *COMMON, *lang, "-c", os.path.join(CSRC, u), "-o", obj]))
        for j in jobs:
            out = j.result()
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


MOCK = os.path.join(BUILD, "libbgtq_mock.so")
MOCK_SAN = os.path.join(BUILD, "libbgtq_mock_san.so")


def build_mock(sanitize: bool = False) -> str:
    """Host C ABI linked against mock launchers (test-only; checks kernel arguments without a GPU).
    sanitize: a separate copy built with AddressSanitizer and UndefinedBehaviorSanitizer (host code
    only; load it in a process that preloads the ASan runtime)."""
    os.makedirs(BUILD, exist_ok=True)
    gen_dir = os.path.join(CSRC, "generated")
    os.makedirs(gen_dir, exist_ok=True)
    gen_exe = os.path.join(BUILD, "gen_codebook")
    _run(["g++", "-O2", "-std=c++17", "-o", gen_exe, os.path.join(CSRC, "gen_codebook.cpp")])
    _run([gen_exe, os.path.join(gen_dir, "bgtq_codebook_data.h")])
    flags = ["-O1", "-std=c++17", "-fPIC", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include"]
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]
    out = MOCK_SAN if sanitize else MOCK
    tag = "mock_san_" if sanitize else "mock_"
    objs = []
    for u in ("bgtq_host.cpp", "mock_launch.cpp"):
        obj = os.path.join(BUILD, tag + u + ".o")
        _run(["g++", *flags, *(san if sanitize else []), "-c", os.path.join(CSRC, u), "-o", obj])
        objs.append(obj)
    tmp = out + ".tmp"
    _run(["g++", "-shared", *(san if sanitize else []), "-o", tmp, *objs, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib"])
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
