"""Builds ``libfp4w.so`` (the gfx950 HIP kernels behind the C ABI of
``include/fp4w.h``) in place, with hipcc.

Every call compiles from source.  Flags: gfx950 only, -O3, packed-fp32 VALU
instructions disabled (they are not used by this library), IEEE-conformant
single-precision division (hipcc's default) and no fast-math.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfp4w.so")
# measurement references for the benchmark (plain streaming read, clock probe); not the path
MEMBENCH_LIB = os.path.join(HERE, "libfp4w_membench.so")
SOURCES = ["api.hip", "quantize.hip", "dequantize.hip", "merge.hip", "linear.hip", "decode.hip", "decode_xs.hip", "grouped.hip", "gemm.hip", "a4w4.hip", "backward.hip", "lora_grad.hip", "delta_grad.hip", "aqn.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the fp4w library needs the ROCm toolchain")


def flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", "-I", os.path.join(HERE, "..", "include")]


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the same
# library (device code unchanged), for the CPU test run of the host validation;
# each sanitizer flag applies to the host compilation only.
SAN_LIB = os.path.join(HERE, "libfp4w_san.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-g"]


def build(verbose: bool = False, jobs: int = 6, sanitize: bool = False) -> str:
    cc = hipcc()
    objdir = os.path.join(HERE, "_build_san" if sanitize else "_build")
    os.makedirs(objdir, exist_ok=True)
    extra = SAN_FLAGS if sanitize else []
    out_lib = SAN_LIB if sanitize else LIB

    def compile_one(src):
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [cc, *flags(), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops" not in l and "ignoring feature" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{out}")
        if out.strip() and verbose:
            print(out)
        return obj

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = out_lib + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *(["-shared-libsan", *extra] if sanitize else []),
           "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out_lib)
    if sanitize:
        return out_lib
    obj = compile_one("membench.hip")
    tmp = MEMBENCH_LIB + ".tmp"
    subprocess.run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, obj], check=True)
    os.replace(tmp, MEMBENCH_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
