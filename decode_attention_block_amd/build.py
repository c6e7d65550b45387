"""Builds libkvq.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Flags that matter for the results:
  * -fhip-fp32-correctly-rounded-divide-sqrt, no fast-math: x / s in the quantizer is
    the correctly rounded binary32 quotient, so codes and scales are bit-exact;
  * -fno-gpu-flush-denormals-to-zero: fp16 and binary32 subnormals are kept (the
    attention kernel feeds codes to the dot units as fp16 subnormals);
  * -Xclang -target-feature -Xclang -packed-fp32-ops: no packed binary32 VALU ops.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["kvq_quant.hip", "kvq_attn.hip", "kvq_api.hip"]
HEADERS = ["kvq_device.h", "kvq_internal.h", "kvq_append.h"]
LIB = os.path.join(HERE, "libkvq.so")
ARCH = "gfx950"

FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
         "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
         "-fno-fast-math", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES]


def inputs():
    return sources() + [os.path.join(CSRC, h) for h in HEADERS] + [
        os.path.join(ROOT, "include", "kvq.h")]


def build(verbose=False, extra=()):
    cmd = ["hipcc", *FLAGS, *extra, "-o", LIB + ".tmp", *sources()]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns that it does not know the packed-fp32 feature; drop that line
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + msg)
    if msg.strip() and verbose:
        print(msg)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def stale():
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in inputs())


if __name__ == "__main__":
    print(build(verbose=True))
