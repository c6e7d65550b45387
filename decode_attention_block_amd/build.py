"""Builds libkvq.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Flags that matter for the results:
  * -fhip-fp32-correctly-rounded-divide-sqrt, no fast-math: x / s in the quantizer is
    the correctly rounded binary32 quotient, so codes and scales are bit-exact;
  * -fno-gpu-flush-denormals-to-zero: fp16 and binary32 subnormals are kept (the
    attention kernel feeds codes to the dot units as fp16 subnormals);
  * -Xclang -target-feature -Xclang -packed-fp32-ops: no packed binary32 VALU ops.
"""
import hashlib
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["kvq_quant.hip", "kvq_attn.hip", "kvq_api.hip", "kvq_probe.hip", "kvq_layout.hip"]
HEADERS = ["kvq_device.h", "kvq_internal.h", "kvq_append.h"]
LIB = os.path.join(HERE, "libkvq.so")
ARCH = "gfx950"

FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
         "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
         "-fno-fast-math", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # matrix-core results in ordinary VGPRs rather than accumulation registers: the
         # kernels read every result right away (softmax, rescale), and each read from an
         # accumulation register costs a v_accvgpr_read (measured: 8-query grouped-query
         # workload 20.4 -> 19.6 us, 8K attention 41.7 -> 41.4 us)
         "-mllvm", "-amdgpu-mfma-vgpr-form",
         "-Wall", "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES]


def inputs():
    return sources() + [os.path.join(CSRC, h) for h in HEADERS] + [
        os.path.join(ROOT, "include", "kvq.h")]


STAMP = LIB + ".inputs.sha256"  # hash of the sources and flags the library was built from


def inputs_hash(extra=()):
    """sha256 over the build flags and the contents of every source and header."""
    h = hashlib.sha256(" ".join([*FLAGS, *extra]).encode())
    for p in inputs():
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode() + b"\0" + f.read())
    return h.hexdigest()


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
    with open(STAMP, "w") as f:
        f.write(inputs_hash(extra) + "\n")
    return LIB


# Host-side sanitizers: AddressSanitizer and UndefinedBehaviorSanitizer on the host code
# only (argument validation, the split plan, launch set-up); each -fsanitize= is preceded
# by -Xarch_host so that no GPU code is built with them. Device code at -O0 (it is never
# run from this build; only the host paths are exercised, without a GPU).
SANITIZE_FLAGS = ["-O0", "-g", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
                  "-fno-fast-math", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                  "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=all",
                  "-Xarch_host", "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
                  "-I", CSRC]


def build_sanitized(out_path):
    """Builds the library with host-side ASan + UBSan into out_path (for the CPU tests;
    load it with the clang ASan runtime preloaded, see sanitizer_runtime())."""
    cmd = ["hipcc", *SANITIZE_FLAGS, "-o", out_path, *sources()]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc (sanitized) failed:\n" + r.stdout + r.stderr)
    return out_path


def sanitizer_runtime():
    """Path of the clang AddressSanitizer runtime that matches hipcc (its UBSan handlers
    included)."""
    r = subprocess.run(["hipcc", "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip().splitlines()[-1] if r.returncode == 0 and r.stdout.strip() else ""
    return path if os.path.isabs(path) and os.path.exists(path) else None


def stale():
    """True when there is no built library or its sources (or flags) have changed since
    it was built: the recorded hash is compared with the current contents, so copying
    the tree (which may reset file times) does not make a library stale."""
    if not os.path.exists(LIB) or not os.path.exists(STAMP):
        return True
    with open(STAMP) as f:
        return f.read().strip() != inputs_hash()


if __name__ == "__main__":
    print(build(verbose=True))
