"""Builds the CPU oracle (plain C++17, libc/libm only) into oracle/libkvq_oracle.so.

Test infrastructure: the oracle is compiled with IEEE binary32/binary64 semantics
(no fast-math, no FMA contraction) so that its quantizer rounds exactly once per
operation.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kvq_oracle.cpp")
LIB = os.path.join(HERE, "libkvq_oracle.so")


def build(verbose=False):
    cmd = ["g++", "-std=c++17", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def build_sanitized(out_path, clang="/opt/rocm/llvm/bin/clang++"):
    """The oracle with AddressSanitizer + UndefinedBehaviorSanitizer (clang, so that one
    sanitizer runtime serves it and the library's sanitized build in one process)."""
    cmd = [clang, "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-o", out_path, SRC]
    subprocess.run(cmd, check=True, capture_output=True)
    return out_path


if __name__ == "__main__":
    print(build(verbose=True))
