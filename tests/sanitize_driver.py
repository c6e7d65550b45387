"""Runs under AddressSanitizer + UndefinedBehaviorSanitizer (started by
test_sanitizers.py with the clang ASan runtime preloaded; not collected by pytest).

argv: sanitized libkvq, sanitized oracle, cases.npz (inputs and the plain oracle's
outputs). Exercises the library's host code (every argument-validation test of
test_abi.py, which rejects its arguments before any HIP call) and the oracle's
quantize / append / attention on the stored inputs, which must reproduce the plain
build's outputs bit for bit. Any sanitizer report aborts the process."""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path[:0] = [ROOT, HERE]

lib_path, oracle_path, cases_path = sys.argv[1:4]

import decode_attention_block_amd.build as kb  # noqa: E402
kb.LIB = lib_path
kb.stale = lambda: False
import oracle  # noqa: E402
oracle._build.LIB = oracle_path
oracle._lib = None

import test_abi  # noqa: E402

n = 0
for name in sorted(dir(test_abi)):
    fn = getattr(test_abi, name)
    if name.startswith("test_") and callable(fn):
        fn()
        n += 1
print(f"abi: {n} host-validation tests passed under the sanitizers", flush=True)

cases = np.load(cases_path)
k = 0
while f"k{k}" in cases:
    scheme = int(cases[f"scheme{k}"])
    kx, vx, lens = cases[f"k{k}"], cases[f"v{k}"], cases[f"lens{k}"]
    mb = int(cases[f"mb{k}"])
    c = oracle.quantize_cache(scheme, kx, vx, lens, mb)
    for key in ("k_codes", "v_codes", "k_scale", "v_scale", "k_zero", "v_zero"):
        assert np.array_equal(c[key].view(np.uint8), cases[f"{key}{k}"].view(np.uint8)), (k, key)
    oracle.append(c, cases[f"hk{k}"], cases[f"hv{k}"], lens + 1)
    for key in ("k_codes", "v_codes", "k_scale", "v_scale"):
        assert np.array_equal(c[key].view(np.uint8), cases[f"a_{key}{k}"].view(np.uint8)), (k, key)
    o = oracle.attention(c, cases[f"q{k}"], lens + 1, float(cases[f"sm{k}"]))
    assert np.array_equal(o.view(np.uint64), cases[f"o{k}"].view(np.uint64)), k
    k += 1
print(f"oracle: {k} cases reproduced bit for bit under the sanitizers", flush=True)
print("sanitizers ok", flush=True)
