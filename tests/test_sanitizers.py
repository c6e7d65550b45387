"""The library's host code and the oracle under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only): both are rebuilt with the sanitizers
(decode_attention_block_amd.build.build_sanitized: host code only, each -fsanitize= after
-Xarch_host; oracle.build.build_sanitized), and tests/sanitize_driver.py runs in a child
process with the clang ASan runtime preloaded: every argument-validation test of
test_abi.py, and the oracle's quantize / append / attention on small inputs of every
scheme, which must reproduce the plain build's outputs bit for bit."""
import os
import shutil
import subprocess
import sys

import numpy as np
import pytest

import oracle
from decode_attention_block_amd import build as kb
from decode_attention_block_amd import workloads as wl

HERE = os.path.dirname(os.path.abspath(__file__))

pytestmark = pytest.mark.skipif(
    shutil.which("hipcc") is None or not os.path.exists("/opt/rocm/llvm/bin/clang++")
    or os.path.exists("/dev/kfd"),
    reason="needs hipcc and ROCm's clang; host-validation cases run only without a GPU")


def _cases(path):
    out = {}
    for k, (scheme, B, H, D, S, lens, mb) in enumerate([
            (oracle.INT4_SYM, 2, 3, 64, 200, (130, 63), 4),
            (oracle.UINT8_ASYM, 2, 2, 128, 150, (64, 1), 3),
            (oracle.FP8_E4M3, 1, 4, 64, 140, (100,), 3)]):
        g = wl.rng(wl.WORKLOADS[0], 500 + k, scheme, D)
        kx = wl.draw(g, "normal_outliers", (B, S, H, D))
        vx = wl.draw(g, "normal0.5", (B, S, H, D))
        q = wl.draw(g, "normal0", (B, H, D))
        lens = np.array(lens, np.int32)
        c = oracle.quantize_cache(scheme, kx, vx, lens, mb)
        out.update({f"scheme{k}": scheme, f"k{k}": kx, f"v{k}": vx, f"lens{k}": lens,
                    f"mb{k}": mb, f"hk{k}": kx, f"hv{k}": vx, f"q{k}": q,
                    f"sm{k}": 1.0 / np.sqrt(D)})
        for key in ("k_codes", "v_codes", "k_scale", "v_scale", "k_zero", "v_zero"):
            out[f"{key}{k}"] = c[key].copy()
        oracle.append(c, kx, vx, lens + 1)
        for key in ("k_codes", "v_codes", "k_scale", "v_scale"):
            out[f"a_{key}{k}"] = c[key].copy()
        out[f"o{k}"] = oracle.attention(c, q, lens + 1, 1.0 / np.sqrt(D))
    np.savez(path, **out)


def test_host_code_and_oracle_under_asan_and_ubsan(tmp_path):
    rt = kb.sanitizer_runtime()
    if rt is None:
        pytest.skip("no clang AddressSanitizer runtime next to hipcc")
    lib = kb.build_sanitized(str(tmp_path / "libkvq_san.so"))
    orc = oracle._build.build_sanitized(str(tmp_path / "libkvq_oracle_san.so"))
    cases = str(tmp_path / "cases.npz")
    _cases(cases)
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, os.path.join(HERE, "sanitize_driver.py"), lib, orc,
                        cases], capture_output=True, text=True, env=env, timeout=600)
    print(r.stdout[-2000:], r.stderr[-4000:])
    assert r.returncode == 0 and "sanitizers ok" in r.stdout
