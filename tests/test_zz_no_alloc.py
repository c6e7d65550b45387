"""decode_attn_qkv_noalloc (the entry point that allocates nothing and works in the
library's static device array) against decode_attn_qkv with a caller workspace, through
the C ABI: bitwise equal outputs on consecutive calls of different shapes (a larger
call, a smaller one, then a larger one again, so that the array's counters and partial
states are reused across shapes), with several splits per row, and within the attention
tolerance of the oracle."""
import numpy as np
import pytest

import oracle
from decode_attention_block_amd import workloads as wl
from helpers import ATTN_TOL, attn_errors, gpu_quantize, say, to_gpu

pytestmark = pytest.mark.gpu


def _case(scheme, B, H, D, S, lens, seed):
    g = wl.rng(wl.WORKLOADS[0], 300 + seed, scheme, D)
    k = wl.draw(g, "normal_outliers", (B, S, H, D))
    v = wl.draw(g, "normal_outliers", (B, S, H, D))
    q = wl.draw(g, "normal0", (B, H, D))
    return k, v, q, np.asarray(lens, np.int32)


def test_noalloc_equals_workspace_call_on_consecutive_shapes():
    import decode_attention_block_amd as kvq
    import torch
    cases = [  # (scheme, B, H, D, S, lens, blocks_per_split)
        (oracle.INT4_SYM, 4, 8, 128, 700, (700, 1, 333, 64), 2),
        (oracle.FP8_E4M3, 1, 2, 64, 200, (200,), 1),
        (oracle.UINT8_ASYM, 3, 16, 128, 900, (900, 450, 0), 3),
        (oracle.INT4_SYM, 2, 4, 64, 300, (300, 129), 0),
    ]
    for i, (scheme, B, H, D, S, lens, bps) in enumerate(cases):
        say("noalloc case", i, "scheme", scheme, "B", B, "H", H, "D", D, "bps", bps)
        k, v, q, lens = _case(scheme, B, H, D, S, lens, i)
        MB = (S + 63) // 64
        c = gpu_quantize(scheme, k, v, lens, MB)
        max_len = int(lens.max())
        qt = to_gpu(q)
        ref = torch.empty((B, H, D), dtype=torch.float16, device="cuda")
        ws = kvq.make_workspace(c, max_len, bps)
        kvq.decode_attn_qkv(c, qt, 1.0 / np.sqrt(D), ref, ws, max_len, bps)
        out = torch.full((B, H, D), float("nan"), dtype=torch.float16, device="cuda")
        kvq.decode_attn_qkv_noalloc(c, qt, 1.0 / np.sqrt(D), out, max_len, bps)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), i
        o_ref = oracle.attention(c.host_arrays(), q, lens, 1.0 / np.sqrt(D))
        norm_err, _ = attn_errors(out.cpu().numpy(), o_ref)
        assert norm_err <= ATTN_TOL, (i, norm_err)
