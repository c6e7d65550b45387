"""The C-ABI library loads, exports every entry point include/kvq.h declares, and
rejects bad arguments on the host before launching anything (no GPU needed: every
case below fails validation, so no HIP call is made; device pointers are fake)."""
import ctypes
import os
import re

import pytest

import decode_attention_block_amd as kvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x100000  # 16-byte aligned stand-in for device memory, never dereferenced

# The cases below pass fake device pointers and rely on host validation rejecting
# them; they never run where a GPU is present, so a validation bug cannot launch.
no_gpu_only = pytest.mark.skipif(os.path.exists("/dev/kfd"),
                                 reason="fake-pointer validation cases run only without a GPU")


def declared_functions():
    text = open(os.path.join(ROOT, "include", "kvq.h"), encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\s*\(", text, flags=re.M)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(kvq.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = kvq.load_library()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert kvq.kvq_version() == 5


def cache(scheme=0, B=2, H=4, D=128, MB=3, **kw):
    fields = dict(k_codes=FAKE, v_codes=FAKE, k_scale=FAKE, v_scale=FAKE, k_zero=FAKE,
                  v_zero=FAKE, k_tail=FAKE, v_tail=FAKE, seq_lens=FAKE, block_table=None,
                  num_pages=0)
    fields.update(kw)
    return kvq.kvq_cache(scheme, B, H, D, MB, *[fields[f] for f in (
        "k_codes", "v_codes", "k_scale", "v_scale", "k_zero", "v_zero", "k_tail", "v_tail",
        "seq_lens", "block_table", "num_pages")])


def rc_quant(c, k=FAKE, v=FAKE, strides=(3 * 64 * 4 * 128, 4 * 128, 128), max_len=100):
    L = kvq.load_library()
    return L.kv_quantize_blocks(ctypes.byref(c), k, v, *strides, max_len, None)


def rc_attn(c, q=FAKE, out=FAKE, ws=FAKE, ws_bytes=1 << 30, max_len=100, bps=0):
    L = kvq.load_library()
    return L.decode_attn_qkv(ctypes.byref(c), q, 0.1, out, ws, ws_bytes, max_len, bps, None)


def rc_append(c, k=FAKE, v=FAKE, max_len_after=100):
    return kvq.load_library().kv_append(ctypes.byref(c), k, v, max_len_after, None)


def rc_step(c, k=FAKE, v=FAKE, q=FAKE, out=FAKE, ws=FAKE, ws_bytes=1 << 30, max_len_after=100,
            bps=0):
    return kvq.load_library().decode_step_qkv(ctypes.byref(c), k, v, q, 0.1, out, ws, ws_bytes,
                                              max_len_after, bps, None)


EINVAL, ENOTSUP, ECAP, EALIGN, EWS = -1, -2, -3, -4, -5


@no_gpu_only
def test_null_and_bad_descriptor():
    L = kvq.load_library()
    assert L.kv_quantize_blocks(None, FAKE, FAKE, 0, 0, 0, 10, None) == EINVAL
    assert rc_quant(cache(scheme=3)) == EINVAL
    assert rc_quant(cache(scheme=-1)) == EINVAL
    assert rc_quant(cache(B=0)) == EINVAL
    assert rc_quant(cache(H=-1)) == EINVAL
    assert rc_quant(cache(MB=0)) == EINVAL
    assert rc_quant(cache(D=96)) == ENOTSUP
    assert rc_quant(cache(k_codes=0)) == EINVAL
    assert rc_quant(cache(seq_lens=0)) == EINVAL
    assert rc_quant(cache(scheme=1, v_zero=0)) == EINVAL
    assert rc_quant(cache(), k=0) == EINVAL


@no_gpu_only
def test_alignment_rules():
    assert rc_quant(cache(k_codes=FAKE + 8)) == EALIGN
    assert rc_quant(cache(), k=FAKE + 2) == EALIGN
    assert rc_quant(cache(), strides=(3 * 64 * 4 * 128, 4 * 128, 4)) == EALIGN
    assert rc_attn(cache(), q=FAKE + 4) == EALIGN
    assert rc_attn(cache(), out=FAKE + 4) == EALIGN
    assert rc_append(cache(), k=FAKE + 2) == EALIGN


@no_gpu_only
def test_capacity_and_lengths():
    assert rc_quant(cache(MB=3), max_len=3 * 64 + 1) == ECAP
    assert rc_quant(cache(), max_len=-1) == EINVAL
    assert rc_attn(cache(MB=3), max_len=193) == ECAP
    assert rc_append(cache(MB=3), max_len_after=193) == ECAP
    assert rc_append(cache(), max_len_after=0) == EINVAL
    assert rc_append(cache(k_tail=0)) == EINVAL
    assert rc_append(cache(H=256)) == ENOTSUP           # arrival count must fit 8 bits
    assert rc_append(cache(MB=1 << 18), max_len_after=100) == ENOTSUP  # lengths < 2^24
    # a row's codes are addressed with 32-bit offsets: below 2^31 bytes
    assert rc_attn(cache(MB=(1 << 19) + 1, D=128)) == ENOTSUP            # int4: 4 KiB blocks
    assert rc_attn(cache(MB=(1 << 19) - 1, D=128), ws=0) == EWS           # just fits
    assert rc_attn(cache(scheme=1, MB=(1 << 18) + 1, D=128)) == ENOTSUP  # uint8: 8 KiB
    assert rc_attn(cache(scheme=2, MB=(1 << 18) + 1, D=128)) == ENOTSUP  # FP8: 8 KiB
    assert rc_attn(cache(scheme=1, MB=1 << 18, D=64), ws=0) == EWS


@no_gpu_only
def test_paged_layout_rules():
    # a block table needs a pool, and page * heads must stay a 32-bit index
    assert rc_quant(cache(block_table=FAKE, num_pages=0)) == EINVAL
    assert rc_quant(cache(block_table=FAKE, num_pages=-3)) == EINVAL
    assert rc_quant(cache(H=64, block_table=FAKE, num_pages=(1 << 25) + 1)) == EINVAL
    assert rc_attn(cache(H=64, block_table=FAKE, num_pages=(1 << 25) - 1), ws=0) == EWS
    # pages are addressed one by one: rows of 2^31 bytes or more are fine
    assert rc_attn(cache(MB=(1 << 19) + 1, D=128, block_table=FAKE, num_pages=8), ws=0) == EWS
    assert rc_step(cache(B=1, H=1, MB=4, block_table=FAKE, num_pages=0)) == EINVAL


def rc_gqa(c, q=FAKE, group=2, out=FAKE, ws=FAKE, ws_bytes=1 << 30, max_len=100, bps=0):
    return kvq.load_library().decode_attn_gqa(ctypes.byref(c), q, group, 0.1, out, ws, ws_bytes,
                                              max_len, bps, None)


@no_gpu_only
def test_grouped_query_rules():
    assert rc_gqa(cache(), group=3) == EINVAL
    assert rc_gqa(cache(), group=16) == EINVAL
    assert rc_gqa(cache(), group=0) == EINVAL
    assert rc_gqa(cache(scheme=1), group=2, q=FAKE + 2) == EALIGN   # every scheme is taken
    assert rc_gqa(cache(scheme=2), group=8, q=FAKE + 2) == EALIGN
    assert rc_gqa(cache(scheme=1), group=5) == EINVAL
    assert rc_gqa(cache(), q=FAKE + 2) == EALIGN
    assert rc_gqa(cache(), out=0) == EINVAL
    c = cache(B=2, H=4, D=128, MB=3)
    need = kvq.decode_attn_gqa_workspace_bytes(c, 4, 192, 1)
    assert need == 256 + 2 * 4 * 4 * 3 * (128 + 2) * 4     # partial states per query row
    assert kvq.decode_attn_gqa_workspace_bytes(c, 1, 192, 1) == \
        kvq.decode_attn_workspace_bytes(c, 192, 1)
    assert rc_gqa(c, group=4, ws_bytes=need - 1, max_len=192, bps=1) == EWS
    assert rc_gqa(c, group=4, max_len=193) == ECAP


@no_gpu_only
def test_workspace_rules():
    c = cache(B=2, H=4, D=128, MB=3)
    need = kvq.decode_attn_workspace_bytes(c, 192, 1)
    assert need == 256 + 2 * 4 * 3 * (128 + 2) * 4      # counters (padded) + partials
    assert rc_attn(c, ws_bytes=need - 1, max_len=192, bps=1) == EWS
    assert rc_attn(c, ws=0, max_len=192, bps=1) == EWS
    assert rc_attn(c, ws=FAKE + 4, ws_bytes=need, max_len=192, bps=1) == EALIGN
    assert rc_attn(c, max_len=192, bps=-1) == EINVAL
    assert kvq.decode_attn_workspace_bytes(cache(D=96), 10) == 0


@no_gpu_only
def test_decode_step_validates_like_append_and_attention():
    # every rule of kv_append and of decode_attn_qkv, checked before anything launches
    assert rc_step(cache(), q=0) == EINVAL
    assert rc_step(cache(), out=0) == EINVAL
    assert rc_step(cache(), k=0) == EINVAL
    assert rc_step(cache(), v=FAKE + 2) == EALIGN
    assert rc_step(cache(), q=FAKE + 4) == EALIGN
    assert rc_step(cache(), out=FAKE + 4) == EALIGN
    assert rc_step(cache(scheme=3)) == EINVAL
    assert rc_step(cache(D=96)) == ENOTSUP
    assert rc_step(cache(v_tail=0)) == EINVAL
    assert rc_step(cache(H=256)) == ENOTSUP
    assert rc_step(cache(MB=3), max_len_after=193) == ECAP
    assert rc_step(cache(), max_len_after=0) == EINVAL
    assert rc_step(cache(MB=(1 << 19) + 1, D=128, B=1, H=1), max_len_after=100) == ENOTSUP
    c = cache(B=2, H=4, D=128, MB=3)
    need = kvq.decode_attn_workspace_bytes(c, 192, 1)
    assert rc_step(c, ws_bytes=need - 1, max_len_after=192, bps=1) == EWS
    assert rc_step(c, ws=0, max_len_after=192, bps=1) == EWS
    assert rc_step(c, ws=FAKE + 4, ws_bytes=need, max_len_after=192, bps=1) == EALIGN
    assert rc_step(c, max_len_after=192, bps=-1) == EINVAL


def test_plan_is_whole_blocks_and_covers_context():
    c = cache(B=8, H=32, D=128, MB=129)
    for max_len in (1, 64, 65, 8192, 8256):
        nb = (max_len + 63) // 64
        for bps in (1, 5, 64, 200):
            assert kvq.decode_attn_plan(c, max_len, bps) == (bps, (nb + bps - 1) // bps)
    assert kvq.decode_attn_plan(c, 0) == (0, 0)
    assert kvq.decode_attn_plan(c, 0, 5) == (5, 0)


def test_automatic_plan_bounds_the_pieces_a_row_may_take():
    # the split of each row is chosen on the device (blocks_per_split_out = 0); the host
    # bounds it: 3 pieces once the rows alone fill the 256 CUs (a ragged batch cuts its
    # long rows in two or three) ...
    assert kvq.decode_attn_plan(cache(B=8, H=32, MB=129), 8192) == (0, 3)
    assert kvq.decode_attn_plan(cache(B=16, H=32, MB=514), 32832) == (0, 3)
    assert kvq.decode_attn_plan(cache(B=8, H=32, MB=129), 64) == (0, 1)   # one block
    # ... else one more than the pieces that equal rows take to reach about 256
    # workgroups, never more than the blocks
    assert kvq.decode_attn_plan(cache(B=1, H=32, MB=2048), 131072) == (0, 9)
    assert kvq.decode_attn_plan(cache(B=1, H=2, MB=4), 256) == (0, 4)
    assert kvq.decode_attn_plan(cache(B=3, H=5, MB=64), 4096) == (0, 19)


def test_decode_step_is_one_launch_when_every_row_is_one_piece():
    assert kvq.decode_step_launches(cache(B=8, H=32, MB=129), 8193) == 1
    assert kvq.decode_step_launches(cache(B=16, H=32, MB=514), 32832) == 1
    assert kvq.decode_step_launches(cache(B=1, H=32, MB=2048), 8193) == 2
    assert kvq.decode_step_launches(cache(B=1, H=2, MB=4), 200, 4) == 1
    assert kvq.decode_step_launches(cache(B=8, H=32, MB=129), 8193, 64) == 2
    with pytest.raises(kvq.KvqError):
        kvq.decode_step_launches(cache(B=8, H=32, MB=129), 129 * 64 + 1)


def test_grouped_query_plan_aims_at_two_workgroups_per_cu_int4_one_8bit():
    # 8 sequences x 8 cached heads, 8K: 64 rows; over an int4 cache equal rows take
    # 512 / 64 = 8 pieces of 16 blocks on the device, over the 8-bit caches 256 / 64 = 4
    # of 32, and the grid allows one more
    c = cache(B=8, H=8, MB=128)
    assert kvq.decode_attn_gqa_plan(c, 8, 8192) == (0, 9)
    for scheme in (1, 2):
        assert kvq.decode_attn_gqa_plan(cache(scheme, B=8, H=8, MB=128), 8, 8192) == (0, 5)
    assert kvq.decode_attn_gqa_plan(c, 1, 8192) == kvq.decode_attn_plan(c, 8192) == (0, 5)
    assert kvq.decode_attn_gqa_plan(c, 4, 8192, 5) == (5, (128 + 4) // 5)
    # the workspace follows the grouped plan
    assert kvq.decode_attn_gqa_workspace_bytes(c, 8, 8192, 0) == \
        kvq.decode_attn_gqa_workspace_bytes(c, 8, 8192, 15)   # ceil(128 / 15) = 9 splits
    with pytest.raises(kvq.KvqError):
        kvq.decode_attn_gqa_plan(c, 0, 8192)


@no_gpu_only
def test_split_count_limit_of_the_grid():
    # a row may take at most 65,535 splits (the grid's split dimension)
    L = kvq.load_library()
    c = cache(B=1, H=1, MB=(1 << 24) // 64 - 1)
    rc = L.decode_attn_qkv(ctypes.byref(c), FAKE, 0.1, FAKE, FAKE, 1 << 40, 70000 * 64, 1, None)
    assert rc == ENOTSUP


def test_strerror_names_every_status():
    for code in range(-6, 1):
        assert kvq.kvq_strerror(code) != "unknown status"
    assert kvq.kvq_strerror(-99) == "unknown status"


@no_gpu_only
def test_stream_read_probe_validation():
    L = kvq.load_library()
    probe = L.kvq_probe_stream_read
    assert probe(None, 4096, 256, FAKE, None) == EINVAL
    assert probe(FAKE, 0, 256, FAKE, None) == EINVAL
    assert probe(FAKE, 4096, 0, FAKE, None) == EINVAL
    assert probe(FAKE, 4096, 256, None, None) == EINVAL
    assert probe(FAKE + 8, 4096, 256, FAKE, None) == EALIGN
    # one workgroup cannot stream 3 GiB in a slab below 2^31 bytes
    assert probe(FAKE, 3 << 30, 1, FAKE, None) == ENOTSUP


@no_gpu_only
def test_hold_probe_validation():
    hold = kvq.load_library().kvq_probe_hold
    assert hold(0, None) == EINVAL
    assert hold(100001, None) == EINVAL


def rc_noalloc(c, q=FAKE, out=FAKE, max_len=100, bps=0):
    return kvq.load_library().decode_attn_qkv_noalloc(ctypes.byref(c), q, 0.1, out, max_len,
                                                      bps, None)


@no_gpu_only
def test_noalloc_validation_before_any_hip_call():
    assert rc_noalloc(cache(), q=0) == EINVAL
    assert rc_noalloc(cache(), out=FAKE + 4) == EALIGN
    assert rc_noalloc(cache(MB=3), max_len=3 * 64 + 1) == ECAP
    assert rc_noalloc(cache(), bps=-1) == EINVAL
    # more rows than the static array has counters for
    assert rc_noalloc(cache(B=300, H=256)) == EWS
    # partial states beyond the array: 1024 rows x 2048 splits x 130 floats
    assert rc_noalloc(cache(B=32, H=32, MB=2048), max_len=2048 * 64, bps=1) == EWS
