"""decode_attention_block_amd — block-quantized KV cache and single-token decode
attention for AMD Instinct MI355X (gfx950).

A thin binding over the C ABI of libkvq.so (include/kvq.h): the functions here carry
the same names as the library's entry points and only marshal arguments (tensor data
pointers, strides, the current HIP stream). Every step of the computation runs in the
library's HIP kernels; there is no CPU fallback, and a missing or unloadable library
raises. PyTorch provides device memory and streams.
"""
import ctypes

import numpy as np

from . import build as _build

INT4_SYM = 0
UINT8_ASYM = 1
FP8_E4M3 = 2
BLOCK_TOKENS = 64

STATUS = {0: "KVQ_OK", -1: "KVQ_EINVAL", -2: "KVQ_ENOTSUP", -3: "KVQ_ECAPACITY",
          -4: "KVQ_EALIGN", -5: "KVQ_EWORKSPACE", -6: "KVQ_EHIP"}

EXPORTS = ["kv_quantize_blocks", "kv_append", "decode_attn_plan", "decode_step_launches",
           "decode_attn_workspace_bytes", "decode_attn_qkv", "decode_attn_qkv_noalloc",
           "decode_attn_split",
           "decode_attn_combine", "decode_step_qkv", "decode_attn_gqa",
           "decode_attn_gqa_workspace_bytes", "decode_attn_gqa_plan", "kvq_int4_to_natural",
           "kvq_int4_from_natural", "kvq_probe_stream_read", "kvq_probe_hold",
           "kvq_strerror", "kvq_version"]


class KvqError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({kvq_strerror(status)})")


class kvq_cache(ctypes.Structure):
    """Mirror of struct kvq_cache in include/kvq.h."""
    _fields_ = [("scheme", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("max_blocks", ctypes.c_int32),
                ("k_codes", ctypes.c_void_p), ("v_codes", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("k_zero", ctypes.c_void_p), ("v_zero", ctypes.c_void_p),
                ("k_tail", ctypes.c_void_p), ("v_tail", ctypes.c_void_p),
                ("seq_lens", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("num_pages", ctypes.c_int32)]


_lib = None


def lib_path():
    return _build.LIB


def load_library():
    """Loads libkvq.so, building it first if there is none or its sources have changed
    since it was built (build.stale())."""
    global _lib
    if _lib is not None:
        return _lib
    if _build.stale():
        _build.build()
    L = ctypes.CDLL(_build.LIB)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    C = ctypes.POINTER(kvq_cache)
    sig = {
        "kv_quantize_blocks": ([C, P, P, i64, i64, i64, i32, P], ctypes.c_int),
        "kv_append": ([C, P, P, i32, P], ctypes.c_int),
        "decode_attn_plan": ([C, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i32)],
                             ctypes.c_int),
        "decode_step_launches": ([C, i32, i32], ctypes.c_int),
        "decode_attn_workspace_bytes": ([C, i32, i32], sz),
        "decode_attn_qkv": ([C, P, ctypes.c_float, P, P, sz, i32, i32, P], ctypes.c_int),
        "decode_attn_qkv_noalloc": ([C, P, ctypes.c_float, P, i32, i32, P], ctypes.c_int),
        "decode_attn_split": ([C, P, ctypes.c_float, P, sz, i32, i32, P], ctypes.c_int),
        "decode_attn_combine": ([C, P, P, sz, i32, i32, P], ctypes.c_int),
        "decode_step_qkv": ([C, P, P, P, ctypes.c_float, P, P, sz, i32, i32, P], ctypes.c_int),
        "decode_attn_gqa": ([C, P, i32, ctypes.c_float, P, P, sz, i32, i32, P], ctypes.c_int),
        "decode_attn_gqa_workspace_bytes": ([C, i32, i32, i32], sz),
        "decode_attn_gqa_plan": ([C, i32, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i32)],
                                 ctypes.c_int),
        "kvq_int4_to_natural": ([P, P, i32, i32, i64], ctypes.c_int),
        "kvq_int4_from_natural": ([P, P, i32, i32, i64], ctypes.c_int),
        "kvq_probe_stream_read": ([P, sz, i32, P, P], ctypes.c_int),
        "kvq_probe_hold": ([ctypes.c_uint32, P], ctypes.c_int),
        "kvq_strerror": ([ctypes.c_int], ctypes.c_char_p),
        "kvq_version": ([], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    _lib = L
    return L


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _check(rc, where):
    if rc != 0:
        raise KvqError(rc, where)


def _desc(cache):
    return ctypes.byref(cache.desc if isinstance(cache, KVCache) else cache)


def kvq_strerror(status):
    return load_library().kvq_strerror(status).decode()


def kvq_version():
    return load_library().kvq_version()


def kv_quantize_blocks(cache, k, v, max_len, stream=None):
    """k, v: fp16 CUDA tensors [B][S][H][D] (any strides, channels contiguous)."""
    if k.dim() != 4 or tuple(k.stride()) != tuple(v.stride()) or k.shape != v.shape:
        raise ValueError("k and v must be 4-D [B][S][H][D] tensors with equal strides")
    if k.stride(3) != 1:
        raise ValueError("channels must be contiguous")
    sb, st, sh = k.stride(0), k.stride(1), k.stride(2)
    rc = load_library().kv_quantize_blocks(_desc(cache), _ptr(k), _ptr(v), sb, st, sh,
                                           int(max_len), _stream(stream))
    _check(rc, "kv_quantize_blocks")


def kv_append(cache, k_new, v_new, max_len_after, stream=None):
    """k_new, v_new: fp16 CUDA tensors [B][H][D] contiguous."""
    if not (k_new.is_contiguous() and v_new.is_contiguous()):
        raise ValueError("k_new and v_new must be contiguous [B][H][D]")
    rc = load_library().kv_append(_desc(cache), _ptr(k_new), _ptr(v_new), int(max_len_after),
                                  _stream(stream))
    _check(rc, "kv_append")


def decode_attn_plan(cache, max_len, blocks_per_split=0):
    bps, ns = ctypes.c_int32(), ctypes.c_int32()
    rc = load_library().decode_attn_plan(_desc(cache), int(max_len), int(blocks_per_split),
                                         ctypes.byref(bps), ctypes.byref(ns))
    _check(rc, "decode_attn_plan")
    return bps.value, ns.value


def decode_step_launches(cache, max_len_after, blocks_per_split=0):
    """1 when decode_step_qkv runs as one kernel launch for these arguments, else 2."""
    rc = load_library().decode_step_launches(_desc(cache), int(max_len_after),
                                             int(blocks_per_split))
    if rc < 0:
        raise KvqError(rc, "decode_step_launches")
    return rc


def decode_attn_gqa_plan(cache, group, max_len, blocks_per_split=0):
    bps, ns = ctypes.c_int32(), ctypes.c_int32()
    rc = load_library().decode_attn_gqa_plan(_desc(cache), int(group), int(max_len),
                                             int(blocks_per_split), ctypes.byref(bps),
                                             ctypes.byref(ns))
    _check(rc, "decode_attn_gqa_plan")
    return bps.value, ns.value


def decode_attn_workspace_bytes(cache, max_len, blocks_per_split=0):
    return load_library().decode_attn_workspace_bytes(_desc(cache), int(max_len),
                                                      int(blocks_per_split))


def decode_attn_gqa_workspace_bytes(cache, group, max_len, blocks_per_split=0):
    return load_library().decode_attn_gqa_workspace_bytes(_desc(cache), int(group), int(max_len),
                                                          int(blocks_per_split))


def make_workspace(cache, max_len, blocks_per_split=0, device="cuda", group=1):
    """A zero-filled device workspace of decode_attn_workspace_bytes(...) bytes (or
    decode_attn_gqa_workspace_bytes(...) for group > 1; its arrival counters must start
    at zero, and the library leaves them zero)."""
    import torch
    n = (decode_attn_workspace_bytes(cache, max_len, blocks_per_split) if group == 1 else
         decode_attn_gqa_workspace_bytes(cache, group, max_len, blocks_per_split))
    return torch.zeros(max(n, 16), dtype=torch.uint8, device=device)


def decode_attn_qkv(cache, q, softmax_scale, out, workspace, max_len, blocks_per_split=0,
                    stream=None):
    """q, out: fp16 CUDA tensors [B][H][D] contiguous; workspace: CUDA tensor of at least
    decode_attn_workspace_bytes(...) bytes."""
    if not (q.is_contiguous() and out.is_contiguous()):
        raise ValueError("q and out must be contiguous [B][H][D]")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = load_library().decode_attn_qkv(_desc(cache), _ptr(q), float(softmax_scale), _ptr(out),
                                        _ptr(workspace), ws_bytes, int(max_len),
                                        int(blocks_per_split), _stream(stream))
    _check(rc, "decode_attn_qkv")


def decode_attn_qkv_noalloc(cache, q, softmax_scale, out, max_len, blocks_per_split=0,
                            stream=None):
    """decode_attn_qkv with no workspace argument: the library works in a static device
    array of its own (KVQ_NOALLOC_SCRATCH_BYTES per GPU); calls on one GPU must not
    overlap."""
    if not (q.is_contiguous() and out.is_contiguous()):
        raise ValueError("q and out must be contiguous [B][H][D]")
    rc = load_library().decode_attn_qkv_noalloc(_desc(cache), _ptr(q), float(softmax_scale),
                                                _ptr(out), int(max_len), int(blocks_per_split),
                                                _stream(stream))
    _check(rc, "decode_attn_qkv_noalloc")


def decode_attn_gqa(cache, q, group, softmax_scale, out, workspace, max_len, blocks_per_split=0,
                    stream=None):
    """Grouped-query attention: q, out fp16 CUDA tensors [B][H * group][D] contiguous,
    query head h * group + g reading cache head h."""
    if not (q.is_contiguous() and out.is_contiguous()):
        raise ValueError("q and out must be contiguous [B][H * group][D]")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = load_library().decode_attn_gqa(_desc(cache), _ptr(q), int(group), float(softmax_scale),
                                        _ptr(out), _ptr(workspace), ws_bytes, int(max_len),
                                        int(blocks_per_split), _stream(stream))
    _check(rc, "decode_attn_gqa")


def decode_attn_split(cache, q, softmax_scale, workspace, max_len, blocks_per_split=0,
                      stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = load_library().decode_attn_split(_desc(cache), _ptr(q), float(softmax_scale),
                                          _ptr(workspace), ws_bytes, int(max_len),
                                          int(blocks_per_split), _stream(stream))
    _check(rc, "decode_attn_split")


def decode_attn_combine(cache, out, workspace, max_len, blocks_per_split=0, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = load_library().decode_attn_combine(_desc(cache), _ptr(out), _ptr(workspace), ws_bytes,
                                            int(max_len), int(blocks_per_split),
                                            _stream(stream))
    _check(rc, "decode_attn_combine")


def decode_step_qkv(cache, k_new, v_new, q, softmax_scale, out, workspace, max_len_after,
                    blocks_per_split=0, stream=None):
    """kv_append(k_new, v_new) then decode_attn_qkv(q) over the lengths after the append,
    as one launch when the plan has one split per row. k_new, v_new, q, out: fp16 CUDA
    tensors [B][H][D] contiguous; workspace: at least
    decode_attn_workspace_bytes(cache, max_len_after, blocks_per_split) bytes."""
    for name, t in (("k_new", k_new), ("v_new", v_new), ("q", q), ("out", out)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous [B][H][D]")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = load_library().decode_step_qkv(_desc(cache), _ptr(k_new), _ptr(v_new), _ptr(q),
                                        float(softmax_scale), _ptr(out), _ptr(workspace),
                                        ws_bytes, int(max_len_after), int(blocks_per_split),
                                        _stream(stream))
    _check(rc, "decode_step_qkv")


def kvq_probe_stream_read(buf, workgroups, sink, stream=None):
    """Measurement aid: one streaming read of the device tensor `buf` (its whole storage)
    by at most `workgroups` workgroups; sink: int32/uint32 device tensor of at least
    workgroups * 256 elements."""
    nbytes = buf.numel() * buf.element_size()
    if sink.numel() * sink.element_size() < 4 * 256 * int(workgroups):
        raise ValueError("sink too small")
    rc = load_library().kvq_probe_stream_read(_ptr(buf), nbytes, int(workgroups), _ptr(sink),
                                              _stream(stream))
    _check(rc, "kvq_probe_stream_read")


def kvq_probe_hold(microseconds, stream=None):
    """Measurement aid: holds the stream for `microseconds` (1 .. 100000) of the GPU's
    real-time counter with one sleeping wave, so that a timing event recorded next marks
    when the GPU reaches the work queued after it."""
    _check(load_library().kvq_probe_hold(int(microseconds), _stream(stream)), "kvq_probe_hold")


class KVCache:
    """Device buffers of one quantized cache, allocated with torch, plus the C
    descriptor pointing at them. Code buffers start zeroed.

    num_pages=None gives the dense layout ([B][H][max_blocks] blocks). With num_pages the
    cache is paged: codes, scales and zero points are pools of num_pages pages (one
    64-token block of one sequence for all heads each) and `block_table` (int32
    [B][max_blocks], device) says which page holds block j of sequence b; it starts at
    block_table[b][j] = b * max_blocks + j when the pool has room for that, else -1, and
    the caller may set any mapping before the calls that use it."""

    def __init__(self, scheme, batch, heads, head_dim, max_blocks, device="cuda",
                 with_tail=True, with_zero=None, num_pages=None):
        import torch
        self.scheme, self.batch, self.heads = scheme, batch, heads
        self.head_dim, self.max_blocks = head_dim, max_blocks
        self.num_pages = num_pages
        rb = head_dim // 2 if scheme == INT4_SYM else head_dim
        if num_pages is None:
            lead = (batch, heads, max_blocks)
        else:
            lead = (num_pages, heads)
        self.k_codes = torch.zeros(lead + (BLOCK_TOKENS, rb), dtype=torch.uint8, device=device)
        self.v_codes = torch.zeros_like(self.k_codes)
        self.k_scale = torch.zeros(lead, dtype=torch.float32, device=device)
        self.v_scale = torch.zeros_like(self.k_scale)
        if with_zero is None:
            with_zero = True
        self.k_zero = torch.zeros_like(self.k_scale) if with_zero else None
        self.v_zero = torch.zeros_like(self.k_scale) if with_zero else None
        tshape = (batch, heads, BLOCK_TOKENS, head_dim)
        self.k_tail = torch.zeros(tshape, dtype=torch.float16, device=device) if with_tail else None
        self.v_tail = torch.zeros(tshape, dtype=torch.float16, device=device) if with_tail else None
        self.seq_lens = torch.zeros(batch, dtype=torch.int32, device=device)
        self.block_table = None
        if num_pages is not None:
            ident = torch.arange(batch * max_blocks, dtype=torch.int32, device=device)
            self.block_table = torch.where(ident < num_pages, ident,
                                           torch.full_like(ident, -1)).view(batch, max_blocks)
        self.desc = kvq_cache(scheme, batch, heads, head_dim, max_blocks,
                              _ptr(self.k_codes), _ptr(self.v_codes), _ptr(self.k_scale),
                              _ptr(self.v_scale), _ptr(self.k_zero), _ptr(self.v_zero),
                              _ptr(self.k_tail), _ptr(self.v_tail), _ptr(self.seq_lens),
                              _ptr(self.block_table), 0 if num_pages is None else num_pages)

    @property
    def capacity(self):
        return self.max_blocks * BLOCK_TOKENS

    def host_arrays(self, natural=True, seqs=None, blocks=None):
        """The cache buffers copied to numpy, keyed like the oracle's cache dicts
        (dense [B][H][max_blocks] order; a paged cache is gathered through its block
        table, entries clamped to the pool as the kernels do). With natural=True int4
        codes are returned in natural [token][channel] order (see layout.py); otherwise
        as stored. `seqs` (a list of sequence indices) and `blocks` (a slice of block
        indices) restrict the copy; "B" and "max_blocks" then give the sizes of what was
        copied."""
        from . import layout
        sel_b = slice(None) if seqs is None else list(seqs)
        sel_j = slice(None) if blocks is None else blocks
        b_list = list(range(self.batch))[sel_b] if seqs is None else sel_b
        j_list = list(range(self.max_blocks))[sel_j]
        out = {"scheme": self.scheme, "B": len(b_list), "H": self.heads, "D": self.head_dim,
               "max_blocks": len(j_list)}
        if self.num_pages is not None:
            table = self.block_table.cpu().numpy()[np.ix_(b_list, j_list)]
            pages = np.clip(table, 0, self.num_pages - 1)
        for key in ("k_codes", "v_codes", "k_scale", "v_scale", "k_zero", "v_zero"):
            t = getattr(self, key)
            if t is None:
                out[key] = None
            elif self.num_pages is None:
                out[key] = np.ascontiguousarray(t[sel_b][:, :, sel_j].cpu().numpy())
            else:
                pool = t.cpu().numpy()                      # [pages][H] + block shape
                out[key] = np.ascontiguousarray(np.moveaxis(pool[pages], 2, 1))
        if natural and self.scheme == INT4_SYM:
            out["k_codes"] = layout.int4_to_natural(out["k_codes"], "k")
            out["v_codes"] = layout.int4_to_natural(out["v_codes"], "v")
        return out
