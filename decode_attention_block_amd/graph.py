"""A multi-layer decode step captured once as a HIP graph and replayed every step.

One decode step of an L-layer model calls the library once per layer; replaying a graph
of those calls replaces L launches from the host (argument checks, ctypes, queueing) by
one. The calls and their kernels are the library's own (decode_step_qkv, or
decode_attn_qkv for attention over a fixed cache); only the host side changes:

  * every input is read from a fixed device buffer that the caller fills before each
    replay (`k_new`, `v_new`, `q` per layer), and the outputs land in fixed buffers
    (`out` per layer);
  * lengths advance on the device (seq_lens), as in eager calls, so the graph stays
    valid from step to step; the host length bound is fixed at capture (max_len, by
    default the caches' capacity). With the automatic split plan (blocks_per_split = 0)
    each row's split is chosen on the device from the actual lengths, so the bound only
    sizes the grid;
  * nothing in the captured calls clears memory (the workspaces' arrival counters are
    zeroed once, before capture, and the kernels leave them zero).
"""
import decode_attention_block_amd as kvq


class DecodeGraph:
    """caches: one KVCache per layer (same shape). append=True captures
    decode_step_qkv per layer (append the layer's new K and V token, then attend);
    append=False captures decode_attn_qkv per layer. max_len: the host bound on the
    lengths during the replays (after the append), at most the capacity."""

    def __init__(self, caches, softmax_scale, append=True, blocks_per_split=0, max_len=None):
        import torch
        c0 = caches[0]
        self.caches = list(caches)
        self.append = append
        self.max_len = c0.capacity if max_len is None else int(max_len)
        shape = (c0.batch, c0.heads, c0.head_dim)
        dev = c0.seq_lens.device
        new = lambda: torch.zeros(shape, dtype=torch.float16, device=dev)
        self.q = [new() for _ in caches]
        self.out = [new() for _ in caches]
        self.k_new = [new() for _ in caches] if append else None
        self.v_new = [new() for _ in caches] if append else None
        self.workspace = [kvq.make_workspace(c, self.max_len, blocks_per_split, device=dev)
                          for c in caches]
        kvq.load_library()
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            for i, c in enumerate(self.caches):
                if append:
                    kvq.decode_step_qkv(c, self.k_new[i], self.v_new[i], self.q[i],
                                        softmax_scale, self.out[i], self.workspace[i],
                                        self.max_len, blocks_per_split)
                else:
                    kvq.decode_attn_qkv(c, self.q[i], softmax_scale, self.out[i],
                                        self.workspace[i], self.max_len, blocks_per_split)

    def replay(self):
        """Queues the captured step on the current stream."""
        self.graph.replay()
