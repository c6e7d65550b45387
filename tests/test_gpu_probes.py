"""The measurement aids on the GPU: the stream-read probe folds every 16-byte chunk of its
buffer into its sink (checked against the same fold done with numpy), and the hold probe
keeps its stream busy for about the requested time."""
import numpy as np
import pytest

from helpers import say

pytestmark = pytest.mark.gpu


def test_stream_read_probe_reads_every_chunk():
    import decode_attention_block_amd as kvq
    import torch
    say("stream read probe")
    n, wgs = 1 << 20, 4                      # 4 slabs of 256 KiB (whole 4 KiB units)
    host = np.random.default_rng(5).integers(0, 256, n, dtype=np.uint8)
    buf = torch.from_numpy(host).cuda()
    sink = torch.zeros(wgs * 256, dtype=torch.int32, device="cuda")
    kvq.kvq_probe_stream_read(buf, wgs, sink)
    torch.cuda.synchronize()
    words = host.view(np.uint32).reshape(wgs, -1, 256, 4)   # slab, 4 KiB unit, thread, dword
    expect = np.bitwise_xor.reduce(np.bitwise_xor.reduce(words, axis=3), axis=1).reshape(-1)
    assert np.array_equal(sink.cpu().numpy().view(np.uint32), expect)


def test_hold_probe_holds_the_stream():
    import decode_attention_block_amd as kvq
    import torch
    say("hold probe")
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    kvq.kvq_probe_hold(2000)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    print(f"hold of 2000 us measured {ms * 1e3:.1f} us")
    assert 1.8 <= ms <= 20.0
