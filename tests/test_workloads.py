"""The seeded input recipes: determinism, independence of the per-sequence streams,
and the distributions the workloads name (N(0,1) with 0.1% x20 outliers, N(0.5,1),
0.5 * Student-t with 3 degrees of freedom, ragged lengths in [1024, 8192])."""
import numpy as np
import pytest

from decode_attention_block_amd import workloads as wl


def test_host_recipe_is_deterministic_and_per_sequence():
    w = wl.WORKLOADS[1]
    a = wl.prefill_batch(w, 0, 0, n_tokens=16, seqs=[0, 1])
    b = wl.prefill_batch(w, 0, 0, n_tokens=16, seqs=[1])
    assert a.dtype == np.float16 and a.shape == (2, 16, 32, 128)
    assert np.array_equal(a[1], b[0])
    assert not np.array_equal(a[0], a[1])
    assert not np.array_equal(wl.prefill_batch(w, 0, 1, n_tokens=16, seqs=[0])[0], a[0])


def test_outlier_mixture_statistics():
    w = wl.WORKLOADS[1]
    x = wl.prefill_kv(w, 0, 0, 0, n_tokens=512).astype(np.float64).ravel()
    big = np.abs(x) > 6.0                 # N(0,1) alone exceeds 6 with probability 2e-9
    assert 0.0006 < big.mean() < 0.0011   # 0.1% outliers, ~82% of them beyond 6 after x20
    assert abs(x[~big].std() - 1.0) < 0.01 and abs(x.mean()) < 0.01


def test_outlier_positions_are_distinct():
    """Each outlier is scaled once (x20, never x400): the positions are distinct, and
    their number has the Binomial(n, 0.001) mean."""
    counts = []
    for seed in range(20):
        g = np.random.Generator(np.random.PCG64(seed))
        pos = wl.outlier_positions(g, 200_000)
        assert len(np.unique(pos)) == len(pos)
        assert pos.min() >= 0 and pos.max() < 200_000
        counts.append(len(pos))
    assert abs(np.mean(counts) - 200.0) < 3 * np.sqrt(200.0 / 20)


def test_uint8_workload_value_mean():
    w = wl.WORKLOADS[2]
    v = wl.prefill_kv(w, 0, 0, 1, n_tokens=256).astype(np.float64)
    assert abs(v.mean() - 0.5) < 0.01 and abs(v.std() - 1.0) < 0.01


def test_student_t3_half_quantiles():
    # 0.5 * t_3: P(|t_3| > 3.182) = 0.05 (two-sided 95% quantile), variance of t_3 is 3
    w = wl.WORKLOADS[4]
    x = wl.prefill_kv(w, 0, 0, 0, n_tokens=256).astype(np.float64).ravel() / 0.5
    assert abs(np.mean(np.abs(x) > 3.182) - 0.05) < 0.002
    assert abs(np.median(np.abs(x)) - 0.765) < 0.01   # median of |t_3|


def test_ragged_lengths_in_range_and_shared():
    w = wl.WORKLOADS[4]
    lens = wl.lengths(w)
    assert lens.shape == (8,) and lens.min() >= 1024 and lens.max() <= 8192
    assert np.array_equal(lens, wl.lengths(w))
    assert (lens % 64 != 0).any()


@pytest.mark.parametrize("index", [1, 2, 4])
def test_device_recipe_matches_distributions_on_cpu(index):
    torch = pytest.importorskip("torch")
    w = wl.WORKLOADS[index]
    which = 1
    x = wl.prefill_batch_device(w, 3, which, n_tokens=64, device="cpu")
    y = wl.prefill_batch_device(w, 3, which, n_tokens=64, device="cpu")
    assert x.dtype == torch.float16 and tuple(x.shape) == (w.batch, 64, w.heads, w.head_dim)
    assert torch.equal(x, y)
    h = wl.prefill_batch(w, 3, which, n_tokens=64).astype(np.float64).ravel()
    d = x.double().numpy().ravel()
    for qtl in (0.01, 0.25, 0.5, 0.75, 0.99):
        assert abs(np.quantile(d, qtl) - np.quantile(h, qtl)) < 0.03, qtl
