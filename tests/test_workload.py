"""Layouts and seeded inputs (CPU)."""

import numpy as np
import pytest

from sparse_communication_distributed_amd import workload as W


@pytest.mark.parametrize("name,n,P,K,k,tensors", [
    ("tiny", 1_048_576, 4, 2, 26_214, 1),
    ("gpt345m", 354_823_168, 32, 8, 1_108_822, 292),
    ("llama500m", 557_774_080, 32, 8, 174_304, 219),
    ("llama1.8b", 1_775_372_288, 32, 4, 554_803, 291),
    ("stress", 1_775_372_288, 64, 4, 27_740, 291),
])
def test_config_sizes(name, n, P, K, k, tensors):
    c = W.CONFIGS[name]
    assert (c.n, c.P, c.K, c.k, len(c.tensors)) == (n, P, K, k, tensors)
    assert c.n_p * c.P == c.n


def test_k_exact_and_sparsity_zero():
    assert W.flat_config("a", 1000, 1, 1, "0").k == 1000
    assert W.flat_config("a", 1000, 1, 1, "0.999").k == 1
    assert W.flat_config("a", 100, 1, 1, "0.999").k == 1
    assert W.flat_config("a", 30, 3, 1, "0.9").k == 1


def test_partition_streams_reproducible_and_independent():
    c = W.flat_config("s", 4 * 1000, 4, 3, "0.9", grad_law="tensor_sigma")
    full = W.grads(c, step=2, seed=0)
    sub = W.grads(c, step=2, seed=0, partitions=[2])
    assert np.array_equal(full[:, 2000:3000], sub)
    assert not np.array_equal(W.grads(c, 3, 0), full)
    assert full.dtype == np.float32 and np.all(np.isfinite(full))
    w = W.init_params(c)
    assert np.array_equal(w[1000:2000], W.init_params(c, partitions=[1]))
    assert abs(float(w.std()) - 0.02) < 2e-3


def test_partition_scale_law_and_stress_duplicates():
    t = W.flat_config("t", 4 * 4096, 4, 2, "0.9", grad_law="partition_scale")
    g = W.grads(t, 1)
    s = W.partition_scales(t)
    for p in range(4):
        std = float(g[0, p * 4096:(p + 1) * 4096].std())
        assert abs(std / (s[p] * 1e-3) - 1) < 0.1
    st = W.flat_config("st", 2 * 20000, 2, 2, "0.99", grad_law="stress_t3")
    gs = W.grads(st, 1)
    for p in range(2):
        mag = np.abs(gs[0, p * 20000:(p + 1) * 20000])
        vals, counts = np.unique(mag, return_counts=True)
        assert counts.max() >= 5          # planted duplicate magnitudes
        assert np.all(np.isfinite(mag))


def test_device_stress_law_plants_host_drawn_duplicates():
    """The device generator's stress law, run here on a CPU tensor through
    the same code: it is the base draw (sigma * t_3) except at the
    floor(1% n_p) distinct positions that duplicate_draws gives for each
    (step, worker, partition), which hold sign-preserving copies of the
    donor magnitudes ranked k-8 .. k+7 of that partition's base draw."""
    torch = pytest.importorskip("torch")
    cfg = W.flat_config("dstress", 3 * 30_000, 3, 2, "0.999", grad_law="stress_t3")
    n_p, k = cfg.n_p, cfg.k
    sigma = W.device_sigma(cfg, 0, "cpu")
    base = torch.empty((cfg.K, cfg.n), dtype=torch.float32)
    g = torch.empty_like(base)
    W.device_base_grads(cfg, 2, 0, sigma, base)
    W.device_grads(cfg, 2, 0, sigma, g)
    b, gg = base.numpy(), g.numpy()
    assert W.donor_count(cfg) == 16
    for i in range(cfg.K):
        for p in range(cfg.P):
            sl = slice(p * n_p, (p + 1) * n_p)
            bs, gs = b[i, sl], gg[i, sl]
            pos, pick = W.duplicate_draws(cfg, 0, 2, i, p)
            assert pos.size == n_p // 100 == np.unique(pos).size
            assert pos.min() >= 0 and pos.max() < n_p and pick.min() >= 0 and pick.max() < 16
            off = np.ones(n_p, bool)
            off[pos] = False
            assert np.array_equal(gs[off].view(np.uint32), bs[off].view(np.uint32))
            donors = np.sort(np.abs(bs))[::-1][k - 8:k + 8]
            assert np.array_equal(np.abs(gs[pos]), donors[pick])
            assert np.all(np.signbit(gs[pos]) == (bs[pos] < 0))
            # the planted magnitudes straddle the k-th largest: exact ties there
            assert np.count_nonzero(np.abs(gs) == donors[7]) >= 2


def test_duplicate_draws_are_the_host_law_draws():
    """The host law plants at duplicate_draws' positions and picks too."""
    cfg = W.flat_config("hstress", 2 * 20_000, 2, 2, "0.99", grad_law="stress_t3")
    g = W.grads_partition(cfg, 1, 1, 1)
    r = W.rng(0, cfg.config_id, W.STREAM_GRADS, 1, 1, 1)
    base = (W.sigma_per_element(cfg, 0, cfg.n_p, 2 * cfg.n_p) *
            r.standard_t(3, size=cfg.n_p).astype(np.float32)).astype(np.float32)
    pos, pick = W.duplicate_draws(cfg, 0, 1, 1, 1)
    off = np.ones(cfg.n_p, bool)
    off[pos] = False
    assert np.array_equal(g[off], base[off])
    donors = np.sort(np.abs(base))[::-1][cfg.k - 8:cfg.k + 8]
    assert np.array_equal(np.abs(g[pos]), donors[pick])
