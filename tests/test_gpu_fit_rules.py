"""GPU parity of the rank rule and the quantiser's division on inputs built
to expose them:

  * planted per-group spectra with distinct 90%-energy crossings: the GPU's
    per-group ranks equal the oracle's and the shared rank is their minimum
    (PALU page, "How it works", prefill step 3), with the captured energy of
    every group within 1e-4 of the oracle's;
  * latents equal to crafted fp16 values (unit-column bases, zero means) in
    which a reciprocal multiply would change codes: the GPU's records equal
    the oracle's bit for bit;
  * a fit that fails its rank check leaves the previous bases and stored
    tokens untouched.
"""
import numpy as np
import pytest

import oracle
from rank_latent_kv_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    if not _t.cuda.is_available():
        pytest.skip("no GPU")
    return _t


def _dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _energy(rows, mu, V):
    c = rows.astype(np.float64) - mu.astype(np.float64)
    proj = c @ V.astype(np.float64)
    return np.sum(proj * proj) / np.sum(c * c)


def test_shared_rank_minimum_with_distinct_group_ranks(torch):
    from rank_latent_kv_amd.palu import LatentKVCache
    N = 2048
    planted = {0: [12, 3, 20, 7], 1: [5, 9, 4, 16]}
    xs = {t: synth.planted_spectrum_groups(c, N, 128, seed=10 + t) for t, c in planted.items()}
    cache = LatentKVCache(128, 4, 8, 4, 1, N, rank=0, energy_threshold=0.90)
    cache.fit(_dev(torch, xs[0]), _dev(torch, xs[1]), [N])
    st = cache.stats()
    for t in (0, 1):
        f = oracle.fit(xs[t], [N], 4, rank=0, tau=0.90)
        assert list(f.r_groups) == planted[t]
        rg, e_prev, e_at = cache.fit_info(t)
        assert list(rg) == list(f.r_groups), (t, rg, f.r_groups)
        r, basis, mu, _ = cache.get_basis(t)
        assert r == f.r == min(planted[t])
        for g in range(4):
            rows = xs[t][0, g]
            assert abs(_energy(rows, f.mu[g], basis[g]) - _energy(rows, f.mu[g], f.V(g))) <= 1e-4
            # energy fractions at the shared rank against the oracle's spectrum
            s2 = f.sigma[g] ** 2
            assert abs(e_at[g] - s2[:r].sum() / s2.sum()) <= 1e-4
            assert abs(e_prev[g] - s2[:r - 1].sum() / s2.sum()) <= 1e-4
            np.testing.assert_allclose(basis[g].T.astype(np.float64) @ basis[g], np.eye(r), atol=1e-5)
        margin = st["energy_margin_k" if t == 0 else "energy_margin_v"]
        assert 0.015 <= margin <= 0.1, margin


def test_quantiser_division_cases_bit_exact(torch):
    """Unit-column bases and zero means make every latent equal to the
    crafted fp16 input value, so the GPU quantises the crafted groups."""
    from quant_cases import division_sensitive_group
    from rank_latent_kv_amd.palu import LatentKVCache
    r, n_groups, H = 8, 6, 2
    n_hi = oracle.n_hi_channels(r, 0.25)
    rng = np.random.default_rng(99)
    x = np.zeros((1, H, 32 * n_groups + 5, 128), np.float16)
    sensitive = 0
    for h in range(H):
        for j in range(n_groups):
            for c in range(r):
                l, n = division_sensitive_group(rng, 4 if c < n_hi else 2)
                x[0, h, 32 * j:32 * j + 32, c] = rng.permutation(l).astype(np.float16)
                sensitive += n
    x[0, :, 32 * n_groups:, :r] = rng.standard_normal((H, 5, r)).astype(np.float16)
    assert sensitive >= 40
    basis = np.zeros((1, 128, r), np.float32)
    basis[0, np.arange(r), np.arange(r)] = 1.0
    mu = np.zeros((1, 128), np.float32)
    cache = LatentKVCache(128, H, H, 1, 1, x.shape[2], rank=r)
    cache.set_basis(0, basis, mu)
    cache.set_basis(1, basis, mu)
    xd = _dev(torch, x)
    cache.encode_append(xd, xd)
    torch.cuda.synchronize()
    fit = oracle.Fit(r, np.array([r], np.int32), np.pad(basis, ((0, 0), (0, 0), (0, 128 - r))), mu,
                     np.zeros((1, 128)))
    layer = oracle.OracleLayer(128, H, H, 1, fit, fit)
    for h in range(H):
        # the latents are the inputs themselves
        assert np.array_equal(layer.latents(x[0, h], h, 0), x[0, h, :, :r].astype(np.float32))
        for t in (0, 1):
            st = layer.encode_head(x[0, h], h, t)
            rec, tail = cache.read_codes(0, h, t)
            assert np.array_equal(rec, st["records"]), (h, t)
            assert np.array_equal(tail.view(np.uint32), st["tail"].view(np.uint32)), (h, t)


def test_failed_fit_keeps_bases_and_tokens(torch):
    """A fit whose shared rank exceeds max_rank fails with CAPACITY before
    touching the cache: the old bases, lengths, records and attention stay."""
    from rank_latent_kv_amd.palu import LatentKVCache, PaluError
    N = 512
    good = synth.planted_spectrum_groups([3, 4, 3, 5], N, 128, seed=3)
    bad = synth.planted_spectrum_groups([12, 10, 20, 15], N, 128, seed=4)
    cache = LatentKVCache(128, 4, 8, 4, 1, N, rank=0, energy_threshold=0.90, max_rank=8)
    g = _dev(torch, good)
    cache.fit(g, g, [N])
    cache.encode_append(g[:, :, :100].contiguous(), g[:, :, :100].contiguous())
    q = _dev(torch, np.random.default_rng(1).standard_normal((1, 8, 128)).astype(np.float16))
    before = (cache.get_basis(0)[1].copy(), cache.read_codes(0, 2, 0), cache.decode_attend(q).cpu().numpy())
    b = _dev(torch, bad)
    with pytest.raises(PaluError) as ei:
        cache.fit(b, b, [N])
    assert ei.value.code == 4
    assert cache.seq_len(0) == 100
    assert np.array_equal(cache.get_basis(0)[1], before[0])
    rec, tail = cache.read_codes(0, 2, 0)
    assert np.array_equal(rec, before[1][0]) and np.array_equal(tail, before[1][1])
    after = cache.decode_attend(q).cpu().numpy()
    assert np.array_equal(after.view(np.uint16), before[2].view(np.uint16))
