"""GPU parity with per-sequence bases (per_seq_basis = 1): every slot holds
its own K and V bases and means, fitted from its own prompt.

The oracle side is the shared-basis fit applied to one sequence's rows:
slot b's expected basis is oracle.fit of row b alone, and its expected
codes and attention come from an oracle layer built on that fit.  Rows are
drawn from workloads with different seeds, so their planted subspaces and
means differ and a kernel that read another slot's basis would fail.

  * fit: per slot, identical rank and captured energy within 1e-4 of the
    oracle's, means within 1e-5;
  * codes and tails bit-exact, decode and prefill attention within
    2e-3 + 1e-2 |ref|, for PALU splits (fp16 and bf16 inputs, fp16 value
    latents) and a bit schedule (the generic coder path);
  * re-fitting some slots leaves the others' bases, codes and outputs as
    they were;
  * a slot exported with its bases and imported into another cache (whose
    slot held other bases) restores codes and decode output bitwise;
  * slots without bases are refused.
"""
import numpy as np
import pytest

import oracle
from rank_latent_kv_amd import synth

from test_gpu_parity import _check_attention, _dev, _energy

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    if not _t.cuda.is_available():
        pytest.skip("no GPU")
    return _t


def _rows(ws, tensor, total, bf16=False):
    """Row b from workload ws[b] (its own subspace and mean): [B, H, total, D]."""
    return np.concatenate([synth.batch_kv(w, tensor, total, seqs=[b], bf16=bf16) for b, w in enumerate(ws)])


def _workloads(B, gqa, groups, rank, vq, seed):
    return [synth.small_workload(batch=B, n_q_heads=2 * gqa, n_kv_heads=2, n_head_groups=groups, prefill=96,
                                 rank=rank, quantize_values=vq, seed=seed + 31 * b) for b in range(B)]


def _cache(torch, w, B, total, rank, **kw):
    from rank_latent_kv_amd.palu import LatentKVCache
    return LatentKVCache(128, w.n_kv_heads, w.n_q_heads, w.n_head_groups, B, total, rank=rank,
                         quantize_values=w.quantize_values, per_seq_basis=True, **kw)


def _bdev(torch, x, bf16):
    if not bf16:
        return _dev(torch, x)
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)


def _out(t, bf16):
    if not bf16:
        return t.cpu().numpy()
    return oracle.bf16_to_float(t.cpu().view(__import__("torch").int16).numpy().view(np.uint16))


def _state_equal(cache, layer, xk, xv, slot):
    for tensor, x in ((0, xk), (1, xv)):
        for h in range(x.shape[0]):
            st = layer.encode_head(x[h], h, tensor)
            rec, tail = cache.read_codes(slot, h, tensor)
            if "fp16" in st:
                continue
            assert np.array_equal(rec, st["records"]), (slot, h, tensor)
            assert np.array_equal(tail.view(np.uint32), st["tail"].view(np.uint32)), (slot, h, tensor)


def _fit_of_slot(cache, seq, tensor):
    """The slot's installed basis as an oracle Fit."""
    r, basis, mu, sigma = cache.get_basis(tensor, seq=seq)
    G, D = basis.shape[0], basis.shape[1]
    full = np.zeros((G, D, D), np.float32)
    full[:, :, :r] = basis
    return oracle.Fit(r, np.full(G, r, np.int32), full, mu, sigma)


def test_fit_per_slot_matches_oracle(torch):
    B, rank, groups = 3, 14, 2
    ws = _workloads(B, 2, groups, rank, True, 70)
    lens = np.array([96, 41, 70], np.int32)
    k, v = _rows(ws, 0, 96), _rows(ws, 1, 96)
    cache = _cache(torch, ws[0], B, 96, rank)
    cache.fit(_dev(torch, k), _dev(torch, v), lens)
    hpg = 1
    bases = []
    for b in range(B):
        for tensor, x in ((0, k), (1, v)):
            f = oracle.fit(x[b:b + 1], lens[b:b + 1], groups, rank=rank)
            r, basis, mu, sigma = cache.get_basis(tensor, seq=b)
            assert r == f.r == rank
            np.testing.assert_allclose(mu, f.mu, atol=1e-5)
            np.testing.assert_allclose(sigma[:, :rank], f.sigma[:, :rank], rtol=1e-3)
            for g in range(groups):
                rows = np.concatenate([x[b, h, :lens[b]] for h in range(g * hpg, (g + 1) * hpg)])
                assert abs(_energy(rows, f.mu[g], basis[g]) - _energy(rows, f.mu[g], f.V(g))) <= 1e-4
            if tensor == 0:
                bases.append(basis)
    # the slots' key subspaces differ (different planted subspaces)
    assert np.abs(np.abs(bases[0][0].T @ bases[1][0]) - np.eye(rank)).max() > 0.1
    with pytest.raises(Exception):
        cache.get_basis(0)          # no shared basis in this mode


CASES = [
    dict(gqa=4, rank=16, vq=True, bf16=False, schedule=None),
    dict(gqa=3, rank=24, vq=False, bf16=False, schedule=None),
    dict(gqa=2, rank=20, vq=True, bf16=True, schedule=None),
    dict(gqa=4, rank=32, vq=True, bf16=False, schedule=(8, 4, 2, 1, 1, 0, 0, 0)),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_codes_decode_prefill_per_slot(torch, case):
    gqa, rank, vq, bf16, sched = case["gqa"], case["rank"], case["vq"], case["bf16"], case["schedule"]
    B, groups, total = 4, 2, 100
    ws = _workloads(B, gqa, groups, rank, vq, 80 + rank)
    lens = np.array([70, 33, 5, 96], np.int32)
    k, v = _rows(ws, 0, total, bf16), _rows(ws, 1, total, bf16)
    cache = _cache(torch, ws[0], B, total, rank, input_dtype="bf16" if bf16 else "fp16", bit_schedule=sched)
    layers = []
    for b in range(B):
        fk = oracle.fit(k[b:b + 1, :, :96], lens[b:b + 1], groups, rank=rank, bf16=bf16)
        fv = oracle.fit(v[b:b + 1, :, :96], lens[b:b + 1], groups, rank=rank, bf16=bf16)
        cache.set_basis(0, fk.bases(), fk.mu, seq=b)
        cache.set_basis(1, fv.bases(), fv.mu, seq=b)
        layers.append(oracle.OracleLayer(128, 2 * gqa, 2, groups, fk, fv, quantize_values=vq, bf16=bf16,
                                         schedule=sched))
    cache.encode_append(_bdev(torch, k[:, :, :96], bf16), _bdev(torch, v[:, :, :96], bf16), n_new=lens)
    kt = np.stack([k[b, :, lens[b]:lens[b] + 1] for b in range(B)])
    vt = np.stack([v[b, :, lens[b]:lens[b] + 1] for b in range(B)])
    cache.encode_append(_bdev(torch, kt, bf16), _bdev(torch, vt, bf16))
    q = np.concatenate([synth.queries(w, b, 1, bf16=bf16) for b, w in enumerate(ws)])
    out = _out(cache.decode_attend(_bdev(torch, q, bf16)), bf16)
    for b in range(B):
        n = int(lens[b]) + 1
        layer = layers[b]
        _state_equal(cache, layer, k[b, :, :n], v[b, :, :n], b)
        ks = [layer.encode_head(k[b, h, :n], h, 0) for h in range(2)]
        vs = [layer.encode_head(v[b, h, :n], h, 1) for h in range(2)]
        _check_attention(out[b], layer.attend(ks, vs, q[b]), f"decode row {b}")
        m = min(40, n)
        qp = synth.prefill_queries(ws[b], b, n, bf16=bf16)[:, n - m:]
        pre = _out(cache.prefill_attend(_bdev(torch, qp[None], bf16), seq_ids=[b], n_q=[m]), bf16)[0]
        _check_attention(pre, layer.prefill_attend(ks, vs, qp, np.arange(n - m, n)), f"prefill row {b}")


def test_refit_some_slots_keeps_the_others(torch):
    B, rank, groups = 3, 12, 1
    ws = _workloads(B, 2, groups, rank, True, 90)
    lens = np.array([64, 50, 77], np.int32)
    k, v = _rows(ws, 0, 96), _rows(ws, 1, 96)
    cache = _cache(torch, ws[0], B, 96, rank)
    cache.fit(_dev(torch, k), _dev(torch, v), lens)
    cache.encode_append(_dev(torch, k), _dev(torch, v), n_new=lens)
    q = np.concatenate([synth.queries(w, b, 1) for b, w in enumerate(ws)])
    before = cache.decode_attend(_dev(torch, q[1:2]), seq_ids=[1]).cpu().numpy()
    keep = [cache.read_codes(1, h, t) for h in range(2) for t in (0, 1)]
    kb1 = cache.get_basis(0, seq=1)[1]
    # re-fit slots 2 and 0 from other data (rows swapped)
    k2, v2 = _rows(list(reversed(ws)), 0, 96), _rows(list(reversed(ws)), 1, 96)
    cache.fit(_dev(torch, k2[[0, 2]]), _dev(torch, v2[[0, 2]]), [60, 33], seq_ids=[2, 0])
    assert cache.seq_len(0) == 0 and cache.seq_len(2) == 0 and cache.seq_len(1) == lens[1]
    np.testing.assert_array_equal(cache.get_basis(0, seq=1)[1], kb1)
    f2 = oracle.fit(k2[0:1], [60], groups, rank=rank)
    assert np.allclose(cache.get_basis(0, seq=2)[2], f2.mu, atol=1e-5)
    for (a, ta), (c, tc) in zip(keep, [cache.read_codes(1, h, t) for h in range(2) for t in (0, 1)]):
        assert np.array_equal(a, c) and np.array_equal(ta.view(np.uint32), tc.view(np.uint32))
    after = cache.decode_attend(_dev(torch, q[1:2]), seq_ids=[1]).cpu().numpy()
    assert np.array_equal(after.view(np.uint16), before.view(np.uint16))
    # re-fitted slots take new tokens under their new bases
    cache.encode_append(_dev(torch, k2[[0, 2], :, :60]), _dev(torch, v2[[0, 2], :, :60]), seq_ids=[2, 0],
                        n_new=[60, 33])
    # (the codes are checked under the slot's installed basis: fits agree
    # with the oracle's only to the energy tolerance)
    layer = oracle.OracleLayer(128, 4, 2, groups, _fit_of_slot(cache, 0, 0), _fit_of_slot(cache, 0, 1))
    _state_equal(cache, layer, k2[2, :, :33], v2[2, :, :33], 0)
    rows = np.concatenate([k2[2, h, :33] for h in range(2)])
    f = oracle.fit(k2[2:3], [33], groups, rank=rank)
    assert abs(_energy(rows, f.mu[0], layer.fit[0].V(0)) - _energy(rows, f.mu[0], f.V(0))) <= 1e-4


def test_export_import_carries_bases(torch):
    B, rank, groups = 2, 16, 2
    ws = _workloads(B, 2, groups, rank, True, 95)
    lens = np.array([75, 40], np.int32)
    k, v = _rows(ws, 0, 96), _rows(ws, 1, 96)
    src = _cache(torch, ws[0], B, 96, rank)
    src.fit(_dev(torch, k), _dev(torch, v), lens)
    src.encode_append(_dev(torch, k), _dev(torch, v), n_new=lens)
    img = src.export_seq(0)
    dst = _cache(torch, ws[0], 3, 96, rank)
    # slot 2 of dst holds other bases and tokens first
    dst.fit(_dev(torch, k[1:2]), _dev(torch, v[1:2]), [40], seq_ids=[2])
    dst.encode_append(_dev(torch, k[1:2]), _dev(torch, v[1:2]), seq_ids=[2], n_new=[40])
    dst.import_seq(2, img)
    assert dst.seq_len(2) == 75
    for t in (0, 1):
        a, c = src.get_basis(t, seq=0), dst.get_basis(t, seq=2)
        np.testing.assert_array_equal(a[1], c[1])
        np.testing.assert_array_equal(a[2], c[2])
        for h in range(2):
            ra, ta = src.read_codes(0, h, t)
            rb, tb = dst.read_codes(2, h, t)
            assert np.array_equal(ra, rb) and np.array_equal(ta.view(np.uint32), tb.view(np.uint32))
    q = synth.queries(ws[0], 0, 1)
    a = src.decode_attend(_dev(torch, q), seq_ids=[0]).cpu().numpy()
    c = dst.decode_attend(_dev(torch, q), seq_ids=[2]).cpu().numpy()
    assert np.array_equal(a.view(np.uint16), c.view(np.uint16))
    # a corrupted basis byte is caught by the hash
    bad = bytearray(img)
    bad[64 + 5] ^= 0x40
    with pytest.raises(Exception):
        dst.import_seq(1, bytes(bad))


def test_fit_tiny_prompts(torch):
    """Per-sequence fits of 1- to 3-token prompts (a zero or rank-deficient
    scatter matrix): the fit converges, the bases are orthonormal, the mean
    is the prompt's mean, and codes and decode match the oracle under the
    installed bases."""
    B, rank, groups = 3, 8, 1
    ws = _workloads(B, 2, groups, rank, True, 97)
    lens = np.array([1, 2, 3], np.int32)
    k, v = _rows(ws, 0, 8), _rows(ws, 1, 8)
    cache = _cache(torch, ws[0], B, 8, rank)
    cache.fit(_dev(torch, k), _dev(torch, v), lens)
    cache.encode_append(_dev(torch, k), _dev(torch, v), n_new=lens + 1)
    q = np.concatenate([synth.queries(w, b, 1) for b, w in enumerate(ws)])
    out = cache.decode_attend(_dev(torch, q)).cpu().numpy()
    for b in range(B):
        for tensor, x in ((0, k), (1, v)):
            r, basis, mu, _ = cache.get_basis(tensor, seq=b)
            np.testing.assert_allclose(basis[0].T.astype(np.float64) @ basis[0], np.eye(r), atol=1e-5)
            rows = np.concatenate([x[b, h, :lens[b]] for h in range(2)]).astype(np.float64)
            np.testing.assert_allclose(mu[0], rows.mean(axis=0), atol=1e-5)
        layer = oracle.OracleLayer(128, 4, 2, groups, _fit_of_slot(cache, b, 0), _fit_of_slot(cache, b, 1))
        n = int(lens[b]) + 1
        _state_equal(cache, layer, k[b, :, :n], v[b, :, :n], b)
        ks = [layer.encode_head(k[b, h, :n], h, 0) for h in range(2)]
        vs = [layer.encode_head(v[b, h, :n], h, 1) for h in range(2)]
        _check_attention(out[b], layer.attend(ks, vs, q[b]), f"decode row {b}")


def test_slots_without_bases_are_refused(torch):
    from rank_latent_kv_amd.palu import PaluError
    ws = _workloads(2, 2, 1, 8, True, 99)
    k, v = _rows(ws, 0, 40), _rows(ws, 1, 40)
    cache = _cache(torch, ws[0], 2, 40, 8)
    cache.fit(_dev(torch, k[:1]), _dev(torch, v[:1]), [40], seq_ids=[0])
    cache.encode_append(_dev(torch, k[:1]), _dev(torch, v[:1]), seq_ids=[0])
    for call in (lambda: cache.encode_append(_dev(torch, k[1:]), _dev(torch, v[1:]), seq_ids=[1]),
                 lambda: cache.decode_attend(_dev(torch, synth.queries(ws[1], 1, 1)), seq_ids=[1]),
                 lambda: cache.read_codes(1, 0, 0)):
        with pytest.raises(PaluError) as ei:
            call()
        assert ei.value.code == 3                       # PALU_ERR_NOT_FITTED
    st = cache.stats()
    assert st["tokens"] == 40 and st["r_k"] == 8
