"""GPU parity with bf16 inputs (input_dtype = bf16): K, V and q arrive as
bf16 and outputs leave as bf16, with no fp16 cast of the raw inputs.

  * fit: identical rank and captured energy within 1e-4 of the oracle's;
  * codes and tails bit-exact against the oracle encode (bf16 widening);
  * decode and prefill attention within 2e-3 + 1e-2 |ref| of the oracle;
  * keys whose raw values lie beyond the fp16 range (a channel mean of
    1e5): codes exact, attention finite and within tolerance; queries of
    very different magnitudes (the per-row rescale into the fp16 MFMA).
"""
import numpy as np
import pytest

import oracle
from rank_latent_kv_amd import synth

from test_gpu_parity import ATOL, RTOL, _energy

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    if not _t.cuda.is_available():
        pytest.skip("no GPU")
    return _t


def _bdev(torch, bits):
    """bf16 bit patterns (uint16) -> a bf16 CUDA tensor holding them."""
    t = torch.from_numpy(np.array(bits, dtype=np.uint16).view(np.int16)).cuda()
    return t.view(torch.bfloat16)


def _bits(t):
    return t.cpu().view(__import__("torch").int16).numpy().view(np.uint16)


def _cache(w, max_seq_len, rank=None):
    from rank_latent_kv_amd.palu import LatentKVCache
    return LatentKVCache(w.head_dim, w.n_kv_heads, w.n_q_heads, w.n_head_groups, w.batch, max_seq_len,
                         rank=(w.rank or 0) if rank is None else rank, energy_threshold=w.energy,
                         quantize_values=w.quantize_values, input_dtype="bf16")


def _check(got_bits, ref, what):
    got = oracle.bf16_to_float(got_bits).astype(np.float64)
    assert np.all(np.isfinite(got)), what
    err = np.abs(got - ref)
    excess = np.max(err - (ATOL + RTOL * np.abs(ref)))
    assert excess <= 0, f"{what}: max excess {excess:.3e}, max abs err {err.max():.3e}"


def _state_equal(cache, layer, xk, xv, slot):
    for tensor, x in ((0, xk), (1, xv)):
        for h in range(x.shape[0]):
            st = layer.encode_head(x[h], h, tensor)
            rec, tail = cache.read_codes(slot, h, tensor)
            if "fp16" in st:
                continue
            assert np.array_equal(rec, st["records"]), (slot, h, tensor)
            assert np.array_equal(tail.view(np.uint32), st["tail"].view(np.uint32)), (slot, h, tensor)


def test_fit_matches_oracle(torch):
    w = synth.small_workload(batch=2, n_q_heads=8, n_kv_heads=4, n_head_groups=2, prefill=300,
                             rank=0, seed=61)
    lens = np.array([300, 170], np.int32)
    k = synth.batch_kv(w, 0, 300, bf16=True)
    v = synth.batch_kv(w, 1, 300, bf16=True)
    cache = _cache(w, 300)
    cache.fit(_bdev(torch, k), _bdev(torch, v), lens)
    hpg = 2
    for tensor, x in ((0, k), (1, v)):
        f = oracle.fit(x, lens, 2, rank=0, tau=w.energy, bf16=True)
        r, basis, mu, _ = cache.get_basis(tensor)
        assert r == f.r, (tensor, r, f.r)
        xf = oracle.bf16_to_float(x)
        for g in range(2):
            rows = np.concatenate([xf[b, h, :lens[b]] for b in range(2) for h in range(g * hpg, (g + 1) * hpg)])
            assert abs(_energy(rows, f.mu[g], basis[g]) - _energy(rows, f.mu[g], f.V(g))) <= 1e-4
            np.testing.assert_allclose(mu[g], f.mu[g], atol=1e-5)


# ranks 27 and 40 take the encode projection's runtime-stride chunks (a
# width rounded up to 4; two chunks of 32 and 8 channels)
@pytest.mark.parametrize("vq,rank", [(True, 16), (False, 16), (True, 27), (True, 40)])
def test_encode_decode_prefill(torch, vq, rank):
    lens = np.array([45, 96, 7], np.int32)
    w = synth.small_workload(batch=3, n_q_heads=8, n_kv_heads=2, n_head_groups=1, prefill=96,
                             rank=rank, quantize_values=vq, seed=62)
    total = 100
    k = synth.batch_kv(w, 0, total, bf16=True)
    v = synth.batch_kv(w, 1, total, bf16=True)
    fk = oracle.fit(k[:, :, :96], lens, 1, rank=rank, tau=w.energy, bf16=True)
    fv = oracle.fit(v[:, :, :96], lens, 1, rank=rank, tau=w.energy, bf16=True)
    cache = _cache(w, total)
    cache.set_basis(0, fk.bases(), fk.mu)
    cache.set_basis(1, fv.bases(), fv.mu)
    layer = oracle.OracleLayer(128, 8, 2, 1, fk, fv, quantize_values=vq, bf16=True)
    cache.encode_append(_bdev(torch, k[:, :, :96]), _bdev(torch, v[:, :, :96]), n_new=lens)
    # one decode step per row
    kt = np.stack([k[b, :, lens[b]:lens[b] + 1] for b in range(3)])
    vt = np.stack([v[b, :, lens[b]:lens[b] + 1] for b in range(3)])
    cache.encode_append(_bdev(torch, kt), _bdev(torch, vt))
    q = synth.queries(w, 0, 3, bf16=True)                       # [3, Hq, D] bf16 bits
    out = cache.decode_attend(_bdev(torch, q))
    assert out.dtype == torch.bfloat16
    out = _bits(out)
    for b in range(3):
        n = int(lens[b]) + 1
        _state_equal(cache, layer, k[b, :, :n], v[b, :, :n], b)
        ks = [layer.encode_head(k[b, h, :n], h, 0) for h in range(2)]
        vs = [layer.encode_head(v[b, h, :n], h, 1) for h in range(2)]
        _check(out[b], layer.attend(ks, vs, q[b]), f"decode row {b}")
        # prefill attention of the last 20 positions (or all of them)
        m = min(20, n)
        qp = synth.prefill_queries(w, b, n, bf16=True)[:, n - m:]
        pre = _bits(cache.prefill_attend(_bdev(torch, qp[None]), seq_ids=[b], n_q=[m]))[0]
        _check(pre, layer.prefill_attend(ks, vs, qp, np.arange(n - m, n)), f"prefill row {b}")


def test_keys_beyond_fp16_range_and_query_magnitudes(torch):
    lens = np.array([80, 33], np.int32)
    w = synth.small_workload(batch=2, n_q_heads=4, n_kv_heads=2, n_head_groups=1, prefill=80,
                             rank=12, seed=63)
    kf = oracle.bf16_to_float(synth.batch_kv(w, 0, 80, bf16=True))
    kf[..., 7] += 1.0e5                                          # raw keys far beyond 65504
    k = synth.to_bf16_bits(kf)
    v = synth.batch_kv(w, 1, 80, bf16=True)
    assert np.abs(oracle.bf16_to_float(k)).max() > 65504
    fk = oracle.fit(k, lens, 1, rank=12, tau=w.energy, bf16=True)
    fv = oracle.fit(v, lens, 1, rank=12, tau=w.energy, bf16=True)
    cache = _cache(w, 80)
    cache.set_basis(0, fk.bases(), fk.mu)
    cache.set_basis(1, fv.bases(), fv.mu)
    layer = oracle.OracleLayer(128, 4, 2, 1, fk, fv, bf16=True)
    cache.encode_append(_bdev(torch, k), _bdev(torch, v), n_new=lens)
    qf = oracle.bf16_to_float(synth.queries(w, 0, 2, bf16=True))
    qf[0, 1] *= 2.0 ** -20                                      # tiny query row
    qf[1, 2] *= 2.0 ** 6                                        # large query row
    q = synth.to_bf16_bits(qf)
    out = _bits(cache.decode_attend(_bdev(torch, q)))
    for b in range(2):
        n = int(lens[b])
        _state_equal(cache, layer, k[b, :, :n], v[b, :, :n], b)
        ks = [layer.encode_head(k[b, h, :n], h, 0) for h in range(2)]
        vs = [layer.encode_head(v[b, h, :n], h, 1) for h in range(2)]
        _check(out[b], layer.attend(ks, vs, q[b]), f"decode row {b}")
        qp = np.ascontiguousarray(np.broadcast_to(q[b][:, None, :], (4, 1, 128)))
        pre = _bits(cache.prefill_attend(_bdev(torch, qp[None]), seq_ids=[b], n_q=[1]))[0]
        _check(pre, layer.prefill_attend(ks, vs, qp, [n - 1]), f"prefill row {b}")
    # the GPU fit on these keys stays finite and keeps the large channel in its mean
    cache2 = _cache(w, 80)
    cache2.fit(_bdev(torch, k), _bdev(torch, v), lens)
    _, basis, mu, _ = cache2.get_basis(0)
    assert np.all(np.isfinite(basis)) and abs(mu[0][7] - fk.mu[0][7]) < 1.0


def test_wrong_dtype_rejected(torch):
    w = synth.small_workload(batch=1, n_q_heads=4, n_kv_heads=2, prefill=40, rank=8)
    cache = _cache(w, 40)
    k16 = torch.zeros((1, 2, 40, 128), dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError):
        cache.fit(k16, k16)
