"""The allocation-free decode entry point (split partials in the library's
static device array) against palu_decode_attend on the same cache: two calls
in a row, the second with fewer rows and a different slot set, outputs equal
bit for bit and within the attention tolerance of the oracle; a launch whose
partials exceed the array is refused before any device work."""
import numpy as np
import pytest

import oracle
from rank_latent_kv_amd import synth

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-3, 1e-2


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    if not _t.cuda.is_available():
        pytest.skip("no GPU")
    return _t


def _dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def test_noalloc_matches_decode_attend_twice(torch):
    from rank_latent_kv_amd.palu import LatentKVCache
    w = synth.small_workload(batch=5, n_q_heads=16, n_kv_heads=4, n_head_groups=2, prefill=700,
                             steps=1, rank=12, seed=808)
    lens = np.array([700, 33, 415, 96, 1], np.int32)
    S = int(lens.max())
    k, v = synth.batch_kv(w, 0, S), synth.batch_kv(w, 1, S)
    fk = oracle.fit(k, lens, 2, rank=12)
    fv = oracle.fit(v, lens, 2, rank=12)
    cache = LatentKVCache(128, 4, 16, 2, 5, S, rank=12)
    cache.set_basis(0, fk.bases(), fk.mu)
    cache.set_basis(1, fv.bases(), fv.mu)
    cache.encode_append(_dev(torch, k), _dev(torch, v), n_new=lens)
    layer = oracle.OracleLayer(128, 16, 4, 2, fk, fv)
    q = synth.queries(w, 0, 5)                       # [5, 16, 128]
    for rows in ([0, 1, 2, 3, 4], [3, 0]):           # second call: fewer rows
        qd = _dev(torch, q[:len(rows)])
        ref_out = cache.decode_attend(qd, seq_ids=rows)
        out = torch.full_like(qd, float("nan"))
        cache.decode_attend_noalloc(qd, out, seq_ids=rows)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.array_equal(got.view(np.uint16), ref_out.cpu().numpy().view(np.uint16)), rows
        for i, slot in enumerate(rows):
            n = int(lens[slot])
            ks = [layer.encode_head(k[slot, h, :n], h, 0) for h in range(4)]
            vs = [layer.encode_head(v[slot, h, :n], h, 1) for h in range(4)]
            ref = layer.attend(ks, vs, q[i])
            err = np.abs(got[i].astype(np.float64) - ref)
            assert np.all(err <= ATOL + RTOL * np.abs(ref)), (rows, slot, err.max())


def test_noalloc_refuses_partials_beyond_the_array(torch):
    from rank_latent_kv_amd.palu import LatentKVCache, PaluError
    # 64 rows x 32 query heads x 128 splits (one group each) x 34 floats > 16 MiB
    cache = LatentKVCache(128, 8, 32, 8, 64, 4096, rank=32, split_groups=1)
    basis = np.zeros((8, 128, 32), np.float32)
    basis[:, np.arange(32), np.arange(32)] = 1.0
    mu = np.zeros((8, 128), np.float32)
    cache.set_basis(0, basis, mu)
    cache.set_basis(1, basis, mu)
    x = torch.zeros((64, 8, 4096, 128), dtype=torch.float16, device="cuda")
    cache.encode_append(x, x)
    q = torch.zeros((64, 32, 128), dtype=torch.float16, device="cuda")
    out = torch.zeros_like(q)
    with pytest.raises(PaluError) as ei:
        cache.decode_attend_noalloc(q, out)
    assert ei.value.code == 2
    torch.cuda.synchronize()
    assert not out.any()                                 # nothing was launched
    cache.decode_attend_noalloc(q[:8].contiguous(), out[:8])   # 8 rows fit
    torch.cuda.synchronize()
