"""A captured decode step replays correctly for later steps: palu_decode_step
(one-token append + decode attention, lengths in device memory) is captured
once in a HIP graph and replayed with new inputs copied in between; every
replay's output matches the oracle at that step's length, and after
palu_sync_lengths the lengths and stored codes match the oracle encode of all
appended tokens.  Also: the eager step equals encode_append + decode_attend
bit for bit."""
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


def _setup(torch, lens, steps, rank=12, seed=515, quantize_values=True):
    from rank_latent_kv_amd.palu import LatentKVCache
    lens = np.asarray(lens, np.int32)
    B = len(lens)
    w = synth.small_workload(batch=B, n_q_heads=8, n_kv_heads=4, n_head_groups=2, prefill=int(lens.max()),
                             steps=steps, rank=rank, seed=seed, quantize_values=quantize_values)
    total = int(lens.max()) + steps
    k = synth.batch_kv(w, 0, total)
    v = synth.batch_kv(w, 1, total)
    S = int(lens.max())
    fk = oracle.fit(k[:, :, :S], lens, 2, rank=rank)
    fv = oracle.fit(v[:, :, :S], lens, 2, rank=rank)
    cache = LatentKVCache(128, 4, 8, 2, B, total, rank=rank, quantize_values=quantize_values)
    cache.set_basis(0, fk.bases(), fk.mu)
    cache.set_basis(1, fv.bases(), fv.mu)
    kd = torch.from_numpy(np.ascontiguousarray(k[:, :, :S])).cuda()
    vd = torch.from_numpy(np.ascontiguousarray(v[:, :, :S])).cuda()
    cache.encode_append(kd, vd, n_new=lens)
    layer = oracle.OracleLayer(128, 8, 4, 2, fk, fv, quantize_values=quantize_values)
    q = np.stack([synth.queries(w, b, steps) for b in range(B)], axis=1)   # [steps, B, Hq, D]
    return cache, layer, k, v, q


def _step_inputs(k, v, lens, step):
    B = len(lens)
    kn = np.stack([k[b, :, lens[b] + step:lens[b] + step + 1] for b in range(B)])
    vn = np.stack([v[b, :, lens[b] + step:lens[b] + step + 1] for b in range(B)])
    return kn, vn


def _check(layer, k, v, lens, step, q, got, what):
    for b in range(len(lens)):
        n = int(lens[b]) + step + 1
        ks = [layer.encode_head(k[b, h, :n], h, 0) for h in range(4)]
        vs = [layer.encode_head(v[b, h, :n], h, 1) for h in range(4)]
        ref = layer.attend(ks, vs, q[b])
        err = np.abs(got[b].astype(np.float64) - ref)
        assert np.all(err <= ATOL + RTOL * np.abs(ref)), (what, step, b, err.max())


@pytest.mark.parametrize("vq", [True, False])
def test_captured_step_replays(torch, vq):
    lens = np.array([100, 31, 64], np.int32)     # crosses group ends during the steps
    steps = 40
    cache, layer, k, v, q = _setup(torch, lens, steps, quantize_values=vq)
    B = len(lens)
    kn0, vn0 = _step_inputs(k, v, lens, 0)
    ks = torch.from_numpy(kn0).cuda()
    vs = torch.from_numpy(vn0).cuda()
    qs = torch.from_numpy(np.ascontiguousarray(q[0])).cuda()
    outs = torch.empty_like(qs)
    # step 0 eagerly (also initialises the kernels outside the capture)
    cache.decode_step(ks, vs, qs, outs)
    torch.cuda.synchronize()
    _check(layer, k, v, lens, 0, q[0], outs.cpu().numpy(), "eager")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cache.decode_step(ks, vs, qs, outs)
    for step in range(1, steps):
        kn, vn = _step_inputs(k, v, lens, step)
        ks.copy_(torch.from_numpy(kn))
        vs.copy_(torch.from_numpy(vn))
        qs.copy_(torch.from_numpy(np.ascontiguousarray(q[step])))
        g.replay()
        got = outs.cpu().numpy()                  # waits for the replay
        _check(layer, k, v, lens, step, q[step], got, "replay")
    cache.sync_lengths()
    for b in range(B):
        n = int(lens[b]) + steps
        assert cache.seq_len(b) == n
        for t, x in ((0, k), (1, v)):
            for h in range(4):
                st = layer.encode_head(x[b, h, :n], h, t)
                rec, tail = cache.read_codes(b, h, t)
                if "fp16" in st:
                    got = rec.view(np.uint16).reshape(st["fp16"].shape)
                    for j in range(got.shape[0]):
                        valid = min(32, n - 32 * j)
                        r = layer.fit[1].r
                        assert np.array_equal(got[j].reshape(r, 32)[:, :valid],
                                              st["fp16"][j].reshape(r, 32)[:, :valid]), (b, h, t, j)
                else:
                    assert np.array_equal(rec, st["records"]), (b, h, t)
                    assert np.array_equal(tail.view(np.uint32), st["tail"].view(np.uint32)), (b, h, t)
    # the host path continues from the synchronised lengths
    kn, vn = _step_inputs(k, v, lens, steps - 1)
    out = cache.decode_attend(qs)
    torch.cuda.synchronize()
    _check(layer, k, v, lens, steps - 1, q[steps - 1], out.cpu().numpy(), "after sync")


def test_step_equals_append_then_attend(torch):
    lens = np.array([70, 33], np.int32)
    cache_a, layer, k, v, q = _setup(torch, lens, 3, seed=616)
    cache_b, _, _, _, _ = _setup(torch, lens, 3, seed=616)
    for step in range(3):
        kn, vn = _step_inputs(k, v, lens, step)
        kd, vd = torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda()
        qd = torch.from_numpy(np.ascontiguousarray(q[step])).cuda()
        oa = cache_a.decode_step(kd, vd, qd, torch.empty_like(qd))
        cache_b.encode_append(kd, vd)
        ob = cache_b.decode_attend(qd)
        torch.cuda.synchronize()
        assert np.array_equal(oa.cpu().numpy().view(np.uint16), ob.cpu().numpy().view(np.uint16)), step
        assert cache_a.seq_len(0) == cache_b.seq_len(0) == lens[0] + step + 1


def test_step_refuses_full_and_repeated_slots(torch):
    from rank_latent_kv_amd.palu import PaluError
    lens = np.array([5, 5], np.int32)
    cache, layer, k, v, q = _setup(torch, lens, 1, seed=717)
    kn, vn = _step_inputs(k, v, lens, 0)
    kd, vd = torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda()
    qd = torch.from_numpy(np.ascontiguousarray(q[0])).cuda()
    with pytest.raises(PaluError) as ei:
        cache.decode_step(kd, vd, qd, torch.empty_like(qd), seq_ids=[1, 1])
    assert ei.value.code == 1
    cache.decode_step(kd, vd, qd, torch.empty_like(qd))          # fills both slots (capacity 6)
    with pytest.raises(PaluError) as ei:
        cache.decode_step(kd, vd, qd, torch.empty_like(qd))
    assert ei.value.code == 4
    torch.cuda.synchronize()
