"""GPU: save / restore of sequence slots (palu_export_seq / palu_import_seq).

A slot exported from one cache and imported into another cache that holds
the same basis must hold the same records and tails (bitwise), give bitwise
identical decode outputs for the same call, match the oracle's encode of the
sequence, and keep doing so as tokens are appended after the import (the
import normalises the double-buffered tail to buffer 0).  Malformed or
mismatched images are rejected and leave the slot unchanged.
"""
import struct

import numpy as np
import pytest

import oracle
from rank_latent_kv_amd import synth

from test_gpu_parity import _cache, _check_attention, _compare_state, _dev

pytestmark = pytest.mark.gpu

HEADER = 64


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    if not _t.cuda.is_available():
        pytest.skip("no GPU")
    return _t


def _setup(torch, vq, lens, extra, max_batch=None, max_seq_len=None, rank=20, groups=2, seed=57):
    w = synth.small_workload(batch=len(lens), n_q_heads=8, n_kv_heads=4, n_head_groups=groups,
                             prefill=int(max(lens)), steps=1, rank=rank, seed=seed,
                             quantize_values=vq)
    total = int(max(lens)) + extra
    k_all = synth.batch_kv(w, 0, total)
    v_all = synth.batch_kv(w, 1, total)
    S = int(max(lens))
    fk = oracle.fit(k_all[:, :, :S], np.asarray(lens, np.int32), groups, rank=rank, tau=w.energy)
    fv = oracle.fit(v_all[:, :, :S], np.asarray(lens, np.int32), groups, rank=rank, tau=w.energy)
    layer = oracle.OracleLayer(w.head_dim, w.n_q_heads, w.n_kv_heads, groups, fk, fv,
                               quantize_values=vq)

    def make(mb=None, msl=None):
        c = _cache(torch, w, msl or max_seq_len or total, max_batch=mb or max_batch or len(lens))
        c.set_basis(0, fk.bases(), fk.mu)
        c.set_basis(1, fv.bases(), fv.mu)
        return c

    return w, k_all, v_all, layer, make


def _append(torch, cache, k_all, v_all, pos, n_new, slots):
    c = int(max(n_new))
    B, H, _, D = k_all.shape
    kc = np.zeros((B, H, c, D), np.float16)
    vc = np.zeros_like(kc)
    for b in range(B):
        kc[b, :, :n_new[b]] = k_all[b, :, pos[b]:pos[b] + n_new[b]]
        vc[b, :, :n_new[b]] = v_all[b, :, pos[b]:pos[b] + n_new[b]]
    cache.encode_append(_dev(torch, kc), _dev(torch, vc), seq_ids=np.asarray(slots, np.int32),
                        n_new=np.asarray(n_new, np.int32))


@pytest.mark.parametrize("vq", [True, False])
def test_round_trip_bitwise_and_continued_decode(torch, vq):
    # lengths: tail-only, exact multiple of 32, partial groups; the 30-token
    # append moves slot 0 (37 -> 67) across a group boundary with a partial
    # group on both sides, so its tail sits in buffer 1 when exported
    lens = [37, 96, 5, 64]
    first = [30, 1, 0, 31]
    then = [40, 33, 7, 1]
    w, k_all, v_all, layer, make = _setup(torch, vq, lens, extra=80)
    src = make()
    B = len(lens)
    S = int(max(lens))
    src.encode_append(_dev(torch, k_all[:, :, :S]), _dev(torch, v_all[:, :, :S]),
                      n_new=np.asarray(lens, np.int32))
    pos = np.asarray(lens)
    _append(torch, src, k_all, v_all, pos, first, range(B))
    pos = pos + np.asarray(first)
    torch.cuda.synchronize()

    # destination: more slots; target slots already hold other sequences
    dst = make(mb=B + 2)
    perm = [4, 0, 5, 2]
    junk = [50, 3, 0, 70, 33, 12]
    _append(torch, dst, k_all[[0, 1, 2, 3, 0, 1]], v_all[[0, 1, 2, 3, 0, 1]],
            np.zeros(6, np.int64), junk, range(6))
    images = []
    for b in range(B):
        img = src.export_seq(b)
        magic, version = struct.unpack_from("<II", img, 0)
        assert (magic, version) == (0x564B4C50, 1)
        assert struct.unpack_from("<i", img, 48)[0] == pos[b]
        images.append(img)
        dst.import_seq(perm[b], img)
        assert dst.seq_len(perm[b]) == pos[b]
    torch.cuda.synchronize()

    for b in range(B):
        # the imported slot exports to the same bytes
        assert dst.export_seq(perm[b]) == images[b]
        for t in (0, 1):
            for h in range(w.n_kv_heads):
                ra, ta = src.read_codes(b, h, t)
                rb, tb = dst.read_codes(perm[b], h, t)
                assert np.array_equal(ra, rb) and np.array_equal(ta.view(np.uint32), tb.view(np.uint32))
        _compare_state(dst, layer, (k_all[b, :, :pos[b]], v_all[b, :, :pos[b]]), perm[b])

    q = np.stack([synth.queries(w, b, 1)[0] for b in range(B)])
    oa = src.decode_attend(_dev(torch, q)).cpu().numpy()
    ob = dst.decode_attend(_dev(torch, q), seq_ids=np.asarray(perm, np.int32)).cpu().numpy()
    assert np.array_equal(oa.view(np.uint16), ob.view(np.uint16))

    # keep going on both caches: tails continue correctly from buffer 0
    _append(torch, src, k_all, v_all, pos, then, range(B))
    _append(torch, dst, k_all, v_all, pos, then, perm)
    pos = pos + np.asarray(then)
    torch.cuda.synchronize()
    oa = src.decode_attend(_dev(torch, q)).cpu().numpy()
    ob = dst.decode_attend(_dev(torch, q), seq_ids=np.asarray(perm, np.int32)).cpu().numpy()
    assert np.array_equal(oa.view(np.uint16), ob.view(np.uint16))
    for b in range(B):
        xs = (k_all[b, :, :pos[b]], v_all[b, :, :pos[b]])
        _compare_state(dst, layer, xs, perm[b])
        ks = [layer.encode_head(xs[0][h], h, 0) for h in range(w.n_kv_heads)]
        vs = [layer.encode_head(xs[1][h], h, 1) for h in range(w.n_kv_heads)]
        _check_attention(ob[b], layer.attend(ks, vs, q[b]), f"imported slot {perm[b]}")


def test_export_sizes_and_empty_slot(torch):
    lens = [37, 64]
    w, k_all, v_all, layer, make = _setup(torch, True, lens, extra=0)
    c = make()
    c.encode_append(_dev(torch, k_all), _dev(torch, v_all), n_new=np.asarray(lens, np.int32))
    torch.cuda.synchronize()
    for b, n in enumerate(lens):
        img = c.export_seq(b)
        size = HEADER
        for t in (0, 1):
            r = layer.fit[t].r
            words = c.read_codes(b, 0, t)[0].shape[1]
            size += w.n_kv_heads * ((n // 32) * words * 4 + (n % 32) * r * 4)
        assert len(img) == size
    # an empty image (len 0, header only) empties a slot
    empty = make(mb=1)
    img0 = empty.export_seq(0)
    assert len(img0) == HEADER
    c.import_seq(1, img0)
    assert c.seq_len(1) == 0
    assert c.export_seq(1) == img0


def test_import_rejects_mismatches(torch):
    from rank_latent_kv_amd.palu import PaluError
    lens = [40, 33]
    w, k_all, v_all, layer, make = _setup(torch, True, lens, extra=0)
    c = make()
    c.encode_append(_dev(torch, k_all), _dev(torch, v_all), n_new=np.asarray(lens, np.int32))
    torch.cuda.synchronize()
    img = c.export_seq(0)
    before = c.export_seq(1)

    def code_of(fn):
        with pytest.raises(PaluError) as ei:
            fn()
        return ei.value.code

    bad_magic = bytearray(img)
    bad_magic[0] ^= 1
    assert code_of(lambda: c.import_seq(1, bytes(bad_magic))) == 1
    bad_version = bytearray(img)
    struct.pack_into("<I", bad_version, 4, 2)
    assert code_of(lambda: c.import_seq(1, bytes(bad_version))) == 1
    assert code_of(lambda: c.import_seq(1, img[:-4])) == 1          # truncated payload
    assert code_of(lambda: c.import_seq(1, img + b"\0" * 4)) == 1   # trailing bytes
    assert code_of(lambda: c.import_seq(1, img[:HEADER - 1])) == 1  # shorter than a header
    assert code_of(lambda: c.import_seq(7, img)) == 4               # slot out of range
    bad_hash = bytearray(img)
    bad_hash[52] ^= 0x80
    assert code_of(lambda: c.import_seq(1, bytes(bad_hash))) == 1
    # a slot saved under another basis (same shapes, other rank)
    _, k2, v2, _, make2 = _setup(torch, True, lens, extra=0, rank=12, seed=58)
    other = make2()
    other.encode_append(_dev(torch, k2), _dev(torch, v2), n_new=np.asarray(lens, np.int32))
    torch.cuda.synchronize()
    assert code_of(lambda: c.import_seq(1, other.export_seq(0))) == 1
    # same basis, but the length does not fit the destination's capacity
    small = make(mb=1, msl=36)
    assert code_of(lambda: small.import_seq(0, img)) == 4
    # every failed import left slot 1 as it was
    assert c.export_seq(1) == before
    assert c.seq_len(1) == lens[1]
