"""C-ABI tests that need no GPU: the library loads, exports every entry point
include/palu.h declares, and rejects bad arguments on the host before any
device work (every error path below returns before a HIP call)."""
import ctypes
import os
import re

import pytest

from rank_latent_kv_amd import palu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "palu.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(palu_[a-z_]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert _declared() == sorted(palu.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(palu.LIB_PATH)
    for name in _declared():
        assert hasattr(L, name), name


def _cfg(**kw):
    cfg = palu.palu_config_default(128, 8, 32)
    for k, v in kw.items():
        setattr(cfg, k, v)
    return cfg


def test_config_defaults_follow_usage_section():
    cfg = palu.palu_config_default(128, 8, 32)
    assert (cfg.rank, cfg.n_head_groups, cfg.hi_bit, cfg.lo_bit, cfg.group_size,
            cfg.quantize_values, cfg.max_rank, cfg.split_groups, cfg.input_dtype) == (0, 4, 4, 2, 32, 1, 0, 0, 0)
    assert abs(cfg.energy_threshold - 0.90) < 1e-7 and abs(cfg.hi_fraction - 0.25) < 1e-7


@pytest.mark.parametrize("kw,code", [
    (dict(n_head_groups=3), 1),          # H % G != 0
    (dict(n_q_heads=12), 1),             # Hq % H != 0
    (dict(energy_threshold=0.0), 1),
    (dict(energy_threshold=1.5), 1),
    (dict(hi_fraction=-0.1), 1),
    (dict(rank=-1), 1),
    (dict(max_rank=129), 1),
    (dict(split_groups=-1), 1),
    (dict(quantize_values=2), 1),
    (dict(input_dtype=2), 1),
    (dict(head_dim=96), 2),              # kernels built for D = 128
    (dict(hi_bit=3), 2),
    (dict(lo_bit=5), 2),
    (dict(schedule_len=9), 1),
    (dict(schedule_len=-1), 1),
    (dict(group_size=64), 2),
    (dict(n_q_heads=8 * 16), 2),         # more than 8 query heads per kv head
])
def test_create_rejects_bad_config(kw, code):
    with pytest.raises(palu.PaluError) as ei:
        palu.palu_cache_create(_cfg(**kw), 4, 1024)
    assert ei.value.code == code
    assert palu.palu_last_error()


@pytest.mark.parametrize("sched,code", [((8, 4, 3), 2), ((0, 0), 1), ((0, 16), 2)])
def test_create_rejects_bad_schedule(sched, code):
    cfg = _cfg(schedule_len=len(sched))
    for i, b in enumerate(sched):
        cfg.bit_schedule[i] = b
    with pytest.raises(palu.PaluError) as ei:
        palu.palu_cache_create(cfg, 4, 1024)
    assert ei.value.code == code


def test_create_accepts_schedules_and_widths():
    for kw in (dict(hi_bit=8, lo_bit=1), dict(hi_bit=1, lo_bit=8)):
        h = palu.palu_cache_create(_cfg(**kw), 2, 64)
        palu.lib().palu_cache_destroy(h)
    cfg = _cfg(schedule_len=8)
    for i, b in enumerate((8, 4, 2, 1, 1, 0, 0, 0)):
        cfg.bit_schedule[i] = b
    h = palu.palu_cache_create(cfg, 2, 64)
    assert palu.palu_cache_required_bytes(h) > 0
    palu.lib().palu_cache_destroy(h)


def test_create_rejects_bad_sizes():
    for mb, ms in [(0, 10), (4, 0), (-1, 5)]:
        with pytest.raises(palu.PaluError) as ei:
            palu.palu_cache_create(_cfg(), mb, ms)
        assert ei.value.code == 1


def test_required_bytes_and_bind_validation():
    h = palu.palu_cache_create(_cfg(max_rank=32), 4, 1000)
    try:
        n = palu.palu_cache_required_bytes(h)
        assert n > 0 and n % 256 == 0
        # capacity covers records at max_rank: 4 slots * 8 heads * 32 groups *
        # (3*32 + 2*8) words * 4 bytes per tensor, plus the rest
        assert n > 2 * 4 * 8 * 32 * (3 * 32 + 2 * 8) * 4
        with pytest.raises(palu.PaluError) as ei:
            palu.palu_cache_bind(h, 0, n)
        assert ei.value.code == 1
        with pytest.raises(palu.PaluError) as ei:
            palu.palu_cache_bind(h, 4096, n - 1)          # too small
        assert ei.value.code == 1
        with pytest.raises(palu.PaluError) as ei:
            palu.palu_cache_bind(h, 4096 + 16, n)         # misaligned
        assert ei.value.code == 1
    finally:
        palu.palu_cache_destroy(h)


def test_calls_before_bind_or_fit_fail_cleanly():
    h = palu.palu_cache_create(_cfg(), 2, 256)
    try:
        with pytest.raises(palu.PaluError) as ei:
            palu.palu_fit(h, 1, 1, [16, 16], 2, 16, 0)
        assert ei.value.code == 5                          # not bound
        with pytest.raises(palu.PaluError) as ei:
            palu.palu_encode_append(h, 1, 1, None, None, 2, 1, 0)
        assert ei.value.code == 5
        # bind to a fake (never dereferenced) aligned address: everything
        # below fails validation before any device call
        palu.palu_cache_bind(h, 1 << 20, palu.palu_cache_required_bytes(h))
        with pytest.raises(palu.PaluError) as ei:
            palu.palu_encode_append(h, 1, 1, None, None, 2, 1, 0)
        assert ei.value.code == 3                          # not fitted
        with pytest.raises(palu.PaluError) as ei:
            palu.palu_decode_attend(h, 1, 1, None, 2, 0.0, 0)
        assert ei.value.code == 3
        with pytest.raises(palu.PaluError) as ei:
            palu.palu_get_stats(h)
        assert ei.value.code == 3
        for lens, B, S in [([17, 3], 2, 16), ([-1, 3], 2, 16), ([0, 0], 2, 16), ([4, 4, 4], 3, 16),
                           ([300, 3], 2, 300)]:
            with pytest.raises(palu.PaluError) as ei:
                palu.palu_fit(h, 1, 1, lens, B, S, 0)
            assert ei.value.code == 1, (lens, B, S)
        with pytest.raises(palu.PaluError) as ei:
            palu.palu_set_basis(h, 2, 4, [0.0] * (4 * 128 * 4), [0.0] * (4 * 128))
        assert ei.value.code == 1
        with pytest.raises(palu.PaluError) as ei:
            palu.palu_set_basis(h, 0, 0, [0.0], [0.0])
        assert ei.value.code == 1
        with pytest.raises(palu.PaluError) as ei:
            palu.palu_seq_len(h, 2)
        assert ei.value.code == 4
        assert palu.palu_seq_len(h, 1) == 0
    finally:
        palu.palu_cache_destroy(h)


def test_per_seq_basis_config_and_host_checks():
    with pytest.raises(palu.PaluError) as ei:
        palu.palu_cache_create(_cfg(per_seq_basis=1), 2, 64)      # energy rule: layout unknown
    assert ei.value.code == 2
    with pytest.raises(palu.PaluError) as ei:
        palu.palu_cache_create(_cfg(per_seq_basis=2, rank=8), 2, 64)
    assert ei.value.code == 1
    shared = palu.palu_cache_create(_cfg(rank=16), 3, 256)
    h = palu.palu_cache_create(_cfg(per_seq_basis=1, rank=16), 3, 256)
    one = palu.palu_cache_create(_cfg(per_seq_basis=1, rank=16), 1, 256)
    try:
        # the record layout is fixed at creation: rank 16 splits 4 channels
        # at 4 bits and 12 at 2 bits, plus 16 scale/zero words
        assert palu.palu_record_words(h, 0) == 4 * 4 + 12 * 2 + 16
        st = palu.palu_get_stats(h)
        assert (st.r_k, st.r_v, st.tokens, st.compressed_key_bytes) == (16, 16, 0, 0)
        assert palu.palu_cache_required_bytes(h) > palu.palu_cache_required_bytes(one)
        basis, mu = [0.0] * (4 * 128 * 16), [0.0] * (4 * 128)
        for c in (h, shared):
            palu.palu_cache_bind(c, 1 << 20, palu.palu_cache_required_bytes(c))
        calls = [
            (lambda: palu.palu_get_basis(h, 0, 4, 128), 1),              # no shared basis
            (lambda: palu.palu_set_basis(h, 0, 8, basis, mu), 1),        # rank fixed at 16
            (lambda: palu.palu_set_basis_seq(h, 3, 0, 16, basis, mu), 4),
            (lambda: palu.palu_set_basis_seq(h, 0, 0, 8, basis, mu), 1),
            (lambda: palu.palu_get_basis_seq(h, 0, 0, 4, 128), 3),
            (lambda: palu.palu_fit_seq(h, 1, 1, [0, 1], [4, 0], 2, 16, 0), 1),   # empty row
            (lambda: palu.palu_fit_seq(h, 1, 1, [1, 1], [4, 4], 2, 16, 0), 1),   # repeated slot
            (lambda: palu.palu_fit_seq(h, 1, 1, [0, 5], [4, 4], 2, 16, 0), 4),
            (lambda: palu.palu_encode_append(h, 1, 1, None, None, 2, 1, 0), 3),  # slots without bases
            (lambda: palu.palu_decode_attend(h, 1, 1, None, 2, 0.0, 0), 3),
            (lambda: palu.palu_export_bytes(h, 0), 3),
            (lambda: palu.palu_import_seq(h, 0, b"x" * 10), 1),
            (lambda: palu.palu_fit_seq(shared, 1, 1, [0], [4], 1, 16, 0), 1),   # shared-basis cache
            (lambda: palu.palu_set_basis_seq(shared, 0, 0, 16, basis, mu), 1),
            (lambda: palu.palu_get_basis_seq(shared, 0, 0, 4, 128), 1),
        ]
        for i, (call, code) in enumerate(calls):
            with pytest.raises(palu.PaluError) as ei:
                call()
            assert ei.value.code == code, (i, ei.value)
    finally:
        for c in (h, shared, one):
            palu.palu_cache_destroy(c)


# ------------------------------------------- binding checks before any call

def _host_cache(**kw):
    """A LatentKVCache-shaped object whose bound storage is a CPU tensor:
    every check below must raise before anything reaches the library."""
    import torch
    c = palu.LatentKVCache.__new__(palu.LatentKVCache)
    c.torch = torch
    c.cfg = _cfg(**kw)
    c.D, c.H, c.Hq, c.G = 128, 8, 32, 4
    c.max_batch, c.max_seq_len = 4, 64
    c.storage = torch.empty(0, dtype=torch.uint8)
    c.handle = None
    return c


def test_binding_rejects_bad_out_before_launch():
    import torch
    c = _host_cache()
    q = torch.zeros((2, 32, 128), dtype=torch.float16)
    bad_outs = [torch.zeros((1, 32, 128), dtype=torch.float16),        # too few rows
                torch.zeros((2, 32, 64), dtype=torch.float16),         # short rows
                torch.zeros((2, 32, 128), dtype=torch.float32),        # wrong type
                torch.zeros((2, 128, 32), dtype=torch.float16).transpose(1, 2)]   # not contiguous
    for out in bad_outs:
        with pytest.raises(ValueError):
            c.decode_attend(q, out=out)
    qp = torch.zeros((2, 32, 16, 128), dtype=torch.float16)
    for out in (torch.zeros((2, 32, 8, 128), dtype=torch.float16),
                torch.zeros((2, 32, 16, 128), dtype=torch.bfloat16)):
        with pytest.raises(ValueError):
            c.prefill_attend(qp, out=out)
    # the tile workspace: a uint8 device tensor (checked before any call)
    for ws in (torch.zeros(64, dtype=torch.uint8), torch.zeros(16, dtype=torch.float32), 1234):
        with pytest.raises(ValueError):
            c.prefill_attend(qp, workspace=ws)
    with pytest.raises(ValueError):
        c.decode_attend(torch.zeros((32, 128), dtype=torch.float16))  # missing batch dim
    with pytest.raises(ValueError):
        c.decode_attend(torch.zeros((2, 8, 128), dtype=torch.float16))  # wrong head count


def test_binding_rejects_tensors_on_another_device():
    import torch
    c = _host_cache()
    c.storage = torch.empty(0, dtype=torch.uint8, device="meta")
    q = torch.zeros((2, 32, 128), dtype=torch.float16)
    with pytest.raises(ValueError):
        c.decode_attend(q, out=torch.empty_like(q))


@pytest.mark.parametrize("call", ["fit", "fit_seq", "encode", "decode", "prefill"])
def test_per_row_arrays_must_have_one_entry_per_row(call):
    """The C side reads B entries of every per-row host array: shorter or
    longer arrays are rejected in the binding."""
    B = 3
    with pytest.raises(ValueError):
        if call == "fit":
            palu.palu_fit(0, 0, 0, [5, 5], B, 8, 0)
        elif call == "fit_seq":
            palu.palu_fit_seq(0, 0, 0, [0, 1, 2, 3], [5, 5, 5], B, 8, 0)
        elif call == "encode":
            palu.palu_encode_append(0, 0, 0, None, [1, 1], B, 1, 0)
        elif call == "decode":
            palu.palu_decode_attend(0, 0, 0, [0, 1], B, 0.0, 0)
        else:
            palu.palu_prefill_attend(0, 0, 0, [0, 1, 2], [4], B, 4, 0.0, 0)
    # and through the cache object, with tensors of the right shapes
    import torch
    c = _host_cache()
    k = torch.zeros((B, 8, 4, 128), dtype=torch.float16)
    with pytest.raises(ValueError):
        if call in ("fit", "fit_seq"):
            c.fit(k, k.clone(), seq_lens=[4, 4], seq_ids=None if call == "fit" else [0, 1, 2])
        elif call == "encode":
            c.encode_append(k, k.clone(), seq_ids=[0, 1])
        elif call == "decode":
            q = torch.zeros((B, 32, 128), dtype=torch.float16)
            c.decode_attend(q, seq_ids=[0, 1, 2, 3])
        else:
            q = torch.zeros((B, 32, 4, 128), dtype=torch.float16)
            c.prefill_attend(q, n_q=[1, 1])


def test_fit_info_needs_a_fit():
    h = palu.palu_cache_create(_cfg(), 2, 64)
    try:
        with pytest.raises(palu.PaluError) as ei:
            palu.palu_get_fit_info(h, 0, 4)
        assert ei.value.code == 3
        with pytest.raises(palu.PaluError) as ei:
            palu.palu_get_fit_info(h, 2, 4)
        assert ei.value.code == 1
    finally:
        palu.palu_cache_destroy(h)


def test_read_probe_rejects_bad_arguments():
    for args in [(0, 1 << 20, 1, 64), (16, 1 << 20, 0, 64), (16, 0, 16, 64), (16, 24, 16, 64),
                 (8, 1 << 20, 16, 64), (16, 1 << 20, 16, 0), (16, 1 << 20, 16, 65537)]:
        with pytest.raises(palu.PaluError) as ei:
            palu.palu_probe_read(args[0], args[1], args[2], args[3], 0)
        assert ei.value.code == 1, args
