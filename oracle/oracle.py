"""NumPy-facing wrapper of the plain-C oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke entry point and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP library or its binding.

Every function is a thin marshalling layer over one oracle.c routine, whose
header comment cites the passage of the pages it follows; the few pieces of
arithmetic done here (the hi-channel count, the effective-bit formulas and
the per-layer composition in OracleLayer) cite their passages inline.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
_u32p = np.ctypeslib.ndpointer(np.uint32, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(np.int64, flags="C_CONTIGUOUS")
_c_int, _c_i64, _c_dbl = ctypes.c_int, ctypes.c_int64, ctypes.c_double


def lib():
    """Load oracle/liboracle.so, compiling it first if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build_oracle
            build_oracle.build()
        L = ctypes.CDLL(_LIB_PATH)
        L.orc_half_to_float_n.argtypes = [_u16p, _f32p, _c_i64]
        L.orc_float_to_half_n.argtypes = [_f32p, _u16p, _c_i64]
        L.orc_energy_rank.argtypes = [_f64p, _c_int, _c_dbl]
        L.orc_energy_rank.restype = _c_int
        L.orc_fit_group.argtypes = [_u16p, _i32p, _c_int, _c_int, _c_int, _c_int,
                                    _c_int, _c_int, _c_int, _c_dbl, _f32p, _f32p,
                                    _f64p, _c_int]
        L.orc_fit_group.restype = _c_int
        L.orc_fit.argtypes = [_u16p, _i32p, _c_int, _c_int, _c_int, _c_int, _c_int,
                              _c_int, _c_dbl, _f32p, _f32p, _f64p, _i32p, _c_int]
        L.orc_fit.restype = _c_int
        L.orc_project.argtypes = [_u16p, _c_i64, _c_int, _f32p, _f32p, _c_int,
                                  _c_int, _f32p, _c_int]
        L.orc_bf16_to_float_n.argtypes = [_u16p, _f32p, _c_i64]
        L.orc_quantize_group.argtypes = [_f32p, _c_int, _c_int, _c_int, _c_int,
                                         _u8p, _u16p, _u16p]
        L.orc_record_words.argtypes = [_c_int, _c_int]
        L.orc_record_words.restype = _c_int
        L.orc_pack_group.argtypes = [_u8p, _u16p, _u16p, _c_int, _c_int, _c_int,
                                     _u32p]
        L.orc_unpack_group.argtypes = [_u32p, _c_int, _c_int, _c_int, _u8p, _u16p,
                                       _u16p]
        L.orc_encode_stream.argtypes = [_f32p, _c_i64, _c_int, _c_int, _c_int,
                                        _c_int, _c_int, _u32p, _f32p]
        L.orc_encode_fp16_stream.argtypes = [_f32p, _c_i64, _c_int, _u16p]
        L.orc_decode_stream.argtypes = [_u32p, _f32p, _c_i64, _c_int, _c_int,
                                        _c_int, _f64p]
        L.orc_decode_fp16_stream.argtypes = [_u16p, _c_i64, _c_int, _f64p]
        L.orc_coded_channels.argtypes = [_c_int, _i32p, _i32p]
        L.orc_coded_channels.restype = _c_int
        L.orc_record_words_seg.argtypes = [_c_int, _i32p, _i32p]
        L.orc_record_words_seg.restype = _c_int
        L.orc_quantize_group_seg.argtypes = [_f32p, _c_int, _c_int, _i32p, _i32p, _u8p, _u16p,
                                             _u16p]
        L.orc_pack_group_seg.argtypes = [_u8p, _u16p, _u16p, _c_int, _c_int, _i32p, _i32p,
                                         _c_int, _u32p]
        L.orc_unpack_group_seg.argtypes = [_u32p, _c_int, _c_int, _i32p, _i32p, _c_int, _u8p,
                                           _u16p, _u16p]
        L.orc_encode_stream_seg.argtypes = [_f32p, _c_i64, _c_int, _c_int, _i32p, _i32p,
                                            _c_int, _u32p, _f32p]
        L.orc_decode_stream_seg.argtypes = [_u32p, _f32p, _c_i64, _c_int, _c_int, _i32p,
                                            _i32p, _c_int, _f64p]
        L.orc_attend.argtypes = [_f64p, _f32p, _c_int, _f32p, _c_int, _f64p, _f32p,
                                 _c_int, _f32p, _c_int, _c_i64, _c_int, _f32p,
                                 _c_dbl, _f64p]
        L.orc_prefill_attend.argtypes = [_f64p, _f32p, _c_int, _f32p, _c_int, _f64p,
                                         _f32p, _c_int, _f32p, _c_int, _c_i64, _c_int,
                                         _f32p, _i64p, _c_i64, _c_dbl, _f64p]
        _lib = L
    return _lib


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def _bits16(x) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype == np.float16:
        return _c(x, np.float16).view(np.uint16)
    return _c(x, np.uint16)


# --------------------------------------------------------------------- fp16

def half_to_float(h) -> np.ndarray:
    h = _bits16(h)
    out = np.empty(h.shape, np.float32)
    lib().orc_half_to_float_n(h.reshape(-1), out.reshape(-1), h.size)
    return out


def bf16_to_float(b) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32, exactly."""
    b = _c(b, np.uint16)
    out = np.empty(b.shape, np.float32)
    lib().orc_bf16_to_float_n(b.reshape(-1), out.reshape(-1), b.size)
    return out


def widen(x, bf16: bool = False) -> np.ndarray:
    """An input array (fp16 values, or bf16 bit patterns when bf16) -> float32."""
    return bf16_to_float(x) if bf16 else half_to_float(x)


def float_to_half_bits(f) -> np.ndarray:
    f = _c(f, np.float32)
    out = np.empty(f.shape, np.uint16)
    lib().orc_float_to_half_n(f.reshape(-1), out.reshape(-1), f.size)
    return out


# ---------------------------------------------------------------------- fit

def n_hi_channels(r: int, hi_fraction: float) -> int:
    """Number of hi-bit latent channels: the channels whose 1-based position
    in descending-singular-value order is at most hi_fraction * r (PALU page,
    "Usage": palu_hi_bit for the top-25% channels by singular value)."""
    return int(math.floor(hi_fraction * r))


def energy_rank(s2, tau: float) -> int:
    s2 = _c(s2, np.float64)
    return lib().orc_energy_rank(s2, s2.size, tau)


@dataclasses.dataclass
class Fit:
    r: int                 # shared rank (minimum over groups)
    r_groups: np.ndarray   # [G] per-group ranks
    basis: np.ndarray      # [G, D, D] fp32, columns sorted by singular value
    mu: np.ndarray         # [G, D] fp32
    sigma: np.ndarray      # [G, D] fp64

    def V(self, g: int) -> np.ndarray:
        """fp32 [D, r] truncated basis of group g (d-major)."""
        return np.ascontiguousarray(self.basis[g][:, :self.r])

    def bases(self) -> np.ndarray:
        """fp32 [G, D, r]."""
        return np.ascontiguousarray(self.basis[:, :, :self.r])


def fit(x, lens, n_groups: int, rank: int = 0, tau: float = 0.90, bf16: bool = False) -> Fit:
    """x: fp16 [B, H, S, D] (bf16 bit patterns, uint16, when bf16); lens: [B]
    valid tokens; rank 0 -> energy rule."""
    x = _bits16(x)
    B, H, S, D = x.shape
    lens = _c(lens, np.int32)
    basis = np.empty((n_groups, D, D), np.float32)
    mu = np.empty((n_groups, D), np.float32)
    sigma = np.empty((n_groups, D), np.float64)
    rg = np.empty(n_groups, np.int32)
    r = lib().orc_fit(x, lens, B, H, S, D, n_groups, int(rank or 0), tau, basis,
                      mu, sigma, rg, 1 if bf16 else 0)
    if r < 0:
        raise ValueError("oracle fit: bad arguments")
    return Fit(r, rg, basis, mu, sigma)


def fit_group(x, lens, n_groups: int, g: int, rank: int = 0, tau: float = 0.90, bf16: bool = False):
    """One group only: (rank_g, basis [D, D], mu [D], sigma [D])."""
    x = _bits16(x)
    B, H, S, D = x.shape
    lens = _c(lens, np.int32)
    basis = np.empty((D, D), np.float32)
    mu = np.empty(D, np.float32)
    sigma = np.empty(D, np.float64)
    r = lib().orc_fit_group(x, lens, B, H, S, D, n_groups, g, int(rank or 0), tau,
                            basis, mu, sigma, 1 if bf16 else 0)
    if r < 0:
        raise ValueError("oracle fit: bad arguments")
    return r, basis, mu, sigma


# ------------------------------------------------------------ encode/decode

def project(x, mu, V, bf16: bool = False) -> np.ndarray:
    """x fp16 [n, D] (bf16 bit patterns when bf16); mu fp32 [D]; V fp32
    [D, r] -> fp32 [n, r]."""
    x = _bits16(x)
    n, D = x.shape
    V = _c(V, np.float32)
    r = V.shape[1]
    out = np.empty((n, r), np.float32)
    lib().orc_project(x.reshape(-1), n, D, _c(mu, np.float32), V, r, r, out, 1 if bf16 else 0)
    return out


def quantize_group(l, n_hi: int, hi_bit: int = 4, lo_bit: int = 2):
    """l fp32 [32, r] -> (codes u8 [32, r], scale16 u16 [r], zero16 u16 [r])."""
    l = _c(l, np.float32)
    r = l.shape[1]
    codes = np.empty((32, r), np.uint8)
    sc = np.empty(r, np.uint16)
    zr = np.empty(r, np.uint16)
    lib().orc_quantize_group(l, r, n_hi, hi_bit, lo_bit, codes, sc, zr)
    return codes, sc, zr


def record_words(r: int, n_hi: int) -> int:
    return lib().orc_record_words(r, n_hi)


def pack_group(codes, scale16, zero16, n_hi: int, layout: int) -> np.ndarray:
    codes = _c(codes, np.uint8)
    r = codes.shape[1]
    rec = np.empty(record_words(r, n_hi), np.uint32)
    lib().orc_pack_group(codes, _c(scale16, np.uint16), _c(zero16, np.uint16), r,
                         n_hi, layout, rec)
    return rec


def unpack_group(rec, r: int, n_hi: int, layout: int):
    codes = np.empty((32, r), np.uint8)
    sc = np.empty(r, np.uint16)
    zr = np.empty(r, np.uint16)
    lib().orc_unpack_group(_c(rec, np.uint32), r, n_hi, layout, codes, sc, zr)
    return codes, sc, zr


def encode_stream(lat, n_hi: int, hi_bit: int, lo_bit: int, layout: int):
    """lat fp32 [n, r] -> (records u32 [n // 32, W], tail fp32 [n % 32, r])."""
    lat = _c(lat, np.float32)
    n, r = lat.shape
    W = record_words(r, n_hi)
    rec = np.zeros((n // 32, W), np.uint32)
    tail = np.zeros((n % 32, r), np.float32)
    lib().orc_encode_stream(lat, n, r, n_hi, hi_bit, lo_bit, layout,
                            rec.reshape(-1) if rec.size else np.zeros(1, np.uint32),
                            tail.reshape(-1) if tail.size else np.zeros(1, np.float32))
    return rec, tail


def encode_fp16_stream(lat) -> np.ndarray:
    """lat fp32 [n, r] -> fp16 bits [ceil(n / 32), r * 32] (channel-major)."""
    lat = _c(lat, np.float32)
    n, r = lat.shape
    rec = np.zeros(((n + 31) // 32, r * 32), np.uint16)
    if n:
        lib().orc_encode_fp16_stream(lat, n, r, rec.reshape(-1))
    return rec


def decode_stream(records, tail, n: int, r: int, n_hi: int, layout: int):
    out = np.empty((n, r), np.float64)
    if n == 0:
        return out
    rec = _c(records, np.uint32).reshape(-1)
    tl = _c(tail, np.float32).reshape(-1)
    lib().orc_decode_stream(rec if rec.size else np.zeros(1, np.uint32),
                            tl if tl.size else np.zeros(1, np.float32), n, r, n_hi,
                            layout, out)
    return out


# -------------------------------------------------------- segment coder

@dataclasses.dataclass
class Segments:
    """Latent channels in contiguous segments, descending singular value
    first: seg_n[s] channels coded with seg_bits[s] bits (0 = not stored)."""
    seg_n: np.ndarray     # int32 [nseg]
    seg_bits: np.ndarray  # int32 [nseg]

    @property
    def r(self) -> int:
        return int(self.seg_n.sum())

    @property
    def coded(self) -> int:
        return lib().orc_coded_channels(len(self.seg_n), self.seg_n, self.seg_bits)

    def words(self) -> int:
        return lib().orc_record_words_seg(len(self.seg_n), self.seg_n, self.seg_bits)


def palu_segments(r: int, hi_fraction: float = 0.25, hi_bit: int = 4, lo_bit: int = 2) -> Segments:
    """PALU's split (PALU page, "Usage"): the first floor(hi_fraction r)
    channels at hi_bit, the rest at lo_bit."""
    n_hi = n_hi_channels(r, hi_fraction)
    return Segments(np.array([n_hi, r - n_hi], np.int32), np.array([hi_bit, lo_bit], np.int32))


def schedule_segments(r: int, schedule) -> Segments:
    """A bit schedule (SVDq cache page): r channels split into len(schedule)
    contiguous groups of equal size, the first r % len(schedule) groups one
    channel larger (the plain reading when r is not a multiple), group i
    coded with schedule[i] bits."""
    L = len(schedule)
    base, extra = divmod(r, L)
    n = np.array([base + (1 if i < extra else 0) for i in range(L)], np.int32)
    return Segments(n, np.array(schedule, np.int32))


def schedule_effective_bits(r: int, D: int, schedule) -> float:
    """Nominal key rate (r / D) * mean(schedule) of the SVDq cache page."""
    return (r / D) * float(np.mean(schedule))


def quantize_group_seg(l, seg: Segments):
    l = _c(l, np.float32)
    r = l.shape[1]
    codes = np.empty((32, r), np.uint8)
    sc = np.empty(r, np.uint16)
    zr = np.empty(r, np.uint16)
    lib().orc_quantize_group_seg(l, r, len(seg.seg_n), seg.seg_n, seg.seg_bits, codes, sc, zr)
    return codes, sc, zr


def pack_group_seg(codes, scale16, zero16, seg: Segments, layout: int) -> np.ndarray:
    codes = _c(codes, np.uint8)
    rec = np.empty(seg.words(), np.uint32)
    lib().orc_pack_group_seg(codes, _c(scale16, np.uint16), _c(zero16, np.uint16), codes.shape[1],
                             len(seg.seg_n), seg.seg_n, seg.seg_bits, layout, rec)
    return rec


def unpack_group_seg(rec, seg: Segments, layout: int):
    r = seg.r
    codes = np.empty((32, r), np.uint8)
    sc = np.empty(r, np.uint16)
    zr = np.empty(r, np.uint16)
    lib().orc_unpack_group_seg(_c(rec, np.uint32), r, len(seg.seg_n), seg.seg_n, seg.seg_bits,
                               layout, codes, sc, zr)
    return codes, sc, zr


def encode_stream_seg(lat, seg: Segments, layout: int):
    """lat fp32 [n, r] -> (records u32 [n // 32, W], tail fp32 [n % 32, coded])."""
    lat = _c(lat, np.float32)
    n, r = lat.shape
    rec = np.zeros((n // 32, seg.words()), np.uint32)
    tail = np.zeros((n % 32, seg.coded), np.float32)
    lib().orc_encode_stream_seg(lat, n, r, len(seg.seg_n), seg.seg_n, seg.seg_bits, layout,
                                rec.reshape(-1) if rec.size else np.zeros(1, np.uint32),
                                tail.reshape(-1) if tail.size else np.zeros(1, np.float32))
    return rec, tail


def decode_stream_seg(records, tail, n: int, seg: Segments, layout: int) -> np.ndarray:
    r = seg.r
    out = np.empty((n, r), np.float64)
    if n == 0:
        return out
    rec = _c(records, np.uint32).reshape(-1)
    tl = _c(tail, np.float32).reshape(-1)
    lib().orc_decode_stream_seg(rec if rec.size else np.zeros(1, np.uint32),
                                tl if tl.size else np.zeros(1, np.float32), n, r,
                                len(seg.seg_n), seg.seg_n, seg.seg_bits, layout, out)
    return out


def decode_fp16_stream(records, n: int, r: int) -> np.ndarray:
    out = np.empty((n, r), np.float64)
    if n:
        lib().orc_decode_fp16_stream(_c(records, np.uint16).reshape(-1), n, r, out)
    return out


def attend(lk, Bk, muk, lv, Bv, muv, q, scale: float) -> np.ndarray:
    """Single-query attention over the reconstructed tokens, fp64 [D]."""
    lk = _c(lk, np.float64)
    lv = _c(lv, np.float64)
    Bk = _c(Bk, np.float32)
    Bv = _c(Bv, np.float32)
    n, rk = lk.shape
    rv = lv.shape[1]
    D = Bk.shape[0]
    qf = half_to_float(q) if np.asarray(q).dtype in (np.float16, np.uint16) \
        else _c(q, np.float32)
    out = np.empty(D, np.float64)
    lib().orc_attend(lk, Bk, Bk.shape[1], _c(muk, np.float32), rk, lv, Bv,
                     Bv.shape[1], _c(muv, np.float32), rv, n, D, _c(qf, np.float32),
                     scale, out)
    return out


def prefill_attend(lk, Bk, muk, lv, Bv, muv, q, positions, scale: float) -> np.ndarray:
    """Causal attention of queries q [nq, D] at the given positions over the
    reconstructed tokens (query i sees tokens 0..positions[i]); fp64 [nq, D]."""
    lk = _c(lk, np.float64)
    lv = _c(lv, np.float64)
    Bk = _c(Bk, np.float32)
    Bv = _c(Bv, np.float32)
    n, rk = lk.shape
    rv = lv.shape[1]
    D = Bk.shape[0]
    qf = half_to_float(q) if np.asarray(q).dtype in (np.float16, np.uint16) \
        else _c(q, np.float32)
    qf = _c(qf, np.float32).reshape(-1, D)
    pos = _c(positions, np.int64).reshape(-1)
    if pos.size != qf.shape[0] or (pos.size and (pos.min() < 0 or pos.max() >= n)):
        raise ValueError("positions must give one position in [0, n) per query")
    out = np.empty((qf.shape[0], D), np.float64)
    if qf.shape[0]:
        lib().orc_prefill_attend(lk, Bk, Bk.shape[1], _c(muk, np.float32), rk, lv, Bv,
                                 Bv.shape[1], _c(muv, np.float32), rv, n, D, qf, pos,
                                 qf.shape[0], scale, out)
    return out


# ------------------------------------------------------------ bit accounting

def effective_bits(r: int, D: int, hi_fraction: float, hi_bit: int, lo_bit: int):
    """Nominal rate (r / D) * (h * b_hi + (1 - h) * b_lo) of the PALU page,
    section "Effective bit-width"."""
    return (r / D) * (hi_fraction * hi_bit + (1.0 - hi_fraction) * lo_bit)


def realised_bits(r: int, D: int, n_hi: int, hi_bit: int, lo_bit: int):
    """Code bits actually stored per element: (n_hi b_hi + n_lo b_lo) / D."""
    return (n_hi * hi_bit + (r - n_hi) * lo_bit) / D


def fp16_latent_bits(r: int, D: int):
    """Value latents kept in fp16: 16 r / D bits per element (PALU page,
    "Effective bit-width")."""
    return 16.0 * r / D


# ------------------------------------------------------------- one layer

class OracleLayer:
    """The whole path for one attention layer, composed from the routines
    above: per-sequence encode of K and V with the group bases, and decode
    attention of one query per query head over everything stored.

    Query head i reads kv head i // (Hq / Hkv) (contiguous grouped-query
    mapping); kv head h uses the basis of group h // (Hkv / G)."""

    def __init__(self, D, n_q_heads, n_kv_heads, n_groups, fitK: Fit, fitV: Fit,
                 hi_fraction=0.25, hi_bit=4, lo_bit=2, quantize_values=True, bf16=False,
                 schedule=None):
        self.D, self.Hq, self.Hkv, self.G = D, n_q_heads, n_kv_heads, n_groups
        self.fit = (fitK, fitV)
        self.hi_fraction, self.hi_bit, self.lo_bit = hi_fraction, hi_bit, lo_bit
        self.quantize_values = quantize_values
        self.bf16 = bf16          # inputs (K, V, q) are bf16 bit patterns
        self.schedule = None if schedule is None else list(schedule)   # bit schedule or PALU split

    def n_hi(self, tensor):
        return n_hi_channels(self.fit[tensor].r, self.hi_fraction)

    def segments(self, tensor) -> Segments:
        r = self.fit[tensor].r
        if self.schedule is not None:
            return schedule_segments(r, self.schedule)
        return palu_segments(r, self.hi_fraction, self.hi_bit, self.lo_bit)

    def group_of(self, h):
        return h // (self.Hkv // self.G)

    def latents(self, x_head, h, tensor):
        f = self.fit[tensor]
        g = self.group_of(h)
        return project(x_head, f.mu[g], f.V(g), bf16=self.bf16)

    def encode_head(self, x_head, h, tensor):
        """x_head fp16 [n, D] -> stored state of one (sequence, head, tensor)."""
        lat = self.latents(x_head, h, tensor)
        if tensor == 1 and not self.quantize_values:
            return {"fp16": encode_fp16_stream(lat), "n": lat.shape[0]}
        rec, tail = encode_stream_seg(lat, self.segments(tensor), tensor)
        return {"records": rec, "tail": tail, "n": lat.shape[0]}

    def decode_head(self, st, tensor):
        r = self.fit[tensor].r
        if "fp16" in st:
            return decode_fp16_stream(st["fp16"], st["n"], r)
        return decode_stream_seg(st["records"], st["tail"], st["n"], self.segments(tensor), tensor)

    def attend(self, kstates, vstates, q, scale=None):
        """kstates / vstates: per kv head stored state; q fp16 [Hq, D].
        Returns fp64 [Hq, D]."""
        if scale is None:
            scale = 1.0 / math.sqrt(self.D)
        if self.bf16:
            q = bf16_to_float(q)
        g = self.Hq // self.Hkv
        fK, fV = self.fit
        out = np.empty((self.Hq, self.D), np.float64)
        lks = [self.decode_head(s, 0) for s in kstates]
        lvs = [self.decode_head(s, 1) for s in vstates]
        for i in range(self.Hq):
            h = i // g
            grp = self.group_of(h)
            out[i] = attend(lks[h], fK.V(grp), fK.mu[grp], lvs[h], fV.V(grp),
                            fV.mu[grp], q[i], scale)
        return out

    def prefill_attend(self, kstates, vstates, q, positions, scale=None):
        """Causal prefill attention.  q fp16 [Hq, nq, D]; query j of every
        head sits at positions[j] and sees the stored tokens 0..positions[j].
        Returns fp64 [Hq, nq, D]."""
        if scale is None:
            scale = 1.0 / math.sqrt(self.D)
        if self.bf16:
            q = bf16_to_float(q)
        g = self.Hq // self.Hkv
        fK, fV = self.fit
        nq = len(positions)
        out = np.empty((self.Hq, nq, self.D), np.float64)
        lks = [self.decode_head(s, 0) for s in kstates]
        lvs = [self.decode_head(s, 1) for s in vstates]
        for i in range(self.Hq):
            h = i // g
            grp = self.group_of(h)
            out[i] = prefill_attend(lks[h], fK.V(grp), fK.mu[grp], lvs[h], fV.V(grp),
                                    fV.mu[grp], q[i], positions, scale)
        return out
