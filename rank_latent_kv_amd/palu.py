"""ctypes binding of libpalu.so (include/palu.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels and host runtime.  The module-level functions carry the C names and
raise PaluError on a non-zero status.  LatentKVCache wraps one cache whose
device storage is a torch uint8 tensor and whose stream is torch's current
stream.  There is no fallback: if the library cannot be loaded, importing
the binding's functions raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpalu.so")

PALU_OK = 0
ERROR_NAMES = {1: "PALU_ERR_INVALID_ARG", 2: "PALU_ERR_UNSUPPORTED", 3: "PALU_ERR_NOT_FITTED",
               4: "PALU_ERR_CAPACITY", 5: "PALU_ERR_NOT_BOUND", 6: "PALU_ERR_HIP"}

EXPORTED = ["palu_config_default", "palu_cache_create", "palu_cache_required_bytes",
            "palu_cache_bind", "palu_fit", "palu_set_basis", "palu_get_basis",
            "palu_fit_seq", "palu_set_basis_seq", "palu_get_basis_seq",
            "palu_encode_append", "palu_decode_attend", "palu_decode_step", "palu_sync_lengths",
            "palu_decode_attend_noalloc",
            "palu_prefill_attend", "palu_prefill_workspace_bytes", "palu_prefill_attend_ws", "palu_seq_len",
            "palu_read_codes",
            "palu_get_stats", "palu_reset", "palu_record_words", "palu_export_bytes",
            "palu_export_seq", "palu_import_seq", "palu_get_fit_info", "palu_probe_read",
            "palu_last_error", "palu_cache_destroy"]


class PaluError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERROR_NAMES.get(code, code)}: {msg}")
        self.code = code


class palu_config(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_head_groups", ctypes.c_int32),
                ("rank", ctypes.c_int32), ("energy_threshold", ctypes.c_float),
                ("hi_bit", ctypes.c_int32), ("lo_bit", ctypes.c_int32),
                ("hi_fraction", ctypes.c_float), ("group_size", ctypes.c_int32),
                ("quantize_values", ctypes.c_int32), ("max_rank", ctypes.c_int32),
                ("split_groups", ctypes.c_int32), ("input_dtype", ctypes.c_int32),
                ("schedule_len", ctypes.c_int32), ("bit_schedule", ctypes.c_int32 * 8),
                ("per_seq_basis", ctypes.c_int32)]


class palu_stats(ctypes.Structure):
    _fields_ = [("r_k", ctypes.c_int32), ("r_v", ctypes.c_int32), ("n_hi_k", ctypes.c_int32),
                ("n_hi_v", ctypes.c_int32), ("tokens", ctypes.c_int64),
                ("compressed_key_bytes", ctypes.c_int64), ("compressed_value_bytes", ctypes.c_int64),
                ("fp16_key_bytes", ctypes.c_int64), ("fp16_value_bytes", ctypes.c_int64),
                ("nominal_bits_k", ctypes.c_double), ("nominal_bits_v", ctypes.c_double),
                ("realised_bits_k", ctypes.c_double), ("realised_bits_v", ctypes.c_double),
                ("assigned_avg_bits", ctypes.c_double), ("coded_k", ctypes.c_int32),
                ("coded_v", ctypes.c_int32), ("energy_margin_k", ctypes.c_double),
                ("energy_margin_v", ctypes.c_double)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


_lib = None
_vp, _i32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
_i32p = ctypes.POINTER(ctypes.c_int32)


def lib():
    """Load libpalu.so (building it first only if it does not exist)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build
        build.build()
    L = ctypes.CDLL(LIB_PATH)
    sig = {
        "palu_config_default": [ctypes.POINTER(palu_config), _i32, _i32, _i32],
        "palu_cache_create": [ctypes.POINTER(palu_config), _i32, _i32, ctypes.POINTER(_vp)],
        "palu_cache_required_bytes": [_vp, ctypes.POINTER(_sz)],
        "palu_cache_bind": [_vp, _vp, _sz],
        "palu_fit": [_vp, _vp, _vp, _i32p, _i32, _i32, _vp],
        "palu_set_basis": [_vp, _i32, _i32, _vp, _vp],
        "palu_get_basis": [_vp, _i32, _i32p, _vp, _vp, _vp],
        "palu_fit_seq": [_vp, _vp, _vp, _i32p, _i32p, _i32, _i32, _vp],
        "palu_set_basis_seq": [_vp, _i32, _i32, _i32, _vp, _vp],
        "palu_get_basis_seq": [_vp, _i32, _i32, _i32p, _vp, _vp, _vp],
        "palu_encode_append": [_vp, _vp, _vp, _i32p, _i32p, _i32, _i32, _vp],
        "palu_decode_attend": [_vp, _vp, _vp, _i32p, _i32, ctypes.c_float, _vp],
        "palu_decode_attend_noalloc": [_vp, _vp, _vp, _i32p, _i32, ctypes.c_float, _vp],
        "palu_decode_step": [_vp, _vp, _vp, _vp, _vp, _i32p, _i32, ctypes.c_float, _vp],
        "palu_sync_lengths": [_vp],
        "palu_prefill_attend": [_vp, _vp, _vp, _i32p, _i32p, _i32, _i32, ctypes.c_float, _vp],
        "palu_prefill_workspace_bytes": [_vp, _i32p, _i32, ctypes.POINTER(_sz)],
        "palu_prefill_attend_ws": [_vp, _vp, _vp, _i32p, _i32p, _i32, _i32, ctypes.c_float, _vp, _sz, _vp],
        "palu_seq_len": [_vp, _i32, _i32p],
        "palu_read_codes": [_vp, _i32, _i32, _i32, _vp, _sz, _vp, _sz],
        "palu_get_stats": [_vp, ctypes.POINTER(palu_stats)],
        "palu_get_fit_info": [_vp, _i32, _i32p, _vp, _vp],
        "palu_probe_read": [_vp, _sz, _vp, _i32, _vp],
        "palu_reset": [_vp],
        "palu_record_words": [_vp, _i32, _i32p],
        "palu_export_bytes": [_vp, _i32, ctypes.POINTER(_sz)],
        "palu_export_seq": [_vp, _i32, _vp, _sz],
        "palu_import_seq": [_vp, _i32, _vp, _sz],
        "palu_cache_destroy": [_vp],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = None if name == "palu_cache_destroy" else ctypes.c_int
    L.palu_last_error.argtypes = []
    L.palu_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(code: int):
    if code != PALU_OK:
        raise PaluError(code, lib().palu_last_error().decode())


def _i32_array(vals, n: Optional[int] = None, name: str = "array"):
    """int32 copy of a per-row host array and its pointer; None stays None.
    With n given the array must hold exactly n entries (the C side reads n)."""
    if vals is None:
        return None
    arr = np.ascontiguousarray(vals, dtype=np.int32).reshape(-1)
    if n is not None and arr.size != n:
        raise ValueError(f"{name} has {arr.size} entries, expected one per row ({n})")
    return arr, arr.ctypes.data_as(_i32p)


# ------------------------------------------------------------------ C names

def palu_config_default(head_dim: int, n_kv_heads: int, n_q_heads: int) -> palu_config:
    cfg = palu_config()
    _check(lib().palu_config_default(ctypes.byref(cfg), head_dim, n_kv_heads, n_q_heads))
    return cfg


def palu_cache_create(cfg: palu_config, max_batch: int, max_seq_len: int) -> int:
    h = _vp()
    _check(lib().palu_cache_create(ctypes.byref(cfg), max_batch, max_seq_len, ctypes.byref(h)))
    return h.value


def palu_cache_required_bytes(cache: int) -> int:
    n = _sz()
    _check(lib().palu_cache_required_bytes(cache, ctypes.byref(n)))
    return n.value


def palu_cache_bind(cache: int, dev_ptr: int, nbytes: int):
    _check(lib().palu_cache_bind(cache, dev_ptr, nbytes))


def palu_fit(cache: int, k_ptr: int, v_ptr: int, seq_lens, B: int, S_stride: int, stream: int):
    if seq_lens is None:
        raise ValueError("seq_lens is required")
    arr, p = _i32_array(seq_lens, B, "seq_lens")
    _check(lib().palu_fit(cache, k_ptr, v_ptr, p, B, S_stride, stream))


def palu_set_basis(cache: int, tensor: int, r: int, basis: np.ndarray, mu: np.ndarray):
    basis = np.ascontiguousarray(basis, dtype=np.float32)
    mu = np.ascontiguousarray(mu, dtype=np.float32)
    _check(lib().palu_set_basis(cache, tensor, r, basis.ctypes.data, mu.ctypes.data))


def palu_get_basis(cache: int, tensor: int, G: int, D: int):
    r = ctypes.c_int32()
    _check(lib().palu_get_basis(cache, tensor, ctypes.byref(r), None, None, None))
    basis = np.empty((G, D, r.value), np.float32)
    mu = np.empty((G, D), np.float32)
    sigma = np.empty((G, D), np.float64)
    _check(lib().palu_get_basis(cache, tensor, ctypes.byref(r), basis.ctypes.data,
                                mu.ctypes.data, sigma.ctypes.data))
    return r.value, basis, mu, sigma


def palu_fit_seq(cache: int, k_ptr: int, v_ptr: int, seq_ids, seq_lens, B: int, S_stride: int,
                 stream: int):
    s = _i32_array(seq_ids, B, "seq_ids")
    n = _i32_array(seq_lens, B, "seq_lens")
    _check(lib().palu_fit_seq(cache, k_ptr, v_ptr, s[1] if s else None, n[1] if n else None, B,
                              S_stride, stream))


def palu_set_basis_seq(cache: int, seq: int, tensor: int, r: int, basis: np.ndarray, mu: np.ndarray):
    basis = np.ascontiguousarray(basis, dtype=np.float32)
    mu = np.ascontiguousarray(mu, dtype=np.float32)
    _check(lib().palu_set_basis_seq(cache, seq, tensor, r, basis.ctypes.data, mu.ctypes.data))


def palu_get_basis_seq(cache: int, seq: int, tensor: int, G: int, D: int):
    r = ctypes.c_int32()
    _check(lib().palu_get_basis_seq(cache, seq, tensor, ctypes.byref(r), None, None, None))
    basis = np.empty((G, D, r.value), np.float32)
    mu = np.empty((G, D), np.float32)
    sigma = np.empty((G, D), np.float64)
    _check(lib().palu_get_basis_seq(cache, seq, tensor, ctypes.byref(r), basis.ctypes.data,
                                    mu.ctypes.data, sigma.ctypes.data))
    return r.value, basis, mu, sigma


def palu_encode_append(cache: int, k_ptr: int, v_ptr: int, seq_ids, n_new, B: int,
                       T_stride: int, stream: int):
    s = _i32_array(seq_ids, B, "seq_ids")
    n = _i32_array(n_new, B, "n_new")
    _check(lib().palu_encode_append(cache, k_ptr, v_ptr, s[1] if s else None,
                                    n[1] if n else None, B, T_stride, stream))


def palu_decode_attend(cache: int, q_ptr: int, out_ptr: int, seq_ids, B: int,
                       softmax_scale: float, stream: int):
    s = _i32_array(seq_ids, B, "seq_ids")
    _check(lib().palu_decode_attend(cache, q_ptr, out_ptr, s[1] if s else None, B,
                                    softmax_scale, stream))


def palu_decode_step(cache: int, k_ptr: int, v_ptr: int, q_ptr: int, out_ptr: int, seq_ids, B: int,
                     softmax_scale: float, stream: int):
    s = _i32_array(seq_ids, B, "seq_ids")
    _check(lib().palu_decode_step(cache, k_ptr, v_ptr, q_ptr, out_ptr, s[1] if s else None, B,
                                  softmax_scale, stream))


def palu_sync_lengths(cache: int):
    _check(lib().palu_sync_lengths(cache))


def palu_decode_attend_noalloc(cache: int, q_ptr: int, out_ptr: int, seq_ids, B: int,
                               softmax_scale: float, stream: int):
    s = _i32_array(seq_ids, B, "seq_ids")
    _check(lib().palu_decode_attend_noalloc(cache, q_ptr, out_ptr, s[1] if s else None, B,
                                            softmax_scale, stream))


def palu_prefill_attend(cache: int, q_ptr: int, out_ptr: int, seq_ids, n_q, B: int,
                        T_stride: int, softmax_scale: float, stream: int):
    s = _i32_array(seq_ids, B, "seq_ids")
    n = _i32_array(n_q, B, "n_q")
    _check(lib().palu_prefill_attend(cache, q_ptr, out_ptr, s[1] if s else None,
                                     n[1] if n else None, B, T_stride, softmax_scale, stream))


def palu_prefill_workspace_bytes(cache: int, seq_ids, B: int) -> int:
    s = _i32_array(seq_ids, B, "seq_ids")
    n = _sz()
    _check(lib().palu_prefill_workspace_bytes(cache, s[1] if s else None, B, ctypes.byref(n)))
    return n.value


def palu_prefill_attend_ws(cache: int, q_ptr: int, out_ptr: int, seq_ids, n_q, B: int, T_stride: int,
                           softmax_scale: float, ws_ptr: int, ws_bytes: int, stream: int):
    s = _i32_array(seq_ids, B, "seq_ids")
    n = _i32_array(n_q, B, "n_q")
    _check(lib().palu_prefill_attend_ws(cache, q_ptr, out_ptr, s[1] if s else None, n[1] if n else None, B,
                                        T_stride, softmax_scale, ws_ptr, ws_bytes, stream))


def palu_seq_len(cache: int, seq: int) -> int:
    n = ctypes.c_int32()
    _check(lib().palu_seq_len(cache, seq, ctypes.byref(n)))
    return n.value


def palu_record_words(cache: int, tensor: int) -> int:
    n = ctypes.c_int32()
    _check(lib().palu_record_words(cache, tensor, ctypes.byref(n)))
    return n.value


def palu_export_bytes(cache: int, seq: int) -> int:
    n = _sz()
    _check(lib().palu_export_bytes(cache, seq, ctypes.byref(n)))
    return n.value


def palu_export_seq(cache: int, seq: int) -> bytes:
    n = palu_export_bytes(cache, seq)
    buf = ctypes.create_string_buffer(n)
    _check(lib().palu_export_seq(cache, seq, buf, n))
    return buf.raw


def palu_import_seq(cache: int, seq: int, data: bytes):
    buf = ctypes.create_string_buffer(bytes(data), len(data))
    _check(lib().palu_import_seq(cache, seq, buf, len(data)))


def palu_read_codes(cache: int, seq: int, head: int, tensor: int, n_records: int, words: int,
                    n_tail: int, r: int):
    rec = np.zeros((n_records, words), np.uint32)
    tail = np.zeros((n_tail, r), np.float32)
    _check(lib().palu_read_codes(cache, seq, head, tensor,
                                 rec.ctypes.data if rec.size else None, rec.nbytes,
                                 tail.ctypes.data if tail.size else None, tail.nbytes))
    return rec, tail


def palu_get_stats(cache: int) -> palu_stats:
    st = palu_stats()
    _check(lib().palu_get_stats(cache, ctypes.byref(st)))
    return st


def palu_get_fit_info(cache: int, tensor: int, G: int):
    """(per-group ranks int32 [G], energy fractions at r - 1 and at r
    float64 [G] each) of the last shared fit of `tensor`."""
    rg = np.empty(G, np.int32)
    ep = np.empty(G, np.float64)
    ea = np.empty(G, np.float64)
    _check(lib().palu_get_fit_info(cache, tensor, rg.ctypes.data_as(_i32p), ep.ctypes.data,
                                   ea.ctypes.data))
    return rg, ep, ea


def palu_probe_read(buf_ptr: int, nbytes: int, sink_ptr: int, grid: int, stream: int):
    _check(lib().palu_probe_read(buf_ptr, nbytes, sink_ptr, grid, stream))


def palu_reset(cache: int):
    _check(lib().palu_reset(cache))


def palu_last_error() -> str:
    return lib().palu_last_error().decode()


def palu_cache_destroy(cache: int):
    lib().palu_cache_destroy(cache)


# -------------------------------------------------------------- torch side

class LatentKVCache:
    """One layer's latent KV cache on the current GPU.

    torch supplies the bound device storage (a uint8 tensor) and the stream
    (torch.cuda.current_stream()); every computation happens in libpalu."""

    def __init__(self, head_dim: int, n_kv_heads: int, n_q_heads: int, n_head_groups: int,
                 max_batch: int, max_seq_len: int, rank: int = 0, energy_threshold: float = 0.90,
                 hi_bit: int = 4, lo_bit: int = 2, hi_fraction: float = 0.25,
                 group_size: int = 32, quantize_values: bool = True, max_rank: int = 0,
                 split_groups: int = 0, input_dtype: str = "fp16", bit_schedule=None,
                 per_seq_basis: bool = False, device=None):
        import torch
        self.torch = torch
        cfg = palu_config_default(head_dim, n_kv_heads, n_q_heads)
        cfg.n_head_groups = n_head_groups
        cfg.rank = rank or 0
        cfg.energy_threshold = energy_threshold
        cfg.hi_bit, cfg.lo_bit, cfg.hi_fraction = hi_bit, lo_bit, hi_fraction
        cfg.group_size = group_size
        cfg.quantize_values = 1 if quantize_values else 0
        cfg.max_rank = max_rank
        cfg.split_groups = split_groups
        if input_dtype not in ("fp16", "bf16"):
            raise ValueError("input_dtype must be 'fp16' or 'bf16'")
        cfg.input_dtype = 1 if input_dtype == "bf16" else 0
        if bit_schedule is not None:
            sched = [int(b) for b in bit_schedule]
            if not 1 <= len(sched) <= 8:
                raise ValueError("bit_schedule needs 1 to 8 entries")
            cfg.schedule_len = len(sched)
            for i, b in enumerate(sched):
                cfg.bit_schedule[i] = b
        cfg.per_seq_basis = 1 if per_seq_basis else 0
        self.cfg = cfg
        self.D, self.H, self.Hq, self.G = head_dim, n_kv_heads, n_q_heads, n_head_groups
        self.max_batch, self.max_seq_len = max_batch, max_seq_len
        self.handle = palu_cache_create(cfg, max_batch, max_seq_len)
        self._destroy = lib().palu_cache_destroy
        nbytes = palu_cache_required_bytes(self.handle)
        dev = torch.device("cuda") if device is None else torch.device(device)
        self.storage = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        palu_cache_bind(self.handle, self.storage.data_ptr(), nbytes)

    def __del__(self):
        # the library handle is kept on the instance: module globals may
        # already be gone when this runs at interpreter exit
        h, destroy = getattr(self, "handle", None), getattr(self, "_destroy", None)
        if h and destroy is not None:
            destroy(h)
            self.handle = None

    def _stream(self):
        return self.torch.cuda.current_stream(self.storage.device).cuda_stream

    def _check_rank(self, t, dims, name):
        if not isinstance(t, self.torch.Tensor) or t.dim() != dims:
            raise ValueError(f"{name} must be a {dims}-dimensional tensor")

    def _check_half(self, t, shape_tail, name, shape=None):
        """t must be a contiguous tensor of the input type on the cache's
        device, ending in shape_tail (or of exactly `shape`)."""
        torch = self.torch
        want = torch.bfloat16 if self.cfg.input_dtype == 1 else torch.float16
        if not isinstance(t, torch.Tensor) or t.dtype != want or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {want} tensor")
        if t.device != self.storage.device:
            raise ValueError(f"{name} is on {t.device}, the cache on {self.storage.device}")
        if shape is not None:
            if tuple(t.shape) != tuple(shape):
                raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        elif t.dim() < len(shape_tail) or tuple(t.shape[-len(shape_tail):]) != tuple(shape_tail):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected [..., {shape_tail}]")

    def fit(self, k, v, seq_lens: Optional[Sequence[int]] = None, seq_ids=None):
        """k, v: fp16 [B, H, S, D].  With per-sequence bases, row b is fitted
        into slot seq_ids[b] (default b)."""
        self._check_rank(k, 4, "k")
        self._check_half(k, (self.H, k.shape[2], self.D), "k")
        self._check_half(v, None, "v", tuple(k.shape))
        B, _, S, _ = k.shape
        lens = [S] * B if seq_lens is None else list(seq_lens)
        _i32_array(lens, B, "seq_lens")
        _i32_array(seq_ids, B, "seq_ids")
        if seq_ids is None:
            palu_fit(self.handle, k.data_ptr(), v.data_ptr(), lens, B, S, self._stream())
        else:
            palu_fit_seq(self.handle, k.data_ptr(), v.data_ptr(), seq_ids, lens, B, S, self._stream())

    def set_basis(self, tensor: int, basis: np.ndarray, mu: np.ndarray, seq: Optional[int] = None):
        """Install a basis: the shared one, every slot's (per-sequence bases,
        seq None) or one slot's."""
        basis = np.asarray(basis, np.float32)
        if seq is None:
            palu_set_basis(self.handle, tensor, basis.shape[-1], basis, mu)
        else:
            palu_set_basis_seq(self.handle, seq, tensor, basis.shape[-1], basis, mu)

    def get_basis(self, tensor: int, seq: Optional[int] = None):
        if seq is None:
            return palu_get_basis(self.handle, tensor, self.G, self.D)
        return palu_get_basis_seq(self.handle, seq, tensor, self.G, self.D)

    def encode_append(self, k, v, seq_ids=None, n_new=None):
        """k, v: fp16 [B, H, T, D]; appends n_new[b] (default T) tokens of row
        b to slot seq_ids[b] (default b)."""
        self._check_rank(k, 4, "k")
        self._check_half(k, (self.H, k.shape[2], self.D), "k")
        self._check_half(v, None, "v", tuple(k.shape))
        B, _, T, _ = k.shape
        _i32_array(seq_ids, B, "seq_ids")
        _i32_array(n_new, B, "n_new")
        palu_encode_append(self.handle, k.data_ptr(), v.data_ptr(), seq_ids, n_new, B, T,
                           self._stream())

    def decode_attend(self, q, seq_ids=None, softmax_scale: float = 0.0, out=None):
        """q: fp16 [B, Hq, D] -> fp16 [B, Hq, D]."""
        self._check_rank(q, 3, "q")
        self._check_half(q, (self.Hq, self.D), "q")
        if out is None:
            out = self.torch.empty_like(q)
        self._check_half(out, None, "out", tuple(q.shape))
        _i32_array(seq_ids, q.shape[0], "seq_ids")
        palu_decode_attend(self.handle, q.data_ptr(), out.data_ptr(), seq_ids, q.shape[0],
                           softmax_scale, self._stream())
        return out

    def decode_step(self, k_new, v_new, q, out, seq_ids=None, softmax_scale: float = 0.0):
        """Append one token per row (k_new, v_new: [B, H, 1, D]) and attend
        (q, out: [B, Hq, D]) in one graph-replayable call."""
        self._check_rank(q, 3, "q")
        self._check_half(q, (self.Hq, self.D), "q")
        B = q.shape[0]
        self._check_half(k_new, None, "k_new", (B, self.H, 1, self.D))
        self._check_half(v_new, None, "v_new", (B, self.H, 1, self.D))
        self._check_half(out, None, "out", tuple(q.shape))
        _i32_array(seq_ids, B, "seq_ids")
        palu_decode_step(self.handle, k_new.data_ptr(), v_new.data_ptr(), q.data_ptr(), out.data_ptr(),
                         seq_ids, B, softmax_scale, self._stream())
        return out

    def sync_lengths(self):
        """Host lengths <- device lengths (after replaying captured steps)."""
        palu_sync_lengths(self.handle)

    def decode_attend_noalloc(self, q, out, seq_ids=None, softmax_scale: float = 0.0):
        """decode_attend with the split partials in the library's static
        device array: allocates nothing (the caller passes out)."""
        self._check_rank(q, 3, "q")
        self._check_half(q, (self.Hq, self.D), "q")
        self._check_half(out, None, "out", tuple(q.shape))
        _i32_array(seq_ids, q.shape[0], "seq_ids")
        palu_decode_attend_noalloc(self.handle, q.data_ptr(), out.data_ptr(), seq_ids, q.shape[0],
                                   softmax_scale, self._stream())
        return out

    def prefill_attend(self, q, seq_ids=None, n_q=None, softmax_scale: float = 0.0, out=None,
                       workspace=None):
        """q: fp16 [B, Hq, T, D]; row b's first n_q[b] (default T) queries
        sit at the slot's last n_q[b] positions and attend causally.
        Returns fp16 [B, Hq, T, D] (entries past n_q[b] are left as they were).
        workspace: None = a device buffer this object keeps and grows for the
        pre-decoded tiles (palu_prefill_attend_ws); a uint8 device tensor =
        that buffer; False = no workspace (palu_prefill_attend, which decodes
        each group in the attention kernel; the same output bits)."""
        self._check_rank(q, 4, "q")
        self._check_half(q, (self.Hq, q.shape[2], self.D), "q")
        if q.data_ptr() % 16:
            raise ValueError("q must be 16-byte aligned")
        if out is None:
            out = self.torch.empty_like(q)
        self._check_half(out, None, "out", tuple(q.shape))
        if out.data_ptr() % 16:
            raise ValueError("out must be 16-byte aligned")
        _i32_array(seq_ids, q.shape[0], "seq_ids")
        _i32_array(n_q, q.shape[0], "n_q")
        if workspace is False:
            palu_prefill_attend(self.handle, q.data_ptr(), out.data_ptr(), seq_ids, n_q, q.shape[0],
                                q.shape[2], softmax_scale, self._stream())
            return out
        if workspace is not None:
            ws = workspace
            if (not isinstance(ws, self.torch.Tensor) or ws.dtype != self.torch.uint8 or not ws.is_cuda
                    or not ws.is_contiguous()):
                raise ValueError("workspace must be a contiguous uint8 device tensor")
            if ws.device != q.device:
                raise ValueError("workspace must be on q's device")
        need = palu_prefill_workspace_bytes(self.handle, seq_ids, q.shape[0])
        if workspace is None:
            ws = getattr(self, "_prefill_ws", None)
            if ws is None or ws.numel() < need:
                ws = self.torch.empty(max(need, 256), dtype=self.torch.uint8, device=q.device)
                self._prefill_ws = ws
        palu_prefill_attend_ws(self.handle, q.data_ptr(), out.data_ptr(), seq_ids, n_q, q.shape[0], q.shape[2],
                               softmax_scale, ws.data_ptr(), ws.numel(), self._stream())
        return out

    def seq_len(self, seq: int) -> int:
        return palu_seq_len(self.handle, seq)

    def read_codes(self, seq: int, head: int, tensor: int):
        """(records uint32 [n, words], tail fp32 [len % 32, r]) of one
        (slot, kv head, tensor); fp16 value latents come back as uint32
        words holding two halves each."""
        st = self.stats()
        r = st["coded_k"] if tensor == 0 else st["coded_v"]
        words = palu_record_words(self.handle, tensor)
        n = self.seq_len(seq)
        fp16 = tensor == 1 and not self.cfg.quantize_values
        nrec = (n + 31) // 32 if fp16 else n // 32
        ntail = 0 if fp16 else n % 32
        return palu_read_codes(self.handle, seq, head, tensor, nrec, words, ntail, r)

    def export_seq(self, seq: int) -> bytes:
        """Serialized codes and tails of one slot (header + records + tails)."""
        return palu_export_seq(self.handle, seq)

    def import_seq(self, seq: int, data: bytes):
        """Replace one slot's contents with an exported slot; with shared
        bases the cache must hold the basis the slot was saved under, with
        per-sequence bases the slot's own bases come with it."""
        palu_import_seq(self.handle, seq, data)

    def stats(self) -> dict:
        return palu_get_stats(self.handle).as_dict()

    def fit_info(self, tensor: int):
        """(per-group ranks, energy fraction at r - 1, at r) of the last
        shared fit of tensor 0 (K) or 1 (V)."""
        return palu_get_fit_info(self.handle, tensor, self.G)

    def reset(self):
        palu_reset(self.handle)
