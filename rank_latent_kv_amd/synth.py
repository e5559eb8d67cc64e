"""Seeded synthetic inputs for the latent KV cache workloads.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no fit, projection, quantisation or attention).  Both the
CPU oracle and the HIP path consume the arrays it returns.

Recipe (one workload = one single attention layer):
  * per (tensor in {K, V}, head group g): A_g = k orthonormal rows in R^D
    (QR of a D x k Gaussian, transposed), row i scaled by rho**i; the group
    mean mu_g ~ N(0, 0.5^2)^D; optional outlier channels (round(frac * D)
    of them, picked at random) that are multiplied by 8 after the noise;
  * per (sequence, kv head, token): x = mu_g + z A_g + eps with
    z ~ N(0, 1)^k and eps ~ N(0, sigma_n^2)^D, drawn and summed in fp32,
    then rounded to fp16;
  * prefill tokens and decode tokens come from the same process (decode
    tokens are simply the positions after the prefill);
  * queries ~ N(0, 1)^D per (sequence, decode step, query head), fp16.

The shapes and distributions follow the PALU page ("How it works",
"Evidence": low-rank synthetic K/V with a planted subspace) and the five
workload descriptions below.  Every sequence has its own generator stream,
so any single sequence can be regenerated without the others.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

K_TENSOR, V_TENSOR = 0, 1


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int            # sequences
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_head_groups: int    # contiguous kv-head groups sharing one basis
    prefill: Optional[int]          # fixed prefill length (None -> ragged)
    ragged: Optional[tuple]         # (lo, hi) inclusive prefill lengths
    steps: int            # decode steps
    rank: Optional[int]   # explicit rank, None -> energy rule
    energy: float
    latent_rank: int      # k of the generator
    rho: float
    sigma_n: float
    quantize_values: bool
    outlier_frac: float
    seed: int
    hi_bit: int = 4
    lo_bit: int = 2
    hi_fraction: float = 0.25
    group_size: int = 32

    @property
    def gqa(self) -> int:
        return self.n_q_heads // self.n_kv_heads


WORKLOADS = {
    # one layer, B1, 8 q = 8 kv heads, 4 groups of 2, prefill 512 + 16 steps, r = 32
    "single_b1_s512_r32": Workload(
        "single_b1_s512_r32", 1, 8, 8, 128, 4, 512, None, 16, 32, 0.90,
        24, 0.85, 0.01, True, 0.0, 1001),
    # Llama-3.2-3B-shaped layer: 24 q / 8 kv heads, 4 groups, 4096 + 256, energy rank
    "gqa3_b1_s4096_e90": Workload(
        "gqa3_b1_s4096_e90", 1, 24, 8, 128, 4, 4096, None, 256, None, 0.90,
        32, 0.90, 0.02, True, 0.0, 1002),
    # fp16 value latents: 32 q / 8 kv, 2 groups, B8, 8192 + 128, r = 64
    "vlat16_b8_s8192_r64": Workload(
        "vlat16_b8_s8192_r64", 8, 32, 8, 128, 2, 8192, None, 128, 64, 0.90,
        48, 0.92, 0.02, False, 0.0, 1003),
    # long context: 32 q / 8 kv, 4 groups, B4, 32768 + 64, energy rank, 1% outliers
    "long_b4_s32768_e90": Workload(
        "long_b4_s32768_e90", 4, 32, 8, 128, 4, 32768, None, 64, None, 0.90,
        32, 0.90, 0.02, True, 0.01, 1004),
    # batched serving: 64 ragged sequences in [1024, 16384], 8 groups of 1, r = 32
    "serve_b64_s1k16k_r32": Workload(
        "serve_b64_s1k16k_r32", 64, 32, 8, 128, 8, None, (1024, 16384), 100, 32,
        0.90, 24, 0.88, 0.02, True, 0.0, 1005),
}


def prefill_lengths(w: Workload) -> np.ndarray:
    """Per-sequence prefill lengths (int32)."""
    if w.ragged is None:
        return np.full(w.batch, w.prefill, dtype=np.int32)
    rng = np.random.default_rng([w.seed, 7])
    lo, hi = w.ragged
    return rng.integers(lo, hi, endpoint=True, size=w.batch).astype(np.int32)


@dataclasses.dataclass
class GroupParams:
    A: np.ndarray        # [G, k, D] float64, scaled orthonormal rows
    mu: np.ndarray       # [G, D] float64
    outliers: np.ndarray  # [G, n_out] int channel indices


def group_params(w: Workload, tensor: int) -> GroupParams:
    rng = np.random.default_rng([w.seed, 11, tensor])
    D, k, G = w.head_dim, w.latent_rank, w.n_head_groups
    A = np.empty((G, k, D))
    mu = np.empty((G, D))
    n_out = int(round(w.outlier_frac * D))
    outl = np.zeros((G, n_out), dtype=np.int64)
    scales = w.rho ** np.arange(k)
    for g in range(G):
        q, _ = np.linalg.qr(rng.standard_normal((D, k)))
        A[g] = q.T * scales[:, None]
        mu[g] = rng.normal(0.0, 0.5, D)
        if n_out:
            outl[g] = rng.choice(D, size=n_out, replace=False)
    return GroupParams(A, mu, outl)


def to_bf16_bits(x) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def kv_sequence(w: Workload, tensor: int, b: int, n_tokens: int,
                gp: Optional[GroupParams] = None, bf16: bool = False) -> np.ndarray:
    """K or V of sequence b: fp16 [n_kv_heads, n_tokens, D] (bf16 bit
    patterns, uint16, when bf16).

    Tokens [0, prefill) are the prefill, later ones the decode appends; a
    shorter n_tokens returns a prefix of the same stream."""
    if gp is None:
        gp = group_params(w, tensor)
    D, k = w.head_dim, w.latent_rank
    hpg = w.n_kv_heads // w.n_head_groups
    out = np.empty((w.n_kv_heads, n_tokens, D), dtype=np.uint16 if bf16 else np.float16)
    for h in range(w.n_kv_heads):
        g = h // hpg
        rng = np.random.default_rng([w.seed, 13, tensor, b, h])
        z = rng.standard_normal((n_tokens, k), dtype=np.float32)
        eps = rng.standard_normal((n_tokens, D), dtype=np.float32)
        eps *= np.float32(w.sigma_n)
        x = z @ gp.A[g].astype(np.float32)
        x += eps
        x += gp.mu[g].astype(np.float32)[None, :]
        if gp.outliers.shape[1]:
            x[:, gp.outliers[g]] *= 8.0
        out[h] = to_bf16_bits(x) if bf16 else x.astype(np.float16)
    return out


def queries(w: Workload, b: int, n_steps: Optional[int] = None, bf16: bool = False) -> np.ndarray:
    """Decode queries of sequence b: fp16 [n_steps, n_q_heads, D] (bf16 bit
    patterns when bf16)."""
    n = w.steps if n_steps is None else n_steps
    rng = np.random.default_rng([w.seed, 17, b])
    x = rng.standard_normal((n, w.n_q_heads, w.head_dim))
    return to_bf16_bits(x.astype(np.float32)) if bf16 else x.astype(np.float16)


def prefill_queries(w: Workload, b: int, n: int, bf16: bool = False) -> np.ndarray:
    """Prefill queries of sequence b, one per prompt position: fp16
    [n_q_heads, n, D], N(0, 1) like the decode queries (bf16 bit patterns
    when bf16)."""
    rng = np.random.default_rng([w.seed, 19, b])
    x = rng.standard_normal((w.n_q_heads, n, w.head_dim), dtype=np.float32)
    return to_bf16_bits(x) if bf16 else x.astype(np.float16)


def batch_kv(w: Workload, tensor: int, n_tokens: int, seqs=None, bf16: bool = False) -> np.ndarray:
    """[len(seqs), n_kv_heads, n_tokens, D] fp16 (each sequence's own stream,
    truncated or generated to n_tokens positions; bf16 bit patterns when bf16)."""
    gp = group_params(w, tensor)
    seqs = range(w.batch) if seqs is None else seqs
    return np.stack([kv_sequence(w, tensor, b, n_tokens, gp, bf16) for b in seqs])


def small_workload(name: str = "tiny", *, batch=2, n_q_heads=4, n_kv_heads=2,
                   head_dim=128, n_head_groups=1, prefill=96, ragged=None,
                   steps=4, rank=16, energy=0.90, latent_rank=12, rho=0.85,
                   sigma_n=0.02, quantize_values=True, outlier_frac=0.0,
                   seed=4242, hi_bit=4, lo_bit=2, hi_fraction=0.25) -> Workload:
    """A reduced workload with the same recipe, for tests the oracle finishes
    in seconds."""
    return Workload(name, batch, n_q_heads, n_kv_heads, head_dim, n_head_groups,
                    prefill, ragged, steps, rank, energy, latent_rank, rho,
                    sigma_n, quantize_values, outlier_frac, seed, hi_bit,
                    lo_bit, hi_fraction)


def planted_spectrum_groups(crossings, n_rows: int, head_dim: int = 128, seed: int = 0,
                            reach: float = 0.925, floor_dims: int = 30) -> np.ndarray:
    """Rows with an exactly planted spectrum per group, for checking rank
    rules: fp16 [1, G, n_rows, head_dim], group g = kv head g.

    Group g is 1 mu^T + U diag(sigma) W^T with U orthonormal columns
    orthogonal to the ones vector and W orthonormal, so the centred rows have
    singular values sigma exactly (before the fp16 rounding).  The squared
    sigmas are crossings[g] leading directions of energy about 1 (slightly
    decreasing), then floor_dims equal ones holding the rest, sized so that
    the leading directions hold the fraction `reach` of the energy."""
    rng = np.random.default_rng([seed, 23])
    G = len(crossings)
    out = np.empty((1, G, n_rows, head_dim), np.float16)
    for g, k in enumerate(crossings):
        big = 1.0 + 0.01 * np.arange(k)[::-1]
        floor_e = (big.sum() / reach - big.sum()) / floor_dims
        e = np.concatenate([big, np.full(floor_dims, floor_e)])
        s = np.sqrt(e / e.sum()) * 40.0
        n = len(s)
        U = rng.standard_normal((n_rows, n))
        U -= U.mean(axis=0)
        U, _ = np.linalg.qr(U)
        W, _ = np.linalg.qr(rng.standard_normal((head_dim, n)))
        mu = rng.normal(0.0, 0.5, head_dim)
        out[0, g] = (mu[None, :] + (U * s[None, :]) @ W.T).astype(np.float16)
    return out
