"""Crafted quantiser inputs: 32-token groups of fp16-representable latents
in which rounding (l - min) / scale to a code gives a different result when
the division is replaced by a multiplication with the rounded reciprocal.

Only numpy fp32 arithmetic picks the candidates (input generation); the
expected codes are computed separately by each test.
"""
import numpy as np


def division_sensitive_group(rng, bits, tries=200):
    """fp32 [32] latents of one channel (every value an fp16 number):
    token 0 holds the minimum, token 1 the maximum, and as many of the other
    30 tokens as the search finds are values whose code differs between
    IEEE division and reciprocal multiplication.  Returns (l, n_sensitive)."""
    levels = np.float32(2 ** bits - 1)
    pos = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32)
    grid = np.concatenate([-pos[::-1], pos])
    best = None
    for _ in range(tries):
        mn = np.float32(np.float16(rng.uniform(-4.0, 4.0)))
        mx = np.float32(np.float16(mn + rng.uniform(0.05, 8.0)))
        scale = np.float32(np.float32(mx - mn) / levels)
        if not scale > 0:
            continue
        cand = grid[(grid > mn) & (grid < mx)]
        d = (cand - mn).astype(np.float32)
        q_div = np.rint(d / scale)
        q_rcp = np.rint(d * np.float32(np.float32(1.0) / scale))
        hit = cand[q_div != q_rcp]
        if best is None or len(hit) > len(best[2]):
            best = (mn, mx, hit, cand)
        if len(hit) >= 30:
            break
    mn, mx, hit, cand = best
    pick = list(hit[:30])
    while len(pick) < 30:
        pick.append(cand[rng.integers(len(cand))])
    l = np.array([mn, mx] + pick, np.float32)
    return l, min(len(hit), 30)
