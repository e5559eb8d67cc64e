"""Host-side logic of bench.py (no GPU): the one-GPU refusal and the
algorithmic byte counts behind every roofline figure, checked on small
cases counted term by term."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr


def test_attend_bytes_quantised_values():
    # two sequences: 33 tokens (1 complete group + 1 tail token) and 64 (2 groups)
    H, Hq, D, G = 2, 4, 128, 1
    wk, rk, wv, rv = 20, 8, 18, 7
    per_head_33 = (1 * wk * 4 + 1 * rk * 4) + (1 * wv * 4 + 1 * rv * 4)
    per_head_64 = (2 * wk * 4) + (2 * wv * 4)
    bases = G * D * (rk + 1) * 4 + G * D * (rv + 1) * 4       # fp32 basis columns + mean
    q_and_out = 2 * Hq * D * 2 * 2                            # fp16 query in, output out
    want = H * (per_head_33 + per_head_64) + bases + q_and_out
    assert bench.attend_bytes([33, 64], H, Hq, D, G, wk, rk, wv, rv, True) == want
    # one basis set per sequence
    assert bench.attend_bytes([33, 64], H, Hq, D, G, wk, rk, wv, rv, True, basis_sets=2) == want + bases


def test_attend_bytes_fp16_value_latents():
    H, Hq, D, G = 1, 2, 128, 2
    wk, rk, rv = 12, 5, 6
    n = 40                                                    # 1 group + 8 tail tokens
    keys = 1 * wk * 4 + 8 * rk * 4
    values = n * rv * 2                                       # fp16 latents of every token
    bases = G * D * (rk + 1) * 4 + G * D * (rv + 1) * 4
    want = H * (keys + values) + bases + 1 * Hq * D * 2 * 2
    assert bench.attend_bytes([n], H, Hq, D, G, wk, rk, 0, rv, False) == want


@pytest.mark.parametrize("vq", [True, False])
def test_encode_bytes(vq):
    H, D, wk, rk, wv, rv = 2, 128, 20, 8, 18, 7
    lens = [70, 5]                                            # 2 groups + 6, 0 groups + 5
    read = 2 * (70 + 5) * H * D * 2                           # fp16 K and V
    k_written = H * (2 * wk * 4 + 6 * rk * 4) + H * (5 * rk * 4)
    v_written = (H * (2 * wv * 4 + 6 * rv * 4) + H * (5 * rv * 4)) if vq else H * (70 + 5) * rv * 2
    assert bench.encode_bytes(lens, H, D, wk, rk, wv, rv, vq) == read + k_written + v_written
