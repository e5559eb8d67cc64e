"""Benchmark of the latent KV cache hot path on one MI355X.

One step = one pass of the whole path over the long-context workload
(4 sequences x 32768 prefill tokens, 32 query / 8 kv heads, D = 128, 4 head
groups, 90%-energy rank, 64 decode steps):
  fit (Gram kernels + host eigensolve) -> encode of the prefill ->
  causal prefill attention of every prompt position over the latent cache ->
  64 x (append one token per sequence -> decode-attend).
All inputs are resident in HBM before the timed region.

`value` is decode-attend throughput: sequences x decode steps per second of
decode-attend time, measured with HIP events recorded on the stream the
library launches on, around every decode-attend call.  The events are
created without the system-scope fence a default HIP event adds (its cache
writeback and invalidation would otherwise land between the timed kernels).  The roofline object
prices the decode-attend call against MI355X's 8 TB/s HBM with the
algorithmic bytes of each call (packed codes + metadata + fp32 tails + bases
and means + query and output).  The CPU baseline times the plain oracle's
decode attention for one sequence on the host.  The prefill-attention
object reports its time and score pairs per second (query head x key pairs
under the causal mask) against the vector-ALU issue rate, counting 2.5 lane
operations per pair (exp2, running max, half an fp16 conversion).

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from rank_latent_kv_amd import synth  # noqa: E402

HBM_PEAK_GBPS = 8000.0
# Non-packed fp32 VALU issue rate of MI355X: 256 CUs x 4 SIMDs x 16 lanes x
# 2.4 GHz (the published 157.3 TFLOP/s counts packed fp32 FMAs: x2 x2).
VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
# Lane operations a causal softmax pair needs at least on the vector unit:
# one exp2, one running-max comparison and half of an fp32 -> fp16 pair
# conversion (the two contractions run on the matrix cores).
PREFILL_OPS_PER_PAIR = 2.5
METRIC = "latent decode-attend tok/s + HBM GB/s (% of peak); encode Mtok/s"


def attend_bytes(lens, H, Hq, D, G, wk, rk, wv, rv, vq, basis_sets=1):
    """Algorithmic bytes of one decode-attend call over sequences of lengths
    `lens`: complete-group records (wk / wv words: codes + fp16 scale/zero
    words), fp32 tail latents of the rk / rv coded channels, fp16 value
    latents of valid tokens, K/V bases and means (one set, or one per
    sequence), query in and output out."""
    tot = 0
    for n in lens:
        nf, nt = n // 32, n % 32
        tot += H * (nf * wk * 4 + nt * rk * 4)
        tot += H * ((nf * wv * 4 + nt * rv * 4) if vq else n * rv * 2)
    tot += basis_sets * (G * D * (rk + 1) * 4 + G * D * (rv + 1) * 4)
    tot += len(lens) * Hq * D * 2 * 2
    return tot


KERNEL_SRC = os.path.join(ROOT, "rank_latent_kv_amd", "csrc", "palu_decode.hip")
PROFILE = os.path.join(ROOT, "profiles", "decode_attend_long_b4_s32768_e90.md")


# GPU clock cycles of the spin queued ahead of the prefill encode's start
# event (about 50 us)
ENCODE_LEAD_CYCLES = 120_000


def measured_traffic(workload):
    """HBM bytes per decode-attend call from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel calibration), if it
    was taken for this workload on the current kernel source; else None."""
    if workload != "long_b4_s32768_e90" or not os.path.exists(PROFILE):
        return None
    import hashlib
    src = hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()
    for line in open(PROFILE):
        if line.startswith("traffic_bytes_per_call:"):
            parts = dict(kv.split("=") for kv in line.split(":", 1)[1].split())
            if parts.get("kernel_sha256") == src:
                return int(parts["bytes"])
    return None


class TimingEvent:
    """A HIP event for timing only, created with hipEventDisableSystemFence
    in the HIP runtime torch has loaded (its streams are only valid there)."""
    _lib = None

    @classmethod
    def _hip(cls):
        if cls._lib is None:
            import ctypes
            path = next(line.split()[-1] for line in open("/proc/self/maps") if "libamdhip64" in line)
            L = ctypes.CDLL(path)
            L.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            L.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._lib = L
        return cls._lib

    def __init__(self):
        import ctypes
        self.ev = ctypes.c_void_p()
        if self._hip().hipEventCreateWithFlags(ctypes.byref(self.ev), 0x20000000) != 0:   # hipEventDisableSystemFence
            raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self, stream):
        if self._hip().hipEventRecord(self.ev, stream.cuda_stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end):
        """milliseconds from this event to `end` (both complete)"""
        import ctypes
        ms = ctypes.c_float()
        if self._hip().hipEventElapsedTime(ctypes.byref(ms), self.ev, end.ev) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        if self._lib is not None and self.ev:
            self._lib.hipEventDestroy(self.ev)


def copy_calibration():
    """A plain device copy of known size, for scaling HBM byte counters."""
    import torch
    n = 256 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    for _ in range(20):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "copies": 20}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="long_b4_s32768_e90")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--input-dtype", choices=("fp16", "bf16"), default="fp16",
                    help="element type of K, V and q (the workload's values, rounded to it)")
    ap.add_argument("--bit-schedule", default="",
                    help="comma-separated bit schedule (e.g. 8,4,2,1,1,0,0,0); default: PALU's 25%%/75%% 4/2-bit split")
    ap.add_argument("--per-seq-rank", type=int, default=0,
                    help="per-sequence bases (each prompt fitted alone) at this explicit rank; "
                         "default: one basis per head group shared by the batch")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 256 MiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the latent KV path is built and measured "
              "on a single MI355X (multi-GPU sharding is a design note, not built).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from rank_latent_kv_amd.palu import LatentKVCache

    w = synth.WORKLOADS[args.workload]
    bf16 = args.input_dtype == "bf16"
    schedule = [int(b) for b in args.bit_schedule.split(",")] if args.bit_schedule else None
    tdt = torch.bfloat16 if bf16 else torch.float16

    def to_dev(a):
        """host input (fp16 values, or bf16 bit patterns) -> device tensor of the input type"""
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16) if bf16 else np.ascontiguousarray(a))
        return (t.view(torch.bfloat16) if bf16 else t).to(dev)
    lens = synth.prefill_lengths(w)
    S = int(lens.max())
    T = w.steps
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    # ---- inputs, generated on the host and made resident in HBM
    t0 = time.time()
    gpk, gpv = synth.group_params(w, 0), synth.group_params(w, 1)
    kpre = torch.zeros((w.batch, w.n_kv_heads, S, w.head_dim), dtype=tdt, device=dev)
    vpre = torch.zeros_like(kpre)
    kdec = torch.empty((T, w.batch, w.n_kv_heads, 1, w.head_dim), dtype=tdt, device=dev)
    vdec = torch.empty_like(kdec)
    host_k0 = host_v0 = None
    for b in range(w.batch):
        kb = synth.kv_sequence(w, 0, b, int(lens[b]) + T, gpk, bf16)
        vb = synth.kv_sequence(w, 1, b, int(lens[b]) + T, gpv, bf16)
        kpre[b, :, :lens[b]] = to_dev(kb[:, :lens[b]])
        vpre[b, :, :lens[b]] = to_dev(vb[:, :lens[b]])
        kdec[:, b, :, 0] = to_dev(kb[:, lens[b]:].transpose(1, 0, 2))
        vdec[:, b, :, 0] = to_dev(vb[:, lens[b]:].transpose(1, 0, 2))
        if b == 0:
            host_k0, host_v0 = kb, vb
    q_host = np.stack([synth.queries(w, b, T, bf16) for b in range(w.batch)], axis=1)
    q_all = to_dev(q_host)
    # prefill queries: one per prompt position and query head
    qpre = torch.zeros((w.batch, w.n_q_heads, S, w.head_dim), dtype=tdt, device=dev)
    for b in range(w.batch):
        qpre[b, :, :lens[b]] = to_dev(synth.prefill_queries(w, b, int(lens[b]), bf16))
    gen_s = time.time() - t0

    cache = LatentKVCache(w.head_dim, w.n_kv_heads, w.n_q_heads, w.n_head_groups, w.batch,
                          S + T, rank=args.per_seq_rank or w.rank or 0, energy_threshold=w.energy,
                          quantize_values=w.quantize_values, input_dtype=args.input_dtype,
                          bit_schedule=schedule, per_seq_basis=args.per_seq_rank > 0)
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=tdt, device=dev)
    out_pre = torch.empty_like(qpre)
    stream = torch.cuda.current_stream(dev)

    # every timing event of a pass is created up front, so that no event
    # creation sits between the calls it brackets
    pass_events = [[tuple(TimingEvent() for _ in range(3)) for _ in range(T)] + [tuple(TimingEvent() for _ in range(3))]
                   for _ in range(args.steps + args.warmup)]

    def one_pass(pi):
        ev = []
        torch.cuda.synchronize()       # the fit is host-synchronous: time it alone
        t_fit = time.perf_counter()
        cache.fit(kpre, vpre, lens)
        t_fit = time.perf_counter() - t_fit
        e_enc0, e_enc1, e_pre1 = pass_events[pi][T]
        # the fit left the GPU idle: a short spin on the stream keeps it busy
        # while the host records the event and launches the encode, so the
        # events bracket the encode's device time, not the host's launch path
        torch.cuda._sleep(ENCODE_LEAD_CYCLES)
        e_enc0.record(stream)
        cache.encode_append(kpre, vpre, n_new=lens)
        e_enc1.record(stream)
        cache.prefill_attend(qpre, n_q=lens, out=out_pre)
        e_pre1.record(stream)
        for t in range(T):
            ea, eb, ec = pass_events[pi][t]
            ea.record(stream)
            cache.encode_append(kdec[t], vdec[t])
            eb.record(stream)
            cache.decode_attend(q_all[t], out=out)
            ec.record(stream)
            ev.append((ea, eb, ec))
        return t_fit, (e_enc0, e_enc1, e_pre1), ev

    for wi in range(args.warmup):
        one_pass(args.steps + wi)
    torch.cuda.synchronize()

    fit_s, enc_ms, pre_ms, app_ms, att_ms = [], [], [], [], []
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    results = [one_pass(pi) for pi in range(args.steps)]
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    for t_fit, (e0, e1, e2), ev in results:
        fit_s.append(t_fit)
        enc_ms.append(e0.elapsed_time(e1))
        pre_ms.append(e1.elapsed_time(e2))
        for ea, eb, ec in ev:
            app_ms.append(ea.elapsed_time(eb))
            att_ms.append(eb.elapsed_time(ec))

    st = cache.stats()
    rk, rv, nhk, nhv = st["r_k"], st["r_v"], st["n_hi_k"], st["n_hi_v"]
    from rank_latent_kv_amd.palu import palu_record_words
    wk, wv = palu_record_words(cache.handle, 0), palu_record_words(cache.handle, 1)
    per_call_bytes = [attend_bytes([int(n) + t + 1 for n in lens], w.n_kv_heads, w.n_q_heads,
                                   w.head_dim, w.n_head_groups, wk, st["coded_k"], wv, st["coded_v"],
                                   w.quantize_values, w.batch if args.per_seq_rank else 1) for t in range(T)]
    mean_bytes = float(np.mean(per_call_bytes))
    att_mean_ms = float(np.mean(att_ms))
    decode_tok_s = w.batch * len(att_ms) / (sum(att_ms) / 1e3)
    achieved_gbps = mean_bytes / (att_mean_ms / 1e3) / 1e9
    enc_positions = float(lens.sum())
    encode_mtok_s = enc_positions / (float(np.mean(enc_ms)) / 1e3) / 1e6

    pairs = float(sum(int(n) * (int(n) + 1) // 2 for n in lens)) * w.n_q_heads
    pre_mean_ms = float(np.mean(pre_ms))
    pre_ops = pairs * PREFILL_OPS_PER_PAIR / (pre_mean_ms / 1e3) / 1e12

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, cache, host_k0, host_v0, lens, q_host[0, 0], bf16, schedule,
                           seq=0 if args.per_seq_rank else None)

    line = {
        "metric": METRIC,
        "value": round(decode_tok_s, 1),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "prefill": S, "decode_steps": T,
                   "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "head_groups": w.n_head_groups,
                   "rank_k": rk, "rank_v": rv, "quantize_values": w.quantize_values,
                   "input_dtype": args.input_dtype,
                   "bit_schedule": schedule if schedule else "palu 25% x 4 bit + 75% x 2 bit",
                   "bases": "per sequence" if args.per_seq_rank else "shared per head group"},
        "roofline": {"bound": "hbm", "kernel": "palu_decode_attend (attend + combine)",
                     "achieved": round(achieved_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved_gbps / HBM_PEAK_GBPS, 4), "traffic": measured_traffic(w.name) if not (bf16 or schedule or args.per_seq_rank) else None,
                     "bytes_per_launch": int(mean_bytes), "launch_us": round(att_mean_ms * 1e3, 2)},
        "decode_attend_us": round(att_mean_ms * 1e3, 2),
        "append_us": round(float(np.mean(app_ms)) * 1e3, 2),
        "encode_mtok_s": round(encode_mtok_s, 2),
        "prefill_attend": {"ms": round(pre_mean_ms, 3), "score_pairs_per_s": round(pairs / (pre_mean_ms / 1e3), 1),
                           "tok_per_s": round(float(lens.sum()) / (pre_mean_ms / 1e3), 1),
                           "roofline": {"bound": "alu", "achieved": round(pre_ops, 2),
                                        "peak": round(VALU_PEAK_TOPS, 2), "unit": "T lane-op/s",
                                        "frac": round(pre_ops / VALU_PEAK_TOPS, 4),
                                        "ops_per_pair": PREFILL_OPS_PER_PAIR}},
        "encode_ms": round(float(np.mean(enc_ms)), 3),
        "fit_ms": round(float(np.mean(fit_s)) * 1e3, 2),
        "input_gen_s": round(gen_s, 1),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(w, cache, k0, v0, lens, q0, bf16=False, schedule=None, seq=None, budget_s=10.0):
    """The oracle's decode attention (dequantise the stored records,
    reconstruct K/V in fp64, softmax per query head) for the first decode step
    of sequence 0 with the GPU's basis, repeated until about `budget_s`
    seconds of single-threaded CPU time have been spent (at least 3 runs)."""
    import oracle
    fits = []
    for t in (0, 1):
        r, basis, mu, sigma = cache.get_basis(t, seq=seq)
        full = np.zeros((w.n_head_groups, w.head_dim, w.head_dim), np.float32)
        full[:, :, :r] = basis
        fits.append(oracle.Fit(r, np.full(w.n_head_groups, r, np.int32), full, mu, sigma))
    layer = oracle.OracleLayer(w.head_dim, w.n_q_heads, w.n_kv_heads, w.n_head_groups, *fits,
                               quantize_values=w.quantize_values, bf16=bf16, schedule=schedule)
    n = int(lens[0]) + 1
    ks = [layer.encode_head(k0[h, :n], h, 0) for h in range(w.n_kv_heads)]
    vs = [layer.encode_head(v0[h, :n], h, 1) for h in range(w.n_kv_heads)]
    q = np.ascontiguousarray(q0)
    runs, t0 = 0, time.perf_counter()
    while runs < 3 or time.perf_counter() - t0 < budget_s:
        layer.attend(ks, vs, q)
        runs += 1
    dt = time.perf_counter() - t0
    return {"value": round(runs / dt, 4), "unit": "tok/s", "cores": 1, "kind": "oracle",
            "sample": f"{runs} x decode-attend of sequence 0 at its first decode step "
                      f"({w.n_q_heads} query heads over {n} tokens, fp64), "
                      f"{dt:.1f} s single-threaded"}


if __name__ == "__main__":
    main()
