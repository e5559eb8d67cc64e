"""Benchmark of the latent KV cache hot path on one MI355X.

Headline step (the long-context workload: 4 sequences x 32768 prefill
tokens, 32 query / 8 kv heads, D = 128, 4 head groups, 90%-energy rank,
64 decode steps):
  fit (Gram kernels + host eigensolve) -> encode of the prefill ->
  causal prefill attention of every prompt position over the latent cache ->
  64 x (append one token per sequence -> decode-attend).
All inputs are resident in HBM before the timed region.

`value` is decode-attend throughput: sequences x decode steps per second of
decode-attend time, measured with HIP events recorded on the stream the
library launches on, around every decode-attend call of the steps above
(warm: the calls run back to back, as decode does, and the call's few MB
stay in the last-level cache).  The events are created without the
system-scope fence a default HIP event adds.  Next to it the line reports:
  * decode_attend: the same call timed warm in a decode-only loop and cold,
    each call preceded (outside its events) by a 1 GiB read that evicts the
    256 MB last-level cache, with algorithmic bytes per second against the
    8 TB/s HBM peak;
  * read_bandwidth: what a plain 16-byte-load stream over 1 GiB reaches on
    the same device (the library's read probe);
  * workloads: decode-only warm and cold times, bytes and bandwidth, the
    prefill encode rate and the prefill attention time (back-to-back calls),
    for each of the five workloads;
  * encode_roofline: the prefill encode against HBM (fp16 K/V read, records
    and tails written) and against the non-packed fp32 VALU issue rate;
  * prefill_attend: time inside the step and causal score pairs per second
    against the VALU issue rate (3.5 lane-operation slots per pair);
  * cpu_baseline: the oracle on the host cores (decode, encode, fit), one
    thread and all threads of the job's CPU share.

    python bench.py [--steps K] [--warmup W] [--workload NAME]
                    [--workloads all|none|NAME,...] [--no-cpu-baseline]
"""
import argparse
import json
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
# Vector issue slots a causal softmax pair needs at least, in lane
# operations: one exp2 (a transcendental, issued at half the rate: two
# slots), one running-max comparison and half of an fp32 -> fp16 pair
# conversion (the two contractions run on the matrix cores).
PREFILL_OPS_PER_PAIR = 3.5
METRIC = "latent decode-attend tok/s + HBM GB/s (% of peak); encode Mtok/s"
# Host threads a benchmark job may use (a CPU share of 16 threads per GPU).
MAX_HOST_THREADS = 16
FLUSH_BYTES = 1 << 30          # > 256 MB last-level cache
PROBE_GRID = 4096


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


def encode_bytes(lens, H, D, wk, rk, wv, rv, vq):
    """Algorithmic bytes of a prefill encode: fp16 K and V read, complete
    records and tail latents written (fp16 value latents: 2 r_v bytes per
    token)."""
    lens = [int(m) for m in lens]
    rd = 2 * sum(lens) * H * D * 2
    wr = sum(H * ((m // 32) * wk * 4 + (m % 32) * rk * 4) for m in lens)
    wr += sum(H * (((m // 32) * wv * 4 + (m % 32) * rv * 4) if vq else m * rv * 2) for m in lens)
    return rd + wr


KERNEL_SRC = os.path.join(ROOT, "rank_latent_kv_amd", "csrc", "palu_decode.hip")
PROFILE = os.path.join(ROOT, "profiles", "decode_attend_long_b4_s32768_e90.md")

# GPU clock cycles of the spin queued ahead of the prefill encode's start
# event (about 200 us: the host's launch path, about 30 us, now and then
# took longer than a 50 us lead and the wait entered the encode's events)
ENCODE_LEAD_CYCLES = 480_000


def measured_traffic(workload):
    """HBM bytes per decode-attend call from the committed counter summary
    (rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE runs, scaled by the
    copy-kernel calibration), if it was taken for this workload on the
    current kernel source; else None."""
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


def host_threads():
    return max(1, min(MAX_HOST_THREADS, len(os.sched_getaffinity(0))))


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


class Flush:
    """A 1 GiB device buffer read by the library's read probe: evicts the
    last-level cache, and times the device's plain read bandwidth."""

    def __init__(self, torch, dev):
        self.torch = torch
        self.buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.int32, device=dev)
        self.sink = torch.zeros(PROBE_GRID, dtype=torch.int32, device=dev)

    def run(self, stream, grid=PROBE_GRID):
        from rank_latent_kv_amd.palu import palu_probe_read
        palu_probe_read(self.buf.data_ptr(), FLUSH_BYTES, self.sink.data_ptr(), grid, stream.cuda_stream)

    def bandwidth(self, stream, reps=10):
        best = None
        for grid in (1024, 2048, PROBE_GRID):
            evs = [(TimingEvent(), TimingEvent()) for _ in range(reps + 2)]
            for a, b in evs:
                a.record(stream)
                self.run(stream, grid)
                b.record(stream)
            self.torch.cuda.synchronize()
            ms = sorted(a.elapsed_time(b) for a, b in evs[2:])
            gbps = FLUSH_BYTES / (ms[len(ms) // 2] / 1e3) / 1e9
            if best is None or gbps > best[0]:
                best = (gbps, grid, ms[len(ms) // 2])
        return {"gbps": round(best[0], 1), "frac_of_peak": round(best[0] / HBM_PEAK_GBPS, 4),
                "bytes": FLUSH_BYTES, "grid": best[1], "us": round(best[2] * 1e3, 1),
                "kernel": "palu_probe_read: grid-stride 16-byte loads, 256 threads per workgroup, median of "
                          f"{reps} launches, best of grids 1024/2048/{PROBE_GRID}"}


def time_decode(torch, cache, q, out, stream, n, flush=None):
    """Mean milliseconds of n decode-attend calls on the cache's current
    state, each between its own events; with flush, every call is preceded
    (outside the events) by the 1 GiB read."""
    evs = [(TimingEvent(), TimingEvent()) for _ in range(n)]
    cache.decode_attend(q, out=out)                 # one untimed call
    for a, b in evs:
        if flush is not None:
            flush.run(stream)
        a.record(stream)
        cache.decode_attend(q, out=out)
        b.record(stream)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in evs]
    return float(np.mean(ms)), float(np.median(ms))


# Steps the cache holds room for after the timed passes: the eager and
# graph-replayed decode steps of time_step_graph append one token each.
GRAPH_STEPS = 48


def time_step_graph(torch, cache, k_new, v_new, q, stream, n_eager=8, n_graph=8, n_replay=3):
    """One decode step (palu_decode_step: one-token append per row, then
    decode-attend) run eagerly, then n_graph steps captured in one HIP graph
    (torch.cuda.graph over the library's launches on the capture stream) and
    replayed n_replay times, and a one-step graph replayed n_replay times:
    mean time per step between fence-free events.  Appends
    n_eager + (n_graph + 1) n_replay tokens (within GRAPH_STEPS) and
    resynchronises the host's lengths afterwards."""
    out = torch.empty_like(q)
    evs = [(TimingEvent(), TimingEvent()) for _ in range(n_eager + 2 * n_replay)]

    def timed(i, fn):
        a, b = evs[i]
        a.record(stream)
        fn()
        b.record(stream)
        return a, b

    eager = [timed(i, lambda: cache.decode_step(k_new, v_new, q, out)) for i in range(n_eager)]
    torch.cuda.synchronize()
    graphs = []
    for n in (n_graph, 1):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n):
                cache.decode_step(k_new, v_new, q, out)
        torch.cuda.synchronize()
        graphs.append(g)
    multi = [timed(n_eager + i, graphs[0].replay) for i in range(n_replay)]
    single = [timed(n_eager + n_replay + i, graphs[1].replay) for i in range(n_replay)]
    torch.cuda.synchronize()
    cache.sync_lengths()
    del graphs
    us = lambda pairs, n: float(np.mean([a.elapsed_time(b) for a, b in pairs])) * 1e3 / n
    return {"eager_us": round(us(eager[1:], 1), 2), "graph_us": round(us(multi, n_graph), 2),
            "graph_steps": n_graph, "one_step_graph_us": round(us(single, 1), 2),
            "note": "per step: one-token append of every sequence + decode-attend (palu_decode_step): "
                    "launched eagerly; as one captured graph of graph_steps steps (time per step); as a "
                    "captured graph of one step (time per replay, which includes the graph launch)"}


def gen_inputs(w, n_extra, bf16=False):
    """Host K/V of every sequence (prefill + n_extra positions), generated on
    host threads: two lists of fp16 [H, len + n_extra, D] arrays."""
    from concurrent.futures import ThreadPoolExecutor
    lens = synth.prefill_lengths(w)
    gp = (synth.group_params(w, 0), synth.group_params(w, 1))
    with ThreadPoolExecutor(host_threads()) as pool:
        out = [list(pool.map(lambda b: synth.kv_sequence(w, t, b, int(lens[b]) + n_extra, gp[t], bf16),
                             range(w.batch))) for t in (0, 1)]
    return lens, out


def workload_prefill(torch, dev, stream, cache, w, lens, n_calls=3):
    """Causal prefill attention of every prompt position over the encoded
    prompt: mean ms of n_calls back-to-back calls after one untimed call."""
    from concurrent.futures import ThreadPoolExecutor
    S = int(lens.max())
    qpre = torch.zeros((w.batch, w.n_q_heads, S, w.head_dim), dtype=torch.float16, device=dev)
    with ThreadPoolExecutor(host_threads()) as pool:
        for b, qb in enumerate(pool.map(lambda b: synth.prefill_queries(w, b, int(lens[b])), range(w.batch))):
            qpre[b, :, :lens[b]] = torch.from_numpy(qb).to(dev)
    out = torch.empty_like(qpre)
    cache.prefill_attend(qpre, n_q=lens, out=out)
    evs = [(TimingEvent(), TimingEvent()) for _ in range(n_calls)]
    for e0, e1 in evs:
        e0.record(stream)
        cache.prefill_attend(qpre, n_q=lens, out=out)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
    del qpre, out
    return ms


def workload_decode(torch, dev, stream, flush, w, n_warm=32, n_cold=16):
    """One workload's decode-only figures: fit and encode the prefill, time
    the prefill attention, append one token per sequence, then time
    decode-attend warm and cold."""
    from rank_latent_kv_amd.palu import LatentKVCache, palu_record_words
    t0 = time.time()
    lens, host = gen_inputs(w, 1)
    S = int(lens.max())
    kpre = torch.zeros((w.batch, w.n_kv_heads, S, w.head_dim), dtype=torch.float16, device=dev)
    vpre = torch.zeros_like(kpre)
    knew = torch.empty((w.batch, w.n_kv_heads, 1, w.head_dim), dtype=torch.float16, device=dev)
    vnew = torch.empty_like(knew)
    for b in range(w.batch):
        n = int(lens[b])
        kpre[b, :, :n] = torch.from_numpy(host[0][b][:, :n]).to(dev)
        vpre[b, :, :n] = torch.from_numpy(host[1][b][:, :n]).to(dev)
        knew[b] = torch.from_numpy(np.ascontiguousarray(host[0][b][:, n:n + 1])).to(dev)
        vnew[b] = torch.from_numpy(np.ascontiguousarray(host[1][b][:, n:n + 1])).to(dev)
    del host
    gen_s = time.time() - t0
    cache = LatentKVCache(w.head_dim, w.n_kv_heads, w.n_q_heads, w.n_head_groups, w.batch, S + 1,
                          rank=w.rank or 0, energy_threshold=w.energy, quantize_values=w.quantize_values)
    cache.fit(kpre, vpre, lens)
    enc_ms = []
    for _ in range(3):
        cache.reset()
        e0, e1 = TimingEvent(), TimingEvent()
        torch.cuda._sleep(ENCODE_LEAD_CYCLES)
        e0.record(stream)
        cache.encode_append(kpre, vpre, n_new=lens)
        e1.record(stream)
        torch.cuda.synchronize()
        enc_ms.append(e0.elapsed_time(e1))
    pre_ms = workload_prefill(torch, dev, stream, cache, w, lens)
    pairs = w.n_q_heads * float(np.sum(lens.astype(np.float64) * (lens + 1) / 2))
    cache.encode_append(knew, vnew)
    q = torch.from_numpy(np.stack([synth.queries(w, b, 1)[0] for b in range(w.batch)])).to(dev)
    out = torch.empty_like(q)
    warm_mean, warm_med = time_decode(torch, cache, q, out, stream, n_warm)
    cold_mean, cold_med = time_decode(torch, cache, q, out, stream, n_cold, flush)
    st = cache.stats()
    wk, wv = palu_record_words(cache.handle, 0), palu_record_words(cache.handle, 1)
    nb = attend_bytes([int(n) + 1 for n in lens], w.n_kv_heads, w.n_q_heads, w.head_dim, w.n_head_groups,
                      wk, st["coded_k"], wv, st["coded_v"], w.quantize_values)
    eb = encode_bytes(lens, w.n_kv_heads, w.head_dim, wk, st["coded_k"], wv, st["coded_v"], w.quantize_values)
    enc = float(np.median(enc_ms))
    res = {"rank_k": st["r_k"], "rank_v": st["r_v"], "bytes_per_call": int(nb),
           "warm_us": round(warm_mean * 1e3, 2), "warm_gbps": round(nb / (warm_mean / 1e3) / 1e9, 1),
           "warm_frac": round(nb / (warm_mean / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
           "cold_us": round(cold_mean * 1e3, 2), "cold_gbps": round(nb / (cold_mean / 1e3) / 1e9, 1),
           "cold_frac": round(nb / (cold_mean / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
           "decode_tok_s_warm": round(w.batch / (warm_mean / 1e3), 1),
           "encode_ms": round(enc, 4), "encode_mtok_s": round(float(lens.sum()) / (enc / 1e3) / 1e6, 2),
           "encode_gbps": round(eb / (enc / 1e3) / 1e9, 1),
           "prefill_ms": round(pre_ms, 3), "prefill_pairs_per_s": round(pairs / (pre_ms / 1e3), 1),
           "input_gen_s": round(gen_s, 1)}
    del cache, kpre, vpre
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="long_b4_s32768_e90")
    ap.add_argument("--workloads", default="all",
                    help="decode-only figures for: all (the five workloads), none, or a comma-separated list")
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
    variant = bool(bf16 or schedule or args.per_seq_rank)
    tdt = torch.bfloat16 if bf16 else torch.float16
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    def to_dev(a):
        """host input (fp16 values, or bf16 bit patterns) -> device tensor of the input type"""
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16) if bf16 else np.ascontiguousarray(a))
        return (t.view(torch.bfloat16) if bf16 else t).to(dev)
    T = w.steps

    # ---- inputs, generated on the host and made resident in HBM
    t0 = time.time()
    lens, host = gen_inputs(w, T, bf16)
    S = int(lens.max())
    kpre = torch.zeros((w.batch, w.n_kv_heads, S, w.head_dim), dtype=tdt, device=dev)
    vpre = torch.zeros_like(kpre)
    kdec = torch.empty((T, w.batch, w.n_kv_heads, 1, w.head_dim), dtype=tdt, device=dev)
    vdec = torch.empty_like(kdec)
    for b in range(w.batch):
        kb, vb = host[0][b], host[1][b]
        kpre[b, :, :lens[b]] = to_dev(kb[:, :lens[b]])
        vpre[b, :, :lens[b]] = to_dev(vb[:, :lens[b]])
        kdec[:, b, :, 0] = to_dev(kb[:, lens[b]:].transpose(1, 0, 2))
        vdec[:, b, :, 0] = to_dev(vb[:, lens[b]:].transpose(1, 0, 2))
    q_host = np.stack([synth.queries(w, b, T, bf16) for b in range(w.batch)], axis=1)
    q_all = to_dev(q_host)
    # prefill queries: one per prompt position and query head
    qpre = torch.zeros((w.batch, w.n_q_heads, S, w.head_dim), dtype=tdt, device=dev)
    for b in range(w.batch):
        qpre[b, :, :lens[b]] = to_dev(synth.prefill_queries(w, b, int(lens[b]), bf16))
    gen_s = time.time() - t0

    cache = LatentKVCache(w.head_dim, w.n_kv_heads, w.n_q_heads, w.n_head_groups, w.batch,
                          S + T + GRAPH_STEPS, rank=args.per_seq_rank or w.rank or 0, energy_threshold=w.energy,
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
    rk, rv = st["r_k"], st["r_v"]
    from rank_latent_kv_amd.palu import palu_record_words
    wk, wv = palu_record_words(cache.handle, 0), palu_record_words(cache.handle, 1)
    basis_sets = w.batch if args.per_seq_rank else 1
    per_call_bytes = [attend_bytes([int(n) + t + 1 for n in lens], w.n_kv_heads, w.n_q_heads,
                                   w.head_dim, w.n_head_groups, wk, st["coded_k"], wv, st["coded_v"],
                                   w.quantize_values, basis_sets) for t in range(T)]
    mean_bytes = float(np.mean(per_call_bytes))
    att_mean_ms = float(np.mean(att_ms))
    decode_tok_s = w.batch * len(att_ms) / (sum(att_ms) / 1e3)
    achieved_gbps = mean_bytes / (att_mean_ms / 1e3) / 1e9
    enc_positions = float(lens.sum())
    enc_mean_ms = float(np.mean(enc_ms))
    encode_mtok_s = enc_positions / (enc_mean_ms / 1e3) / 1e6
    eb = encode_bytes(lens, w.n_kv_heads, w.head_dim, wk, st["coded_k"], wv, st["coded_v"], w.quantize_values)
    enc_gbps = eb / (enc_mean_ms / 1e3) / 1e9
    # fixed-order fp32 projection: one fma lane operation per (position,
    # kv head, coded channel, d)
    enc_ops = enc_positions * w.n_kv_heads * (st["coded_k"] + st["coded_v"]) * w.head_dim
    enc_tops = enc_ops / (enc_mean_ms / 1e3) / 1e12

    pairs = float(sum(int(n) * (int(n) + 1) // 2 for n in lens)) * w.n_q_heads
    pre_mean_ms = float(np.mean(pre_ms))
    pre_ops = pairs * PREFILL_OPS_PER_PAIR / (pre_mean_ms / 1e3) / 1e12

    # ---- decode-only loops on the final state: warm, and cold (1 GiB read
    #      before every call, outside its events); device read bandwidth
    flush = Flush(torch, dev)
    read_bw = flush.bandwidth(stream)
    q_last = q_all[T - 1]
    dw_mean, dw_med = time_decode(torch, cache, q_last, out, stream, 64)
    dc_mean, dc_med = time_decode(torch, cache, q_last, out, stream, 32, flush)
    last_bytes = per_call_bytes[-1]
    decode_only = {
        "bytes_per_call": int(last_bytes),
        "warm_us": round(dw_mean * 1e3, 2), "warm_median_us": round(dw_med * 1e3, 2),
        "warm_gbps": round(last_bytes / (dw_mean / 1e3) / 1e9, 1),
        "warm_frac": round(last_bytes / (dw_mean / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
        "cold_us": round(dc_mean * 1e3, 2), "cold_median_us": round(dc_med * 1e3, 2),
        "cold_gbps": round(last_bytes / (dc_mean / 1e3) / 1e9, 1),
        "cold_frac": round(last_bytes / (dc_mean / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
        "cold_frac_of_read_bw": round(last_bytes / (dc_mean / 1e3) / 1e9 / read_bw["gbps"], 4),
        "note": "warm: 64 back-to-back calls (working set resident in the 256 MB last-level cache); "
                "cold: 32 calls, each after a 1 GiB read (outside the events) that evicts that cache"}
    rg, ep, ea = ([], [], [])
    fit_info = None
    if not args.per_seq_rank:
        fit_info = {}
        for t, name in ((0, "k"), (1, "v")):
            rg, ep, ea = cache.fit_info(t)
            fit_info[name] = {"rank": int(st["r_" + name]), "group_ranks": [int(x) for x in rg],
                              "energy_at_r": [round(float(x), 6) for x in ea],
                              "energy_at_r_minus_1": [round(float(x), 6) for x in ep],
                              "margin": round(float(st["energy_margin_" + name]), 6)}

    step_graph = time_step_graph(torch, cache, kdec[T - 1], vdec[T - 1], q_last, stream)

    workloads = {}
    if not variant and args.workloads != "none":
        names = list(synth.WORKLOADS) if args.workloads == "all" else args.workloads.split(",")
        held = (kpre, vpre, qpre, out_pre)
        del kpre, vpre, qpre, out_pre, held
        torch.cuda.empty_cache()
        for name in names:
            workloads[name] = workload_decode(torch, dev, stream, flush, synth.WORKLOADS[name])
            print(f"# workload {name}: {json.dumps(workloads[name])}", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, cache, host, lens, q_host[0], bf16, schedule,
                           per_seq=bool(args.per_seq_rank))

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
        "dtype": "fp16 mfma operands, fp32 accumulate",
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
                     "frac": round(achieved_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(w.name) if not variant else None,
                     "traffic_source": "rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE runs of this kernel source "
                                       "(profiles/decode_attend_long_b4_s32768_e90.md), scaled by a plain copy",
                     "bytes_per_launch": int(mean_bytes), "launch_us": round(att_mean_ms * 1e3, 2),
                     "cache": "warm (steps back to back); cold figures under decode_attend"},
        "decode_attend": decode_only,
        "read_bandwidth": read_bw,
        "decode_attend_us": round(att_mean_ms * 1e3, 2),
        "append_us": round(float(np.mean(app_ms)) * 1e3, 2),
        "decode_step_graph": step_graph,
        "encode_mtok_s": round(encode_mtok_s, 2),
        "encode_ms": round(enc_mean_ms, 4),
        "encode_roofline": {"bound": "hbm", "achieved": round(enc_gbps, 1), "peak": HBM_PEAK_GBPS,
                            "unit": "GB/s", "frac": round(enc_gbps / HBM_PEAK_GBPS, 4),
                            "bytes_per_launch": int(eb),
                            "valu": {"achieved": round(enc_tops, 2), "peak": round(VALU_PEAK_TOPS, 2),
                                     "unit": "T lane-op/s", "frac": round(enc_tops / VALU_PEAK_TOPS, 4),
                                     "ops": "one fp32 fma per (position, kv head, coded channel, d)"}},
        "prefill_attend": {"ms": round(pre_mean_ms, 3), "score_pairs_per_s": round(pairs / (pre_mean_ms / 1e3), 1),
                           "tok_per_s": round(float(lens.sum()) / (pre_mean_ms / 1e3), 1),
                           "roofline": {"bound": "alu", "achieved": round(pre_ops, 2),
                                        "peak": round(VALU_PEAK_TOPS, 2), "unit": "T lane-op/s",
                                        "frac": round(pre_ops / VALU_PEAK_TOPS, 4),
                                        "ops_per_pair": PREFILL_OPS_PER_PAIR}},
        "fit_ms": round(float(np.mean(fit_s)) * 1e3, 2),
        "fit_rank_rule": fit_info,
        "workloads": workloads,
        "input_gen_s": round(gen_s, 1),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(w, cache, host, lens, q0, bf16=False, schedule=None, per_seq=False):
    """The plain oracle on the host, one thread and all threads of the job's
    CPU share (independent (sequence, kv head) or (tensor, group) problems on
    a thread pool; the oracle's C routines release the interpreter lock):
      * encode: the oracle's projection + quantisation of every kv head of
        K and V (sequence 0 on one thread, the other sequences on the pool);
      * decode: one decode step's attention (dequantise, reconstruct in fp64,
        softmax per query head) with the GPU's basis, at the first decode
        position: sequence 0 on one thread, every sequence on the pool;
      * fit: the oracle fit of one (tensor, group) on one thread, all of
        them on the pool (shared bases only)."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    nthr = host_threads()
    seqs = list(range(w.batch))
    fits = []
    for t in (0, 1):
        r, basis, mu, sigma = cache.get_basis(t, seq=0 if per_seq else None)
        full = np.zeros((w.n_head_groups, w.head_dim, w.head_dim), np.float32)
        full[:, :, :r] = basis
        fits.append(oracle.Fit(r, np.full(w.n_head_groups, r, np.int32), full, mu, sigma))
    layer = oracle.OracleLayer(w.head_dim, w.n_q_heads, w.n_kv_heads, w.n_head_groups, *fits,
                               quantize_values=w.quantize_values, bf16=bf16, schedule=schedule)
    H, g = w.n_kv_heads, w.gqa

    def enc_job(job):
        b, h = job
        n = int(lens[b]) + 1
        return (layer.encode_head(host[0][b][h, :n], h, 0), layer.encode_head(host[1][b][h, :n], h, 1))

    # encode: sequence 0 on one thread, the rest on the pool
    t0 = time.perf_counter()
    states = {(0, h): enc_job((0, h)) for h in range(H)}
    enc1 = time.perf_counter() - t0
    rest = [(b, h) for b in seqs[1:] for h in range(H)]
    t0 = time.perf_counter()
    with ThreadPoolExecutor(nthr) as pool:
        states.update(zip(rest, pool.map(enc_job, rest)))
    encn = time.perf_counter() - t0 if rest else None
    n_rest = float(sum(int(lens[b]) + 1 for b in seqs[1:]))

    scale = 1.0 / np.sqrt(w.head_dim)
    qf = oracle.bf16_to_float(q0) if bf16 else q0

    def dec_job(job):
        b, h = job
        ks, vs = states[(b, h)]
        lk, lv = layer.decode_head(ks, 0), layer.decode_head(vs, 1)
        grp = layer.group_of(h)
        fK, fV = layer.fit
        return [oracle.attend(lk, fK.V(grp), fK.mu[grp], lv, fV.V(grp), fV.mu[grp], qf[b, i], scale)
                for i in range(h * g, (h + 1) * g)]

    # decode: one step of sequence 0 on one thread, repeated ~8 s
    runs, t0 = 0, time.perf_counter()
    while runs < 2 or time.perf_counter() - t0 < 8.0:
        for h in range(H):
            dec_job((0, h))
        runs += 1
    dec1 = (time.perf_counter() - t0) / runs
    jobs = [(b, h) for b in seqs for h in range(H)]
    runs_n, t0 = 0, time.perf_counter()
    with ThreadPoolExecutor(nthr) as pool:
        while runs_n < 2 or time.perf_counter() - t0 < 6.0:
            list(pool.map(dec_job, jobs))
            runs_n += 1
    decn = (time.perf_counter() - t0) / runs_n

    fit_1 = fit_n = None
    if not per_seq:
        hpg = w.n_kv_heads // w.n_head_groups
        S = int(lens.max())

        def fit_job(job):
            t, grp = job
            x = np.zeros((w.batch, hpg, S, w.head_dim), host[t][0].dtype)
            for b in seqs:
                x[b, :, :lens[b]] = host[t][b][grp * hpg:(grp + 1) * hpg, :lens[b]]
            t1 = time.perf_counter()
            oracle.fit_group(x, lens, 1, 0, rank=w.rank or 0, tau=w.energy, bf16=bf16)
            return time.perf_counter() - t1

        fit_1 = fit_job((0, 0))
        fjobs = [(t, grp) for t in (0, 1) for grp in range(w.n_head_groups)]
        t0 = time.perf_counter()
        with ThreadPoolExecutor(nthr) as pool:
            list(pool.map(fit_job, fjobs))
        fit_n = time.perf_counter() - t0
    n_pos0 = int(lens[0]) + 1
    return {"value": round(w.batch / decn, 4), "unit": "tok/s", "cores": nthr, "kind": "oracle",
            "sample": f"decode-attend of all {w.batch} sequences at their first decode position "
                      f"({w.n_q_heads} query heads each, fp64), {runs_n} runs on {nthr} threads",
            "nproc": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "single_thread": {"value": round(1.0 / dec1, 4), "unit": "tok/s", "cores": 1,
                              "sample": f"sequence 0, {runs} runs"},
            "encode_mtok_s": {"cores_1": round(n_pos0 / enc1 / 1e6, 6),
                              f"cores_{nthr}": round(n_rest / encn / 1e6, 6) if encn else None,
                              "sample": f"every kv head of K and V: sequence 0 ({n_pos0} positions) on one "
                                        f"thread, the other {w.batch - 1} on {nthr} threads"},
            "fit_ms": None if fit_1 is None else
            {"one_group_cores_1": round(fit_1 * 1e3, 1),
             "all_groups_extrapolated_cores_1": round(fit_1 * 2 * w.n_head_groups * 1e3, 1),
             f"all_groups_cores_{nthr}": round(fit_n * 1e3, 1),
             "sample": f"fp64 two-pass scatter + Jacobi per (tensor, group); {2 * w.n_head_groups} problems"}}


if __name__ == "__main__":
    main()
