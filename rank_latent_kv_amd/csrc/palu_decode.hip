// Decode attention over the latent cache, for gfx950 (MI355X).
//
//   attend_kernel / combine_kernel : single-query decode attention computed
//       from the stored latents (PALU page, "How it works", decode step 3)
//       with the query absorbed into the key basis, split over token ranges,
//       then merged by log-sum-exp and projected back with the value basis.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>
#include <type_traits>

#include "palu_device.h"
#include "palu_internal.h"

namespace palu {

namespace {

// -------------------------------------------------------------- attend ----
//
// Workgroup = (kv head h, call row i, split s).  Split s covers complete
// token groups [s*chunk, min(nfull, (s+1)*chunk)); the last split also
// covers the incomplete group (fp32 tail latents).  With the query absorbed
// into the key basis, score_t = qs * q . (V_K l_t + mu_K) = qt . l_t + const
// with qt = qs V_K^T q (qs = scale * log2 e); the constant q . mu_K is the
// same for every token of a head and cancels in the softmax.
//
// Each wave owns 16 "streams" n = slot * g + head: per iteration it takes
// S = 16 / g consecutive token groups (slots) and runs, for both 16-token
// halves of the groups,
//   scores  D[t][n] = sum_k A[t][k] B[k][n]    (v_mfma_f32_16x16x32_f16)
// where k runs over (slot, 8-channel block) pairs, A holds the token's
// latents of that block dequantised to fp16 (code * scale16 + zero16 with
// packed fp16 arithmetic), and B is the block-diagonal constant qt in fp16
// (B[(slot j, block)][n] = qt[head(n)][block] if j == slot(n), else 0), so
// every output lane is a useful score.  Values use a second MFMA per slot,
//   O[n][c] += sum_t p[n][t] lv[t][c],
// with A = softmax weights of the slot's streams (fp16) and B = that group's
// dequantised value latents.  The online softmax keeps one running max per
// stream and rescales only when a new block maximum exceeds it by more than
// kRescaleSlack (log2 units), so weights stay <= 2^kRescaleSlack.
//
// Channel order inside an 8-channel block follows the code extraction:
// halves [c0, c4, c1, c5, c2, c6, c3, c7]; A and B use the same order.

constexpr int kWaves = 4;
constexpr float kRescaleSlack = 8.0f;
constexpr int kStageBudgetWords = 24 * 1024;   // both record buffers together (96 KiB)

// LDS layout of one attend workgroup (byte offsets).  Shared by the kernel
// and the host, which sizes the dynamic LDS from it.
struct AttendLds {
    int qt, qt16, kpw, blk, stage, sb;           // sb: words per stage buffer
    int pp;                                      // token groups per pass
    int ts, mst, lst, ost, tp;                   // merge state: byte offsets inside a stage buffer
    int total, nbk, nub;
};


// Dynamic LDS of one attend workgroup; the same for every split size.
__host__ __device__ inline AttendLds attend_lds(int g, int nbk, int rk, int rv, int wk, int wv, bool vq) {
    AttendLds L;
    const int S = 16 / g, P = kWaves * S;
    L.nbk = nbk;
    L.nub = (S * L.nbk + 3) / 4;
    int o = 0;
    L.qt = lds_take(o, g * kHeadDim * 4);
    L.qt16 = lds_take(o, g * 16 * 16);
    L.kpw = lds_take(o, kWaves * S * L.nbk * 8 * 4);
    L.blk = lds_take(o, L.nbk * 16);             // key block addressing (base, stride, width, channels)
    // two stage buffers.  Each holds one pass of records (+ 16-byte
    // alignment slack); a pass is the 4 S groups the waves take, fewer when
    // that would not fit the budget.  The last split's tail latents go to
    // the buffer its last pass leaves free, and after the main loop the
    // other buffer holds the merge state.
    const int rec_words = wk + (vq ? wv : 0);
    const int fit = (kStageBudgetWords / 2 - 16) / rec_words;
    L.pp = fit < P ? (fit > 1 ? fit : 1) : P;
    int m = 0;
    L.ts = lds_take(m, g * (kWaves * 16 + 1) * 4);
    L.mst = lds_take(m, (kWaves + 1) * 16 * 4);
    L.lst = lds_take(m, (kWaves + 1) * 16 * 4);
    L.ost = lds_take(m, (kWaves + 1) * 16 * rv * 4);
    L.tp = lds_take(m, g * 32 * 4);
    int sb = L.pp * rec_words + 16;
    const int tail_words = 32 * rk + (vq ? 32 * rv : 16 * rv);
    sb = sb > tail_words ? sb : tail_words;
    sb = sb > m / 4 ? sb : m / 4;
    L.sb = (sb + 3) & ~3;
    L.stage = lds_take(o, 2 * L.sb * 4);
    L.total = o;
    return L;
}


// Workgroup = (kv head h, call row i, split s); see the section comment.
// GEN = false serves PALU-shaped layouts (a 4-bit segment, then 2-bit
// channels) with closed-form record addressing; GEN = true any coder, through
// a per-block address table in LDS.
// G = query heads per kv head, NBV = value-channel blocks of 16.  A split is
// processed in passes of up to 4 S token groups (S per wave); the records of
// pass p + 1 are copied global -> LDS (direct 16-byte loads into LDS, no
// registers) into the other of two buffers while pass p is computed.
// The fast variants with up to two value blocks are held to 128 VGPRs (four
// waves per SIMD); the widest of them would otherwise take 129.
template <int G, int NBV, bool VQ, bool GEN, int NBKF>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NBKF > 0 && NBV <= 2 ? 4 : 1)))
void attend_kernel(AttendArgs a) {
    constexpr int g = G, S = 16 / G, NS = S * G;
    constexpr bool vq = VQ;                      // V stored as mixed-bit codes
    extern __shared__ __align__(16) unsigned char lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int ln = lane & 15, kb = lane >> 4;

    // ---- work item: grid (kv head, row, split), kv head fastest.  Workgroups
    //      go to the XCDs round-robin by linear id, so every XCD gets the same
    //      mix of heads and rows (with the split fastest, ragged rows left
    //      the XCDs that draw high split indices idle while others queued
    //      work); one 16-byte row descriptor
    const int h = blockIdx.x, i = blockIdx.y, z = blockIdx.z;
    const AttendRow rw = a.row[i];
    // Pin the kernel arguments the prologue needs before the first branch so
    // their scalar loads are issued together (one round trip instead of a
    // chain of dependent ones).
    asm volatile("" ::"s"(a.k.records), "s"(a.v.records), "s"(a.k.tail), "s"(a.v.tail), "s"(a.k.basis_t16),
                 "s"(a.q), "s"(a.k.head_stride), "s"(a.v.head_stride), "s"(a.k.r), "s"(a.k.cd.meta0), "s"(a.k.words),
                 "s"(a.v.r), "s"(a.v.cd.meta0), "s"(a.v.words), "s"(a.v.fp16_latents), "s"(a.chunk), "s"(a.hpg),
                 "s"(a.Hq), "s"(a.Hkv), "s"(a.qscale), "s"(rw.slot), "s"(rw.len), "s"(rw.qi), "s"(rw.sel_ns));
    const int qi = rw.qi, slot = rw.slot;
    int ns = rw.sel_ns >> 1, len = rw.len, tsl = rw.sel_ns & 1;
    if (a.dev_len) {
        // decode step: the row's length after this step's one-token append
        // (none at the capacity), its tail buffer, and its splits; one
        // workgroup hands (length, splits) to the combine kernel
        len = min(a.len_dev[slot] + 1, a.max_len);
        tsl = a.sel_dev[slot];
        ns = max(1, ((len >> 5) + a.chunk - 1) / a.chunk);
        if (h == 0 && z == 0 && threadIdx.x == 0) {
            a.row_info[2 * qi] = len;
            a.row_info[2 * qi + 1] = ns;
        }
    }
    if (z >= ns) return;                          // whole workgroup: no barrier reached
    const int nfull = len >> 5, ntail = len & 31;
    // split of this workgroup: when the row's last split is a full chunk
    // and also carries the incomplete group it is the heaviest one, and it
    // goes first in the dispatch order; otherwise splits go in order
    const bool tail_first = ntail > 0 && nfull - (ns - 1) * a.chunk >= a.chunk;
    const int s = tail_first ? (z == 0 ? ns - 1 : z - 1) : z;
    const int jb = s * a.chunk;
    const int je = jb + a.chunk < nfull ? jb + a.chunk : nfull;
    const int ntg = je > jb ? je - jb : 0;
    const bool do_tail = (s == ns - 1) && ntail > 0;
    const int grp = h / a.hpg;
    const int rk = a.k.r;
    const int rv = a.v.r;
    const int WK = a.k.words, WV = a.v.words;
    const int kmeta = a.k.cd.meta0, vmeta = a.v.cd.meta0;
    // PALU-shaped layouts: nhk 4-bit channels, then 2-bit ones
    const int nhk = a.k.cd.bits[0] == 4 ? a.k.cd.c0[1] : 0, nlk = rk - nhk, nbh = (nhk + 7) >> 3;
    const int nhv = a.v.cd.bits[0] == 4 ? a.v.cd.c0[1] : 0;

    const AttendLds L = attend_lds(g, coder_blocks(a.k.cd), rk, rv, WK, WV, vq);
    const int nbk = L.nbk, nub = L.nub, npair = S * nbk;
    const int PP = L.pp;                          // groups per pass (<= P)
    const int npass = (ntg + PP - 1) / PP;
    float *qt = reinterpret_cast<float *>(lds + L.qt);
    uint4 *qt16 = reinterpret_cast<uint4 *>(lds + L.qt16);
    _Float16 *qt16h = reinterpret_cast<_Float16 *>(lds + L.qt16);
    // stage buffer tb holds the tail latents (the one the last pass leaves
    // free); after the main loop the other one holds the merge state
    const int tb = npass & 1;
    const int tail_off = L.stage + tb * L.sb * 4, post = L.stage + (1 - tb) * L.sb * 4;
    const uint32_t *tails = reinterpret_cast<const uint32_t *>(lds + tail_off);
    float *ts = reinterpret_cast<float *>(lds + post + L.ts);
    float *mst = reinterpret_cast<float *>(lds + post + L.mst);
    float *lst = reinterpret_cast<float *>(lds + post + L.lst);
    float *ost = reinterpret_cast<float *>(lds + post + L.ost);
    float *tp = reinterpret_cast<float *>(lds + post + L.tp);

    const int64_t hb = static_cast<int64_t>(slot) * a.Hkv + h;
    const uint32_t *kg = a.k.records + hb * a.k.head_stride;
    const uint32_t *vg = a.v.records + hb * a.v.head_stride;

    // ---- 1. copies global -> LDS: a pass of records (K records, then V
    //         records; each block starts at the 16-byte boundary at or below
    //         its first word) and, in the last split, the tail latents
    auto pass_words = [&](int p, int &nk4, int &nv4, int &koff, int &voff) {
        const int64_t g0 = jb + p * PP, g1 = g0 + PP < je ? g0 + PP : je;
        const int64_t ka = (g0 * WK) & ~3LL, va = (g0 * WV) & ~3LL;
        nk4 = static_cast<int>((g1 * WK - ka + 3) >> 2);
        nv4 = vq ? static_cast<int>((g1 * WV - va + 3) >> 2) : 0;
        koff = static_cast<int>(g0 * WK - ka);
        voff = 4 * nk4 + static_cast<int>(g0 * WV - va);
    };
    // (dst = the LDS base the copies write through)
    auto copy_pass = [&](unsigned char *dst, int p) {
        int nk4, nv4, koff, voff;
        pass_words(p, nk4, nv4, koff, voff);
        const int64_t g0 = jb + p * PP;
        const u4v *ks = reinterpret_cast<const u4v *>(kg + ((g0 * WK) & ~3LL));
        const u4v *vs = reinterpret_cast<const u4v *>(vg + ((g0 * WV) & ~3LL));
        const int n4 = nk4 + nv4, boff = L.stage + (p & 1) * L.sb * 4;
        for (int c = wv; c * 64 < n4; c += kWaves) {
            const int e = c * 64 + lane;
            if (e < n4)
                __builtin_amdgcn_global_load_lds(e < nk4 ? ks + e : vs + (e - nk4), dst + boff + c * 1024, 16, 0, 0);
        }
    };
    const int64_t tsel = (hb * 2 + tsl) * kTokGroup;
    const int tk_words = do_tail ? min((ntail * rk + 3) & ~3, kTokGroup * rk) : 0;
    const int tv_words = do_tail ? (vq ? min((ntail * rv + 3) & ~3, kTokGroup * rv) : 16 * rv) : 0;
    auto copy_tail = [&](unsigned char *dst) {
        const u4v *tks = reinterpret_cast<const u4v *>(a.k.tail + tsel * rk);
        const u4v *tvs = vq ? reinterpret_cast<const u4v *>(a.v.tail + tsel * rv)
                            : reinterpret_cast<const u4v *>(vg + static_cast<int64_t>(nfull) * WV);
        const int ntk4 = tk_words >> 2, n4 = ntk4 + (tv_words >> 2);
        for (int c = wv; c * 64 < n4; c += kWaves) {
            const int e = c * 64 + lane;
            if (e < n4)
                __builtin_amdgcn_global_load_lds(e < ntk4 ? tks + e : tvs + (e - ntk4), dst + tail_off + c * 1024, 16,
                                                 0, 0);
        }
    };
    // With fp16 value latents, what the first pass would copy while it runs
    // (the second pass's records, or the tail latents when there is one
    // pass) goes out now too: the second buffer is free, and the first pass
    // then waits only on its value loads (fp16-value batch 29.9 -> 29.0 us
    // per call).  With quantised values it stays in the first pass: issuing
    // it here left the memory pipe idle during that pass and measured
    // slower on many-pass splits (serving batch 51.5 -> 53.0 us).
    constexpr bool kEarly = !VQ;
    if (npass > 0) copy_pass(lds, 0);
    else if (do_tail) copy_tail(lds);
    if (kEarly) {
        if (npass > 1) copy_pass(lds, 1);
        else if (npass == 1 && do_tail) copy_tail(lds);
    }

    // ---- 2. absorbed query qt = qs V_K^T q on MFMA: rows = query heads of
    //         this kv head, K = d, columns = 16 score-operand positions of
    //         the position-ordered fp16 key basis (wave w takes blocks w and
    //         w + 4).  The result goes straight to the fp16 score operand
    //         qt16[head][position] (padding positions come out 0) and, for
    //         the tail stream, to fp32 qt[head][channel]; only the waves
    //         that own a block load the query and the basis.
    {
        const int np = 8 * nbk;                      // positions (<= 128)
        const int nbc = (np + 15) >> 4;              // 16-position blocks (<= 8)
        const bool own0 = wv < nbc, own1 = wv + kWaves < nbc;
        if (own0) {
            const int qrow = qi * a.Hq + h * g;
            // rows ln >= g repeat a valid query; their MFMA output rows are never stored
            const uint16_t *qsrc = a.q + static_cast<int64_t>(qrow + (ln < g ? ln : 0)) * kHeadDim + 8 * kb;
            uint4 qa[4], bb[2][4];
#pragma unroll
            for (int st = 0; st < 4; ++st) qa[st] = *reinterpret_cast<const uint4 *>(qsrc + 32 * st);
            // bf16 queries: exact per-row power-of-two rescale into fp16,
            // undone on the MFMA result (output row 4 kb + v = query row)
            float qsc[4] = {a.qscale, a.qscale, a.qscale, a.qscale};
            if (a.bf16) {
                const int kq = bf16_rows_to_fp16(qa);
#pragma unroll
                for (int v = 0; v < 4; ++v) qsc[v] = ldexpf(a.qscale, __shfl(kq, 4 * kb + v));
            }
            const uint16_t *bt = a.k.basis_t16 + slot * a.k.set_bt16 + static_cast<int64_t>(grp) * np * kHeadDim;
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                if (x == 1 && !own1) break;
                int n = 16 * (wv + kWaves * x) + ln;
                n = n < np ? n : np - 1;              // clamped rows are never stored
#pragma unroll
                for (int st = 0; st < 4; ++st)
                    bb[x][st] = *reinterpret_cast<const uint4 *>(bt + static_cast<int64_t>(n) * kHeadDim + 32 * st +
                                                                 8 * kb);
            }
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                if (x == 1 && !own1) break;
                f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int st = 0; st < 4; ++st)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h8(qa[st].x, qa[st].y, qa[st].z, qa[st].w),
                                                                as_h8(bb[x][st].x, bb[x][st].y, bb[x][st].z,
                                                                      bb[x][st].w),
                                                                acc, 0, 0, 0);
                const int n = 16 * (wv + kWaves * x) + ln;
                const int q = n >> 3, idx = n & 7;
                const KBlock kbq = key_block(a.k.cd, q < nbk ? q : nbk - 1);
                const int chan0 = kbq.chan0, chanend = kbq.chanend;
                const int c = chan0 + (idx >> 1) + 4 * (idx & 1);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int hh = 4 * kb + v;
                    if (hh < g && n < np) {
                        const float val = acc[v] * qsc[v];
                        qt16h[hh * np + n] = static_cast<_Float16>(val);
                        if (c < chanend) qt[hh * rk + c] = val;
                    }
                }
            }
        }
    }
    // ---- 3. key block addressing table (one entry per 8-channel block)
    int4 *blk = reinterpret_cast<int4 *>(lds + L.blk);
    if (GEN && tid < nbk) {
        const KBlock b = key_block(a.k.cd, tid);
        blk[tid] = make_int4(b.base, b.stride, b.w, b.chan0 | (b.chanend << 16));
    }
    __builtin_amdgcn_s_waitcnt(0);                    // this wave's copies have landed
    __syncthreads();

    // ---- 4. main loop: passes of PP token groups, wave w takes pass-relative
    //         groups [w S, w S + S)
    const int slot_n = ln / g, head_n = ln - (ln / g) * g;
    const bool live_n = ln < NS;
    float m_run = -INFINITY, l_run = 0.0f;
    f4 oacc[NBV];
#pragma unroll
    for (int nb = 0; nb < NBV; ++nb) oacc[nb] = (f4){0.0f, 0.0f, 0.0f, 0.0f};
    // per-lane value-channel addressing (column c = 16 nb + ln, clamped)
    int vch[NBV], vw0[NBV], vw1[NBV], vs0[NBV], vs1[NBV], vwid[NBV], vwc[NBV];
    uint32_t vcm[NBV];
    int row_slot[4];                                 // slot of value-output row 4*kb + v
#pragma unroll
    for (int v = 0; v < 4; ++v) row_slot[v] = (4 * kb + v) / g;
#pragma unroll
    for (int nb = 0; nb < NBV; ++nb) {
        int c = 16 * nb + ln;
        c = c < rv ? c : rv - 1;
        int2 vc = make_int2(0, 2);                   // base bit, width
        if constexpr (VQ && GEN) vc = value_channel(a.v.cd, c);
        else if constexpr (VQ) vc = c < nhv ? make_int2(128 * c, 4) : make_int2(128 * nhv + 64 * (c - nhv), 2);
        const int wc = vc.y;
        const int b0 = vc.x + 4 * kb * wc, b1 = b0 + 16 * wc;
        vch[nb] = c;
        vw0[nb] = b0 >> 5;
        vw1[nb] = b1 >> 5;
        vs0[nb] = b0 & 31;
        vs1[nb] = b1 & 31;          // differs from vs0 only for 1-bit codes (b1 - b0 = 16 wc)
        vwid[nb] = 4 * wc;          // 4 tokens; width 8 takes whole words instead
        vwc[nb] = wc;
        const uint32_t m = (1u << wc) - 1u;
        vcm[nb] = m | (m << 16);
    }
    const uint32_t kmagic = vgpr_const(0x64006400u), km4 = vgpr_const(0x000F000Fu),
                   km2 = vgpr_const(0x00030003u);
    const FastDiv div_nbk4(a.inv_nbk4);
    const int tb0 = wv * S;                          // pass-relative group of slot 0
    // (a) below gathers S nbk 4 (slot, block, pair) items per pass.  When
    // one round of 64 lanes covers them, each lane's item is fixed: its
    // slot, the two metadata words it reads (padding channels read word 0
    // and are masked to 0) and the word it writes are computed once here.
    const bool kp_one = S * nbk * 4 <= 64;
    int kp_m = 0, kp_ca = 0, kp_cb = 0, kp_dst = 0;
    uint32_t kp_ma = 0u, kp_mb = 0u;
    if (kp_one && lane < S * nbk * 4) {
        const int m = div_nbk4.quo(lane), r2 = lane - m * nbk * 4;
        const int q = r2 >> 2, k = r2 & 3;
        int chan0, chanend;
        if constexpr (GEN) {
            const int cc = blk[q].w;
            chan0 = cc & 0xFFFF;
            chanend = cc >> 16;
        } else {
            chan0 = q < nbh ? 8 * q : nhk + 8 * (q - nbh);
            chanend = q < nbh ? nhk : rk;
        }
        kp_m = m;
        kp_ca = chan0 + k < chanend ? kmeta + chan0 + k : 0;
        kp_cb = chan0 + k + 4 < chanend ? kmeta + chan0 + k + 4 : 0;
        kp_ma = chan0 + k < chanend ? 0xFFFFFFFFu : 0u;
        kp_mb = chan0 + k + 4 < chanend ? 0xFFFFFFFFu : 0u;
        kp_dst = (m * nbk + q) * 8 + k;
    }
    // the score operand B of the first two score steps (the same in every
    // pass), held in registers when there are at most two steps
    auto score_b = [&](const uint4 *q16, int u) -> uint4 {
        const int p = 4 * u + kb;
        int q, j;
        if constexpr (S % 4 == 0) {
            q = (4 * u) / S;
            j = p - q * S;
        } else {
            q = p / S;
            j = p - q * S;
        }
        const int qc = q < nbk ? q : nbk - 1;
        const bool ok = p < npair && live_n && j == slot_n;
        return ok ? q16[head_n * nbk + qc] : make_uint4(0u, 0u, 0u, 0u);
    };
    uint4 bq_pre[2] = {make_uint4(0u, 0u, 0u, 0u), make_uint4(0u, 0u, 0u, 0u)};
    // Fast path: 4 query heads per kv head (S = 4), PALU layout, quantised
    // values, at most 4 key blocks.  Lane kb then always serves slot kb and
    // score step u is key block u, so everything a lane addresses is fixed:
    // the score operands B of every step stay in registers, the metadata of
    // (slot kb, block u) is at a constant offset, and the bit of the lane's
    // token in block u's plane is precomputed.  The score MFMA's row ln of
    // half h holds token 8 (ln / 4) + 4 h + ln % 4, so the softmax weights
    // a lane holds (rows 4 kb .. 4 kb + 3 of both halves) are the tokens
    // 8 kb .. 8 kb + 7, and each value operand comes from one word: the
    // lane's 8 tokens of its channel (4-bit: word kb of the channel; 2-bit:
    // half kb % 2 of word kb / 2, its second byte moved up by a permute).
    // (the host launches this variant only with 4 query heads per kv
    // head, quantised values and a PALU key coder of at most 4 blocks whose
    // first block is the only 4-bit one: 1 to 8 hi channels)
    // NBKF > 0: this variant, for exactly NBKF key blocks
    constexpr bool FAST = NBKF > 0 && G == 4 && !GEN && VQ;
    constexpr bool fast = FAST;
    constexpr int NF = NBKF > 0 ? NBKF : 1;
    uint4 bqf[NF];
    int bitA[NF];
    int vwf[NBV];
    uint32_t vsel[NBV];
    if constexpr (FAST) {
        if (fast) {
            const int t0 = 8 * (ln >> 2) + (ln & 3);
#pragma unroll
            for (int u = 0; u < NF; ++u) {
                bqf[u] = score_b(qt16, u);
                const bool w4 = u == 0;
                const int base = w4 ? 32 * u : 128 * nhk + 16 * (u - nbh);
                const int stride = w4 ? 4 * nhk : 2 * nlk;
                bitA[u] = base + t0 * stride;
            }
#pragma unroll
            for (int nb = 0; nb < NBV; ++nb) {
                const int c = vch[nb];
                if (c < nhv) {
                    vwf[nb] = 4 * c + kb;
                    vsel[nb] = 0x03020100u;
                } else {
                    vwf[nb] = 4 * nhv + 2 * (c - nhv) + (kb >> 1);
                    vsel[nb] = (kb & 1) ? 0x0C030C02u : 0x0C010C00u;
                }
            }
        }
    }
    if constexpr (!fast) {
        if (nub <= 2) {
            bq_pre[0] = score_b(qt16, 0);
            if (nub == 2) bq_pre[1] = score_b(qt16, 1);
        }
    }
    // One pass.  Every LDS access in it goes through lw, and the copies of
    // the next pass through ldma; both are restrict-qualified and both are
    // the LDS base.  As distinct values (fp16 value latents) they tell the
    // compiler that the copies in flight write nothing the pass reads, and
    // it no longer waits for those copies at the pass's first LDS read (nor,
    // counters being in order, at the value loads issued before them).  As
    // one value (quantised values) the qualification is dropped and the
    // first LDS read waits for the copies: letting them overlap the pass
    // measured 1% slower on the long-context shape there.  Either way the
    // copies land before the barrier that ends the pass (explicit wait).
    // (everything else by value: capturing all by reference cost 2 to 4
    // VGPRs in most variants)
    using LdsPtr = std::conditional_t<VQ, unsigned char *, unsigned char *__restrict__>;
    auto run_pass = [=, &oacc, &m_run, &l_run](int pi, LdsPtr lw, LdsPtr ldma) mutable {
        uint32_t *kpw = reinterpret_cast<uint32_t *>(lw + L.kpw) + wv * (S * nbk * 8);
        const uint4 *qt16 = reinterpret_cast<const uint4 *>(lw + L.qt16);
        const int4 *blk = reinterpret_cast<const int4 *>(lw + L.blk);
        const int npg = min(PP, ntg - pi * PP);      // groups in this pass (>= 1)
        const int64_t g0 = jb + pi * PP;             // absolute group of pass group 0
        // fp16 value latents are read from memory straight into the value
        // operands.  With at most 16 (slot, block) pairs all of a pass's
        // loads are issued here, before the next pass's copies, so that they
        // are in flight while the scores are computed and the wait for them
        // does not also wait for those copies; otherwise each slot's loads
        // are issued right before its MFMAs.  Slots past the pass read the
        // last group (never used).
        constexpr bool kPreV = !VQ && S * NBV <= 16;
        uint2 vlo[kPreV ? S : 1][NBV], vhi[kPreV ? S : 1][NBV];
        if constexpr (kPreV) {
#pragma unroll
            for (int m = 0; m < S; ++m) {
                const int tg = tb0 + m < npg ? tb0 + m : npg - 1;
#pragma unroll
                for (int nb = 0; nb < NBV; ++nb) {
                    const uint16_t *r16 = reinterpret_cast<const uint16_t *>(vg + (g0 + tg) * WV) + vch[nb] * 32;
                    vlo[m][nb] = *reinterpret_cast<const uint2 *>(r16 + 4 * kb);
                    vhi[m][nb] = *reinterpret_cast<const uint2 *>(r16 + 16 + 4 * kb);
                }
            }
        }
        if (pi > 0 || !kEarly) {                      // (else pass 0's went out with the first)
            if (pi + 1 < npass) copy_pass(ldma, pi + 1);  // into the other buffer
            else if (do_tail) copy_tail(ldma);            // the last pass leaves buffer tb free
        }
        int nk4, nv4, koff, voff;
        pass_words(pi, nk4, nv4, koff, voff);
        const uint32_t *stage = reinterpret_cast<const uint32_t *>(lw + L.stage) + (pi & 1) * L.sb;

        // (a) this wave's K scale/zero pairs per (slot, channel block):
        //     words 0..3 scale pairs (k, k + 4), words 4..7 zero pairs;
        //     padding channels are 0; slots past the pass repeat its last group
        // (with S a multiple of 4, only the slots of live score steps: the
        // pass's slots rounded up to a multiple of 4)
        int n_gather = S * nbk * 4;
        if constexpr (S % 4 == 0) {
            const int live = tb0 < npg ? min(S, (npg - tb0 + 3) & ~3) : 0;
            n_gather = live * nbk * 4;
        }
        if (kp_one) {
            if (lane < S * nbk * 4) {
                int tg = tb0 + kp_m;
                tg = tg < npg ? tg : npg - 1;
                const uint32_t *rec = stage + koff + tg * WK;
                const uint32_t wa = rec[kp_ca] & kp_ma, wb = rec[kp_cb] & kp_mb;
                kpw[kp_dst] = perm_b32(wb, wa, 0x05040100u);
                kpw[kp_dst + 4] = perm_b32(wb, wa, 0x07060302u);
            }
        } else for (int e = lane; e < n_gather; e += 64) {
            const int m = div_nbk4.quo(e), r2 = e - m * nbk * 4;
            const int q = r2 >> 2, k = r2 & 3;
            int chan0, chanend;
            if constexpr (GEN) {
                const int cc = blk[q].w;
                chan0 = cc & 0xFFFF;
                chanend = cc >> 16;
            } else {
                chan0 = q < nbh ? 8 * q : nhk + 8 * (q - nbh);
                chanend = q < nbh ? nhk : rk;
            }
            int tg = tb0 + m;
            tg = tg < npg ? tg : npg - 1;
            const uint32_t *rec = stage + koff + tg * WK + kmeta;
            const uint32_t wa = chan0 + k < chanend ? rec[chan0 + k] : 0u;
            const uint32_t wb = chan0 + k + 4 < chanend ? rec[chan0 + k + 4] : 0u;
            uint32_t *dst = kpw + (m * nbk + q) * 8;
            dst[k] = perm_b32(wb, wa, 0x05040100u);
            dst[4 + k] = perm_b32(wb, wa, 0x07060302u);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // (b) scores.  PALU-shaped layouts: A = the codes as exact fp16
        //     1024 + code, B = qt16 * scale16 (the group's scales folded into
        //     the query operand, the same for all 32 tokens); the rest of
        //     sum_c qt_c (s_c code_c + z_c) comes from two more MFMAs into
        //     zacc whose A rows are all equal: the fp16 zeros against qt16
        //     (products exact) and -1024 against the scaled operand.  Every
        //     row of zacc holds the same value, the stream's constant.
        f4 sacc0 = {0.0f, 0.0f, 0.0f, 0.0f}, sacc1 = {0.0f, 0.0f, 0.0f, 0.0f}, zacc = {0.0f, 0.0f, 0.0f, 0.0f};
        const f16x8 kneg1024 = as_h8(0xE400E400u, 0xE400E400u, 0xE400E400u, 0xE400E400u);
        auto score_step = [&](int u, const uint4 bq) {
            const int p = 4 * u + kb;
            int q, j;
            if constexpr (S % 4 == 0) {
                q = (4 * u) / S;            // the same for every lane of the wave
                j = p - q * S;
            } else {
                q = p / S;
                j = p - q * S;
            }
            // invalid pairs and groups past the pass are read from a valid
            // (clamped) record; their scores belong to masked streams
            int tg = tb0 + j;
            tg = tg < npg ? tg : npg - 1;
            const int qc = q < nbk ? q : nbk - 1;
            const uint32_t *rec = stage + koff + tg * WK;
            const uint4 *kp = reinterpret_cast<const uint4 *>(kpw + (j * nbk + qc) * 8);
            const uint4 sp = kp[0], zp = kp[1];
            const f16x8 bop = as_h8(bq.x, bq.y, bq.z, bq.w);
            f16x8 a0, a1;
            if constexpr (!GEN) {
                const bool w4 = qc < nbh;
                const int base = w4 ? 32 * qc : 128 * nhk + 16 * (qc - nbh);
                const int stride = w4 ? 4 * nhk : 2 * nlk;
                const int bit0 = base + ln * stride, bit1 = bit0 + 16 * stride;
                const uint32_t X0 = __builtin_amdgcn_alignbit(rec[(bit0 >> 5) + 1], rec[bit0 >> 5], bit0 & 31);
                const uint32_t X1 = __builtin_amdgcn_alignbit(rec[(bit1 >> 5) + 1], rec[bit1 >> 5], bit1 & 31);
                if constexpr (S % 4 == 0) {
                    if (w4) {
                        a0 = codes8<true>(X0, km4, kmagic);
                        a1 = codes8<true>(X1, km4, kmagic);
                    } else {
                        a0 = codes8<false>(X0, km2, kmagic);
                        a1 = codes8<false>(X1, km2, kmagic);
                    }
                } else {
                    a0 = codes8_any(X0, w4);
                    a1 = codes8_any(X1, w4);
                }
                const f16x8 bs = bop * as_h8(sp.x, sp.y, sp.z, sp.w);
                sacc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, bs, sacc0, 0, 0, 0);
                sacc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, bs, sacc1, 0, 0, 0);
                zacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h8(zp.x, zp.y, zp.z, zp.w), bop, zacc, 0, 0, 0);
                zacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kneg1024, bs, zacc, 0, 0, 0);
                return;
            } else {
                const int4 bq4 = blk[qc];                // base, stride, width
                const int wq = bq4.z;
                const int bit0 = bq4.x + ln * bq4.y, bit1 = bit0 + 16 * bq4.y;
                const uint32_t X0 = __builtin_amdgcn_alignbit(rec[(bit0 >> 5) + 1], rec[bit0 >> 5], bit0 & 31);
                const uint32_t X1 = __builtin_amdgcn_alignbit(rec[(bit1 >> 5) + 1], rec[bit1 >> 5], bit1 & 31);
                // 8-bit blocks span 64 bits: the second word of each window
                const uint32_t Y0 = wq == 8 ? __builtin_amdgcn_alignbit(rec[(bit0 >> 5) + 2], rec[(bit0 >> 5) + 1],
                                                                       bit0 & 31) : 0u;
                const uint32_t Y1 = wq == 8 ? __builtin_amdgcn_alignbit(rec[(bit1 >> 5) + 2], rec[(bit1 >> 5) + 1],
                                                                       bit1 & 31) : 0u;
                a0 = dequant8_w(X0, Y0, wq, sp, zp);
                a1 = dequant8_w(X1, Y1, wq, sp, zp);
            }
            sacc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, bop, sacc0, 0, 0, 0);
            sacc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, bop, sacc1, 0, 0, 0);
        };
        if constexpr (fast) {
            const int tgl = tb0 + kb < npg ? tb0 + kb : npg - 1;
            const uint32_t *rec = stage + koff + tgl * WK;
            const uint4 *kpl = reinterpret_cast<const uint4 *>(kpw + kb * nbk * 8);
#pragma unroll
            for (int u = 0; u < NF; ++u) {
                {
                    // the second half's token is 4 tokens further (stride: bits per token)
                    const int stride = u == 0 ? 4 * nhk : 2 * nlk;
                    const int bitB = bitA[u] + 4 * stride;
                    const int wa = bitA[u] >> 5, wb = bitB >> 5;
                    const uint32_t X0 = __builtin_amdgcn_alignbit(rec[wa + 1], rec[wa], bitA[u] & 31);
                    const uint32_t X1 = __builtin_amdgcn_alignbit(rec[wb + 1], rec[wb], bitB & 31);
                    const uint4 sp = kpl[2 * u], zp = kpl[2 * u + 1];
                    const f16x8 a0 = u == 0 ? codes8<true>(X0, km4, kmagic) : codes8<false>(X0, km2, kmagic);
                    const f16x8 a1 = u == 0 ? codes8<true>(X1, km4, kmagic) : codes8<false>(X1, km2, kmagic);
                    const f16x8 bop = as_h8(bqf[u].x, bqf[u].y, bqf[u].z, bqf[u].w);
                    const f16x8 bs = bop * as_h8(sp.x, sp.y, sp.z, sp.w);
                    sacc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, bs, sacc0, 0, 0, 0);
                    sacc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, bs, sacc1, 0, 0, 0);
                    zacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h8(zp.x, zp.y, zp.z, zp.w), bop, zacc, 0, 0,
                                                                  0);
                    zacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kneg1024, bs, zacc, 0, 0, 0);
                }
            }
        } else {
            // with S a multiple of 4, step u covers slots 4 (u % (S / 4)) ..
            // + 3 of one key block; a step whose slots all lie past the pass
            // only feeds masked streams and is skipped (one or two query heads
            // per kv head on short passes: 4 of 16 steps when the pass has
            // at most 4 groups)
            auto step_live = [&](int u) {
                if constexpr (S % 4 == 0) return tb0 + 4 * (u % (S / 4)) < npg;
                else return true;
            };
            if (nub <= 2) {
                score_step(0, bq_pre[0]);
                if (nub == 2 && step_live(1)) score_step(1, bq_pre[1]);
            } else {
                for (int u = 0; u < nub; ++u)
                    if (step_live(u)) score_step(u, score_b(qt16, u));   // wave-uniform
            }
        }

        // (c) online softmax of stream ln (rows 4*kb + v of both 16-token halves)
        const bool sv = live_n && (tb0 + slot_n) < npg;
        const float sc[8] = {sacc0[0], sacc0[1], sacc0[2], sacc0[3], sacc1[0], sacc1[1], sacc1[2], sacc1[3]};
        // the stream's constant (0 for the generic coders): score = sc + zc
        const float zc = zacc[0];
        float mloc = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])),
                           fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7]))) + zc;
        mloc = sv ? mloc : -INFINITY;
        const bool need = mloc > m_run + kRescaleSlack;
        if (__any(need)) {
            float mm = fmaxf(mloc, __shfl_xor(mloc, 16));
            mm = fmaxf(mm, __shfl_xor(mm, 32));
            const bool upd = mm > m_run + kRescaleSlack;
            const float m_new = upd ? mm : m_run;
            const float alpha = upd ? exp2f(m_run - m_new) : 1.0f;
            l_run *= alpha;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float av = __shfl(alpha, 4 * kb + v);
#pragma unroll
                for (int nb = 0; nb < NBV; ++nb) oacc[nb][v] *= av;
            }
            m_run = m_new;
        }
        // weights of streams whose group is past the pass never reach a
        // value MFMA (their slot's A rows are zero), so only l is masked
        const float msafe = (m_run == -INFINITY ? 0.0f : m_run) - zc;
        float pr[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) pr[k] = __builtin_amdgcn_exp2f(sc[k] - msafe);
        const float psum = ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
        l_run += sv ? psum : 0.0f;
        const uint32_t pp0 = pack_rtz(pr[0], pr[4]), pp1 = pack_rtz(pr[1], pr[5]);
        const uint32_t pp2 = pack_rtz(pr[2], pr[6]), pp3 = pack_rtz(pr[3], pr[7]);

        // (d) values: one MFMA per slot and 16-channel block on exact codes
        //     (1024 + code in fp16); per-group scale and zero are applied in
        //     the epilogue: sum_t p (code s + z) = s (D - 1024 P) + z P, with
        //     the weight sum P = sum_t p of each stream from one more MFMA
        //     against a constant-one operand (so it sums exactly the fp16
        //     weights used).  fp16 value latents come from registers
        //     loaded at the start of the pass, or from memory per slot.
        f4 dacc[NBV];
#pragma unroll
        for (int nb = 0; nb < NBV; ++nb) dacc[nb] = (f4){0.0f, 0.0f, 0.0f, 0.0f};
        f4 dP = {0.0f, 0.0f, 0.0f, 0.0f};
        const f16x8 ones8 = as_h8(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);
#pragma unroll
        for (int m = 0; m < S; ++m) {
            if (tb0 + m >= npg) break;               // wave-uniform
            const bool arow = live_n && slot_n == m;
            const f16x8 aop = arow ? as_h8(pp0, pp1, pp2, pp3) : as_h8(0u, 0u, 0u, 0u);
            if (vq) dP = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, ones8, dP, 0, 0, 0);
#pragma unroll
            for (int nb = 0; nb < NBV; ++nb) {
                uint32_t bp0, bp1, bp2, bp3;
                if constexpr (fast) {
                    // tokens (8 kb + j, 8 kb + 4 + j) of channel vch[nb] in pair j
                    const uint32_t *rec = stage + voff + (tb0 + m) * WV;
                    const uint32_t Wd = rec[vwf[nb]];
                    const uint32_t U = perm_b32(Wd, Wd, vsel[nb]);
                    const int wc = vwc[nb];
                    bp0 = (U & vcm[nb]) | kmagic;
                    bp1 = ((U >> wc) & vcm[nb]) | kmagic;
                    bp2 = ((U >> (2 * wc)) & vcm[nb]) | kmagic;
                    bp3 = ((U >> (3 * wc)) & vcm[nb]) | kmagic;
                } else if constexpr (VQ) {
                    const uint32_t *rec = stage + voff + (tb0 + m) * WV;
                    const uint32_t L0 = rec[vw0[nb]], L1 = rec[vw1[nb]];
                    const int wc = vwc[nb];
                    if (GEN && wc == 8) {
                        // tokens 4 kb + k (word L0, byte k) and 16 + 4 kb + k (L1)
                        bp0 = perm_b32(L1, L0, 0x0C040C00u) | kmagic;
                        bp1 = perm_b32(L1, L0, 0x0C050C01u) | kmagic;
                        bp2 = perm_b32(L1, L0, 0x0C060C02u) | kmagic;
                        bp3 = perm_b32(L1, L0, 0x0C070C03u) | kmagic;
                    } else {
                        const uint32_t X = __builtin_amdgcn_ubfe(L0, vs0[nb], vwid[nb]) |
                                           (__builtin_amdgcn_ubfe(L1, GEN ? vs1[nb] : vs0[nb], vwid[nb]) << 16);
                        bp0 = (X & vcm[nb]) | kmagic;
                        bp1 = ((X >> wc) & vcm[nb]) | kmagic;
                        bp2 = ((X >> (2 * wc)) & vcm[nb]) | kmagic;
                        bp3 = ((X >> (3 * wc)) & vcm[nb]) | kmagic;
                    }
                } else {
                    uint2 lo, hi;
                    if constexpr (kPreV) {
                        lo = vlo[m][nb];
                        hi = vhi[m][nb];
                    } else {
                        const uint16_t *r16 =
                            reinterpret_cast<const uint16_t *>(vg + (g0 + tb0 + m) * WV) + vch[nb] * 32;
                        lo = *reinterpret_cast<const uint2 *>(r16 + 4 * kb);
                        hi = *reinterpret_cast<const uint2 *>(r16 + 16 + 4 * kb);
                    }
                    bp0 = perm_b32(hi.x, lo.x, 0x05040100u);
                    bp1 = perm_b32(hi.x, lo.x, 0x07060302u);
                    bp2 = perm_b32(hi.y, lo.y, 0x05040100u);
                    bp3 = perm_b32(hi.y, lo.y, 0x07060302u);
                }
                dacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, as_h8(bp0, bp1, bp2, bp3), dacc[nb], 0, 0, 0);
            }
        }
        if (vq && G % 4 == 0) {
            // (e) epilogue: with 4 or 8 query heads a lane's four output rows
            //     4 kb + v belong to one token group, so its scale s and
            //     z - 1024 s are decoded once per channel block
            int tgr = tb0 + row_slot[0];
            tgr = tgr < npg ? tgr : npg - 1;
            const uint32_t *meta = stage + voff + tgr * WV + vmeta;
#pragma unroll
            for (int nb = 0; nb < NBV; ++nb) {
                const uint32_t mw = meta[vch[nb]];
                const float sc16 = h2f(mw);
                const float zr = fmaf(-1024.0f, sc16, h2f(mw >> 16));
#pragma unroll
                for (int v = 0; v < 4; ++v) oacc[nb][v] = fmaf(sc16, dacc[nb][v], fmaf(zr, dP[v], oacc[nb][v]));
            }
        } else if (vq) {
            // (e) epilogue per output row 4*kb + v (stream): the row's group
            //     scale s and z - 1024 s from its metadata word; rows of
            //     groups past the pass have D = P = 0
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                int tgr = tb0 + row_slot[v];
                tgr = tgr < npg ? tgr : npg - 1;
                const uint32_t *meta = stage + voff + tgr * WV + vmeta;
#pragma unroll
                for (int nb = 0; nb < NBV; ++nb) {
                    const uint32_t mw = meta[vch[nb]];
                    const float sc16 = h2f(mw);
                    const float zr = fmaf(-1024.0f, sc16, h2f(mw >> 16));
                    oacc[nb][v] = fmaf(sc16, dacc[nb][v], fmaf(zr, dP[v], oacc[nb][v]));
                }
            }
        } else {
#pragma unroll
            for (int nb = 0; nb < NBV; ++nb) oacc[nb] += dacc[nb];
        }
        __builtin_amdgcn_s_waitcnt(0);                // the next pass's copies have landed
        __syncthreads();                              // and every wave is done with this buffer
    };
    // two opaque zero offsets make the bases distinct values
    int lz0 = 0, lz1 = 0;
    if constexpr (!VQ) {
        asm volatile("" : "+s"(lz0));
        asm volatile("" : "+s"(lz1));
    }
    for (int pi = 0; pi < npass; ++pi) run_pass(pi, lds + lz0, lds + lz1);

    // A wave past its main loop takes a higher issue priority (within the
    // kernel, s_setprio): workgroups that are merging finish sooner and free
    // their CU slots for workgroups still queued (ragged batches launch more
    // workgroups than the CUs hold at once).
    __builtin_amdgcn_s_setprio(2);
    // ---- 5. per-wave stream results to LDS
    const FastDiv div_rv(a.inv_rv);
    float lsum = l_run;
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    float msum = fmaxf(m_run, __shfl_xor(m_run, 16));
    msum = fmaxf(msum, __shfl_xor(msum, 32));
    if (lane < 16) {
        mst[wv * 16 + lane] = msum;
        lst[wv * 16 + lane] = lsum;
    }
#pragma unroll
    for (int nb = 0; nb < NBV; ++nb) {
        const int c = 16 * nb + ln;
        if (c < rv) {
#pragma unroll
            for (int v = 0; v < 4; ++v) ost[(wv * 16 + 4 * kb + v) * rv + c] = oacc[nb][v];
        }
    }

    // ---- 6. incomplete group (fp32 latents staged in LDS; fp16 value
    //         latents of the partial record), as one more stream per head:
    //         thread (head tid / 32, token tid % 32), softmax within the 32
    //         lanes of a head
    if (do_tail) {
        const float *tk = reinterpret_cast<const float *>(tails);
        const int hh = tid >> 5, t = tid & 31;
        const bool ok = hh < g && t < ntail;
        float sc = -INFINITY;
        if (ok) {
            // four independent chains; lane t starts at channel t mod rk and
            // wraps, so the 32 lanes of a head read different LDS banks (the
            // row stride of rk floats put them on one or two banks when rk
            // is a multiple of 32)
            const float *qrow = qt + hh * rk, *krow = tk + t * rk;
            const int t0 = t - rk * (t / rk);
            float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
            auto span = [&](int c, int ce) {
                for (; c + 4 <= ce; c += 4) {
                    a0 = fmaf(qrow[c], krow[c], a0);
                    a1 = fmaf(qrow[c + 1], krow[c + 1], a1);
                    a2 = fmaf(qrow[c + 2], krow[c + 2], a2);
                    a3 = fmaf(qrow[c + 3], krow[c + 3], a3);
                }
                for (; c < ce; ++c) a0 = fmaf(qrow[c], krow[c], a0);
            };
            span(t0, rk);
            span(0, t0);
            sc = (a0 + a1) + (a2 + a3);
        }
        float mx = row_max(sc);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        const float pv = ok ? exp2f(sc - mx) : 0.0f;
        float ls = row_sum(pv);
        ls += __shfl_xor(ls, 16);
        if (hh < g) {
            tp[hh * 32 + t] = pv;
            if (t == 0) {
                mst[kWaves * 16 + hh] = mx;
                lst[kWaves * 16 + hh] = ls;
            }
        }
        __syncthreads();
        for (int e = tid; e < g * rv; e += 256) {
            const int hv = div_rv.quo(e), c = e - hv * rv;
            const float *pw = tp + hv * 32;
            float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;   // four independent chains
            int t2 = 0;
            if (vq) {
                const float *tv = reinterpret_cast<const float *>(tails + tk_words) + c;
                for (; t2 + 4 <= ntail; t2 += 4) {
                    a0 = fmaf(pw[t2], tv[t2 * rv], a0);
                    a1 = fmaf(pw[t2 + 1], tv[(t2 + 1) * rv], a1);
                    a2 = fmaf(pw[t2 + 2], tv[(t2 + 2) * rv], a2);
                    a3 = fmaf(pw[t2 + 3], tv[(t2 + 3) * rv], a3);
                }
                for (; t2 < ntail; ++t2) a0 = fmaf(pw[t2], tv[t2 * rv], a0);
            } else {
                const _Float16 *tv = reinterpret_cast<const _Float16 *>(tails + tk_words) + c * 32;
                for (; t2 + 4 <= ntail; t2 += 4) {
                    a0 = fmaf(pw[t2], static_cast<float>(tv[t2]), a0);
                    a1 = fmaf(pw[t2 + 1], static_cast<float>(tv[t2 + 1]), a1);
                    a2 = fmaf(pw[t2 + 2], static_cast<float>(tv[t2 + 2]), a2);
                    a3 = fmaf(pw[t2 + 3], static_cast<float>(tv[t2 + 3]), a3);
                }
                for (; t2 < ntail; ++t2) a0 = fmaf(pw[t2], static_cast<float>(tv[t2]), a0);
            }
            ost[(kWaves * 16 + hv) * rv + c] = (a0 + a1) + (a2 + a3);
        }
    }
    __syncthreads();

    // ---- 7. merge the streams of each head and write the split's partial.
    //         Stream k of a head: k < kWaves * S -> wave k / S, slot k % S
    //         (LDS stream (k / S) * 16 + (k % S) * g + head); k = kWaves * S
    //         -> the tail stream kWaves * 16 + head.  Wave w merges heads
    //         w, w + 4 with its lanes over streams.
    const int nsw = kWaves * S + (do_tail ? 1 : 0);   // <= 65
    float *wts = ts;                                   // [g][65]
    float *part = a.partial + (static_cast<int64_t>(qi) * a.Hq + h * g) * a.nsplit_max * (rv + 2) +
                  static_cast<int64_t>(s) * (rv + 2);
    const int64_t head_stride = static_cast<int64_t>(a.nsplit_max) * (rv + 2);
    for (int hh = wv; hh < g; hh += kWaves) {
        const int k1 = lane + 64;
        const int sid0 = lane < kWaves * S ? (lane / S) * 16 + (lane % S) * g + hh : kWaves * 16 + hh;
        const float m0 = lane < nsw ? mst[sid0] : -INFINITY;
        const float l0 = lane < nsw ? lst[sid0] : 0.0f;
        const float m1 = k1 < nsw ? mst[kWaves * 16 + hh] : -INFINITY;   // only k = 64 (the tail at S = 16)
        const float l1 = k1 < nsw ? lst[kWaves * 16 + hh] : 0.0f;
        const float M = wave_max(fmaxf(m0, m1));
        const float w0 = m0 == -INFINITY ? 0.0f : exp2f(m0 - M);
        const float w1 = m1 == -INFINITY ? 0.0f : exp2f(m1 - M);
        const float lt = wave_sum(fmaf(w0, l0, w1 * l1));
        if (lane < nsw) wts[hh * 65 + lane] = w0;
        if (k1 < nsw) wts[hh * 65 + k1] = w1;
        if (lane == 0) {
            part[hh * head_stride] = M;
            part[hh * head_stride + 1] = lt;
        }
    }
    __syncthreads();
    // weighted sum over the streams of every (head, channel) output: four
    // lanes of a quad per output, each over every fourth stream, then a quad
    // reduction (one lane per output with four independent chains when
    // there are more than 64 outputs)
    auto stream_row = [&](int k, int hh) {
        return k < kWaves * S ? (k / S) * 16 + (k % S) * g + hh : kWaves * 16 + hh;
    };
    if (g * rv <= 64) {
        const int e = tid >> 2, sub = tid & 3;
        const bool live = e < g * rv;
        const int ee = live ? e : 0;
        const int hh = div_rv.quo(ee), c = ee - hh * rv;
        const float *wrow = wts + hh * 65;
        float acc = 0.0f;
        for (int k = sub; k < nsw; k += 4) acc = fmaf(wrow[k], ost[stream_row(k, hh) * rv + c], acc);
        acc += dpp<kDppXor1>(acc);
        acc += dpp<kDppXor2>(acc);
        if (live && sub == 0) part[hh * head_stride + 2 + c] = acc;
    } else {
        for (int e = tid; e < g * rv; e += 256) {
            const int hh = div_rv.quo(e), c = e - hh * rv;
            const float *wrow = wts + hh * 65;
            float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
            int k = 0;
            for (; k + 4 <= nsw; k += 4) {
                a0 = fmaf(wrow[k], ost[stream_row(k, hh) * rv + c], a0);
                a1 = fmaf(wrow[k + 1], ost[stream_row(k + 1, hh) * rv + c], a1);
                a2 = fmaf(wrow[k + 2], ost[stream_row(k + 2, hh) * rv + c], a2);
                a3 = fmaf(wrow[k + 3], ost[stream_row(k + 3, hh) * rv + c], a3);
            }
            for (; k < nsw; ++k) a0 = fmaf(wrow[k], ost[stream_row(k, hh) * rv + c], a0);
            part[hh * head_stride + 2 + c] = (a0 + a1) + (a2 + a3);
        }
    }
}

// One workgroup of one wave per (call row, query head): merge the splits by
// log-sum-exp and project back with the value basis,
// o = V_V (o_lat / l) + mu_V, rounded to fp16.  The row's split partials and
// its group's value basis and mean are first copied to LDS with independent
// 16-byte loads, so the kernel waits on memory once; all later steps read LDS.
__host__ __device__ inline int combine_lds_floats(int ns, int rv) {
    return ((ns * (rv + 2) + 3) & ~3) + kHeadDim * rv + kHeadDim + ((ns + 3) & ~3) + ((rv + 3) & ~3);
}

__global__ __launch_bounds__(64) void combine_kernel(AttendArgs a) {
    extern __shared__ __align__(16) float cl[];
    const int lane = threadIdx.x;
    const int qh = blockIdx.x, i = blockIdx.y;   // grid (Hq, B)
    // all argument loads issued together (one scalar round trip)
    asm volatile("" ::"s"(a.partial), "s"(a.out), "s"(a.v.basis_cm), "s"(a.v.mu), "s"(a.v.r), "s"(a.gqa),
                 "s"(a.hpg), "s"(a.Hq), "s"(a.nsplit_call[i]), "s"(a.slot_call[i]), "s"(a.v.set_bcm), "s"(a.v.set_mu));
    const int h = qh / a.gqa, grp = h / a.hpg, rv = a.v.r;
    const int64_t slot = a.slot_call[i];
    int ns = a.nsplit_call[i];
    if (a.dev_len) {
        // decode step: splits from the attend kernel; the row's new length
        // is committed here, after every reader of the old one has run
        ns = a.row_info[2 * i + 1];
        if (qh == 0 && lane == 0) a.len_dev[slot] = a.row_info[2 * i];
    }
    const int np = ns * (rv + 2), npa = (np + 3) & ~3;
    float *pl = cl;                            // [ns][rv + 2]: m, l, o_lat
    float *bl = cl + npa;                      // [rv][D] value basis (channel-major)
    float *ml = bl + kHeadDim * rv;            // [D] value mean
    float *wl = ml + kHeadDim;                 // [ns] split weights
    float *ol = wl + ((ns + 3) & ~3);          // [rv] merged latent output
    const float *part = a.partial + (static_cast<int64_t>(i) * a.Hq + qh) * a.nsplit_max * (rv + 2);
    const float *bv = a.v.basis_cm + slot * a.v.set_bcm + static_cast<int64_t>(grp) * rv * kHeadDim;
    const float *mv = a.v.mu + slot * a.v.set_mu + grp * kHeadDim;

    if (ns <= 64 && rv <= 16) {
        // Register path: lane s holds split s's (m, l, latent output) and,
        // for its two outputs d = 2 lane, 2 lane + 1, the value basis of every
        // channel and the mean; every load is issued before the first use, and
        // the merge is a handful of wave reductions (no LDS round trips).
        const bool live = lane < ns;
        const float *ps = part + lane * (rv + 2);
        const float m = live ? ps[0] : -INFINITY;
        const float ls = live ? ps[1] : 0.0f;
        float oz[16];
        float2 bz[16];
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            oz[c] = 0.0f;
            bz[c] = make_float2(0.0f, 0.0f);
            if (c < rv) {
                if (live) oz[c] = ps[2 + c];
                bz[c] = *reinterpret_cast<const float2 *>(bv + c * kHeadDim + 2 * lane);
            }
        }
        const float2 mu = *reinterpret_cast<const float2 *>(mv + 2 * lane);
        const float M = wave_max(m);
        const float w = live ? exp2f(m - M) : 0.0f;
        const float inv_l = 1.0f / wave_sum(w * ls);
        // all 16 channel sums, unguarded: they are independent, so their
        // DPP steps interleave (channels past r_V sum zeros and add 0 * 0)
        float oc[16];
#pragma unroll
        for (int c = 0; c < 16; ++c) oc[c] = wave_sum(w * oz[c]) * inv_l;
        float o0 = mu.x, o1 = mu.y;
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            o0 = fmaf(bz[c].x, oc[c], o0);
            o1 = fmaf(bz[c].y, oc[c], o1);
        }
        reinterpret_cast<uint32_t *>(a.out + (static_cast<int64_t>(i) * a.Hq + qh) * kHeadDim)[lane] =
            out_bits(o0, a.bf16) | (out_bits(o1, a.bf16) << 16);
        return;
    }

    if (ns <= 64 && rv <= 64) {
        // Channel path: lane c owns latent channel c.  Lane s's split
        // maximum gives the row maximum and the split weights w_s (broadcast
        // by readlane); lane c sums w_s o_s[c] over the splits (one coalesced
        // row of the partials per split), then every lane projects its two
        // outputs d = 2 lane, 2 lane + 1 with the value basis, 16 channels
        // at a time (loads issued before the first use), taking channel c's
        // merged latent from lane c.  No LDS.
        const bool live = lane < ns;
        const float m = live ? part[lane * (rv + 2)] : -INFINITY;
        const float ls = live ? part[lane * (rv + 2) + 1] : 0.0f;
        const float M = wave_max(m);
        const float w = live ? exp2f(m - M) : 0.0f;
        const float inv_l = 1.0f / wave_sum(w * ls);
        const int cc = lane < rv ? lane : rv - 1;
        float acc = 0.0f;
        for (int s0 = 0; s0 < ns; s0 += 8) {
            float oz[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) oz[u] = s0 + u < ns ? part[(s0 + u) * (rv + 2) + 2 + cc] : 0.0f;
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (s0 + u < ns) acc = fmaf(lane_value(w, s0 + u), oz[u], acc);
        }
        const float oc = acc * inv_l;
        const float2 mu = *reinterpret_cast<const float2 *>(mv + 2 * lane);
        float o0 = mu.x, o1 = mu.y;
        for (int c0 = 0; c0 < rv; c0 += 16) {
            float2 bz[16];
#pragma unroll
            for (int u = 0; u < 16; ++u)
                bz[u] = c0 + u < rv ? *reinterpret_cast<const float2 *>(bv + (c0 + u) * kHeadDim + 2 * lane)
                                    : make_float2(0.0f, 0.0f);
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                if (c0 + u < rv) {
                    const float occ = lane_value(oc, c0 + u);
                    o0 = fmaf(bz[u].x, occ, o0);
                    o1 = fmaf(bz[u].y, occ, o1);
                }
            }
        }
        reinterpret_cast<uint32_t *>(a.out + (static_cast<int64_t>(i) * a.Hq + qh) * kHeadDim)[lane] =
            out_bits(o0, a.bf16) | (out_bits(o1, a.bf16) << 16);
        return;
    }

    // 1. copy to LDS: whole 16-byte pieces of the partials, the basis
    //    (128 rv floats) and the mean; the < 4 trailing partial floats singly
    {
        const int n4p = np >> 2, n4b = (kHeadDim * rv) >> 2, n4 = n4p + n4b + kHeadDim / 4;
        for (int base = 0; base < n4; base += 64 * 8) {
            float4 buf[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int e = base + 64 * u + lane;
                const float4 *src = e < n4p ? reinterpret_cast<const float4 *>(part) + e
                                  : e < n4p + n4b ? reinterpret_cast<const float4 *>(bv) + (e - n4p)
                                                  : reinterpret_cast<const float4 *>(mv) + (e - n4p - n4b);
                buf[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                if (e < n4) buf[u] = *src;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int e = base + 64 * u + lane;
                float4 *dst = e < n4p ? reinterpret_cast<float4 *>(pl) + e
                            : e < n4p + n4b ? reinterpret_cast<float4 *>(bl) + (e - n4p)
                                            : reinterpret_cast<float4 *>(ml) + (e - n4p - n4b);
                if (e < n4) *dst = buf[u];
            }
        }
        if (lane < np - 4 * n4p) pl[4 * n4p + lane] = part[4 * n4p + lane];
    }
    __syncthreads();

    // 2. split weights relative to the largest split maximum, and l
    const bool s0 = lane < ns, s1 = lane + 64 < ns;
    const float m0 = s0 ? pl[lane * (rv + 2)] : -INFINITY;
    const float m1 = s1 ? pl[(lane + 64) * (rv + 2)] : -INFINITY;
    const float M = wave_max(fmaxf(m0, m1));
    const float w0 = s0 ? exp2f(m0 - M) : 0.0f, w1 = s1 ? exp2f(m1 - M) : 0.0f;
    const float l = wave_sum(fmaf(w0, s0 ? pl[lane * (rv + 2) + 1] : 0.0f,
                                  w1 * (s1 ? pl[(lane + 64) * (rv + 2) + 1] : 0.0f)));
    if (s0) wl[lane] = w0;
    if (s1) wl[lane + 64] = w1;
    __syncthreads();

    // 3. merged latent output per channel: with r_v <= 16, four lanes per
    //    channel (lanes c, c + 16, c + 32, c + 48), each over every fourth
    //    split, then summed across the four rows of 16 lanes
    const float inv_l = 1.0f / l;
    if (rv <= 16) {
        const int c = lane & 15, part0 = lane >> 4;
        const int cc = c < rv ? c : 0;
        float acc = 0.0f;
        for (int sp = part0; sp < ns; sp += 4) acc = fmaf(wl[sp], pl[sp * (rv + 2) + 2 + cc], acc);
        acc += __shfl_xor(acc, 16);
        acc += __shfl_xor(acc, 32);
        if (lane < rv) ol[lane] = acc * inv_l;
    } else {
        for (int c = lane; c < rv; c += 64) {
            float acc = 0.0f;
            for (int sp = 0; sp < ns; ++sp) acc = fmaf(wl[sp], pl[sp * (rv + 2) + 2 + c], acc);
            ol[c] = acc * inv_l;
        }
    }
    __syncthreads();

    // 4. output projection, two adjacent outputs per lane
    const int d0 = 2 * lane;
    float o0 = ml[d0], o1 = ml[d0 + 1];
    for (int c = 0; c < rv; ++c) {
        const float oc = ol[c];
        const float2 b = *reinterpret_cast<const float2 *>(bl + c * kHeadDim + d0);   // conflict-free
        o0 = fmaf(b.x, oc, o0);
        o1 = fmaf(b.y, oc, o1);
    }
    reinterpret_cast<uint32_t *>(a.out + (static_cast<int64_t>(i) * a.Hq + qh) * kHeadDim)[lane] =
        out_bits(o0, a.bf16) | (out_bits(o1, a.bf16) << 16);
}

}  // namespace

size_t attend_lds_bytes(int gqa, int nbk, int r_k, int r_v, int words_k, int words_v, bool vq) {
    return static_cast<size_t>(attend_lds(gqa, nbk, r_k, r_v, words_k, words_v, vq).total);
}

template <int G, int NBV, bool VQ, bool GEN, int NBKF>
static hipError_t launch_attend_tgf(const AttendArgs &a, size_t lds_bytes, hipStream_t s) {
    // set once per process (thread-safe static initialisation)
    static const hipError_t attr =
        hipFuncSetAttribute(reinterpret_cast<const void *>(&attend_kernel<G, NBV, VQ, GEN, NBKF>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((attend_kernel<G, NBV, VQ, GEN, NBKF>), dim3(a.Hkv, a.B, a.nsplit_max), dim3(256), lds_bytes, s,
                       a);
    return hipGetLastError();
}

// The fast variant serves 4 query heads per kv head with a PALU-shaped key
// coder of at most 4 channel blocks and quantised values.
template <int G, int NBV, bool VQ, bool GEN>
static hipError_t launch_attend_tg(const AttendArgs &a, size_t lds_bytes, hipStream_t s) {
    const bool hi_first = a.k.cd.nseg == 2 && a.k.cd.bits[0] == 4 && a.k.cd.bits[1] == 2 && a.k.cd.c0[1] >= 1 &&
                          a.k.cd.c0[1] <= 8;
    if constexpr (G == 4 && VQ && !GEN) {
        if (hi_first) switch (coder_blocks(a.k.cd)) {
            case 1: return launch_attend_tgf<G, NBV, VQ, GEN, 1>(a, lds_bytes, s);
            case 2: return launch_attend_tgf<G, NBV, VQ, GEN, 2>(a, lds_bytes, s);
            case 3: return launch_attend_tgf<G, NBV, VQ, GEN, 3>(a, lds_bytes, s);
            case 4: return launch_attend_tgf<G, NBV, VQ, GEN, 4>(a, lds_bytes, s);
            default: break;
        }
    }
    return launch_attend_tgf<G, NBV, VQ, GEN, 0>(a, lds_bytes, s);
}

// A PALU-shaped coder: one 4-bit or 2-bit segment, or 4-bit then 2-bit.
static bool palu_shaped(const Coder &cd) {
    if (cd.nseg == 1) return cd.bits[0] == 4 || cd.bits[0] == 2;
    return cd.nseg == 2 && cd.bits[0] == 4 && cd.bits[1] == 2;
}

template <int G, int NBV, bool VQ>
static hipError_t launch_attend_t(const AttendArgs &a, size_t lds_bytes, hipStream_t s) {
    const bool gen = !palu_shaped(a.k.cd) || (VQ && !palu_shaped(a.v.cd));
    return gen ? launch_attend_tg<G, NBV, VQ, true>(a, lds_bytes, s) : launch_attend_tg<G, NBV, VQ, false>(a, lds_bytes, s);
}

template <int G, bool VQ>
static hipError_t launch_attend_v(const AttendArgs &a, size_t lds_bytes, hipStream_t s) {
    const int nbv = (a.v.r + 15) / 16;
    if (nbv <= 1) return launch_attend_t<G, 1, VQ>(a, lds_bytes, s);
    if (nbv <= 2) return launch_attend_t<G, 2, VQ>(a, lds_bytes, s);
    if (nbv <= 4) return launch_attend_t<G, 4, VQ>(a, lds_bytes, s);
    return launch_attend_t<G, 8, VQ>(a, lds_bytes, s);
}

template <int G>
static hipError_t launch_attend_g(const AttendArgs &a, size_t lds_bytes, hipStream_t s) {
    return a.v.fp16_latents ? launch_attend_v<G, false>(a, lds_bytes, s) : launch_attend_v<G, true>(a, lds_bytes, s);
}

hipError_t launch_attend(const AttendArgs &a, size_t lds_bytes, hipStream_t s) {
    switch (a.gqa) {
        case 1: return launch_attend_g<1>(a, lds_bytes, s);
        case 2: return launch_attend_g<2>(a, lds_bytes, s);
        case 3: return launch_attend_g<3>(a, lds_bytes, s);
        case 4: return launch_attend_g<4>(a, lds_bytes, s);
        case 5: return launch_attend_g<5>(a, lds_bytes, s);
        case 6: return launch_attend_g<6>(a, lds_bytes, s);
        case 7: return launch_attend_g<7>(a, lds_bytes, s);
        case 8: return launch_attend_g<8>(a, lds_bytes, s);
        default: return hipErrorInvalidValue;
    }
}

// Split partials of the allocation-free decode entry point: one array per
// device, alive until the process ends.  Host code never passes the array's
// name to a kernel (on the host it only stands for the symbol); it passes the
// device address looked up below.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

hipError_t static_scratch_address(void **ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        // with this device current: its own copy of the array
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_combine(const AttendArgs &a, hipStream_t s) {
    // set once per process (thread-safe static initialisation)
    static const hipError_t attr =
        hipFuncSetAttribute(reinterpret_cast<const void *>(combine_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (attr != hipSuccess) return attr;
    // the register and channel paths (at most 64 splits, r_V <= 64) use no LDS
    const size_t lds = a.nsplit_max <= 64 && a.v.r <= 64
                           ? 0
                           : static_cast<size_t>(combine_lds_floats(a.nsplit_max, a.v.r)) * sizeof(float);
    hipLaunchKernelGGL(combine_kernel, dim3(a.Hq, a.B), dim3(64), lds, s, a);
    return hipGetLastError();
}

}  // namespace palu
