// Causal prefill attention over the latent cache, for gfx950 (MI355X).
//
// The PALU page ("How it works", prefill step 6) reconstructs K/V from the
// stored latents for the attention call that follows the encode.  This
// kernel computes that attention without materialising K or V in head
// space.  With the query absorbed into the key basis,
//   score(p, t) = qs q_p . (V_K l_t + mu_K) = qt_p . l_t + const(p),
//   qt_p = qs V_K^T q_p,  qs = softmax scale * log2 e,
// and the per-query constant cancels in the softmax.  The value side
// accumulates o_lat = sum_t w_t lv_t in latent space and projects once at
// the end: o = V_V o_lat / l + mu_V.
//
// Workgroup = (kv head h, query tile x, call row i), four waves.  Its 64 NQ
// columns are (query position, query head) pairs: column c holds position
// c / g and head c % g of the kv head's g query heads.  Wave w owns columns
// [16 NQ w, 16 NQ (w + 1)) as NQ MFMA tiles of 16.  The key loop walks the
// 32-token groups 0 .. (last position) / 32.  Each group is staged once per
// workgroup as two fp16 tiles in LDS:
//   key tile   [32 tokens][32 KS positions]: score-operand position order
//              (8-channel blocks, hi blocks first, channels c0,c4,c1,c5,...
//              inside a block; padding positions 0), matching the
//              position-ordered fp16 key basis the query is absorbed with;
//   value tile [16 NBV channels][32 tokens]: natural channel order; channel
//              r_V is all ones, so the value MFMA also sums the weights.
// A complete group comes from its packed record (code * fp16 scale + fp16
// zero in fp16, the decode kernel's dequantisation).  The incomplete group
// comes from the fp32 tail (or the partial fp16 record) rounded to fp16.
// Groups go in pairs, one barrier per pair.  Without a workspace (PRE =
// false) records are copied global -> LDS two pairs ahead (direct 16-byte
// loads into LDS) and the tiles built one pair ahead; with one (PRE = true)
// prefill_tiles_kernel has decoded every complete group's tile pair into it
// once, with the same arithmetic, and the tile pairs are copied global ->
// LDS one pair ahead instead (only the incomplete group is built here).
//
// Per wave and group: scores S^T[t][col] = sum_k Khat[t][k] Qt[col][k] on
// v_mfma_f32_16x16x32_f16 (two 16-token halves, KS K-steps, NQ column
// tiles), with the running maximum folded into the accumulator input
// (C = -m).  Causal masking runs only on groups that reach past one of the
// wave's positions.  The online softmax is lazy: it rescales only when a
// group's maximum exceeds the running one by more than kPfSlack (log2
// units).  Weights 2^(s - m) are rounded to fp16, and
// O[col][c] += sum_t P[col][t] Vhat[t][c] runs on MFMA.  In both MFMAs K
// index i stands for token (or position) i: score half hh takes the tokens
// 2 row + hh as its rows (and the query absorption the positions likewise),
// so the accumulator values v of halves 0 and 1 are the adjacent tokens
// 8 kb + 2 v and 8 kb + 2 v + 1, and every operand is one 16-byte LDS read
// of 8 consecutive tile elements.
#include "palu_device.h"
#include "palu_internal.h"

namespace palu {

namespace {

constexpr int kPfWaves = kPrefillWaves;
constexpr int kPfThreads = 64 * kPfWaves;
constexpr float kPfSlack = 8.0f;
constexpr int kVRow = 40;   // halves per value-tile row: 32 tokens + 8 padding


__host__ __device__ constexpr int pf_krow(int ks) { return 32 * ks + 8; }   // halves per key-tile row

// Rings of raw record buffers and tile pairs: groups 2i and 2i + 1 are
// computed while 2i + 2 and 2i + 3 are built and 2i + 4 and 2i + 5 copied.
constexpr int kPfRing = 4;

struct PrefillLds {
    int raw, raw_words;    // kPfRing raw record buffers (K record, then V record)
    int tiles, ktile, vtile;   // kPfRing (key tile, value tile) pairs; bytes of each tile
    int basis;             // epilogue: fp32 value basis [D][r_V] + mean [D] (aliases the above)
    int tab;               // key block table (int4 per block) + value channel table (int2 per channel)
    int olat;              // per wave [16 NQ][16 NBV] fp32 normalised latent outputs
    int total;
};

__host__ __device__ inline PrefillLds prefill_lds(int ks, int nbv, int nq, int wk, int wv, int rv, int nbk) {
    PrefillLds L;
    L.raw_words = ((wk + 3) & ~3) + 4 + ((wv + 3) & ~3) + 4;
    L.ktile = 32 * pf_krow(ks) * 2;
    L.vtile = 16 * nbv * kVRow * 2;
    int a = 0;
    L.raw = lds_take(a, kPfRing * L.raw_words * 4);
    L.tiles = lds_take(a, kPfRing * (L.ktile + L.vtile));
    int b = 0;
    L.basis = lds_take(b, (kHeadDim * rv + kHeadDim) * 4);
    int o = a > b ? a : b;
    L.olat = lds_take(o, kPfWaves * 16 * nq * 16 * nbv * 4);
    L.tab = lds_take(o, nbk * 16 + rv * 8);
    L.total = o;
    return L;
}

// Query tiles per wave: the query operand (4 KS registers per tile) and the
// value accumulators (4 NBV per tile) stay within about 64 registers.
__host__ __device__ constexpr int prefill_nq_c(int ks, int nbv) {
    return 16 / (ks + nbv) >= 4 ? 4 : (16 / (ks + nbv) >= 2 ? 2 : 1);
}

// ---- one 16-byte item of a complete group's fp16 tiles for the tile
//      pre-decode kernel: the same operations in the same order as the
//      prefill kernel's own decode of a complete group (build_tiles there,
//      kept inline: as a shared function it changed that kernel's register
//      allocation), so both write the same bits
// Key item: the 8 score-operand positions of key block kq (base bit, bit
// stride, width, chan0 | chanend << 16) for token t, dequantised from the
// group's K record kr (scale/zero words from kmeta).
template <bool GEN>
__device__ __forceinline__ uint4 tile_key_item(const uint32_t *kr, int kmeta, int4 kq, int t) {
    const int chan0 = kq.w & 0xFFFF, chanend = kq.w >> 16;
    const int bit = kq.x + t * kq.y;
    const uint32_t X = __builtin_amdgcn_alignbit(kr[(bit >> 5) + 1], kr[bit >> 5], bit & 31);
    const uint32_t Y = GEN && kq.z == 8 ? __builtin_amdgcn_alignbit(kr[(bit >> 5) + 2], kr[(bit >> 5) + 1], bit & 31)
                                        : 0u;
    uint32_t sp[4], zp[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t wa = chan0 + k < chanend ? kr[kmeta + chan0 + k] : 0u;
        const uint32_t wb = chan0 + k + 4 < chanend ? kr[kmeta + chan0 + k + 4] : 0u;
        sp[k] = perm_b32(wb, wa, 0x05040100u);
        zp[k] = perm_b32(wb, wa, 0x07060302u);
    }
    const uint4 spv = make_uint4(sp[0], sp[1], sp[2], sp[3]), zpv = make_uint4(zp[0], zp[1], zp[2], zp[3]);
    return __builtin_bit_cast(uint4, GEN ? dequant8_w(X, Y, kq.z, spv, zpv) : dequant8_any(X, kq.z == 4, spv, zpv));
}

// Value item of a complete group with quantised values: tokens 8 tb ..
// 8 tb + 7 of channel c (vcw = base bit, width), dequantised from the
// group's V record vr (scale/zero word of the channel at vmeta + c).
template <bool GEN>
__device__ __forceinline__ uint4 tile_value_item(const uint32_t *vr, int vmeta, int2 vcw, int c, int tb) {
    const int wc = vcw.y;
    const int bit = vcw.x + 8 * tb * wc;
    const uint32_t mw = vr[vmeta + c];
    const uint32_t spair = (mw & 0xFFFFu) | (mw << 16), zpair = (mw >> 16) | (mw & 0xFFFF0000u);
    uint32_t wd[4];
    if (GEN && wc == 8) {
        // 8 tokens = 2 whole words; token u is byte u of the pair
        const uint32_t Xa = vr[bit >> 5], Xb = vr[(bit >> 5) + 1];
        wd[0] = dequant_pair(perm_b32(Xb, Xa, 0x0C010C00u) | 0x64006400u, spair, zpair);
        wd[1] = dequant_pair(perm_b32(Xb, Xa, 0x0C030C02u) | 0x64006400u, spair, zpair);
        wd[2] = dequant_pair(perm_b32(Xb, Xa, 0x0C050C04u) | 0x64006400u, spair, zpair);
        wd[3] = dequant_pair(perm_b32(Xb, Xa, 0x0C070C06u) | 0x64006400u, spair, zpair);
    } else {
        const uint32_t X = __builtin_amdgcn_alignbit(vr[(bit >> 5) + 1], vr[bit >> 5], bit & 31);
        const uint32_t m = (1u << wc) - 1u;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t lo = (X >> (2 * k * wc)) & m, hi = (X >> ((2 * k + 1) * wc)) & m;
            wd[k] = dequant_pair(lo | (hi << 16) | 0x64006400u, spair, zpair);
        }
    }
    return make_uint4(wd[0], wd[1], wd[2], wd[3]);
}

// Tile pre-decode: the fp16 key and value tiles of every complete group of
// the call's rows, byte for byte as the prefill kernel lays a tile pair out
// in LDS (zero key positions past the key blocks, the all-ones value
// channel r_V, zero channels after it, zero row padding), into the
// workspace at tile tile_base[call row] + kv head * nfull + group.  One wave
// per group, one 16-byte item per lane and round.  A prompt's groups are
// then decoded once, not once per query tile that reads them.
template <int KS, int NBV, bool GEN>
__global__ __launch_bounds__(256) void prefill_tiles_kernel(PrefillArgs a) {
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = blockIdx.y, i = blockIdx.z;
    const PrefillRow rw = a.row[i];
    const int nfull = rw.len >> 5;
    const int j = blockIdx.x * 4 + wv;
    if (j >= nfull) return;                          // per wave: the kernel has no barrier
    const int64_t ci = rw.sel_qi >> 1;
    const int rk = a.k.r, rv = a.v.r, nbk = coder_blocks(a.k.cd);
    const bool vq = !a.v.fp16_latents;
    const int nhk = a.k.cd.bits[0] == 4 ? a.k.cd.c0[1] : 0, nlk = rk - nhk, nbh = (nhk + 7) >> 3;
    const int nhv = a.v.cd.bits[0] == 4 ? a.v.cd.c0[1] : 0;
    const int64_t hb = static_cast<int64_t>(rw.slot) * a.Hkv + h;
    const uint32_t *kr = a.k.records + hb * a.k.head_stride + static_cast<int64_t>(j) * a.k.words;
    const uint32_t *vr = a.v.records + hb * a.v.head_stride + static_cast<int64_t>(j) * a.v.words;
    constexpr int kq16 = pf_krow(KS) / 8, vq16 = kVRow / 8;   // 16-byte items per key / value tile row
    constexpr int nk16 = 32 * kq16, nv16 = 16 * NBV * vq16;
    uint4 *dst = reinterpret_cast<uint4 *>(a.ws_tiles + (a.tile_base[ci] + static_cast<int64_t>(h) * nfull + j) *
                                                            static_cast<int64_t>(a.tile_bytes));
    for (int e = lane; e < nk16 + nv16; e += 64) {
        uint4 val = make_uint4(0u, 0u, 0u, 0u);
        if (e < nk16) {
            const int t = e / kq16, q = e - t * kq16;   // token, 8-position block
            if (q < nbk) {
                int4 kq;
                if constexpr (GEN) {
                    const KBlock b = key_block(a.k.cd, q);
                    kq = make_int4(b.base, b.stride, b.w, b.chan0 | (b.chanend << 16));
                } else {
                    const bool w4 = q < nbh;
                    kq = make_int4(w4 ? 32 * q : 128 * nhk + 16 * (q - nbh), w4 ? 4 * nhk : 2 * nlk, w4 ? 4 : 2,
                                   (w4 ? 8 * q : nhk + 8 * (q - nbh)) | ((w4 ? nhk : rk) << 16));
                }
                val = tile_key_item<GEN>(kr, a.k.cd.meta0, kq, t);
            }
        } else {
            const int e2 = e - nk16, c = e2 / vq16, tb = e2 - c * vq16;   // channel, 8-token block
            if (tb < 4) {
                if (c < rv) {
                    if (vq) {
                        const int2 vcw = GEN ? value_channel(a.v.cd, c)
                                             : (c < nhv ? make_int2(128 * c, 4)
                                                        : make_int2(128 * nhv + 64 * (c - nhv), 2));
                        val = tile_value_item<GEN>(vr, a.v.cd.meta0, vcw, c, tb);
                    } else {
                        val = *reinterpret_cast<const uint4 *>(vr + c * 16 + 4 * tb);
                    }
                } else if (c == rv) {
                    val = make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);
                }
            }
        }
        dst[e] = val;
    }
}

// GEN = false: PALU-shaped layouts (a 4-bit segment, then 2-bit channels),
// closed-form record addressing; GEN = true: any coder, through LDS tables.
// PRE = true: complete groups come pre-decoded from a.ws_tiles (a
// compile-time choice: a runtime one cost both variants registers).
template <int KS, int NBV, int NQ, bool GEN, bool PRE>
__global__ __launch_bounds__(kPfThreads) __attribute__((amdgpu_waves_per_eu(KS + NBV <= 2 ? 4 : 1)))
void prefill_kernel(PrefillArgs a) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ln = lane & 15, kb = lane >> 4;
    // grid (kv head, query tile, row), head fastest: round-robin XCD
    // placement keeps the tiles of one (row, kv head) on one XCD, whose L2
    // then serves their shared records and basis, and the row slowest keeps
    // the rows in flight (the records the L2s must hold) few
    const int h = blockIdx.x, i = blockIdx.z;
    const PrefillRow rw = a.row[i];
    const int64_t ci = rw.sel_qi >> 1;                       // the row's index in the call
    const int nq = rw.nq;
    const int ntiles = (nq + a.qp - 1) / a.qp;
    if (static_cast<int>(blockIdx.y) >= ntiles) return;   // whole workgroup, before any barrier
    const int x = ntiles - 1 - static_cast<int>(blockIdx.y);   // longest tiles first
    const int g = a.gqa, len = rw.len;
    const int nfull = len >> 5, ntail = len & 31;
    const int grp = h / a.hpg;
    const int rk = a.k.r;
    const int nbk = coder_blocks(a.k.cd), np = 8 * nbk;
    const int rv = a.v.r;
    const int WK = a.k.words, WV = a.v.words;
    const bool vq = !a.v.fp16_latents;
    const int kmeta = a.k.cd.meta0, vmeta = a.v.cd.meta0;
    const PrefillLds L = prefill_lds(KS, NBV, NQ, WK, WV, rv, nbk);
    int4 *ktab = reinterpret_cast<int4 *>(lds + L.tab);          // base, stride, width, chan0 | chanend << 16
    int2 *vtab = reinterpret_cast<int2 *>(lds + L.tab + nbk * 16);   // base bit, width
    // PALU-shaped layouts: nhk (nhv) 4-bit channels, then 2-bit ones
    const int nhk = a.k.cd.bits[0] == 4 ? a.k.cd.c0[1] : 0, nlk = rk - nhk, nbh = (nhk + 7) >> 3;
    const int nhv = a.v.cd.bits[0] == 4 ? a.v.cd.c0[1] : 0;
    constexpr int krow = 32 * KS + 8;

    // ---- query columns: index qi -> position len - nq + qi; columns past
    //      the tile or the call repeat the tile's last query and are not stored
    const int q0 = x * a.qp;
    const int qlast = min(q0 + a.qp, nq) - 1;
    const int pbase = len - nq;
    const int c_lo = wv * 16 * NQ;
    const int pw_lo = pbase + min(q0 + c_lo / g, qlast);
    const int pw_hi = pbase + min(q0 + (c_lo + 16 * NQ - 1) / g, qlast);
    const int ngroups = (pbase + qlast) / 32 + 1;
    int pcol[NQ];
    const uint16_t *qsrc[NQ];
#pragma unroll
    for (int t = 0; t < NQ; ++t) {
        const int c = c_lo + 16 * t + ln, pl = c / g, hd = c - pl * g;
        const int qi = min(q0 + pl, qlast);
        pcol[t] = pbase + qi;
        qsrc[t] = a.q + ((ci * a.Hq + h * g + hd) * a.T_stride + qi) * kHeadDim;
    }

    const int64_t hb = static_cast<int64_t>(rw.slot) * a.Hkv + h;
    const uint32_t *kg = a.k.records + hb * a.k.head_stride;
    const uint32_t *vg = a.v.records + hb * a.v.head_stride;

    // ---- raw records of group j (< nfull) -> raw buffer j % kPfRing
    auto rec_offsets = [&](int j, int &koff, int &nk4, int &voff, int &nv4) {
        const int64_t ka = (static_cast<int64_t>(j) * WK) & ~3LL, va = (static_cast<int64_t>(j) * WV) & ~3LL;
        koff = static_cast<int>(static_cast<int64_t>(j) * WK - ka);
        nk4 = static_cast<int>((static_cast<int64_t>(j + 1) * WK - ka + 3) >> 2);
        voff = 4 * nk4 + static_cast<int>(static_cast<int64_t>(j) * WV - va);
        nv4 = static_cast<int>((static_cast<int64_t>(j + 1) * WV - va + 3) >> 2);
    };
    auto copy_raw = [&](unsigned char *base, int j) {
        int koff, nk4, voff, nv4;
        rec_offsets(j, koff, nk4, voff, nv4);
        const u4v *ks = reinterpret_cast<const u4v *>(kg + ((static_cast<int64_t>(j) * WK) & ~3LL));
        const u4v *vs = reinterpret_cast<const u4v *>(vg + ((static_cast<int64_t>(j) * WV) & ~3LL));
        const int n4 = nk4 + nv4;
        unsigned char *dst = base + L.raw + (j & (kPfRing - 1)) * L.raw_words * 4;
        for (int c = wv; c * 64 < n4; c += kPfWaves) {
            const int e = c * 64 + lane;
            if (e < n4) __builtin_amdgcn_global_load_lds(e < nk4 ? ks + e : vs + (e - nk4), dst + c * 1024, 16, 0, 0);
        }
    };

    // ---- pre-decoded tiles of group j (< nfull) -> tile pair j % kPfRing,
    //      whole (data and constant parts), with direct 16-byte loads
    constexpr bool pre = PRE;
    auto copy_tile = [&](unsigned char *base, int j) {
        const int nb16 = a.tile_bytes >> 4;
        const u4v *src = reinterpret_cast<const u4v *>(
            a.ws_tiles + (a.tile_base[ci] + static_cast<int64_t>(h) * nfull + j) * static_cast<int64_t>(a.tile_bytes));
        unsigned char *dst = base + L.tiles + (j & (kPfRing - 1)) * (L.ktile + L.vtile);
        for (int c = wv; c * 64 < nb16; c += kPfWaves) {
            const int e = c * 64 + lane;
            if (e < nb16) __builtin_amdgcn_global_load_lds(src + e, dst + c * 1024, 16, 0, 0);
        }
    };

    // ---- fp16 tiles of group j -> tile pair j % kPfRing (data parts only).
    //      The items come in rounds of 64 (one per lane): key rounds, then
    //      value rounds; round r goes to wave (rot + r) % 4, so whole waves
    //      build (no partly filled item loops in every wave) and the two
    //      groups built together share the waves evenly.
    const int nrk = (32 * nbk + 63) >> 6, nrv = (4 * rv + 63) >> 6;
    auto build_tiles = [&](unsigned char *base, int j, int rot) {
        const int slot = j & (kPfRing - 1);
        _Float16 *kt = reinterpret_cast<_Float16 *>(base + L.tiles + slot * (L.ktile + L.vtile));
        _Float16 *vt = reinterpret_cast<_Float16 *>(base + L.tiles + slot * (L.ktile + L.vtile) + L.ktile);
        const int4 *ktab = reinterpret_cast<const int4 *>(base + L.tab);
        const int2 *vtab = reinterpret_cast<const int2 *>(base + L.tab + nbk * 16);
        const bool full = j < nfull;
        int koff = 0, nk4 = 0, voff = 0, nv4 = 0;
        if (full) rec_offsets(j, koff, nk4, voff, nv4);
        const uint32_t *raw = reinterpret_cast<const uint32_t *>(base + L.raw) + slot * L.raw_words;
        const uint32_t *kr = raw + koff, *vr = raw + voff;
        const float *tk = a.k.tail + (hb * 2 + (rw.sel_qi & 1)) * kTokGroup * rk;
        const float *tv = vq ? a.v.tail + (hb * 2 + (rw.sel_qi & 1)) * kTokGroup * rv : nullptr;
        const uint16_t *r16 = reinterpret_cast<const uint16_t *>(vg + static_cast<int64_t>(nfull) * WV);
        for (int r = (wv - rot) & (kPfWaves - 1); r < nrk + nrv; r += kPfWaves) {
            if (r < nrk) {
                // key item: (8-position block q < nbk, token t)
                const int e = 64 * r + lane;
                if (e >= 32 * nbk) continue;
                const int q = e >> 5, t = e & 31;
                int4 kq;                                  // base, stride, width, channels
                if constexpr (GEN) {
                    kq = ktab[q];
                } else {
                    const bool w4 = q < nbh;
                    kq = make_int4(w4 ? 32 * q : 128 * nhk + 16 * (q - nbh), w4 ? 4 * nhk : 2 * nlk, w4 ? 4 : 2,
                                   (w4 ? 8 * q : nhk + 8 * (q - nbh)) | ((w4 ? nhk : rk) << 16));
                }
                const int chan0 = kq.w & 0xFFFF, chanend = kq.w >> 16;
                uint4 val;
                if (full) {
                    const int bit = kq.x + t * kq.y;
                    const uint32_t X = __builtin_amdgcn_alignbit(kr[(bit >> 5) + 1], kr[bit >> 5], bit & 31);
                    const uint32_t Y = GEN && kq.z == 8 ? __builtin_amdgcn_alignbit(kr[(bit >> 5) + 2],
                                                                                   kr[(bit >> 5) + 1], bit & 31)
                                                        : 0u;
                    uint32_t sp[4], zp[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const uint32_t wa = chan0 + k < chanend ? kr[kmeta + chan0 + k] : 0u;
                        const uint32_t wb = chan0 + k + 4 < chanend ? kr[kmeta + chan0 + k + 4] : 0u;
                        sp[k] = perm_b32(wb, wa, 0x05040100u);
                        zp[k] = perm_b32(wb, wa, 0x07060302u);
                    }
                    const uint4 spv = make_uint4(sp[0], sp[1], sp[2], sp[3]), zpv = make_uint4(zp[0], zp[1], zp[2], zp[3]);
                    val = __builtin_bit_cast(uint4, GEN ? dequant8_w(X, Y, kq.z, spv, zpv)
                                                        : dequant8_any(X, kq.z == 4, spv, zpv));
                } else {
                    // incomplete group: fp32 tail rounded to fp16, 0 past ntail
                    uint32_t wd[4] = {0u, 0u, 0u, 0u};
                    if (t < ntail) {
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            const float fa = chan0 + k < chanend ? tk[t * rk + chan0 + k] : 0.0f;
                            const float fb = chan0 + k + 4 < chanend ? tk[t * rk + chan0 + k + 4] : 0.0f;
                            wd[k] = f2h_bits(fa) | (f2h_bits(fb) << 16);
                        }
                    }
                    val = make_uint4(wd[0], wd[1], wd[2], wd[3]);
                }
                *reinterpret_cast<uint4 *>(kt + t * krow + 8 * q) = val;
            } else {
                // value item: (channel c < r_V, 8-token block tb)
                const int e = 64 * (r - nrk) + lane;
                if (e >= 4 * rv) continue;
                const int c = e >> 2, tb = e & 3;
                uint4 val;
                if (full && vq) {
                    const int2 vcw = GEN ? vtab[c]
                                         : (c < nhv ? make_int2(128 * c, 4) : make_int2(128 * nhv + 64 * (c - nhv), 2));
                    const int wc = vcw.y;
                    const int bit = vcw.x + 8 * tb * wc;
                    const uint32_t mw = vr[vmeta + c];
                    const uint32_t spair = (mw & 0xFFFFu) | (mw << 16), zpair = (mw >> 16) | (mw & 0xFFFF0000u);
                    uint32_t wd[4];
                    if (GEN && wc == 8) {
                        // 8 tokens = 2 whole words; token u is byte u of the pair
                        const uint32_t Xa = vr[bit >> 5], Xb = vr[(bit >> 5) + 1];
                        wd[0] = dequant_pair(perm_b32(Xb, Xa, 0x0C010C00u) | 0x64006400u, spair, zpair);
                        wd[1] = dequant_pair(perm_b32(Xb, Xa, 0x0C030C02u) | 0x64006400u, spair, zpair);
                        wd[2] = dequant_pair(perm_b32(Xb, Xa, 0x0C050C04u) | 0x64006400u, spair, zpair);
                        wd[3] = dequant_pair(perm_b32(Xb, Xa, 0x0C070C06u) | 0x64006400u, spair, zpair);
                    } else {
                        const uint32_t X = __builtin_amdgcn_alignbit(vr[(bit >> 5) + 1], vr[bit >> 5], bit & 31);
                        const uint32_t m = (1u << wc) - 1u;
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            const uint32_t lo = (X >> (2 * k * wc)) & m, hi = (X >> ((2 * k + 1) * wc)) & m;
                            wd[k] = dequant_pair(lo | (hi << 16) | 0x64006400u, spair, zpair);
                        }
                    }
                    val = make_uint4(wd[0], wd[1], wd[2], wd[3]);
                } else if (full) {
                    val = *reinterpret_cast<const uint4 *>(vr + c * 16 + 4 * tb);
                } else {
                    uint32_t wd[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        uint32_t hv[2];
#pragma unroll
                        for (int u = 0; u < 2; ++u) {
                            const int tok = 8 * tb + 2 * k + u;
                            hv[u] = tok < ntail ? (vq ? f2h_bits(tv[tok * rv + c]) : static_cast<uint32_t>(r16[c * 32 + tok]))
                                                : 0u;
                        }
                        wd[k] = hv[0] | (hv[1] << 16);
                    }
                    val = make_uint4(wd[0], wd[1], wd[2], wd[3]);
                }
                *reinterpret_cast<uint4 *>(vt + c * kVRow + 8 * tb) = val;
            }
        }
    };

    // ---- the tiles' constant parts, written once for every buffer: key
    //      positions past the last channel block are 0; value channel r_V is
    //      all ones and the channels after it are 0
    for (int e = tid; e < kPfRing * 32 * (4 * KS - nbk); e += kPfThreads) {
        const int bf = e & (kPfRing - 1), r = e / kPfRing, t = r & 31, q = nbk + (r >> 5);
        *reinterpret_cast<uint4 *>(lds + L.tiles + bf * (L.ktile + L.vtile) + (t * krow + 8 * q) * 2) =
            make_uint4(0u, 0u, 0u, 0u);
    }
    for (int e = tid; e < kPfRing * 4 * (16 * NBV - rv); e += kPfThreads) {
        const int bf = e & (kPfRing - 1), r = e / kPfRing, tb = r & 3, c = rv + (r >> 2);
        const uint32_t w = c == rv ? 0x3C003C00u : 0u;
        *reinterpret_cast<uint4 *>(lds + L.tiles + bf * (L.ktile + L.vtile) + L.ktile + (c * kVRow + 8 * tb) * 2) =
            make_uint4(w, w, w, w);
    }

    // ---- record addressing tables (per key block, per value channel)
    if (GEN && tid < nbk) {
        const KBlock b = key_block(a.k.cd, tid);
        ktab[tid] = make_int4(b.base, b.stride, b.w, b.chan0 | (b.chanend << 16));
    }
    if (GEN && vq && tid < rv) vtab[tid] = value_channel(a.v.cd, tid);

    // ---- prologue: records of groups 0 and 1 in flight while the query is
    //      absorbed: qt = qs V_K^T q on MFMA, A = position-ordered key basis
    //      rows (16 positions x 32 d), B = the column's query (32 d x 16
    //      columns; block 2 ks + hh takes positions 32 ks + 2 row + hh);
    //      D[position][column] packed straight into the fp16 score operand
    //      qb (K index 8 kb + 2 v + hh <- position 32 ks + 8 kb + 2 v + hh)
    if constexpr (pre) {
        for (int j = 0; j < 2; ++j)
            if (j < nfull && j < ngroups) copy_tile(lds, j);
    } else {
        for (int j = 0; j < kPfRing; ++j)
            if (j < nfull && j < ngroups) copy_raw(lds, j);
    }
    f16x8 qb[NQ][KS];
    {
        const uint16_t *bt = a.k.basis_t16 + rw.slot * a.k.set_bt16 + static_cast<int64_t>(grp) * np * kHeadDim;
#pragma unroll
        for (int t = 0; t < NQ; ++t) {
            uint4 qa[4];
#pragma unroll
            for (int st = 0; st < 4; ++st) qa[st] = *reinterpret_cast<const uint4 *>(qsrc[t] + 32 * st + 8 * kb);
            // bf16 queries: exact per-column power-of-two rescale into fp16
            // (the MFMA result of column ln sits in this lane)
            const float qsc = a.bf16 ? ldexpf(a.qscale, bf16_rows_to_fp16(qa)) : a.qscale;
            f4 acc[2 * KS];
#pragma unroll
            for (int blk = 0; blk < 2 * KS; ++blk) {
                const int n = 32 * (blk >> 1) + 2 * ln + (blk & 1);
                acc[blk] = (f4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int st = 0; st < 4; ++st) {
                    const uint4 bb = n < np ? *reinterpret_cast<const uint4 *>(bt + static_cast<int64_t>(n) * kHeadDim +
                                                                               32 * st + 8 * kb)
                                            : make_uint4(0u, 0u, 0u, 0u);
                    acc[blk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h8(bb.x, bb.y, bb.z, bb.w),
                                                                     as_h8(qa[st].x, qa[st].y, qa[st].z, qa[st].w),
                                                                     acc[blk], 0, 0, 0);
                }
            }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                uint32_t wd[4];
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    wd[v] = pack_half2(acc[2 * ks][v] * qsc, acc[2 * ks + 1][v] * qsc);
                qb[t][ks] = as_h8(wd[0], wd[1], wd[2], wd[3]);
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // (with pre-decoded tiles only the incomplete group is built here)
    if (!pre || nfull == 0) build_tiles(lds, 0, 0);
    if (ngroups > 1 && (!pre || nfull <= 1)) build_tiles(lds, 1, nrk + nrv);
    __syncthreads();

    // ---- key loop
    f4 negm[NQ];            // -(running maximum) of each column, as the score MFMA's C operand
    f4 oacc[NQ][NBV];
#pragma unroll
    for (int t = 0; t < NQ; ++t) {
        negm[t] = (f4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int nb = 0; nb < NBV; ++nb) oacc[t][nb] = (f4){0.0f, 0.0f, 0.0f, 0.0f};
    }
    // group j's scores, softmax and value contraction from its tiles
    auto compute_group = [&](const unsigned char *base, int j) {
        if (32 * j <= pw_hi) {                       // wave-uniform
            const int slot = j & (kPfRing - 1);
            const _Float16 *kt = reinterpret_cast<const _Float16 *>(base + L.tiles + slot * (L.ktile + L.vtile));
            const _Float16 *vt = reinterpret_cast<const _Float16 *>(base + L.tiles + slot * (L.ktile + L.vtile) +
                                                                    L.ktile);
            f16x8 ka[2][KS];     // half hh, row ln: token 2 ln + hh
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const uint4 w = *reinterpret_cast<const uint4 *>(kt + (2 * ln + hh) * krow + 32 * ks + 8 * kb);
                    ka[hh][ks] = as_h8(w.x, w.y, w.z, w.w);
                }
            }
            f16x8 vb[NBV];       // channel 16 nb + ln, tokens 8 kb .. 8 kb + 7
#pragma unroll
            for (int nb = 0; nb < NBV; ++nb) {
                const uint4 w = *reinterpret_cast<const uint4 *>(vt + (16 * nb + ln) * kVRow + 8 * kb);
                vb[nb] = as_h8(w.x, w.y, w.z, w.w);
            }
            const bool masked = 32 * j + 31 > pw_lo;    // wave-uniform
            // (a) every tile's scores first (the softmax of tile t then finds
            //     its MFMA results long done); running max as the C operand
            float xv[NQ][8];
#pragma unroll
            for (int t = 0; t < NQ; ++t) {
                f4 s0 = negm[t], s1 = negm[t];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[0][ks], qb[t][ks], s0, 0, 0, 0);
                    s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[1][ks], qb[t][ks], s1, 0, 0, 0);
                }
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    xv[t][v] = s0[v];
                    xv[t][4 + v] = s1[v];
                }
            }
            // (b) causal mask on the groups that reach past a column's position
            if (masked) {
#pragma unroll
                for (int t = 0; t < NQ; ++t) {
                    const int lim = pcol[t] - 32 * j - 8 * kb;   // token 8 kb + 2 v + hh allowed iff 2 v + hh <= lim
#pragma unroll
                    for (int k = 0; k < 8; ++k) xv[t][k] = 2 * (k & 3) + (k >> 2) <= lim ? xv[t][k] : -INFINITY;
                }
            }
            // (c) lazy rescale: one test for the whole wave and all tiles,
            //     on the maximum of all the lane's values (three-input max
            //     steps); the per-tile maxima only when a rescale is due
            float mall = xv[0][0];
#pragma unroll
            for (int i = 1; i + 1 < 8 * NQ; i += 2) mall = fmaxf(fmaxf(mall, xv[i / 8][i % 8]), xv[(i + 1) / 8][(i + 1) % 8]);
            mall = fmaxf(mall, xv[NQ - 1][7]);
            if (j == 0 || __builtin_amdgcn_ballot_w64(mall > kPfSlack) != 0) {
                float mloc[NQ];
#pragma unroll
                for (int t = 0; t < NQ; ++t)
                    mloc[t] = fmaxf(fmaxf(fmaxf(xv[t][0], xv[t][1]), fmaxf(xv[t][2], xv[t][3])),
                                    fmaxf(fmaxf(xv[t][4], xv[t][5]), fmaxf(xv[t][6], xv[t][7])));
#pragma unroll
                for (int t = 0; t < NQ; ++t) {
                    // column maximum of s - m over the 4 lanes that hold the
                    // column; every valid column sees token 0 in group 0
                    float mm = fmaxf(mloc[t], __shfl_xor(mloc[t], 16));
                    mm = fmaxf(mm, __shfl_xor(mm, 32));
                    const bool upd = j == 0 || mm > kPfSlack;
                    const float delta = upd ? mm : 0.0f;
                    const float alpha = j == 0 ? 0.0f : exp2f(-delta);
                    negm[t] -= (f4){delta, delta, delta, delta};
#pragma unroll
                    for (int k = 0; k < 8; ++k) xv[t][k] -= delta;
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const float av = __shfl(alpha, 4 * kb + v);
#pragma unroll
                        for (int nb = 0; nb < NBV; ++nb) oacc[t][nb][v] *= av;
                    }
                }
            }
            // (d) weights 2^(s - m) in fp16 and the value contraction
#pragma unroll
            for (int t = 0; t < NQ; ++t) {
                float pr[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) pr[k] = __builtin_amdgcn_exp2f(xv[t][k]);
                const f16x8 pa = as_h8(pack_rtz(pr[0], pr[4]), pack_rtz(pr[1], pr[5]), pack_rtz(pr[2], pr[6]),
                                       pack_rtz(pr[3], pr[7]));
#pragma unroll
                for (int nb = 0; nb < NBV; ++nb)
                    oacc[t][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, vb[nb], oacc[t][nb], 0, 0, 0);
            }
        }
    };
    // groups in pairs: copy the raw records two pairs ahead, build the
    // tiles of the next pair, compute this pair; one barrier per pair.  The
    // pair's LDS accesses go through lw and its copies through ldma, both
    // restrict-qualified (the LDS base plus an opaque zero each, distinct
    // values): the compiler then knows that the copies in flight write
    // nothing the pair reads, and the tile building no longer waits for the
    // copies issued at the pair's start (which undid the two-pair lead).
    // They land before the barrier that ends the pair (explicit wait).
    // (The helpers are captured by value; they hold the loop-carried state
    // by reference.)
    auto pair = [=](int j, unsigned char *__restrict__ lw, unsigned char *__restrict__ ldma) {
        if constexpr (pre) {
            // pre-decoded tiles of the next pair (the incomplete group built)
            if (j + 2 < ngroups) {
                if (j + 2 < nfull) copy_tile(ldma, j + 2);
                else build_tiles(lw, j + 2, j + 2);
            }
            if (j + 3 < ngroups) {
                if (j + 3 < nfull) copy_tile(ldma, j + 3);
                else build_tiles(lw, j + 3, j + 2 + nrk + nrv);
            }
        } else {
            if (j + 4 < ngroups && j + 4 < nfull) copy_raw(ldma, j + 4);
            if (j + 5 < ngroups && j + 5 < nfull) copy_raw(ldma, j + 5);
            if (j + 2 < ngroups) build_tiles(lw, j + 2, j + 2);
            if (j + 3 < ngroups) build_tiles(lw, j + 3, j + 2 + nrk + nrv);
        }
        compute_group(lw, j);
        if (j + 1 < ngroups) compute_group(lw, j + 1);
        __builtin_amdgcn_s_waitcnt(0);                // this wave's record copies have landed
        __syncthreads();                              // and every wave is done with this pair's tiles
    };
    int lz0 = 0, lz1 = 0;
    asm volatile("" : "+s"(lz0));
    asm volatile("" : "+s"(lz1));
    for (int j = 0; j < ngroups; j += 2) pair(j, lds + lz0, lds + lz1);

    // ---- normalise by the ones column (channel r_V) and park the latent
    //      outputs: row 4 kb + v of tile t, channel 16 nb + ln
    float *ol = reinterpret_cast<float *>(lds + L.olat) + wv * (16 * NQ) * (16 * NBV);
    const int nbl = rv >> 4, lnl = rv & 15;
#pragma unroll
    for (int t = 0; t < NQ; ++t) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            float lq = 0.0f;
#pragma unroll
            for (int nb = 0; nb < NBV; ++nb) lq = nb == nbl ? oacc[t][nb][v] : lq;
            lq = __shfl(lq, 16 * kb + lnl);
            const float inv = 1.0f / lq;
#pragma unroll
            for (int nb = 0; nb < NBV; ++nb) ol[(16 * t + 4 * kb + v) * (16 * NBV) + 16 * nb + ln] = oacc[t][nb][v] * inv;
        }
    }
    // channel-major value basis [r_V][D] and mean into the (now idle)
    //      record/tile area, 16 bytes per thread and step
    float *bl = reinterpret_cast<float *>(lds + L.basis);
    float *ml = bl + kHeadDim * rv;
    {
        const float4 *bv = reinterpret_cast<const float4 *>(a.v.basis_cm + rw.slot * a.v.set_bcm +
                                                            static_cast<int64_t>(grp) * rv * kHeadDim);
        for (int e = tid; e < kHeadDim * rv / 4; e += kPfThreads) reinterpret_cast<float4 *>(bl)[e] = bv[e];
        if (tid < kHeadDim) ml[tid] = a.v.mu[rw.slot * a.v.set_mu + grp * kHeadDim + tid];
    }
    __syncthreads();

    // ---- output projection o = V_V o_lat + mu_V (fp32 fma chain in channel
    //      order), two adjacent outputs per lane (8 consecutive bytes of a
    //      basis row: conflict-free LDS reads), one column at a time
    const int d0 = 2 * lane;
    for (int col = 0; col < 16 * NQ; ++col) {
        const int c = c_lo + col, pl = c / g, hd = c - pl * g, qi = q0 + pl;
        if (pl >= a.qp || qi >= nq) continue;       // wave-uniform
        const float *o = ol + col * (16 * NBV);
        float acc0 = ml[d0], acc1 = ml[d0 + 1];
        for (int cc = 0; cc < rv; ++cc) {
            const float oc = o[cc];
            const float2 b = *reinterpret_cast<const float2 *>(bl + cc * kHeadDim + d0);
            acc0 = fmaf(b.x, oc, acc0);
            acc1 = fmaf(b.y, oc, acc1);
        }
        uint16_t *dst = a.out + ((ci * a.Hq + h * g + hd) * a.T_stride + qi) * kHeadDim;
        reinterpret_cast<uint32_t *>(dst)[lane] = out_bits(acc0, a.bf16) | (out_bits(acc1, a.bf16) << 16);
    }
}

template <int KS, int NBV, bool GEN>
hipError_t launch_prefill_tiles_tg(const PrefillArgs &a, int max_nfull, hipStream_t s) {
    hipLaunchKernelGGL((prefill_tiles_kernel<KS, NBV, GEN>), dim3((max_nfull + 3) / 4, a.Hkv, a.B), dim3(256), 0, s,
                       a);
    return hipGetLastError();
}

template <int KS, int NBV, bool GEN, bool PRE>
hipError_t launch_prefill_tgp(const PrefillArgs &a, size_t lds_bytes, hipStream_t s) {
    constexpr int NQ = prefill_nq_c(KS, NBV);
    // set once per process (thread-safe static initialisation)
    static const hipError_t attr =
        hipFuncSetAttribute(reinterpret_cast<const void *>(&prefill_kernel<KS, NBV, NQ, GEN, PRE>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((prefill_kernel<KS, NBV, NQ, GEN, PRE>), dim3(a.Hkv, a.tiles_max, a.B), dim3(kPfThreads),
                       lds_bytes, s, a);
    return hipGetLastError();
}

template <int KS, int NBV, bool GEN>
hipError_t launch_prefill_tg(const PrefillArgs &a, size_t lds_bytes, hipStream_t s) {
    return a.ws_tiles ? launch_prefill_tgp<KS, NBV, GEN, true>(a, lds_bytes, s)
                      : launch_prefill_tgp<KS, NBV, GEN, false>(a, lds_bytes, s);
}

// A PALU-shaped coder: one 4-bit or 2-bit segment, or 4-bit then 2-bit.
bool palu_shaped_pf(const Coder &cd) {
    if (cd.nseg == 1) return cd.bits[0] == 4 || cd.bits[0] == 2;
    return cd.nseg == 2 && cd.bits[0] == 4 && cd.bits[1] == 2;
}

template <int KS, int NBV>
hipError_t launch_prefill_t(const PrefillArgs &a, size_t lds_bytes, hipStream_t s) {
    const bool gen = !palu_shaped_pf(a.k.cd) || (!a.v.fp16_latents && !palu_shaped_pf(a.v.cd));
    return gen ? launch_prefill_tg<KS, NBV, true>(a, lds_bytes, s) : launch_prefill_tg<KS, NBV, false>(a, lds_bytes, s);
}

template <int KS, int NBV>
hipError_t launch_prefill_tiles_t(const PrefillArgs &a, int max_nfull, hipStream_t s) {
    const bool gen = !palu_shaped_pf(a.k.cd) || (!a.v.fp16_latents && !palu_shaped_pf(a.v.cd));
    return gen ? launch_prefill_tiles_tg<KS, NBV, true>(a, max_nfull, s)
               : launch_prefill_tiles_tg<KS, NBV, false>(a, max_nfull, s);
}

template <int KS>
hipError_t launch_prefill_tiles_v(const PrefillArgs &a, int max_nfull, hipStream_t s) {
    switch (prefill_nbv(a.v.r)) {
        case 1: return launch_prefill_tiles_t<KS, 1>(a, max_nfull, s);
        case 2: return launch_prefill_tiles_t<KS, 2>(a, max_nfull, s);
        case 3: return launch_prefill_tiles_t<KS, 3>(a, max_nfull, s);
        case 5: return launch_prefill_tiles_t<KS, 5>(a, max_nfull, s);
        case 9: return launch_prefill_tiles_t<KS, 9>(a, max_nfull, s);
        default: return hipErrorInvalidValue;
    }
}

template <int KS>
hipError_t launch_prefill_v(const PrefillArgs &a, size_t lds_bytes, hipStream_t s) {
    switch (prefill_nbv(a.v.r)) {
        case 1: return launch_prefill_t<KS, 1>(a, lds_bytes, s);
        case 2: return launch_prefill_t<KS, 2>(a, lds_bytes, s);
        case 3: return launch_prefill_t<KS, 3>(a, lds_bytes, s);
        case 5: return launch_prefill_t<KS, 5>(a, lds_bytes, s);
        case 9: return launch_prefill_t<KS, 9>(a, lds_bytes, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int prefill_ks(int nbk) {
    const int np = 8 * nbk;
    const int ks = (np + 31) / 32;
    return ks <= 1 ? 1 : (ks <= 2 ? 2 : 4);
}

int prefill_nbv(int r_v) {
    const int n = (r_v + 1 + 15) / 16;
    return n <= 1 ? 1 : n <= 2 ? 2 : n <= 3 ? 3 : n <= 5 ? 5 : 9;
}

int prefill_nq(int ks, int nbv) { return prefill_nq_c(ks, nbv); }

size_t prefill_lds_bytes(int nbk, int r_k, int r_v, int words_k, int words_v) {
    (void)r_k;
    const int ks = prefill_ks(nbk), nbv = prefill_nbv(r_v);
    return static_cast<size_t>(prefill_lds(ks, nbv, prefill_nq(ks, nbv), words_k, words_v, r_v, nbk).total);
}

size_t prefill_tile_bytes(int nbk, int r_v) {
    const int ks = prefill_ks(nbk), nbv = prefill_nbv(r_v);
    return static_cast<size_t>(32 * pf_krow(ks) * 2 + 16 * nbv * kVRow * 2);
}

hipError_t launch_prefill_tiles(const PrefillArgs &a, int max_nfull, hipStream_t s) {
    if (max_nfull <= 0) return hipSuccess;
    switch (prefill_ks(coder_blocks(a.k.cd))) {
        case 1: return launch_prefill_tiles_v<1>(a, max_nfull, s);
        case 2: return launch_prefill_tiles_v<2>(a, max_nfull, s);
        case 4: return launch_prefill_tiles_v<4>(a, max_nfull, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_prefill(const PrefillArgs &a, size_t lds_bytes, hipStream_t s) {
    switch (prefill_ks(coder_blocks(a.k.cd))) {
        case 1: return launch_prefill_v<1>(a, lds_bytes, s);
        case 2: return launch_prefill_v<2>(a, lds_bytes, s);
        case 4: return launch_prefill_v<4>(a, lds_bytes, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace palu
