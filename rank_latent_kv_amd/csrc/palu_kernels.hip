// HIP kernels of the latent KV cache for gfx950 (MI355X).
//
//   gram_kernel / gram_reduce_kernel : per (tensor, head group) Gram matrix
//       X^T X and column sums X^T 1 of the stacked fp16 rows (the fit's data
//       pass; PALU page, "How it works", prefill steps 1-2).  fp16 products
//       are exact, tiles accumulate in fp32 on MFMA, tiles are summed in fp64.
//   encode_kernel : projection L = (x - mu_g) V_g as a fixed-order fp32 fma
//       chain, min/max quantisation of complete 32-token groups, bit packing,
//       fp32 tail of the incomplete group (prefill steps 4-6, decode steps
//       1-2).
//   attend_kernel / combine_kernel : single-query decode attention computed
//       from the stored latents (decode step 3) with the query absorbed into
//       the key basis, split over token ranges, then merged by log-sum-exp
//       and projected back with the value basis.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "palu_internal.h"

namespace palu {

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float h2f(uint32_t bits) {
    return __half2float(__ushort_as_half(static_cast<unsigned short>(bits & 0xffffu)));
}

__device__ __forceinline__ uint32_t f2h_bits(float f) {
    return static_cast<uint32_t>(__half_as_ushort(__float2half_rn(f)));
}

__device__ __forceinline__ float wave_max(float v) {
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// ---------------------------------------------------------------- Gram ----
//
// Workgroup (block, group g, tensor) owns rows [block*rpb, (block+1)*rpb) of
// the group's stacked rows.  Row index -> (sequence b, head in group, token)
// through the prefix over (b, head) segments.  64-row tiles are staged in
// LDS; wave w accumulates the 32-row band I = w of the 128 x 128 Gram matrix
// (four 32x32 MFMA tiles) plus the column sums of feature block w (an MFMA
// with an all-ones A operand).

constexpr int kGramTile = 64;
constexpr int kGramPad = 136;   // LDS row stride in halves

__global__ __launch_bounds__(256) void gram_kernel(GramArgs a) {
    const int blk = blockIdx.x, g = blockIdx.y, tz = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t row0 = static_cast<int64_t>(blk) * a.rows_per_block;
    const int64_t row1 = row0 + a.rows_per_block < a.n_rows ? row0 + a.rows_per_block : a.n_rows;
    const uint16_t *x = a.x[tz];
    const int nseg = a.B * a.hpg;

    __shared__ _Float16 tile[kGramTile][kGramPad];

    f32x16 acc0 = {}, acc1 = {}, acc2 = {}, acc3 = {}, accs = {};
    f16x8 ones;
    for (int u = 0; u < 8; ++u) ones[u] = static_cast<_Float16>(1.0f);

    for (int64_t base = row0; base < row1; base += kGramTile) {
        for (int k = 0; k < 4; ++k) {
            const int id = tid + 256 * k;
            const int rr = id >> 4, fc = id & 15;
            const int64_t row = base + rr;
            uint4 val = make_uint4(0u, 0u, 0u, 0u);
            if (row < row1) {
                int lo = 0, hi = nseg - 1;
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (a.seg_pref[mid] <= row) lo = mid; else hi = mid - 1;
                }
                const int b = lo / a.hpg, hh = lo - b * a.hpg;
                const int64_t t = row - a.seg_pref[lo];
                const uint16_t *src =
                    x + ((static_cast<int64_t>(b) * a.H + g * a.hpg + hh) * a.S_stride + t) * kHeadDim +
                    fc * 8;
                val = *reinterpret_cast<const uint4 *>(src);
            }
            *reinterpret_cast<uint4 *>(&tile[rr][fc * 8]) = val;
        }
        __syncthreads();
        for (int ks = 0; ks < kGramTile / 16; ++ks) {
            const int rb = ks * 16 + (lane >> 5) * 8;
            const int f = lane & 31;
            f16x8 o0, o1, o2, o3;
            for (int u = 0; u < 8; ++u) {
                o0[u] = tile[rb + u][f];
                o1[u] = tile[rb + u][32 + f];
                o2[u] = tile[rb + u][64 + f];
                o3[u] = tile[rb + u][96 + f];
            }
            const f16x8 oa = w == 0 ? o0 : w == 1 ? o1 : w == 2 ? o2 : o3;
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(oa, o0, acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(oa, o1, acc1, 0, 0, 0);
            acc2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(oa, o2, acc2, 0, 0, 0);
            acc3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(oa, o3, acc3, 0, 0, 0);
            accs = __builtin_amdgcn_mfma_f32_32x32x16_f16(ones, oa, accs, 0, 0, 0);
        }
        __syncthreads();
    }

    constexpr int kElems = kHeadDim * kHeadDim + kHeadDim;
    float *out = a.partial + ((static_cast<int64_t>(tz) * a.G + g) * a.nb + blk) * kElems;
    const int j = lane & 31;
    for (int v = 0; v < 16; ++v) {
        // 32x32 accumulator layout: column = lane % 32,
        // row = 8 * (v / 4) + 4 * (lane / 32) + v % 4
        const int i = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        float *orow = out + (32 * w + i) * kHeadDim;
        orow[j] = acc0[v];
        orow[32 + j] = acc1[v];
        orow[64 + j] = acc2[v];
        orow[96 + j] = acc3[v];
    }
    if (lane < 32) out[kHeadDim * kHeadDim + 32 * w + lane] = accs[0];
}

__global__ __launch_bounds__(256) void gram_reduce_kernel(GramReduceArgs a) {
    constexpr int kElems = kHeadDim * kHeadDim + kHeadDim;
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= kElems) return;
    const int g = blockIdx.y, tz = blockIdx.z;
    const float *p = a.partial + (static_cast<int64_t>(tz) * a.G + g) * a.nb * kElems + e;
    double s = 0.0;
    for (int b = 0; b < a.nb; ++b) s += static_cast<double>(p[static_cast<int64_t>(b) * kElems]);
    a.out[(static_cast<int64_t>(tz) * a.G + g) * kElems + e] = s;
}

// -------------------------------------------------------------- encode ----
//
// Workgroup (touched group u, call row bi * H + head h, tensor tz).  The
// group index is j = old_len / 32 + u; its new positions are
// [max(32j, old), min(32j + 32, old + n)).

__global__ __launch_bounds__(256) void encode_kernel(EncodeArgs a) {
    const int u = blockIdx.x;
    const int bi = blockIdx.y / a.H, h = blockIdx.y - (blockIdx.y / a.H) * a.H;
    const int tz = blockIdx.z;
    const int o = a.old_len[bi], n = a.n_new[bi];
    if (n <= 0) return;
    const int j0 = o >> 5, jl = (o + n - 1) >> 5, j = j0 + u;
    if (j > jl) return;
    const TensorDev &T = tz ? a.t[1] : a.t[0];
    const int r = T.r, n_hi = T.n_hi, n_lo = T.r - T.n_hi;
    const int g = h / a.hpg, slot = a.slot[bi], tid = threadIdx.x;
    const int pb = 32 * j > o ? 32 * j : o;
    const int pe = 32 * j + 32 < o + n ? 32 * j + 32 : o + n;
    const bool complete = (o + n) >= 32 * j + 32;

    __shared__ float ys[kHeadDim][33];       // (x - mu) transposed: [d][t]
    __shared__ float vs[kHeadDim][32];       // basis columns chunk [d][c]
    __shared__ float lat[32][kHeadDim + 1];  // latents [t][c]
    __shared__ uint8_t codes[32][kHeadDim];
    __shared__ uint32_t meta[kHeadDim];

    // 1. y = float(x) - mu for the new tokens
    const uint16_t *xin = a.x[tz] + (static_cast<int64_t>(bi) * a.H + h) * a.T_stride * kHeadDim;
    const float *mu = T.mu + g * kHeadDim;
    for (int e = tid; e < 32 * 16; e += 256) {
        const int t = e >> 4, dc = e & 15;
        const int p = 32 * j + t;
        if (p >= pb && p < pe) {
            const uint4 v = *reinterpret_cast<const uint4 *>(xin + static_cast<int64_t>(p - o) * kHeadDim + dc * 8);
            const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
            for (int q = 0; q < 4; ++q) {
                const int d = dc * 8 + 2 * q;
                ys[d][t] = h2f(wv[q]) - mu[d];
                ys[d + 1][t] = h2f(wv[q] >> 16) - mu[d + 1];
            }
        }
    }

    // 2. latents: acc = fma(y_d, V[d][c], acc) for d = 0..D-1, in order
    const float *basis = T.basis + static_cast<int64_t>(g) * kHeadDim * r;
    for (int c0 = 0; c0 < r; c0 += 32) {
        const int nc = r - c0 < 32 ? r - c0 : 32;
        __syncthreads();
        for (int e = tid; e < kHeadDim * 32; e += 256) {
            const int d = e >> 5, c = e & 31;
            vs[d][c] = c < nc ? basis[d * r + c0 + c] : 0.0f;
        }
        __syncthreads();
        const int t = tid & 31, cq = tid >> 5;
        const int p = 32 * j + t;
        if (p >= pb && p < pe && 4 * cq < nc) {
            float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
            for (int d = 0; d < kHeadDim; ++d) {
                const float y = ys[d][t];
                const float4 v = *reinterpret_cast<const float4 *>(&vs[d][4 * cq]);
                a0 = __builtin_fmaf(y, v.x, a0);
                a1 = __builtin_fmaf(y, v.y, a1);
                a2 = __builtin_fmaf(y, v.z, a2);
                a3 = __builtin_fmaf(y, v.w, a3);
            }
            const int c = c0 + 4 * cq;
            lat[t][c] = a0;
            if (4 * cq + 1 < nc) lat[t][c + 1] = a1;
            if (4 * cq + 2 < nc) lat[t][c + 2] = a2;
            if (4 * cq + 3 < nc) lat[t][c + 3] = a3;
        }
    }
    __syncthreads();

    const int64_t head_base = (static_cast<int64_t>(slot) * a.H + h);
    if (T.fp16_latents) {
        uint16_t *rec16 = reinterpret_cast<uint16_t *>(T.records + head_base * T.head_stride +
                                                       static_cast<int64_t>(j) * T.words);
        for (int e = tid; e < 32 * r; e += 256) {
            const int c = e >> 5, t = e & 31;
            const int p = 32 * j + t;
            if (p >= pb && p < pe) rec16[c * 32 + t] = static_cast<uint16_t>(f2h_bits(lat[t][c]));
        }
        return;
    }
    if (!complete) {
        float *tl = T.tail + (head_base * 2 + a.sel_new[bi]) * 32 * r;
        for (int e = tid; e < 32 * r; e += 256) {
            const int t = e / r, c = e - (e / r) * r;
            const int p = 32 * j + t;
            if (p >= pb && p < pe) tl[t * r + c] = lat[t][c];
        }
        return;
    }
    // 3. the group is complete: older latents of the group come from the tail
    if (j == j0 && (o & 31)) {
        const float *tl = T.tail + (head_base * 2 + a.sel_old[bi]) * 32 * r;
        const int nold = o & 31;
        for (int e = tid; e < nold * r; e += 256) {
            const int t = e / r, c = e - (e / r) * r;
            lat[t][c] = tl[t * r + c];
        }
    }
    __syncthreads();
    // 4. min/max quantiser per channel
    for (int c = tid; c < r; c += 256) {
        const int bits = c < n_hi ? a.hi_bit : a.lo_bit;
        const float levels = static_cast<float>((1 << bits) - 1);
        float mn = lat[0][c], mx = lat[0][c];
        for (int t = 1; t < 32; ++t) {
            const float v = lat[t][c];
            mn = v < mn ? v : mn;
            mx = v > mx ? v : mx;
        }
        const float scale = (mx - mn) / levels;
        for (int t = 0; t < 32; ++t) {
            int q = 0;
            if (scale > 0.0f) {
                float uq = rintf((lat[t][c] - mn) / scale);
                uq = uq < 0.0f ? 0.0f : (uq > levels ? levels : uq);
                q = static_cast<int>(uq);
            }
            codes[t][c] = static_cast<uint8_t>(q);
        }
        meta[c] = f2h_bits(scale) | (f2h_bits(mn) << 16);
    }
    __syncthreads();
    // 5. pack: each thread assembles whole words
    uint32_t *rec = T.records + head_base * T.head_stride + static_cast<int64_t>(j) * T.words;
    for (int wd = tid; wd < T.words; wd += 256) {
        uint32_t word = 0;
        if (wd < 4 * n_hi) {
            for (int m = 0; m < 8; ++m) {
                const int pos = 32 * wd + 4 * m;
                int t, c;
                if (tz == 0) { t = pos / (4 * n_hi); c = (pos - t * 4 * n_hi) >> 2; }
                else { c = pos >> 7; t = (pos & 127) >> 2; }
                word |= static_cast<uint32_t>(codes[t][c]) << (4 * m);
            }
        } else if (wd < 4 * n_hi + 2 * n_lo) {
            const int wl = wd - 4 * n_hi;
            for (int m = 0; m < 16; ++m) {
                const int pos = 32 * wl + 2 * m;
                int t, c;
                if (tz == 0) { t = pos / (2 * n_lo); c = n_hi + ((pos - t * 2 * n_lo) >> 1); }
                else { c = n_hi + (pos >> 6); t = (pos & 63) >> 1; }
                word |= static_cast<uint32_t>(codes[t][c]) << (2 * m);
            }
        } else {
            word = meta[wd - 4 * n_hi - 2 * n_lo];
        }
        rec[wd] = word;
    }
}

// -------------------------------------------------------------- attend ----
//
// Workgroup = (call row i, kv head h, split s).  Split s covers complete
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
constexpr int kBtabMaxU = 16;   // score B-operand table kept in LDS up to this many MFMA k-steps

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));

// LDS layout of one attend workgroup (byte offsets).  Shared by the kernel
// and the host, which sizes the dynamic LDS from it.
struct AttendLds {
    int qt, qt16, ts, mst, lst, ost, tp, hm, btab, kpair, vpair, stage, total;
    int nbk, nub;
    bool use_btab;
};

__host__ __device__ inline int lds_take(int &o, int bytes) {
    const int r = o;
    o += (bytes + 15) & ~15;
    return r;
}

__host__ __device__ inline AttendLds attend_lds(int g, int rk, int nhk, int rv, int chunk, int wk, int wv, bool vq) {
    AttendLds L;
    const int S = 16 / g;
    L.nbk = (nhk + 7) / 8 + (rk - nhk + 7) / 8;
    L.nub = (S * L.nbk + 3) / 4;
    L.use_btab = L.nub <= kBtabMaxU;
    int o = 0;
    L.qt = lds_take(o, g * kHeadDim * 4);
    L.qt16 = lds_take(o, g * 16 * 16);
    L.ts = lds_take(o, g * (kWaves * 16 + 1) * 4);
    L.mst = lds_take(o, (kWaves + 1) * 16 * 4);
    L.lst = lds_take(o, (kWaves + 1) * 16 * 4);
    L.ost = lds_take(o, (kWaves + 1) * 16 * rv * 4);
    L.tp = lds_take(o, g * 32 * 4);
    L.hm = lds_take(o, kMaxGqa * 4);
    L.btab = lds_take(o, L.use_btab ? L.nub * 64 * 16 : 0);
    L.kpair = lds_take(o, chunk * L.nbk * 8 * 4);
    L.vpair = lds_take(o, vq ? chunk * rv * 2 * 4 : 0);
    L.stage = lds_take(o, (chunk * (wk + (vq ? wv : 0)) + 16) * 4);
    L.total = o;
    return L;
}

__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// (code * scale + zero) for a pair of magic halves 1024 + code, in fp16
__device__ __forceinline__ uint32_t dequant_pair(uint32_t magic, uint32_t spair, uint32_t zpair) {
    const h2 code = __builtin_bit_cast(h2, magic) - (h2){(_Float16)1024.0f, (_Float16)1024.0f};
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(code, __builtin_bit_cast(h2, spair),
                                                                   __builtin_bit_cast(h2, zpair)));
}

__device__ __forceinline__ uint32_t pack_half2(float a, float b) {
    const h2 v = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
    return __builtin_bit_cast(uint32_t, v);
}

// fp16 pair, round toward zero (one instruction); used for softmax weights
__device__ __forceinline__ uint32_t pack_rtz(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}

// A 32-bit constant held in a VGPR, so that three-operand ALU forms
// (v_and_or_b32) can take it without a literal encoding.
__device__ __forceinline__ uint32_t vgpr_const(uint32_t v) {
    uint32_t r;
    asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "i"(v));
    return r;
}

__device__ __forceinline__ f16x8 as_h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    const u4v t = {a, b, c, d};
    return __builtin_bit_cast(f16x8, t);
}

// 8 codes of one token from a 32-bit window (channel k at bit w*k) ->
// dequantised fp16 pairs (channel k, channel k + 4), k = 0..3.
template <bool W4>
__device__ __forceinline__ f16x8 dequant8(uint32_t X, const uint4 &sp, const uint4 &zp, uint32_t cm,
                                          uint32_t magic) {
    // 2-bit codes: move codes 4..7 (bits 8..15) up to bits 16..23
    const uint32_t U = W4 ? X : perm_b32(X, X, 0x0C010C00u);
    constexpr int wc = W4 ? 4 : 2;
    return as_h8(dequant_pair((U & cm) | magic, sp.x, zp.x),
                 dequant_pair(((U >> wc) & cm) | magic, sp.y, zp.y),
                 dequant_pair(((U >> (2 * wc)) & cm) | magic, sp.z, zp.z),
                 dequant_pair(((U >> (3 * wc)) & cm) | magic, sp.w, zp.w));
}

__device__ __forceinline__ f16x8 dequant8_any(uint32_t X, bool w4, const uint4 &sp, const uint4 &zp) {
    const uint32_t U = w4 ? X : perm_b32(X, X, 0x0C010C00u);
    const int wc = w4 ? 4 : 2;
    const uint32_t cm = w4 ? 0x000F000Fu : 0x00030003u;
    return as_h8(dequant_pair((U & cm) | 0x64006400u, sp.x, zp.x),
                 dequant_pair(((U >> wc) & cm) | 0x64006400u, sp.y, zp.y),
                 dequant_pair(((U >> (2 * wc)) & cm) | 0x64006400u, sp.z, zp.z),
                 dequant_pair(((U >> (3 * wc)) & cm) | 0x64006400u, sp.w, zp.w));
}

// Workgroup = (call row i, kv head h, split s); see the section comment.
// S = 16 / gqa token groups (slots) per wave iteration, NBV = value-channel
// blocks of 16.
template <int S, int NBV>
__global__ __launch_bounds__(256) void attend_kernel(AttendArgs a) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int ln = lane & 15, kb = lane >> 4;

    // ---- work item
    const int wid = blockIdx.x;
    int i = 0;
    while (i + 1 < a.B && a.work_prefix[i + 1] <= wid) ++i;
    const int rem = wid - a.work_prefix[i];
    const int ns = a.nsplit[i];
    const int h = rem / ns, s = rem - (rem / ns) * ns;
    const int slot = a.slot[i], len = a.len[i];
    const int nfull = len >> 5, ntail = len & 31;
    const int jb = s * a.chunk;
    const int je = jb + a.chunk < nfull ? jb + a.chunk : nfull;
    const int ntg = je > jb ? je - jb : 0;
    const bool do_tail = (s == ns - 1) && ntail > 0;
    const int g = a.gqa, grp = h / a.hpg;
    const int NS = S * g;
    const int rk = a.k.r, nhk = a.k.n_hi, nlk = rk - nhk;
    const int nbh = (nhk + 7) >> 3;
    const int rv = a.v.r, nhv = a.v.n_hi;
    const int WK = a.k.words, WV = a.v.words;
    const bool vq = !a.v.fp16_latents;
    const int kmeta = 4 * nhk + 2 * nlk, vmeta = 4 * nhv + 2 * (rv - nhv);

    const AttendLds L = attend_lds(g, rk, nhk, rv, a.chunk, WK, WV, vq);
    const int nbk = L.nbk, nub = L.nub, npair = S * nbk;
    float *qt = reinterpret_cast<float *>(lds + L.qt);
    uint4 *qt16 = reinterpret_cast<uint4 *>(lds + L.qt16);
    _Float16 *qt16h = reinterpret_cast<_Float16 *>(lds + L.qt16);
    float *ts = reinterpret_cast<float *>(lds + L.ts);
    float *mst = reinterpret_cast<float *>(lds + L.mst);
    float *lst = reinterpret_cast<float *>(lds + L.lst);
    float *ost = reinterpret_cast<float *>(lds + L.ost);
    float *tp = reinterpret_cast<float *>(lds + L.tp);
    float *hm = reinterpret_cast<float *>(lds + L.hm);
    uint4 *btab = reinterpret_cast<uint4 *>(lds + L.btab);
    uint32_t *kpair = reinterpret_cast<uint32_t *>(lds + L.kpair);
    uint32_t *vpair = reinterpret_cast<uint32_t *>(lds + L.vpair);
    uint32_t *stage = reinterpret_cast<uint32_t *>(lds + L.stage);

    const int64_t hb = static_cast<int64_t>(slot) * a.Hkv + h;
    const uint32_t *kg = a.k.records + hb * a.k.head_stride;
    const uint32_t *vg = a.v.records + hb * a.v.head_stride;

    // ---- 1. stage the split's packed records in LDS (16-byte loads, all
    //         issued before the first store)
    const int64_t k_a = (static_cast<int64_t>(jb) * WK) & ~3LL;
    const int k_words = ntg ? static_cast<int>((static_cast<int64_t>(je) * WK - k_a + 3) & ~3LL) : 0;
    const int64_t v_a = (static_cast<int64_t>(jb) * WV) & ~3LL;
    const int v_words = (vq && ntg) ? static_cast<int>((static_cast<int64_t>(je) * WV - v_a + 3) & ~3LL) : 0;
    const int koff = static_cast<int>(static_cast<int64_t>(jb) * WK - k_a);          // record 0 of the split
    const int voff = k_words + static_cast<int>(static_cast<int64_t>(jb) * WV - v_a);
    {
        const int nk4 = k_words >> 2, nv4 = v_words >> 2, n4 = nk4 + nv4;
        const uint4 *ksrc = reinterpret_cast<const uint4 *>(kg + k_a);
        const uint4 *vsrc = reinterpret_cast<const uint4 *>(vg + v_a);
        uint4 *dst = reinterpret_cast<uint4 *>(stage);
        for (int base = 0; base < n4; base += 256 * 8) {
            uint4 buf[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int e = base + u * 256 + tid;
                const uint4 *src = e < nk4 ? ksrc + e : vsrc + (e - nk4);
                buf[u] = make_uint4(0u, 0u, 0u, 0u);
                if (e < n4) buf[u] = *src;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int e = base + u * 256 + tid;
                if (e < n4) dst[e] = buf[u];
            }
        }
    }

    // ---- 2. absorbed query qt = qs V_K^T q on MFMA: rows = query heads of
    //         this kv head, K = d, columns = 16-channel blocks of the fp16
    //         channel-major key basis (wave w takes blocks w, w + 4, ...)
    {
        const int nbc = (rk + 15) >> 4;
        const int qrow = i * a.Hq + h * g;
        const bool qv = ln < g;
        const uint16_t *qsrc = a.q + static_cast<int64_t>(qrow + (qv ? ln : 0)) * kHeadDim + 8 * kb;
        uint4 qa[4];
#pragma unroll
        for (int st = 0; st < 4; ++st)
            qa[st] = qv ? *reinterpret_cast<const uint4 *>(qsrc + 32 * st) : make_uint4(0u, 0u, 0u, 0u);
        const uint16_t *bt = a.k.basis_t16 + static_cast<int64_t>(grp) * rk * kHeadDim;
        for (int cb = wv; cb < nbc; cb += kWaves) {
            const int c = 16 * cb + ln;
            const bool cvq = c < rk;
            uint4 bb[4];
#pragma unroll
            for (int st = 0; st < 4; ++st)
                bb[st] = cvq ? *reinterpret_cast<const uint4 *>(bt + static_cast<int64_t>(c) * kHeadDim + 32 * st + 8 * kb)
                             : make_uint4(0u, 0u, 0u, 0u);
            f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int st = 0; st < 4; ++st)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h8(qa[st].x, qa[st].y, qa[st].z, qa[st].w),
                                                            as_h8(bb[st].x, bb[st].y, bb[st].z, bb[st].w), acc, 0, 0, 0);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int hh = 4 * kb + v;
                if (hh < g && cvq) qt[hh * rk + c] = acc[v] * a.qscale;
            }
        }
    }
    __syncthreads();

    // ---- 3. per-split tables
    // (a) qt in fp16 per (head, channel block), channel order [c0,c4,c1,c5,..]
    for (int e = tid; e < g * nbk * 8; e += 256) {
        const int hh = e / (nbk * 8), r2 = e - hh * nbk * 8;
        const int q = r2 >> 3, idx = r2 & 7;
        const int kk = (idx >> 1) + 4 * (idx & 1);
        const int chan0 = q < nbh ? 8 * q : nhk + 8 * (q - nbh);
        const int chanend = q < nbh ? nhk : rk;
        const int c = chan0 + kk;
        qt16h[(hh * nbk + q) * 8 + idx] = c < chanend ? static_cast<_Float16>(qt[hh * rk + c])
                                                      : static_cast<_Float16>(0.0f);
    }
    // (b) K scale/zero pairs per (group, channel block): words 0..3 scale
    //     pairs (k, k + 4), words 4..7 zero pairs; padding channels are 0
    for (int e = tid; e < ntg * nbk * 4; e += 256) {
        const int tg = e / (nbk * 4), r2 = e - tg * nbk * 4;
        const int q = r2 >> 2, k = r2 & 3;
        const int chan0 = q < nbh ? 8 * q : nhk + 8 * (q - nbh);
        const int chanend = q < nbh ? nhk : rk;
        const uint32_t *rec = stage + koff + tg * WK + kmeta;
        const uint32_t wa = chan0 + k < chanend ? rec[chan0 + k] : 0u;
        const uint32_t wb = chan0 + k + 4 < chanend ? rec[chan0 + k + 4] : 0u;
        uint32_t *dst = kpair + (tg * nbk + q) * 8;
        dst[k] = perm_b32(wb, wa, 0x05040100u);
        dst[4 + k] = perm_b32(wb, wa, 0x07060302u);
    }
    // (c) V per (group, channel): fp32 scale and zero - 1024 * scale, for
    //     the value epilogue (the value MFMA runs on 1024 + code)
    float *vsz = reinterpret_cast<float *>(vpair);
    if (vq) {
        for (int e = tid; e < ntg * rv; e += 256) {
            const int tg = e / rv, c = e - (e / rv) * rv;
            const uint32_t mw = stage[voff + tg * WV + vmeta + c];
            const float sc = h2f(mw), zr = h2f(mw >> 16);
            vsz[2 * e] = sc;
            vsz[2 * e + 1] = fmaf(-1024.0f, sc, zr);
        }
    }
    __syncthreads();
    // (d) block-diagonal score B operand per k-step u and lane
    if (L.use_btab) {
        for (int e = tid; e < nub * 64; e += 256) {
            const int u = e >> 6, l2 = e & 63, n2 = l2 & 15;
            const int p = 4 * u + (l2 >> 4);
            const int q = p / S, j = p - (p / S) * S;
            const bool ok = p < npair && n2 < NS && j == n2 / g;
            btab[e] = ok ? qt16[(n2 - (n2 / g) * g) * nbk + q] : make_uint4(0u, 0u, 0u, 0u);
        }
        __syncthreads();
    }

    // ---- 4. main loop over token groups
    const int slot_n = ln / g, head_n = ln - (ln / g) * g;
    const bool live_n = ln < NS;
    float m_run = -INFINITY, l_run = 0.0f;
    f4 oacc[NBV];
#pragma unroll
    for (int nb = 0; nb < NBV; ++nb) oacc[nb] = (f4){0.0f, 0.0f, 0.0f, 0.0f};
    // per-lane value-channel addressing (column c = 16 nb + ln, clamped)
    int vch[NBV], vw0[NBV], vw1[NBV], vs0[NBV], vwid[NBV], vwc[NBV];
    uint32_t vcm[NBV], vbase[NBV];
    const bool ones_col = vq && (rv & 15) != 0;     // column 15 of the last block is free
    int row_slot[4];                                 // slot of value-output row 4*kb + v
#pragma unroll
    for (int v = 0; v < 4; ++v) row_slot[v] = (4 * kb + v) / g;
#pragma unroll
    for (int nb = 0; nb < NBV; ++nb) {
        int c = 16 * nb + ln;
        c = c < rv ? c : rv - 1;
        const bool w4c = c < nhv;
        const int wc = w4c ? 4 : 2;
        const int bitbase = w4c ? 128 * c : 128 * nhv + 64 * (c - nhv);
        const int b0 = bitbase + 4 * kb * wc, b1 = b0 + 16 * wc;
        vch[nb] = c;
        vw0[nb] = b0 >> 5;
        vw1[nb] = b1 >> 5;
        vs0[nb] = b0 & 31;          // b1 - b0 = 16 wc is a multiple of 32 bits
        vwid[nb] = 4 * wc;
        vwc[nb] = wc;
        const bool one = ones_col && nb == NBV - 1 && ln == 15;
        vcm[nb] = one ? 0u : (w4c ? 0x000F000Fu : 0x00030003u);
        vbase[nb] = one ? 0x3C003C00u : 0x64006400u;
    }
    const uint32_t kmagic = vgpr_const(0x64006400u), km4 = vgpr_const(0x000F000Fu),
                   km2 = vgpr_const(0x00030003u);
    constexpr int per_iter = kWaves * S;
    const int n_iter = (ntg + per_iter - 1) / per_iter;
    for (int it = 0; it < n_iter; ++it) {
        const int tb0 = (it * kWaves + wv) * S;      // split-relative group of slot 0
        f4 sacc0 = {0.0f, 0.0f, 0.0f, 0.0f}, sacc1 = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int u = 0; u < nub; ++u) {
            const int p = 4 * u + kb;
            int q, j;
            if constexpr (S % 4 == 0) {
                q = (4 * u) / S;            // the same for every lane of the wave
                j = p - q * S;
            } else {
                q = p / S;
                j = p - q * S;
            }
            // invalid pairs and groups past the split are read from a valid
            // (clamped) record; their scores belong to masked streams
            int tg = tb0 + j;
            tg = tg < ntg ? tg : ntg - 1;
            const int qc = q < nbk ? q : nbk - 1;
            const uint32_t *rec = stage + koff + tg * WK;
            const uint4 *kp = reinterpret_cast<const uint4 *>(kpair + (tg * nbk + qc) * 8);
            const uint4 sp = kp[0], zp = kp[1];
            uint4 bq;
            if (L.use_btab) {
                bq = btab[u * 64 + lane];
            } else {
                const bool ok = p < npair && live_n && j == slot_n;
                bq = ok ? qt16[head_n * nbk + qc] : make_uint4(0u, 0u, 0u, 0u);
            }
            const f16x8 bop = as_h8(bq.x, bq.y, bq.z, bq.w);
            const bool w4 = qc < nbh;
            const int base = w4 ? 32 * qc : 128 * nhk + 16 * (qc - nbh);
            const int stride = w4 ? 4 * nhk : 2 * nlk;
            const int bit0 = base + ln * stride, bit1 = bit0 + 16 * stride;
            const uint32_t X0 = __builtin_amdgcn_alignbit(rec[(bit0 >> 5) + 1], rec[bit0 >> 5], bit0 & 31);
            const uint32_t X1 = __builtin_amdgcn_alignbit(rec[(bit1 >> 5) + 1], rec[bit1 >> 5], bit1 & 31);
            f16x8 a0, a1;
            if constexpr (S % 4 == 0) {
                if (w4) {
                    a0 = dequant8<true>(X0, sp, zp, km4, kmagic);
                    a1 = dequant8<true>(X1, sp, zp, km4, kmagic);
                } else {
                    a0 = dequant8<false>(X0, sp, zp, km2, kmagic);
                    a1 = dequant8<false>(X1, sp, zp, km2, kmagic);
                }
            } else {
                a0 = dequant8_any(X0, w4, sp, zp);
                a1 = dequant8_any(X1, w4, sp, zp);
            }
            sacc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, bop, sacc0, 0, 0, 0);
            sacc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, bop, sacc1, 0, 0, 0);
        }

        // online softmax of stream ln (rows 4*kb + v of both 16-token halves)
        const bool sv = live_n && (tb0 + slot_n) < ntg;
        const float sc[8] = {sacc0[0], sacc0[1], sacc0[2], sacc0[3], sacc1[0], sacc1[1], sacc1[2], sacc1[3]};
        float mloc = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])),
                           fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
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
        // weights of streams whose group is past the split never reach a
        // value MFMA (that slot is skipped), so only the sums (l and P) are
        // masked
        const float msafe = m_run == -INFINITY ? 0.0f : m_run;
        float pr[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) pr[k] = __builtin_amdgcn_exp2f(sc[k] - msafe);
        const float psum = ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
        l_run += sv ? psum : 0.0f;
        const uint32_t pp0 = pack_rtz(pr[0], pr[4]), pp1 = pack_rtz(pr[1], pr[5]);
        const uint32_t pp2 = pack_rtz(pr[2], pr[6]), pp3 = pack_rtz(pr[3], pr[7]);

        // values: one MFMA per slot and 16-channel block on exact codes
        // (1024 + code in fp16); per-group scale and zero are applied in the
        // epilogue: sum_t p (code s + z) = s (D - 1024 P) + z P, with
        // P = sum_t p read from a constant-one column when one is free.
        f4 dacc[NBV];
#pragma unroll
        for (int nb = 0; nb < NBV; ++nb) dacc[nb] = (f4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int m = 0; m < S; ++m) {
            const int tg = tb0 + m;
            if (tg >= ntg) break;
            const bool arow = live_n && slot_n == m;
            const f16x8 aop = arow ? as_h8(pp0, pp1, pp2, pp3) : as_h8(0u, 0u, 0u, 0u);
#pragma unroll
            for (int nb = 0; nb < NBV; ++nb) {
                uint32_t bp0, bp1, bp2, bp3;
                if (vq) {
                    const uint32_t *rec = stage + voff + tg * WV;
                    const uint32_t X = __builtin_amdgcn_ubfe(rec[vw0[nb]], vs0[nb], vwid[nb]) |
                                       (__builtin_amdgcn_ubfe(rec[vw1[nb]], vs0[nb], vwid[nb]) << 16);
                    const int wc = vwc[nb];
                    bp0 = (X & vcm[nb]) | vbase[nb];
                    bp1 = ((X >> wc) & vcm[nb]) | vbase[nb];
                    bp2 = ((X >> (2 * wc)) & vcm[nb]) | vbase[nb];
                    bp3 = ((X >> (3 * wc)) & vcm[nb]) | vbase[nb];
                } else {
                    const uint16_t *r16 =
                        reinterpret_cast<const uint16_t *>(vg + static_cast<int64_t>(jb + tg) * WV) + vch[nb] * 32;
                    const uint2 lo = *reinterpret_cast<const uint2 *>(r16 + 4 * kb);
                    const uint2 hi = *reinterpret_cast<const uint2 *>(r16 + 16 + 4 * kb);
                    bp0 = perm_b32(hi.x, lo.x, 0x05040100u);
                    bp1 = perm_b32(hi.x, lo.x, 0x07060302u);
                    bp2 = perm_b32(hi.y, lo.y, 0x05040100u);
                    bp3 = perm_b32(hi.y, lo.y, 0x07060302u);
                }
                dacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, as_h8(bp0, bp1, bp2, bp3), dacc[nb], 0, 0, 0);
            }
        }
        if (vq) {
            // P per output row 4*kb + v (stream); rows of invalid groups are 0
            float Pv[4];
            if (ones_col) {
#pragma unroll
                for (int v = 0; v < 4; ++v) Pv[v] = __shfl(dacc[NBV - 1][v], (lane & 48) | 15);
            } else {
                const h2 q0 = __builtin_bit_cast(h2, pp0), q1 = __builtin_bit_cast(h2, pp1);
                const h2 q2 = __builtin_bit_cast(h2, pp2), q3 = __builtin_bit_cast(h2, pp3);
                float P = ((static_cast<float>(q0[0]) + static_cast<float>(q0[1])) +
                           (static_cast<float>(q1[0]) + static_cast<float>(q1[1]))) +
                          ((static_cast<float>(q2[0]) + static_cast<float>(q2[1])) +
                           (static_cast<float>(q3[0]) + static_cast<float>(q3[1])));
                P = sv ? P : 0.0f;        // weights of masked streams are not zeroed
                P += __shfl_xor(P, 16);
                P += __shfl_xor(P, 32);
#pragma unroll
                for (int v = 0; v < 4; ++v) Pv[v] = __shfl(P, 4 * kb + v);
            }
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                int tgr = tb0 + row_slot[v];
                tgr = tgr < ntg ? tgr : ntg - 1;
#pragma unroll
                for (int nb = 0; nb < NBV; ++nb) {
                    const float2 sz = *reinterpret_cast<const float2 *>(vsz + 2 * (tgr * rv + vch[nb]));
                    oacc[nb][v] = fmaf(sz.x, dacc[nb][v], fmaf(sz.y, Pv[v], oacc[nb][v]));
                }
            }
        } else {
#pragma unroll
            for (int nb = 0; nb < NBV; ++nb) oacc[nb] += dacc[nb];
        }
    }

    // ---- 5. per-wave stream results to LDS
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

    // ---- 6. incomplete group (fp32 latents; fp16 value latents live in
    //         the partial record), as one more stream per head
    if (do_tail) {
        const int64_t tb = (hb * 2 + a.sel[i]) * 32;
        const float *kt = a.k.tail + tb * rk;
        for (int e = tid; e < g * 32; e += 256) {
            const int hh = e >> 5, t = e & 31;
            float acc = -INFINITY;
            if (t < ntail) {
                acc = 0.0f;
                for (int c = 0; c < rk; ++c) acc = fmaf(qt[hh * rk + c], kt[t * rk + c], acc);
            }
            ts[e] = acc;
        }
        __syncthreads();
        if (tid < g) {
            float mx = -INFINITY;
            for (int t = 0; t < ntail; ++t) mx = fmaxf(mx, ts[tid * 32 + t]);
            float l = 0.0f;
            for (int t = 0; t < 32; ++t) {
                const float pv = t < ntail ? exp2f(ts[tid * 32 + t] - mx) : 0.0f;
                tp[tid * 32 + t] = pv;
                l += pv;
            }
            mst[kWaves * 16 + tid] = mx;
            lst[kWaves * 16 + tid] = l;
        }
        __syncthreads();
        for (int e = tid; e < g * rv; e += 256) {
            const int hh = e / rv, c = e - (e / rv) * rv;
            float acc = 0.0f;
            if (vq) {
                const float *vt = a.v.tail + tb * rv;
                for (int t = 0; t < ntail; ++t) acc = fmaf(tp[hh * 32 + t], vt[t * rv + c], acc);
            } else {
                const uint16_t *r16 =
                    reinterpret_cast<const uint16_t *>(vg + static_cast<int64_t>(nfull) * WV) + c * 32;
                for (int t = 0; t < ntail; ++t) acc = fmaf(tp[hh * 32 + t], h2f(r16[t]), acc);
            }
            ost[(kWaves * 16 + hh) * rv + c] = acc;
        }
    }
    __syncthreads();

    // ---- 7. merge the streams of each head; write the split's partial.
    //         Stream index sidx: waves' streams w*16 + slot*g + head, then the
    //         tail stream kWaves*16 + head.
    const int nsw = kWaves * S + (do_tail ? 1 : 0);   // streams per head
    float *wts = ts;                                   // reuse: [g][<= 4*16 + 1]
    if (tid < g) {
        float M = -INFINITY;
        for (int k = 0; k < nsw; ++k) {
            const int sidx = k < kWaves * S ? (k / S) * 16 + (k % S) * g + tid : kWaves * 16 + tid;
            M = fmaxf(M, mst[sidx]);
        }
        hm[tid] = M;
    }
    __syncthreads();
    for (int e = tid; e < g * nsw; e += 256) {
        const int hh = e / nsw, k = e - (e / nsw) * nsw;
        const int sidx = k < kWaves * S ? (k / S) * 16 + (k % S) * g + hh : kWaves * 16 + hh;
        const float ms = mst[sidx];
        wts[e] = ms == -INFINITY ? 0.0f : exp2f(ms - hm[hh]);
    }
    __syncthreads();
    for (int e = tid; e < g * (rv + 2); e += 256) {
        const int hh = e / (rv + 2), k = e - (e / (rv + 2)) * (rv + 2);
        const float *wrow = wts + hh * nsw;
        float val;
        if (k == 0) {
            val = hm[hh];
        } else {
            const int c = k - 2;
            float acc = 0.0f;
#pragma unroll 4
            for (int kk = 0; kk < nsw; ++kk) {
                const int sidx = kk < kWaves * S ? (kk / S) * 16 + (kk % S) * g + hh : kWaves * 16 + hh;
                acc = fmaf(wrow[kk], k == 1 ? lst[sidx] : ost[sidx * rv + c], acc);
            }
            val = acc;
        }
        a.partial[((static_cast<int64_t>(i) * a.Hq + h * g + hh) * kMaxSplits + s) * (rv + 2) + k] = val;
    }

}

// One wave per (call row, query head): merge the splits by log-sum-exp and
// project back with the value basis, o = V_V (o_lat / l) + mu_V, in fp16.
// Lane sp holds split sp (and sp + 64); every partial is read once, all
// loads of a wave are independent.
__global__ __launch_bounds__(256) void combine_kernel(AttendArgs a) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int task = blockIdx.x * 4 + wv;
    const bool active = task < a.B * a.Hq;
    __shared__ float ov[4][kHeadDim];
    const int i = active ? task / a.Hq : 0, qh = active ? task - (task / a.Hq) * a.Hq : 0;
    const int h = qh / a.gqa, grp = h / a.hpg, ns = a.nsplit[i], rv = a.v.r;
    const float *part = a.partial + (static_cast<int64_t>(i) * a.Hq + qh) * kMaxSplits * (rv + 2);
    const bool s0 = lane < ns, s1 = lane + 64 < ns;
    const float m0 = s0 ? part[lane * (rv + 2)] : -INFINITY;
    const float m1 = s1 ? part[(lane + 64) * (rv + 2)] : -INFINITY;
    const float l0 = s0 ? part[lane * (rv + 2) + 1] : 0.0f;
    const float l1 = s1 ? part[(lane + 64) * (rv + 2) + 1] : 0.0f;
    const float M = wave_max(fmaxf(m0, m1));
    const float w0 = s0 ? exp2f(m0 - M) : 0.0f, w1 = s1 ? exp2f(m1 - M) : 0.0f;
    const float l = wave_sum(fmaf(w0, l0, w1 * l1));
    const float inv_l = 1.0f / l;
    for (int c0 = 0; c0 < rv; c0 += 4) {
        float acc[4];
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            const int c = c0 + cc;
            float t = 0.0f;
            if (c < rv) {
                if (s0) t = w0 * part[lane * (rv + 2) + 2 + c];
                if (s1) t = fmaf(w1, part[(lane + 64) * (rv + 2) + 2 + c], t);
            }
            acc[cc] = t;
        }
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) acc[cc] = wave_sum(acc[cc]);
        if (lane < 4 && c0 + lane < rv && active)
            ov[wv][c0 + lane] = (lane == 0 ? acc[0] : lane == 1 ? acc[1] : lane == 2 ? acc[2] : acc[3]) * inv_l;
    }
    __syncthreads();
    if (!active) return;
    const float *bv = a.v.basis + static_cast<int64_t>(grp) * kHeadDim * rv;
    for (int d = lane; d < kHeadDim; d += 64) {
        float o = a.v.mu[grp * kHeadDim + d];
        for (int c = 0; c < rv; ++c) o = fmaf(bv[d * rv + c], ov[wv][c], o);
        a.out[(static_cast<int64_t>(i) * a.Hq + qh) * kHeadDim + d] = static_cast<uint16_t>(f2h_bits(o));
    }
}

__global__ __launch_bounds__(256) void basis_t16_kernel(const float *src, uint16_t *dst, int G, int r) {
    const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int64_t n = static_cast<int64_t>(G) * r * kHeadDim;
    if (e >= n) return;
    const int d = static_cast<int>(e % kHeadDim);
    const int64_t gc = e / kHeadDim;
    const int c = static_cast<int>(gc % r), g = static_cast<int>(gc / r);
    dst[e] = static_cast<uint16_t>(f2h_bits(src[(static_cast<int64_t>(g) * kHeadDim + d) * r + c]));
}

}  // namespace

hipError_t launch_gram(const GramArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(gram_kernel, dim3(a.nb, a.G, 2), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_gram_reduce(const GramReduceArgs &a, hipStream_t s) {
    constexpr int kElems = kHeadDim * kHeadDim + kHeadDim;
    hipLaunchKernelGGL(gram_reduce_kernel, dim3((kElems + 255) / 256, a.G, 2), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_encode(const EncodeArgs &a, int max_touched, hipStream_t s) {
    hipLaunchKernelGGL(encode_kernel, dim3(max_touched, a.B * a.H, 2), dim3(256), 0, s, a);
    return hipGetLastError();
}

size_t attend_lds_bytes(int gqa, int r_k, int n_hi_k, int r_v, int chunk, int words_k, int words_v, bool vq) {
    return static_cast<size_t>(attend_lds(gqa, r_k, n_hi_k, r_v, chunk, words_k, words_v, vq).total);
}

template <int S, int NBV>
static hipError_t launch_attend_t(const AttendArgs &a, int n_work, size_t lds_bytes, hipStream_t s) {
    static bool configured = false;
    if (!configured) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&attend_kernel<S, NBV>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return e;
        configured = true;
    }
    hipLaunchKernelGGL((attend_kernel<S, NBV>), dim3(n_work), dim3(256), lds_bytes, s, a);
    return hipGetLastError();
}

template <int S>
static hipError_t launch_attend_s(const AttendArgs &a, int n_work, size_t lds_bytes, hipStream_t s) {
    const int nbv = (a.v.r + 15) / 16;
    if (nbv <= 1) return launch_attend_t<S, 1>(a, n_work, lds_bytes, s);
    if (nbv <= 2) return launch_attend_t<S, 2>(a, n_work, lds_bytes, s);
    if (nbv <= 4) return launch_attend_t<S, 4>(a, n_work, lds_bytes, s);
    return launch_attend_t<S, 8>(a, n_work, lds_bytes, s);
}

hipError_t launch_attend(const AttendArgs &a, int n_work, size_t lds_bytes, hipStream_t s) {
    switch (16 / a.gqa) {
        case 16: return launch_attend_s<16>(a, n_work, lds_bytes, s);
        case 8: return launch_attend_s<8>(a, n_work, lds_bytes, s);
        case 5: return launch_attend_s<5>(a, n_work, lds_bytes, s);
        case 4: return launch_attend_s<4>(a, n_work, lds_bytes, s);
        case 3: return launch_attend_s<3>(a, n_work, lds_bytes, s);
        default: return launch_attend_s<2>(a, n_work, lds_bytes, s);
    }
}

hipError_t launch_basis_t16(const float *src, uint16_t *dst, int G, int r, hipStream_t s) {
    const int64_t n = static_cast<int64_t>(G) * r * kHeadDim;
    hipLaunchKernelGGL(basis_t16_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, src, dst, G, r);
    return hipGetLastError();
}

hipError_t launch_combine(const AttendArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(combine_kernel, dim3((a.B * a.Hq + 3) / 4), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace palu
