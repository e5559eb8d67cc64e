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
//   append1_kernel : one-token appends (decode steps 1-2).
//   basis_t16_kernel : position-ordered fp16 copy of the key basis (query
//       absorption operand of the decode and prefill attention kernels).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "palu_device.h"
#include "palu_internal.h"

namespace palu {

namespace {

// ---------------------------------------------------------------- Gram ----
//
// Workgroup (block, group g, tensor) owns one block of rows: tokens
// [t0, t1) of one (sequence, head-in-group) segment, so its rows are
// consecutive in memory.  64-row tiles go global -> registers -> LDS,
// transposed to feature-major order (two rows per 32-bit word) so that an
// MFMA operand (8 rows of one feature) is one 16-byte LDS read; the loads of
// the next two tiles are in flight while the current one is multiplied (two
// register buffers, two LDS buffers, one barrier per tile).  Wave w accumulates the 32-row band I = w
// of the 128 x 128 Gram matrix (four 32x32 MFMA tiles) plus the column sums
// of feature block w (an MFMA with an all-ones A operand).

constexpr int kGramTile = 64;      // rows per tile
constexpr int kGramTStride = 72;   // LDS halves per feature run of a tile (64 rows + 8; 16-byte aligned,
                                   // 36 words = 4 mod 32 keeps 8 lanes' 16-byte reads on distinct banks)

// bf16 rows use the bf16 MFMA: bf16 x bf16 products are exact in fp32 just
// like fp16 x fp16.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

template <bool BF16>
__global__ __launch_bounds__(256) void gram_kernel(GramArgs a) {
    const int blk = blockIdx.x, g = blockIdx.y, tz = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const GramBlock bd = a.blocks[blk];
    const int sb = bd.seg / a.hpg, hh = bd.seg - sb * a.hpg;
    const int nrows = bd.t1 - bd.t0;
    const uint16_t *src =
        a.x[tz] + ((static_cast<int64_t>(sb) * a.H + g * a.hpg + hh) * a.S_stride + bd.t0) * kHeadDim;

    __shared__ __align__(16) uint32_t tt[2][kHeadDim][kGramTStride / 2];

    using vec8 = typename std::conditional<BF16, bf16x8, f16x8>::type;
    using elem = typename std::conditional<BF16, __bf16, _Float16>::type;
    const uint16_t one_bits = BF16 ? 0x3F80 : 0x3C00;   // 1.0
    vec8 ones;
    for (int u = 0; u < 8; ++u) ones[u] = __builtin_bit_cast(elem, one_bits);

    // loads: thread (w, lane) takes rows 2p, 2p + 1 (p = lane % 32) and the
    // 16-byte feature chunks c0, c0 + 1 (c0 = 4 w + 2 (lane / 32)); rows past
    // the block read as zero
    const int p = lane & 31, c0 = 4 * w + 2 * (lane >> 5);
    // two register buffers [row of the pair][chunk], for even and odd tiles
    uint4 buf0[2][2], buf1[2][2];
    auto load = [&](int t, uint4 (&bt)[2][2]) {
#pragma unroll
        for (int rp = 0; rp < 2; ++rp) {
            const int r = t * bd.stride + 2 * p + rp;
#pragma unroll
            for (int c = 0; c < 2; ++c)
                bt[rp][c] = r < nrows ? *reinterpret_cast<const uint4 *>(src + static_cast<int64_t>(r) * kHeadDim +
                                                                         8 * (c0 + c))
                                      : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    // word p of feature f's run = (row 2p, row 2p + 1) of feature f
    auto store = [&](int t, const uint4 (&bt)[2][2]) {
        uint32_t(*T)[kGramTStride / 2] = tt[t & 1];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const uint32_t r0[4] = {bt[0][c].x, bt[0][c].y, bt[0][c].z, bt[0][c].w};
            const uint32_t r1[4] = {bt[1][c].x, bt[1][c].y, bt[1][c].z, bt[1][c].w};
            const int f0 = 8 * (c0 + c);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                T[f0 + 2 * u][p] = __builtin_amdgcn_perm(r1[u], r0[u], 0x05040100u);
                T[f0 + 2 * u + 1][p] = __builtin_amdgcn_perm(r1[u], r0[u], 0x07060302u);
            }
        }
    };

    f32x16 acc0 = {}, acc1 = {}, acc2 = {}, acc3 = {}, accs = {};
    const int ntile = (nrows + bd.stride - 1) / bd.stride;
    const int f = lane & 31, kh = lane >> 5;
    auto tile = [&](int t) {
        const uint32_t(*T)[kGramTStride / 2] = tt[t & 1];
#pragma unroll
        for (int ks = 0; ks < kGramTile / 16; ++ks) {
            // operand of feature 32 j + f: rows 16 ks + 8 kh .. + 7 (words 8 ks + 4 kh .. + 3)
            uint4 q[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) q[j] = *reinterpret_cast<const uint4 *>(&T[32 * j + f][8 * ks + 4 * kh]);
            const vec8 o0 = __builtin_bit_cast(vec8, q[0]), o1 = __builtin_bit_cast(vec8, q[1]);
            const vec8 o2 = __builtin_bit_cast(vec8, q[2]), o3 = __builtin_bit_cast(vec8, q[3]);
            const vec8 oa = w == 0 ? o0 : w == 1 ? o1 : w == 2 ? o2 : o3;
            if constexpr (BF16) {
                acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, o0, acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, o1, acc1, 0, 0, 0);
                acc2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, o2, acc2, 0, 0, 0);
                acc3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, o3, acc3, 0, 0, 0);
                accs = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, oa, accs, 0, 0, 0);
            } else {
                acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(oa, o0, acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(oa, o1, acc1, 0, 0, 0);
                acc2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(oa, o2, acc2, 0, 0, 0);
                acc3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(oa, o3, acc3, 0, 0, 0);
                accs = __builtin_amdgcn_mfma_f32_32x32x16_f16(ones, oa, accs, 0, 0, 0);
            }
        }
    };
    // tile t: store it from its register buffer, refill that buffer with
    // tile t + 2, barrier (tile t stored; every wave is past tile t - 1,
    // whose LDS buffer the next store reuses), multiply
    if (ntile > 0) load(0, buf0);
    if (ntile > 1) load(1, buf1);
    int t = 0;
    for (; t + 1 < ntile; t += 2) {
        store(t, buf0);
        if (t + 2 < ntile) load(t + 2, buf0);
        __syncthreads();
        tile(t);
        store(t + 1, buf1);
        if (t + 3 < ntile) load(t + 3, buf1);
        __syncthreads();
        tile(t + 1);
    }
    if (t < ntile) {
        store(t, buf0);
        __syncthreads();
        tile(t);
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
    // blocks in order; loads issued eight at a time
    double s = 0.0;
    int b = 0;
    for (; b + 8 <= a.nb; b += 8) {
        float x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = p[static_cast<int64_t>(b + u) * kElems];
#pragma unroll
        for (int u = 0; u < 8; ++u) s += static_cast<double>(x[u]);
    }
    for (; b < a.nb; ++b) s += static_cast<double>(p[static_cast<int64_t>(b) * kElems]);
    a.out[(static_cast<int64_t>(tz) * a.G + g) * kElems + e] = s;
}

// -------------------------------------------------------------- encode ----
//
// One wave per pair of token groups (64 positions, lane = position) of one
// (call row, kv head, tensor); four independent waves per workgroup, no
// workgroup barriers.  Wave unit u of a row covers groups 2 (j0/2 + u) and
// 2 (j0/2 + u) + 1, j0 = old_len / 32.  A lane's position is new (in
// [old, old + n)), old (an earlier position of group j0, read back from the
// tail buffer) or outside the call.  Per lane y_d = float(x_d) - mu_d in
// fp32, then per channel the fixed-order chain acc = fma(y_d, V[d][c], acc),
// d = 0..D-1; the group's basis (rows padded to a multiple of 4 floats) and
// mean are staged in LDS once per workgroup and read as broadcasts.  The 32
// lanes of a complete group quantise it (min/max by lane reductions, IEEE
// division, round-half-even) and OR their codes into an LDS copy of the
// record at the layout's bit positions; an incomplete group's new latents go
// to the tail buffer; fp16 value latents are stored directly.

constexpr int kEncWaves = 4;

// max / min over the 32 lanes of each half-wave
__device__ __forceinline__ float half_max(float v) {
    v = row_max(v);
    return fmaxf(v, __shfl_xor(v, 16));
}
__device__ __forceinline__ float half_min(float v) { return -half_max(-v); }

struct EncLane {
    int t, half;                // token in its group, which group of the pair
    bool is_new, is_old, complete, touched;
};

// Quantise / store channel c of this lane's latent (see the section comment).
// ct = the channel's entry of the code table: bit of token 0, bits per
// token, width, metadata word.
__device__ __forceinline__ void encode_channel(const EncLane &e, int c, int r, bool fp16, const int4 ct, float lat,
                                               const float *told, float *tnew, uint32_t *rec_lds, uint16_t *rec16,
                                               bool any_complete) {
    // fp16 latents have no tail buffer (told and tnew are null): only new
    // positions are stored
    if (fp16) {
        if (e.is_new) rec16[c * 32 + e.t] = static_cast<uint16_t>(f2h_bits(lat));
        return;
    }
    if (e.is_old) lat = told[e.t * r + c];
    if (!any_complete) {                             // wave-uniform: no group completes
        if (e.touched && e.is_new) tnew[e.t * r + c] = lat;
        return;
    }
    // every lane takes part in the half-wave reductions; only complete
    // groups use the result
    const float mn = half_min(lat), mx = half_max(lat);
    if (e.complete) {
        const int bit = ct.x + e.t * ct.y;
        const float levels = static_cast<float>((1 << ct.z) - 1);
        const float scale = (mx - mn) / levels;
        int q = 0;
        if (scale > 0.0f) {
            float uq = rintf((lat - mn) / scale);
            uq = uq < 0.0f ? 0.0f : (uq > levels ? levels : uq);
            q = static_cast<int>(uq);
        }
        // codes never straddle a word: a code of width w sits at a multiple of w
        if (q) atomicOr(rec_lds + (bit >> 5), static_cast<uint32_t>(q) << (bit & 31));
        if (e.t == 0) rec_lds[ct.w] = f2h_bits(scale) | (f2h_bits(mn) << 16);
    } else if (e.touched && e.is_new) {
        tnew[e.t * r + c] = lat;
    }
}

// W consecutive channels of this lane's latent: W independent fixed-order
// chains over d = 0..D-1, run in four quarters of 32 rows so that only 32
// values y_d = float(x_d) - mu_d are live at a time.  vch is the channel
// chunk's basis in LDS, [D][RW] with RW = W rounded up to 4 (a compile-time
// stride, so every row is an immediate offset); rows are read as 16-byte
// broadcasts (8- and 4-byte ones for the last W % 4 channels).
template <int W, bool BF16>
__device__ __forceinline__ void project_to_lds(const uint16_t *xrow, const float *msh, const float *vch, float *lat,
                                               int lane) {
    constexpr int RW = (W + 3) & ~3;
    float l[W];
#pragma unroll
    for (int k = 0; k < W; ++k) l[k] = 0.0f;
    // the next quarter's 64 bytes are loaded while this one is computed
    uint4 xa[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) xa[k] = *reinterpret_cast<const uint4 *>(xrow + 8 * k);
    for (int q = 0; q < kHeadDim / 32; ++q) {
        uint4 xb[4];
        const int qn = q + 1 < kHeadDim / 32 ? q + 1 : q;
#pragma unroll
        for (int k = 0; k < 4; ++k) xb[k] = *reinterpret_cast<const uint4 *>(xrow + 32 * qn + 8 * k);
        float y[32];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t wq[4] = {xa[k].x, xa[k].y, xa[k].z, xa[k].w};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                y[8 * k + 2 * m] = in2f<BF16>(wq[m]) - msh[32 * q + 8 * k + 2 * m];
                y[8 * k + 2 * m + 1] = in2f_hi<BF16>(wq[m]) - msh[32 * q + 8 * k + 2 * m + 1];
            }
        }
#pragma unroll
        for (int dd = 0; dd < 32; ++dd) {
            const float *vrow = vch + (32 * q + dd) * RW;
#pragma unroll
            for (int k = 0; k + 4 <= W; k += 4) {
                const float4 v = *reinterpret_cast<const float4 *>(vrow + k);
                l[k] = __builtin_fmaf(y[dd], v.x, l[k]);
                l[k + 1] = __builtin_fmaf(y[dd], v.y, l[k + 1]);
                l[k + 2] = __builtin_fmaf(y[dd], v.z, l[k + 2]);
                l[k + 3] = __builtin_fmaf(y[dd], v.w, l[k + 3]);
            }
            constexpr int k2 = W & ~3;
            if constexpr ((W & 3) >= 2) {
                const float2 v = *reinterpret_cast<const float2 *>(vrow + k2);
                l[k2] = __builtin_fmaf(y[dd], v.x, l[k2]);
                l[k2 + 1] = __builtin_fmaf(y[dd], v.y, l[k2 + 1]);
            }
            if constexpr (W & 1) l[W - 1] = __builtin_fmaf(y[dd], vrow[W - 1], l[W - 1]);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) xa[k] = xb[k];
    }
#pragma unroll
    for (int k = 0; k < W; ++k) lat[k * 64 + lane] = l[k];
}

// Dynamic LDS of one encode workgroup: basis (chunks of 32 channels, each
// [D][32] except the last, [D][nc rounded up to 4]: D rp floats in all) +
// mean [D] + per wave two record buffers (none for fp16 latents) and a
// [channels][64 lanes] latent buffer (rows for the widest chunk: r rounded
// up to 4, at most 32), then the code table (one int4 per channel).
__host__ __device__ inline int encode_rec_words(int words, bool fp16) { return fp16 ? 0 : words; }
__host__ __device__ inline int encode_lat_rows(int r) { return ((r + 3) & ~3) < 32 ? ((r + 3) & ~3) : 32; }
__host__ __device__ inline int encode_lds_bytes(int r, int words, bool fp16) {
    const int rp = (r + 3) & ~3;
    return (kHeadDim * rp + kHeadDim + kEncWaves * (2 * encode_rec_words(words, fp16) + encode_lat_rows(r) * 64) +
            4 * r) * 4;
}

// Five waves per SIMD (at most 96 VGPRs; the latent buffer is sized by the
// rank so that LDS admits five workgroups per CU at ranks up to 16): the
// projection's LDS broadcast reads and the quantiser's reductions are latency
// chains that the extra wave hides.
template <bool BF16>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(5))) void encode_kernel(EncodeArgs a) {
    extern __shared__ __align__(16) float esh[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int u = blockIdx.x * kEncWaves + wv;
    const int bi = blockIdx.y / a.H, h = blockIdx.y - (blockIdx.y / a.H) * a.H;
    const int tz = blockIdx.z;
    const int o = a.old_len[bi], n = a.n_new[bi];
    // the row's new length and tail buffer, mirrored in device memory
    if (blockIdx.x == 0 && h == 0 && tz == 0 && tid == 0 && a.len_dev) {
        a.len_dev[a.slot[bi]] = o + n;
        a.sel_dev[a.slot[bi]] = a.sel_new[bi];
    }
    if (n <= 0) return;                              // whole workgroup
    const int j0 = o >> 5, jl = (o + n - 1) >> 5;
    if (2 * ((j0 >> 1) + blockIdx.x * kEncWaves) > jl) return;   // whole workgroup
    const TensorDev &T = tz ? a.t[1] : a.t[0];
    const int r = T.r, rp = (r + 3) & ~3, W = T.words;
    const int grp = h / a.hpg, slot = a.slot[bi];

    // 0. the group's basis in 32-channel chunks (chunk j = channels 32 j ..,
    //    [D][32], the last [D][rwl], rwl = its channels rounded up to 4,
    //    zero-padded) and mean -> LDS
    float *vsh = esh;
    float *msh = esh + kHeadDim * rp;
    {
        const float *vb = T.basis + slot * T.set_basis + static_cast<int64_t>(grp) * kHeadDim * r;
        const int cl = (r - 1) & ~31;                 // first channel of the last chunk
        const int rwl = rp - cl, full = kHeadDim * cl;
        for (int e = tid; e < kHeadDim * rp; e += 256) {
            int d, c;
            if (e < full) {
                d = (e & 4095) >> 5;
                c = ((e >> 12) << 5) + (e & 31);
            } else {
                d = (e - full) / rwl;
                c = cl + (e - full) - d * rwl;
            }
            vsh[e] = c < r ? vb[d * r + c] : 0.0f;
        }
        if (tid < kHeadDim) msh[tid] = T.mu[slot * T.set_mu + grp * kHeadDim + tid];
    }
    // code table: per channel the record bit of token 0, the bits between
    // consecutive tokens, the width and the metadata word (read as one
    // broadcast per channel instead of a walk over the segment list)
    const int WR = encode_rec_words(W, T.fp16_latents);
    const int LR = encode_lat_rows(r);
    int4 *ctab = reinterpret_cast<int4 *>(msh + kHeadDim + kEncWaves * (2 * WR + LR * 64));
    if (tid < r && !T.fp16_latents) {
        const int2 b0 = code_bit(T.cd, tz, tid, 0), b1 = code_bit(T.cd, tz, tid, 1);
        ctab[tid] = make_int4(b0.x, b1.x - b0.x, b0.y, T.cd.meta0 + tid);
    }
    __syncthreads();
    const int jp = (j0 >> 1) + u;                    // group pair of this wave
    if (2 * jp > jl) return;                         // wave-uniform; no barrier follows

    const int p = 64 * jp + lane;                    // this lane's position
    EncLane e;
    const int j = p >> 5;
    e.t = p & 31;
    e.half = lane >> 5;
    e.is_new = p >= o && p < o + n;
    e.is_old = p < o && j == j0;
    e.touched = j >= j0 && j <= jl;
    e.complete = e.touched && o + n >= 32 * j + 32;
    // complete groups that get a quantised record (fp16 latents have none)
    const bool fp16 = T.fp16_latents;
    const bool any_complete = !fp16 && __any(e.complete);
    const int64_t head_base = static_cast<int64_t>(slot) * a.H + h;

    uint32_t *rec_lds = reinterpret_cast<uint32_t *>(msh + kHeadDim) + (wv * 2 + e.half) * WR;
    float *lat = msh + kHeadDim + kEncWaves * 2 * WR + wv * LR * 64;   // this wave's [LR][64]
    if (any_complete) {
        for (int w = e.t; w < W; w += 32) rec_lds[w] = 0u;
    }

    // 1. this lane's input row (a valid row is read for every lane; only
    //    new positions use theirs)
    const int row = e.is_new ? p - o : 0;
    const uint16_t *xrow = a.x[tz] + (static_cast<int64_t>(bi) * a.H + h) * a.T_stride * kHeadDim +
                           static_cast<int64_t>(row) * kHeadDim;

    // 2. latents in chunks of up to 32 channels (one fma chain per channel),
    //    parked in LDS, then quantised / stored channel by channel
    const float *told = T.fp16_latents ? nullptr : T.tail + (head_base * 2 + a.sel_old[bi]) * 32 * r;
    float *tnew = T.fp16_latents ? nullptr : T.tail + (head_base * 2 + a.sel_new[bi]) * 32 * r;
    uint16_t *rec16 = reinterpret_cast<uint16_t *>(T.records + head_base * T.head_stride +
                                                   static_cast<int64_t>(j) * W);
    for (int c0 = 0; c0 < r; c0 += 32) {
        const int nc = r - c0 < 32 ? r - c0 : 32;
        // exactly nc chains up to 16 channels, a multiple of 4 above
        switch (nc <= 16 ? nc : 16 + ((nc - 13) >> 2)) {
            case 1: project_to_lds<1, BF16>(xrow, msh, vsh + kHeadDim * c0, lat, lane); break;
            case 2: project_to_lds<2, BF16>(xrow, msh, vsh + kHeadDim * c0, lat, lane); break;
            case 3: project_to_lds<3, BF16>(xrow, msh, vsh + kHeadDim * c0, lat, lane); break;
            case 4: project_to_lds<4, BF16>(xrow, msh, vsh + kHeadDim * c0, lat, lane); break;
            case 5: project_to_lds<5, BF16>(xrow, msh, vsh + kHeadDim * c0, lat, lane); break;
            case 6: project_to_lds<6, BF16>(xrow, msh, vsh + kHeadDim * c0, lat, lane); break;
            case 7: project_to_lds<7, BF16>(xrow, msh, vsh + kHeadDim * c0, lat, lane); break;
            case 8: project_to_lds<8, BF16>(xrow, msh, vsh + kHeadDim * c0, lat, lane); break;
            case 9: project_to_lds<9, BF16>(xrow, msh, vsh + kHeadDim * c0, lat, lane); break;
            case 10: project_to_lds<10, BF16>(xrow, msh, vsh + kHeadDim * c0, lat, lane); break;
            case 11: project_to_lds<11, BF16>(xrow, msh, vsh + kHeadDim * c0, lat, lane); break;
            case 12: project_to_lds<12, BF16>(xrow, msh, vsh + kHeadDim * c0, lat, lane); break;
            case 13: project_to_lds<13, BF16>(xrow, msh, vsh + kHeadDim * c0, lat, lane); break;
            case 14: project_to_lds<14, BF16>(xrow, msh, vsh + kHeadDim * c0, lat, lane); break;
            case 15: project_to_lds<15, BF16>(xrow, msh, vsh + kHeadDim * c0, lat, lane); break;
            case 16: project_to_lds<16, BF16>(xrow, msh, vsh + kHeadDim * c0, lat, lane); break;
            case 17: project_to_lds<20, BF16>(xrow, msh, vsh + kHeadDim * c0, lat, lane); break;
            case 18: project_to_lds<24, BF16>(xrow, msh, vsh + kHeadDim * c0, lat, lane); break;
            case 19: project_to_lds<28, BF16>(xrow, msh, vsh + kHeadDim * c0, lat, lane); break;
            default: project_to_lds<32, BF16>(xrow, msh, vsh + kHeadDim * c0, lat, lane); break;
        }
        for (int k = 0; k < nc; ++k)
            encode_channel(e, c0 + k, r, fp16, fp16 ? make_int4(0, 0, 0, 0) : ctab[c0 + k], lat[k * 64 + lane], told,
                           tnew, rec_lds, rec16, any_complete);
    }

    // 3. complete groups: LDS record -> memory
    if (any_complete) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (e.complete) {
            uint32_t *rec = T.records + head_base * T.head_stride + static_cast<int64_t>(j) * W;
            for (int w = e.t; w < W; w += 32) rec[w] = rec_lds[w];
        }
    }
}

// ------------------------------------------------------ append one token ----
//
// Appends of at most one token per row (the decode step).  Workgroup =
// (call row x kv head, tensor), 128 threads, thread c < r owns latent
// channel c.  y = float(x) - mu and the group's basis are staged in LDS; each
// channel runs the fixed-order fma chain over d.  The token either extends
// the fp32 tail of the incomplete group or completes it; then every
// channel's 32 latents (31 from the tail, the new one) are quantised in
// token order and the codes OR-ed into an LDS copy of the record.

// One wave per (call row x kv head, tensor).  Lane c owns latent channel c
// (and c + 64 when r > 64): its basis row (channel-major copy, 128 floats)
// comes into registers with the first loads, the centred input y = x - mu is
// broadcast through LDS, and the channel's latent is the fixed-order fp32
// chain fma(y_d, V[d][c], acc), d = 0..D-1.  An incomplete group keeps the
// latent in the fp32 tail; a token that completes its group quantises the
// group's 32 latents per channel (lane = channel) and ORs the codes into an
// LDS copy of the record.
constexpr int kApp1Threads = 64;

__host__ __device__ inline int append1_lds_bytes(int words) { return (kHeadDim + words) * 4; }

template <bool BF16>
__global__ __launch_bounds__(kApp1Threads) void append1_kernel(EncodeArgs a) {
    extern __shared__ __align__(16) float ash[];
    const int lane = threadIdx.x;
    const int bi = blockIdx.x / a.H, h = blockIdx.x - (blockIdx.x / a.H) * a.H;
    const int tz = blockIdx.y;
    const int slot = a.slot[bi];
    int o, n, sel_old, sel_new;
    if (a.dev_len) {
        // one token per row at the stored length (nothing past the capacity)
        o = a.len_dev[slot];
        n = o < a.max_len ? 1 : 0;
        sel_old = sel_new = a.sel_dev[slot];   // one token never moves the tail buffer
    } else {
        o = a.old_len[bi];
        n = a.n_new[bi];
        sel_old = a.sel_old[bi];
        sel_new = a.sel_new[bi];
        if (h == 0 && tz == 0 && lane == 0 && a.len_dev) {
            a.len_dev[slot] = o + n;
            a.sel_dev[slot] = sel_new;
        }
    }
    if (n <= 0) return;                               // whole workgroup
    const TensorDev &T = tz ? a.t[1] : a.t[0];
    const int r = T.r, W = T.words;
    const int grp = h / a.hpg;
    const int64_t head_base = static_cast<int64_t>(slot) * a.H + h;
    const int j = o >> 5, t = o & 31;                 // group and position of the new token
    const bool complete = t == 31 && !T.fp16_latents;
    float *ys = ash;
    uint32_t *rec = reinterpret_cast<uint32_t *>(ash + kHeadDim);

    // 1. y = float(x) - mu, two elements per lane, to LDS; the record copy
    //    is cleared when the group completes
    const uint16_t *xin = a.x[tz] + (static_cast<int64_t>(bi) * a.H + h) * a.T_stride * kHeadDim;
    const uint32_t xp = reinterpret_cast<const uint32_t *>(xin)[lane];
    const float2 mu = reinterpret_cast<const float2 *>(T.mu + slot * T.set_mu + grp * kHeadDim)[lane];
    reinterpret_cast<float2 *>(ys)[lane] = make_float2(in2f<BF16>(xp & 0xFFFFu) - mu.x, in2f<BF16>(xp >> 16) - mu.y);
    if (complete)
        for (int w = lane; w < W; w += kApp1Threads) rec[w] = 0u;
    __syncthreads();

    const float *bcm = T.basis_cm + slot * T.set_bcm + static_cast<int64_t>(grp) * r * kHeadDim;
    const float4 *ys4 = reinterpret_cast<const float4 *>(ys);
    const float *told = T.tail + (head_base * 2 + sel_old) * 32 * r;
    for (int c = lane; c < r; c += kApp1Threads) {
        // 2. the chain, with the channel's basis row in registers; when the
        //    group completes, its 31 older latents are loaded alongside
        float4 vb[kHeadDim / 4];
        const float4 *row = reinterpret_cast<const float4 *>(bcm + static_cast<int64_t>(c) * kHeadDim);
#pragma unroll
        for (int d4 = 0; d4 < kHeadDim / 4; ++d4) vb[d4] = row[d4];
        float lv[32];
        if (complete) {
#pragma unroll
            for (int tt = 0; tt < 31; ++tt) lv[tt] = told[tt * r + c];
        }
        float lat = 0.0f;
#pragma unroll
        for (int d4 = 0; d4 < kHeadDim / 4; ++d4) {
            const float4 y = ys4[d4];
            lat = __builtin_fmaf(y.x, vb[d4].x, lat);
            lat = __builtin_fmaf(y.y, vb[d4].y, lat);
            lat = __builtin_fmaf(y.z, vb[d4].z, lat);
            lat = __builtin_fmaf(y.w, vb[d4].w, lat);
        }
        if (T.fp16_latents) {                         // uniform: no tail, no quantiser
            uint16_t *rec16 = reinterpret_cast<uint16_t *>(T.records + head_base * T.head_stride +
                                                           static_cast<int64_t>(j) * W);
            rec16[c * 32 + t] = static_cast<uint16_t>(f2h_bits(lat));
            continue;
        }
        if (!complete) {                              // uniform
            T.tail[(head_base * 2 + sel_new) * 32 * r + t * r + c] = lat;
            continue;
        }
        // 3. the group completes: channel c over its 32 latents in token order
        lv[31] = lat;
        float mn = lv[0], mx = mn;
#pragma unroll
        for (int tt = 1; tt < 32; ++tt) {
            mn = lv[tt] < mn ? lv[tt] : mn;
            mx = lv[tt] > mx ? lv[tt] : mx;
        }
        const int2 b0 = code_bit(T.cd, tz, c, 0);    // token 0's bit, width
        const int tstep = tz == 0 ? code_bit(T.cd, 0, c, 1).x - b0.x : b0.y;   // bits between tokens
        const float levels = static_cast<float>((1 << b0.y) - 1);
        const float scale = (mx - mn) / levels;
#pragma unroll
        for (int tt = 0; tt < 32; ++tt) {
            int q = 0;
            if (scale > 0.0f) {
                float uq = rintf((lv[tt] - mn) / scale);
                uq = uq < 0.0f ? 0.0f : (uq > levels ? levels : uq);
                q = static_cast<int>(uq);
            }
            const int bit = b0.x + tt * tstep;
            if (q) atomicOr(rec + (bit >> 5), static_cast<uint32_t>(q) << (bit & 31));
        }
        rec[T.cd.meta0 + c] = f2h_bits(scale) | (f2h_bits(mn) << 16);
    }
    if (!complete) return;                            // uniform
    __syncthreads();
    uint32_t *dst = T.records + head_base * T.head_stride + static_cast<int64_t>(j) * W;
    for (int w = lane; w < W; w += kApp1Threads) dst[w] = rec[w];
}

// dst[g][n][d] = fp16(V[g][d][chan(n)]) for the score-operand position n
// (block q = n / 8 of 8 channels, hi blocks first; slot idx = n % 8 holds
// channel (idx >> 1) + 4 (idx & 1) of the block), 0 where n is padding.
__global__ __launch_bounds__(256) void basis_t16_kernel(const float *src, uint16_t *dst, int G, int r, Coder cd) {
    const int rows = 8 * cd.q0[cd.nseg];
    const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (e >= static_cast<int64_t>(G) * rows * kHeadDim) return;
    const int d = static_cast<int>(e % kHeadDim);
    const int64_t gn = e / kHeadDim;
    const int n = static_cast<int>(gn % rows), g = static_cast<int>(gn / rows);
    const int q = n >> 3, idx = n & 7;
    const KBlock kbq = key_block(cd, q);
    const int chan0 = kbq.chan0, chanend = kbq.chanend;
    const int c = chan0 + (idx >> 1) + 4 * (idx & 1);
    dst[e] = c < chanend ? static_cast<uint16_t>(f2h_bits(src[(static_cast<int64_t>(g) * kHeadDim + d) * r + c]))
                         : static_cast<uint16_t>(0);
}

}  // namespace

hipError_t gram_resident_blocks(int *n) {
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(gram_kernel<false>), 256,
                                                         0);
    *n = cus * per_cu;
    return e;
}

hipError_t launch_gram(const GramArgs &a, hipStream_t s) {
    if (a.bf16) hipLaunchKernelGGL(gram_kernel<true>, dim3(a.nb, a.G, 2), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(gram_kernel<false>, dim3(a.nb, a.G, 2), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_gram_reduce(const GramReduceArgs &a, hipStream_t s) {
    constexpr int kElems = kHeadDim * kHeadDim + kHeadDim;
    hipLaunchKernelGGL(gram_reduce_kernel, dim3((kElems + 255) / 256, a.G, 2), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <bool BF16>
static hipError_t launch_append1_t(const EncodeArgs &a, hipStream_t s) {
    // set once per process (thread-safe static initialisation)
    static const hipError_t attr =
        hipFuncSetAttribute(reinterpret_cast<const void *>(append1_kernel<BF16>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (attr != hipSuccess) return attr;
    const int l0 = append1_lds_bytes(a.t[0].words), l1 = append1_lds_bytes(a.t[1].words);
    hipLaunchKernelGGL(append1_kernel<BF16>, dim3(a.B * a.H, 2), dim3(kApp1Threads),
                       static_cast<size_t>(l0 > l1 ? l0 : l1), s, a);
    return hipGetLastError();
}

hipError_t launch_append1(const EncodeArgs &a, hipStream_t s) {
    return a.bf16 ? launch_append1_t<true>(a, s) : launch_append1_t<false>(a, s);
}

template <bool BF16>
static hipError_t launch_encode_t(const EncodeArgs &a, int max_units, hipStream_t s) {
    // set once per process (thread-safe static initialisation)
    static const hipError_t attr =
        hipFuncSetAttribute(reinterpret_cast<const void *>(encode_kernel<BF16>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (attr != hipSuccess) return attr;
    const int l0 = encode_lds_bytes(a.t[0].r, a.t[0].words, a.t[0].fp16_latents),
              l1 = encode_lds_bytes(a.t[1].r, a.t[1].words, a.t[1].fp16_latents);
    hipLaunchKernelGGL(encode_kernel<BF16>, dim3((max_units + kEncWaves - 1) / kEncWaves, a.B * a.H, 2), dim3(256),
                       static_cast<size_t>(l0 > l1 ? l0 : l1), s, a);
    return hipGetLastError();
}

hipError_t launch_encode(const EncodeArgs &a, int max_units, hipStream_t s) {
    return a.bf16 ? launch_encode_t<true>(a, max_units, s) : launch_encode_t<false>(a, max_units, s);
}

hipError_t launch_basis_t16(const float *src, uint16_t *dst, int G, int r, const Coder &cd, hipStream_t s) {
    const int64_t n = static_cast<int64_t>(G) * basis_t16_rows(cd) * kHeadDim;
    hipLaunchKernelGGL(basis_t16_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, src, dst, G, r,
                       cd);
    return hipGetLastError();
}


// ---------------------------------------------------------- read probe ----
//
// Measurement aid: every thread walks the buffer with a grid stride, four
// independent 16-byte loads in flight per step, XOR-folding what it reads;
// one lane per workgroup stores the workgroup's fold so no load is dead.
__global__ __launch_bounds__(256) void read_probe_kernel(const uint4 *__restrict__ src, size_t n16,
                                                         uint32_t *__restrict__ sink) {
    const size_t stride = static_cast<size_t>(gridDim.x) * 256;
    size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
        acc ^= (a.x ^ a.y ^ a.z ^ a.w) ^ (b.x ^ b.y ^ b.z ^ b.w) ^ (c.x ^ c.y ^ c.z ^ c.w) ^ (d.x ^ d.y ^ d.z ^ d.w);
    }
    for (; i < n16; i += stride) {
        const uint4 a = src[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
    __shared__ uint32_t wf[4];
    if ((threadIdx.x & 63) == 0) wf[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = wf[0] ^ wf[1] ^ wf[2] ^ wf[3];
}

hipError_t launch_read_probe(const void *src, size_t n16, uint32_t *sink, int grid, hipStream_t s) {
    hipLaunchKernelGGL(read_probe_kernel, dim3(grid), dim3(256), 0, s, static_cast<const uint4 *>(src), n16, sink);
    return hipGetLastError();
}

}  // namespace palu
