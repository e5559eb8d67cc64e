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
// One wave per REPS consecutive pairs of token groups, one pair (64
// positions, lane = position) after the other, of one (call row, kv head,
// tensor); four independent waves per workgroup, no workgroup barriers after
// the code table.  Unit u of a row covers groups 2 (j0/2 + u) and
// 2 (j0/2 + u) + 1, j0 = old_len / 32.  A lane's
// position is new (in [old, old + n)), old (an earlier position of group j0,
// read back from the tail buffer) or outside the call.  Per lane
// y_d = float(x_d) - mu_d in fp32 (one mixed-precision fma per fp16 element,
// the same single rounding), then per channel the fixed-order chain
// acc = fma(y_d, V[d][c], acc), d = 0..D-1.  The basis and the mean are the
// same for every lane: they come in through scalar loads and enter the fmas
// as SGPR operands, so the projection reads no LDS.
//
// A complete group is quantised in three passes over its channels: (1) the
// minimum and maximum over each 32-lane half by DPP (the results land in
// lanes 31 and 63); (2) one lane per (group, channel) forms
// scale = (max - min) / levels by IEEE division, its reciprocal and the
// metadata word; (3) every lane forms its code
// round-half-even((l - min) / scale) and ORs it into an LDS copy of the
// record at the layout's bit position.  The IEEE quotient decides each code:
// the reciprocal product is within 2^-21 relative of it (reciprocal within
// 1 ulp, one product rounding), so for quotients below 256 the two round to
// the same integer unless the product lies within 2^-11 of a half-integer,
// and there the lane divides.  An incomplete group's new latents go to the
// tail buffer; fp16 value latents are stored directly.

constexpr int kEncWaves = 4;

struct EncLane {
    int t, half;                // token in its group, which group of the pair
    bool is_new, is_old, complete, touched;
};


// Constant-address-space view of a basis or mean: uniform loads from it are
// scalar loads, and the values are SGPR operands of the fmas.
typedef const float __attribute__((address_space(4))) ConstF;

// float(h) - mu for the low (HI = false) or high fp16 half of a word: the
// mixed-precision fma h * 1 - mu, exact product and one rounding, equal to
// the fp32 subtraction.
template <bool HI>
__device__ __forceinline__ float centred_f16(uint32_t w, float mu) {
    float y;
    if constexpr (HI)
        asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(y) : "v"(w), "s"(mu));
    else
        asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel_hi:[1,0,0]" : "=v"(y) : "v"(w), "s"(mu));
    return y;
}

// The value of lane 15 of the previous 16-lane row, in rows 1 and 3 (rows 0
// and 2 keep their own): after a row reduction, lanes 31 and 63 combine it
// into the reduction over their 32-lane half.
__device__ __forceinline__ float from_prev_row(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v),
                                                                 0x142, 0xA, 0xF, false));
}

// W consecutive channels of this lane's latent: W independent fixed-order
// chains over d = 0..D-1, run in steps of QD rows (32, or 16 for more than 16
// chains) so that only QD values y_d are live at a time.  vb points at the
// chunk's first channel in the [D][r] basis.  RS = r when it is known at
// compile time (the chunk is the whole row and W = r: constant offsets);
// RS = 0 strides the rows by the runtime r, and W may exceed the chunk's
// channels by up to 3: those chains read the next row's first values (or,
// after the last row, the basis region's slack) and are not used.
template <int W, int RS, bool BF16>
__device__ __forceinline__ void project_chunk(const uint16_t *xrow, ConstF *mu, ConstF *vb, int r, float *lat,
                                              int lane) {
    constexpr int QD = W > 16 ? 16 : 32, NX = QD / 8;   // rows per step, 16-byte input pieces per step
    constexpr int kSteps = kHeadDim / QD, kStepUnroll = W > 16 ? 2 : kSteps;
    const int rs = RS ? RS : r;
    float l[W];
#pragma unroll
    for (int k = 0; k < W; ++k) l[k] = 0.0f;
    // the next step's input is loaded while this one is computed
    uint4 xa[NX];
#pragma unroll
    for (int k = 0; k < NX; ++k) xa[k] = *reinterpret_cast<const uint4 *>(xrow + 8 * k);
#pragma unroll kStepUnroll
    for (int q = 0; q < kSteps; ++q) {
        uint4 xb[NX];
        const int qn = q + 1 < kHeadDim / QD ? q + 1 : q;
#pragma unroll
        for (int k = 0; k < NX; ++k) xb[k] = *reinterpret_cast<const uint4 *>(xrow + QD * qn + 8 * k);
        float y[QD];
#pragma unroll
        for (int k = 0; k < NX; ++k) {
            const uint32_t wq[4] = {xa[k].x, xa[k].y, xa[k].z, xa[k].w};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int d = QD * q + 8 * k + 2 * m;
                if constexpr (BF16) {
                    y[8 * k + 2 * m] = in2f<true>(wq[m]) - mu[d];
                    y[8 * k + 2 * m + 1] = in2f_hi<true>(wq[m]) - mu[d + 1];
                } else {
                    y[8 * k + 2 * m] = centred_f16<false>(wq[m], mu[d]);
                    y[8 * k + 2 * m + 1] = centred_f16<true>(wq[m], mu[d + 1]);
                }
            }
        }
        // a runtime stride is re-read per step (opaque to the compiler), so
        // the row offsets are formed here rather than hoisted out of every
        // width's code into the kernel's prologue
        int rsq = rs;
        if constexpr (RS == 0) asm volatile("" : "+s"(rsq));
        ConstF *vq = vb + QD * q * rsq;
#pragma unroll
        for (int dd = 0; dd < QD; ++dd) {
            ConstF *vrow = vq + dd * rsq;
#pragma unroll
            for (int k = 0; k < W; ++k) l[k] = __builtin_fmaf(y[dd], vrow[k], l[k]);
        }
#pragma unroll
        for (int k = 0; k < NX; ++k) xa[k] = xb[k];
    }
#pragma unroll
    for (int k = 0; k < W; ++k) lat[k * 64 + lane] = l[k];
}

// Dynamic LDS of one encode workgroup, per wave: the quantiser's 64 (group,
// channel) entries (float4; none for fp16 latents), two record buffers
// (words rounded up to even; none for fp16 latents) and a [channels][64
// lanes] latent buffer (rows for the widest chunk: r rounded up to 4, at most
// 32); then the code table (one int4 per channel).  Every part starts on a
// 16-byte boundary.
__host__ __device__ inline int encode_rec_words(int words, bool fp16) { return fp16 ? 0 : (words + 1) & ~1; }
__host__ __device__ inline int encode_lat_rows(int r) { return ((r + 3) & ~3) < 32 ? ((r + 3) & ~3) : 32; }
__host__ __device__ inline int encode_sc_floats(bool fp16) { return fp16 ? 0 : 256; }
__host__ __device__ inline int encode_lds_bytes(int r, int words, bool fp16) {
    return (kEncWaves * (encode_sc_floats(fp16) + 2 * encode_rec_words(words, fp16) + encode_lat_rows(r) * 64) +
            4 * r) * 4;
}

// Ranks up to 16 (REPS = 1): five waves per SIMD (at most 96 VGPRs), the
// quantiser's reductions and the scalar-load waits of the projection being
// latency chains that the extra waves hide.  Wider ranks (REPS = 2): up to
// 32 fma chains per lane need the registers of four waves per SIMD, and
// each wave takes two group pairs, so that the basis it streams through
// scalar loads serves twice the positions.
template <bool BF16, int REPS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(REPS > 1 ? 4 : 5))) void encode_kernel(
    EncodeArgs a) {
    extern __shared__ __align__(16) float esh[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int u = (blockIdx.x * kEncWaves + wv) * REPS;      // first unit of this wave
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
    if (2 * ((j0 >> 1) + blockIdx.x * kEncWaves * REPS) > jl) return;   // whole workgroup
    const TensorDev &T = tz ? a.t[1] : a.t[0];
    const int r = T.r, W = T.words;
    const int grp = h / a.hpg, slot = a.slot[bi];
    const bool fp16 = T.fp16_latents;
    const int SC = encode_sc_floats(fp16), WR = encode_rec_words(W, fp16), LR = encode_lat_rows(r);

    // code table: per channel the record bit of token 0, the bits between
    // consecutive tokens, the width and the metadata word (read as one
    // broadcast per channel instead of a walk over the segment list)
    int4 *ctab = reinterpret_cast<int4 *>(esh + kEncWaves * (SC + 2 * WR + LR * 64));
    if (tid < r && !fp16) {
        const int2 b0 = code_bit(T.cd, tz, tid, 0), b1 = code_bit(T.cd, tz, tid, 1);
        ctab[tid] = make_int4(b0.x, b1.x - b0.x, b0.y, T.cd.meta0 + tid);
    }
    __syncthreads();
    for (int rep = 0; rep < REPS; ++rep) {
        const int jp = (j0 >> 1) + u + rep;              // group pair of this pass
        if (2 * jp > jl) break;                          // wave-uniform; no barrier follows

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
        const bool any_complete = !fp16 && __any(e.complete);
        const bool any_old = !fp16 && __any(e.is_old);
        const int64_t head_base = static_cast<int64_t>(slot) * a.H + h;

        float4 *sc = reinterpret_cast<float4 *>(esh) + wv * (SC / 4);                     // [2 halves][32 channels]
        uint32_t *rec_lds = reinterpret_cast<uint32_t *>(esh + kEncWaves * SC) + (wv * 2 + e.half) * WR;
        float *lat = esh + kEncWaves * (SC + 2 * WR) + wv * LR * 64;                       // this wave's [LR][64]
        if (any_complete) {
            for (int w = e.t; w < W; w += 32) rec_lds[w] = 0u;
        }

        // 1. this lane's input row (a valid row is read for every lane; only
        //    new positions use theirs)
        const int row = e.is_new ? p - o : 0;
        const uint16_t *xrow = a.x[tz] + (static_cast<int64_t>(bi) * a.H + h) * a.T_stride * kHeadDim +
                               static_cast<int64_t>(row) * kHeadDim;
        ConstF *mu = (ConstF *)(T.mu + slot * T.set_mu + grp * kHeadDim);   // address-space cast
        ConstF *vbase = (ConstF *)(T.basis + slot * T.set_basis + static_cast<int64_t>(grp) * kHeadDim * r);

        // 2. latents in chunks of up to 32 channels (one fma chain per channel),
        //    parked in LDS, then quantised / stored channel by channel
        const float *told = fp16 ? nullptr : T.tail + (head_base * 2 + a.sel_old[bi]) * 32 * r;
        float *tnew = fp16 ? nullptr : T.tail + (head_base * 2 + a.sel_new[bi]) * 32 * r;
        uint16_t *rec16 = reinterpret_cast<uint16_t *>(T.records + head_base * T.head_stride +
                                                       static_cast<int64_t>(j) * W);
        for (int c0 = 0; c0 < r; c0 += 32) {
            const int nc = r - c0 < 32 ? r - c0 : 32;
            ConstF *vb = vbase + c0;
            if (nc == r && (nc <= 16 || (nc & 3) == 0)) {
                // the whole row in one chunk of a compiled width
                switch (nc <= 16 ? nc : 12 + (nc >> 2)) {
                    case 1: project_chunk<1, 1, BF16>(xrow, mu, vb, r, lat, lane); break;
                    case 2: project_chunk<2, 2, BF16>(xrow, mu, vb, r, lat, lane); break;
                    case 3: project_chunk<3, 3, BF16>(xrow, mu, vb, r, lat, lane); break;
                    case 4: project_chunk<4, 4, BF16>(xrow, mu, vb, r, lat, lane); break;
                    case 5: project_chunk<5, 5, BF16>(xrow, mu, vb, r, lat, lane); break;
                    case 6: project_chunk<6, 6, BF16>(xrow, mu, vb, r, lat, lane); break;
                    case 7: project_chunk<7, 7, BF16>(xrow, mu, vb, r, lat, lane); break;
                    case 8: project_chunk<8, 8, BF16>(xrow, mu, vb, r, lat, lane); break;
                    case 9: project_chunk<9, 9, BF16>(xrow, mu, vb, r, lat, lane); break;
                    case 10: project_chunk<10, 10, BF16>(xrow, mu, vb, r, lat, lane); break;
                    case 11: project_chunk<11, 11, BF16>(xrow, mu, vb, r, lat, lane); break;
                    case 12: project_chunk<12, 12, BF16>(xrow, mu, vb, r, lat, lane); break;
                    case 13: project_chunk<13, 13, BF16>(xrow, mu, vb, r, lat, lane); break;
                    case 14: project_chunk<14, 14, BF16>(xrow, mu, vb, r, lat, lane); break;
                    case 15: project_chunk<15, 15, BF16>(xrow, mu, vb, r, lat, lane); break;
                    case 16: project_chunk<16, 16, BF16>(xrow, mu, vb, r, lat, lane); break;
                    case 17: project_chunk<20, 20, BF16>(xrow, mu, vb, r, lat, lane); break;
                    case 18: project_chunk<24, 24, BF16>(xrow, mu, vb, r, lat, lane); break;
                    case 19: project_chunk<28, 28, BF16>(xrow, mu, vb, r, lat, lane); break;
                    default: project_chunk<32, 32, BF16>(xrow, mu, vb, r, lat, lane); break;
                }
            } else {
                // other chunks: runtime row stride, width rounded up to 4
                switch ((nc + 3) >> 2) {
                    case 1: project_chunk<4, 0, BF16>(xrow, mu, vb, r, lat, lane); break;
                    case 2: project_chunk<8, 0, BF16>(xrow, mu, vb, r, lat, lane); break;
                    case 3: project_chunk<12, 0, BF16>(xrow, mu, vb, r, lat, lane); break;
                    case 4: project_chunk<16, 0, BF16>(xrow, mu, vb, r, lat, lane); break;
                    case 5: project_chunk<20, 0, BF16>(xrow, mu, vb, r, lat, lane); break;
                    case 6: project_chunk<24, 0, BF16>(xrow, mu, vb, r, lat, lane); break;
                    case 7: project_chunk<28, 0, BF16>(xrow, mu, vb, r, lat, lane); break;
                    default: project_chunk<32, 0, BF16>(xrow, mu, vb, r, lat, lane); break;
                }
            }
            if (fp16) {
                // fp16 latents: only new positions are stored
                if (e.is_new)
                    for (int k = 0; k < nc; ++k) rec16[(c0 + k) * 32 + e.t] = static_cast<uint16_t>(f2h_bits(lat[k * 64 + lane]));
                continue;
            }
            // pass 1: each channel's value (old positions from the tail buffer),
            // new latents of an incomplete group to the tail, and per half the
            // minimum and maximum (lanes 31 and 63 record them)
            if (any_old) {
                // old positions of the first group: their latents from the tail
                // buffer, into the latent buffer
                for (int k = 0; k < nc; ++k)
                    if (e.is_old) lat[k * 64 + lane] = told[e.t * r + c0 + k];
            }
            for (int k = 0; k < nc; ++k) {
                const int c = c0 + k;
                const float v = lat[k * 64 + lane];
                if (!e.complete && e.touched && e.is_new) tnew[e.t * r + c] = v;
                if (any_complete) {                      // wave-uniform
                    float mx = row_max(v), mn = -row_max(-v);
                    mx = fmaxf(mx, from_prev_row(mx));
                    mn = fminf(mn, from_prev_row(mn));
                    if (e.t == 31) *reinterpret_cast<float2 *>(sc + e.half * 32 + k) = make_float2(mn, mx);
                }
            }
            if (!any_complete) continue;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // pass 2: lane (half, k) takes its group's channel c0 + k: scale by
            // IEEE division, the reciprocal (normal scales only; 0 makes every
            // code of the channel a division) and the metadata word
            {
                const int k = lane & 31;
                if (k < nc && e.complete) {
                    const int c = c0 + k;
                    const int4 ct = ctab[c];
                    const float2 mm = *reinterpret_cast<const float2 *>(sc + e.half * 32 + k);
                    const float levels = static_cast<float>((1 << ct.z) - 1);
                    const float scale = (mm.y - mm.x) / levels;
                    const float inv = scale >= 0x1p-126f && scale < 0x1p+126f ? __builtin_amdgcn_rcpf(scale) : 0.0f;
                    sc[e.half * 32 + k] = make_float4(mm.x, scale, inv, levels);
                    rec_lds[ct.w] = f2h_bits(scale) | (f2h_bits(mm.x) << 16);
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // pass 3: codes of the complete groups
            if (e.complete) {
                for (int k = 0; k < nc; ++k) {
                    const float4 s = sc[e.half * 32 + k];
                    const int4 ct = ctab[c0 + k];
                    const float x = lat[k * 64 + lane] - s.x;
                    float uq = 0.0f;
                    if (s.y > 0.0f) {
                        const float pq = x * s.z;
                        const float f = __builtin_amdgcn_fractf(pq);
                        uq = s.z == 0.0f || fabsf(f - 0.5f) <= 0x1p-11f ? rintf(x / s.y) : rintf(pq);
                        uq = uq < 0.0f ? 0.0f : (uq > s.w ? s.w : uq);
                    }
                    const int bit = ct.x + static_cast<int>(__umul24(e.t, ct.y));
                    // codes never straddle a word: a code of width w sits at a multiple of w
                    atomicOr(rec_lds + (bit >> 5), static_cast<uint32_t>(static_cast<int>(uq)) << (bit & 31));
                }
            }
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
        // the next pass reuses this wave's LDS buffers
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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
    const TensorDev &T = tz ? a.t[1] : a.t[0];
    const int r = T.r, W = T.words;
    const int grp = h / a.hpg;
    // The loads that do not depend on the row's stored length go out with
    // it, in one round trip: the token, the mean and this lane's basis row
    // (channel lane; a second pass takes channels from 64 on).  Every
    // address is valid whatever the length; an empty append discards them.
    const uint16_t *xin = a.x[tz] + (static_cast<int64_t>(bi) * a.H + h) * a.T_stride * kHeadDim;
    const uint32_t xp = reinterpret_cast<const uint32_t *>(xin)[lane];
    const float2 mu = reinterpret_cast<const float2 *>(T.mu + slot * T.set_mu + grp * kHeadDim)[lane];
    const float *bcm = T.basis_cm + slot * T.set_bcm + static_cast<int64_t>(grp) * r * kHeadDim;
    float4 vb[kHeadDim / 4];
    if (lane < r) {
        const float4 *row = reinterpret_cast<const float4 *>(bcm + static_cast<int64_t>(lane) * kHeadDim);
#pragma unroll
        for (int d4 = 0; d4 < kHeadDim / 4; ++d4) vb[d4] = row[d4];
    }
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
    const int64_t head_base = static_cast<int64_t>(slot) * a.H + h;
    const int j = o >> 5, t = o & 31;                 // group and position of the new token
    const bool complete = t == 31 && !T.fp16_latents;
    float *ys = ash;
    uint32_t *rec = reinterpret_cast<uint32_t *>(ash + kHeadDim);

    // 1. y = float(x) - mu, two elements per lane, to LDS; the record copy
    //    is cleared when the group completes
    reinterpret_cast<float2 *>(ys)[lane] = make_float2(in2f<BF16>(xp & 0xFFFFu) - mu.x, in2f<BF16>(xp >> 16) - mu.y);
    if (complete)
        for (int w = lane; w < W; w += kApp1Threads) rec[w] = 0u;
    __syncthreads();

    const float4 *ys4 = reinterpret_cast<const float4 *>(ys);
    const float *told = T.tail + (head_base * 2 + sel_old) * 32 * r;
    for (int c = lane; c < r; c += kApp1Threads) {
        // 2. the chain, with the channel's basis row in registers; when the
        //    group completes, its 31 older latents are loaded alongside
        if (c != lane) {
            const float4 *row = reinterpret_cast<const float4 *>(bcm + static_cast<int64_t>(c) * kHeadDim);
#pragma unroll
            for (int d4 = 0; d4 < kHeadDim / 4; ++d4) vb[d4] = row[d4];
        }
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

template <bool BF16, int REPS>
static hipError_t launch_encode_t(const EncodeArgs &a, int max_units, hipStream_t s) {
    // set once per process (thread-safe static initialisation)
    static const hipError_t attr =
        hipFuncSetAttribute(reinterpret_cast<const void *>(encode_kernel<BF16, REPS>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (attr != hipSuccess) return attr;
    const int l0 = encode_lds_bytes(a.t[0].r, a.t[0].words, a.t[0].fp16_latents),
              l1 = encode_lds_bytes(a.t[1].r, a.t[1].words, a.t[1].fp16_latents);
    constexpr int per_wg = kEncWaves * REPS;
    hipLaunchKernelGGL((encode_kernel<BF16, REPS>), dim3((max_units + per_wg - 1) / per_wg, a.B * a.H, 2), dim3(256),
                       static_cast<size_t>(l0 > l1 ? l0 : l1), s, a);
    return hipGetLastError();
}

hipError_t launch_encode(const EncodeArgs &a, int max_units, hipStream_t s) {
    // two group pairs per wave above rank 16 (either tensor)
    const bool wide = a.t[0].r > 16 || a.t[1].r > 16;
    if (a.bf16) return wide ? launch_encode_t<true, 2>(a, max_units, s) : launch_encode_t<true, 1>(a, max_units, s);
    return wide ? launch_encode_t<false, 2>(a, max_units, s) : launch_encode_t<false, 1>(a, max_units, s);
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
