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
// covers the incomplete group.  With the query absorbed into the key basis,
//   score_t = qs * (q . (V_K l_t + mu_K)) = sum_c qt_c l_tc + c0,
// where qt = qs V_K^T q and c0 = qs q . mu_K (qs = scale * log2 e, so the
// softmax uses exp2).  The workgroup keeps a running max m, denominator l
// and latent accumulator o_c = sum_t p_t lv_tc for each of its query heads.

__device__ __forceinline__ float wave_max(float v) {
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

__global__ __launch_bounds__(256) void attend_kernel(AttendArgs a) {
    const int wid = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int i = 0;
    while (i + 1 < a.B && a.work_prefix[i + 1] <= wid) ++i;
    const int rem = wid - a.work_prefix[i];
    const int ns = a.nsplit[i];
    const int h = rem / ns, s = rem - (rem / ns) * ns;
    const int slot = a.slot[i], len = a.len[i];
    const int nfull = len >> 5, ntail = len & 31;
    const int jb = s * a.chunk;
    const int je = jb + a.chunk < nfull ? jb + a.chunk : nfull;
    const bool do_tail = (s == ns - 1) && ntail > 0;
    const int g = a.gqa, grp = h / a.hpg;
    const int rk = a.k.r, rv = a.v.r, nhk = a.k.n_hi, nlk = a.k.r - a.k.n_hi;
    const int nhv = a.v.n_hi;

    __shared__ float qf[kMaxGqa][kHeadDim];
    __shared__ float qt[kMaxGqa][kHeadDim];
    __shared__ float c0s[kMaxGqa];
    __shared__ float sp[kMaxGqa][256];
    __shared__ float ot[kMaxGqa][kHeadDim];
    __shared__ float mst[kMaxGqa], lst[kMaxGqa], alp[kMaxGqa];
    __shared__ float red[4][kMaxGqa];

    for (int e = tid; e < g * kHeadDim; e += 256) {
        const int hh = e >> 7, d = e & 127;
        qf[hh][d] = h2f(a.q[(static_cast<int64_t>(i) * a.Hq + h * g + hh) * kHeadDim + d]);
        ot[hh][d] = 0.0f;
    }
    if (tid < g) {
        mst[tid] = -INFINITY;
        lst[tid] = 0.0f;
    }
    __syncthreads();
    const float *bk = a.k.basis + static_cast<int64_t>(grp) * kHeadDim * rk;
    for (int e = tid; e < g * rk; e += 256) {
        const int hh = e / rk, c = e - (e / rk) * rk;
        float acc = 0.0f;
        for (int d = 0; d < kHeadDim; ++d) acc = fmaf(qf[hh][d], bk[d * rk + c], acc);
        qt[hh][c] = acc * a.qscale;
    }
    for (int hh = tid; hh < g; hh += 256) {
        float acc = 0.0f;
        for (int d = 0; d < kHeadDim; ++d) acc = fmaf(qf[hh][d], a.k.mu[grp * kHeadDim + d], acc);
        c0s[hh] = acc * a.qscale;
    }
    __syncthreads();

    const int64_t hb = static_cast<int64_t>(slot) * a.Hkv + h;
    const uint32_t *krec0 = a.k.records + hb * a.k.head_stride;
    const uint32_t *vrec0 = a.v.records + hb * a.v.head_stride;
    const float *ktail = a.k.tail ? a.k.tail + (hb * 2 + a.sel[i]) * 32 * rk : nullptr;
    const float *vtail = a.v.tail ? a.v.tail + (hb * 2 + a.sel[i]) * 32 * rv : nullptr;

    const int ncoded = (je - jb + 7) >> 3;
    const int nblk = ncoded + (do_tail ? 1 : 0);
    for (int blk = 0; blk < nblk; ++blk) {
        const bool tb = blk == ncoded;
        const int p0 = tb ? 32 * nfull : 32 * (jb + 8 * blk);
        const int p1 = tb ? len : (32 * je < p0 + 256 ? 32 * je : p0 + 256);
        const int p = p0 + tid;
        const bool valid = p < p1;
        // scores
        if (valid) {
            float sc[kMaxGqa];
            for (int hh = 0; hh < kMaxGqa; ++hh) sc[hh] = hh < g ? c0s[hh] : 0.0f;
            if (!tb) {
                const uint32_t *rec = krec0 + static_cast<int64_t>(p >> 5) * a.k.words;
                const int t = p & 31;
                const uint32_t *meta = rec + 4 * nhk + 2 * nlk;
                for (int c = 0; c < rk; ++c) {
                    uint32_t code;
                    if (c < nhk) {
                        const int pos = t * 4 * nhk + 4 * c;
                        code = (rec[pos >> 5] >> (pos & 31)) & 15u;
                    } else {
                        const int pos = t * 2 * nlk + 2 * (c - nhk);
                        code = (rec[4 * nhk + (pos >> 5)] >> (pos & 31)) & 3u;
                    }
                    const uint32_t mw = meta[c];
                    const float l = fmaf(static_cast<float>(code), h2f(mw), h2f(mw >> 16));
                    for (int hh = 0; hh < kMaxGqa; ++hh)
                        if (hh < g) sc[hh] = fmaf(qt[hh][c], l, sc[hh]);
                }
            } else {
                const float *tl = ktail + (p & 31) * rk;
                for (int c = 0; c < rk; ++c) {
                    const float l = tl[c];
                    for (int hh = 0; hh < kMaxGqa; ++hh)
                        if (hh < g) sc[hh] = fmaf(qt[hh][c], l, sc[hh]);
                }
            }
            for (int hh = 0; hh < g; ++hh) sp[hh][tid] = sc[hh];
        }
        __syncthreads();
        for (int hh = 0; hh < g; ++hh) {
            const float m = wave_max(valid ? sp[hh][tid] : -INFINITY);
            if (lane == 0) red[wv][hh] = m;
        }
        __syncthreads();
        if (tid < g) {
            const float bm = fmaxf(fmaxf(red[0][tid], red[1][tid]), fmaxf(red[2][tid], red[3][tid]));
            const float mo = mst[tid];
            const float mn = fmaxf(mo, bm);
            alp[tid] = exp2f(mo - mn);
            mst[tid] = mn;
        }
        __syncthreads();
        for (int hh = 0; hh < g; ++hh) {
            const float pv = valid ? exp2f(sp[hh][tid] - mst[hh]) : 0.0f;
            if (valid) sp[hh][tid] = pv;
            const float sum = wave_sum(pv);
            if (lane == 0) red[wv][hh] = sum;
        }
        __syncthreads();
        if (tid < g) lst[tid] = lst[tid] * alp[tid] + (red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid]);
        // values
        for (int e = tid; e < g * rv; e += 256) {
            const int hh = e / rv, c = e - (e / rv) * rv;
            float acc = ot[hh][c] * alp[hh];
            if (!tb) {
                for (int jj = p0 >> 5; jj < (p1 + 31) >> 5; ++jj) {
                    const float *pr = &sp[hh][32 * jj - p0];
                    const uint32_t *rec = vrec0 + static_cast<int64_t>(jj) * a.v.words;
                    if (a.v.fp16_latents) {
                        const uint16_t *r16 = reinterpret_cast<const uint16_t *>(rec) + c * 32;
                        for (int t = 0; t < 32; ++t) acc = fmaf(pr[t], h2f(r16[t]), acc);
                    } else {
                        const uint32_t mw = rec[4 * nhv + 2 * (rv - nhv) + c];
                        float spc = 0.0f, sps = 0.0f;
                        if (c < nhv) {
                            for (int t = 0; t < 32; ++t) {
                                const uint32_t code = (rec[4 * c + (t >> 3)] >> (4 * (t & 7))) & 15u;
                                spc = fmaf(pr[t], static_cast<float>(code), spc);
                                sps += pr[t];
                            }
                        } else {
                            const int cl = c - nhv;
                            for (int t = 0; t < 32; ++t) {
                                const uint32_t code = (rec[4 * nhv + 2 * cl + (t >> 4)] >> (2 * (t & 15))) & 3u;
                                spc = fmaf(pr[t], static_cast<float>(code), spc);
                                sps += pr[t];
                            }
                        }
                        acc = fmaf(h2f(mw), spc, fmaf(h2f(mw >> 16), sps, acc));
                    }
                }
            } else {
                const int nt = p1 - p0;
                if (a.v.fp16_latents) {
                    const uint16_t *r16 = reinterpret_cast<const uint16_t *>(
                        vrec0 + static_cast<int64_t>(nfull) * a.v.words) + c * 32;
                    for (int t = 0; t < nt; ++t) acc = fmaf(sp[hh][t], h2f(r16[t]), acc);
                } else {
                    for (int t = 0; t < nt; ++t) acc = fmaf(sp[hh][t], vtail[t * rv + c], acc);
                }
            }
            ot[hh][c] = acc;
        }
        __syncthreads();
    }

    // partials: [i][q head][split][m, l, o_0 .. o_{rv-1}]
    for (int e = tid; e < g * (rv + 2); e += 256) {
        const int hh = e / (rv + 2), k = e - (e / (rv + 2)) * (rv + 2);
        float *part = a.partial +
            ((static_cast<int64_t>(i) * a.Hq + h * g + hh) * kMaxSplits + s) * (rv + 2);
        part[k] = k == 0 ? mst[hh] : (k == 1 ? lst[hh] : ot[hh][k - 2]);
    }
}

__global__ __launch_bounds__(128) void combine_kernel(AttendArgs a) {
    const int i = blockIdx.x / a.Hq, qh = blockIdx.x - (blockIdx.x / a.Hq) * a.Hq;
    const int h = qh / a.gqa, grp = h / a.hpg, ns = a.nsplit[i], rv = a.v.r;
    const int tid = threadIdx.x;
    const float *part = a.partial + (static_cast<int64_t>(i) * a.Hq + qh) * kMaxSplits * (rv + 2);
    __shared__ float wsp[kMaxSplits];
    __shared__ float ov[kHeadDim];
    __shared__ float ltot;
    if (tid == 0) {
        float m = -INFINITY;
        for (int s = 0; s < ns; ++s) m = fmaxf(m, part[s * (rv + 2)]);
        float l = 0.0f;
        for (int s = 0; s < ns; ++s) {
            const float w = exp2f(part[s * (rv + 2)] - m);
            wsp[s] = w;
            l = fmaf(w, part[s * (rv + 2) + 1], l);
        }
        ltot = l;
    }
    __syncthreads();
    for (int c = tid; c < rv; c += 128) {
        float acc = 0.0f;
        for (int s = 0; s < ns; ++s) acc = fmaf(wsp[s], part[s * (rv + 2) + 2 + c], acc);
        ov[c] = acc / ltot;
    }
    __syncthreads();
    const float *bv = a.v.basis + static_cast<int64_t>(grp) * kHeadDim * rv;
    float o = a.v.mu[grp * kHeadDim + tid];
    for (int c = 0; c < rv; ++c) o = fmaf(bv[tid * rv + c], ov[c], o);
    a.out[(static_cast<int64_t>(i) * a.Hq + qh) * kHeadDim + tid] = static_cast<uint16_t>(f2h_bits(o));
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

hipError_t launch_attend(const AttendArgs &a, int n_work, hipStream_t s) {
    hipLaunchKernelGGL(attend_kernel, dim3(n_work), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_combine(const AttendArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(combine_kernel, dim3(a.B * a.Hq), dim3(128), 0, s, a);
    return hipGetLastError();
}

}  // namespace palu
