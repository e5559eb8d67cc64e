// Device helpers shared by the HIP kernel sources of libpalu.so: vector
// types, fp16 conversions, lane exchanges inside a 64-lane wave, the fp16
// dequantisation of packed codes and exact small integer division.  Each
// source that includes this gets its own internal copy (anonymous
// namespace); nothing here is part of the C ABI.
#pragma once

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

// bf16 bits (low 16 bits of the argument) -> float, exact.
__device__ __forceinline__ float bf2f(uint32_t bits) { return __uint_as_float(bits << 16); }

// An input element (fp16 or bf16 bits in the low half) -> float, exact.
template <bool BF16>
__device__ __forceinline__ float in2f(uint32_t bits) {
    if constexpr (BF16) return bf2f(bits & 0xFFFFu);
    else return __half2float(__ushort_as_half(static_cast<unsigned short>(bits & 0xFFFFu)));
}
// The high half of a 32-bit pair of inputs -> float.
template <bool BF16>
__device__ __forceinline__ float in2f_hi(uint32_t pair) {
    if constexpr (BF16) return __uint_as_float(pair & 0xFFFF0000u);
    else return __half2float(__ushort_as_half(static_cast<unsigned short>(pair >> 16)));
}

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f2bf_bits(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// An output element in the input type (fp16 or bf16), round to nearest even.
__device__ __forceinline__ uint32_t out_bits(float f, bool bf16) { return bf16 ? f2bf_bits(f) : f2h_bits(f); }

// Lane exchange inside rows of 16 lanes through DPP (no LDS round trip).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E;            // quad_perm [1,0,3,2], [2,3,0,1]
constexpr int kDppHalfMirror = 0x141, kDppMirror = 0x140;  // lane i <- 7-i (per 8), 15-i

// Every lane of a 16-lane row gets the row's max / sum: pairs, quads, then
// the mirrored halves of 8 and of 16 lanes.
__device__ __forceinline__ float row_max(float v) {
    v = fmaxf(v, dpp<kDppXor1>(v));
    v = fmaxf(v, dpp<kDppXor2>(v));
    v = fmaxf(v, dpp<kDppHalfMirror>(v));
    return fmaxf(v, dpp<kDppMirror>(v));
}
__device__ __forceinline__ float row_sum(float v) {
    v += dpp<kDppXor1>(v);
    v += dpp<kDppXor2>(v);
    v += dpp<kDppHalfMirror>(v);
    return v + dpp<kDppMirror>(v);
}
__device__ __forceinline__ float lane_value(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Whole-wave max / sum, the same (wave-uniform) value in every lane.
__device__ __forceinline__ float wave_max(float v) {
    v = row_max(v);
    return fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)), fmaxf(lane_value(v, 32), lane_value(v, 48)));
}
__device__ __forceinline__ float wave_sum(float v) {
    v = row_sum(v);
    return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

// floor(e / d) for 0 <= e < 2^21 and d >= 1 from a correctly rounded fp32
// reciprocal: (e + 1/2) / d lies at least 1/(2d) away from an integer, and
// the two roundings perturb it by at most (e + 1/2) / d * 2^-23 < 1/(2d).
struct FastDiv {
    float inv;   // the correctly rounded fp32 1 / d
    __device__ explicit FastDiv(float inv_d) : inv(inv_d) {}
    __device__ int quo(int e) const { return static_cast<int>((static_cast<float>(e) + 0.5f) * inv); }
};

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));

// bf16 query rows for an fp16 MFMA: the 32 elements a lane holds (4 x 8
// bf16 in qa) of a row spread over the 4 lanes ln, ln + 16, ln + 32, ln + 48
// are scaled by 2^-k, with k chosen per row so that the row's largest
// magnitude lands in [2^14, 2^15), and rounded to fp16.  bf16 carries 8
// significand bits, so every element that stays in the fp16 normal range
// converts exactly; elements more than 2^28 below the row maximum may round
// (fp16 subnormals), far below what any dot product resolves.  Returns k;
// qa is rewritten in place as fp16.
__device__ __forceinline__ int bf16_rows_to_fp16(uint4 (&qa)[4]) {
    uint32_t emax = 0;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        const uint32_t w[4] = {qa[st].x, qa[st].y, qa[st].z, qa[st].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t e0 = w[i] & 0x7F80u, e1 = (w[i] >> 16) & 0x7F80u;
            emax = emax > e0 ? emax : e0;
            emax = emax > e1 ? emax : e1;
        }
    }
    uint32_t o = __shfl_xor(emax, 16);
    emax = emax > o ? emax : o;
    o = __shfl_xor(emax, 32);
    emax = emax > o ? emax : o;
    // |x| < 2^(E - 126) with E the biased exponent: scale by 2^-(E - 141)
    const int E = static_cast<int>(emax >> 7);
    int k = E == 0 ? 0 : E - 141;
    k = k < -100 ? -100 : (k > 100 ? 100 : k);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        uint32_t w[4] = {qa[st].x, qa[st].y, qa[st].z, qa[st].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float lo = ldexpf(bf2f(w[i] & 0xFFFFu), -k), hi = ldexpf(__uint_as_float(w[i] & 0xFFFF0000u), -k);
            w[i] = f2h_bits(lo) | (f2h_bits(hi) << 16);
        }
        qa[st] = make_uint4(w[0], w[1], w[2], w[3]);
    }
    return k;
}

// ---- segment coder lookups (see Coder).  Select chains over the fixed
//      8-entry arrays: no dynamic indexing of kernel arguments.
template <int N>
__device__ __forceinline__ int pick(const int (&v)[N], int s) {
    int r = v[0];
#pragma unroll
    for (int k = 1; k < N; ++k) r = s == k ? v[k] : r;
    return r;
}
// segment holding channel c / 8-channel block q
__device__ __forceinline__ int seg_of_channel(const Coder &cd, int c) {
    int s = 0;
#pragma unroll
    for (int k = 1; k < kMaxSegs; ++k) s += (k < cd.nseg && c >= cd.c0[k]) ? 1 : 0;
    return s;
}
__device__ __forceinline__ int seg_of_block(const Coder &cd, int q) {
    int s = 0;
#pragma unroll
    for (int k = 1; k < kMaxSegs; ++k) s += (k < cd.nseg && q >= cd.q0[k]) ? 1 : 0;
    return s;
}

// Key-record addressing of 8-channel block q (token-major planes): the
// block's codes of token t start at bit base + t * stride, channel k of the
// block at bit w * k after that; channels [chan0, chanend) are real.
struct KBlock {
    int base, stride, w, chan0, chanend;
};
__device__ __forceinline__ KBlock key_block(const Coder &cd, int q) {
    const int s = seg_of_block(cd, q);
    const int c0 = pick(cd.c0, s), c1 = pick(cd.c0, s + 1), w = pick(cd.bits, s), qq = q - pick(cd.q0, s);
    KBlock b;
    b.base = 32 * pick(cd.plane0, s) + 8 * qq * w;
    b.stride = w * (c1 - c0);
    b.w = w;
    b.chan0 = c0 + 8 * qq;
    b.chanend = c1;
    return b;
}
// Value-record addressing of channel c (channel-major planes): token t's
// code at bit base + w * t.
__device__ __forceinline__ int2 value_channel(const Coder &cd, int c) {
    const int s = seg_of_channel(cd, c);
    const int w = pick(cd.bits, s);
    return make_int2(32 * pick(cd.plane0, s) + 32 * w * (c - pick(cd.c0, s)), w);
}
// Bit of (token t, channel c) in a record of either layout (0 = K, 1 = V),
// and the channel's width.
__device__ __forceinline__ int2 code_bit(const Coder &cd, int layout, int c, int t) {
    const int s = seg_of_channel(cd, c);
    const int w = pick(cd.bits, s), c0 = pick(cd.c0, s), n = pick(cd.c0, s + 1) - c0;
    const int p = 32 * pick(cd.plane0, s);
    return make_int2(layout == 0 ? p + t * w * n + w * (c - c0) : p + 32 * w * (c - c0) + w * t, w);
}

// Bump allocator for a workgroup's dynamic LDS (16-byte aligned pieces).
__host__ __device__ inline int lds_take(int &o, int bytes) {
    const int r = o;
    o += (bytes + 15) & ~15;
    return r;
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

[[maybe_unused]] __device__ __forceinline__ uint32_t pack_half2(float a, float b) {
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

// 8 codes of one token from a 32-bit window -> fp16 pairs 1024 + code
// (channel k, channel k + 4), k = 0..3, exact.
template <bool W4>
__device__ __forceinline__ f16x8 codes8(uint32_t X, uint32_t cm, uint32_t magic) {
    const uint32_t U = W4 ? X : perm_b32(X, X, 0x0C010C00u);
    constexpr int wc = W4 ? 4 : 2;
    return as_h8((U & cm) | magic, ((U >> wc) & cm) | magic, ((U >> (2 * wc)) & cm) | magic,
                 ((U >> (3 * wc)) & cm) | magic);
}

__device__ __forceinline__ f16x8 codes8_any(uint32_t X, bool w4) {
    const uint32_t U = w4 ? X : perm_b32(X, X, 0x0C010C00u);
    const int wc = w4 ? 4 : 2;
    const uint32_t cm = w4 ? 0x000F000Fu : 0x00030003u;
    return as_h8((U & cm) | 0x64006400u, ((U >> wc) & cm) | 0x64006400u, ((U >> (2 * wc)) & cm) | 0x64006400u,
                 ((U >> (3 * wc)) & cm) | 0x64006400u);
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

// 8 codes of width w (1, 2, 4 or 8) of one token: channel k at bit w * k of
// the 64-bit window X1:X0 -> dequantised fp16 pairs (channel k, k + 4).
__device__ __forceinline__ f16x8 dequant8_w(uint32_t X0, uint32_t X1, int w, const uint4 &sp, const uint4 &zp) {
    constexpr uint32_t magic = 0x64006400u;
    if (w == 8) {
        // pair k: byte k of X0 (channel k) and byte k of X1 (channel k + 4)
        return as_h8(dequant_pair(perm_b32(X1, X0, 0x0C040C00u) | magic, sp.x, zp.x),
                     dequant_pair(perm_b32(X1, X0, 0x0C050C01u) | magic, sp.y, zp.y),
                     dequant_pair(perm_b32(X1, X0, 0x0C060C02u) | magic, sp.z, zp.z),
                     dequant_pair(perm_b32(X1, X0, 0x0C070C03u) | magic, sp.w, zp.w));
    }
    if (w == 1) {
        // channels 4..7 (bits 4..7) up to bits 16..19
        const uint32_t U = (X0 & 0x0Fu) | ((X0 & 0xF0u) << 12);
        return as_h8(dequant_pair((U & 0x00010001u) | magic, sp.x, zp.x),
                     dequant_pair(((U >> 1) & 0x00010001u) | magic, sp.y, zp.y),
                     dequant_pair(((U >> 2) & 0x00010001u) | magic, sp.z, zp.z),
                     dequant_pair(((U >> 3) & 0x00010001u) | magic, sp.w, zp.w));
    }
    return dequant8_any(X0, w == 4, sp, zp);
}

}  // namespace
}  // namespace palu
