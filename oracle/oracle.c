/*
 * Plain CPU oracle for the PALU-style low-rank latent KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke entry and the benchmark's
 * CPU-baseline leg may load this library.  The product path never calls it,
 * and it shares no code, header, table or helper with the HIP library.
 *
 * What it computes, step by step, in the order of the PALU page
 * (veloxquant-mlx docs, "PALU", section "How it works"):
 *   fit      : per head group, stack the group's heads along the token axis,
 *              centre by the fp64 mean, eigendecompose the fp64 scatter
 *              matrix by cyclic Jacobi, sort descending, choose the rank by
 *              an explicit value or by the singular-value-energy rule, and
 *              take the minimum rank over groups.
 *   encode   : L = (x - mu_g) V_g as a fixed-order fp32 fused multiply-add
 *              chain over d = 0..D-1 (the operation order the GPU reproduces).
 *   quantise : asymmetric min/max round-to-nearest per channel over groups of
 *              32 tokens (quantiser of the "KIVI 0.8.0" blog post, section
 *              "What KIVI is"), top channels by singular value at hi_bit,
 *              the rest at lo_bit (PALU page, "Usage" and "How it works").
 *   pack     : LSB-first sub-byte packing (VeloxQuant blog post, section
 *              "The Bit-Packing Problem") in the record layout below.
 *   attend   : reconstruct K/V = l_hat V_g^T + mu_g in fp64 and run plain
 *              single-query softmax attention over every stored token.
 *   prefill  : reconstruct K/V of every stored token the same way, then
 *              causal softmax attention of each prefill query over the
 *              tokens up to and including its own position (prefill step 6:
 *              the reconstruction feeds the downstream attention call).
 *
 * Record layout (one record per sequence, kv head, tensor and complete
 * 32-token group; 32-bit little-endian words):
 *   K records (token-major planes)
 *     hi plane, 4*n_hi words : code of token t, channel c < n_hi sits at bit
 *                              t*4*n_hi + 4*c of the plane
 *     lo plane, 2*n_lo words : code of token t, channel n_hi + c' sits at bit
 *                              t*2*n_lo + 2*c' of the plane
 *   V records (channel-major planes)
 *     hi plane, 4*n_hi words : channel c, token t at bit 128*c + 4*t
 *     lo plane, 2*n_lo words : channel n_hi + c', token t at bit 64*c' + 2*t
 *   both, then r meta words  : word c = scale16[c] | zero16[c] << 16
 *   fp16 value latents       : record = r*32 halves, channel-major (c*32 + t)
 * A group that is not yet complete is kept as fp32 latents (the "tail").
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16 conversion, written from the format definition          */
/* ------------------------------------------------------------------------ */

float orc_half_to_float(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    float v;
    if (e == 0)
        v = ldexpf((float)m, -24);               /* zero / subnormal */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexpf((float)(m | 0x400), e - 25);  /* 1.m * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16 bits -> float: the 16 bits are the high half of the binary32
 * pattern, so the widening is exact. */
float orc_bf16_to_float(uint16_t b)
{
    union {
        uint32_t u;
        float f;
    } v;
    v.u = (uint32_t)b << 16;
    return v.f;
}

/* An input element (K, V or q) in its storage format: fmt 0 = fp16,
 * fmt 1 = bf16; both widen to float exactly. */
static float orc_in_to_float(uint16_t v, int fmt)
{
    return fmt ? orc_bf16_to_float(v) : orc_half_to_float(v);
}

void orc_bf16_to_float_n(const uint16_t *b, float *f, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        f[i] = orc_bf16_to_float(b[i]);
}

/* Round-to-nearest-even conversion float -> binary16. */
uint16_t orc_float_to_half(float f)
{
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    double a = fabs((double)f);
    if (isnan(f))
        return (uint16_t)(sign | 0x7e00);
    if (isinf(f))
        return (uint16_t)(sign | 0x7c00);
    if (a < ldexp(1.0, -14)) {
        /* subnormal grid: multiples of 2^-24 (a result of 1024 is the
         * smallest normal number, whose encoding is the same integer) */
        double q = nearbyint(a * 16777216.0);
        return (uint16_t)(sign | (uint16_t)q);
    }
    int e;
    frexp(a, &e);                      /* a in [2^(e-1), 2^e) */
    double q = nearbyint(ldexp(a, 11 - e));   /* significand in [1024, 2048] */
    int E = e - 1 + 15;
    if (q == 2048.0) {
        q = 1024.0;
        E += 1;
    }
    if (E >= 31)
        return (uint16_t)(sign | 0x7c00);
    return (uint16_t)(sign | (E << 10) | ((int)q - 1024));
}

void orc_half_to_float_n(const uint16_t *h, float *f, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        f[i] = orc_half_to_float(h[i]);
}

void orc_float_to_half_n(const float *f, uint16_t *h, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        h[i] = orc_float_to_half(f[i]);
}

/* ------------------------------------------------------------------------ */
/* Symmetric eigensolver: cyclic Jacobi (Golub & Van Loan, "Matrix           */
/* Computations", the symmetric Schur decomposition and cyclic Jacobi).     */
/* a: n x n row-major, destroyed (diagonal = eigenvalues on return).        */
/* v: n x n row-major, columns = eigenvectors.                              */
/* ------------------------------------------------------------------------ */

static void jacobi_eigen(double *a, double *v, int n)
{
    for (int i = 0; i < n; i++)
        for (int j = 0; j < n; j++)
            v[i * n + j] = (i == j) ? 1.0 : 0.0;

    double frob = 0.0;
    for (int i = 0; i < n * n; i++)
        frob += a[i] * a[i];
    if (frob == 0.0)
        return;

    for (int sweep = 0; sweep < 100; sweep++) {
        double off = 0.0;
        for (int p = 0; p < n; p++)
            for (int q = p + 1; q < n; q++)
                off += a[p * n + q] * a[p * n + q];
        if (off <= 1e-30 * frob)
            break;
        for (int p = 0; p < n - 1; p++) {
            for (int q = p + 1; q < n; q++) {
                double apq = a[p * n + q];
                if (apq == 0.0)
                    continue;
                /* rotation that annihilates a[p][q] */
                double theta = (a[q * n + q] - a[p * n + p]) / (2.0 * apq);
                double t = (theta >= 0 ? 1.0 : -1.0) /
                           (fabs(theta) + sqrt(theta * theta + 1.0));
                double c = 1.0 / sqrt(t * t + 1.0);
                double s = t * c;
                /* A <- J^T A J with J the (p,q) rotation */
                for (int k = 0; k < n; k++) {
                    double akp = a[k * n + p], akq = a[k * n + q];
                    a[k * n + p] = c * akp - s * akq;
                    a[k * n + q] = s * akp + c * akq;
                }
                for (int k = 0; k < n; k++) {
                    double apk = a[p * n + k], aqk = a[q * n + k];
                    a[p * n + k] = c * apk - s * aqk;
                    a[q * n + k] = s * apk + c * aqk;
                }
                for (int k = 0; k < n; k++) {
                    double vkp = v[k * n + p], vkq = v[k * n + q];
                    v[k * n + p] = c * vkp - s * vkq;
                    v[k * n + q] = s * vkp + c * vkq;
                }
            }
        }
    }
}

/* Energy rule: smallest k >= 1 with sum_{i<k} s2[i] >= tau * sum_i s2[i]
 * (s2 = squared singular values, descending, non-negative).  Energy is the
 * sum of squared singular values.  Zero total energy gives rank 1. */
int orc_energy_rank(const double *s2, int n, double tau)
{
    double total = 0.0;
    for (int i = 0; i < n; i++)
        total += s2[i];
    if (total <= 0.0)
        return 1;
    double acc = 0.0;
    for (int k = 1; k <= n; k++) {
        acc += s2[k - 1];
        if (acc >= tau * total)
            return k;
    }
    return n;
}

/*
 * Group-head fit of one head group (PALU page, "How it works", prefill
 * steps 1-2).
 *   x      : fp16 (fmt 0) or bf16 (fmt 1) [B][H][S_stride][D]; group g owns
 *            heads [g*H/G, (g+1)*H/G)
 *   lens   : valid tokens per sequence
 *   rank   : > 0 explicit rank (clamped to D), 0 -> energy rule with tau
 * Outputs (every column of the sorted eigenbasis is returned; the rank picks
 * the leading ones):
 *   basis  : fp32 [D][D], basis[d][c] = component d of direction c
 *   mu     : fp32 [D]
 *   sigma  : fp64 [D] singular values of the centred stack, descending
 * Returns the group's rank, or -1 on bad arguments.
 */
int orc_fit_group(const uint16_t *x, const int32_t *lens, int B, int H,
                  int S_stride, int D, int G, int g, int rank, double tau,
                  float *basis, float *mu, double *sigma, int fmt)
{
    if (B <= 0 || H <= 0 || D <= 0 || G <= 0 || H % G != 0 || g < 0 || g >= G)
        return -1;
    int hpg = H / G;
    double *mean = malloc(sizeof(double) * D);
    double *cov = malloc(sizeof(double) * D * D);
    double *vec = malloc(sizeof(double) * D * D);
    double *row = malloc(sizeof(double) * D);
    int *order = malloc(sizeof(int) * D);
    double *s2 = malloc(sizeof(double) * D);

    /* pass 1: mean of all valid rows of the group's heads */
    int64_t N = 0;
    for (int d = 0; d < D; d++)
        mean[d] = 0.0;
    for (int b = 0; b < B; b++)
        for (int h = g * hpg; h < (g + 1) * hpg; h++)
            for (int t = 0; t < lens[b]; t++) {
                const uint16_t *xr = x + (((int64_t)b * H + h) * S_stride + t) * D;
                for (int d = 0; d < D; d++)
                    mean[d] += (double)orc_in_to_float(xr[d], fmt);
                N++;
            }
    for (int d = 0; d < D; d++)
        mean[d] = N ? mean[d] / (double)N : 0.0;

    /* pass 2: scatter matrix of the centred rows (upper triangle, mirrored) */
    for (int i = 0; i < D * D; i++)
        cov[i] = 0.0;
    for (int b = 0; b < B; b++)
        for (int h = g * hpg; h < (g + 1) * hpg; h++)
            for (int t = 0; t < lens[b]; t++) {
                const uint16_t *xr = x + (((int64_t)b * H + h) * S_stride + t) * D;
                for (int d = 0; d < D; d++)
                    row[d] = (double)orc_in_to_float(xr[d], fmt) - mean[d];
                for (int i = 0; i < D; i++)
                    for (int j = i; j < D; j++)
                        cov[i * D + j] += row[i] * row[j];
            }
    for (int i = 0; i < D; i++)
        for (int j = 0; j < i; j++)
            cov[i * D + j] = cov[j * D + i];

    jacobi_eigen(cov, vec, D);

    /* sort eigenpairs by eigenvalue, descending (stable on ties) */
    for (int i = 0; i < D; i++)
        order[i] = i;
    for (int i = 1; i < D; i++) {
        int key = order[i];
        int j = i - 1;
        while (j >= 0 && cov[order[j] * D + order[j]] < cov[key * D + key]) {
            order[j + 1] = order[j];
            j--;
        }
        order[j + 1] = key;
    }
    for (int c = 0; c < D; c++) {
        int src = order[c];
        double lam = cov[src * D + src];
        s2[c] = lam > 0.0 ? lam : 0.0;
        sigma[c] = sqrt(s2[c]);
        /* sign: the entry of largest magnitude is positive (lowest index
         * wins a tie) */
        int arg = 0;
        for (int d = 1; d < D; d++)
            if (fabs(vec[d * D + src]) > fabs(vec[arg * D + src]))
                arg = d;
        double sgn = vec[arg * D + src] < 0.0 ? -1.0 : 1.0;
        for (int d = 0; d < D; d++)
            basis[(int64_t)d * D + c] = (float)(sgn * vec[d * D + src]);
    }
    for (int d = 0; d < D; d++)
        mu[d] = (float)mean[d];

    int r;
    if (rank > 0)
        r = rank < D ? rank : D;
    else
        r = orc_energy_rank(s2, D, tau);
    free(mean);
    free(cov);
    free(vec);
    free(row);
    free(order);
    free(s2);
    return r;
}

/* All groups; the shared rank is the minimum over groups (PALU page, "How it
 * works", prefill step 3).  basis [G][D][D], mu [G][D], sigma [G][D],
 * rg [G] = per-group ranks.  Returns the shared rank or -1. */
int orc_fit(const uint16_t *x, const int32_t *lens, int B, int H, int S_stride,
            int D, int G, int rank, double tau, float *basis, float *mu,
            double *sigma, int32_t *rg, int fmt)
{
    int shared = -1;
    for (int g = 0; g < G; g++) {
        int r = orc_fit_group(x, lens, B, H, S_stride, D, G, g, rank, tau,
                              basis + (int64_t)g * D * D, mu + (int64_t)g * D,
                              sigma + (int64_t)g * D, fmt);
        if (r < 0)
            return -1;
        rg[g] = r;
        if (shared < 0 || r < shared)
            shared = r;
    }
    return shared;
}

/* ------------------------------------------------------------------------ */
/* Projection: l_c = fma chain over d of (float(x_d) - mu_d) * V[d][c]       */
/* x: fp16 or bf16 [n][D] (fmt); V: fp32 [D][ldv] (first r columns used);     */
/* out [n][r]                                                                */
/* ------------------------------------------------------------------------ */

void orc_project(const uint16_t *x, int64_t n, int D, const float *mu,
                 const float *V, int ldv, int r, float *out, int fmt)
{
    for (int64_t i = 0; i < n; i++) {
        for (int c = 0; c < r; c++) {
            float acc = 0.0f;
            for (int d = 0; d < D; d++) {
                float y = orc_in_to_float(x[i * D + d], fmt) - mu[d];
                acc = fmaf(y, V[(int64_t)d * ldv + c], acc);
            }
            out[i * r + c] = acc;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Quantiser: one 32-token group, every channel.                             */
/*   zero = min, scale = (max - min) / (2^b - 1), q = round((l - zero)/scale) */
/* fp32 throughout, IEEE division, round-half-to-even, q clamped to the       */
/* code range; a constant channel (scale 0) gets code 0.                     */
/* l: fp32 [32][r]; codes: [32][r]; scale16/zero16: fp16 bits [r]            */
/* ------------------------------------------------------------------------ */

/*
 * The coder works on segments: contiguous ranges of latent channels in
 * descending-singular-value order, segment s holding seg_n[s] channels coded
 * with seg_bits[s] bits (0, 1, 2, 4 or 8).  PALU's split (PALU page,
 * "Usage": the top hi_fraction of channels at hi_bit, the rest at lo_bit) is
 * the two-segment case; the SVDq cache page's bit schedule (section on the
 * SVDq cache: r channels split into len(schedule) equal contiguous groups,
 * 0 bits truncating a group to exactly zero) is the general one.  A 0-bit
 * channel is not stored in any form: no codes, no metadata, no tail entry;
 * its latent is exactly 0.
 */
static int seg_of(int c, int nseg, const int *seg_n, int *c0)
{
    int start = 0;
    for (int s = 0; s < nseg; s++) {
        if (c < start + seg_n[s]) {
            *c0 = start;
            return s;
        }
        start += seg_n[s];
    }
    *c0 = start;
    return nseg;
}

/* channels with a nonzero bit width */
int orc_coded_channels(int nseg, const int *seg_n, const int *seg_bits)
{
    int n = 0;
    for (int s = 0; s < nseg; s++)
        if (seg_bits[s] > 0)
            n += seg_n[s];
    return n;
}

/* words of one record: a code plane of seg_n * seg_bits words per coded
 * segment (32 tokens), then one metadata word per coded channel */
int orc_record_words_seg(int nseg, const int *seg_n, const int *seg_bits)
{
    int w = 0;
    for (int s = 0; s < nseg; s++)
        w += seg_n[s] * seg_bits[s];
    return w + orc_coded_channels(nseg, seg_n, seg_bits);
}

void orc_quantize_group_seg(const float *l, int r, int nseg, const int *seg_n,
                            const int *seg_bits, uint8_t *codes,
                            uint16_t *scale16, uint16_t *zero16)
{
    for (int c = 0; c < r; c++) {
        int c0;
        int s = seg_of(c, nseg, seg_n, &c0);
        int bits = s < nseg ? seg_bits[s] : 0;
        if (bits == 0) {
            for (int t = 0; t < 32; t++)
                codes[t * r + c] = 0;
            scale16[c] = 0;
            zero16[c] = 0;
            continue;
        }
        int levels = (1 << bits) - 1;
        float mn = l[c], mx = l[c];
        for (int t = 1; t < 32; t++) {
            float v = l[t * r + c];
            if (v < mn) mn = v;
            if (v > mx) mx = v;
        }
        float scale = (mx - mn) / (float)levels;
        for (int t = 0; t < 32; t++) {
            int q = 0;
            if (scale > 0.0f) {
                float u = rintf((l[t * r + c] - mn) / scale);
                if (u < 0.0f) u = 0.0f;
                if (u > (float)levels) u = (float)levels;
                q = (int)u;
            }
            codes[t * r + c] = (uint8_t)q;
        }
        scale16[c] = orc_float_to_half(scale);
        zero16[c] = orc_float_to_half(mn);
    }
}

static void put_bits(uint32_t *w, int64_t bitpos, uint32_t val)
{
    w[bitpos >> 5] |= val << (bitpos & 31);
}

static uint32_t get_bits(const uint32_t *w, int64_t bitpos, int width)
{
    return (w[bitpos >> 5] >> (bitpos & 31)) & ((1u << width) - 1u);
}

/* Bit of (token t, channel c) inside its segment's plane.  layout 0 = K
 * (token-major: t * bits * n + bits * c'), 1 = V (channel-major:
 * 32 * bits * c' + bits * t), c' = channel index inside the segment. */
static int64_t code_bit(int layout, int t, int cc, int bits, int n)
{
    return layout == 0 ? (int64_t)t * bits * n + (int64_t)bits * cc
                       : (int64_t)32 * bits * cc + (int64_t)bits * t;
}

void orc_pack_group_seg(const uint8_t *codes, const uint16_t *scale16,
                        const uint16_t *zero16, int r, int nseg,
                        const int *seg_n, const int *seg_bits, int layout,
                        uint32_t *rec)
{
    int words = orc_record_words_seg(nseg, seg_n, seg_bits);
    memset(rec, 0, sizeof(uint32_t) * words);
    int plane = 0, c0 = 0, m = 0;
    int meta0 = words - orc_coded_channels(nseg, seg_n, seg_bits);
    for (int s = 0; s < nseg; s++) {
        int n = seg_n[s], bits = seg_bits[s];
        if (bits > 0) {
            for (int t = 0; t < 32; t++)
                for (int cc = 0; cc < n; cc++)
                    put_bits(rec + plane, code_bit(layout, t, cc, bits, n),
                             codes[t * r + c0 + cc]);
            for (int cc = 0; cc < n; cc++, m++)
                rec[meta0 + m] = (uint32_t)scale16[c0 + cc] | ((uint32_t)zero16[c0 + cc] << 16);
        }
        plane += n * bits;
        c0 += n;
    }
    (void)r;
}

void orc_unpack_group_seg(const uint32_t *rec, int r, int nseg, const int *seg_n,
                          const int *seg_bits, int layout, uint8_t *codes,
                          uint16_t *scale16, uint16_t *zero16)
{
    int words = orc_record_words_seg(nseg, seg_n, seg_bits);
    int meta0 = words - orc_coded_channels(nseg, seg_n, seg_bits);
    int plane = 0, c0 = 0, m = 0;
    for (int s = 0; s < nseg; s++) {
        int n = seg_n[s], bits = seg_bits[s];
        for (int cc = 0; cc < n; cc++) {
            int c = c0 + cc;
            if (bits > 0) {
                for (int t = 0; t < 32; t++)
                    codes[t * r + c] = (uint8_t)get_bits(rec + plane, code_bit(layout, t, cc, bits, n), bits);
                scale16[c] = (uint16_t)(rec[meta0 + m] & 0xffff);
                zero16[c] = (uint16_t)(rec[meta0 + m] >> 16);
                m++;
            } else {
                for (int t = 0; t < 32; t++)
                    codes[t * r + c] = 0;
                scale16[c] = 0;
                zero16[c] = 0;
            }
        }
        plane += n * bits;
        c0 += n;
    }
}

/*
 * Encode a stream of n latents [n][r] (token order) of one (sequence, head,
 * tensor): complete 32-token groups are quantised and packed into records;
 * the last n % 32 latents of the coded channels (in channel order) are
 * copied to the fp32 tail [n % 32][coded channels].
 */
void orc_encode_stream_seg(const float *lat, int64_t n, int r, int nseg,
                           const int *seg_n, const int *seg_bits, int layout,
                           uint32_t *records, float *tail)
{
    int words = orc_record_words_seg(nseg, seg_n, seg_bits);
    int rc = orc_coded_channels(nseg, seg_n, seg_bits);
    int64_t full = n / 32;
    uint8_t *codes = malloc((size_t)32 * (r > 0 ? r : 1));
    uint16_t *sc = malloc(sizeof(uint16_t) * (r > 0 ? r : 1)), *zr = malloc(sizeof(uint16_t) * (r > 0 ? r : 1));
    for (int64_t j = 0; j < full; j++) {
        orc_quantize_group_seg(lat + j * 32 * r, r, nseg, seg_n, seg_bits, codes, sc, zr);
        orc_pack_group_seg(codes, sc, zr, r, nseg, seg_n, seg_bits, layout, records + j * words);
    }
    for (int64_t i = full * 32; i < n; i++) {
        int k = 0;
        for (int c = 0; c < r; c++) {
            int c0;
            int s = seg_of(c, nseg, seg_n, &c0);
            if (s < nseg && seg_bits[s] > 0)
                tail[(i - full * 32) * rc + k++] = lat[i * r + c];
        }
    }
    free(codes);
    free(sc);
    free(zr);
}

/* Dequantised latents (fp64) [n][r] of n tokens: complete groups from
 * records, l_hat = code * scale16 + zero16 evaluated exactly in fp64; the
 * remaining n % 32 from the fp32 tail; 0-bit channels are 0. */
void orc_decode_stream_seg(const uint32_t *records, const float *tail, int64_t n,
                           int r, int nseg, const int *seg_n, const int *seg_bits,
                           int layout, double *out)
{
    int words = orc_record_words_seg(nseg, seg_n, seg_bits);
    int rc = orc_coded_channels(nseg, seg_n, seg_bits);
    int64_t full = n / 32;
    uint8_t *codes = malloc((size_t)32 * (r > 0 ? r : 1));
    uint16_t *sc = malloc(sizeof(uint16_t) * (r > 0 ? r : 1)), *zr = malloc(sizeof(uint16_t) * (r > 0 ? r : 1));
    for (int64_t j = 0; j < full; j++) {
        orc_unpack_group_seg(records + j * words, r, nseg, seg_n, seg_bits, layout, codes, sc, zr);
        for (int t = 0; t < 32; t++)
            for (int c = 0; c < r; c++)
                out[(j * 32 + t) * r + c] =
                    (double)codes[t * r + c] * (double)orc_half_to_float(sc[c]) +
                    (double)orc_half_to_float(zr[c]);
    }
    for (int64_t i = full * 32; i < n; i++) {
        int k = 0;
        for (int c = 0; c < r; c++) {
            int c0;
            int s = seg_of(c, nseg, seg_n, &c0);
            out[i * r + c] = (s < nseg && seg_bits[s] > 0) ? (double)tail[(i - full * 32) * rc + k++] : 0.0;
        }
    }
    free(codes);
    free(sc);
    free(zr);
}

/* The PALU split as segments: [n_hi channels at hi_bit, the rest at lo_bit]. */
static void palu_segments(int r, int n_hi, int hi_bit, int lo_bit, int *seg_n, int *seg_bits)
{
    seg_n[0] = n_hi;
    seg_bits[0] = hi_bit;
    seg_n[1] = r - n_hi;
    seg_bits[1] = lo_bit;
}

void orc_quantize_group(const float *l, int r, int n_hi, int hi_bit, int lo_bit,
                        uint8_t *codes, uint16_t *scale16, uint16_t *zero16)
{
    int sn[2], sb[2];
    palu_segments(r, n_hi, hi_bit, lo_bit, sn, sb);
    orc_quantize_group_seg(l, r, 2, sn, sb, codes, scale16, zero16);
}

int orc_record_words(int r, int n_hi)
{
    return 4 * n_hi + 2 * (r - n_hi) + r;
}

/* Pack one complete group with the PALU split at 4 / 2 bits.  layout 0 = K
 * (token-major planes), 1 = V (channel-major planes). */
void orc_pack_group(const uint8_t *codes, const uint16_t *scale16,
                    const uint16_t *zero16, int r, int n_hi, int layout,
                    uint32_t *rec)
{
    int sn[2], sb[2];
    palu_segments(r, n_hi, 4, 2, sn, sb);
    orc_pack_group_seg(codes, scale16, zero16, r, 2, sn, sb, layout, rec);
}

void orc_unpack_group(const uint32_t *rec, int r, int n_hi, int layout,
                      uint8_t *codes, uint16_t *scale16, uint16_t *zero16)
{
    int sn[2], sb[2];
    palu_segments(r, n_hi, 4, 2, sn, sb);
    orc_unpack_group_seg(rec, r, 2, sn, sb, layout, codes, scale16, zero16);
}

void orc_encode_stream(const float *lat, int64_t n, int r, int n_hi,
                       int hi_bit, int lo_bit, int layout, uint32_t *records,
                       float *tail)
{
    int sn[2], sb[2];
    palu_segments(r, n_hi, hi_bit, lo_bit, sn, sb);
    orc_encode_stream_seg(lat, n, r, 2, sn, sb, layout, records, tail);
}

/* fp16 value latents: records of r*32 halves (channel-major); the last,
 * partially filled record has zeros in its unused slots. */
void orc_encode_fp16_stream(const float *lat, int64_t n, int r, uint16_t *records)
{
    int64_t nrec = (n + 31) / 32;
    memset(records, 0, sizeof(uint16_t) * nrec * 32 * r);
    for (int64_t i = 0; i < n; i++) {
        int64_t j = i / 32;
        int t = (int)(i % 32);
        for (int c = 0; c < r; c++)
            records[j * 32 * r + c * 32 + t] = orc_float_to_half(lat[i * r + c]);
    }
}

/* Dequantised latents (fp64) of n tokens with the PALU split at 4 / 2 bits. */
void orc_decode_stream(const uint32_t *records, const float *tail, int64_t n,
                       int r, int n_hi, int layout, double *out)
{
    int sn[2], sb[2];
    palu_segments(r, n_hi, 4, 2, sn, sb);
    orc_decode_stream_seg(records, tail, n, r, 2, sn, sb, layout, out);
}

void orc_decode_fp16_stream(const uint16_t *records, int64_t n, int r, double *out)
{
    for (int64_t i = 0; i < n; i++)
        for (int c = 0; c < r; c++)
            out[i * r + c] = (double)orc_half_to_float(
                records[(i / 32) * 32 * r + c * 32 + (i % 32)]);
}

/*
 * Single-query attention over n reconstructed tokens (PALU page, "How it
 * works": reconstruct K/V = L V_g^T + mu_g, then attention).
 *   lk, lv : fp64 dequantised latents [n][rk], [n][rv]
 *   Bk, Bv : fp32 bases [D][ldk], [D][ldv] (first rk / rv columns used)
 *   q      : fp32 query [D] (fp16 values widened)
 *   out    : fp64 [D]
 * Everything is fp64; the softmax subtracts the maximum score.
 */
void orc_attend(const double *lk, const float *Bk, int ldk, const float *muk,
                int rk, const double *lv, const float *Bv, int ldv,
                const float *muv, int rv, int64_t n, int D, const float *q,
                double scale, double *out)
{
    double *s = malloc(sizeof(double) * (n > 0 ? n : 1));
    double *kt = malloc(sizeof(double) * D);
    double smax = -INFINITY;
    for (int64_t t = 0; t < n; t++) {
        for (int d = 0; d < D; d++) {
            double acc = (double)muk[d];
            for (int c = 0; c < rk; c++)
                acc += (double)Bk[(int64_t)d * ldk + c] * lk[t * rk + c];
            kt[d] = acc;
        }
        double dot = 0.0;
        for (int d = 0; d < D; d++)
            dot += (double)q[d] * kt[d];
        s[t] = dot * scale;
        if (s[t] > smax)
            smax = s[t];
    }
    double denom = 0.0;
    for (int64_t t = 0; t < n; t++) {
        s[t] = exp(s[t] - smax);
        denom += s[t];
    }
    for (int d = 0; d < D; d++)
        out[d] = 0.0;
    for (int64_t t = 0; t < n; t++) {
        double p = s[t] / denom;
        for (int d = 0; d < D; d++) {
            double acc = (double)muv[d];
            for (int c = 0; c < rv; c++)
                acc += (double)Bv[(int64_t)d * ldv + c] * lv[t * rv + c];
            out[d] += p * acc;
        }
    }
    free(s);
    free(kt);
}

/*
 * Causal prefill attention over n reconstructed tokens (PALU page, "How it
 * works", prefill step 6: K/V are reconstructed as L V_g^T + mu_g for the
 * attention call that follows).  The whole K and V are reconstructed first,
 * then each query i, sitting at position pos[i], attends to tokens
 * 0..pos[i] (causal mask, the plain reading for a prefill).
 *   lk, lv : fp64 dequantised latents [n][rk], [n][rv]
 *   Bk, Bv : fp32 bases [D][ldk], [D][ldv] (first rk / rv columns used)
 *   q      : fp32 queries [nq][D] (fp16 values widened)
 *   pos    : [nq] positions, 0 <= pos[i] < n
 *   out    : fp64 [nq][D]
 * Everything is fp64; each softmax subtracts its row's maximum score.
 */
void orc_prefill_attend(const double *lk, const float *Bk, int ldk, const float *muk,
                        int rk, const double *lv, const float *Bv, int ldv,
                        const float *muv, int rv, int64_t n, int D, const float *q,
                        const int64_t *pos, int64_t nq, double scale, double *out)
{
    double *kh = malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * D);
    double *vh = malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * D);
    double *s = malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    /* 1. reconstruction of every stored token */
    for (int64_t t = 0; t < n; t++)
        for (int d = 0; d < D; d++) {
            double ak = (double)muk[d], av = (double)muv[d];
            for (int c = 0; c < rk; c++)
                ak += (double)Bk[(int64_t)d * ldk + c] * lk[t * rk + c];
            for (int c = 0; c < rv; c++)
                av += (double)Bv[(int64_t)d * ldv + c] * lv[t * rv + c];
            kh[t * D + d] = ak;
            vh[t * D + d] = av;
        }
    /* 2. one causal softmax attention row per query */
    for (int64_t i = 0; i < nq; i++) {
        const int64_t last = pos[i];
        double smax = -INFINITY;
        for (int64_t t = 0; t <= last; t++) {
            double dot = 0.0;
            for (int d = 0; d < D; d++)
                dot += (double)q[i * D + d] * kh[t * D + d];
            s[t] = dot * scale;
            if (s[t] > smax)
                smax = s[t];
        }
        double denom = 0.0;
        for (int64_t t = 0; t <= last; t++) {
            s[t] = exp(s[t] - smax);
            denom += s[t];
        }
        for (int d = 0; d < D; d++)
            out[i * D + d] = 0.0;
        for (int64_t t = 0; t <= last; t++) {
            const double p = s[t] / denom;
            for (int d = 0; d < D; d++)
                out[i * D + d] += p * vh[t * D + d];
        }
    }
    free(kh);
    free(vh);
    free(s);
}
