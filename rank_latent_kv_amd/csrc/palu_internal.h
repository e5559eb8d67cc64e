// Internal declarations shared by the host runtime and the HIP kernels of
// libpalu.so.  Nothing here is part of the C ABI.
#pragma once

#include <cstddef>
#include <cstdint>
#include <vector>

#include <hip/hip_runtime_api.h>

// Helpers used by both the host runtime and the kernels.
#if defined(__HIP__)
#define PALU_HD __host__ __device__
#else
#define PALU_HD
#endif

namespace palu {

constexpr int kTokGroup = 32;      // tokens per quantisation group
constexpr int kHeadDim = 128;      // head_dim the kernels are built for
constexpr int kMaxCallSeqs = 64;   // sequences per launch (argument arrays)
constexpr int kMaxSplits = 128;    // token splits per (sequence, kv head)
constexpr int kMaxGqa = 8;         // query heads per kv head in the attend kernel
constexpr int kGramRowsPerBlockMin = 512;

constexpr int kMaxSegs = 8;        // coded segments of a tensor's latent channels

// The coded latent channels of a tensor as contiguous segments, descending
// singular value first (0-bit channels are removed before this point):
// segment s holds channels [c0[s], c0[s+1]) at bits[s] bits (1, 2, 4 or 8);
// its code plane starts at record word plane0[s] (32 tokens x bits x
// channels bits long); its channels fill the 8-channel blocks
// [q0[s], q0[s+1]) of the score-operand position order (each segment's
// last block padded); one metadata word per channel follows all planes, at
// meta0 + c.  PALU's split is the two-segment case (hi channels at 4 bits,
// the rest at 2).
struct Coder {
    int nseg;
    int bits[kMaxSegs];
    int c0[kMaxSegs + 1];
    int plane0[kMaxSegs];
    int q0[kMaxSegs + 1];
    int meta0;
};

// Segments (channels, bits) with channels > 0 and bits > 0 -> Coder.
PALU_HD inline Coder make_coder(const int *seg_n, const int *seg_bits, int nseg) {
    Coder cd{};
    int c = 0, w = 0, q = 0;
    for (int s = 0; s < nseg; ++s) {
        cd.bits[s] = seg_bits[s];
        cd.c0[s] = c;
        cd.plane0[s] = w;
        cd.q0[s] = q;
        c += seg_n[s];
        w += seg_n[s] * seg_bits[s];
        q += (seg_n[s] + 7) / 8;
    }
    cd.nseg = nseg;
    cd.c0[nseg] = c;
    cd.q0[nseg] = q;
    cd.meta0 = w;
    return cd;
}
PALU_HD inline int coder_channels(const Coder &cd) { return cd.c0[cd.nseg]; }
PALU_HD inline int coder_blocks(const Coder &cd) { return cd.q0[cd.nseg]; }
// Words of one record: the code planes, then one meta word per channel.
PALU_HD inline int coder_words(const Coder &cd) { return cd.meta0 + coder_channels(cd); }
// fp16 latents: r channels x 32 tokens of 2 bytes = 16 r words.
inline int fp16_record_words(int r) { return 16 * r; }

// Stored state of one tensor (K or V) in the bound device buffer.
struct TensorDev {
    uint32_t *records;   // [slots][H][max_groups][words]
    float *tail;         // [slots][H][2][32][r]  (nullptr for fp16 latents)
    float *basis;        // [G][D][r] fp32, d-major
    uint16_t *basis_t16; // K only: [G][P][D] fp16 copy, row n = channel of score-operand position n
                         // (8-channel blocks, hi blocks first, [c0,c4,c1,c5,..] inside a
                         // block; zero rows for padding), P = 8 * blocks (query absorption)
    float *basis_cm;     // [G][r][D] fp32, channel-major copy (output projection)
    float *mu;           // [G][D] fp32
    int r, words;        // coded latent channels, words per record
    int fp16_latents;    // V stored as fp16 latents (no tail, no meta)
    Coder cd;            // segments of the quantised records (unused for fp16 latents)
    int64_t head_stride; // words between consecutive (slot, head): max_groups * words
                         // rounded up to a multiple of 4 (16-byte aligned streams)
    // elements between the basis sets of consecutive slots (per-sequence
    // bases); 0 when one basis set serves every slot
    int64_t set_basis, set_bt16, set_bcm, set_mu;
};

// One Gram block of segment seg = b * hpg + head-in-group: the 64-token
// tiles starting at t0, t0 + stride, t0 + 2 stride, ... below t1 (the
// segment's length).  The k blocks of a segment take every k-th tile
// (stride 64 k), so the blocks of a segment stream adjacent tiles.
struct GramBlock {
    int seg, t0, t1, stride;
};

struct GramArgs {
    const uint16_t *x[2];     // K, V fp16 or bf16 [B][H][S_stride][D]
    const GramBlock *blocks;  // [nb], device
    float *partial;           // [2][G][nb][D*D + D]
    int B, H, S_stride, G, hpg, nb;
    int bf16;                 // inputs are bf16 (else fp16)
};

struct GramReduceArgs {
    const float *partial;     // [2][G][nb][D*D + D]
    double *out;              // [2][G][D*D + D]
    int G, nb;
};

struct EncodeArgs {
    const uint16_t *x[2];     // K, V fp16 or bf16 [B][H][T_stride][D]
    TensorDev t[2];
    int B, H, T_stride, hpg;
    int bf16;                 // inputs are bf16 (else fp16)
    // Per-slot stored length and live tail buffer in device memory.  With
    // dev_len = 0 the lengths below come from the host and one workgroup per
    // row writes the new length and buffer there; with dev_len = 1 (one token
    // per row, lengths read from there) nothing writes them: the decode step
    // that follows commits the new length.
    int *len_dev, *sel_dev;
    int dev_len, max_len;
    int slot[kMaxCallSeqs];
    int old_len[kMaxCallSeqs];
    int n_new[kMaxCallSeqs];
    int sel_old[kMaxCallSeqs];
    int sel_new[kMaxCallSeqs];
};

// One decode row (16 bytes, one load): cache slot, stored length, the
// call's row index of its query/output, and sel | nsplit << 1 (live tail
// buffer, number of splits).  Rows are ordered longest first so that the
// longest workgroups are dispatched first.
struct AttendRow {
    int slot, len, qi, sel_ns;
};

struct AttendArgs {
    const uint16_t *q;        // fp16 or bf16 [B][Hq][D]
    uint16_t *out;            // same type as q, [B][Hq][D]
    float *partial;           // [B][Hq][nsplit_max][2 + r_v]
    TensorDev k, v;
    int B, Hq, Hkv, gqa, hpg;
    int chunk;                // complete token groups per split
    int nsplit_max;           // grid x; splits s >= row.nsplit exit at once
    float qscale;             // softmax scale * log2(e)
    // correctly rounded fp32 reciprocals of index divisors: r_v and 4 times
    // the key channel blocks
    float inv_rv, inv_nbk4;
    int bf16;                 // q and out are bf16 (else fp16)
    // dev_len = 1 (decode step after a one-token append): a row's length is
    // min(len_dev[slot] + 1, max_len) and its tail buffer sel_dev[slot], its
    // split count follows from chunk; the attend kernel hands (length,
    // splits) of call row i to the combine kernel in row_info[2 i], which
    // then commits the length to len_dev.
    int *len_dev;
    const int *sel_dev;
    int *row_info;
    int dev_len, max_len;
    AttendRow row[kMaxCallSeqs];       // grid y order (longest first)
    int nsplit_call[kMaxCallSeqs];     // splits of call row i (combine)
    int slot_call[kMaxCallSeqs];       // cache slot of call row i (combine)
};

// One call row of a prefill attention launch: the queries are the last nq
// positions [len - nq, len) of the slot.
// One prefill row (16 bytes): cache slot, stored length, queries, and the
// tail buffer in use | call index of the row << 1 (rows are launched
// heaviest first; the call index addresses its queries and outputs).
struct PrefillRow {
    int slot, len, nq, sel_qi;
};

struct PrefillArgs {
    const uint16_t *q;        // fp16 or bf16 [B][Hq][T_stride][D]
    uint16_t *out;            // same type as q, [B][Hq][T_stride][D]
    TensorDev k, v;
    int B, Hq, Hkv, gqa, hpg, T_stride;
    int qp;                   // query positions per workgroup
    int tiles_max;            // grid x; tiles past a row's last exit at once
    float qscale;             // softmax scale * log2(e)
    int bf16;                 // q and out are bf16 (else fp16)
    PrefillRow row[kMaxCallSeqs];
    // Pre-decoded tiles (nullptr: the prefill kernel decodes each group
    // itself): the fp16 key and value tiles of complete group j of call row
    // i and kv head h are tile_bytes bytes at tile tile_base[i] + h nfull + j
    // (nfull = the row's complete groups).
    uint8_t *ws_tiles;
    int tile_bytes;
    int64_t tile_base[kMaxCallSeqs];
};

// Waves of one prefill attention workgroup (16 NQ query columns each).
constexpr int kPrefillWaves = 4;

// Score K-steps (32 key-basis positions each), value blocks (16 channels,
// one of them the all-ones column that yields the softmax denominator) and
// query tiles per wave (16 columns each) of the prefill kernel variant that
// serves these ranks.
int prefill_ks(int nbk);             // nbk = key channel blocks (coder_blocks)
int prefill_nbv(int r_v);
int prefill_nq(int ks, int nbv);
// LDS bytes of one prefill workgroup.
size_t prefill_lds_bytes(int nbk, int r_k, int r_v, int words_k, int words_v);
// Bytes of one complete group's pre-decoded key + value tiles.
size_t prefill_tile_bytes(int nbk, int r_v);
// Grid (tiles_max, Hkv, B), 64 kPrefillWaves threads (defined in palu_prefill.hip).
hipError_t launch_prefill(const PrefillArgs &a, size_t lds_bytes, hipStream_t s);
// Pre-decodes the tiles of every complete group of the call's rows into
// a.ws_tiles (one wave per group; max_nfull = the rows' largest count).
hipError_t launch_prefill_tiles(const PrefillArgs &a, int max_nfull, hipStream_t s);

// LDS bytes of one attend workgroup (independent of the split size).
size_t attend_lds_bytes(int gqa, int nbk, int r_k, int r_v, int words_k, int words_v, bool vq);

// Launchers (defined in palu_kernels.hip).  They return the launch status.
hipError_t launch_gram(const GramArgs &a, hipStream_t s);
// Gram workgroups the current device holds at once (CUs x blocks per CU).
hipError_t gram_resident_blocks(int *n);
hipError_t launch_gram_reduce(const GramReduceArgs &a, hipStream_t s);
// One wave per (pair of touched token groups, call row x head, tensor).
hipError_t launch_encode(const EncodeArgs &a, int max_units, hipStream_t s);
// Appends of at most one token per row: one workgroup of one wave per (call
// row x head, tensor), one lane per latent channel.
hipError_t launch_append1(const EncodeArgs &a, hipStream_t s);
// Grid (Hkv, B, nsplit_max): one workgroup per (kv head, row, split), the head fastest.
hipError_t launch_attend(const AttendArgs &a, size_t lds_bytes, hipStream_t s);
hipError_t launch_combine(const AttendArgs &a, hipStream_t s);
// Bytes of the file-scope device array that holds the split partials of the
// allocation-free decode entry point, and its address on the current device
// (looked up once per device; defined in palu_decode.hip).
constexpr size_t kStaticScratchBytes = size_t(16) << 20;
hipError_t static_scratch_address(void **ptr);
// Position-ordered fp16 copy of a basis [G][D][r]: dst[g][n][d] =
// fp16(src[g][d][channel of position n]) for the coder's blocks, 0 where n
// is padding.
hipError_t launch_basis_t16(const float *src, uint16_t *dst, int G, int r, const Coder &cd, hipStream_t s);
// Read-bandwidth probe: grid workgroups of 256 threads stream n16 16-byte
// words of src and write one fold per workgroup to sink[grid].
hipError_t launch_read_probe(const void *src, size_t n16, uint32_t *sink, int grid, hipStream_t s);
// rows of the position-ordered fp16 basis copy (8 per channel block)
PALU_HD inline int basis_t16_rows(const Coder &cd) { return 8 * coder_blocks(cd); }

// Host symmetric eigensolver (palu_eigen.cpp), in two steps for the fit:
// sym_eigenvalues reduces a (n x n row-major symmetric, destroyed) to
// tridiagonal form, keeps the reflectors and finds every eigenvalue
// (descending in w; false if the iteration did not converge);
// sym_top_vectors then writes the eigenvectors of the k largest into z
// (n x k row-major, column j <-> w[j]), unit length and mutually orthogonal.
struct SymEigen {
    int n = 0;
    std::vector<double> hv, beta;   // reflector vectors [n][n] and coefficients
    std::vector<double> d, e;       // tridiagonal matrix
    std::vector<double> w;          // eigenvalues, descending
};
bool sym_eigenvalues(double *a, int n, SymEigen &s);
void sym_top_vectors(const SymEigen &s, int k, double *z);

}  // namespace palu
