/*
 * palu.h -- C ABI of the low-rank latent KV cache library (libpalu.so).
 *
 * The method is the PALU-style latent cache of the veloxquant-mlx "PALU"
 * page: per head group, a mean mu_g and a truncated basis V_g (D x r) are
 * fitted from the prefill (section "How it works", prefill steps 1-3); keys
 * and values are stored as latents L = (x - mu_g) V_g quantised with mixed
 * bit widths over 32-token groups (steps 4-6 and the decode steps); decode
 * attention is computed directly from the stored latents, which equals
 * attention over the reconstruction L V_g^T + mu_g.
 *
 * Conventions for every entry point:
 *   - Return value: PALU_OK (0) or a PALU_ERR_* code.  No exception, abort
 *     or HIP error escapes; palu_last_error() gives a message for the last
 *     failing call on the calling thread.
 *   - Every argument is validated on the host before any device work, so a
 *     failing call leaves the cache and the stream untouched.
 *   - "device" pointers are HIP device memory owned by the caller; "host"
 *     pointers are ordinary host memory owned by the caller and only read
 *     or written during the call.
 *   - stream is a hipStream_t (NULL = the null stream).  Calls marked
 *     "stream-ordered" only enqueue work; calls marked "synchronous" return
 *     after their device work has finished.
 *   - fp16 tensors are IEEE binary16, little-endian, densely packed in the
 *     stated index order (last index fastest).
 *   - A cache object must not be used by two threads at once.
 */
#ifndef PALU_H
#define PALU_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    PALU_OK = 0,
    PALU_ERR_INVALID_ARG = 1,   /* null pointer, bad size, bad config       */
    PALU_ERR_UNSUPPORTED = 2,   /* valid but not implemented (e.g. D > 128) */
    PALU_ERR_NOT_FITTED = 3,    /* encode/decode/read before a basis exists */
    PALU_ERR_CAPACITY = 4,      /* append beyond max_seq_len, bad seq slot  */
    PALU_ERR_NOT_BOUND = 5,     /* device storage not bound yet             */
    PALU_ERR_HIP = 6            /* a HIP runtime call failed                */
};

/* Method configuration.  Mirrors the PALU fields of KVCacheConfig on the
 * PALU page, section "Usage" (palu_rank, palu_energy_threshold,
 * palu_n_head_groups, palu_hi_bit, palu_lo_bit, palu_hi_fraction,
 * palu_group_size, palu_quantize_values). */
typedef struct palu_config {
    int32_t head_dim;          /* D; the kernels are built for D = 128 only      */
    int32_t n_kv_heads;        /* H: heads stored by the cache                     */
    int32_t n_q_heads;         /* query heads, a multiple of n_kv_heads; query head
                                  i attends with kv head i / (n_q_heads/n_kv_heads) */
    int32_t n_head_groups;     /* G contiguous groups of kv heads sharing a basis;
                                  group g owns heads [g*H/G, (g+1)*H/G)           */
    int32_t rank;              /* explicit rank (clamped to D); 0 = energy rule   */
    float energy_threshold;    /* tau of the energy rule, in (0, 1]               */
    int32_t hi_bit;            /* bits of the top channels: 1, 2, 4 or 8          */
    int32_t lo_bit;            /* bits of the other channels: 1, 2, 4 or 8        */
    float hi_fraction;         /* n_hi = floor(hi_fraction * r) channels at hi_bit */
    int32_t group_size;        /* tokens per quantisation group; only 32          */
    int32_t quantize_values;   /* 1: V mixed-bit like K; 0: V as fp16 latents     */
    int32_t max_rank;          /* storage is sized for ranks up to this (0 = D)   */
    int32_t split_groups;      /* decode: complete token groups per split (work of
                                  one workgroup); 0 = automatic.  Raised to fit the
                                  split limit (128 splits per sequence and head);
                                  a value whose LDS need exceeds 160 KiB makes
                                  palu_decode_attend fail with UNSUPPORTED.      */
    int32_t input_dtype;       /* element type of every K, V and q input and of the
                                  attention outputs: 0 = fp16, 1 = bf16 (review
                                  thread of the "add TurboQuant KV cache
                                  compression" pull-request page: bf16 keys beyond
                                  the fp16 range must not be cast).  Codes,
                                  their fp16 scale/zero words and the fp32 tails
                                  are the same for both; with bf16, latents must
                                  stay within the fp16 range like with fp16.     */
    int32_t schedule_len;      /* 0: PALU's split above (hi_fraction, hi_bit,
                                  lo_bit).  1..8: a bit schedule as on the SVDq
                                  cache page: the r latent channels form
                                  schedule_len contiguous groups of equal size
                                  (the first r % schedule_len one channel
                                  larger), largest singular values first, group
                                  i coded with bit_schedule[i] bits; 0 bits drops
                                  the group (its latent is exactly zero and is
                                  stored nowhere).  Applies to K, and to V when
                                  quantize_values is 1.                          */
    int32_t bit_schedule[8];   /* bits per group: 0, 1, 2, 4 or 8; at least one
                                  nonzero among the first schedule_len           */
    int32_t per_seq_basis;     /* 0: one basis per (tensor, head group), fitted
                                  over every sequence given to palu_fit and
                                  shared by all slots.  1: every slot has its own
                                  bases, fitted from its own prompt (palu_fit /
                                  palu_fit_seq) or installed with
                                  palu_set_basis_seq; needs an explicit rank (all
                                  slots share one record layout).                 */
} palu_config;

/* Fills the page's defaults (rank 0 = energy rule, threshold 0.90, G = 4,
 * 4/2 bits, hi_fraction 0.25, group 32, quantised values) for the given
 * shape.  Returns PALU_ERR_INVALID_ARG for a null pointer. */
int palu_config_default(palu_config *cfg, int32_t head_dim, int32_t n_kv_heads,
                        int32_t n_q_heads);

typedef struct palu_cache palu_cache;   /* opaque; host memory only */

/* Creates a cache for up to max_batch sequence slots of up to max_seq_len
 * tokens each.  Allocates host bookkeeping only (no device memory).
 * Errors: INVALID_ARG (null, non-positive sizes, H % G, Hq % H, bad
 * threshold or fraction), UNSUPPORTED (D, bit widths or group size outside
 * what the kernels implement). */
int palu_cache_create(const palu_config *cfg, int32_t max_batch,
                      int32_t max_seq_len, palu_cache **out);

/* Device bytes the cache needs: bases, means, packed records, fp32 tails,
 * the fit workspace and the decode split scratch, for max_rank. */
int palu_cache_required_bytes(const palu_cache *cache, size_t *dev_bytes);

/* Binds caller-allocated device storage of at least the required bytes,
 * 256-byte aligned.  The library never allocates device memory itself.
 * The storage must outlive the cache or the next bind.  Binding drops any
 * fitted basis and empties every sequence. */
int palu_cache_bind(palu_cache *cache, void *dev_buf, size_t bytes);

/* Group-head fit (PALU page, "How it works", prefill steps 1-3): for K and
 * V separately, per group, mean and truncated eigenbasis of the rows of all
 * B sequences (first seq_lens[b] tokens) and all heads of the group; the
 * rank is the explicit one or the smallest meeting the energy threshold
 * (energy = sum of squared singular values), and the minimum over groups
 * is used for every group.
 *   k, v     : device fp16 or bf16 (input_dtype) [B][H][S_stride][D]
 *   seq_lens : host int32 [B], 0 <= seq_lens[b] <= S_stride, sum > 0
 * Synchronous (the eigensolve runs on the host).  Empties every sequence
 * slot (stored codes of an older basis are meaningless) once the fit has
 * succeeded; a fit that fails on its arguments, the fit workspace, the
 * eigensolver or the rank (CAPACITY: rank above max_rank; UNSUPPORTED: a
 * bit schedule that codes no channel at that rank) leaves the previous
 * bases and stored tokens as they were (a HIP error while installing the
 * new bases leaves the cache unfitted).  With per-sequence
 * bases (per_seq_basis = 1) row b is fitted alone into slot b, as
 * palu_fit_seq with seq_ids = 0 .. B-1 (every seq_lens[b] > 0), and only
 * those slots are emptied.  Errors: INVALID_ARG, CAPACITY, NOT_BOUND,
 * UNSUPPORTED, HIP (also when the eigensolver does not converge). */
int palu_fit(palu_cache *cache, const void *k, const void *v,
             const int32_t *seq_lens, int32_t B, int32_t S_stride, void *stream);

/* Installs a basis instead of fitting one (tensor 0 = K, 1 = V):
 *   basis : host fp32 [G][D][r], basis[g][d][c] = component d of channel c,
 *           channels in descending singular-value order
 *   mu    : host fp32 [G][D]
 * 1 <= r <= max_rank.  Synchronous.  Empties every sequence slot.  With
 * per-sequence bases it installs the basis in every slot (r must equal the
 * cache's rank). */
int palu_set_basis(palu_cache *cache, int32_t tensor, int32_t r,
                   const float *basis, const float *mu);

/* Reads the shared basis of tensor 0 (K) or 1 (V) (INVALID_ARG with
 * per-sequence bases: see palu_get_basis_seq).  r receives the rank; basis
 * (host fp32 [G][D][r]), mu (host fp32 [G][D]) and sigma (host fp64 [G][D],
 * singular values of the centred stacks, zeros if set by palu_set_basis)
 * may each be NULL.  Errors: INVALID_ARG, NOT_FITTED. */
int palu_get_basis(const palu_cache *cache, int32_t tensor, int32_t *r,
                   float *basis, float *mu, double *sigma);

/* Per-sequence bases (per_seq_basis = 1): fits row b of k / v
 * ([B][H][S_stride][D], seq_lens[b] valid tokens, > 0) into the bases of
 * slot seq_ids[b] (distinct), with the cache's explicit rank, and empties
 * those slots; other slots keep their bases and tokens.  palu_fit in this
 * mode fits row b into slot b for every row.  Synchronous.
 * Errors: INVALID_ARG (not in per-sequence mode, bad sizes, repeated slot),
 * CAPACITY (slot out of range), NOT_BOUND, HIP. */
int palu_fit_seq(palu_cache *cache, const void *k, const void *v,
                 const int32_t *seq_ids, const int32_t *seq_lens, int32_t B,
                 int32_t S_stride, void *stream);

/* Per-sequence bases: installs (set) or copies out (get) one slot's basis
 * for tensor 0 (K) or 1 (V), in the layout of palu_set_basis /
 * palu_get_basis; r must equal the cache's rank.  set empties the slot. */
int palu_set_basis_seq(palu_cache *cache, int32_t seq, int32_t tensor, int32_t r,
                       const float *basis, const float *mu);
int palu_get_basis_seq(const palu_cache *cache, int32_t seq, int32_t tensor, int32_t *r,
                       float *basis, float *mu, double *sigma);

/* Appends tokens (PALU page, "How it works", decode steps 1-2): projects
 * each new key/value into its group's basis with a fixed-order fp32 chain,
 * quantises every 32-token group that becomes complete (asymmetric min/max,
 * round half to even, each channel at its segment's width: PALU's split or
 * the bit schedule) and keeps the incomplete group's latents of the coded
 * channels in fp32 until it completes.
 *   k, v     : device fp16 or bf16 (input_dtype) [B][H][T_stride][D]
 *   seq_ids  : host int32 [B] slot of each row (NULL = 0..B-1), distinct
 *   n_new    : host int32 [B] tokens to append per row (NULL = T_stride each),
 *              0 <= n_new[b] <= T_stride
 * Row b appends positions [len, len + n_new[b]) of slot seq_ids[b].
 * Stream-ordered.  Errors: INVALID_ARG, NOT_BOUND, NOT_FITTED, CAPACITY
 * (len + n_new > max_seq_len or slot >= max_batch), HIP. */
int palu_encode_append(palu_cache *cache, const void *k, const void *v,
                       const int32_t *seq_ids, const int32_t *n_new, int32_t B,
                       int32_t T_stride, void *stream);

/* Single-query decode attention over every stored token of each slot
 * (PALU page, "How it works", decode step 3, computed directly from the
 * latent codes): out = softmax(q K^T * scale) V with K, V the decoded
 * reconstruction; fp32 scores and accumulation.
 *   q, out        : device fp16 or bf16 (input_dtype) [B][Hq][D]
 *   seq_ids       : host int32 [B] (NULL = 0..B-1); every slot must hold at
 *                   least one token
 *   softmax_scale : 0 means 1/sqrt(D)
 * Stream-ordered.  Uses the split scratch inside the bound storage, so two
 * calls on one cache must not run concurrently on different streams.
 * Errors: INVALID_ARG, NOT_BOUND, NOT_FITTED, CAPACITY (empty slot), HIP. */
int palu_decode_attend(palu_cache *cache, const void *q, void *out,
                       const int32_t *seq_ids, int32_t B, float softmax_scale,
                       void *stream);

/* One decode step (PALU page, "How it works", decode steps 1-3: project,
 * quantise and append the new token, then attend over everything stored),
 * fused so that it can be captured once in a HIP graph and replayed for
 * later steps: row b appends one token (k_new / v_new: device fp16 or bf16
 * [B][H][1][D]) to slot seq_ids[b], then its queries attend over the slot's
 * tokens, including the new one, exactly as palu_encode_append followed by
 * palu_decode_attend.  Every kernel of the call reads the slots' lengths
 * from device memory and the call leaves the new lengths there, so a graph
 * replay appends at the right position without host involvement.  The host
 * keeps its own copy of the lengths, advanced when the call is made (not
 * when a graph replays it): after replaying captured steps call
 * palu_sync_lengths before any other call on the cache.  A replay that
 * finds a slot full stores no token and attends over what is stored.
 *   q, out   : device [B][Hq][D] as in palu_decode_attend
 *   seq_ids  : host int32 [B] (NULL = 0..B-1), distinct; empty slots allowed
 * Stream-ordered; uses the split scratch of the bound storage (no
 * concurrent decode calls on one cache).  Errors: INVALID_ARG, NOT_BOUND,
 * NOT_FITTED, CAPACITY (a slot out of range or full), UNSUPPORTED, HIP. */
int palu_decode_step(palu_cache *cache, const void *k_new, const void *v_new, const void *q,
                     void *out, const int32_t *seq_ids, int32_t B, float softmax_scale,
                     void *stream);

/* Copies the slots' lengths from device memory to the host's copy (after
 * graph replays of palu_decode_step).  Synchronous: waits for all device
 * work.  Errors: INVALID_ARG, NOT_BOUND, HIP. */
int palu_sync_lengths(palu_cache *cache);

/* palu_decode_attend for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same kernels and results, with the split partials in a
 * file-scope device array of the library (16 MiB per GPU, held until the
 * process ends) instead of the bound storage.  The call allocates nothing
 * (no hipMalloc or allocating library routine); the caller still passes q,
 * out and the bound cache.  Every call on a GPU shares that GPU's array, so
 * calls that overlap on one GPU (other streams, other caches, other
 * threads) race: order them on one stream.  Nothing in the array has to
 * start at zero (each call writes every partial it reads).
 * Errors: as palu_decode_attend, and UNSUPPORTED when a launch's partials
 * (rows x n_q_heads x splits x (r_v + 2) x 4 bytes, at most 64 rows per
 * launch) exceed 16 MiB. */
int palu_decode_attend_noalloc(palu_cache *cache, const void *q, void *out,
                               const int32_t *seq_ids, int32_t B, float softmax_scale,
                               void *stream);

/* Causal prefill attention over the stored latents (PALU page, "How it
 * works", prefill step 6: the stored latents feed the attention call that
 * follows the encode), computed directly from the codes like
 * palu_decode_attend.  Row b's queries are the last n_q[b] positions
 * [len - n_q[b], len) of slot seq_ids[b] (append the prompt's K/V first);
 * the query at position p attends to the slot's tokens 0..p.
 *   q, out        : device fp16 or bf16 (input_dtype) [B][Hq][T_stride][D], 16-byte aligned; query
 *                   j of row b at [b][head][j]; only j < n_q[b] is written
 *   seq_ids       : host int32 [B] (NULL = 0..B-1); slots may repeat
 *   n_q           : host int32 [B] (NULL = T_stride each),
 *                   0 <= n_q[b] <= min(T_stride, len of the slot)
 *   softmax_scale : 0 means 1/sqrt(D)
 * Stream-ordered; reads only the cache (no scratch), so calls may overlap.
 * fp32 scores and accumulation, fp16 weights into the value contraction.
 * Errors: INVALID_ARG, NOT_BOUND, NOT_FITTED, CAPACITY (slot out of range or
 * n_q beyond the slot's length), UNSUPPORTED (LDS need above 160 KiB, or
 * more than 65535 query tiles per row: T_stride above 65535 x the tile's
 * query positions, 16 x 4 x (query tiles per wave) / GQA), HIP. */
int palu_prefill_attend(palu_cache *cache, const void *q, void *out,
                        const int32_t *seq_ids, const int32_t *n_q, int32_t B,
                        int32_t T_stride, float softmax_scale, void *stream);

/* Bytes of the workspace palu_prefill_attend_ws needs for these slots at
 * their current lengths: one pre-decoded key + value tile pair per kv head
 * and complete 32-token group (a few KiB each).  seq_ids as in
 * palu_prefill_attend.  Errors: INVALID_ARG, NOT_BOUND, NOT_FITTED,
 * CAPACITY (slot out of range). */
int palu_prefill_workspace_bytes(const palu_cache *cache, const int32_t *seq_ids, int32_t B,
                                 size_t *bytes);

/* palu_prefill_attend with a caller-provided device workspace (PALU page,
 * "How it works", prefill step 6, as above): every complete group's fp16
 * key and value tiles are decoded from the codes once, into the workspace,
 * and the attention kernel streams them instead of decoding each group
 * once per query tile that reads it.  Same arguments, the same output
 * bits as palu_prefill_attend, plus
 *   workspace       : device, 16-byte aligned, at least
 *                     palu_prefill_workspace_bytes for these slots; the call
 *                     writes it (stream-ordered), so calls that share one
 *                     workspace must not overlap
 *   workspace_bytes : its size
 * Errors: as palu_prefill_attend; INVALID_ARG also for a NULL, misaligned
 * or too small workspace. */
int palu_prefill_attend_ws(palu_cache *cache, const void *q, void *out,
                           const int32_t *seq_ids, const int32_t *n_q, int32_t B,
                           int32_t T_stride, float softmax_scale,
                           void *workspace, size_t workspace_bytes, void *stream);

/* Tokens stored in a slot. */
int palu_seq_len(const palu_cache *cache, int32_t seq, int32_t *len);

/* Copies the stored state of one (slot, kv head, tensor) to host memory.
 * Synchronous on the null stream after a device synchronisation.
 *   records : host, receives the complete groups' records in order:
 *             quantised: floor(len/32) records of palu_record_words uint32
 *             fp16 V latents: ceil(len/32) records of r*32 fp16 (c*32 + t);
 *             may be NULL
 *   tail    : host fp32 [len % 32][coded] latents of the incomplete group,
 *             coded = the stats' coded_k / coded_v (NULL allowed; not used
 *             for fp16 V latents)
 * The byte sizes must be at least what is copied.  Record layout: the coded
 * channels (0-bit channels dropped, order kept) form segments of n_s
 * channels at b_s bits; segment s has a code plane of n_s * b_s words, the
 * planes in segment order, then one word scale16[c] | zero16[c] << 16 per
 * coded channel.  Inside a plane (c' = channel index in the segment):
 *   K (tensor 0): token t, channel c' at bit t * b_s * n_s + b_s * c'
 *   V (tensor 1): channel c', token t at bit 32 * b_s * c' + b_s * t
 * PALU's split gives a 4-bit plane of 4 n_hi words and a 2-bit plane of
 * 2 (r - n_hi) words. */
int palu_read_codes(const palu_cache *cache, int32_t seq, int32_t head,
                    int32_t tensor, void *records, size_t records_bytes,
                    float *tail, size_t tail_bytes);

/* Byte accounting and rates (PALU page, "Effective bit-width" and
 * "Evidence"; SVDq cache page, "Byte accounting"). */
typedef struct palu_stats {
    int32_t r_k, r_v, n_hi_k, n_hi_v;  /* fitted ranks; channels of the first coder
                                         segment (PALU: n_hi; 0 for fp16 latents) */
    int64_t tokens;                  /* sum of stored tokens over slots        */
    int64_t compressed_key_bytes;    /* records + tails + K bases and means    */
    int64_t compressed_value_bytes;  /* same for V (fp16 latents if unquantised) */
    int64_t fp16_key_bytes;          /* tokens * H * D * 2                     */
    int64_t fp16_value_bytes;
    double nominal_bits_k, nominal_bits_v;   /* (r/D)(h b_hi + (1-h) b_lo), with a schedule
                                                (r/D) mean(schedule); 16 r/D for fp16 latents */
    double realised_bits_k, realised_bits_v; /* code bits per element: sum over channels of
                                                their widths / D, or 16 r/D            */
    double assigned_avg_bits;        /* max of the realised K and V rates      */
    int32_t coded_k, coded_v;        /* latent channels stored (0-bit channels dropped):
                                        the tail width returned by palu_read_codes */
    double energy_margin_k, energy_margin_v; /* energy-rule fits with shared bases: how far
                                        the groups' spectra sit from changing the shared
                                        rank r, min(max_g E_g(r) - tau, tau - max_g
                                        E_g(r - 1)) with E_g(k) the energy fraction of
                                        group g's first k channels (the first term alone
                                        at r = 1); -1 for explicit ranks, installed bases
                                        and per-sequence bases                        */
} palu_stats;

int palu_get_stats(const palu_cache *cache, palu_stats *out);

/* The rank rule of the last shared-basis fit of tensor 0 (K) or 1 (V)
 * (PALU page, "How it works", prefill step 3: a rank per group, the minimum
 * shared by all groups).  For every group g < G:
 *   r_groups[g]    : the group's own rank (the explicit rank clamped to D,
 *                    or the smallest k whose leading squared singular
 *                    values reach energy_threshold of the group's total)
 *   energy_prev[g] : energy fraction of the group's first r - 1 channels,
 *                    r = the shared rank (0 when r = 1)
 *   energy_at[g]   : energy fraction of its first r channels
 * Each pointer may be NULL; the arrays are host memory of G entries.
 * Errors: INVALID_ARG (bad tensor, per-sequence bases), NOT_FITTED (no fit
 * of this tensor since the last bind or palu_set_basis). */
int palu_get_fit_info(const palu_cache *cache, int32_t tensor, int32_t *r_groups,
                      double *energy_prev, double *energy_at);

/* Empties every slot, keeping the basis. */
int palu_reset(palu_cache *cache);

/* Words of one record: the code planes (channels x bits words per segment)
 * plus one metadata word per coded channel; PALU's split gives
 * 4 n_hi + 2 (r - n_hi) + r; fp16 value latents 16 r. */
int palu_record_words(const palu_cache *cache, int32_t tensor, int32_t *words);

/* Save / restore of one sequence slot: the prompt-cache round trip that the
 * "add TurboQuant KV cache compression" pull-request page lists among its
 * proposed changes and fixes in its review thread, applied here to the
 * latent cache.  The
 * serialized form is a 64-byte header followed by, for K then V, the records
 * of every kv head in head order (len / 32 records of words_t uint32 each;
 * fp16 value latents keep ceil(len / 32), the last one partial) and then the
 * fp32 tail latents of every kv head in head order (len % 32 rows of
 * coded_t floats; none for fp16 value latents).  Header, all
 * little-endian: uint32 magic 0x564B4C50 ("PLKV"), uint32 version 1, int32
 * head_dim, n_kv_heads, n_head_groups, r_K, r_V, coder_K, coder_V (32-bit
 * FNV-1a hashes of each tensor's segment layout), words_K, words_V,
 * quantize_values, len, uint64 FNV-1a hash of the fp32 bases and means of
 * both tensors, uint32 flags.  With shared bases (flags 0) the basis is not
 * included (palu_get_basis / palu_set_basis move it) and must match the
 * cache's.  With per-sequence bases (flags 1) the slot's bases follow the
 * header (K basis [G][D][r_K], K mean [G][D], V basis, V mean, fp32) and
 * an import installs them into the target slot.
 *
 * palu_export_bytes: bytes of the serialized slot.  palu_export_seq:
 * synchronous (waits for the device), writes exactly that many bytes to
 * host_dst.  palu_import_seq: synchronous; replaces the slot's contents.
 * Errors: NOT_BOUND / NOT_FITTED as elsewhere; INVALID_ARG for a NULL
 * buffer, an export buffer smaller than palu_export_bytes, an import buffer
 * whose size differs from what its header describes, a bad magic or version,
 * or a header whose shape, ranks or basis hash differ from the cache's
 * current ones; CAPACITY for a slot out of range or len > max_seq_len.  A
 * failed import leaves the slot unchanged (all checks come first). */
int palu_export_bytes(const palu_cache *cache, int32_t seq, size_t *bytes);
int palu_export_seq(const palu_cache *cache, int32_t seq, void *host_dst, size_t bytes);
int palu_import_seq(palu_cache *cache, int32_t seq, const void *host_src, size_t bytes);

/* Measurement aid, not a step of the method: reads `bytes` (a positive
 * multiple of 16) of device memory at buf (16-byte aligned) with 16-byte
 * loads from `grid` workgroups of 256 threads (1 <= grid <= 65536) and
 * writes one 32-bit fold of what each workgroup read to sink (device,
 * grid entries), so the reads cannot be elided.  Timing it gives the read
 * bandwidth the device sustains; run over a buffer larger than the
 * last-level cache it also evicts that cache between timed calls.
 * Stream-ordered.  Errors: INVALID_ARG, HIP. */
int palu_probe_read(const void *buf, size_t bytes, void *sink, int32_t grid, void *stream);

/* Message of the last failing call on this thread ("" if none). */
const char *palu_last_error(void);

void palu_cache_destroy(palu_cache *cache);

#ifdef __cplusplus
}
#endif

#endif /* PALU_H */
