// Host runtime of libpalu.so: argument validation, cache bookkeeping, the
// device memory layout inside the caller-bound buffer, the fit's host
// eigensolve, and kernel launches.  Implements include/palu.h.
#include <hip/hip_runtime_api.h>

#include <unistd.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <condition_variable>
#include <cstdint>
#include <cstring>
#include <functional>
#include <mutex>
#include <numeric>
#include <string>
#include <thread>
#include <vector>

#include "palu.h"
#include "palu_internal.h"

#define PALU_API extern "C" __attribute__((visibility("default")))

using namespace palu;

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string &msg) {
    g_last_error = msg;
    return code;
}

int hip_fail(hipError_t e, const char *what) {
    return fail(PALU_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

constexpr int kGramElems = kHeadDim * kHeadDim + kHeadDim;
constexpr int kGramMaxRowsPerBlock = 8192;   // bounds fp32 accumulation per block
// full Gram blocks per (tensor, group) at most: 1024 workgroups a fit
inline int gram_nb_target(int G) { return std::max(1, 512 / G); }
constexpr int kAttendTargetGroups = 1024;    // workgroups aimed for per decode launch
constexpr int64_t kMaxGridYZ = 65535;        // largest grid y or z dimension of a launch
constexpr size_t kAttendLdsMax = 160 * 1024; // LDS per workgroup on gfx950

int n_hi_of(int r, float frac) {
    return static_cast<int>(std::floor(static_cast<double>(frac) * static_cast<double>(r)));
}

// The latent channels of rank r as (channels, bits) segments: PALU's split,
// or the bit schedule's equal contiguous groups (the first r % L one larger).
void split_segments(const palu_config &cfg, int r, std::vector<int> &n, std::vector<int> &bits) {
    n.clear();
    bits.clear();
    if (cfg.schedule_len == 0) {
        const int nh = n_hi_of(r, cfg.hi_fraction);
        n = {nh, r - nh};
        bits = {cfg.hi_bit, cfg.lo_bit};
        return;
    }
    const int L = cfg.schedule_len, base = r / L, extra = r % L;
    for (int i = 0; i < L; ++i) {
        n.push_back(base + (i < extra ? 1 : 0));
        bits.push_back(cfg.bit_schedule[i]);
    }
}

// Coder of the coded segments at rank r, and the coded channels' indices.
Coder coder_for(const palu_config &cfg, int r, std::vector<int> *coded) {
    std::vector<int> n, bits, cn, cb;
    split_segments(cfg, r, n, bits);
    int c = 0;
    if (coded) coded->clear();
    for (size_t s = 0; s < n.size(); ++s) {
        if (n[s] > 0 && bits[s] > 0) {
            cn.push_back(n[s]);
            cb.push_back(bits[s]);
            if (coded)
                for (int k = 0; k < n[s]; ++k) coded->push_back(c + k);
        }
        c += n[s];
    }
    return make_coder(cn.data(), cb.data(), static_cast<int>(cn.size()));
}

bool valid_width(int b) { return b == 1 || b == 2 || b == 4 || b == 8; }

uint32_t fnv1a32(const void *p, size_t n) {
    const unsigned char *b = static_cast<const unsigned char *>(p);
    uint32_t h = 0x811C9DC5u;
    for (size_t i = 0; i < n; ++i) {
        h ^= b[i];
        h *= 0x01000193u;
    }
    return h;
}

}  // namespace

struct palu_cache {
    palu_config cfg{};
    int max_batch = 0, max_seq_len = 0;
    int D = 0, H = 0, Hq = 0, G = 0, hpg = 0, gqa = 0, r_max = 0, max_groups = 0;
    int gram_nb_cap = 0;          // Gram blocks (partials) of one launch
    int64_t gram_tab_cap = 0;     // block-table entries of one fit
    int gram_resident = 0;        // Gram workgroups the device holds at once (0: not queried yet)
    int n_cus = 0;                // compute units of the device (0: not queried yet)
    // byte offsets of each region inside the bound buffer
    size_t off_basis[2]{}, off_bt16[2]{}, off_bcm[2]{}, off_mu[2]{}, off_rec[2]{}, off_tail[2]{};
    size_t off_gram_part = 0, off_gram_out = 0, off_seg = 0, off_attend = 0, off_len = 0, total = 0;
    char *dev = nullptr;
    size_t dev_bytes = 0;
    // basis sets: one per slot with per-sequence bases (the rank, and so
    // the record layout, fixed at creation), else one shared by all slots
    bool per_seq = false;
    int nbs = 1;
    int64_t sb_basis = 0, sb_bt16 = 0, sb_bcm = 0, sb_mu = 0;   // device elements per set
    std::vector<char> ready[2];        // set s of tensor t installed
    int r[2] = {0, 0};                 // fitted ranks
    int rc[2] = {0, 0};                // coded (stored) latent channels
    Coder cd[2]{};
    std::vector<int> coded[2];         // fitted-basis column of each coded channel
    std::vector<float> basis_h[2], mu_h[2];   // nbs sets of [G][D][r] and [G][D]
    std::vector<double> sigma_h[2];           // nbs sets of [G][D]
    std::vector<int> len, sel;
    // rank rule of the last shared fit of each tensor: per group its own
    // rank and the energy fractions of the first r - 1 and r channels at
    // the shared rank r (empty after palu_set_basis)
    bool energy_rule[2] = {false, false};
    std::vector<int> rank_g[2];
    std::vector<double> frac_prev[2], frac_at[2];

    bool quantized(int t) const { return t == 0 || cfg.quantize_values; }
    int bset(int slot) const { return per_seq ? slot : 0; }
    bool slot_ready(int slot) const { return ready[0][bset(slot)] && ready[1][bset(slot)]; }
    // rank and record layout of tensor t are known
    bool layout_known(int t) const { return per_seq || ready[t][0]; }
    size_t basis_elems(int t) const { return static_cast<size_t>(G) * D * r[t]; }
    size_t mu_elems() const { return static_cast<size_t>(G) * D; }
    // words of one record at fitted rank rr
    int words_for(int t, int rr) const {
        return quantized(t) ? coder_words(coder_for(cfg, rr, nullptr)) : fp16_record_words(rr);
    }
    TensorDev tensor_dev(int t) const {
        TensorDev d{};
        d.r = rc[t];
        d.cd = cd[t];
        d.words = words_for(t, r[t]);
        d.fp16_latents = quantized(t) ? 0 : 1;
        d.head_stride = (static_cast<int64_t>(max_groups) * d.words + 3) / 4 * 4;
        d.records = reinterpret_cast<uint32_t *>(dev + off_rec[t]);
        d.tail = quantized(t) ? reinterpret_cast<float *>(dev + off_tail[t]) : nullptr;
        d.basis = reinterpret_cast<float *>(dev + off_basis[t]);
        d.basis_t16 = reinterpret_cast<uint16_t *>(dev + off_bt16[t]);
        d.basis_cm = reinterpret_cast<float *>(dev + off_bcm[t]);
        d.mu = reinterpret_cast<float *>(dev + off_mu[t]);
        if (per_seq) {
            d.set_basis = sb_basis;
            d.set_bt16 = sb_bt16;
            d.set_bcm = sb_bcm;
            d.set_mu = sb_mu;
        }
        return d;
    }
};

namespace {

int validate_config(const palu_config *c) {
    if (!c) return fail(PALU_ERR_INVALID_ARG, "config is NULL");
    if (c->head_dim <= 0 || c->n_kv_heads <= 0 || c->n_q_heads <= 0 || c->n_head_groups <= 0)
        return fail(PALU_ERR_INVALID_ARG, "head_dim, n_kv_heads, n_q_heads and n_head_groups must be positive");
    if (c->n_kv_heads % c->n_head_groups != 0)
        return fail(PALU_ERR_INVALID_ARG, "n_kv_heads must be a multiple of n_head_groups (contiguous groups)");
    if (c->n_q_heads % c->n_kv_heads != 0)
        return fail(PALU_ERR_INVALID_ARG, "n_q_heads must be a multiple of n_kv_heads");
    if (c->rank < 0) return fail(PALU_ERR_INVALID_ARG, "rank must be >= 0 (0 selects the energy rule)");
    if (!(c->energy_threshold > 0.0f && c->energy_threshold <= 1.0f))
        return fail(PALU_ERR_INVALID_ARG, "energy_threshold must be in (0, 1]");
    if (!(c->hi_fraction >= 0.0f && c->hi_fraction <= 1.0f))
        return fail(PALU_ERR_INVALID_ARG, "hi_fraction must be in [0, 1]");
    if (c->max_rank < 0 || c->max_rank > c->head_dim)
        return fail(PALU_ERR_INVALID_ARG, "max_rank must be in [0, head_dim]");
    if (c->split_groups < 0) return fail(PALU_ERR_INVALID_ARG, "split_groups must be >= 0 (0 = automatic)");
    if (c->quantize_values != 0 && c->quantize_values != 1)
        return fail(PALU_ERR_INVALID_ARG, "quantize_values must be 0 or 1");
    if (c->input_dtype != 0 && c->input_dtype != 1)
        return fail(PALU_ERR_INVALID_ARG, "input_dtype must be 0 (fp16) or 1 (bf16)");
    if (c->head_dim != kHeadDim)
        return fail(PALU_ERR_UNSUPPORTED, "only head_dim = 128 is implemented by the kernels");
    if (!valid_width(c->hi_bit) || !valid_width(c->lo_bit))
        return fail(PALU_ERR_UNSUPPORTED, "hi_bit and lo_bit must be 1, 2, 4 or 8");
    if (c->schedule_len < 0 || c->schedule_len > 8)
        return fail(PALU_ERR_INVALID_ARG, "schedule_len must be in [0, 8]");
    if (c->schedule_len > 0) {
        bool any = false;
        for (int i = 0; i < c->schedule_len; ++i) {
            if (c->bit_schedule[i] != 0 && !valid_width(c->bit_schedule[i]))
                return fail(PALU_ERR_UNSUPPORTED, "bit_schedule entries must be 0, 1, 2, 4 or 8");
            any = any || c->bit_schedule[i] > 0;
        }
        if (!any) return fail(PALU_ERR_INVALID_ARG, "bit_schedule codes no channel (all entries 0)");
    }
    if (c->group_size != kTokGroup)
        return fail(PALU_ERR_UNSUPPORTED, "only group_size = 32 is implemented");
    if (c->n_q_heads / c->n_kv_heads > kMaxGqa)
        return fail(PALU_ERR_UNSUPPORTED, "at most 8 query heads per kv head are implemented");
    if (c->per_seq_basis != 0 && c->per_seq_basis != 1)
        return fail(PALU_ERR_INVALID_ARG, "per_seq_basis must be 0 or 1");
    if (c->per_seq_basis && c->rank <= 0)
        return fail(PALU_ERR_UNSUPPORTED, "per-sequence bases need an explicit rank (all slots share one record layout)");
    return PALU_OK;
}

int check_bound(const palu_cache *c) {
    if (!c) return fail(PALU_ERR_INVALID_ARG, "cache is NULL");
    if (!c->dev) return fail(PALU_ERR_NOT_BOUND, "no device storage bound (call palu_cache_bind)");
    return PALU_OK;
}

// Bound, and with shared bases both installed (per-sequence bases are
// checked per slot by check_slot).
int check_fitted(const palu_cache *c) {
    if (int e = check_bound(c)) return e;
    if (!c->per_seq && (!c->ready[0][0] || !c->ready[1][0]))
        return fail(PALU_ERR_NOT_FITTED, "no basis for K and V yet (call palu_fit or palu_set_basis)");
    return PALU_OK;
}

// slot in range and its bases installed
int check_slot(const palu_cache *c, int slot) {
    if (slot < 0 || slot >= c->max_batch)
        return fail(PALU_ERR_CAPACITY, "sequence slot " + std::to_string(slot) + " out of [0, max_batch)");
    if (!c->slot_ready(slot))
        return fail(PALU_ERR_NOT_FITTED, "no K and V bases for slot " + std::to_string(slot) +
                                             " (call palu_fit_seq or palu_set_basis_seq)");
    return PALU_OK;
}

void reset_seqs(palu_cache *c) {
    std::fill(c->len.begin(), c->len.end(), 0);
    std::fill(c->sel.begin(), c->sel.end(), 0);
}

int *dev_len(const palu_cache *c) { return reinterpret_cast<int *>(c->dev + c->off_len); }
int *dev_sel(const palu_cache *c) { return dev_len(c) + c->max_batch; }
int *dev_row_info(const palu_cache *c) { return dev_len(c) + 2 * c->max_batch; }

// The host's lengths and tail buffers -> their device copies (read by the
// decode step).  Called by the synchronous calls that change them on the
// host only; stream-ordered calls keep the copies current in their kernels.
int push_lengths(palu_cache *c) {
    if (!c->dev) return PALU_OK;
    hipError_t e = hipMemcpy(dev_len(c), c->len.data(), sizeof(int) * c->max_batch, hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemcpy(dev_sel(c), c->sel.data(), sizeof(int) * c->max_batch, hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(e, "length upload");
    return PALU_OK;
}

// Fails when tensor t at rank rr would store no latent channel (a bit
// schedule of zeros there); touches nothing of the cache.
int check_coder(const palu_cache *c, int t, int rr) {
    if (!c->quantized(t)) return PALU_OK;
    std::vector<int> coded;
    coder_for(c->cfg, rr, &coded);
    if (coded.empty()) return fail(PALU_ERR_UNSUPPORTED, "the bit schedule codes no channel at rank " + std::to_string(rr));
    return PALU_OK;
}

// Sets tensor t's coder (segments, coded channels) for its rank.
int set_coder(palu_cache *c, int t) {
    const int rr = c->r[t];
    if (c->quantized(t)) {
        c->cd[t] = coder_for(c->cfg, rr, &c->coded[t]);
    } else {
        c->cd[t] = Coder{};
        c->coded[t].resize(rr);
        std::iota(c->coded[t].begin(), c->coded[t].end(), 0);
    }
    const int rc = static_cast<int>(c->coded[t].size());
    if (rc == 0) return fail(PALU_ERR_UNSUPPORTED, "the bit schedule codes no channel at rank " + std::to_string(rr));
    c->rc[t] = rc;
    return PALU_OK;
}

// Uploads basis set `set` of tensor t (host copy in basis_h / mu_h) for the
// coded channels: fp32 [G][D][rc], channel-major fp32 [G][rc][D], the
// position-ordered fp16 copy and the mean.  0-bit channels are left out:
// their latents are zero by definition.  The coder must be set.
int upload_basis(palu_cache *c, int t, int set) {
    const int G = c->G, D = c->D, rr = c->r[t], rc = c->rc[t];
    const float *src = c->basis_h[t].data() + set * c->basis_elems(t);
    std::vector<float> bk(static_cast<size_t>(G) * D * rc), cm(static_cast<size_t>(G) * rc * D);
    for (int g = 0; g < G; ++g)
        for (int d = 0; d < D; ++d)
            for (int k = 0; k < rc; ++k) {
                const float v = src[(static_cast<size_t>(g) * D + d) * rr + c->coded[t][k]];
                bk[(static_cast<size_t>(g) * D + d) * rc + k] = v;
                cm[(static_cast<size_t>(g) * rc + k) * D + d] = v;
            }
    const TensorDev td = c->tensor_dev(t);
    float *basis = td.basis + set * td.set_basis;
    hipError_t e = hipMemcpy(basis, bk.data(), bk.size() * sizeof(float), hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(e, "basis upload");
    e = hipMemcpy(td.mu + set * td.set_mu, c->mu_h[t].data() + set * c->mu_elems(), c->mu_elems() * sizeof(float),
                  hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(e, "mean upload");
    e = hipMemcpy(td.basis_cm + set * td.set_bcm, cm.data(), cm.size() * sizeof(float), hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(e, "channel-major basis upload");
    if (t == 0) {   // only the key basis is absorbed into queries
        e = launch_basis_t16(basis, td.basis_t16 + set * td.set_bt16, G, rc, c->cd[t], nullptr);
        if (e != hipSuccess) return hip_fail(e, "basis fp16 copy");
    }
    e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_fail(e, "basis upload synchronize");
    return PALU_OK;
}

// Installs a basis (host [G][D][r], mean [G][D], sigma [G][D] or null)
// as set `set` of tensor t and uploads it.
int install_basis(palu_cache *c, int t, int set, const float *basis, const float *mu, const double *sigma) {
    const size_t nb = c->basis_elems(t), nm = c->mu_elems();
    c->ready[t][set] = 0;
    std::copy(basis, basis + nb, c->basis_h[t].begin() + set * nb);
    std::copy(mu, mu + nm, c->mu_h[t].begin() + set * nm);
    if (sigma) std::copy(sigma, sigma + nm, c->sigma_h[t].begin() + set * nm);
    else std::fill(c->sigma_h[t].begin() + set * nm, c->sigma_h[t].begin() + (set + 1) * nm, 0.0);
    if (int e = upload_basis(c, t, set)) return e;
    c->ready[t][set] = 1;
    return PALU_OK;
}

// Shared bases: sizes the host copies of tensor t for rank rr.
void size_shared(palu_cache *c, int t, int rr) {
    c->r[t] = rr;
    c->basis_h[t].assign(c->basis_elems(t), 0.0f);
    c->mu_h[t].assign(c->mu_elems(), 0.0f);
    c->sigma_h[t].assign(c->mu_elems(), 0.0);
}

}  // namespace

PALU_API int palu_config_default(palu_config *cfg, int32_t head_dim, int32_t n_kv_heads,
                                 int32_t n_q_heads) {
    if (!cfg) return fail(PALU_ERR_INVALID_ARG, "config is NULL");
    cfg->head_dim = head_dim;
    cfg->n_kv_heads = n_kv_heads;
    cfg->n_q_heads = n_q_heads;
    cfg->n_head_groups = 4;
    cfg->rank = 0;
    cfg->energy_threshold = 0.90f;
    cfg->hi_bit = 4;
    cfg->lo_bit = 2;
    cfg->hi_fraction = 0.25f;
    cfg->group_size = 32;
    cfg->quantize_values = 1;
    cfg->max_rank = 0;
    cfg->split_groups = 0;
    cfg->input_dtype = 0;
    cfg->schedule_len = 0;
    for (int i = 0; i < 8; ++i) cfg->bit_schedule[i] = 0;
    cfg->per_seq_basis = 0;
    return PALU_OK;
}

PALU_API int palu_cache_create(const palu_config *cfg, int32_t max_batch, int32_t max_seq_len,
                               palu_cache **out) {
    if (!out) return fail(PALU_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (int e = validate_config(cfg)) return e;
    if (max_batch <= 0 || max_seq_len <= 0)
        return fail(PALU_ERR_INVALID_ARG, "max_batch and max_seq_len must be positive");
    if (cfg->rank > 0 && cfg->max_rank > 0 && cfg->rank > cfg->max_rank)
        return fail(PALU_ERR_INVALID_ARG, "rank exceeds max_rank");
    palu_cache *c = new palu_cache();
    c->cfg = *cfg;
    c->max_batch = max_batch;
    c->max_seq_len = max_seq_len;
    c->D = cfg->head_dim;
    c->H = cfg->n_kv_heads;
    c->Hq = cfg->n_q_heads;
    c->G = cfg->n_head_groups;
    c->hpg = c->H / c->G;
    c->gqa = c->Hq / c->H;
    c->r_max = cfg->max_rank > 0 ? cfg->max_rank : c->D;
    c->max_groups = (max_seq_len + kTokGroup - 1) / kTokGroup;
    c->len.assign(max_batch, 0);
    c->sel.assign(max_batch, 0);

    // device layout, sized for r_max
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes, 256);
        return o;
    };
    c->per_seq = cfg->per_seq_basis != 0;
    c->nbs = c->per_seq ? max_batch : 1;
    // with per-sequence bases the rank is fixed: regions sized for it
    const int r_alloc = c->per_seq ? std::min(cfg->rank, c->D) : c->r_max;
    c->sb_basis = static_cast<int64_t>(c->G) * c->D * r_alloc;
    c->sb_bt16 = static_cast<int64_t>(c->G) * c->D * (r_alloc + 8 * kMaxSegs);   // >= basis_t16_rows
    c->sb_bcm = c->sb_basis;
    c->sb_mu = static_cast<int64_t>(c->G) * c->D;
    for (int t = 0; t < 2; ++t) {
        c->ready[t].assign(c->nbs, 0);
        // + 4 floats of slack: the encode projection reads whole groups of
        // 4 channels, up to 3 past the last row of the last basis
        c->off_basis[t] = take(sizeof(float) * (c->nbs * c->sb_basis + 4));
        // only the key basis is absorbed into queries: no fp16 copy of V's
        c->off_bt16[t] = t == 0 ? take(sizeof(uint16_t) * c->nbs * c->sb_bt16) : 0;
        c->off_bcm[t] = take(sizeof(float) * c->nbs * c->sb_bcm);
        c->off_mu[t] = take(sizeof(float) * c->nbs * c->sb_mu);
        const size_t head_words = (static_cast<size_t>(c->max_groups) * c->words_for(t, r_alloc) + 3) / 4 * 4;
        c->off_rec[t] = take(sizeof(uint32_t) * static_cast<size_t>(max_batch) * c->H * head_words);
        c->off_tail[t] = c->quantized(t)
                             ? take(sizeof(float) * static_cast<size_t>(max_batch) * c->H * 2 * kTokGroup * r_alloc)
                             : 0;
        if (c->per_seq) {
            c->r[t] = r_alloc;
            if (int e = set_coder(c, t)) {
                delete c;
                return e;
            }
            c->basis_h[t].assign(c->nbs * c->basis_elems(t), 0.0f);
            c->mu_h[t].assign(c->nbs * c->mu_elems(), 0.0f);
            c->sigma_h[t].assign(c->nbs * c->mu_elems(), 0.0);
        }
    }
    // Gram blocks of one fit: at most the target count of full blocks (or
    // the count at the largest block size), plus one partial block per
    // (sequence, head-in-group) segment
    const int64_t n_rows_max = static_cast<int64_t>(max_batch) * max_seq_len * c->hpg;
    c->gram_nb_cap = static_cast<int>(std::max<int64_t>(gram_nb_target(c->G), (n_rows_max + kGramMaxRowsPerBlock - 1) /
                                                                                  kGramMaxRowsPerBlock) +
                                      static_cast<int64_t>(max_batch) * c->hpg);
    c->off_gram_part = take(sizeof(float) * 2 * static_cast<size_t>(c->G) * c->gram_nb_cap * kGramElems);
    c->off_gram_out = take(sizeof(double) * 2 * static_cast<size_t>(c->G) * kGramElems);
    // block tables: one fit's (shared), or one per row (per-sequence fit)
    c->gram_tab_cap = std::max<int64_t>(c->gram_nb_cap, static_cast<int64_t>(max_batch) *
                                                            (gram_nb_target(c->G) + c->hpg));
    c->off_seg = take(sizeof(GramBlock) * static_cast<size_t>(c->gram_tab_cap));
    // decode rows may repeat slots, so a launch can hold kMaxCallSeqs rows
    // whatever max_batch is
    c->off_attend = take(sizeof(float) * static_cast<size_t>(kMaxCallSeqs) * c->Hq * kMaxSplits * (c->r_max + 2));
    // per-slot length and tail buffer (device copies of len / sel), then
    // (length, splits) of each row of a decode step
    c->off_len = take(sizeof(int32_t) * (2 * static_cast<size_t>(max_batch) + 2 * kMaxCallSeqs));
    c->total = off;
    *out = c;
    return PALU_OK;
}

PALU_API int palu_cache_required_bytes(const palu_cache *c, size_t *dev_bytes) {
    if (!c || !dev_bytes) return fail(PALU_ERR_INVALID_ARG, "cache or dev_bytes is NULL");
    *dev_bytes = c->total;
    return PALU_OK;
}

PALU_API int palu_cache_bind(palu_cache *c, void *dev_buf, size_t bytes) {
    if (!c || !dev_buf) return fail(PALU_ERR_INVALID_ARG, "cache or dev_buf is NULL");
    if (bytes < c->total)
        return fail(PALU_ERR_INVALID_ARG, "bound buffer has " + std::to_string(bytes) + " bytes, " +
                                              std::to_string(c->total) + " required");
    if (reinterpret_cast<uintptr_t>(dev_buf) % 256 != 0)
        return fail(PALU_ERR_INVALID_ARG, "bound buffer must be 256-byte aligned");
    c->dev = static_cast<char *>(dev_buf);
    c->dev_bytes = bytes;
    for (int t = 0; t < 2; ++t) {
        std::fill(c->ready[t].begin(), c->ready[t].end(), 0);
        c->rank_g[t].clear();
    }
    // the device copies of the lengths are written by the fit or basis
    // installation that every slot needs before its first token
    reset_seqs(c);
    return PALU_OK;
}

namespace {

// Gram blocks over rows b < B of k / v (seq_lens[b] tokens, every head of
// the group): at most R rows of one (sequence, head-in-group) segment each,
// R chosen for about nb_target full blocks per (tensor, group).
void gram_blocks(const int32_t *seq_lens, int B, int hpg, int G, int nb_target, std::vector<GramBlock> &out) {
    int64_t n_rows = 0;
    for (int b = 0; b < B; ++b) n_rows += static_cast<int64_t>(hpg) * seq_lens[b];
    int64_t R = std::max<int64_t>(kGramRowsPerBlockMin, (n_rows + nb_target - 1) / nb_target);
    R = std::min<int64_t>((R + 63) / 64 * 64, kGramMaxRowsPerBlock);
    // a segment of L rows gets k = ceil(L / R) blocks; block i takes tiles
    // i, i + k, i + 2k, ... (concurrent blocks read adjacent tiles)
    for (int b = 0; b < B; ++b)
        for (int hh = 0; hh < hpg; ++hh) {
            const int64_t L = seq_lens[b], k = (L + R - 1) / R;
            for (int64_t i = 0; i < k; ++i)
                out.push_back(GramBlock{b * hpg + hh, static_cast<int>(64 * i), static_cast<int>(L),
                                        static_cast<int>(64 * k)});
        }
}

// Compute units of the current device (256 when the query fails).
int device_cus(palu_cache *c) {
    if (c->n_cus == 0) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        c->n_cus = n;
    }
    return c->n_cus;
}

// Full Gram blocks per (tensor, group): as many as the device holds at once
// over both tensors and all groups (one round of equal blocks), within
// gram_nb_target.
int gram_target(palu_cache *c) {
    if (c->gram_resident == 0) {
        int n = 0;
        if (gram_resident_blocks(&n) != hipSuccess || n <= 0) n = 1024;
        c->gram_resident = n;
    }
    return std::max(1, std::min(gram_nb_target(c->G), c->gram_resident / (2 * c->G)));
}

// Gram partials of rows [b0, b0 + B) of k / v over the nb blocks at tab
// (device), reduced into the fp64 [2][G][D*D + D] result, whose download
// into gram_host is queued on s.
int queue_gram(palu_cache *c, const void *k, const void *v, int b0, int B, int S_stride, const GramBlock *tab,
               int nb, hipStream_t s, double *gram_host) {
    if (nb > c->gram_nb_cap) return fail(PALU_ERR_CAPACITY, "fit workspace too small for this many rows");
    const size_t row_elems = static_cast<size_t>(c->H) * S_stride * c->D;
    GramArgs ga{};
    ga.x[0] = static_cast<const uint16_t *>(k) + b0 * row_elems;
    ga.x[1] = static_cast<const uint16_t *>(v) + b0 * row_elems;
    ga.blocks = tab;
    ga.partial = reinterpret_cast<float *>(c->dev + c->off_gram_part);
    ga.B = B;
    ga.H = c->H;
    ga.S_stride = S_stride;
    ga.bf16 = c->cfg.input_dtype;
    ga.G = c->G;
    ga.hpg = c->hpg;
    ga.nb = nb;
    hipError_t e = launch_gram(ga, s);
    if (e != hipSuccess) return hip_fail(e, "gram launch");
    GramReduceArgs ra{};
    ra.partial = ga.partial;
    ra.out = reinterpret_cast<double *>(c->dev + c->off_gram_out);
    ra.G = c->G;
    ra.nb = nb;
    if ((e = launch_gram_reduce(ra, s)) != hipSuccess) return hip_fail(e, "gram reduce launch");
    e = hipMemcpyAsync(gram_host, ra.out, sizeof(double) * 2 * c->G * kGramElems, hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return hip_fail(e, "gram download");
    return PALU_OK;
}

// One fitted (tensor, group) problem: eigenvalues of the scatter matrix
// about the mean, X^T X - s s^T / N, then eigenvectors of the k largest.
struct FitProblem {
    const double *gram;   // D*D Gram, then D column sums
    double n;             // rows
    SymEigen se;          // reduction and eigenvalues (descending)
    int k = 0;            // eigenvectors wanted
    std::vector<double> z;   // [D][k]
    bool ok = false;
};

// Host worker threads kept for the life of the process: spawning and
// joining eight threads per call cost 0.1-0.2 ms, and a fit makes two such
// calls.  Items are handed out one at a time to the workers and to the
// calling thread; calls from several host threads queue on call_mu_.  Each
// call waits until every worker has seen it, so no worker still reads a
// call's job when the next one starts.  A forked child (which has none of
// its parent's threads) starts workers of its own.
class HostPool {
public:
    void run(int count, const std::function<void(int)> &f) {
        if (count <= 1) {
            for (int i = 0; i < count; ++i) f(i);
            return;
        }
        std::lock_guard<std::mutex> call(call_mu_);
        start_workers();
        {
            std::lock_guard<std::mutex> lk(mu_);
            job_ = &f;
            count_ = count;
            next_.store(0);
            pending_ = static_cast<int>(workers_->size());
            ++gen_;
        }
        cv_.notify_all();
        take_items();
        std::unique_lock<std::mutex> lk(mu_);
        done_cv_.wait(lk, [&] { return pending_ == 0; });
        job_ = nullptr;
    }
    ~HostPool() {
        if (!workers_ || pid_ != getpid()) return;
        {
            std::lock_guard<std::mutex> lk(mu_);
            stop_ = true;
        }
        cv_.notify_all();
        for (auto &t : *workers_) t.join();
        delete workers_;
    }

private:
    void start_workers() {
        if (workers_ && pid_ == getpid()) return;
        // (after a fork the parent's thread objects are dropped unjoined:
        // leaked on purpose, their threads do not exist here)
        pid_ = getpid();
        stop_ = false;
        const unsigned hw = std::max(1u, std::thread::hardware_concurrency());
        const int n = static_cast<int>(std::min(hw, 16u)) - 1;
        workers_ = new std::vector<std::thread>();
        // the generation before this call's: a worker that starts late
        // still takes part in it (gen_ changes only under call_mu_)
        const uint64_t g0 = gen_;
        for (int w = 0; w < n; ++w) workers_->emplace_back([this, g0] { worker(g0); });
    }
    void take_items() {
        for (int i = next_.fetch_add(1); i < count_; i = next_.fetch_add(1)) (*job_)(i);
    }
    void worker(uint64_t seen) {
        for (;;) {
            {
                std::unique_lock<std::mutex> lk(mu_);
                cv_.wait(lk, [&] { return stop_ || gen_ != seen; });
                if (stop_) return;
                seen = gen_;
            }
            take_items();
            std::lock_guard<std::mutex> lk(mu_);
            if (--pending_ == 0) done_cv_.notify_one();
        }
    }

    std::mutex call_mu_, mu_;
    std::condition_variable cv_, done_cv_;
    std::vector<std::thread> *workers_ = nullptr;
    pid_t pid_ = 0;
    const std::function<void(int)> *job_ = nullptr;
    int count_ = 0, pending_ = 0;
    std::atomic<int> next_{0};
    uint64_t gen_ = 0;
    bool stop_ = false;
};

HostPool &host_pool() {
    static HostPool pool;
    return pool;
}

// f(i) for i < count on host threads (the problems are independent).
template <typename F>
void parallel_for(int count, F f) {
    host_pool().run(count, std::function<void(int)>(f));
}

// Step 1 of every problem: scatter matrix, reduction, eigenvalues.
void solve_values(int D, std::vector<FitProblem> &pr) {
    parallel_for(static_cast<int>(pr.size()), [&](int i) {
        FitProblem &p = pr[i];
        std::vector<double> cov(static_cast<size_t>(D) * D);
        const double *sum = p.gram + D * D;
        for (int a = 0; a < D; ++a)
            for (int b = 0; b < D; ++b) cov[a * D + b] = p.gram[a * D + b] - sum[a] * sum[b] / p.n;
        for (int a = 0; a < D; ++a)
            for (int b = 0; b < a; ++b) {
                const double m = 0.5 * (cov[a * D + b] + cov[b * D + a]);
                cov[a * D + b] = cov[b * D + a] = m;
            }
        p.ok = sym_eigenvalues(cov.data(), D, p.se);
    });
}

// Step 2: eigenvectors of the p.k largest eigenvalues of every problem.
void solve_vectors(int D, std::vector<FitProblem> &pr) {
    parallel_for(static_cast<int>(pr.size()), [&](int i) {
        FitProblem &p = pr[i];
        p.z.assign(static_cast<size_t>(D) * p.k, 0.0);
        sym_top_vectors(p.se, p.k, p.z.data());
    });
}

// Squared singular values s2 (clamped at 0), sigma and the mean of a problem.
void spectrum_of(const FitProblem &p, int D, double *s2, double *sigma, float *mu) {
    for (int c = 0; c < D; ++c) {
        s2[c] = p.se.w[c] > 0.0 ? p.se.w[c] : 0.0;
        sigma[c] = std::sqrt(s2[c]);
    }
    const double *sum = p.gram + D * D;
    for (int d = 0; d < D; ++d) mu[d] = static_cast<float>(sum[d] / p.n);
}

// Basis columns c < r of a problem (descending eigenvalue order), each
// signed so that its largest-magnitude component is positive, into fp32
// dst[d * r + c].
void basis_of(const FitProblem &p, int D, int r, float *dst) {
    for (int c = 0; c < r; ++c) {
        int arg = 0;
        for (int d = 1; d < D; ++d)
            if (std::fabs(p.z[static_cast<size_t>(d) * p.k + c]) > std::fabs(p.z[static_cast<size_t>(arg) * p.k + c]))
                arg = d;
        const double sg = p.z[static_cast<size_t>(arg) * p.k + c] < 0.0 ? -1.0 : 1.0;
        for (int d = 0; d < D; ++d)
            dst[static_cast<size_t>(d) * r + c] = static_cast<float>(sg * p.z[static_cast<size_t>(d) * p.k + c]);
    }
}

// Smallest rank whose leading squared singular values reach tau of the
// total (1 when the total is zero).
int energy_rank(const double *s2, int D, float tau) {
    double tot = 0.0;
    for (int i = 0; i < D; ++i) tot += s2[i];
    if (tot <= 0.0) return 1;
    double acc = 0.0;
    for (int kk = 1; kk <= D; ++kk) {
        acc += s2[kk - 1];
        if (acc >= static_cast<double>(tau) * tot) return kk;
    }
    return D;
}

// Fit argument checks shared by both modes.
int check_fit_args(const palu_cache *c, const void *k, const void *v, const int32_t *seq_lens, int B,
                   int S_stride) {
    if (int e = check_bound(c)) return e;
    if (!k || !v || !seq_lens) return fail(PALU_ERR_INVALID_ARG, "k, v and seq_lens must be non-NULL");
    if (B <= 0 || B > c->max_batch) return fail(PALU_ERR_INVALID_ARG, "B must be in [1, max_batch]");
    if (S_stride <= 0) return fail(PALU_ERR_INVALID_ARG, "S_stride must be positive");
    for (int b = 0; b < B; ++b)
        if (seq_lens[b] < 0 || seq_lens[b] > S_stride || seq_lens[b] > c->max_seq_len)
            return fail(PALU_ERR_INVALID_ARG, "seq_lens[" + std::to_string(b) + "] out of [0, min(S_stride, max_seq_len)]");
    return PALU_OK;
}

// Per-sequence fit: row b of k / v -> basis sets of slot ids[b].
int fit_per_seq(palu_cache *c, const void *k, const void *v, const int32_t *ids, const int32_t *seq_lens, int B,
                int S_stride, hipStream_t s) {
    const int hpg = c->hpg, D = c->D, G = c->G;
    std::vector<char> seen(c->max_batch, 0);
    for (int b = 0; b < B; ++b) {
        const int slot = ids ? ids[b] : b;
        if (slot < 0 || slot >= c->max_batch)
            return fail(PALU_ERR_CAPACITY, "sequence slot " + std::to_string(slot) + " out of [0, max_batch)");
        if (seen[slot]) return fail(PALU_ERR_INVALID_ARG, "sequence slot listed twice in one call");
        seen[slot] = 1;
        if (seq_lens[b] <= 0) return fail(PALU_ERR_INVALID_ARG, "a per-sequence fit needs at least one token per row");
    }
    // each row's block table, all uploaded at once
    std::vector<GramBlock> tab;
    std::vector<size_t> first(B + 1, 0);
    for (int b = 0; b < B; ++b) {
        gram_blocks(seq_lens + b, 1, hpg, G, gram_target(c), tab);
        first[b + 1] = tab.size();
    }
    if (static_cast<int64_t>(tab.size()) > c->gram_tab_cap)
        return fail(PALU_ERR_CAPACITY, "fit workspace too small for this many rows");
    hipError_t e = hipMemcpyAsync(c->dev + c->off_seg, tab.data(), sizeof(GramBlock) * tab.size(),
                                  hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "fit block table upload");
    const size_t per = 2 * static_cast<size_t>(G) * kGramElems;
    std::vector<double> gram(per * B);
    const GramBlock *dtab = reinterpret_cast<const GramBlock *>(c->dev + c->off_seg);
    for (int b = 0; b < B; ++b)
        if (int err = queue_gram(c, k, v, b, 1, S_stride, dtab + first[b], static_cast<int>(first[b + 1] - first[b]),
                                 s, gram.data() + per * b))
            return err;
    if ((e = hipStreamSynchronize(s)) != hipSuccess) return hip_fail(e, "fit synchronize");

    std::vector<FitProblem> pr(static_cast<size_t>(B) * 2 * G);
    for (int b = 0; b < B; ++b)
        for (int pb = 0; pb < 2 * G; ++pb) {
            FitProblem &p = pr[static_cast<size_t>(b) * 2 * G + pb];
            p.gram = gram.data() + per * b + static_cast<size_t>(pb) * kGramElems;
            p.n = static_cast<double>(hpg) * seq_lens[b];
        }
    solve_values(D, pr);
    for (const auto &p : pr)
        if (!p.ok) return fail(PALU_ERR_HIP, "eigensolver did not converge");
    for (int b = 0; b < B; ++b)
        for (int pb = 0; pb < 2 * G; ++pb) pr[static_cast<size_t>(b) * 2 * G + pb].k = c->r[pb / G];
    solve_vectors(D, pr);
    std::vector<double> s2(D);
    for (int b = 0; b < B; ++b) {
        const int slot = ids ? ids[b] : b;
        c->len[slot] = 0;
        c->sel[slot] = 0;
        for (int t = 0; t < 2; ++t) {
            const int rr = c->r[t];
            std::vector<float> basis(c->basis_elems(t)), mu(c->mu_elems());
            std::vector<double> sigma(c->mu_elems());
            for (int g = 0; g < G; ++g) {
                const FitProblem &p = pr[(static_cast<size_t>(b) * 2 + t) * G + g];
                spectrum_of(p, D, s2.data(), sigma.data() + static_cast<size_t>(g) * D,
                            mu.data() + static_cast<size_t>(g) * D);
                basis_of(p, D, rr, basis.data() + static_cast<size_t>(g) * D * rr);
            }
            if (int err = install_basis(c, t, slot, basis.data(), mu.data(), sigma.data())) return err;
        }
    }
    return push_lengths(c);
}

}  // namespace

PALU_API int palu_fit(palu_cache *c, const void *k, const void *v, const int32_t *seq_lens, int32_t B,
                      int32_t S_stride, void *stream) {
    if (int e = check_fit_args(c, k, v, seq_lens, B, S_stride)) return e;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (c->per_seq) return fit_per_seq(c, k, v, nullptr, seq_lens, B, S_stride, s);
    int64_t total = 0;
    for (int b = 0; b < B; ++b) total += seq_lens[b];
    if (total == 0) return fail(PALU_ERR_INVALID_ARG, "no valid tokens to fit");
    // Until every check below has passed (block table, eigensolver, ranks,
    // coder) the cache keeps its bases and stored tokens: the Gram kernels
    // write only the fit scratch.

    const int64_t n_rows = total * c->hpg;
    std::vector<GramBlock> tab;
    gram_blocks(seq_lens, B, c->hpg, c->G, gram_target(c), tab);
    if (static_cast<int64_t>(tab.size()) > c->gram_tab_cap)
        return fail(PALU_ERR_CAPACITY, "fit workspace too small for this many rows");
    hipError_t e = hipMemcpyAsync(c->dev + c->off_seg, tab.data(), sizeof(GramBlock) * tab.size(),
                                  hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "fit block table upload");
    std::vector<double> gram(2 * static_cast<size_t>(c->G) * kGramElems);
    if (int err = queue_gram(c, k, v, 0, B, S_stride, reinterpret_cast<const GramBlock *>(c->dev + c->off_seg),
                             static_cast<int>(tab.size()), s, gram.data()))
        return err;
    if ((e = hipStreamSynchronize(s)) != hipSuccess) return hip_fail(e, "fit synchronize");

    const int D = c->D, G = c->G;
    std::vector<FitProblem> pr(2 * G);
    for (int pb = 0; pb < 2 * G; ++pb) {
        pr[pb].gram = gram.data() + static_cast<size_t>(pb) * kGramElems;
        pr[pb].n = static_cast<double>(n_rows);
    }
    solve_values(D, pr);
    for (const auto &p : pr)
        if (!p.ok) return fail(PALU_ERR_HIP, "eigensolver did not converge");
    // ranks from the eigenvalues (the minimum over groups), then only that
    // many eigenvectors per problem
    int rt[2];
    std::vector<double> s2(static_cast<size_t>(2) * G * D), sigma(static_cast<size_t>(2) * G * D);
    std::vector<float> mu(static_cast<size_t>(2) * G * D);
    std::vector<int> rank_g[2];
    std::vector<double> frac_prev[2], frac_at[2];
    for (int t = 0; t < 2; ++t) {
        int rr = D;
        rank_g[t].resize(G);
        for (int g = 0; g < G; ++g) {
            const size_t off = (static_cast<size_t>(t) * G + g) * D;
            spectrum_of(pr[t * G + g], D, s2.data() + off, sigma.data() + off, mu.data() + off);
            rank_g[t][g] = c->cfg.rank > 0 ? std::min(c->cfg.rank, D)
                                           : energy_rank(s2.data() + off, D, c->cfg.energy_threshold);
            rr = std::min(rr, rank_g[t][g]);
        }
        if (rr > c->r_max)
            return fail(PALU_ERR_CAPACITY, "fitted rank " + std::to_string(rr) + " exceeds max_rank " +
                                               std::to_string(c->r_max));
        if (int err = check_coder(c, t, rr)) return err;
        rt[t] = rr;
        for (int g = 0; g < G; ++g) pr[t * G + g].k = rr;
        // energy fractions of each group's first rr - 1 and rr channels
        frac_prev[t].assign(G, 0.0);
        frac_at[t].assign(G, 0.0);
        for (int g = 0; g < G; ++g) {
            const double *e = s2.data() + (static_cast<size_t>(t) * G + g) * D;
            double tot = 0.0, acc = 0.0;
            for (int i = 0; i < D; ++i) tot += e[i];
            for (int i = 0; i < rr; ++i) {
                if (i == rr - 1) frac_prev[t][g] = tot > 0.0 ? acc / tot : 0.0;
                acc += e[i];
            }
            frac_at[t][g] = tot > 0.0 ? acc / tot : 1.0;
        }
    }
    solve_vectors(D, pr);
    // every check has passed: the old bases and stored tokens go
    c->ready[0][0] = c->ready[1][0] = 0;
    reset_seqs(c);
    if (int err = push_lengths(c)) return err;
    for (int t = 0; t < 2; ++t) {
        c->energy_rule[t] = c->cfg.rank <= 0;
        c->rank_g[t] = rank_g[t];
        c->frac_prev[t] = frac_prev[t];
        c->frac_at[t] = frac_at[t];
    }
    for (int t = 0; t < 2; ++t) {
        const int rr = rt[t];
        size_shared(c, t, rr);
        std::vector<float> basis(c->basis_elems(t));
        for (int g = 0; g < G; ++g) basis_of(pr[t * G + g], D, rr, basis.data() + static_cast<size_t>(g) * D * rr);
        if (int err = set_coder(c, t)) return err;
        const size_t off = static_cast<size_t>(t) * G * D;
        if (int err = install_basis(c, t, 0, basis.data(), mu.data() + off, sigma.data() + off)) return err;
    }
    return PALU_OK;
}

PALU_API int palu_fit_seq(palu_cache *c, const void *k, const void *v, const int32_t *seq_ids,
                          const int32_t *seq_lens, int32_t B, int32_t S_stride, void *stream) {
    if (int e = check_fit_args(c, k, v, seq_lens, B, S_stride)) return e;
    if (!c->per_seq) return fail(PALU_ERR_INVALID_ARG, "palu_fit_seq needs per_seq_basis = 1");
    if (!seq_ids) return fail(PALU_ERR_INVALID_ARG, "seq_ids must be non-NULL");
    return fit_per_seq(c, k, v, seq_ids, seq_lens, B, S_stride, static_cast<hipStream_t>(stream));
}

PALU_API int palu_set_basis(palu_cache *c, int32_t tensor, int32_t r, const float *basis, const float *mu) {
    if (int e = check_bound(c)) return e;
    if (tensor != 0 && tensor != 1) return fail(PALU_ERR_INVALID_ARG, "tensor must be 0 (K) or 1 (V)");
    if (!basis || !mu) return fail(PALU_ERR_INVALID_ARG, "basis and mu must be non-NULL");
    if (c->per_seq) {
        // the same basis in every slot
        if (r != c->r[tensor]) return fail(PALU_ERR_INVALID_ARG, "r must equal the cache's rank");
        for (int set = 0; set < c->nbs; ++set)
            if (int e = install_basis(c, tensor, set, basis, mu, nullptr)) return e;
        reset_seqs(c);
        return push_lengths(c);
    }
    if (r < 1 || r > c->r_max) return fail(PALU_ERR_INVALID_ARG, "r must be in [1, max_rank]");
    if (int e = check_coder(c, tensor, r)) return e;
    c->ready[tensor][0] = 0;
    c->rank_g[tensor].clear();
    reset_seqs(c);
    if (int e = push_lengths(c)) return e;
    size_shared(c, tensor, r);
    if (int e = set_coder(c, tensor)) return e;
    return install_basis(c, tensor, 0, basis, mu, nullptr);
}

PALU_API int palu_set_basis_seq(palu_cache *c, int32_t seq, int32_t tensor, int32_t r, const float *basis,
                                const float *mu) {
    if (int e = check_bound(c)) return e;
    if (!c->per_seq) return fail(PALU_ERR_INVALID_ARG, "palu_set_basis_seq needs per_seq_basis = 1");
    if (tensor != 0 && tensor != 1) return fail(PALU_ERR_INVALID_ARG, "tensor must be 0 (K) or 1 (V)");
    if (seq < 0 || seq >= c->max_batch) return fail(PALU_ERR_CAPACITY, "sequence slot out of range");
    if (!basis || !mu) return fail(PALU_ERR_INVALID_ARG, "basis and mu must be non-NULL");
    if (r != c->r[tensor]) return fail(PALU_ERR_INVALID_ARG, "r must equal the cache's rank");
    c->len[seq] = 0;
    c->sel[seq] = 0;
    if (int e = push_lengths(c)) return e;
    return install_basis(c, tensor, seq, basis, mu, nullptr);
}

namespace {

int get_set(const palu_cache *c, int tensor, int set, int32_t *r, float *basis, float *mu, double *sigma) {
    if (!c->ready[tensor][set]) return fail(PALU_ERR_NOT_FITTED, "no basis for this tensor");
    const size_t nb = c->basis_elems(tensor), nm = c->mu_elems();
    if (r) *r = c->r[tensor];
    if (basis) std::memcpy(basis, c->basis_h[tensor].data() + set * nb, nb * sizeof(float));
    if (mu) std::memcpy(mu, c->mu_h[tensor].data() + set * nm, nm * sizeof(float));
    if (sigma) std::memcpy(sigma, c->sigma_h[tensor].data() + set * nm, nm * sizeof(double));
    return PALU_OK;
}

}  // namespace

PALU_API int palu_get_basis(const palu_cache *c, int32_t tensor, int32_t *r, float *basis, float *mu,
                            double *sigma) {
    if (!c) return fail(PALU_ERR_INVALID_ARG, "cache is NULL");
    if (tensor != 0 && tensor != 1) return fail(PALU_ERR_INVALID_ARG, "tensor must be 0 (K) or 1 (V)");
    if (c->per_seq) return fail(PALU_ERR_INVALID_ARG, "per-sequence bases: use palu_get_basis_seq");
    return get_set(c, tensor, 0, r, basis, mu, sigma);
}

PALU_API int palu_get_basis_seq(const palu_cache *c, int32_t seq, int32_t tensor, int32_t *r, float *basis,
                                float *mu, double *sigma) {
    if (!c) return fail(PALU_ERR_INVALID_ARG, "cache is NULL");
    if (!c->per_seq) return fail(PALU_ERR_INVALID_ARG, "palu_get_basis_seq needs per_seq_basis = 1");
    if (tensor != 0 && tensor != 1) return fail(PALU_ERR_INVALID_ARG, "tensor must be 0 (K) or 1 (V)");
    if (seq < 0 || seq >= c->max_batch) return fail(PALU_ERR_CAPACITY, "sequence slot out of range");
    return get_set(c, tensor, seq, r, basis, mu, sigma);
}

PALU_API int palu_encode_append(palu_cache *c, const void *k, const void *v, const int32_t *seq_ids,
                                const int32_t *n_new, int32_t B, int32_t T_stride, void *stream) {
    if (int e = check_fitted(c)) return e;
    if (!k || !v) return fail(PALU_ERR_INVALID_ARG, "k and v must be non-NULL");
    if (B <= 0) return fail(PALU_ERR_INVALID_ARG, "B must be positive");
    if (T_stride <= 0) return fail(PALU_ERR_INVALID_ARG, "T_stride must be positive");
    std::vector<char> seen(c->max_batch, 0);
    for (int b = 0; b < B; ++b) {
        const int slot = seq_ids ? seq_ids[b] : b;
        if (int e = check_slot(c, slot)) return e;
        if (seen[slot]) return fail(PALU_ERR_INVALID_ARG, "sequence slot listed twice in one call");
        seen[slot] = 1;
        const int n = n_new ? n_new[b] : T_stride;
        if (n < 0 || n > T_stride) return fail(PALU_ERR_INVALID_ARG, "n_new must be in [0, T_stride]");
        if (static_cast<int64_t>(c->len[slot]) + n > c->max_seq_len)
            return fail(PALU_ERR_CAPACITY, "append to slot " + std::to_string(slot) + " exceeds max_seq_len");
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t row_elems = static_cast<size_t>(c->H) * T_stride * c->D;
    for (int b0 = 0; b0 < B; b0 += kMaxCallSeqs) {
        const int nb = std::min(kMaxCallSeqs, B - b0);
        EncodeArgs ea{};
        ea.x[0] = static_cast<const uint16_t *>(k) + b0 * row_elems;
        ea.x[1] = static_cast<const uint16_t *>(v) + b0 * row_elems;
        ea.t[0] = c->tensor_dev(0);
        ea.t[1] = c->tensor_dev(1);
        ea.B = nb;
        ea.H = c->H;
        ea.T_stride = T_stride;
        ea.hpg = c->hpg;
        ea.bf16 = c->cfg.input_dtype;
        ea.len_dev = dev_len(c);
        ea.sel_dev = dev_sel(c);
        ea.max_len = c->max_seq_len;
        int max_units = 0;   // group pairs touched by a row (one wave each)
        for (int i = 0; i < nb; ++i) {
            const int b = b0 + i;
            const int slot = seq_ids ? seq_ids[b] : b;
            const int n = n_new ? n_new[b] : T_stride;
            const int o = c->len[slot];
            ea.slot[i] = slot;
            ea.old_len[i] = o;
            ea.n_new[i] = n;
            ea.sel_old[i] = c->sel[slot];
            // the incomplete group after the append lives in the other tail
            // buffer whenever a different group was incomplete before, so
            // the workgroup that completes the old group can still read it
            int sel_new = c->sel[slot];
            if (n > 0 && (o + n) % kTokGroup != 0 && (o % kTokGroup) != 0 &&
                (o + n) / kTokGroup != o / kTokGroup)
                sel_new = 1 - sel_new;
            ea.sel_new[i] = sel_new;
            if (n > 0) max_units = std::max(max_units, (o + n - 1) / kTokGroup / 2 - o / kTokGroup / 2 + 1);
        }
        int max_new = 0;
        for (int i = 0; i < nb; ++i) max_new = std::max(max_new, ea.n_new[i]);
        if (max_new == 1) {
            hipError_t e = launch_append1(ea, s);
            if (e != hipSuccess) return hip_fail(e, "append launch");
        } else if (max_units > 0) {
            hipError_t e = launch_encode(ea, max_units, s);
            if (e != hipSuccess) return hip_fail(e, "encode launch");
        }
        for (int i = 0; i < nb; ++i) {
            c->len[ea.slot[i]] += ea.n_new[i];
            c->sel[ea.slot[i]] = ea.sel_new[i];
        }
    }
    return PALU_OK;
}

namespace {

// Decode attention of palu_decode_attend and palu_decode_attend_noalloc.
// The split partials go to the bound buffer (fixed == nullptr) or to the
// file-scope device array at `fixed` (kStaticScratchBytes), which every call
// of one launch group reuses in stream order.
// With step (palu_decode_step) every row first appends one token (K and V
// from step[0] / step[1], [B][H][1][D]) and every kernel reads and advances
// the lengths in device memory, so a captured call replays correctly later.
int decode_attend(palu_cache *c, const void *q, void *out, const int32_t *seq_ids, int32_t B,
                  float softmax_scale, void *stream, float *fixed, const void *const *step = nullptr) {
    if (int e = check_fitted(c)) return e;
    if (!q || !out) return fail(PALU_ERR_INVALID_ARG, "q and out must be non-NULL");
    if (B <= 0) return fail(PALU_ERR_INVALID_ARG, "B must be positive");
    if (!(softmax_scale >= 0.0f) || std::isinf(softmax_scale))
        return fail(PALU_ERR_INVALID_ARG, "softmax_scale must be finite and >= 0");
    if (step && (!step[0] || !step[1])) return fail(PALU_ERR_INVALID_ARG, "k_new and v_new must be non-NULL");
    std::vector<char> seen(step ? c->max_batch : 0, 0);
    for (int b = 0; b < B; ++b) {
        const int slot = seq_ids ? seq_ids[b] : b;
        if (int e = check_slot(c, slot)) return e;
        if (step) {
            if (seen[slot]) return fail(PALU_ERR_INVALID_ARG, "sequence slot listed twice in one call");
            seen[slot] = 1;
            if (c->len[slot] + 1 > c->max_seq_len)
                return fail(PALU_ERR_CAPACITY, "append to slot " + std::to_string(slot) + " exceeds max_seq_len");
        } else if (c->len[slot] <= 0) {
            return fail(PALU_ERR_CAPACITY, "sequence slot " + std::to_string(slot) + " holds no tokens");
        }
    }
    const int add = step ? 1 : 0;   // tokens the call appends before attending
    hipStream_t s = static_cast<hipStream_t>(stream);
    const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / std::sqrt(static_cast<float>(c->D));
    const size_t row_elems = static_cast<size_t>(c->Hq) * c->D;
    std::vector<AttendArgs> launches;
    for (int b0 = 0; b0 < B; b0 += kMaxCallSeqs) {
        const int nb = std::min(kMaxCallSeqs, B - b0);
        launches.emplace_back();
        AttendArgs &aa = launches.back();
        aa = AttendArgs{};
        aa.q = static_cast<const uint16_t *>(q) + b0 * row_elems;
        aa.out = static_cast<uint16_t *>(out) + b0 * row_elems;
        aa.partial = fixed ? fixed : reinterpret_cast<float *>(c->dev + c->off_attend);

        aa.k = c->tensor_dev(0);
        aa.v = c->tensor_dev(1);
        aa.B = nb;
        aa.Hq = c->Hq;
        aa.Hkv = c->H;
        aa.gqa = c->gqa;
        aa.hpg = c->hpg;
        aa.qscale = static_cast<float>(scale * 1.4426950408889634);
        aa.bf16 = c->cfg.input_dtype;
        int64_t units = 0;
        int max_full = 0;
        for (int i = 0; i < nb; ++i) {
            const int slot = seq_ids ? seq_ids[b0 + i] : b0 + i;
            aa.row[i].slot = slot;
            aa.row[i].len = c->len[slot] + add;
            aa.row[i].qi = i;
            aa.row[i].sel_ns = c->sel[slot];
            aa.slot_call[i] = slot;
            const int nfull = (c->len[slot] + add) / kTokGroup;
            units += static_cast<int64_t>(c->H) * std::max(1, nfull);
            max_full = std::max(max_full, nfull);
        }
        // split size: a multiple of the groups one workgroup pass covers
        // (double-buffered passes keep the LDS independent of it), about
        // kAttendTargetGroups workgroups per launch, and large enough for the
        // split limit; launches with fewer groups than CUs x one pass split
        // finer.  The same for every row, so a row has ceil(groups / chunk)
        // splits
        const int per_pass = 4 * (16 / c->gqa);
        const bool vq = !aa.v.fp16_latents;
        auto round_up = [](int64_t v, int64_t m) { return (v + m - 1) / m * m; };
        int64_t chunk;
        if (c->cfg.split_groups > 0) {
            chunk = c->cfg.split_groups;
        } else {
            const int cus = device_cus(c);
            if (units / per_pass < cus) {
                // too few groups to fill the CUs with full passes: spread
                // them, about one workgroup per CU (a launch this small is
                // bound by the latency of one workgroup)
                chunk = std::max<int64_t>(1, (units + cus - 1) / cus);
            } else {
                chunk = round_up(std::max<int64_t>(1, (units + kAttendTargetGroups - 1) / kAttendTargetGroups),
                                 per_pass);
                // at least two passes per split while that still leaves a
                // workgroup per CU: the prologue and the merge of a split
                // are then paid once per two passes
                if (chunk < 2 * per_pass && units / (2 * per_pass) >= cus) chunk = 2 * per_pass;
                // and four while that still leaves two per CU
                if (chunk < 4 * per_pass && units / (4 * per_pass) >= 2 * cus) chunk = 4 * per_pass;
                // ragged rows round their last split up: grow the split by
                // whole passes until the launch's exact workgroup count fits
                // the target (no second, partial round of workgroups)
                auto wg_count = [&](int64_t ch) {
                    int64_t n = 0;
                    for (int i = 0; i < nb; ++i)
                        n += std::max<int64_t>(1, (aa.row[i].len / kTokGroup + ch - 1) / ch);
                    return n * c->H;
                };
                while (wg_count(chunk) > kAttendTargetGroups && chunk < max_full) chunk += per_pass;
            }
        }
        chunk = std::max<int64_t>(chunk, (max_full + kMaxSplits - 1) / kMaxSplits);
        if (step) {
            // a replayed step sees longer rows: the grid and the partials'
            // split stride cover any length up to the capacity
            const int cap_full = c->max_seq_len / kTokGroup;
            chunk = std::max<int64_t>(chunk, (cap_full + kMaxSplits - 1) / kMaxSplits);
        }
        int nsplit_max = 1;
        for (int i = 0; i < nb; ++i) {
            const int nfull = aa.row[i].len / kTokGroup;
            const int ns = std::max(1, static_cast<int>((nfull + chunk - 1) / chunk));
            aa.row[i].sel_ns |= ns << 1;
            aa.nsplit_call[i] = ns;
            nsplit_max = std::max(nsplit_max, ns);
        }
        if (step) {
            nsplit_max = std::max(1, static_cast<int>((c->max_seq_len / kTokGroup + chunk - 1) / chunk));
            aa.dev_len = 1;
            aa.len_dev = dev_len(c);
            aa.sel_dev = dev_sel(c);
            aa.row_info = dev_row_info(c);
            aa.max_len = c->max_seq_len;
        }
        // longest rows first in the grid's y order (stable, so equal lengths keep call order)
        std::stable_sort(aa.row, aa.row + nb, [](const AttendRow &x, const AttendRow &y) { return x.len > y.len; });
        const size_t lds = attend_lds_bytes(c->gqa, coder_blocks(aa.k.cd), aa.k.r, aa.v.r, aa.k.words, aa.v.words, vq);
        if (lds > kAttendLdsMax)
            return fail(PALU_ERR_UNSUPPORTED, "decode workgroup needs more than 160 KiB of LDS at these ranks");
        aa.chunk = static_cast<int>(chunk);
        aa.nsplit_max = nsplit_max;
        {
            const int nbk = coder_blocks(aa.k.cd);
            volatile float one = 1.0f;   // IEEE fp32 divisions, not folded to other precisions
            aa.inv_rv = one / static_cast<float>(aa.v.r);
            aa.inv_nbk4 = one / static_cast<float>(4 * nbk);
        }
        if (fixed) {
            const size_t need = sizeof(float) * static_cast<size_t>(nb) * c->Hq * nsplit_max * (aa.v.r + 2);
            if (need > kStaticScratchBytes)
                return fail(PALU_ERR_UNSUPPORTED,
                            "split partials need " + std::to_string(need) + " bytes, above the " +
                                std::to_string(kStaticScratchBytes) + "-byte static scratch (fewer rows per call, "
                                "or a larger split_groups, or palu_decode_attend)");
        }
    }
    for (size_t li = 0; li < launches.size(); ++li) {
        const AttendArgs &aa = launches[li];
        hipError_t e;
        if (step) {
            // this launch's rows append their token (lengths from device memory)
            const int b0 = static_cast<int>(li) * kMaxCallSeqs;
            const size_t kv_elems = static_cast<size_t>(c->H) * c->D;
            EncodeArgs ea{};
            ea.x[0] = static_cast<const uint16_t *>(step[0]) + b0 * kv_elems;
            ea.x[1] = static_cast<const uint16_t *>(step[1]) + b0 * kv_elems;
            ea.t[0] = aa.k;
            ea.t[1] = aa.v;
            ea.B = aa.B;
            ea.H = c->H;
            ea.T_stride = 1;
            ea.hpg = c->hpg;
            ea.bf16 = c->cfg.input_dtype;
            ea.len_dev = dev_len(c);
            ea.sel_dev = dev_sel(c);
            ea.dev_len = 1;
            ea.max_len = c->max_seq_len;
            for (int i = 0; i < aa.B; ++i) ea.slot[i] = aa.slot_call[i];
            if ((e = launch_append1(ea, s)) != hipSuccess) return hip_fail(e, "append launch");
        }
        const size_t lds =
            attend_lds_bytes(c->gqa, coder_blocks(aa.k.cd), aa.k.r, aa.v.r, aa.k.words, aa.v.words, !aa.v.fp16_latents);
        e = launch_attend(aa, lds, s);
        if (e != hipSuccess) return hip_fail(e, "attend launch");
        e = launch_combine(aa, s);
        if (e != hipSuccess) return hip_fail(e, "combine launch");
    }
    if (step)
        for (int b = 0; b < B; ++b) c->len[seq_ids ? seq_ids[b] : b] += 1;   // one token never moves the tail buffer
    return PALU_OK;
}

}  // namespace

PALU_API int palu_decode_attend(palu_cache *c, const void *q, void *out, const int32_t *seq_ids, int32_t B,
                                float softmax_scale, void *stream) {
    return decode_attend(c, q, out, seq_ids, B, softmax_scale, stream, nullptr);
}

PALU_API int palu_decode_step(palu_cache *c, const void *k_new, const void *v_new, const void *q, void *out,
                              const int32_t *seq_ids, int32_t B, float softmax_scale, void *stream) {
    const void *kv[2] = {k_new, v_new};
    return decode_attend(c, q, out, seq_ids, B, softmax_scale, stream, nullptr, kv);
}

PALU_API int palu_sync_lengths(palu_cache *c) {
    if (int e = check_bound(c)) return e;
    hipError_t e = hipDeviceSynchronize();
    if (e == hipSuccess) e = hipMemcpy(c->len.data(), dev_len(c), sizeof(int) * c->max_batch, hipMemcpyDeviceToHost);
    if (e == hipSuccess) e = hipMemcpy(c->sel.data(), dev_sel(c), sizeof(int) * c->max_batch, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "length download");
    return PALU_OK;
}

PALU_API int palu_decode_attend_noalloc(palu_cache *c, const void *q, void *out, const int32_t *seq_ids,
                                        int32_t B, float softmax_scale, void *stream) {
    if (int e = check_fitted(c)) return e;
    void *p = nullptr;
    const hipError_t e = static_scratch_address(&p);
    if (e != hipSuccess) return hip_fail(e, "static scratch address");
    return decode_attend(c, q, out, seq_ids, B, softmax_scale, stream, static_cast<float *>(p));
}

namespace {

// Bytes of the pre-decoded tiles of the complete groups of the given slots.
size_t prefill_ws_need(const palu_cache *c, const int32_t *seq_ids, int32_t B) {
    const TensorDev kd = c->tensor_dev(0), vd = c->tensor_dev(1);
    const size_t tb = prefill_tile_bytes(coder_blocks(kd.cd), vd.r);
    size_t tiles = 0;
    for (int b = 0; b < B; ++b) tiles += static_cast<size_t>(c->H) * (c->len[seq_ids ? seq_ids[b] : b] / kTokGroup);
    return tiles * tb;
}

int prefill_attend(palu_cache *c, const void *q, void *out, const int32_t *seq_ids, const int32_t *n_q, int32_t B,
                   int32_t T_stride, float softmax_scale, void *stream, void *ws, size_t ws_bytes) {
    if (int e = check_fitted(c)) return e;
    if (!q || !out) return fail(PALU_ERR_INVALID_ARG, "q and out must be non-NULL");
    if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(out)) & 15)
        return fail(PALU_ERR_INVALID_ARG, "q and out must be 16-byte aligned");
    if (B <= 0 || T_stride <= 0) return fail(PALU_ERR_INVALID_ARG, "B and T_stride must be positive");
    if (!(softmax_scale >= 0.0f) || std::isinf(softmax_scale))
        return fail(PALU_ERR_INVALID_ARG, "softmax_scale must be finite and >= 0");
    for (int b = 0; b < B; ++b) {
        const int slot = seq_ids ? seq_ids[b] : b;
        if (int e = check_slot(c, slot)) return e;
        const int n = n_q ? n_q[b] : T_stride;
        if (n < 0 || n > T_stride) return fail(PALU_ERR_INVALID_ARG, "n_q must be in [0, T_stride]");
        if (n > c->len[slot])
            return fail(PALU_ERR_CAPACITY, "n_q exceeds the tokens stored in slot " + std::to_string(slot));
    }
    const TensorDev kd = c->tensor_dev(0), vd = c->tensor_dev(1);
    const size_t lds = prefill_lds_bytes(coder_blocks(kd.cd), kd.r, vd.r, kd.words, vd.words);
    if (lds > kAttendLdsMax)
        return fail(PALU_ERR_UNSUPPORTED, "prefill workgroup needs more than 160 KiB of LDS at these ranks");
    if (ws) {
        if (reinterpret_cast<uintptr_t>(ws) & 15) return fail(PALU_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
        const size_t need = prefill_ws_need(c, seq_ids, B);
        if (ws_bytes < need)
            return fail(PALU_ERR_INVALID_ARG, "workspace of " + std::to_string(ws_bytes) + " bytes, " +
                                                  std::to_string(need) + " needed (palu_prefill_workspace_bytes)");
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / std::sqrt(static_cast<float>(c->D));
    const int ks = prefill_ks(coder_blocks(kd.cd)), nbv = prefill_nbv(vd.r);
    const size_t tile_bytes = prefill_tile_bytes(coder_blocks(kd.cd), vd.r);
    int64_t tile_next = 0;                             // first free tile of the workspace
    const int qp = 16 * kPrefillWaves * prefill_nq(ks, nbv) / c->gqa;   // query positions per workgroup
    if ((static_cast<int64_t>(T_stride) + qp - 1) / qp > kMaxGridYZ)
        return fail(PALU_ERR_UNSUPPORTED, "prefill: more query tiles per row than the grid holds (T_stride too large)");
    const size_t row_elems = static_cast<size_t>(c->Hq) * T_stride * c->D;
    for (int b0 = 0; b0 < B; b0 += kMaxCallSeqs) {
        const int nb = std::min(kMaxCallSeqs, B - b0);
        PrefillArgs pa{};
        pa.q = static_cast<const uint16_t *>(q) + b0 * row_elems;
        pa.out = static_cast<uint16_t *>(out) + b0 * row_elems;
        pa.k = kd;
        pa.v = vd;
        pa.B = nb;
        pa.Hq = c->Hq;
        pa.Hkv = c->H;
        pa.gqa = c->gqa;
        pa.hpg = c->hpg;
        pa.T_stride = T_stride;
        pa.qp = qp;
        pa.qscale = static_cast<float>(scale * 1.4426950408889634);
        pa.bf16 = c->cfg.input_dtype;
        int tiles = 0, max_nfull = 0;
        for (int i = 0; i < nb; ++i) {
            const int slot = seq_ids ? seq_ids[b0 + i] : b0 + i;
            pa.row[i].slot = slot;
            pa.row[i].len = c->len[slot];
            pa.row[i].nq = n_q ? n_q[b0 + i] : T_stride;
            pa.row[i].sel_qi = c->sel[slot] | (i << 1);
            tiles = std::max(tiles, (pa.row[i].nq + qp - 1) / qp);
            // tiles of call row i: kv head h's complete groups from tile_base + h nfull
            pa.tile_base[i] = tile_next;
            tile_next += static_cast<int64_t>(c->H) * (c->len[slot] / kTokGroup);
            max_nfull = std::max(max_nfull, c->len[slot] / kTokGroup);
        }
        if (ws) {
            pa.ws_tiles = static_cast<uint8_t *>(ws);
            pa.tile_bytes = static_cast<int>(tile_bytes);
        }
        // heaviest rows first in the grid's z order (the causal work of a row
        // grows with its query count and length; stable for equal rows)
        std::stable_sort(pa.row, pa.row + nb, [](const PrefillRow &x, const PrefillRow &y) {
            return static_cast<int64_t>(x.nq) * x.len > static_cast<int64_t>(y.nq) * y.len;
        });
        if (tiles == 0) continue;
        pa.tiles_max = tiles;
        if (ws) {
            hipError_t e = launch_prefill_tiles(pa, max_nfull, s);
            if (e != hipSuccess) return hip_fail(e, "prefill tile launch");
        }
        hipError_t e = launch_prefill(pa, lds, s);
        if (e != hipSuccess) return hip_fail(e, "prefill launch");
    }
    return PALU_OK;
}

}  // namespace

PALU_API int palu_prefill_attend(palu_cache *c, const void *q, void *out, const int32_t *seq_ids,
                                 const int32_t *n_q, int32_t B, int32_t T_stride, float softmax_scale,
                                 void *stream) {
    return prefill_attend(c, q, out, seq_ids, n_q, B, T_stride, softmax_scale, stream, nullptr, 0);
}

PALU_API int palu_prefill_workspace_bytes(const palu_cache *c, const int32_t *seq_ids, int32_t B, size_t *bytes) {
    if (!c || !bytes) return fail(PALU_ERR_INVALID_ARG, "cache or bytes is NULL");
    if (int e = check_fitted(c)) return e;
    if (B <= 0) return fail(PALU_ERR_INVALID_ARG, "B must be positive");
    for (int b = 0; b < B; ++b)
        if (int e = check_slot(c, seq_ids ? seq_ids[b] : b)) return e;
    *bytes = prefill_ws_need(c, seq_ids, B);
    return PALU_OK;
}

PALU_API int palu_prefill_attend_ws(palu_cache *c, const void *q, void *out, const int32_t *seq_ids,
                                    const int32_t *n_q, int32_t B, int32_t T_stride, float softmax_scale,
                                    void *workspace, size_t workspace_bytes, void *stream) {
    if (!workspace) return fail(PALU_ERR_INVALID_ARG, "workspace is NULL (palu_prefill_attend needs none)");
    return prefill_attend(c, q, out, seq_ids, n_q, B, T_stride, softmax_scale, stream, workspace, workspace_bytes);
}

PALU_API int palu_seq_len(const palu_cache *c, int32_t seq, int32_t *len) {
    if (!c || !len) return fail(PALU_ERR_INVALID_ARG, "cache or len is NULL");
    if (seq < 0 || seq >= c->max_batch) return fail(PALU_ERR_CAPACITY, "sequence slot out of range");
    *len = c->len[seq];
    return PALU_OK;
}

PALU_API int palu_read_codes(const palu_cache *c, int32_t seq, int32_t head, int32_t tensor, void *records,
                             size_t records_bytes, float *tail, size_t tail_bytes) {
    if (int e = check_fitted(c)) return e;
    if (tensor != 0 && tensor != 1) return fail(PALU_ERR_INVALID_ARG, "tensor must be 0 (K) or 1 (V)");
    if (int e = check_slot(c, seq)) return e;
    if (head < 0 || head >= c->H) return fail(PALU_ERR_INVALID_ARG, "head out of range");
    const TensorDev td = c->tensor_dev(tensor);
    const int len = c->len[seq];
    const int nrec = td.fp16_latents ? (len + kTokGroup - 1) / kTokGroup : len / kTokGroup;
    const size_t rbytes = sizeof(uint32_t) * static_cast<size_t>(nrec) * td.words;
    const int ntail = td.fp16_latents ? 0 : len % kTokGroup;
    const size_t tbytes = sizeof(float) * static_cast<size_t>(ntail) * td.r;
    if (records && records_bytes < rbytes) return fail(PALU_ERR_INVALID_ARG, "records buffer too small");
    if (tail && tail_bytes < tbytes) return fail(PALU_ERR_INVALID_ARG, "tail buffer too small");
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_fail(e, "read synchronize");
    const int64_t hb = static_cast<int64_t>(seq) * c->H + head;
    if (records && rbytes) {
        e = hipMemcpy(records, td.records + hb * td.head_stride, rbytes, hipMemcpyDeviceToHost);
        if (e != hipSuccess) return hip_fail(e, "records download");
    }
    if (tail && tbytes) {
        e = hipMemcpy(tail, td.tail + (hb * 2 + c->sel[seq]) * kTokGroup * td.r, tbytes, hipMemcpyDeviceToHost);
        if (e != hipSuccess) return hip_fail(e, "tail download");
    }
    return PALU_OK;
}

PALU_API int palu_get_stats(const palu_cache *c, palu_stats *st) {
    if (!c || !st) return fail(PALU_ERR_INVALID_ARG, "cache or stats is NULL");
    if (!c->layout_known(0) || !c->layout_known(1)) return fail(PALU_ERR_NOT_FITTED, "no basis for K and V yet");
    std::memset(st, 0, sizeof(*st));
    st->r_k = c->r[0];
    st->r_v = c->r[1];
    for (int t = 0; t < 2; ++t) {
        std::vector<int> n, bits;
        split_segments(c->cfg, c->r[t], n, bits);
        const int first = c->quantized(t) ? n[0] : 0;
        if (t == 0) st->n_hi_k = first;
        else st->n_hi_v = first;
    }
    st->coded_k = c->rc[0];
    st->coded_v = c->rc[1];
    int64_t tokens = 0, full_groups = 0, tail_tokens = 0, fp16_groups = 0;
    for (int s = 0; s < c->max_batch; ++s) {
        tokens += c->len[s];
        full_groups += c->len[s] / kTokGroup;
        tail_tokens += c->len[s] % kTokGroup;
        fp16_groups += (c->len[s] + kTokGroup - 1) / kTokGroup;
    }
    st->tokens = tokens;
    const double D = c->D;
    for (int t = 0; t < 2; ++t) {
        const int rr = c->r[t], rc = c->rc[t];
        // stored bases and means: one set, or one per slot that has its own
        const int64_t sets = std::count(c->ready[t].begin(), c->ready[t].end(), 1);
        const int64_t basis_bytes = sets * c->G * c->D * (rc + 1) * 4;
        int64_t bytes;
        double nominal, realised;
        if (c->quantized(t)) {
            bytes = c->H * (full_groups * coder_words(c->cd[t]) * 4 + tail_tokens * rc * 4) + basis_bytes;
            if (c->cfg.schedule_len > 0) {
                double mean = 0.0;
                for (int i = 0; i < c->cfg.schedule_len; ++i) mean += c->cfg.bit_schedule[i];
                nominal = (rr / D) * (mean / c->cfg.schedule_len);
            } else {
                nominal = (rr / D) * (c->cfg.hi_fraction * c->cfg.hi_bit + (1.0 - c->cfg.hi_fraction) * c->cfg.lo_bit);
            }
            // the code planes hold sum(channels x bits) words per 32 tokens,
            // i.e. that many code bits per token
            realised = static_cast<double>(c->cd[t].meta0) / D;
        } else {
            bytes = c->H * fp16_groups * static_cast<int64_t>(fp16_record_words(rr)) * 4 + basis_bytes;
            nominal = realised = 16.0 * rr / D;
        }
        if (t == 0) {
            st->compressed_key_bytes = bytes;
            st->nominal_bits_k = nominal;
            st->realised_bits_k = realised;
        } else {
            st->compressed_value_bytes = bytes;
            st->nominal_bits_v = nominal;
            st->realised_bits_v = realised;
        }
    }
    st->fp16_key_bytes = tokens * c->H * c->D * 2;
    st->fp16_value_bytes = st->fp16_key_bytes;
    st->assigned_avg_bits = std::max(st->realised_bits_k, st->realised_bits_v);
    for (int t = 0; t < 2; ++t) {
        double m = -1.0;
        if (!c->per_seq && c->energy_rule[t] && !c->rank_g[t].empty()) {
            const double tau = c->cfg.energy_threshold;
            const double at = *std::max_element(c->frac_at[t].begin(), c->frac_at[t].end());
            const double prev = *std::max_element(c->frac_prev[t].begin(), c->frac_prev[t].end());
            m = std::min(at - tau, c->r[t] > 1 ? tau - prev : at - tau);
        }
        (t == 0 ? st->energy_margin_k : st->energy_margin_v) = m;
    }
    return PALU_OK;
}

PALU_API int palu_get_fit_info(const palu_cache *c, int32_t tensor, int32_t *r_groups, double *energy_prev,
                               double *energy_at) {
    if (!c) return fail(PALU_ERR_INVALID_ARG, "cache is NULL");
    if (tensor != 0 && tensor != 1) return fail(PALU_ERR_INVALID_ARG, "tensor must be 0 (K) or 1 (V)");
    if (c->per_seq) return fail(PALU_ERR_INVALID_ARG, "no shared fit with per-sequence bases");
    if (c->rank_g[tensor].empty() || !c->ready[tensor][0])
        return fail(PALU_ERR_NOT_FITTED, "no fit of this tensor since the last bind or palu_set_basis");
    for (int g = 0; g < c->G; ++g) {
        if (r_groups) r_groups[g] = c->rank_g[tensor][g];
        if (energy_prev) energy_prev[g] = c->frac_prev[tensor][g];
        if (energy_at) energy_at[g] = c->frac_at[tensor][g];
    }
    return PALU_OK;
}

PALU_API int palu_reset(palu_cache *c) {
    if (!c) return fail(PALU_ERR_INVALID_ARG, "cache is NULL");
    reset_seqs(c);
    return push_lengths(c);
}

PALU_API int palu_record_words(const palu_cache *c, int32_t tensor, int32_t *words) {
    if (!c || !words) return fail(PALU_ERR_INVALID_ARG, "cache or words is NULL");
    if (tensor != 0 && tensor != 1) return fail(PALU_ERR_INVALID_ARG, "tensor must be 0 (K) or 1 (V)");
    if (!c->layout_known(tensor)) return fail(PALU_ERR_NOT_FITTED, "no basis for this tensor");
    *words = c->words_for(tensor, c->r[tensor]);
    return PALU_OK;
}

namespace {

constexpr uint32_t kSeqMagic = 0x564B4C50u;   // "PLKV" little-endian
constexpr uint32_t kSeqVersion = 1;
constexpr size_t kSeqHeaderBytes = 64;
constexpr int kSeqHeaderInts = 13;            // magic .. len

uint64_t fnv1a(uint64_t h, const void *p, size_t n) {
    const unsigned char *b = static_cast<const unsigned char *>(p);
    for (size_t i = 0; i < n; ++i) {
        h ^= b[i];
        h *= 0x100000001B3ull;
    }
    return h;
}

// Hash of K basis, K mean, V basis, V mean (fp32), each given as a pointer.
uint64_t basis_hash(const palu_cache *c, const float *const part[4]) {
    uint64_t h = 0xCBF29CE484222325ull;
    for (int t = 0; t < 2; ++t) {
        h = fnv1a(h, part[2 * t], c->basis_elems(t) * sizeof(float));
        h = fnv1a(h, part[2 * t + 1], c->mu_elems() * sizeof(float));
    }
    return h;
}

// The four parts of basis set `set` in the host copies.
void set_parts(const palu_cache *c, int set, const float *part[4]) {
    for (int t = 0; t < 2; ++t) {
        part[2 * t] = c->basis_h[t].data() + set * c->basis_elems(t);
        part[2 * t + 1] = c->mu_h[t].data() + set * c->mu_elems();
    }
}

// Bytes of a slot's bases and means stored after the header (per-sequence
// bases only).
size_t seq_basis_bytes(const palu_cache *c) {
    if (!c->per_seq) return 0;
    return sizeof(float) * (c->basis_elems(0) + c->basis_elems(1) + 2 * c->mu_elems());
}

// Per-tensor sizes of one slot of length len.
struct SeqPart {
    int nrec, words, ntail, r;
    size_t rec_bytes() const { return sizeof(uint32_t) * static_cast<size_t>(nrec) * words; }
    size_t tail_bytes() const { return sizeof(float) * static_cast<size_t>(ntail) * r; }
};

SeqPart seq_part(const palu_cache *c, int t, int len) {
    const TensorDev td = c->tensor_dev(t);
    SeqPart p;
    p.words = td.words;
    p.r = td.r;
    p.nrec = td.fp16_latents ? (len + kTokGroup - 1) / kTokGroup : len / kTokGroup;
    p.ntail = td.fp16_latents ? 0 : len % kTokGroup;
    return p;
}

size_t seq_bytes(const palu_cache *c, int len) {
    size_t n = kSeqHeaderBytes + seq_basis_bytes(c);
    for (int t = 0; t < 2; ++t) {
        const SeqPart p = seq_part(c, t, len);
        n += static_cast<size_t>(c->H) * (p.rec_bytes() + p.tail_bytes());
    }
    return n;
}

// The header's int fields for this cache at slot length len.
void seq_header(const palu_cache *c, int len, int32_t f[kSeqHeaderInts]) {
    f[0] = static_cast<int32_t>(kSeqMagic);
    f[1] = static_cast<int32_t>(kSeqVersion);
    f[2] = c->D;
    f[3] = c->H;
    f[4] = c->G;
    f[5] = c->r[0];
    f[6] = c->r[1];
    f[7] = static_cast<int32_t>(fnv1a32(&c->cd[0], sizeof(Coder)));
    f[8] = static_cast<int32_t>(fnv1a32(&c->cd[1], sizeof(Coder)));
    f[9] = c->words_for(0, c->r[0]);
    f[10] = c->words_for(1, c->r[1]);
    f[11] = c->cfg.quantize_values;
    f[12] = len;
}

int check_seq(const palu_cache *c, int32_t seq) {
    if (int e = check_fitted(c)) return e;
    return check_slot(c, seq);
}

}  // namespace

PALU_API int palu_export_bytes(const palu_cache *c, int32_t seq, size_t *bytes) {
    if (!bytes) return fail(PALU_ERR_INVALID_ARG, "bytes is NULL");
    if (int e = check_seq(c, seq)) return e;
    *bytes = seq_bytes(c, c->len[seq]);
    return PALU_OK;
}

PALU_API int palu_export_seq(const palu_cache *c, int32_t seq, void *host_dst, size_t bytes) {
    if (int e = check_seq(c, seq)) return e;
    if (!host_dst) return fail(PALU_ERR_INVALID_ARG, "destination is NULL");
    const int len = c->len[seq];
    if (bytes < seq_bytes(c, len)) return fail(PALU_ERR_INVALID_ARG, "destination smaller than palu_export_bytes");
    char *out = static_cast<char *>(host_dst);
    std::memset(out, 0, kSeqHeaderBytes);
    int32_t f[kSeqHeaderInts];
    seq_header(c, len, f);
    std::memcpy(out, f, sizeof(f));
    const float *part[4];
    set_parts(c, c->bset(seq), part);
    const uint64_t h = basis_hash(c, part);
    std::memcpy(out + sizeof(f), &h, sizeof(h));
    const uint32_t flags = c->per_seq ? 1u : 0u;
    std::memcpy(out + sizeof(f) + sizeof(h), &flags, sizeof(flags));
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_fail(e, "export synchronize");
    char *p = out + kSeqHeaderBytes;
    if (c->per_seq)
        for (int i = 0; i < 4; ++i) {
            const size_t n = sizeof(float) * (i % 2 ? c->mu_elems() : c->basis_elems(i / 2));
            std::memcpy(p, part[i], n);
            p += n;
        }
    const int64_t hb0 = static_cast<int64_t>(seq) * c->H;
    for (int t = 0; t < 2; ++t) {
        const TensorDev td = c->tensor_dev(t);
        const SeqPart sp = seq_part(c, t, len);
        if (sp.rec_bytes()) {
            e = hipMemcpy2D(p, sp.rec_bytes(), td.records + hb0 * td.head_stride, td.head_stride * sizeof(uint32_t),
                            sp.rec_bytes(), c->H, hipMemcpyDeviceToHost);
            if (e != hipSuccess) return hip_fail(e, "records download");
            p += sp.rec_bytes() * c->H;
        }
        if (sp.tail_bytes()) {
            const float *src = td.tail + (hb0 * 2 + c->sel[seq]) * kTokGroup * td.r;
            e = hipMemcpy2D(p, sp.tail_bytes(), src, sizeof(float) * 2 * kTokGroup * td.r, sp.tail_bytes(), c->H,
                            hipMemcpyDeviceToHost);
            if (e != hipSuccess) return hip_fail(e, "tail download");
            p += sp.tail_bytes() * c->H;
        }
    }
    return PALU_OK;
}

PALU_API int palu_import_seq(palu_cache *c, int32_t seq, const void *host_src, size_t bytes) {
    // a per-sequence import installs the slot's bases, so they need not be there yet
    if (int e = check_fitted(c)) return e;
    if (seq < 0 || seq >= c->max_batch) return fail(PALU_ERR_CAPACITY, "sequence slot out of range");
    if (!c->per_seq)
        if (int e = check_slot(c, seq)) return e;
    if (!host_src) return fail(PALU_ERR_INVALID_ARG, "source is NULL");
    if (bytes < kSeqHeaderBytes) return fail(PALU_ERR_INVALID_ARG, "source shorter than the header");
    const char *in = static_cast<const char *>(host_src);
    int32_t f[kSeqHeaderInts];
    std::memcpy(f, in, sizeof(f));
    uint64_t h;
    std::memcpy(&h, in + sizeof(f), sizeof(h));
    uint32_t flags;
    std::memcpy(&flags, in + sizeof(f) + sizeof(h), sizeof(flags));
    if (static_cast<uint32_t>(f[0]) != kSeqMagic) return fail(PALU_ERR_INVALID_ARG, "bad magic");
    if (static_cast<uint32_t>(f[1]) != kSeqVersion) return fail(PALU_ERR_INVALID_ARG, "unsupported version");
    const int len = f[12];
    if (len < 0) return fail(PALU_ERR_INVALID_ARG, "negative length");
    int32_t mine[kSeqHeaderInts];
    seq_header(c, len, mine);
    for (int i = 2; i < 12; ++i)
        if (f[i] != mine[i])
            return fail(PALU_ERR_INVALID_ARG, "slot was saved under a different shape, rank or value coding");
    if (flags != (c->per_seq ? 1u : 0u))
        return fail(PALU_ERR_INVALID_ARG, c->per_seq ? "slot was saved without its bases (shared-basis cache)"
                                                     : "slot was saved with its own bases (per-sequence cache)");
    if (len > c->max_seq_len) return fail(PALU_ERR_CAPACITY, "saved length exceeds max_seq_len");
    if (bytes != seq_bytes(c, len)) return fail(PALU_ERR_INVALID_ARG, "source size does not match its header");
    const char *p = in + kSeqHeaderBytes;
    const float *part[4];
    if (c->per_seq) {
        // the bases travel with the slot: check them against the hash, then install
        std::vector<float> buf(seq_basis_bytes(c) / sizeof(float));
        std::memcpy(buf.data(), p, seq_basis_bytes(c));
        p += seq_basis_bytes(c);
        const float *q = buf.data();
        for (int i = 0; i < 4; ++i) {
            part[i] = q;
            q += i % 2 ? c->mu_elems() : c->basis_elems(i / 2);
        }
        if (h != basis_hash(c, part)) return fail(PALU_ERR_INVALID_ARG, "saved bases do not match their hash");
        c->len[seq] = 0;
        c->sel[seq] = 0;
        if (int err = push_lengths(c)) return err;
        for (int t = 0; t < 2; ++t)
            if (int e = install_basis(c, t, seq, part[2 * t], part[2 * t + 1], nullptr)) return e;
    } else {
        set_parts(c, 0, part);
        if (h != basis_hash(c, part)) return fail(PALU_ERR_INVALID_ARG, "slot was saved under a different basis");
    }
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_fail(e, "import synchronize");
    const int64_t hb0 = static_cast<int64_t>(seq) * c->H;
    for (int t = 0; t < 2; ++t) {
        const TensorDev td = c->tensor_dev(t);
        const SeqPart sp = seq_part(c, t, len);
        if (sp.rec_bytes()) {
            e = hipMemcpy2D(td.records + hb0 * td.head_stride, td.head_stride * sizeof(uint32_t), p, sp.rec_bytes(),
                            sp.rec_bytes(), c->H, hipMemcpyHostToDevice);
            if (e != hipSuccess) return hip_fail(e, "records upload");
            p += sp.rec_bytes() * c->H;
        }
        if (sp.tail_bytes()) {
            float *dst = td.tail + hb0 * 2 * kTokGroup * td.r;   // tail buffer 0
            e = hipMemcpy2D(dst, sizeof(float) * 2 * kTokGroup * td.r, p, sp.tail_bytes(), sp.tail_bytes(), c->H,
                            hipMemcpyHostToDevice);
            if (e != hipSuccess) return hip_fail(e, "tail upload");
            p += sp.tail_bytes() * c->H;
        }
    }
    e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_fail(e, "import synchronize");
    c->len[seq] = len;
    c->sel[seq] = 0;
    return push_lengths(c);
}

PALU_API const char *palu_last_error(void) { return g_last_error.c_str(); }

PALU_API void palu_cache_destroy(palu_cache *c) { delete c; }

PALU_API int palu_probe_read(const void *buf, size_t bytes, void *sink, int32_t grid, void *stream) {
    if (!buf || !sink) return fail(PALU_ERR_INVALID_ARG, "buf and sink must be non-NULL");
    if (bytes == 0 || bytes % 16 != 0) return fail(PALU_ERR_INVALID_ARG, "bytes must be a positive multiple of 16");
    if (reinterpret_cast<uintptr_t>(buf) % 16 != 0) return fail(PALU_ERR_INVALID_ARG, "buf must be 16-byte aligned");
    if (grid < 1 || grid > 65536) return fail(PALU_ERR_INVALID_ARG, "grid must be in [1, 65536]");
    const hipError_t e =
        launch_read_probe(buf, bytes / 16, static_cast<uint32_t *>(sink), grid, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "read probe launch");
    return PALU_OK;
}
