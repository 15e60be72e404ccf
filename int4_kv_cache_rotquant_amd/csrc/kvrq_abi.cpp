// C-ABI layer: argument validation, error reporting, the host page pool and
// dispatch to the HIP launchers.  No device memory is allocated here and no
// HIP call is made before every argument has been checked.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/kvrq.h"
#include "kvrq_internal.h"

namespace {

thread_local std::string g_last_error;

kvrq_status fail(kvrq_status st, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int log2_exact(int64_t x)
{
    int l = 0;
    while ((int64_t(1) << l) < x)
        ++l;
    return l;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool valid_block(int b) { return b == 0 || b == 16 || b == 32 || b == 64 || b == 128; }

// Code width of a pool: 0 (the default) and 4 mean INT4, 2 the 2-bit variant.
int code_bits(int32_t b) { return b == 2 ? 2 : 4; }
bool valid_bits(int32_t b) { return b == 0 || b == 2 || b == 4; }

kvrq_status check_desc(const kvrq_cache_desc *d)
{
    if (!d)
        return fail(KVRQ_EINVAL, "cache descriptor is NULL");
    if (d->head_dim != kvrq::kHeadDim)
        return fail(KVRQ_EUNSUPPORTED, "head_dim %d unsupported (only 128)", d->head_dim);
    if (d->num_kv_heads < 1)
        return fail(KVRQ_EINVAL, "num_kv_heads must be >= 1 (got %d)", d->num_kv_heads);
    if (!is_pow2(d->page_size) || d->page_size > 1024)
        return fail(KVRQ_EUNSUPPORTED, "page_size %d unsupported (power of two, 1..1024)", d->page_size);
    if (d->num_pages < 1)
        return fail(KVRQ_EINVAL, "num_pages must be >= 1 (got %d)", d->num_pages);
    if (!valid_block(d->k_block) || !valid_block(d->v_block))
        return fail(KVRQ_EUNSUPPORTED, "rotation blocks (%d, %d) unsupported (0, 16, 32, 64, 128)",
                    d->k_block, d->v_block);
    if (!valid_bits(d->k_bits) || !valid_bits(d->v_bits))
        return fail(KVRQ_EUNSUPPORTED, "code widths (%d, %d) unsupported (0 or 4 = INT4, 2)",
                    d->k_bits, d->v_bits);
    const int64_t cells = int64_t(d->num_pages) * d->num_kv_heads * d->page_size;
    // (page, head, token) cells are 32-bit indexes in the kernels; 2^32 of them would
    // take at least 288 GiB (72 B per cell with 2-bit codes)
    if (cells > (int64_t(1) << 32))
        return fail(KVRQ_EINVAL, "cache too large: num_pages * num_kv_heads * page_size = %lld > 2^32",
                    (long long)cells);
    return KVRQ_OK;
}

kvrq_status check_buffers(const kvrq_cache_buffers *b)
{
    if (!b)
        return fail(KVRQ_EINVAL, "cache buffers struct is NULL");
    if (!b->k_codes || !b->v_codes || !b->k_params || !b->v_params)
        return fail(KVRQ_EINVAL, "a cache buffer pointer is NULL");
    if (!aligned(b->k_codes, 16) || !aligned(b->v_codes, 16) || !aligned(b->k_params, 16) ||
        !aligned(b->v_params, 16))
        return fail(KVRQ_EINVAL, "cache buffers must be 16-byte aligned");
    return KVRQ_OK;
}

kvrq_status check_rows(const kvrq_cache_desc *d, const void *k, const void *v, int64_t T, int64_t ks,
                       int64_t vs, const int32_t *slots)
{
    if (T < 0)
        return fail(KVRQ_EINVAL, "num_tokens must be >= 0 (got %lld)", (long long)T);
    if (T > INT32_MAX)
        return fail(KVRQ_EUNSUPPORTED, "num_tokens %lld above 2^31-1", (long long)T);
    if (T == 0)
        return KVRQ_OK;
    if (!k || !v || !slots)
        return fail(KVRQ_EINVAL, "k, v and slot_mapping must be non-NULL");
    const int64_t row = int64_t(d->num_kv_heads) * d->head_dim;
    if (ks < row || vs < row)
        return fail(KVRQ_EINVAL, "token strides (%lld, %lld) below num_kv_heads*head_dim = %lld",
                    (long long)ks, (long long)vs, (long long)row);
    if (ks % 8 || vs % 8)
        return fail(KVRQ_EINVAL, "token strides must be multiples of 8 elements");
    if (!aligned(k, 16) || !aligned(v, 16))
        return fail(KVRQ_EINVAL, "k and v must be 16-byte aligned");
    if (!aligned(slots, 4))
        return fail(KVRQ_EINVAL, "slot_mapping must be 4-byte aligned");
    return KVRQ_OK;
}

kvrq_status hip_status(int err, const char *what)
{
    if (err == 0)
        return KVRQ_OK;
    return fail(KVRQ_EHIP, "%s: %s", what, kvrq::hip_error_string(err));
}

// The balanced decode (one resident round of workgroups sharing the tiles equally) serves an
// automatic plan with enough work for several rounds of split workgroups; a split grid pays
// where the work is small (one round, little tail) or the split size is forced.
constexpr int64_t kBalancedMinTokens = int64_t(1) << 22;

// The balanced decode can serve the shape: its tile prefix sums fit LDS and int32, and every
// (sequence, KV head) has a counter.
bool balanced_fits(int32_t num_seqs, int32_t num_kv_heads, int32_t max_seq_len)
{
    const int64_t tiles = (int64_t(max_seq_len) + kvrq::kTile - 1) / kvrq::kTile;
    return num_seqs <= kvrq::kBalancedMaxSeqs &&
           int64_t(num_seqs) * num_kv_heads <= kvrq::kSplitCounters &&
           int64_t(num_seqs) * tiles < (int64_t(1) << 31);
}

bool use_balanced(int32_t num_seqs, int32_t num_kv_heads, int32_t max_seq_len, int32_t split_tokens)
{
    if (split_tokens == KVRQ_SPLIT_BALANCED)
        return true;   // checked to fit by check_decode_shape
    return split_tokens == 0 && balanced_fits(num_seqs, num_kv_heads, max_seq_len) &&
           int64_t(num_seqs) * num_kv_heads * max_seq_len >= kBalancedMinTokens;
}

// Decode plan.  Balanced where use_balanced says so; otherwise split workgroups: a workgroup
// of kDecodeWaves waves takes split_tokens consecutive tokens of one (sequence, KV head), each
// wave a quarter.  The automatic size gives every wave split_tokens/4 = clamp(S * Hkv *
// max_len / 8192, 256, 1024) tokens (a multiple of 32): an upper bound of the work spread over
// ~8192 waves, several per SIMD, while each wave still streams enough tiles to hide its
// prologue and the split partials stay a few percent of the cache bytes.
kvrq::DecodePlan plan_decode(int32_t num_seqs, int32_t num_kv_heads, int32_t max_seq_len,
                             int32_t split_tokens)
{
    kvrq::DecodePlan p;
    if (use_balanced(num_seqs, num_kv_heads, max_seq_len, split_tokens)) {
        p.split_tokens = 0;
        p.max_splits = 0;
        p.balanced_wgs = kvrq::kBalancedMaxWgs;   // sized for the most; the launch takes fewer
        return p;
    }
    if (split_tokens <= 0) {
        // tokens per wave: enough (sequence, KV head, split) workgroups to fill the chip,
        // at least 8 tiles per wave so the per-workgroup query set-up and the combine stay
        // small (measured: 1024-token splits beat 512 and 256 on 16 x 1-4k sequences), at
        // most 1024 (one register of page ids) ...
        const int64_t work = int64_t(num_seqs) * num_kv_heads * std::max<int32_t>(max_seq_len, 1);
        int64_t wt = work / 8192;
        wt = std::max<int64_t>(256, std::min<int64_t>(1024, wt));
        // ... but no more than 64 splits, which one wave per output row combines (a 1M-token
        // sequence: 16k-token splits measured 5% faster than 4k ones and their 256-way
        // combine); longer ranges are walked in 1024-token chunks
        wt = std::max<int64_t>(wt, (int64_t(max_seq_len) + 64 * kvrq::kDecodeWaves - 1) /
                                       (64 * kvrq::kDecodeWaves));
        wt = (wt + kvrq::kTile - 1) / kvrq::kTile * kvrq::kTile;
        split_tokens = (int32_t)(wt * kvrq::kDecodeWaves);
    }
    p.split_tokens = split_tokens;
    p.max_splits = std::max<int32_t>(1, (max_seq_len + split_tokens - 1) / split_tokens);
    return p;
}

// Groups of the balanced decode: Hkv workgroups each, at most kBalancedMaxWgs workgroups in
// all (at least one group).
int32_t balanced_groups_max(int32_t num_kv_heads)
{
    return std::max<int32_t>(1, kvrq::kBalancedMaxWgs / num_kv_heads);
}

// Partial slots of the balanced decode: (group + sequence) * Hkv + KV head.
size_t balanced_slots(int32_t num_seqs, int32_t num_kv_heads)
{
    return (size_t(balanced_groups_max(num_kv_heads)) + size_t(num_seqs)) * num_kv_heads;
}

// The split counters, then the split partials; nothing when a single split writes the
// output itself.  Decode and extend lay a workspace out alike, so one workspace serves both
// (the extend leaves the counters alone).
size_t decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, const kvrq::DecodePlan &p,
                              int32_t num_kv_heads = 1)
{
    if (p.balanced_wgs > 0) {
        // partial slots: (group + sequence) * Hkv + KV head, G query heads each
        const size_t slots = balanced_slots(num_seqs, num_kv_heads);
        const size_t rows = slots * size_t(num_q_heads / num_kv_heads);
        return kvrq::kCounterBytes + rows * (kvrq::kHeadDim + 2) * sizeof(float);
    }
    if (p.max_splits == 1)
        return 0;
    const size_t rows = size_t(num_seqs) * num_q_heads * p.max_splits;
    return kvrq::kCounterBytes + rows * (kvrq::kHeadDim + 2) * sizeof(float);
}

kvrq_status check_decode_shape(const kvrq_cache_desc *d, int32_t num_seqs, int32_t num_q_heads,
                               int32_t max_seq_len, int32_t split_tokens)
{
    kvrq_status st = check_desc(d);
    if (st)
        return st;
    if (num_seqs < 0)
        return fail(KVRQ_EINVAL, "num_seqs must be >= 0");
    if (num_q_heads < 1 || num_q_heads % d->num_kv_heads)
        return fail(KVRQ_EINVAL, "num_q_heads %d must be a positive multiple of num_kv_heads %d",
                    num_q_heads, d->num_kv_heads);
    if (num_q_heads / d->num_kv_heads > kvrq::kMaxGroup)
        return fail(KVRQ_EUNSUPPORTED, "more than %d query heads per KV head", kvrq::kMaxGroup);
    if (d->page_size < 16)
        return fail(KVRQ_EUNSUPPORTED, "decode needs page_size >= 16 (got %d)", d->page_size);
    if (max_seq_len < 0)
        return fail(KVRQ_EINVAL, "max_seq_len must be >= 0");
    if (split_tokens == KVRQ_SPLIT_BALANCED) {
        if (!balanced_fits(num_seqs, d->num_kv_heads, max_seq_len))
            return fail(KVRQ_EUNSUPPORTED, "the balanced decode takes at most %d sequences and %d "
                        "(sequence, KV head) pairs", kvrq::kBalancedMaxSeqs, kvrq::kSplitCounters);
    } else if (split_tokens < 0 || split_tokens % (kvrq::kTile * kvrq::kDecodeWaves)) {
        return fail(KVRQ_EINVAL, "split_tokens must be 0, KVRQ_SPLIT_BALANCED or a positive "
                    "multiple of %d", kvrq::kTile * kvrq::kDecodeWaves);
    }
    if (num_seqs > 65535)
        return fail(KVRQ_EUNSUPPORTED, "num_seqs above 65535");
    return KVRQ_OK;
}

// Extend: query rows per workgroup, so that a wave's blocks of 16 MFMA columns hold whole
// rows.
int32_t extend_rows_per_block(int32_t group)
{
    return std::max<int32_t>(1, kvrq::kMaxGroup * kvrq::kExtendBlocks / group);
}

kvrq_status check_extend_shape(const kvrq_cache_desc *d, int32_t num_seqs, int32_t num_q_heads,
                               int32_t total_q, int32_t max_q_len, int32_t max_seq_len,
                               int32_t split_tokens)
{
    if (split_tokens == KVRQ_SPLIT_BALANCED)
        return fail(KVRQ_EUNSUPPORTED, "the extend has no balanced grid (split_tokens -1)");
    kvrq_status st = check_decode_shape(d, num_seqs, num_q_heads, max_seq_len, split_tokens);
    if (st)
        return st;
    if (total_q < 0 || max_q_len < 0)
        return fail(KVRQ_EINVAL, "total_q and max_q_len must be >= 0");
    if (total_q > 0 && max_q_len < 1)
        return fail(KVRQ_EINVAL, "max_q_len must be >= 1 when there are query rows");
    if (max_q_len > max_seq_len)
        return fail(KVRQ_EINVAL, "max_q_len %d exceeds max_seq_len %d", max_q_len, max_seq_len);
    const int64_t r = extend_rows_per_block(num_q_heads / d->num_kv_heads);
    if (int64_t(num_seqs) * ((max_q_len + r - 1) / r) > 0x7fffffff)
        return fail(KVRQ_EUNSUPPORTED, "too many query row blocks");
    return KVRQ_OK;
}

// Extend: split the key range only when the (row block, KV head) workgroups alone are too
// few to fill the chip; at least 512 tokens per split.
kvrq::DecodePlan plan_extend(int32_t num_seqs, int32_t num_kv_heads, int32_t group,
                             int32_t max_q_len, int32_t max_seq_len, int32_t split_tokens)
{
    kvrq::DecodePlan p;
    const int64_t step = int64_t(kvrq::kTile) * kvrq::kDecodeWaves;
    if (split_tokens <= 0) {
        const int64_t r = extend_rows_per_block(group);
        const int64_t blocks = std::max<int64_t>(1, int64_t(num_seqs) * ((max_q_len + r - 1) / r) *
                                                        num_kv_heads);
        int64_t splits = (4096 + blocks - 1) / blocks;
        splits = std::max<int64_t>(1, std::min<int64_t>(splits, (max_seq_len + 511) / 512));
        int64_t st = (std::max<int64_t>(max_seq_len, 1) + splits - 1) / splits;
        st = (st + step - 1) / step * step;
        split_tokens = (int32_t)std::min<int64_t>(st, int64_t(1) << 30);
    }
    p.split_tokens = split_tokens;
    p.max_splits = std::max<int32_t>(1, (max_seq_len + split_tokens - 1) / split_tokens);
    return p;
}

}  // namespace

// --------------------------------------------------------------------------
// host page pool
// --------------------------------------------------------------------------
struct kvrq_pool {
    int32_t num_pages;
    int32_t page_size;
    int32_t max_seqs;
    int32_t max_pages_per_seq;
    std::vector<int32_t> free_list;              // back() is handed out next
    std::vector<std::vector<int32_t>> seq_pages;
    std::vector<int32_t> seq_len;
};

namespace {

uint64_t splitmix64(uint64_t &x)
{
    uint64_t z = (x += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

}  // namespace

extern "C" {

const char *kvrq_status_str(kvrq_status s)
{
    switch (s) {
    case KVRQ_OK: return "KVRQ_OK";
    case KVRQ_EINVAL: return "KVRQ_EINVAL";
    case KVRQ_EUNSUPPORTED: return "KVRQ_EUNSUPPORTED";
    case KVRQ_ENOPAGES: return "KVRQ_ENOPAGES";
    case KVRQ_EHIP: return "KVRQ_EHIP";
    case KVRQ_EWORKSPACE: return "KVRQ_EWORKSPACE";
    default: return "KVRQ_UNKNOWN";
    }
}

const char *kvrq_last_error(void) { return g_last_error.c_str(); }

kvrq_status kvrq_cache_sizes(const kvrq_cache_desc *d, size_t *k_codes_bytes, size_t *v_codes_bytes,
                             size_t *params_bytes)
{
    kvrq_status st = check_desc(d);
    if (st)
        return st;
    const size_t cells = size_t(d->num_pages) * d->num_kv_heads * d->page_size;
    if (k_codes_bytes)
        *k_codes_bytes = cells * (d->head_dim * code_bits(d->k_bits) / 8);
    if (v_codes_bytes)
        *v_codes_bytes = cells * (d->head_dim * code_bits(d->v_bits) / 8);
    if (params_bytes)
        *params_bytes = cells * 2 * sizeof(uint16_t);
    return KVRQ_OK;
}

kvrq_status kvrq_pool_create(int32_t num_pages, int32_t page_size, int32_t max_seqs,
                             int32_t max_pages_per_seq, uint64_t shuffle_seed, kvrq_pool **out)
{
    if (!out)
        return fail(KVRQ_EINVAL, "out pointer is NULL");
    *out = nullptr;
    if (num_pages < 1 || max_seqs < 1 || max_pages_per_seq < 1)
        return fail(KVRQ_EINVAL, "num_pages, max_seqs and max_pages_per_seq must be >= 1");
    if (!is_pow2(page_size) || page_size > 1024)
        return fail(KVRQ_EUNSUPPORTED, "page_size %d unsupported (power of two, 1..1024)", page_size);
    kvrq_pool *p = new (std::nothrow) kvrq_pool;
    if (!p)
        return fail(KVRQ_EINVAL, "out of host memory");
    p->num_pages = num_pages;
    p->page_size = page_size;
    p->max_seqs = max_seqs;
    p->max_pages_per_seq = max_pages_per_seq;
    // page ids in hand-out order: identity, or a seeded Fisher-Yates permutation
    std::vector<int32_t> order(num_pages);
    for (int32_t i = 0; i < num_pages; ++i)
        order[i] = i;
    if (shuffle_seed) {
        uint64_t st = shuffle_seed;
        for (int32_t i = num_pages - 1; i > 0; --i) {
            const uint64_t j = splitmix64(st) % uint64_t(i + 1);
            std::swap(order[i], order[j]);
        }
    }
    p->free_list.assign(order.rbegin(), order.rend());
    p->seq_pages.assign(max_seqs, {});
    p->seq_len.assign(max_seqs, 0);
    *out = p;
    return KVRQ_OK;
}

void kvrq_pool_destroy(kvrq_pool *p) { delete p; }

kvrq_status kvrq_seq_extend(kvrq_pool *p, int32_t seq, int32_t new_len)
{
    if (!p)
        return fail(KVRQ_EINVAL, "pool is NULL");
    if (seq < 0 || seq >= p->max_seqs)
        return fail(KVRQ_EINVAL, "sequence %d outside 0..%d", seq, p->max_seqs - 1);
    if (new_len < p->seq_len[seq])
        return fail(KVRQ_EINVAL, "new_len %d below current length %d", new_len, p->seq_len[seq]);
    const int64_t need = (int64_t(new_len) + p->page_size - 1) / p->page_size;
    const int64_t have = (int64_t)p->seq_pages[seq].size();
    if (need > p->max_pages_per_seq)
        return fail(KVRQ_ENOPAGES, "sequence %d would need %lld pages (max %d)", seq, (long long)need,
                    p->max_pages_per_seq);
    if (need - have > (int64_t)p->free_list.size())
        return fail(KVRQ_ENOPAGES, "pool exhausted: need %lld more pages, %zu free",
                    (long long)(need - have), p->free_list.size());
    for (int64_t i = have; i < need; ++i) {
        p->seq_pages[seq].push_back(p->free_list.back());
        p->free_list.pop_back();
    }
    p->seq_len[seq] = new_len;
    return KVRQ_OK;
}

kvrq_status kvrq_seq_release(kvrq_pool *p, int32_t seq)
{
    if (!p)
        return fail(KVRQ_EINVAL, "pool is NULL");
    if (seq < 0 || seq >= p->max_seqs)
        return fail(KVRQ_EINVAL, "sequence %d outside 0..%d", seq, p->max_seqs - 1);
    auto &pages = p->seq_pages[seq];
    for (auto it = pages.rbegin(); it != pages.rend(); ++it)
        p->free_list.push_back(*it);
    pages.clear();
    p->seq_len[seq] = 0;
    return KVRQ_OK;
}

int32_t kvrq_seq_len(const kvrq_pool *p, int32_t seq)
{
    if (!p || seq < 0 || seq >= p->max_seqs)
        return -1;
    return p->seq_len[seq];
}

kvrq_status kvrq_slots(const kvrq_pool *p, int32_t seq, int32_t first_pos, int32_t count,
                       int32_t *slots_out)
{
    if (!p)
        return fail(KVRQ_EINVAL, "pool is NULL");
    if (seq < 0 || seq >= p->max_seqs)
        return fail(KVRQ_EINVAL, "sequence %d outside 0..%d", seq, p->max_seqs - 1);
    if (count < 0 || first_pos < 0)
        return fail(KVRQ_EINVAL, "first_pos and count must be >= 0");
    if (count > 0 && !slots_out)
        return fail(KVRQ_EINVAL, "slots_out is NULL");
    if (int64_t(first_pos) + count > p->seq_len[seq])
        return fail(KVRQ_EINVAL, "positions %d..%lld beyond sequence length %d", first_pos,
                    (long long)first_pos + count - 1, p->seq_len[seq]);
    if (int64_t(p->num_pages) * p->page_size > INT32_MAX)
        return fail(KVRQ_EUNSUPPORTED, "pool too large for int32 slots");
    const auto &pages = p->seq_pages[seq];
    for (int32_t i = 0; i < count; ++i) {
        const int32_t pos = first_pos + i;
        slots_out[i] = pages[pos / p->page_size] * p->page_size + pos % p->page_size;
    }
    return KVRQ_OK;
}

kvrq_status kvrq_page_table(const kvrq_pool *p, int32_t *table_out, int32_t *seq_lens_out)
{
    if (!p)
        return fail(KVRQ_EINVAL, "pool is NULL");
    if (!table_out)
        return fail(KVRQ_EINVAL, "table_out is NULL");
    for (int32_t s = 0; s < p->max_seqs; ++s) {
        int32_t *row = table_out + int64_t(s) * p->max_pages_per_seq;
        const auto &pages = p->seq_pages[s];
        for (int32_t i = 0; i < p->max_pages_per_seq; ++i)
            row[i] = i < (int32_t)pages.size() ? pages[i] : -1;
        if (seq_lens_out)
            seq_lens_out[s] = p->seq_len[s];
    }
    return KVRQ_OK;
}

int32_t kvrq_pool_free_pages(const kvrq_pool *p) { return p ? (int32_t)p->free_list.size() : -1; }

// --------------------------------------------------------------------------
// hot path
// --------------------------------------------------------------------------
kvrq_status kv_rotquant_write(const kvrq_cache_desc *d, const kvrq_cache_buffers *b, const void *k,
                              const void *v, int64_t num_tokens, int64_t k_token_stride,
                              int64_t v_token_stride, const int32_t *slot_mapping, void *stream)
{
    kvrq_status st = check_desc(d);
    if (st)
        return st;
    st = check_buffers(b);
    if (st)
        return st;
    st = check_rows(d, k, v, num_tokens, k_token_stride, v_token_stride, slot_mapping);
    if (st)
        return st;
    if (num_tokens == 0)
        return KVRQ_OK;
    kvrq::WriteArgs a;
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.num_tokens = num_tokens;
    a.k_stride = k_token_stride;
    a.v_stride = v_token_stride;
    a.slots = slot_mapping;
    a.k_codes = b->k_codes;
    a.v_codes = b->v_codes;
    a.k_params = reinterpret_cast<uint32_t *>(b->k_params);
    a.v_params = reinterpret_cast<uint32_t *>(b->v_params);
    a.num_slots = int64_t(d->num_pages) * d->page_size;
    a.num_kv_heads = d->num_kv_heads;
    a.page_log2 = log2_exact(d->page_size);
    a.k_bits = code_bits(d->k_bits);
    a.v_bits = code_bits(d->v_bits);
    return hip_status(kvrq::launch_rotquant_write(d->k_block, d->v_block, a, stream), "kv_rotquant_write");
}

kvrq_status kv_int4_paged_decode_workspace(const kvrq_cache_desc *d, int32_t num_seqs,
                                           int32_t num_q_heads, int32_t max_seq_len,
                                           int32_t split_tokens, size_t *bytes)
{
    kvrq_status st = check_decode_shape(d, num_seqs, num_q_heads, max_seq_len, split_tokens);
    if (st)
        return st;
    if (!bytes)
        return fail(KVRQ_EINVAL, "bytes is NULL");
    *bytes = decode_workspace_bytes(num_seqs, num_q_heads,
                                    plan_decode(num_seqs, d->num_kv_heads, max_seq_len, split_tokens),
                                    d->num_kv_heads);
    return KVRQ_OK;
}

namespace {

// The new token rows of a fused decode step.
struct StepRows {
    const void *k, *v;
    int64_t k_stride, v_stride;
    const int32_t *slots;
};

kvrq_status decode_impl(const kvrq_cache_desc *d, const kvrq_cache_buffers *b, const void *q,
                        int32_t num_seqs, int32_t num_q_heads, const int32_t *page_table,
                        int32_t max_pages_per_seq, const int32_t *seq_lens, int32_t max_seq_len,
                        float sm_scale, int32_t split_tokens, float *out, void *workspace,
                        size_t workspace_bytes, void *stream, const StepRows *step,
                        const char *what, bool static_scratch = false)
{
    kvrq_status st = check_decode_shape(d, num_seqs, num_q_heads, max_seq_len, split_tokens);
    if (st)
        return st;
    st = check_buffers(b);
    if (st)
        return st;
    if (step) {
        st = check_rows(d, step->k, step->v, num_seqs, step->k_stride, step->v_stride, step->slots);
        if (st)
            return st;
    }
    if (num_seqs == 0)
        return KVRQ_OK;
    if (!q || !page_table || !seq_lens || !out)
        return fail(KVRQ_EINVAL, "q, page_table, seq_lens and out must be non-NULL");
    if (!aligned(q, 16) || !aligned(out, 16) || !aligned(page_table, 4) || !aligned(seq_lens, 4))
        return fail(KVRQ_EINVAL, "q and out must be 16-byte aligned, page_table and seq_lens 4-byte");
    if (max_pages_per_seq < 1)
        return fail(KVRQ_EINVAL, "max_pages_per_seq must be >= 1");
    if (int64_t(max_pages_per_seq) * d->page_size < max_seq_len)
        return fail(KVRQ_EINVAL, "max_seq_len %d exceeds max_pages_per_seq*page_size", max_seq_len);
    if (!std::isfinite(sm_scale))
        return fail(KVRQ_EINVAL, "sm_scale must be finite");
    const kvrq::DecodePlan plan = plan_decode(num_seqs, d->num_kv_heads, max_seq_len, split_tokens);
    const size_t need = decode_workspace_bytes(num_seqs, num_q_heads, plan, d->num_kv_heads);
    if (static_scratch) {
        // the library's own per-device scratch: the last check before the first HIP call
        if (need > kvrq::kNoallocScratchBytes)
            return fail(KVRQ_EWORKSPACE, "%s: this decode needs %zu bytes of scratch, the static "
                        "scratch holds %zu (fewer sequences, query heads or splits, or "
                        "kv_int4_paged_decode with a workspace)", what, need,
                        kvrq::kNoallocScratchBytes);
        if (plan.balanced_wgs == 0 && plan.max_splits > 65535 * 64)
            return fail(KVRQ_EUNSUPPORTED, "too many splits");
        workspace = nullptr;
        workspace_bytes = 0;
        if (need > 0) {
            st = hip_status(kvrq::noalloc_scratch(&workspace, stream), what);
            if (st)
                return st;
            workspace_bytes = kvrq::kNoallocScratchBytes;
        }
    }
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(KVRQ_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : size_t(0));
    if (need > 0 && !aligned(workspace, 16))
        return fail(KVRQ_EINVAL, "workspace must be 16-byte aligned");
    if (plan.balanced_wgs == 0 && plan.max_splits > 65535 * 64)
        return fail(KVRQ_EUNSUPPORTED, "too many splits");

    kvrq::DecodeArgs a;
    a.k_codes = b->k_codes;
    a.v_codes = b->v_codes;
    a.k_params = reinterpret_cast<const uint32_t *>(b->k_params);
    a.v_params = reinterpret_cast<const uint32_t *>(b->v_params);
    a.q = static_cast<const uint16_t *>(q);
    a.page_table = page_table;
    a.seq_lens = seq_lens;
    a.out = out;
    if (plan.balanced_wgs > 0) {
        const size_t slots = balanced_slots(num_seqs, d->num_kv_heads);
        const size_t rows = slots * size_t(num_q_heads / d->num_kv_heads);
        a.part_o = reinterpret_cast<float *>(static_cast<char *>(workspace) + kvrq::kCounterBytes);
        a.part_ml = a.part_o + rows * kvrq::kHeadDim;
        a.counters = static_cast<int32_t *>(workspace);
        // one resident round, in whole groups of Hkv workgroups
        const int32_t groups = std::max<int32_t>(1, std::min<int32_t>(
            kvrq::decode_resident_wgs(num_q_heads / d->num_kv_heads) / d->num_kv_heads,
            balanced_groups_max(d->num_kv_heads)));
        a.balanced_wgs = groups * d->num_kv_heads;
        // pairs that span many groups (few sequences: the long-context decode) are merged by
        // a combine launch, 32 partials at a time; otherwise by their last workgroup
        a.balanced_combine = int64_t(num_seqs) * 8 <= groups ? 1 : 0;
    } else if (plan.max_splits > 1) {
        const size_t rows = size_t(num_seqs) * num_q_heads * plan.max_splits;
        a.part_o = reinterpret_cast<float *>(static_cast<char *>(workspace) + kvrq::kCounterBytes);
        a.part_ml = a.part_o + rows * kvrq::kHeadDim;
        // counters for every (sequence, KV head): the launch may then merge the partials in
        // the split kernel (where that pays) instead of a combine launch
        if (int64_t(num_seqs) * d->num_kv_heads <= kvrq::kSplitCounters)
            a.counters = static_cast<int32_t *>(workspace);
    }
    a.num_seqs = num_seqs;
    a.num_pages = d->num_pages;
    a.max_seq_len = max_seq_len;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = d->num_kv_heads;
    a.group = num_q_heads / d->num_kv_heads;
    a.page_log2 = log2_exact(d->page_size);
    a.max_pages = max_pages_per_seq;
    a.k_bits = code_bits(d->k_bits);
    a.v_bits = code_bits(d->v_bits);
    a.v_block = d->v_block;
    a.split_tokens = plan.split_tokens;
    a.max_splits = plan.max_splits;
    const float scale = sm_scale > 0.0f ? sm_scale : 1.0f / std::sqrt(float(d->head_dim));
    a.q_scale = scale * 1.4426950408889634f;
    a.qo_start = nullptr;
    a.num_rows = num_seqs;
    a.rows_per_block = 1;
    a.blocks_per_seq = 1;
    if (step) {
        a.new_slots = step->slots;
        a.k_new = static_cast<const uint16_t *>(step->k);
        a.v_new = static_cast<const uint16_t *>(step->v);
        a.k_new_stride = step->k_stride;
        a.v_new_stride = step->v_stride;
        a.k_codes_w = b->k_codes;
        a.v_codes_w = b->v_codes;
        a.k_params_w = reinterpret_cast<uint32_t *>(b->k_params);
        a.v_params_w = reinterpret_cast<uint32_t *>(b->v_params);
        a.num_slots = int64_t(d->num_pages) * d->page_size;
        a.v_block = d->v_block;
    }
    return hip_status(kvrq::launch_decode(d->k_block, d->v_block, a, stream), what);
}

}  // namespace

kvrq_status kv_int4_paged_decode(const kvrq_cache_desc *d, const kvrq_cache_buffers *b, const void *q,
                                 int32_t num_seqs, int32_t num_q_heads, const int32_t *page_table,
                                 int32_t max_pages_per_seq, const int32_t *seq_lens,
                                 int32_t max_seq_len, float sm_scale, int32_t split_tokens, float *out,
                                 void *workspace, size_t workspace_bytes, void *stream)
{
    return decode_impl(d, b, q, num_seqs, num_q_heads, page_table, max_pages_per_seq, seq_lens,
                       max_seq_len, sm_scale, split_tokens, out, workspace, workspace_bytes, stream,
                       nullptr, "kv_int4_paged_decode");
}

KVRQ_API kvrq_status kv_int4_paged_decode_noalloc(const kvrq_cache_desc *d,
                                                  const kvrq_cache_buffers *b, const void *q,
                                                  int32_t num_seqs, int32_t num_q_heads,
                                                  const int32_t *page_table,
                                                  int32_t max_pages_per_seq, const int32_t *seq_lens,
                                                  int32_t max_seq_len, float sm_scale,
                                                  int32_t split_tokens, float *out, void *stream)
{
    return decode_impl(d, b, q, num_seqs, num_q_heads, page_table, max_pages_per_seq, seq_lens,
                       max_seq_len, sm_scale, split_tokens, out, nullptr, 0, stream, nullptr,
                       "kv_int4_paged_decode_noalloc", true);
}

KVRQ_API kvrq_status kv_int4_paged_decode_step(const kvrq_cache_desc *d, const kvrq_cache_buffers *b,
                                               const void *k_new, const void *v_new,
                                               int64_t k_token_stride, int64_t v_token_stride,
                                               const int32_t *new_slots, const void *q,
                                               int32_t num_seqs, int32_t num_q_heads,
                                               const int32_t *page_table, int32_t max_pages_per_seq,
                                               const int32_t *seq_lens, int32_t max_seq_len,
                                               float sm_scale, int32_t split_tokens, float *out,
                                               void *workspace, size_t workspace_bytes, void *stream)
{
    const StepRows step{k_new, v_new, k_token_stride, v_token_stride, new_slots};
    return decode_impl(d, b, q, num_seqs, num_q_heads, page_table, max_pages_per_seq, seq_lens,
                       max_seq_len, sm_scale, split_tokens, out, workspace, workspace_bytes, stream,
                       &step, "kv_int4_paged_decode_step");
}

KVRQ_API kvrq_status kv_int4_paged_extend_workspace(const kvrq_cache_desc *d, int32_t num_seqs,
                                                    int32_t num_q_heads, int32_t total_q,
                                                    int32_t max_q_len, int32_t max_seq_len,
                                                    int32_t split_tokens, size_t *bytes)
{
    kvrq_status st = check_extend_shape(d, num_seqs, num_q_heads, total_q, max_q_len, max_seq_len,
                                        split_tokens);
    if (st)
        return st;
    if (!bytes)
        return fail(KVRQ_EINVAL, "bytes is NULL");
    const kvrq::DecodePlan plan = plan_extend(num_seqs, d->num_kv_heads, num_q_heads / d->num_kv_heads,
                                              max_q_len, max_seq_len, split_tokens);
    *bytes = decode_workspace_bytes(total_q, num_q_heads, plan);
    return KVRQ_OK;
}

KVRQ_API kvrq_status kv_int4_paged_extend(const kvrq_cache_desc *d, const kvrq_cache_buffers *b,
                                          const void *q, int32_t total_q, int32_t num_seqs,
                                          int32_t num_q_heads, const int32_t *qo_start,
                                          const int32_t *page_table, int32_t max_pages_per_seq,
                                          const int32_t *seq_lens, int32_t max_seq_len,
                                          int32_t max_q_len, float sm_scale, int32_t split_tokens,
                                          float *out, void *workspace, size_t workspace_bytes,
                                          void *stream)
{
    kvrq_status st = check_extend_shape(d, num_seqs, num_q_heads, total_q, max_q_len, max_seq_len,
                                        split_tokens);
    if (st)
        return st;
    st = check_buffers(b);
    if (st)
        return st;
    if (num_seqs == 0 || total_q == 0)
        return KVRQ_OK;
    if (!q || !qo_start || !page_table || !seq_lens || !out)
        return fail(KVRQ_EINVAL, "q, qo_start, page_table, seq_lens and out must be non-NULL");
    if (!aligned(q, 16) || !aligned(out, 16) || !aligned(page_table, 4) || !aligned(seq_lens, 4) ||
        !aligned(qo_start, 4))
        return fail(KVRQ_EINVAL, "q and out must be 16-byte aligned, the int32 arrays 4-byte");
    if (max_pages_per_seq < 1)
        return fail(KVRQ_EINVAL, "max_pages_per_seq must be >= 1");
    if (int64_t(max_pages_per_seq) * d->page_size < max_seq_len)
        return fail(KVRQ_EINVAL, "max_seq_len %d exceeds max_pages_per_seq*page_size", max_seq_len);
    if (!std::isfinite(sm_scale))
        return fail(KVRQ_EINVAL, "sm_scale must be finite");
    const int32_t group = num_q_heads / d->num_kv_heads;
    const kvrq::DecodePlan plan = plan_extend(num_seqs, d->num_kv_heads, group, max_q_len,
                                              max_seq_len, split_tokens);
    const size_t need = decode_workspace_bytes(total_q, num_q_heads, plan);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(KVRQ_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : size_t(0));
    if (need > 0 && !aligned(workspace, 16))
        return fail(KVRQ_EINVAL, "workspace must be 16-byte aligned");
    if (plan.max_splits > 65535)
        return fail(KVRQ_EUNSUPPORTED, "too many splits");

    kvrq::DecodeArgs a;
    a.k_codes = b->k_codes;
    a.v_codes = b->v_codes;
    a.k_params = reinterpret_cast<const uint32_t *>(b->k_params);
    a.v_params = reinterpret_cast<const uint32_t *>(b->v_params);
    a.q = static_cast<const uint16_t *>(q);
    a.page_table = page_table;
    a.seq_lens = seq_lens;
    a.out = out;
    const size_t rows = size_t(total_q) * num_q_heads * plan.max_splits;
    if (plan.max_splits > 1) {
        a.part_o = reinterpret_cast<float *>(static_cast<char *>(workspace) + kvrq::kCounterBytes);
        a.part_ml = a.part_o + rows * kvrq::kHeadDim;
    }
    a.num_seqs = num_seqs;
    a.num_pages = d->num_pages;
    a.max_seq_len = max_seq_len;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = d->num_kv_heads;
    a.group = group;
    a.page_log2 = log2_exact(d->page_size);
    a.max_pages = max_pages_per_seq;
    a.k_bits = code_bits(d->k_bits);
    a.v_bits = code_bits(d->v_bits);
    a.v_block = d->v_block;
    a.split_tokens = plan.split_tokens;
    a.max_splits = plan.max_splits;
    const float scale = sm_scale > 0.0f ? sm_scale : 1.0f / std::sqrt(float(d->head_dim));
    a.q_scale = scale * 1.4426950408889634f;
    a.qo_start = qo_start;
    a.num_rows = total_q;
    a.rows_per_block = extend_rows_per_block(group);
    a.blocks_per_seq = (max_q_len + a.rows_per_block - 1) / a.rows_per_block;
    return hip_status(kvrq::launch_decode(d->k_block, d->v_block, a, stream), "kv_int4_paged_extend");
}

kvrq_status kvrq_bf16_paged_write(const kvrq_cache_desc *d, void *k_cache, void *v_cache, const void *k,
                                  const void *v, int64_t num_tokens, int64_t k_token_stride,
                                  int64_t v_token_stride, const int32_t *slot_mapping, void *stream)
{
    if (!d)
        return fail(KVRQ_EINVAL, "cache descriptor is NULL");
    kvrq_cache_desc dd = *d;
    dd.k_block = dd.v_block = 0;
    kvrq_status st = check_desc(&dd);
    if (st)
        return st;
    if (!k_cache || !v_cache)
        return fail(KVRQ_EINVAL, "bf16 cache pointers must be non-NULL");
    if (!aligned(k_cache, 16) || !aligned(v_cache, 16))
        return fail(KVRQ_EINVAL, "bf16 caches must be 16-byte aligned");
    st = check_rows(&dd, k, v, num_tokens, k_token_stride, v_token_stride, slot_mapping);
    if (st)
        return st;
    if (num_tokens == 0)
        return KVRQ_OK;
    kvrq::CopyArgs a;
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.num_tokens = num_tokens;
    a.k_stride = k_token_stride;
    a.v_stride = v_token_stride;
    a.slots = slot_mapping;
    a.k_cache = static_cast<uint16_t *>(k_cache);
    a.v_cache = static_cast<uint16_t *>(v_cache);
    a.num_slots = int64_t(d->num_pages) * d->page_size;
    a.num_kv_heads = d->num_kv_heads;
    a.page_log2 = log2_exact(d->page_size);
    return hip_status(kvrq::launch_bf16_paged_write(a, stream), "kvrq_bf16_paged_write");
}

kvrq_status kvrq_device_read(const void *src, size_t bytes, uint32_t *sink, void *stream)
{
    if (bytes == 0)
        return KVRQ_OK;
    if (!src || !sink)
        return fail(KVRQ_EINVAL, "src and sink must be non-NULL");
    if (bytes % 16 || !aligned(src, 16) || !aligned(sink, 4))
        return fail(KVRQ_EINVAL, "bytes must be a multiple of 16, src 16-byte and sink 4-byte aligned");
    return hip_status(kvrq::launch_device_read(src, bytes, sink, stream), "kvrq_device_read");
}

kvrq_status kvrq_paged_read(const kvrq_cache_desc *d, const kvrq_cache_buffers *b, const int32_t *pages,
                            int64_t num_list, int32_t pattern, int32_t wgs_per_cu, uint32_t *sink,
                            void *stream)
{
    kvrq_status st = check_desc(d);
    if (st != KVRQ_OK)
        return st;
    if ((st = check_buffers(b)) != KVRQ_OK)
        return st;
    if (code_bits(d->k_bits) != 4 || code_bits(d->v_bits) != 4)
        return fail(KVRQ_EUNSUPPORTED, "kvrq_paged_read reads 4-bit pools only");
    if (pattern < 0 || pattern > 3)
        return fail(KVRQ_EINVAL, "pattern must be 0, 1, 2 or 3 (got %d)", pattern);
    if (pattern == 0 && ((int64_t)d->num_kv_heads * d->page_size) % 128 != 0)
        return fail(KVRQ_EUNSUPPORTED, "kvrq_paged_read pattern 0 needs num_kv_heads * page_size to be a "
                                       "multiple of 128 (got %d * %d)", d->num_kv_heads, d->page_size);
    if (pattern != 0 && d->page_size % 16 != 0)
        return fail(KVRQ_EUNSUPPORTED, "kvrq_paged_read patterns 1 to 3 need page_size to be a multiple "
                                       "of 16 (got %d)", d->page_size);
    if (num_list < 0)
        return fail(KVRQ_EINVAL, "num_list must be >= 0");
    if (wgs_per_cu < 1 || wgs_per_cu > 4)
        return fail(KVRQ_EINVAL, "wgs_per_cu must be 1..4 (got %d)", wgs_per_cu);
    if (num_list == 0)
        return KVRQ_OK;
    if (!pages || !sink || !aligned(sink, 4))
        return fail(KVRQ_EINVAL, "pages and a 4-byte aligned sink must be given");
    kvrq::PagedReadArgs a{};
    a.k_codes = b->k_codes;
    a.v_codes = b->v_codes;
    a.k_params = reinterpret_cast<const uint8_t *>(b->k_params);
    a.v_params = reinterpret_cast<const uint8_t *>(b->v_params);
    a.pages = pages;
    a.num_list = num_list;
    a.units_per_page = d->num_kv_heads * d->page_size / 128;
    a.num_pages = d->num_pages;
    a.num_kv_heads = d->num_kv_heads;
    a.page_size = d->page_size;
    a.pattern = pattern;
    a.sink = sink;
    a.magic = 0x9E3779B9u;
    return hip_status(kvrq::launch_paged_read(a, wgs_per_cu, stream), "kvrq_paged_read");
}

kvrq_status kvrq_device_copy(void *dst, const void *src, size_t bytes, void *stream)
{
    if (bytes == 0)
        return KVRQ_OK;
    if (!dst || !src)
        return fail(KVRQ_EINVAL, "dst and src must be non-NULL");
    if (bytes % 16 || !aligned(dst, 16) || !aligned(src, 16))
        return fail(KVRQ_EINVAL, "bytes must be a multiple of 16 and pointers 16-byte aligned");
    return hip_status(kvrq::launch_device_copy(dst, src, bytes, stream), "kvrq_device_copy");
}

}  // extern "C"
