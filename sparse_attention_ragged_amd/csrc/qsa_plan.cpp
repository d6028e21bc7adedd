// Host-side argument checks and the split-K launch plan. Pure C++: nothing here
// touches the device, so every check can be exercised without a GPU.
#include <cstdarg>
#include <cstdio>
#include <string>

#include "qsa_host.hpp"

namespace qsa {

namespace {
thread_local std::string g_error;

// Workgroups a launch should provide: two per compute unit of an MI355X (8 XCDs x
// 32 CUs) keeps every CU streaming; more, shorter workgroups only add prologue and
// split-K combine cost.
constexpr int64_t kTargetWorkgroups = 256 * 2;
// A split shorter than this many keys spends more on its prologue/epilogue than on
// gathering.
constexpr int64_t kMinKeysPerSplit = 128;
constexpr int32_t kMaxSplits = 64;
// Head-split matrix-core kernel: workgroups resident at once (one per CU), and the most
// splits a tail row of a short last round is cut into (more would cost the combine
// step more than the round saves).
constexpr int64_t kWideSlots = 256;
constexpr int64_t kMaxTailSplits = 8;

// ceil(a / b) for a >= 0, b > 0, without forming a + b - 1 (which can overflow)
int64_t ceil_div(int64_t a, int64_t b) { return a / b + (a % b != 0); }
}  // namespace

qsa_status fail(qsa_status code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_error = buf;
    return code;
}

void clear_error() { g_error.clear(); }

const char *last_error_text() { return g_error.c_str(); }

static bool valid_dtype(int32_t d) { return d == QSA_F32 || d == QSA_BF16 || d == QSA_FP8_E4M3; }

int64_t elem_bytes(int32_t d) { return d == QSA_F32 ? 4 : d == QSA_BF16 ? 2 : 1; }

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

qsa_status check_cache(const qsa_paged_cache *c, const char *what, int64_t planes)
{
    if (!c)
        return fail(QSA_ERR_NULL, "%s: cache descriptor is NULL", what);
    if (!c->blocks || !c->lookup_table || !c->cache_lengths)
        return fail(QSA_ERR_NULL, "%s: blocks, lookup_table and cache_lengths are required", what);
    if (!valid_dtype(c->dtype))
        return fail(QSA_ERR_DTYPE, "%s: unknown dtype %d", what, c->dtype);
    if (c->num_pages < 1 || c->num_layers < 1 || c->page_size < 1 || c->num_kv_heads < 1 ||
        c->head_dim < 1 || c->max_pages < 1)
        return fail(QSA_ERR_SHAPE, "%s: num_pages, num_layers, page_size, num_kv_heads, head_dim "
                                   "and max_pages must be >= 1", what);
    if (c->num_planes != planes)
        return fail(QSA_ERR_SHAPE, "%s: num_planes is %lld, expected %lld", what,
                    (long long)c->num_planes, (long long)planes);
    if (c->page_size > (1 << 30) || c->max_pages > (int64_t(1) << 31) ||
        c->num_pages > (int64_t(1) << 32))
        return fail(QSA_ERR_SHAPE, "%s: page_size, max_pages or num_pages out of range", what);
    // elements of a packed page, with the product checked: a page must stay below 4 GiB
    int64_t packed = c->num_planes;
    if (__builtin_mul_overflow(packed, c->num_layers, &packed) ||
        __builtin_mul_overflow(packed, c->page_size, &packed) ||
        __builtin_mul_overflow(packed, c->num_kv_heads, &packed) ||
        __builtin_mul_overflow(packed, c->head_dim, &packed) || packed >= (int64_t(1) << 32))
        return fail(QSA_ERR_UNSUPPORTED, "%s: pages of 4 GiB or more are not supported", what);
    if (c->page_stride != -1 && c->page_stride < packed)
        return fail(QSA_ERR_SHAPE, "%s: page_stride %lld is smaller than a packed page (%lld)", what,
                    (long long)c->page_stride, (long long)packed);
    // in-page offsets and the page stride are 32-bit byte quantities in the kernels
    // (packed < 2^32 and head_dim <= packed, so the products below stay in range)
    const int64_t eb = elem_bytes(c->dtype);
    const int64_t stride = c->page_stride == -1 ? packed : c->page_stride;
    if (stride >= (int64_t(1) << 32) || stride * eb >= (int64_t(1) << 32))
        return fail(QSA_ERR_UNSUPPORTED, "%s: pages of 4 GiB or more (page_stride %lld elements) are not "
                                         "supported", what, (long long)stride);
    // every K/V row is fetched with 16-byte loads
    if (!aligned16(c->blocks) || (c->head_dim * eb) % 16 != 0 || (stride * eb) % 16 != 0)
        return fail(QSA_ERR_SHAPE, "%s: blocks, head_dim rows and page_stride must keep 16-byte "
                                   "alignment", what);
    return QSA_OK;
}

qsa_status check_q(const qsa_ragged_q *q, const qsa_paged_cache *c, bool same_heads_as_cache)
{
    if (!q)
        return fail(QSA_ERR_NULL, "q descriptor is NULL");
    if (!q->input_row_offsets)
        return fail(QSA_ERR_NULL, "input_row_offsets is required");
    if (q->total_q < 0 || q->batch < 1 || q->num_q_heads < 1 || q->head_dim < 1)
        return fail(QSA_ERR_SHAPE, "q: total_q >= 0, batch >= 1, num_q_heads >= 1, head_dim >= 1");
    if (q->total_q > 0 && !q->q)
        return fail(QSA_ERR_NULL, "q data pointer is NULL");
    if (q->total_q > (int64_t(1) << 31) - 1 || q->batch > (int64_t(1) << 31) - 1 ||
        q->num_q_heads > 65536)
        return fail(QSA_ERR_SHAPE, "q: total_q, batch or num_q_heads out of range");
    if (q->dtype != c->dtype)
        return fail(QSA_ERR_DTYPE, "q dtype %d differs from the cache dtype %d", q->dtype, c->dtype);
    if (q->head_dim != c->head_dim)
        return fail(QSA_ERR_SHAPE, "q head_dim %lld differs from the cache head_dim %lld",
                    (long long)q->head_dim, (long long)c->head_dim);
    if (q->total_q > 0 && !aligned16(q->q))
        return fail(QSA_ERR_SHAPE, "q must be 16-byte aligned");
    if (same_heads_as_cache && q->num_q_heads % c->num_kv_heads != 0)
        return fail(QSA_ERR_SHAPE, "num_q_heads %lld is not a multiple of num_kv_heads %lld",
                    (long long)q->num_q_heads, (long long)c->num_kv_heads);
    return QSA_OK;
}

// Split plan for a gather launch: grid = total_q x num_kv_heads x num_splits
// workgroups. Each (row, kv head) key list of at most `key_capacity` keys is cut
// into num_splits contiguous ranges of split_keys keys (a multiple of split_unit).
// With more than one split every workgroup writes an (m, l, acc) partial to the
// workspace and a combine kernel merges them; with one split the gather kernel
// writes the output itself.
qsa_status plan_gather(const qsa_ragged_q *q, int64_t num_kv_heads, int32_t dtype, int32_t list_kind,
                       int64_t key_capacity, int64_t split_unit, const qsa_launch_options *opts,
                       Plan *plan)
{
    const int64_t group = q->num_q_heads / num_kv_heads;
    const int32_t G = (int32_t)group, Dh = (int32_t)q->head_dim;
    bool built;
    if (group > 16) {
        plan->path = PATH_MFMA_WIDE;
        built = group <= 64 && mfma_wide_supported(dtype, G, Dh, list_kind);
    } else if (group >= 8) {
        plan->path = PATH_MFMA;
        built = mfma_supported(dtype, G, Dh);
    } else {
        plan->path = PATH_VALU;
        built = valu_supported(dtype, G, Dh);
    }
    if (!built)
        return fail(QSA_ERR_UNSUPPORTED,
                    "no kernel built for dtype %d, group %lld, head_dim %lld", dtype,
                    (long long)group, (long long)q->head_dim);
    plan->split_row0 = 0;
    qsa_launch_options o = {0, 0, 0, 0};
    if (opts)
        o = *opts;
    if (o.num_splits < 0 || o.num_splits > kMaxSplits)
        return fail(QSA_ERR_UNSUPPORTED, "num_splits must be in [0, %d]", kMaxSplits);
    if (o.waves < 0 || o.waves > 8)
        return fail(QSA_ERR_UNSUPPORTED, "waves must be in [0, 8] (0 = automatic)");
    if (o.unroll < 0 || o.unroll > 8)
        return fail(QSA_ERR_UNSUPPORTED, "unroll must be in [0, 8]");
    if (o.reserved != 0)
        return fail(QSA_ERR_UNSUPPORTED, "qsa_launch_options.reserved must be 0");
    plan->waves = o.waves ? o.waves : 4;
    plan->unroll = o.unroll ? o.unroll : 4;
    plan->key_capacity = key_capacity;
    const int64_t cap = key_capacity > 0 ? key_capacity : 1;

    // wavefront kernel: when every kv head reads the same keys and there are too few
    // (row, kv head) items to fill the device without splitting, one workgroup covers a
    // block of kv heads (one team each): a wavefront then reads all of a key's heads at
    // once and computes the key's address once. With enough items, one kv head per
    // workgroup needs no split-K partials (measured faster on the decode workload,
    // where the combine step costs more than the shared addressing saves).
    plan->head_block = 1;
    if (plan->path == PATH_VALU && list_kind != KEYS_BLOCKS && q->total_q * num_kv_heads < kTargetWorkgroups) {
        const int eb = dtype == QSA_F32 ? 4 : dtype == QSA_BF16 ? 2 : 1;
        int64_t a = num_kv_heads, c = 64 / valu_team_lanes(eb, Dh);
        while (c) {
            const int64_t t = a % c;
            a = c;
            c = t;
        }
        plan->head_block = (int32_t)a;  // gcd(kv heads, teams per wavefront)
    }
    // wavefront kernel over index lists with at most one query row per sequence (decode):
    // no other row reads the same K/V rows, so they are loaded non-temporally (measured
    // ~10 % faster at the decode workload; prefill rows, whose selections overlap,
    // measured 4 % slower with it and keep plain loads)
    plan->stream_rows = plan->path == PATH_VALU && (list_kind == KEYS_TOKEN_INDICES || list_kind == KEYS_BLOCKS) &&
                        q->total_q <= q->batch;
    const int64_t items = q->total_q * (num_kv_heads / plan->head_block);
    int64_t splits = o.num_splits;
    if (splits == 0) {
        // the matrix-core kernel gives each wavefront its own (row, kv head, split)
        const int64_t target = plan->path == PATH_MFMA ? kTargetWorkgroups * (plan->waves < 4 ? plan->waves : 4)
                                                       : kTargetWorkgroups;
        // matrix-core wavefronts: round down, so that every item stays resident (two
        // workgroups per CU); a few items over that would run as a short second round
        splits = items > 0 ? (plan->path == PATH_MFMA ? target / items : ceil_div(target, items)) : 1;
        int64_t by_len = ceil_div(cap, kMinKeysPerSplit);
        if (splits > by_len)
            splits = by_len;
        if (splits > kMaxSplits)
            splits = kMaxSplits;
        if (splits < 1)
            splits = 1;
    }
    int64_t unit = split_unit > 0 ? split_unit : 1;
    int64_t sk = ceil_div(ceil_div(cap, splits), unit) * unit;
    splits = ceil_div(cap, sk);   // drop splits that would start past the capacity
    if (splits < 1)
        splits = 1;
    // head-split matrix-core kernel (one workgroup per CU): when the rows fill whole
    // rounds of the 256 CUs plus a short last round, that round would run a few rows
    // alone for a full row's time. Those tail rows run split instead (their partials
    // merged by the combine step), the rows before them unsplit.
    int64_t row0 = 0;
    if (plan->path == PATH_MFMA_WIDE && o.num_splits == 0 && splits == 1) {
        const int64_t tail = q->total_q % kWideSlots;
        if (q->total_q > kWideSlots && tail > 0 && tail <= kWideSlots / 4) {
            int64_t ts = kWideSlots / tail < kMaxTailSplits ? kWideSlots / tail : kMaxTailSplits;
            const int64_t tsk = ceil_div(ceil_div(cap, ts), unit) * unit;
            ts = ceil_div(cap, tsk);
            if (ts > 1) {
                row0 = q->total_q - tail;
                splits = ts;
                sk = tsk;
            }
        }
    }
    plan->split_row0 = row0;
    plan->num_splits = (int32_t)splits;
    plan->split_keys = sk;
    plan->ws_bytes = 0;
    plan->ws_ml_offset = 0;
    if (splits > 1) {
        size_t rows_heads = (size_t)(q->total_q - row0) * (size_t)q->num_q_heads;
        size_t acc = (size_t)splits * rows_heads * (size_t)q->head_dim * sizeof(float);
        acc = (acc + 255) & ~(size_t)255;
        plan->ws_ml_offset = acc;
        plan->ws_bytes = acc + (size_t)splits * rows_heads * 2 * sizeof(float);
    }
    return QSA_OK;
}

CacheAddr cache_addr(const qsa_paged_cache *c, uint32_t layer)
{
    CacheAddr a;
    const int64_t slab = c->page_size * c->num_kv_heads * c->head_dim;
    a.blocks = c->blocks;
    a.lut = c->lookup_table;
    a.page_stride = c->page_stride == -1 ? c->num_planes * c->num_layers * slab : c->page_stride;
    a.plane_stride = c->num_layers * slab;
    a.layer_off = (int64_t)layer * slab;
    a.slot_stride = c->num_kv_heads * c->head_dim;
    a.max_pages = c->max_pages;
    a.num_pages = c->num_pages;
    a.page_size = (int32_t)c->page_size;
    // Division by the page size as a multiply-high: with k = ceil(log2(page_size)) and
    // magic = ceil(2^(31+k) / page_size), (pos * magic) >> (31+k) == pos / page_size
    // for every 0 <= pos < 2^31 (the rounding error stays below 2^-k <= 1/page_size).
    int k = 0;
    while ((int64_t(1) << k) < c->page_size)
        ++k;
    const unsigned __int128 num = (unsigned __int128)1 << (31 + k);
    a.magic = (uint64_t)((num + (unsigned __int128)c->page_size - 1) / (unsigned __int128)c->page_size);
    a.magic_shift = 31 + k;
    const bool pow2 = (c->page_size & (c->page_size - 1)) == 0;
    a.page_shift = pow2 ? k : -1;
    a.page_mask = pow2 ? (uint32_t)(c->page_size - 1) : 0u;
    const int64_t eb = elem_bytes(c->dtype);
    a.page_stride_b = (uint32_t)(a.page_stride * eb);   // < 2^32: checked in check_cache
    a.plane_stride_b = (uint32_t)(a.plane_stride * eb);
    a.layer_off_b = (uint32_t)(a.layer_off * eb);
    a.slot_stride_b = (uint32_t)(a.slot_stride * eb);
    return a;
}

}  // namespace qsa
