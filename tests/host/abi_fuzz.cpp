// Deterministic fuzz of the C ABI's host-side argument checks and launch planning,
// built with address and undefined-behaviour sanitizers (against stub launchers: no
// GPU). Descriptors are drawn from edge values (zero, one, powers of two around 2^31 and
// 2^32, the int64 extremes, negatives), misaligned and null pointers, unknown dtypes
// and launch options. Every call must return a status without a sanitizer report, and
// the statuses must agree with each other: a call given the workspace its
// *_workspace_size query reported never fails for want of workspace. Host buffers
// stand in for device pointers; nothing is dereferenced.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>

#include "qsa.h"

namespace qsa {
extern long g_launches;
}

namespace {

alignas(256) unsigned char g_buf[4096];
std::mt19937_64 g_rng(20261202);

int64_t pick_i64()
{
    static const int64_t edges[] = {0, 1, 2, 3, 4, 7, 8, 16, 63, 64, 127, 128, 256, 512, 1024, 2048, 4096,
                                    65536, 65537, (1LL << 31) - 1, 1LL << 31, 1LL << 32, (1LL << 32) + 1,
                                    1LL << 40, INT64_MAX, -1, -2, INT64_MIN};
    const uint64_t r = g_rng();
    if (r % 4 == 0)
        return (int64_t)(g_rng() % 300);
    return edges[(r >> 8) % (sizeof edges / sizeof edges[0])];
}

int64_t pick_small()   // mostly plausible sizes, sometimes edges
{
    const uint64_t r = g_rng();
    if (r % 3 == 0)
        return pick_i64();
    static const int64_t v[] = {1, 2, 3, 4, 8, 16, 32, 64, 128, 256, 512};
    return v[(r >> 8) % 11];
}

uint32_t pick_u32()
{
    static const uint32_t v[] = {0u, 1u, 2u, 16u, 100u, 1024u, 1u << 31, 0xffffffffu};
    return v[g_rng() % 8];
}

const void *pick_ptr()
{
    const uint64_t r = g_rng() % 10;
    return r == 0 ? nullptr : r == 1 ? (const void *)(g_buf + 4) : (const void *)g_buf;
}

int32_t pick_dtype() { static const int32_t v[] = {0, 1, 1, 2, 3, -1}; return v[g_rng() % 6]; }

qsa_paged_cache make_cache(int64_t head_dim, int32_t dtype)
{
    qsa_paged_cache c;
    std::memset(&c, 0, sizeof c);
    c.blocks = pick_ptr();
    c.dtype = g_rng() % 8 ? dtype : pick_dtype();
    c.num_pages = pick_small();
    c.num_planes = g_rng() % 4 ? 2 : pick_small();
    c.num_layers = pick_small();
    c.page_size = pick_small();
    c.num_kv_heads = pick_small();
    c.head_dim = g_rng() % 4 ? head_dim : pick_i64();
    c.page_stride = g_rng() % 2 ? -1 : pick_i64();
    c.lookup_table = (const uint32_t *)pick_ptr();
    c.max_pages = pick_small();
    c.cache_lengths = (const uint32_t *)pick_ptr();
    c.max_cache_length = pick_u32();
    return c;
}

qsa_ragged_q make_q(int64_t head_dim, int32_t dtype)
{
    qsa_ragged_q q;
    std::memset(&q, 0, sizeof q);
    q.q = pick_ptr();
    q.dtype = dtype;
    q.total_q = pick_small();
    q.num_q_heads = pick_small();
    q.head_dim = head_dim;
    q.batch = pick_small();
    q.input_row_offsets = (const uint32_t *)pick_ptr();
    q.max_prompt_length = pick_u32();
    return q;
}

qsa_launch_options g_opts;
const qsa_launch_options *pick_opts()
{
    if (g_rng() % 2)
        return nullptr;
    static const int32_t v[] = {0, 0, 1, 2, 3, 4, 7, 8, 9, 16, 64, 65, -1};
    g_opts.num_splits = v[g_rng() % 13];
    g_opts.waves = v[g_rng() % 13];
    g_opts.unroll = v[g_rng() % 13];
    g_opts.reserved = g_rng() % 16 ? 0 : 1;
    return &g_opts;
}

long g_fail = 0;
void expect(bool ok, const char *what, long it)
{
    if (!ok) {
        std::fprintf(stderr, "iteration %ld: %s (%s)\n", it, what, qsa_last_error());
        ++g_fail;
    }
}

}  // namespace

int main(int argc, char **argv)
{
    const long iters = argc > 1 ? std::atol(argv[1]) : 200000;
    long ok_calls = 0;
    for (long it = 0; it < iters; ++it) {
        const int64_t D = g_rng() % 3 ? (int64_t)(64 << (g_rng() % 4)) : pick_i64();
        const int32_t dt = pick_dtype();
        qsa_ragged_q q = make_q(D, dt);
        qsa_paged_cache kv = make_cache(D, dt), comp = make_cache(D, dt);
        const qsa_launch_options *o = pick_opts();
        const int64_t W = pick_small();
        const uint32_t layer = (uint32_t)(g_rng() % 4);
        const float scale = g_rng() % 16 ? 0.125f : (g_rng() % 2 ? 1.0f / 0.0f : 0.0f / 0.0f);
        void *out = (void *)pick_ptr();
        size_t n = 7;
        qsa_status s;
        const int which = (int)(g_rng() % 7);
        if (which == 0) {
            s = qsa_sparse_attention_workspace_size(&q, &kv, W, o, &n);
            expect(s != QSA_OK || n < (size_t)1 << 62, "workspace size out of range", it);
            qsa_status c = qsa_sparse_attention(out, dt == 2 ? 1 : dt, &q, &kv, layer, (const int32_t *)pick_ptr(), W,
                                                (const int32_t *)pick_ptr(), scale, o, g_buf, s == QSA_OK ? n : 0, nullptr);
            expect(!(s == QSA_OK && c == QSA_ERR_WORKSPACE), "sized workspace refused", it);
            ok_calls += c == QSA_OK;
            c = qsa_sparse_attention_no_alloc(out, 1, &q, &kv, layer, (const int32_t *)pick_ptr(), W,
                                              (const int32_t *)pick_ptr(), scale, o, nullptr);
            ok_calls += c == QSA_OK;
        } else if (which == 1) {
            const int64_t bs = pick_small();
            s = qsa_block_sparse_attention_workspace_size(&q, &kv, W, bs, o, &n);
            qsa_status c = qsa_block_sparse_attention(out, &q, &kv, layer, (const int32_t *)pick_ptr(), W, bs, scale,
                                                      nullptr, nullptr, o, g_buf, s == QSA_OK ? n : 0, nullptr);
            expect(!(s == QSA_OK && c == QSA_ERR_WORKSPACE), "sized workspace refused (block-sparse)", it);
            ok_calls += c == QSA_OK;
        } else if (which == 2) {
            const int64_t win = pick_small(), nc = pick_small();
            s = qsa_latent_sparse_attention_workspace_size(&q, win, nc, o, &n);
            kv.num_planes = comp.num_planes = 1;
            qsa_status c = qsa_latent_sparse_attention(out, 1, &q, &kv, &comp, layer, win, (const int32_t *)pick_ptr(),
                                                       nc, (const float *)pick_ptr(), scale, o, g_buf,
                                                       s == QSA_OK ? n : 0, nullptr);
            expect(!(s == QSA_OK && c == QSA_ERR_WORKSPACE), "sized workspace refused (latent)", it);
            ok_calls += c == QSA_OK;
        } else if (which == 3) {
            const int64_t hkv = pick_small(), win = g_rng() % 2 ? -1 : pick_small();
            const int32_t causal = (int32_t)(g_rng() % 3);
            s = qsa_ragged_attention_workspace_size(&q, hkv, causal, win, o, &n);
            qsa_status c = qsa_ragged_attention(out, 1, &q, pick_ptr(), pick_ptr(), hkv, causal, win, scale, o, g_buf,
                                                s == QSA_OK ? n : 0, nullptr);
            expect(!(s == QSA_OK && c == QSA_ERR_WORKSPACE), "sized workspace refused (dense)", it);
            ok_calls += c == QSA_OK;
        } else if (which == 4) {
            kv.num_kv_heads = g_rng() % 4 ? 1 : kv.num_kv_heads;
            qsa_status c = qsa_compress_keys(out, pick_small(), pick_ptr(), pick_ptr(), pick_dtype(), pick_i64(),
                                             g_rng() % 2 ? 64 : pick_small(), (const int32_t *)pick_ptr(), &kv,
                                             pick_small(), layer, pick_u32(), pick_small(),
                                             g_rng() % 8 ? 1e-6f : -1.0f, nullptr);
            ok_calls += c == QSA_OK;
        } else if (which == 5) {
            q.num_q_heads = g_rng() % 4 ? 1 : q.num_q_heads;
            const int64_t mb = pick_small(), ratio = pick_small(), topk = pick_small();
            const uint32_t mcl = pick_u32();
            s = qsa_select_blocks_workspace_size(&q, mb, ratio, topk, mcl, &n);
            qsa_status c = qsa_select_blocks((int32_t *)pick_ptr(), pick_i64(), (int32_t *)pick_ptr(),
                                             (int32_t *)pick_ptr(), &q, pick_ptr(), mb, (const uint32_t *)pick_ptr(),
                                             mcl, ratio, topk, g_buf, s == QSA_OK ? n : 0, nullptr);
            expect(!(s == QSA_OK && c == QSA_ERR_WORKSPACE), "sized workspace refused (select)", it);
            ok_calls += c == QSA_OK;
        } else {
            qsa_status c = qsa_stream_read(pick_ptr(), (size_t)pick_i64(), (uint32_t *)pick_ptr(), pick_u32(), nullptr);
            ok_calls += c == QSA_OK;
        }
    }
    std::printf("iterations %ld, OK calls %ld, stub launches %ld, failures %ld\n", iters, ok_calls, qsa::g_launches,
                g_fail);
    return g_fail ? 1 : 0;
}
