// Device-side building blocks shared by the gather kernels (gfx950, wave64):
// element decode, wavefront reductions, sequence lookup and the key-address pipeline.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qsa_host.hpp"

namespace qsa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

typedef const __attribute__((address_space(1))) u32x4 global_u32x4;

constexpr float kNegInf = -__builtin_huge_valf();
// Running reference of a softmax state that has not seen a key yet: finite, so that
// 2^(kNoKey - kNoKey) = 1 and 2^(kNoKey - real) = 0 need no special cases.
constexpr float kNoKey = -1e30f;
// Two bf16 ones packed in a dword (sums a packed pair with one dot instruction).
constexpr uint32_t kBf16OnePair = 0x3F803F80u;

// 16-byte load through the global address space (global_load_dwordx4 rather than a
// flat load: the pointer came out of LDS, so the compiler cannot prove where it points).
__device__ __forceinline__ u32x4 ldg16(const void *p) { return *(global_u32x4 *)(p); }
// The same load marked non-temporal (streaming: the line is not kept for reuse). For
// gathered rows that are read once per call this raised a bare replay of the decode
// workload's rows from 5.6 to 6.5 TB/s on MI355X.
__device__ __forceinline__ u32x4 ldg16_nt(const void *p) { return __builtin_nontemporal_load((global_u32x4 *)(p)); }

// Two floats -> two bf16 (round to nearest even) packed in a dword, low half first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    uint32_t u;
    __builtin_memcpy(&u, &v, sizeof u);
    return u;
}

// Reinterpret one dword as two bf16. (A memcpy from a scalar copy: bit-casting a
// vector element directly has been seen to read element 0 regardless of the index.)
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t u)
{
    bf16x2_t r;
    __builtin_memcpy(&r, &u, sizeof r);
    return r;
}

template <int DT> struct Elem;
template <> struct Elem<QSA_F32> { static constexpr int bytes = 4; };
template <> struct Elem<QSA_BF16> { static constexpr int bytes = 2; };
template <> struct Elem<QSA_FP8_E4M3> { static constexpr int bytes = 1; };

// bf16 holds the upper 16 bits of a binary32: widening is a shift or a mask.
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// binary32 -> bf16 bits, round to nearest even (the hardware conversion; NaN stays a NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) { return pack_bf16x2(f, 0.f) & 0xffffu; }

// Four OCP E4M3 codes (one dword) -> four floats, exact, via the gfx950 converter.
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t w, float *o)
{
    f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    o[0] = a[0];
    o[1] = a[1];
    o[2] = b[0];
    o[3] = b[1];
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over aligned teams of TL lanes (TL a power of two, <= 64). Within a 16-lane
// row the steps are DPP quad permutes and the half-row / row mirrors; wider teams
// finish with lane shuffles.
template <int TL>
__device__ __forceinline__ float team_sum(float x)
{
    if constexpr (TL >= 2) x += dpp_f<0xB1>(x);   // quad_perm [1,0,3,2]
    if constexpr (TL >= 4) x += dpp_f<0x4E>(x);   // quad_perm [2,3,0,1]
    if constexpr (TL >= 8) x += dpp_f<0x141>(x);  // row_half_mirror
    if constexpr (TL >= 16) x += dpp_f<0x140>(x); // row_mirror
    if constexpr (TL >= 32) x += __shfl_xor(x, 16);
    if constexpr (TL >= 64) x += __shfl_xor(x, 32);
    return x;
}

// max(a, b) of two scores as one v_med3(a, b, +inf). fmaxf keeps IEEE NaN quieting, so
// the compiler first canonicalises every operand whose producer it cannot see through
// (an MFMA result, a lane permute): one more instruction per operand. The two agree
// on every non-NaN pair, -inf included.
__device__ __forceinline__ float score_max(float a, float b)
{
    float inf = __builtin_huge_valf();
    asm("" : "+v"(inf));   // opaque, so the med3 is not turned back into fmaxf
    return __builtin_amdgcn_fmed3f(a, b, inf);
}

// Reductions over the lane pairs (l, l^16) and (l, l^32) with the gfx950 row-swap
// permutes: both operands start as x, and after the swap one holds the partner rows.
// VALU only (no trip through the LDS queue, unlike a lane shuffle).
__device__ __forceinline__ float xor16_max(float x)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return score_max(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return score_max(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The value of lane l and of its partner lane l^OFF, as an unordered pair (a, b): one
// of the two is this lane's own value. Symmetric combinations (sums, maxima, softmax
// merges) can use the pair directly. 8: DPP row rotation; 16 and 32: gfx950 row-swap
// permutes; other offsets fall back to a lane shuffle.
template <int OFF>
__device__ __forceinline__ void xor_pair(float x, float &a, float &b)
{
    if constexpr (OFF == 8) {
        a = x;
        b = dpp_f<0x128>(x);                    // row_ror:8 = lane ^ 8 within a 16-lane row
    } else if constexpr (OFF == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        a = __uint_as_float(r[0]);
        b = __uint_as_float(r[1]);
    } else if constexpr (OFF == 32) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        a = __uint_as_float(r[0]);
        b = __uint_as_float(r[1]);
    } else {
        a = x;
        b = __shfl_xor(x, OFF);
    }
}

// Sequence of row r: the b with row_off[b] <= r < row_off[b+1] (binary search; a
// chain of dependent loads, used only for very large batches).
__device__ __forceinline__ int find_seq(const uint32_t *row_off, int batch, uint32_t r)
{
    int lo = 0, hi = batch - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (row_off[mid] <= r)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// Sequence of row r and the row's position (cache_lengths[b] + r - row_off[b]) in one
// memory round trip: lane t also loads cache_lengths[base + t] next to the offsets.
// `pos` is left at 0 when cache_lengths is null.
__device__ __forceinline__ int find_seq_pos_wave(const uint32_t *row_off, const uint32_t *cache_lengths, int batch,
                                                 uint32_t r, int64_t &pos)
{
    if (batch > 1024) {
        const int b = find_seq(row_off, batch, r);
        pos = cache_lengths ? (int64_t)cache_lengths[b] + ((int64_t)r - (int64_t)row_off[b]) : 0;
        return b;
    }
    const int lane = threadIdx.x & 63;
    for (int base = 0; base < batch; base += 64) {
        const int t = base + lane;
        const uint32_t lo = t < batch ? row_off[t] : 0xffffffffu;
        const uint32_t hi = t < batch ? row_off[t + 1] : 0u;
        const uint32_t cl = cache_lengths && t < batch ? cache_lengths[t] : 0u;
        const unsigned long long m = __ballot(lo <= r && r < hi);
        if (m) {
            const int w = __ffsll((long long)m) - 1;
            pos = (int64_t)(uint32_t)__shfl((int)cl, w) + ((int64_t)r - (int64_t)(uint32_t)__shfl((int)lo, w));
            return base + w;
        }
    }
    // rows past the last offset belong to the last sequence
    pos = cache_lengths ? (int64_t)cache_lengths[batch - 1] + ((int64_t)r - (int64_t)row_off[batch - 1]) : 0;
    return batch - 1;
}

// Barrier that waits only for this wavefront's LDS operations (__syncthreads also
// drains every vector-memory load in flight, which stalls a load pipeline).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// A zero the compiler cannot see through, held in a vector register: an address that
// adds it is taken as per-lane, so the load goes through the vector memory path.
__device__ __forceinline__ int32_t opaque_vzero()
{
    int32_t z;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z));
    return z;
}

// Number of keys in the list of row r (before splitting), as a per-lane value. For
// token-index lists counts[r] is read with a vector load: a scalar load would be
// waited for together with every later kernel-argument load (scalar loads complete
// out of order, so every such wait is a wait for all of them); as a vector load it
// completes in order with the loads issued after it.
template <int LIST>
__device__ __forceinline__ int64_t key_list_length_v(const GatherParams &p, int64_t r)
{
    if constexpr (LIST == KEYS_TOKEN_INDICES) {
        const int64_t n = p.counts[r + opaque_vzero()];
        return n < 0 ? 0 : (n > p.width ? p.width : n);
    } else if constexpr (LIST == KEYS_BLOCKS) {
        return p.width * p.block_size;
    } else {
        return p.window + p.width;
    }
}

// Dense ragged attention ("RaggedFlashAttentionGPU"): row r, the i-th of its sequence
// b (L rows starting at row_off[b]), sees the keys i' of the same sequence with
// i' <= i under the causal mask (all of them without) and i' >= i - window + 1 for a
// window > 0. Returns their number and sets `first` to the row index of the first one.
__device__ __forceinline__ int64_t dense_key_range(const GatherParams &p, int64_t r, int b, int64_t &first)
{
    const int64_t start = p.row_off[b], len = (int64_t)p.row_off[b + 1] - start, i = r - start;
    const int64_t hi = p.dense_causal ? i : len - 1;
    const int64_t lo = p.window > 0 && i - p.window + 1 > 0 ? i - p.window + 1 : 0;
    first = start + lo;
    return hi >= lo ? hi - lo + 1 : 0;
}

// Number of keys in the list of row r (before splitting).
__device__ __forceinline__ int64_t key_list_length(const GatherParams &p, int64_t r)
{
    if (p.list_kind == KEYS_TOKEN_INDICES) {
        int64_t n = p.counts[r];
        return n < 0 ? 0 : (n > p.width ? p.width : n);
    }
    if (p.list_kind == KEYS_BLOCKS)
        return p.width * p.block_size;
    return p.window + p.width;
}

// ------------------------------------------------------------------ key pipeline
//
// Key j of (row r, kv head g) reaches its K/V rows through three dependent reads:
//   1. its list entry (a position, a block id, or a compressed entry number);
//   2. the page-table entry of the page holding that position;
//   3. the K and V rows themselves.
// The gather loops run these as a pipeline, several batches apart. Every stage issues
// exactly one load per key whether or not the key is present: a key past the list,
// clipped, unused or outside the cache reads a harmless dummy location and carries
// present = false, so that all code paths issue the same loads and the compiler can
// wait for exactly the oldest batch. Entries at or past counts are never loaded.

// Stage 1: address of key jj's list entry (or a dummy, whose value is not used).
// Block of a block-sparse list slot jj (below 2^31: the host bounds topk * block_size
// by 2^30): a shift for power-of-two block sizes, else a 32-bit division.
__device__ __forceinline__ uint32_t block_of(const GatherParams &p, int64_t jj)
{
    const uint32_t j = (uint32_t)jj;
    return p.block_shift >= 0 ? j >> p.block_shift : j / (uint32_t)p.block_size;
}

template <int LIST>
__device__ __forceinline__ const int32_t *entry_ptr(const GatherParams &p, int64_t r, int g, int64_t jj,
                                                    bool present)
{
    const int32_t *dummy = reinterpret_cast<const int32_t *>(p.row_off);
    if (!present)
        return dummy;
    if constexpr (LIST == KEYS_TOKEN_INDICES)
        return p.indices + r * p.width + jj;
    if constexpr (LIST == KEYS_BLOCKS)
        return p.indices + ((int64_t)g * p.total_q + r) * p.width + block_of(p, jj);
    return jj < p.window ? dummy : p.indices + r * p.width + (jj - p.window);
}

// Stage 2 input: the position the entry names, and which leaf holds it. Positions
// are below 2^31 (int32 lists; a block-sparse position past the row is not present).
struct KeyPos {
    int32_t tok;       // position (or compressed entry); meaningful when present
    bool comp;         // latent: compressed leaf
    bool present;
};

template <int LIST>
__device__ __forceinline__ KeyPos key_pos(const GatherParams &p, int64_t pos, int64_t jj, int32_t raw,
                                          bool present)
{
    KeyPos k{raw, false, present};
    if constexpr (LIST == KEYS_BLOCKS) {
        const int32_t bs = p.block_size;
        const int32_t t = (int32_t)block_of(p, jj);
        const int64_t tok = (int64_t)raw * bs + ((int32_t)jj - t * bs);
        k.present = present && raw >= 0 && tok <= pos;
        k.tok = (int32_t)tok;
    } else if constexpr (LIST == KEYS_LATENT) {
        const bool win = jj < p.window;
        k.tok = win ? (int32_t)(pos - p.window + 1 + jj) : raw;
        k.comp = !win;
    } else if constexpr (LIST == KEYS_DENSE) {
        k.tok = (int32_t)(pos + jj);   // row index of the key in the ragged k/v (pos = the row's first key)
    }
    k.present = k.present && k.tok >= 0;
    return k;
}

// Stage 2 for one leaf: logical page and slot of a position, and whether the page
// table covers it (shift and mask for power-of-two page sizes, else a multiply-high
// that is exact below 2^31).
__device__ __forceinline__ const uint32_t *leaf_entry_ptr(const CacheAddr &c, int b, uint32_t t, bool &in,
                                                          int32_t &slot)
{
    uint32_t lp;
    if (c.page_shift >= 0) {
        lp = t >> c.page_shift;
        slot = (int32_t)(t & c.page_mask);
    } else {
        lp = (uint32_t)(((uint64_t)t * c.magic) >> c.magic_shift);
        slot = (int32_t)(t - lp * (uint32_t)c.page_size);
    }
    in = (int64_t)lp < c.max_pages;
    return c.lut + (uint64_t)(uint32_t)b * (uint64_t)c.max_pages + lp;
}

// Stage 2: address of the page-table entry of k (or a dummy). Updates k.present for
// positions beyond the page table. Latent keys live in one of two leaves: both
// addresses are formed and the result selected, so that every leaf field stays a
// scalar kernel argument (a per-lane choice of leaf would otherwise become a per-lane
// address into the parameter block, loaded with vector loads).
template <int LIST>
__device__ __forceinline__ const uint32_t *page_entry_ptr(const GatherParams &p, int b, KeyPos &k,
                                                          int32_t &slot)
{
    const uint32_t t = (uint32_t)k.tok & 0x7fffffffu;
    bool in;
    const uint32_t *e = leaf_entry_ptr(p.kv, b, t, in, slot);
    if constexpr (LIST == KEYS_LATENT) {
        bool in_c;
        int32_t slot_c;
        const uint32_t *e_c = leaf_entry_ptr(p.comp, b, t, in_c, slot_c);
        e = k.comp ? e_c : e;
        in = k.comp ? in_c : in;
        slot = k.comp ? slot_c : slot;
    }
    k.present = k.present && in;
    return k.present ? e : p.kv.lut;
}

// Stage 3 for one leaf: byte address of (page, slot) of the addressed layer plus
// `head_b` bytes: one 32x32->64 multiply-add on top of a 32-bit in-page offset.
__device__ __forceinline__ const char *leaf_row(const CacheAddr &c, uint32_t page, int32_t slot, uint32_t head_b,
                                                bool &in)
{
    in = (int64_t)page < c.num_pages;
    const uint32_t inpage = c.layer_off_b + (uint32_t)slot * c.slot_stride_b + head_b;
    return static_cast<const char *>(c.blocks) + ((uint64_t)page * c.page_stride_b + inpage);
}

// Stage 3: byte address of k's plane-0 row for kv head g (or `dummy`).
template <int EB, int LIST>
__device__ __forceinline__ const char *row_address(const GatherParams &p, const KeyPos &k, uint32_t page,
                                                   int32_t slot, int g, const char *dummy, bool &present)
{
    if constexpr (LIST == KEYS_DENSE) {
        present = k.present;
        return present ? static_cast<const char *>(p.dense_k) +
                             ((int64_t)k.tok * p.num_kv_heads + g) * (int64_t)p.head_dim * EB
                       : dummy;
    }
    const uint32_t head_b = LIST == KEYS_LATENT ? 0u : (uint32_t)(g * p.head_dim * EB);
    bool in;
    const char *a = leaf_row(p.kv, page, slot, head_b, in);
    if constexpr (LIST == KEYS_LATENT) {
        bool in_c;
        const char *a_c = leaf_row(p.comp, page, slot, head_b, in_c);
        a = k.comp ? a_c : a;
        in = k.comp ? in_c : in;
    }
    present = k.present && in;
    return present ? a : dummy;
}

// Stage 3 without the kv head term: byte address of k's plane-0 row of kv head 0 and
// whether k is present (the caller adds head * head_dim * elem bytes, and uses the
// address only when present).
template <int EB, int LIST>
__device__ __forceinline__ const char *row_base(const GatherParams &p, const KeyPos &k, uint32_t page, int32_t slot,
                                                bool &present)
{
    if constexpr (LIST == KEYS_DENSE) {
        present = k.present;
        return static_cast<const char *>(p.dense_k) + (int64_t)k.tok * p.num_kv_heads * (int64_t)p.head_dim * EB;
    }
    bool in;
    const char *a = leaf_row(p.kv, page, slot, 0u, in);
    if constexpr (LIST == KEYS_LATENT) {
        bool in_c;
        const char *a_c = leaf_row(p.comp, page, slot, 0u, in_c);
        a = k.comp ? a_c : a;
        in = k.comp ? in_c : in;
    }
    present = k.present && in;
    return a;
}

// Normalising factor of a finished softmax state (reference M, sum L, log2 domain):
// out = acc * factor. With a sink logit (natural-log units, not scaled) the sink
// joins the denominator once; a row with no keys is all zeros.
__device__ __forceinline__ float final_factor(const GatherParams &p, int64_t head, float M, float L)
{
    float c = 1.f;
    if (p.sink) {
        const float sl = p.sink[head] * 1.44269504088896340736f;
        const float M2 = fmaxf(M, sl);
        c = __builtin_amdgcn_exp2f(M - M2);
        L = L * c + __builtin_amdgcn_exp2f(sl - M2);
    }
    return L > 0.f ? c / L : 0.f;
}

// ------------------------------------------------------------------ split-K merge
//
// Each split s leaves, per (row, q head), a log2-domain reference m_s, the sum
// l_s = sum_j 2^(t_j - m_s) and acc_s = sum_j 2^(t_j - m_s) V_j. The exact result is
//   out = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s,   M = max_s m_s
// ("Struct_msa_attention_ragged_paged" design notes: partitioned KV bands merged by a
// reduction), with the sink (latent attention) joining the denominator once; a (row,
// head) that saw no key in any split is all zeros.

__device__ __forceinline__ void store_out4(void *out, int32_t out_dtype, int64_t idx, f32x4_t v);

// Merge of outputs d0 .. d0+3 of partial row `rel` (partials are indexed from row
// split_row0 on) into the output of (row, head) `rh`; UNROLL partials' loads go out
// together.
template <int UNROLL = 8>
__device__ __forceinline__ void merge_splits4(const GatherParams &p, int64_t rh, int64_t rel, int d0)
{
    const int S = p.num_splits;
    const int D = p.head_dim;
    const int64_t RH = (p.total_q - p.split_row0) * p.num_q_heads;
    float M = kNoKey;
#pragma unroll UNROLL
    for (int s = 0; s < S; ++s)
        M = fmaxf(M, p.ws_ml[((int64_t)s * RH + rel) * 2]);
    float L = 0.f;
    f32x4_t a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll UNROLL
    for (int s = 0; s < S; ++s) {
        const int64_t srh = (int64_t)s * RH + rel;
        const float c = __builtin_amdgcn_exp2f(p.ws_ml[srh * 2] - M);
        L += c * p.ws_ml[srh * 2 + 1];
        a += c * *reinterpret_cast<const f32x4_t *>(p.ws_acc + srh * D + d0);
    }
    store_out4(p.out, p.out_dtype, rh * D + d0, a * final_factor(p, rh % p.num_q_heads, M, L));
}

// Four consecutive outputs (idx a multiple of 4): bf16 (round to nearest even) or fp32.
__device__ __forceinline__ void store_out4(void *out, int32_t out_dtype, int64_t idx, f32x4_t v)
{
    if (out_dtype == QSA_BF16) {
        typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
        const u32x2v w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        *reinterpret_cast<u32x2v *>(static_cast<uint16_t *>(out) + idx) = w;
    } else {
        *reinterpret_cast<f32x4_t *>(static_cast<float *>(out) + idx) = v;
    }
}

// Two adjacent outputs (idx even): one 4-byte bf16 pair or one 8-byte float pair.
__device__ __forceinline__ void store_out2(void *out, int32_t out_dtype, int64_t idx, float v0, float v1)
{
    if (out_dtype == QSA_BF16)
        *reinterpret_cast<uint32_t *>(static_cast<uint16_t *>(out) + idx) = pack_bf16x2(v0, v1);
    else
        *reinterpret_cast<float2 *>(static_cast<float *>(out) + idx) = make_float2(v0, v1);
}

__device__ __forceinline__ void store_out(void *out, int32_t out_dtype, int64_t idx, float v)
{
    if (out_dtype == QSA_BF16)
        static_cast<uint16_t *>(out)[idx] = (uint16_t)f32_to_bf16_bits(v);
    else
        static_cast<float *>(out)[idx] = v;
}

}  // namespace qsa
