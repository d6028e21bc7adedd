// Device-side building blocks shared by the gather kernels (gfx950, wave64):
// element decode, wavefront reductions, the key-address generator and the
// online-softmax state merge.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qsa_host.hpp"

namespace qsa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

typedef const __attribute__((address_space(1))) u32x4 global_u32x4;

constexpr float kNegInf = -__builtin_huge_valf();

// 16-byte load through the global address space (global_load_dwordx4 rather than a
// flat load: the pointer came out of LDS, so the compiler cannot prove where it points).
__device__ __forceinline__ u32x4 ldg16(const void *p) { return *(global_u32x4 *)(p); }

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

// binary32 -> bf16 with round-to-nearest-even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

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

// Element offset of (position p, plane 0, kv head 0) in a paged leaf, or -1 when
// the entry does not address the cache (position outside the page table, or page
// id past the pool); such entries are skipped, never dereferenced.
__device__ __forceinline__ int64_t key_elem_offset(const CacheAddr &c, int64_t b, int64_t p)
{
    if (p < 0)
        return -1;
    int64_t lp, slot;
    if (c.page_shift >= 0) {
        lp = p >> c.page_shift;
        slot = p & (c.page_size - 1);
    } else {
        lp = p / c.page_size;
        slot = p - lp * c.page_size;
    }
    if (lp >= c.max_pages)
        return -1;
    uint32_t page = c.lut[b * c.max_pages + lp];
    if ((int64_t)page >= c.num_pages)
        return -1;
    return (int64_t)page * c.page_stride + c.layer_off + slot * c.slot_stride;
}

// Sequence of row r: the b with row_off[b] <= r < row_off[b+1] (binary search;
// rows of empty sequences are skipped naturally).
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

// Byte address of the plane-0 row of key j of (row r, sequence b, kv head g), or
// nullptr when the key is not present (past the list, clipped, unused or outside
// the cache). `pos` is the row's position, `n` the key-list length.
template <int eb>
__device__ __forceinline__ const char *key_address(const GatherParams &p, int b, int64_t r,
                                                   int64_t pos, int g, int64_t j)
{
    int64_t off;
    if (p.list_kind == KEYS_TOKEN_INDICES) {
        int64_t tok = p.indices[r * p.width + j];
        off = key_elem_offset(p.kv, b, tok);
        if (off < 0)
            return nullptr;
        return static_cast<const char *>(p.kv.blocks) + (off + (int64_t)g * p.head_dim) * eb;
    }
    if (p.list_kind == KEYS_BLOCKS) {
        int64_t t = j / p.block_size;
        int64_t i = j - t * p.block_size;
        int64_t id = p.indices[((int64_t)g * p.total_q + r) * p.width + t];
        int64_t tok = id * p.block_size + i;
        if (id < 0 || tok > pos)
            return nullptr;
        off = key_elem_offset(p.kv, b, tok);
        if (off < 0)
            return nullptr;
        return static_cast<const char *>(p.kv.blocks) + (off + (int64_t)g * p.head_dim) * eb;
    }
    // KEYS_LATENT: window positions first, then listed compressed entries
    if (j < p.window) {
        int64_t tok = pos - p.window + 1 + j;
        off = key_elem_offset(p.kv, b, tok);
        if (off < 0)
            return nullptr;
        return static_cast<const char *>(p.kv.blocks) + off * eb;
    }
    int64_t e = p.indices[r * p.width + (j - p.window)];
    off = key_elem_offset(p.comp, b, e);
    if (off < 0)
        return nullptr;
    return static_cast<const char *>(p.comp.blocks) + off * eb;
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

// Scale factors for merging two online-softmax states with maxima m and m2
// (log2-domain scores, -inf when a state has seen no key): the merged maximum is
// mnew and the states are weighted by c1 = 2^(m - mnew) and c2 = 2^(m2 - mnew).
__device__ __forceinline__ void merge_scale(float m, float m2, float &c1, float &c2, float &mnew)
{
    mnew = fmaxf(m, m2);
    float ref = mnew == kNegInf ? 0.f : mnew;
    c1 = __builtin_amdgcn_exp2f(m - ref);
    c2 = __builtin_amdgcn_exp2f(m2 - ref);
}

__device__ __forceinline__ void store_out(void *out, int32_t out_dtype, int64_t idx, float v)
{
    if (out_dtype == QSA_BF16)
        static_cast<uint16_t *>(out)[idx] = (uint16_t)f32_to_bf16_bits(v);
    else
        static_cast<float *>(out)[idx] = v;
}

}  // namespace qsa
