// Device-side building blocks shared by the CSR kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <climits>

#include "../../include/csrsa.h"

#define CSR_WAVE 64
#define CSR_BLOCK 256
#define CSR_WAVES_PER_BLOCK (CSR_BLOCK / CSR_WAVE)
// XCDs of an MI355X; a launch's workgroups are dealt to them in turn
#define CSR_XCDS 8

namespace csrk {

// ---------------------------------------------------------------------------
// fp32 vectors of 1, 2 or 4 lanes (one global load / store instruction each)
// ---------------------------------------------------------------------------
template <int VEC> struct vtype;
template <> struct vtype<1> { typedef float t; };
template <> struct vtype<2> { typedef float2 t; };
template <> struct vtype<4> { typedef float4 t; };

template <int VEC>
__device__ __forceinline__ void vload(float (&d)[VEC], const float* p)
{
    typedef typename vtype<VEC>::t T;
    T v = *reinterpret_cast<const T*>(p);
    if constexpr (VEC == 1) {
        d[0] = v;
    } else if constexpr (VEC == 2) {
        d[0] = v.x; d[1] = v.y;
    } else {
        d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
    }
}

template <int VEC>
__device__ __forceinline__ void vstore(float* p, const float (&s)[VEC])
{
    if constexpr (VEC == 8) {
        // two 16-byte stores (the lane layout of bf16 operands read 8 at a time)
        reinterpret_cast<float4*>(p)[0] = make_float4(s[0], s[1], s[2], s[3]);
        reinterpret_cast<float4*>(p)[1] = make_float4(s[4], s[5], s[6], s[7]);
        return;
    } else {
        typedef typename vtype<VEC>::t T;
        T v;
        if constexpr (VEC == 1) {
            v = s[0];
        } else if constexpr (VEC == 2) {
            v.x = s[0]; v.y = s[1];
        } else {
            v.x = s[0]; v.y = s[1]; v.z = s[2]; v.w = s[3];
        }
        *reinterpret_cast<T*>(p) = v;
    }
}

// bfloat16 operands: raw 16-bit patterns in memory, widened exactly to fp32
// in registers (the 16 bits become the float's high half).  bf16_t is a tag
// type; the kernels read it VEC elements at a time (VEC = 2, 4, 8: one 4-,
// 8- or 16-byte load per lane).
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ void widen2(float& lo, float& hi, uint32_t w)
{
    lo = __uint_as_float(w << 16);
    hi = __uint_as_float(w & 0xffff0000u);
}

// VEC consecutive elements of type T at p, as fp32
template <typename T, int VEC>
__device__ __forceinline__ void vload_t(float (&d)[VEC], const T* p)
{
    if constexpr (sizeof(T) == 4) {
        vload<VEC>(d, reinterpret_cast<const float*>(p));
    } else if constexpr (VEC == 2) {
        widen2(d[0], d[1], *reinterpret_cast<const uint32_t*>(p));
    } else if constexpr (VEC == 4) {
        const uint2 r = *reinterpret_cast<const uint2*>(p);
        widen2(d[0], d[1], r.x);
        widen2(d[2], d[3], r.y);
    } else {
        static_assert(VEC == 8, "bf16 operands are read 2, 4 or 8 at a time");
        const uint4 r = *reinterpret_cast<const uint4*>(p);
        widen2(d[0], d[1], r.x);
        widen2(d[2], d[3], r.y);
        widen2(d[4], d[5], r.z);
        widen2(d[6], d[7], r.w);
    }
}

// VEC consecutive bf16 values at p, still packed: VEC / 2 words of two
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <int VEC>
__device__ __forceinline__ void vload_packed(uint32_t (&d)[VEC / 2], const bf16_t* p)
{
    if constexpr (VEC == 2) {
        d[0] = *reinterpret_cast<const uint32_t*>(p);
    } else if constexpr (VEC == 4) {
        const uint2 r = *reinterpret_cast<const uint2*>(p);
        d[0] = r.x;
        d[1] = r.y;
    } else {
        static_assert(VEC == 8, "bf16 operands are read 2, 4 or 8 at a time");
        const uint4 r = *reinterpret_cast<const uint4*>(p);
        d[0] = r.x;
        d[1] = r.y;
        d[2] = r.z;
        d[3] = r.w;
    }
}

// a0 b0 + a1 b1 + c over two packed bf16 pairs, in fp32 (v_dot2 on gfx950:
// the bf16 products are exact in fp32 and the sum keeps fp32 accuracy)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                           false);
}

// the bf16 pair of two fp32 values that are bf16 values widened (exact)
__device__ __forceinline__ uint32_t pack_bf16_exact(float lo, float hi)
{
    return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
}

// Streamed store (an output row written once and not read again by the
// kernel): non-temporal, so that it does not push the gathered feature rows
// out of the caches.
template <int VEC>
__device__ __forceinline__ void vstore_stream(float* p, const float (&s)[VEC])
{
    typedef float T __attribute__((ext_vector_type(VEC == 1 ? 1 : (VEC == 8 ? 4 : VEC))));
    if constexpr (VEC == 8) {
        T v0 = {s[0], s[1], s[2], s[3]}, v1 = {s[4], s[5], s[6], s[7]};
        __builtin_nontemporal_store(v0, reinterpret_cast<T*>(p));
        __builtin_nontemporal_store(v1, reinterpret_cast<T*>(p + 4));
    } else if constexpr (VEC == 1) {
        __builtin_nontemporal_store(s[0], p);
    } else if constexpr (VEC == 2) {
        T v = {s[0], s[1]};
        __builtin_nontemporal_store(v, reinterpret_cast<T*>(p));
    } else {
        T v = {s[0], s[1], s[2], s[3]};
        __builtin_nontemporal_store(v, reinterpret_cast<T*>(p));
    }
}

// Streamed (read-once) loads of the CSR arrays: non-temporal so that they do
// not push the gathered feature rows out of the caches.
__device__ __forceinline__ int ld_stream(const int32_t* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ float ld_stream(const float* p) { return __builtin_nontemporal_load(p); }

// Stages a merge-path chunk in LDS with the 64 lanes of a wave: row_ptr
// entries rp_src[0 .. nr) (nr <= NR * 64) and, for the chunk's entries,
// col_src[0 .. ne) and optionally val_src[0 .. ne) (ne <= NE * 64; a null
// val_src with FILL set stores 1.0), or val_src[val_idx[i]] for i < ne when
// val_idx is given (values kept in another entry order).  Every global load
// is issued before the first LDS store, so the loads of one wave overlap
// instead of each waiting for the previous one.  The per-entry arrays are
// read once: non-temporal.
template <int NR, int NE, bool VALS, typename V>
__device__ __forceinline__ void stage_chunk(int32_t* rp_dst, const int32_t* rp_src, int nr, int32_t* col_dst,
                                            const int32_t* col_src, V* val_dst, const V* val_src, int ne,
                                            const int32_t* val_idx = nullptr)
{
    const int lane = __lane_id();
    int32_t r[NR], c[NE];
    V v[NE];
#pragma unroll
    for (int k = 0; k < NR; ++k) {
        const int i = lane + k * 64;
        if (i < nr) r[k] = rp_src[i];
    }
    if (VALS && val_src && val_idx) {
        int32_t ix[NE];
#pragma unroll
        for (int k = 0; k < NE; ++k) {
            const int i = lane + k * 64;
            if (i < ne) {
                if (col_src) c[k] = __builtin_nontemporal_load(col_src + i);
                ix[k] = __builtin_nontemporal_load(val_idx + i);
            }
        }
#pragma unroll
        for (int k = 0; k < NE; ++k) {
            const int i = lane + k * 64;
            if (i < ne) v[k] = val_src[ix[k]];
        }
    } else {
#pragma unroll
        for (int k = 0; k < NE; ++k) {
            const int i = lane + k * 64;
            if (i < ne) {
                if (col_src) c[k] = __builtin_nontemporal_load(col_src + i);
                if constexpr (VALS) v[k] = val_src ? __builtin_nontemporal_load(val_src + i) : V(1);
            }
        }
    }
#pragma unroll
    for (int k = 0; k < NR; ++k) {
        const int i = lane + k * 64;
        if (i < nr) rp_dst[i] = r[k];
    }
#pragma unroll
    for (int k = 0; k < NE; ++k) {
        const int i = lane + k * 64;
        if (i < ne) {
            if (col_src) col_dst[i] = c[k];
            if constexpr (VALS) val_dst[i] = v[k];
        }
    }
}

// exp(x) for x <= 0 as 2^(x log2 e) on the hardware exp2 unit.
__device__ __forceinline__ float exp_neg(float x)
{
    return __builtin_amdgcn_exp2f(x * 1.44269504088896341f);
}

__device__ __forceinline__ float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, CSR_WAVE); }
__device__ __forceinline__ int lane_id() { return __lane_id(); }

// ---------------------------------------------------------------------------
// Cross-lane moves on the DPP path (VALU, no LDS traffic).  GFX9 controls:
// row_shr:n = 0x110 + n, wave_shl:1 = 0x130, row_bcast:15 = 0x142,
// row_bcast:31 = 0x143.  A lane whose source lies outside its row (or the
// wave), or whose row is masked off, keeps `old`.
// ---------------------------------------------------------------------------
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_i(int old, int v)
{
    return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xf, false);
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f(float old, float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL, ROW_MASK, 0xf,
                                                      false));
}

// Every lane of an aligned group of W lanes (W a power of two <= 64) gets
// the group's sum of v[k].  After the steps for distances 1 and 2 (quad
// permutes [1,0,3,2] and [2,3,0,1]) each quad holds its sum in all lanes, so
// the next steps may pair a lane with any lane of the other half of its
// group: the half-row mirror (lane i of 8 with 7 - i) and the row mirror
// (i of 16 with 15 - i), still on the DPP path; distance 16 is a swizzle
// inside each 32 lanes, distance 32 a permute.  W is uniform over the wave.
template <int N>
__device__ __forceinline__ void group_sum_lanes(float (&v)[N], int W)
{
    if (W > 1) {
#pragma unroll
        for (int k = 0; k < N; ++k) v[k] += dpp_f<0xB1, 0xf>(0.f, v[k]);
    }
    if (W > 2) {
#pragma unroll
        for (int k = 0; k < N; ++k) v[k] += dpp_f<0x4E, 0xf>(0.f, v[k]);
    }
    if (W > 4) {
#pragma unroll
        for (int k = 0; k < N; ++k) v[k] += dpp_f<0x141, 0xf>(0.f, v[k]);
    }
    if (W > 8) {
#pragma unroll
        for (int k = 0; k < N; ++k) v[k] += dpp_f<0x140, 0xf>(0.f, v[k]);
    }
    if (W > 16) {
        // bit mode: and 0x1f, or 0, xor 0x10
#pragma unroll
        for (int k = 0; k < N; ++k) v[k] += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v[k]), 0x401F));
    }
    if (W > 32) {
#pragma unroll
        for (int k = 0; k < N; ++k) v[k] += shfl_xor(v[k], 32);
    }
}

// Lane l + 1's value (lane 63: `old`).
__device__ __forceinline__ int next_lane_i(int old, int v) { return dpp_i<0x130, 0xf>(old, v); }

__device__ __forceinline__ int lane63_i(int v) { return __builtin_amdgcn_readlane(v, CSR_WAVE - 1); }
__device__ __forceinline__ float lane63_f(float v)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), CSR_WAVE - 1));
}

// One step of a segmented sum: add the source lane's partial sum when it
// carries the same run id.
template <int CTRL, int ROW_MASK, int A, int B>
__device__ __forceinline__ void seg_sum_step(int id, float (&v)[A][B])
{
    const bool join = dpp_i<CTRL, ROW_MASK>(INT_MIN, id) == id;
#pragma unroll
    for (int a = 0; a < A; ++a)
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const float o = dpp_f<CTRL, ROW_MASK>(0.f, v[a][b]);
            if (join) v[a][b] += o;
        }
}

// Inclusive segmented sum over the wave: runs are lanes with equal ids, and
// ids never decrease from one lane to the next among the lanes that may
// join (any other lane carries an id no lane shares), so two lanes with one
// id enclose a single run.  Within each row of 16 lanes the partial sums
// shift by 1, 2, 4 and 8 lanes (Hillis-Steele); then lane 15 of rows 0 and 2
// feeds rows 1 and 3, and lane 31 feeds rows 2 and 3, which completes every
// run across rows: each lane ends with the sum over its run up to itself.
template <int A, int B>
__device__ __forceinline__ void seg_sum_wave(int id, float (&v)[A][B])
{
    seg_sum_step<0x111, 0xf>(id, v);
    seg_sum_step<0x112, 0xf>(id, v);
    seg_sum_step<0x114, 0xf>(id, v);
    seg_sum_step<0x118, 0xf>(id, v);
    seg_sum_step<0x142, 0xa>(id, v);
    seg_sum_step<0x143, 0xc>(id, v);
}

// Sum over the lanes l, l ^ from, l ^ 2 from, ... (from a power of two < 64):
// afterwards every lane holds the sum over its coset.
__device__ __forceinline__ float xor_sum_from(float v, int from)
{
    for (int s = from; s < CSR_WAVE; s <<= 1) v += shfl_xor(v, s);
    return v;
}

// Sum over the lanes of an aligned group of W lanes.
template <int W>
__device__ __forceinline__ float group_sum(float v)
{
#pragma unroll
    for (int s = 1; s < W; s <<= 1) v += shfl_xor(v, s);
    return v;
}

template <int W>
__device__ __forceinline__ float group_max(float v)
{
#pragma unroll
    for (int s = 1; s < W; s <<= 1) v = fmaxf(v, shfl_xor(v, s));
    return v;
}

// Online softmax state (m = running maximum, l = sum of exp(t - m)) merged
// across the lanes l ^ s for s = from .. 32.  The lanes of one group must
// hold identical states on entry when from > 1.
__device__ __forceinline__ void softmax_merge_xor(float& m, float& l, int from, int to)
{
    for (int s = from; s < to; s <<= 1) {
        float m2 = shfl_xor(m, s);
        float l2 = shfl_xor(l, s);
        float mm = fmaxf(m, m2);
        float a = (l > 0.f) ? l * exp_neg(m - mm) : 0.f;
        float b = (l2 > 0.f) ? l2 * exp_neg(m2 - mm) : 0.f;
        m = mm;
        l = a + b;
    }
}

// The fix-up kernels give each wavefront a window of 64 consecutive chunks:
// one coalesced load tells which of them hold work (a split row ending
// there), and the wave then handles those one after the other.  Returns the
// window's first chunk, or -1 when the window is past the last chunk.
__device__ __forceinline__ int64_t fixup_window(int64_t n_chunks)
{
    const int64_t base = ((int64_t)blockIdx.x * CSR_WAVES_PER_BLOCK + threadIdx.x / CSR_WAVE) * CSR_WAVE;
    return base < n_chunks ? base : -1;
}

} // namespace csrk
