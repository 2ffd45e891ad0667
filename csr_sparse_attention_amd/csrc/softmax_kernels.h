// Standalone CSR row softmax, the middle stage of the unfused pipeline
// SDDMM -> row-softmax -> SpMM: p_e = exp(scale * s_e - m_i) / l_i over the
// stored entries e of each row i, with m_i the row maximum of scale * s and
// l_i the sum of exponentials.
//
// Three kernels over the merge-path chunks of the fp32 kernels:
//   k_softmax_stats  - (m, l) of every row segment of a chunk (a long segment
//                      by the whole wave, short ones by groups of W lanes);
//                      complete rows write their statistics, split rows leave
//                      (m, l) pieces in the carry slots;
//   k_softmax_fixup  - merges the pieces of each split row in chunk order;
//   k_softmax_norm   - writes p_e for every entry of the chunk.
#pragma once

#include "args.h"
#include "common.h"

namespace csrk {

template <int D>
struct SmShared {
    int32_t rp[CSR_WAVES_PER_BLOCK][D + 2];
    float s[CSR_WAVES_PER_BLOCK][D];
};

// (m, l) of scale * s[e] over e = kb + t, kb + t + n, ... merged over the n
// lanes of an aligned lane set.
__device__ __forceinline__ void sm_stats(const float* s, int kb, int ke, int t, int n, float scale, float& m, float& l)
{
    m = -INFINITY;
    l = 0.f;
    for (int e = kb + t; e < ke; e += n) {
        const float x = s[e] * scale;
        if (x > m) {
            l = l * exp_neg(m - x) + 1.f;
            m = x;
        } else {
            l += exp_neg(x - m);
        }
    }
    for (int k = 1; k < n; k <<= 1) {
        const float m2 = shfl_xor(m, k), l2 = shfl_xor(l, k);
        const float mm = fmaxf(m, m2);
        const float a = (l > 0.f) ? l * exp_neg(m - mm) : 0.f;
        const float b = (l2 > 0.f) ? l2 * exp_neg(m2 - mm) : 0.f;
        m = mm;
        l = a + b;
    }
}

template <int D>
__device__ __forceinline__ bool sm_stage(const SoftmaxArgs& a, SmShared<D>& sh, int wave, int lane, int64_t chunk,
                                         int& x0, int& y0, int& x1, int& y1, int& nrow, bool& slotB)
{
    const bool active = chunk < a.n_chunks;
    if (active) {
        x0 = a.part[2 * chunk];
        y0 = a.part[2 * chunk + 1];
        x1 = a.part[2 * chunk + 2];
        y1 = a.part[2 * chunk + 3];
        const int rpx1 = (x1 < a.n_rows) ? a.row_ptr[x1] : y1;
        slotB = (x1 < a.n_rows) && (max(rpx1, y0) < y1);
        nrow = x1 - x0 + (slotB ? 1 : 0);
        for (int i = lane; i <= nrow; i += CSR_WAVE) sh.rp[wave][i] = a.row_ptr[x0 + i];
        for (int i = lane; i < y1 - y0; i += CSR_WAVE) sh.s[wave][i] = ld_stream(a.scores + y0 + i);
    }
    __syncthreads();
    return active;
}

template <int D>
__global__ __launch_bounds__(CSR_BLOCK) void k_softmax_stats(SoftmaxArgs a)
{
    __shared__ SmShared<D> sh;
    const int wave = threadIdx.x / CSR_WAVE, lane = lane_id();
    const int64_t chunk = (int64_t)blockIdx.x * CSR_WAVES_PER_BLOCK + wave;
    int x0 = 0, y0 = 0, x1 = 0, y1 = 0, nrow = 0;
    bool slotB = false;
    if (!sm_stage<D>(a, sh, wave, lane, chunk, x0, y0, x1, y1, nrow, slotB)) return;
    const int32_t* rp = sh.rp[wave];
    const float* s = sh.s[wave] - y0;
    const bool slotA = (x0 < x1) && (rp[0] < y0);
    if (lane == 0) {
        a.carry_row[2 * chunk] = slotA ? x0 : -1;
        a.carry_row[2 * chunk + 1] = slotB ? x1 : -1;
    }
    const int nend = x1 - x0;
    const int W = a.W, G = CSR_WAVE / W, g = lane / W, lg = lane & (W - 1);
    auto emit = [&](int i, float m, float l) {
        if (i < nend && rp[i] >= y0) {
            a.stats[2 * ((int64_t)x0 + i)] = m;
            a.stats[2 * ((int64_t)x0 + i) + 1] = l;
        } else {
            const int64_t slot = 2 * chunk + ((i == nend) ? 1 : 0);
            a.carry_ml[2 * slot] = m;
            a.carry_ml[2 * slot + 1] = l;
        }
    };
    for (int i = 0; i < nrow; ++i) {
        const int sb = max(rp[i], y0), se = min(rp[i + 1], y1);
        if (se - sb < a.long_row) continue;
        float m, l;
        sm_stats(s, sb, se, lane, CSR_WAVE, a.scale, m, l);
        if (lane == 0) emit(i, m, l);
    }
    for (int i = g; i < nrow; i += G) {
        const int sb = max(rp[i], y0), se = min(rp[i + 1], y1);
        if (se - sb >= a.long_row) continue;
        float m, l;
        sm_stats(s, sb, se, lg, W, a.scale, m, l);
        if (lg == 0) emit(i, m, l);
    }
}

// Merges the (m, l) pieces of rows split across chunks (one wave per chunk
// whose slot A holds a row; the pieces are slot B of the run of chunks before
// it, then slot A).
__global__ __launch_bounds__(CSR_BLOCK) void k_softmax_fixup(SoftmaxArgs a)
{
    const int wave = threadIdx.x / CSR_WAVE, lane = lane_id();
    const int64_t c = (int64_t)blockIdx.x * CSR_WAVES_PER_BLOCK + wave;
    if (c >= a.n_chunks) return;
    const int r = a.carry_row[2 * c];
    if (r < 0) return;
    int64_t k0 = c;
    while (true) {
        const int64_t idx = k0 - 1 - lane;
        const bool ok = idx >= 0 && a.carry_row[2 * idx + 1] == r;
        const uint64_t mask = __ballot(ok);
        const int n = (~mask == 0) ? 64 : __builtin_ctzll(~mask);
        k0 -= n;
        if (n < 64) break;
    }
    const int64_t np = c - k0 + 1;
    float m = -INFINITY, l = 0.f;
    for (int64_t p = lane; p < np; p += CSR_WAVE) {
        const int64_t s = (p < np - 1) ? 2 * (k0 + p) + 1 : 2 * c;
        const float m2 = a.carry_ml[2 * s], l2 = a.carry_ml[2 * s + 1];
        const float mm = fmaxf(m, m2);
        const float x = (l > 0.f) ? l * exp_neg(m - mm) : 0.f;
        const float y = (l2 > 0.f) ? l2 * exp_neg(m2 - mm) : 0.f;
        m = mm;
        l = x + y;
    }
    for (int k = 1; k < CSR_WAVE; k <<= 1) {
        const float m2 = shfl_xor(m, k), l2 = shfl_xor(l, k);
        const float mm = fmaxf(m, m2);
        const float x = (l > 0.f) ? l * exp_neg(m - mm) : 0.f;
        const float y = (l2 > 0.f) ? l2 * exp_neg(m2 - mm) : 0.f;
        m = mm;
        l = x + y;
    }
    if (lane == 0) {
        a.stats[2 * (int64_t)r] = m;
        a.stats[2 * (int64_t)r + 1] = l;
    }
}

template <int D>
__global__ __launch_bounds__(CSR_BLOCK) void k_softmax_norm(SoftmaxArgs a)
{
    __shared__ SmShared<D> sh;
    const int wave = threadIdx.x / CSR_WAVE, lane = lane_id();
    const int64_t chunk = (int64_t)blockIdx.x * CSR_WAVES_PER_BLOCK + wave;
    int x0 = 0, y0 = 0, x1 = 0, y1 = 0, nrow = 0;
    bool slotB = false;
    if (!sm_stage<D>(a, sh, wave, lane, chunk, x0, y0, x1, y1, nrow, slotB)) return;
    const int32_t* rp = sh.rp[wave];
    const float* s = sh.s[wave] - y0;
    const int W = a.W, G = CSR_WAVE / W, g = lane / W, lg = lane & (W - 1);
    auto write = [&](int i, int sb, int se, int t, int n) {
        const int64_t row = (int64_t)x0 + i;
        const float m = a.stats[2 * row], inv = 1.f / a.stats[2 * row + 1];
        for (int e = sb + t; e < se; e += n) a.probs[e] = exp_neg(s[e] * a.scale - m) * inv;
    };
    for (int i = 0; i < nrow; ++i) {
        const int sb = max(rp[i], y0), se = min(rp[i + 1], y1);
        if (se - sb < a.long_row || se <= sb) continue;
        write(i, sb, se, lane, CSR_WAVE);
    }
    for (int i = g; i < nrow; i += G) {
        const int sb = max(rp[i], y0), se = min(rp[i + 1], y1);
        if (se - sb >= a.long_row || se <= sb) continue;
        write(i, sb, se, lg, W);
    }
}

}  // namespace csrk
