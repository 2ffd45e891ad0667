// Standalone CSR row softmax, the middle stage of the unfused pipeline
// SDDMM -> row-softmax -> SpMM: p_e = exp(scale * s_e - m_i) / l_i over the
// stored entries e of each row i, with m_i the row maximum of scale * s and
// l_i the sum of exponentials.
//
// Three kernels over the merge-path chunks of the fp32 kernels:
//   k_softmax_main   - stages the chunk's row_ptr and scores in LDS, forms
//                      (m, l) of every row segment (a long segment by the
//                      whole wave, short ones by groups of W lanes) into LDS,
//                      then writes p_e for every entry of the rows that lie
//                      wholly in the chunk, lanes over consecutive entries
//                      (coalesced); the segments of rows cut by a chunk
//                      boundary leave (m, l) pieces in the carry slots;
//   k_softmax_fixup  - merges the pieces of each split row in chunk order into
//                      that row's statistics;
//   k_softmax_split  - writes p_e for the entries of split rows only, a wave
//                      per chunk, lanes over entries.
// The scores are read once (plus the entries of split rows a second time).
#pragma once

#include "args.h"
#include "common.h"

namespace csrk {

template <int D>
struct SmShared {
    int32_t rp[CSR_WAVES_PER_BLOCK][D + 2];
    float s[CSR_WAVES_PER_BLOCK][D];
    float m[CSR_WAVES_PER_BLOCK][D + 2];
    float l[CSR_WAVES_PER_BLOCK][D + 2];
    uint16_t ri[CSR_WAVES_PER_BLOCK][D];  // row index (within the chunk) of each entry
};

// (m, l) of scale * s[e] over e = kb + t, kb + t + n, ... for the n lanes of
// an aligned lane set: the maximum first (butterfly of max), then the sum of
// exponentials (butterfly of sums), so the cross-lane steps need no rescaling.
__device__ __forceinline__ void sm_stats(const float* s, int kb, int ke, int t, int n, float scale, float& m, float& l)
{
    m = -INFINITY;
    for (int e = kb + t; e < ke; e += n) m = fmaxf(m, s[e] * scale);
    for (int k = 1; k < n; k <<= 1) m = fmaxf(m, shfl_xor(m, k));
    l = 0.f;
    for (int e = kb + t; e < ke; e += n) l += exp_neg(s[e] * scale - m);
    for (int k = 1; k < n; k <<= 1) l += shfl_xor(l, k);
}

template <int D>
__global__ __launch_bounds__(CSR_BLOCK) void k_softmax_main(SoftmaxArgs a)
{
    __shared__ SmShared<D> sh;
    const int wave = threadIdx.x / CSR_WAVE, lane = lane_id();
    const int64_t chunk = (int64_t)blockIdx.x * CSR_WAVES_PER_BLOCK + wave;
    const bool active = chunk < a.n_chunks;
    int x0 = 0, y0 = 0, x1 = 0, y1 = 0, nrow = 0;
    bool slotB = false;
    if (active) {
        x0 = a.part[2 * chunk];
        y0 = a.part[2 * chunk + 1];
        x1 = a.part[2 * chunk + 2];
        y1 = a.part[2 * chunk + 3];
        // rows x0 .. x1 (x1 only if it exists): row_ptr[x0 .. min(x1, n_rows - 1) + 1]
        const int nr = (x1 < a.n_rows ? x1 : (int)a.n_rows - 1) - x0 + 2;
        stage_chunk<(D + 2 + CSR_WAVE - 1) / CSR_WAVE, D / CSR_WAVE, true, float>(
            sh.rp[wave], a.row_ptr + x0, nr, nullptr, nullptr, sh.s[wave], a.scores + y0, y1 - y0);
    }
    __syncthreads();
    const int32_t* rp = sh.rp[wave];
    const float* s = sh.s[wave] - y0;
    const int nend = x1 - x0;
    const int W = a.W, G = CSR_WAVE / W, g = lane / W, lg = lane & (W - 1);
    if (active) {
        slotB = (x1 < a.n_rows) && (max(rp[x1 - x0], y0) < y1);
        nrow = x1 - x0 + (slotB ? 1 : 0);
        const bool slotA = (x0 < x1) && (rp[0] < y0);
        if (lane == 0) {
            a.carry_row[2 * chunk] = slotA ? x0 : -1;
            a.carry_row[2 * chunk + 1] = slotB ? x1 : -1;
        }
        // statistics of every segment; split segments also leave a piece
        auto keep = [&](int i, int sb, int se, float m, float l, bool writer, int t, int n) {
            if (writer) {
                sh.m[wave][i] = m;
                sh.l[wave][i] = l;
                if (!(i < nend && rp[i] >= y0)) {
                    const int64_t slot = 2 * chunk + ((i == nend) ? 1 : 0);
                    a.carry_ml[2 * slot] = m;
                    a.carry_ml[2 * slot + 1] = l;
                }
            }
            for (int e = sb + t; e < se; e += n) sh.ri[wave][e - y0] = (uint16_t)i;
        };
        for (int i = 0; i < nrow; ++i) {
            const int sb = max(rp[i], y0), se = min(rp[i + 1], y1);
            if (se - sb < a.long_row) continue;
            float m, l;
            sm_stats(s, sb, se, lane, CSR_WAVE, a.scale, m, l);
            keep(i, sb, se, m, l, lane == 0, lane, CSR_WAVE);
        }
        for (int i = g; i < nrow; i += G) {
            const int sb = max(rp[i], y0), se = min(rp[i + 1], y1);
            if (se - sb >= a.long_row) continue;
            float m, l;
            sm_stats(s, sb, se, lg, W, a.scale, m, l);
            keep(i, sb, se, m, l, lg == 0, lg, W);
        }
    }
    __syncthreads();
    if (!active) return;
    // probabilities of the rows wholly inside the chunk, lanes over entries
    for (int e = y0 + lane; e < y1; e += CSR_WAVE) {
        const int i = sh.ri[wave][e - y0];
        if (i < nend && rp[i] >= y0) a.probs[e] = exp_neg(s[e] * a.scale - sh.m[wave][i]) / sh.l[wave][i];
    }
}

// Merges the (m, l) pieces of rows split across chunks (one wave per chunk
// whose slot A holds a row; the pieces are slot B of the run of chunks before
// it, then slot A).
__device__ __forceinline__ void softmax_fixup_one(const SoftmaxArgs& a, int64_t c, int r)
{
    const int lane = lane_id();
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

__global__ __launch_bounds__(CSR_BLOCK) void k_softmax_fixup(SoftmaxArgs a)
{
    const int64_t base = fixup_window(a.n_chunks);
    if (base < 0) return;
    const int lane = lane_id();
    const int64_t mine = base + lane;
    const int rl = (mine < a.n_chunks) ? a.carry_row[2 * mine] : -1;
    uint64_t todo = __ballot(rl >= 0);
    while (todo) {
        const int j = __builtin_ctzll(todo);
        todo &= todo - 1;
        softmax_fixup_one(a, base + j, __shfl(rl, j, CSR_WAVE));
    }
}

// Probabilities of the entries of split rows, one wave per chunk: the chunk's
// slot A segment (the end of a row begun earlier: [y0, end of row x0)) and
// slot B segment (the start or middle of a row that continues: [start of row
// x1, y1)) are written with the lanes over consecutive entries (coalesced).
// A wave per chunk keeps every chunk's few dependent loads (slot rows, bounds,
// row statistics, scores) in flight at once across the chip.
__device__ __forceinline__ void softmax_write_segment(const SoftmaxArgs& a, int r, int sb, int se)
{
    const int lane = lane_id();
    const float m = a.stats[2 * (int64_t)r], l = a.stats[2 * (int64_t)r + 1];
    for (int e0 = sb; e0 < se; e0 += 4 * CSR_WAVE) {
        float x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e = e0 + u * CSR_WAVE + lane;
            x[u] = (e < se) ? a.scores[e] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e = e0 + u * CSR_WAVE + lane;
            if (e < se) a.probs[e] = exp_neg(x[u] * a.scale - m) / l;
        }
    }
}

__global__ __launch_bounds__(CSR_BLOCK) void k_softmax_split(SoftmaxArgs a)
{
    const int64_t c = (int64_t)blockIdx.x * CSR_WAVES_PER_BLOCK + threadIdx.x / CSR_WAVE;
    if (c >= a.n_chunks) return;
    const int ra = a.carry_row[2 * c], rb = a.carry_row[2 * c + 1];
    if (ra < 0 && rb < 0) return;
    const int y0 = a.part[2 * c + 1], y1 = a.part[2 * c + 3];
    if (ra >= 0) softmax_write_segment(a, ra, y0, min(a.row_ptr[ra + 1], y1));
    if (rb >= 0) softmax_write_segment(a, rb, max(a.row_ptr[rb], y0), y1);
}

}  // namespace csrk
