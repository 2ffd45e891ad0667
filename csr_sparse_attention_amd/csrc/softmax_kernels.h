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

// ---------------------------------------------------------------------------
// Entry-run variant (mapping "segmented scan").  Chunks are the merge-path
// chunks, re-cut at row starts: a row of at most D entries belongs wholly to
// the chunk that holds its end (its entries before the chunk's start are
// staged too, so a chunk stages fewer than 2 D entries), and only rows of more
// than D entries are cut into pieces, merged by k_softmax_fixup and written by
// k_softmax_split as before.  Lane l of a wave owns the run of R consecutive
// entries [l R, l R + R) of the chunk's range, R = ceil(entries / 64), loads
// its scores straight into registers (between them the wave's lanes read
// whole lines) and walks them alone with an online (m, l) of the row it is in;
// a row that crosses lanes is completed by one inclusive segmented scan of the
// lanes' open pieces (keyed by row), so the cross-lane work is one scan per
// chunk.  Only row_ptr and the per-row statistics go through LDS.  Every lane
// then reads the statistics of its rows and writes its p_e.
// ---------------------------------------------------------------------------
// 4 floats at a 4-byte aligned address: one 16-byte access
typedef float sm_f32x4 __attribute__((ext_vector_type(4), aligned(4)));

template <int D>
struct SmRunShared {
    // chunk row_ptr, then the rows' maxima (float bits); 64 trailing slots take
    // the lanes' writes that have no row to go to
    int32_t rp[CSR_WAVES_PER_BLOCK][D + 4 + CSR_WAVE];
    float l[CSR_WAVES_PER_BLOCK][D + 4 + CSR_WAVE];  // row-start marks (uint16), then the rows' sums
};

// (m1, l1) <- (m1, l1) merged with (m2, l2); maxima in log2 units, an empty
// piece has m = -inf and l = 0.  One of the two exponentials is exp2(0) = 1.
__device__ __forceinline__ void sm_merge2(float& m1, float& l1, float m2, float l2)
{
    const float d = m1 - m2;
    const float e = (fminf(l1, l2) > 0.f) ? __builtin_amdgcn_exp2f(-fabsf(d)) : 0.f;
    const bool first_big = d >= 0.f;
    l1 = first_big ? fmaf(l2, e, l1) : fmaf(l1, e, l2);
    m1 = first_big ? m1 : m2;
}

// largest i in [lo, hi] with rp[i] <= e, given rp[lo] <= e
__device__ __forceinline__ int sm_row_search(const int32_t* rp, int lo, int hi, int e)
{
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (rp[mid] <= e)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// BWD: the softmax backward instead, grad_scores_e = scale p_e (g_e - S_i)
// with S_i the row sum of p g; scores holds p, grad holds g, probs receives
// the result, and the per-row reduction is that plain sum (a piece is (0, S)).
template <int D, bool BWD>
__global__ __launch_bounds__(CSR_BLOCK) void k_softmax_run(SoftmaxArgs a)
{
    constexpr int RMAX = 2 * D / CSR_WAVE;
    constexpr float LOG2E = 1.44269504088896341f, LN2 = 0.693147180559945309f;
    __shared__ SmRunShared<D> sh;
    // the wave index is the same for all of a wave's lanes: in a scalar register,
    // everything derived from the chunk's coordinates is uniform too
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / CSR_WAVE), lane = lane_id();
    const int64_t chunk = (int64_t)blockIdx.x * CSR_WAVES_PER_BLOCK + wave;
    const bool active = chunk < a.n_chunks;
    int x0 = 0, y0 = 0, x1 = 0, y1 = 0, a_beg = 0, a_end = 0, b_beg = 0, b_end = 0;
    if (active) {
        x0 = a.part[2 * chunk];
        y0 = a.part[2 * chunk + 1];
        x1 = a.part[2 * chunk + 2];
        y1 = a.part[2 * chunk + 3];
        a_beg = a.bounds[2 * chunk];  // entries of row x0
        a_end = a.bounds[2 * chunk + 1];
        b_beg = a.bounds[2 * chunk + 2];  // entries of row x1
        b_end = a.bounds[2 * chunk + 3];
    }
    // row x0 ends here: whole if short, its last piece if long (begun earlier);
    // row x1 goes on past the chunk: its first or middle piece if long, left to
    // a later chunk if short
    const bool slotA = active && x0 < x1 && a_end - a_beg > D;
    const bool slotB = active && x1 < a.n_rows && b_end - b_beg > D && max(b_beg, y0) < y1;
    // (for a valid CSR lo > y0 - D and hi <= y1; the clamps keep an invalid
    // row_ptr from reading past the arrays or the LDS)
    const int lo = max((active && x0 < x1 && !slotA) ? a_beg : y0, max(0, y0 - D + 1));
    const int hi = min(min(slotB ? y1 : max(b_beg, lo), y1), lo + 2 * D - 1);
    const int ne = active ? max(0, hi - lo) : 0;
    const int nend = x1 - x0, nrow = nend + (slotB ? 1 : 0);
    int32_t* rp = sh.rp[wave];
    uint16_t* mark = reinterpret_cast<uint16_t*>(sh.l[wave]);
    // lane-owned run of R staged entries [k0, k0 + kn); R is the same for the
    // whole wave, so loops over k stop at R uniformly
    const int R = (ne + CSR_WAVE - 1) / CSR_WAVE;
    const int k0 = lane * R;
    const int kn = max(0, min(R, ne - k0));
    const float c = a.scale * LOG2E;
    float t[RMAX];
    float g[BWD ? RMAX : 1];
    // the run's scores, straight from HBM (the wave's loads cover whole lines
    // between them); read once, so non-temporal.  Four entries per access
    // where the run holds them (a lane's run is only 4-byte aligned): an
    // access costs the address unit about the same whether it moves 4 or 16
    // bytes per lane, and the lanes' runs are R entries apart.
    const float* srun = a.scores + lo + k0;
    const float* grun = BWD ? a.grad + lo + k0 : nullptr;
#pragma unroll
    for (int k = 0; k < RMAX; k += 4) {
        if (k >= R) break;
        if (k + 4 <= kn) {
            const sm_f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const sm_f32x4*>(srun + k));
            t[k] = v.x;
            t[k + 1] = v.y;
            t[k + 2] = v.z;
            t[k + 3] = v.w;
            if constexpr (BWD) {
                const sm_f32x4 w = __builtin_nontemporal_load(reinterpret_cast<const sm_f32x4*>(grun + k));
                g[k] = w.x;
                g[k + 1] = w.y;
                g[k + 2] = w.z;
                g[k + 3] = w.w;
            }
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                t[k + u] = (k + u < kn) ? __builtin_nontemporal_load(srun + k + u) : 0.f;
                if constexpr (BWD) g[k + u] = (k + u < kn) ? __builtin_nontemporal_load(grun + k + u) : 0.f;
            }
        }
    }
    if (active) {
        // row_ptr[x0 .. x0 + nrow]: nrow + 1 <= D + 2 values
        stage_chunk<(D + 2 + CSR_WAVE - 1) / CSR_WAVE, 1, false, float>(rp, a.row_ptr + x0, nrow + 1, nullptr,
                                                                       nullptr, nullptr, nullptr, 0);
        for (int j = lane; j < ne; j += CSR_WAVE) mark[j] = 0;
    }
    __syncthreads();
    // mark the first staged entry of every non-empty row after row 0 with its index + 1
    for (int i = 1 + lane; i < nrow; i += CSR_WAVE) {
        const int b = rp[i];
        if (b < rp[i + 1] && b >= lo && b < lo + ne) mark[b - lo] = (uint16_t)(i + 1);
    }
    __syncthreads();
    // rows of the run's entries and scores in log2 units
    int ri[RMAX] = {};  // zero past the run's R entries: the result loop reads (and drops) up to 3 more
    {
        int cur = (kn > 0) ? sm_row_search(rp, 0, nrow - 1, lo + k0) : 0;
#pragma unroll
        for (int k = 0; k < RMAX; ++k) {
            if (k >= R) break;
            const bool ok = k < kn;
            const int mk = ok ? mark[k0 + k] : 0;
            cur = mk ? mk - 1 : cur;
            ri[k] = cur;  // past the run: the last row again, adding nothing
            if constexpr (!BWD) t[k] = ok ? t[k] * c : -INFINITY;
        }
    }
    __syncthreads();  // rp and the marks are rewritten below
    float* sl = sh.l[wave];
    const int dummy = D + 4 + lane;  // this lane's slot for writes that go nowhere
    const int64_t slot_base = 2 * chunk;
    // the total of row i over this chunk: LDS statistics for a row completed
    // here, a carry piece (natural-log maximum) for a long row
    auto finish = [&](int i, float m, float l) {
        const float mn = BWD ? 0.f : m * LN2;
        if (i == nend && slotB) {
            a.carry_ml[2 * (slot_base + 1)] = mn;
            a.carry_ml[2 * (slot_base + 1) + 1] = l;
        } else if (i == 0 && slotA) {
            a.carry_ml[2 * slot_base] = mn;
            a.carry_ml[2 * slot_base + 1] = l;
        } else {
            rp[i] = __float_as_int(m);
            sl[i] = l;
        }
    };
    // online (max, sum) of the run's row segments; a segment closed inside the
    // run goes to LDS at its row (the first one is finished after the scan)
    const int first = (kn > 0) ? ri[0] : -1;
    int tail = (kn > 0) ? first : -2 - lane;  // row of the open piece
    float m = BWD ? 0.f : -INFINITY, l = 0.f;
#pragma unroll
    for (int k = 0; k < RMAX; ++k) {
        if (k >= R) break;
        const bool close = ri[k] != tail && kn > 0;
        const int w = close ? tail : dummy;
        rp[w] = __float_as_int(m);
        sl[w] = l;
        tail = close ? ri[k] : tail;
        if constexpr (BWD) {
            l = close ? 0.f : l;
            if (k < kn) l = fmaf(t[k], g[k], l);
        } else {
            m = close ? -INFINITY : m;
            l = close ? 0.f : l;
            const float mm = (t[k] > m) ? t[k] : m;
            l = fmaf(l, __builtin_amdgcn_exp2f(m - mm), __builtin_amdgcn_exp2f(t[k] - mm));
            m = mm;
        }
    }
    if (active && lane == 0) {
        a.carry_row[2 * chunk] = slotA ? x0 : -1;
        a.carry_row[2 * chunk + 1] = slotB ? x1 : -1;
        if (slotA && a_end == y0) {  // long row without entries here: empty piece
            a.carry_ml[2 * slot_base] = BWD ? 0.f : -INFINITY;
            a.carry_ml[2 * slot_base + 1] = 0.f;
        }
    }
    // inclusive segmented scan of the open pieces over the lanes, keyed by row
    float sm = m, sq = l;
#pragma unroll
    for (int off = 1; off < CSR_WAVE; off <<= 1) {
        const int r2 = __shfl_up(tail, off, CSR_WAVE);
        const float m2 = __shfl_up(sm, off, CSR_WAVE);
        const float l2 = __shfl_up(sq, off, CSR_WAVE);
        if (lane >= off && r2 == tail) {
            if constexpr (BWD)
                sq += l2;
            else
                sm_merge2(sm, sq, m2, l2);
        }
    }
    // what the lanes before this one hold of this run's first row
    const int prev_tail = __shfl_up(tail, 1, CSR_WAVE);
    const float cm = __shfl_up(sm, 1, CSR_WAVE), cl = __shfl_up(sq, 1, CSR_WAVE);
    const int next_first = __shfl_down(first, 1, CSR_WAVE);
    if (active && kn > 0) {
        if (tail != first) {  // the first row closed inside the run
            float fm = __int_as_float(rp[first]), fl = sl[first];
            if (lane > 0 && prev_tail == first) {
                if constexpr (BWD)
                    fl += cl;
                else
                    sm_merge2(fm, fl, cm, cl);
            }
            finish(first, fm, fl);
        }
        // the open piece is the row's total over the chunk when no later lane continues it
        if (k0 + kn >= ne || next_first != tail) finish(tail, sm, sq);
    }
    __syncthreads();
    // entries of the rows completed here: [ya, yb), run positions [ks, ke)
    const int ya = slotA ? a_end : lo;
    const int yb = slotB ? max(b_beg, y0) : hi;
    const int ks = max(0, ya - lo - k0), ke = min(kn, yb - lo - k0);
    float* prun = a.probs + lo + k0;
#pragma unroll
    for (int k = 0; k < RMAX; k += 4) {
        if (k >= R) break;
        // the run's results, four at a time (k + u may pass R: those are never stored)
        float p[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if constexpr (BWD)
                p[u] = a.scale * t[k + u] * (g[k + u] - sl[ri[k + u]]);
            else
                p[u] = __builtin_amdgcn_exp2f(t[k + u] - __int_as_float(rp[ri[k + u]])) *
                       __builtin_amdgcn_rcpf(sl[ri[k + u]]);
        }
        if (k >= ks && k + 4 <= ke) {
            *reinterpret_cast<sm_f32x4*>(prun + k) = sm_f32x4{p[0], p[1], p[2], p[3]};
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (k + u >= ks && k + u < ke) prun[k + u] = p[u];
        }
    }
}

// Merges the (m, l) pieces of rows split across chunks (one wave per chunk
// whose slot A holds a row; the pieces are slot B of the run of chunks before
// it, then slot A).
template <bool BWD>
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
    if constexpr (BWD) {
        // pieces are (0, partial sum of p g): add them
        float sum = 0.f;
        for (int64_t p = lane; p < np; p += CSR_WAVE) {
            const int64_t s = (p < np - 1) ? 2 * (k0 + p) + 1 : 2 * c;
            sum += a.carry_ml[2 * s + 1];
        }
        sum = xor_sum_from(sum, 1);
        if (lane == 0) {
            a.stats[2 * (int64_t)r] = 0.f;
            a.stats[2 * (int64_t)r + 1] = sum;
        }
        return;
    }
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

// The fix-up and the long-row pass give each wave SM_FIX_CHUNKS consecutive
// chunks (one lane reads each chunk's slots) and handle the chunks with work
// one after the other.  Each such chunk costs a few dependent loads, so the
// window is kept short: more waves share the work and their loads overlap
// (with 64 chunks a wave, a few thousand waves each walked dozens of chunks).
constexpr int SM_FIX_CHUNKS = 16;

__device__ __forceinline__ int64_t sm_fix_window()
{
    return ((int64_t)blockIdx.x * CSR_WAVES_PER_BLOCK + __builtin_amdgcn_readfirstlane(threadIdx.x / CSR_WAVE)) *
           SM_FIX_CHUNKS;
}

template <bool BWD>
__global__ __launch_bounds__(CSR_BLOCK) void k_softmax_fixup(SoftmaxArgs a)
{
    const int64_t base = sm_fix_window();
    if (base >= a.n_chunks) return;
    const int lane = lane_id();
    const int64_t mine = base + lane;
    const int rl = (lane < SM_FIX_CHUNKS && mine < a.n_chunks) ? a.carry_row[2 * mine] : -1;
    uint64_t todo = __ballot(rl >= 0);
    while (todo) {
        const int j = __builtin_ctzll(todo);
        todo &= todo - 1;
        softmax_fixup_one<BWD>(a, base + j, __shfl(rl, j, CSR_WAVE));
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

// Probabilities of the long rows' entries after the entry-run kernel: a wave
// per window of SM_FIX_CHUNKS chunks.  Lane j reads chunk base + j's slot rows, bounds
// (from the row-bound records, no row_ptr reads) and the slot rows' merged
// statistics in two rounds of independent loads; a ballot then lists the
// window's segments and the whole wave writes each one, lanes over
// consecutive entries (at most D entries, one pass of 4 loads per lane for
// D = 256).  Only chunks inside or at the ends of rows longer than D hold
// segments, so a window usually has few.
template <bool BWD>
__global__ __launch_bounds__(CSR_BLOCK) void k_softmax_split_runs(SoftmaxArgs a)
{
    const int64_t base = sm_fix_window();
    if (base >= a.n_chunks) return;
    const int lane = lane_id();
    const int64_t c = base + lane;
    int ra = -1, rb = -1, a0 = 0, a1 = 0, b0 = 0, b1 = 0;
    if (lane < SM_FIX_CHUNKS && c < a.n_chunks) {
        ra = a.carry_row[2 * c];
        rb = a.carry_row[2 * c + 1];
        const int y0 = a.part[2 * c + 1], y1 = a.part[2 * c + 3];
        a0 = y0;
        a1 = min(a.bounds[2 * c + 1], y1);            // end of row x0
        b0 = min(max(a.bounds[2 * c + 2], y0), y1);   // start of row x1
        b1 = y1;
    }
    float ma = 0.f, la = 1.f, mb = 0.f, lb = 1.f;
    if (ra >= 0) {
        ma = a.stats[2 * (int64_t)ra];
        la = a.stats[2 * (int64_t)ra + 1];
    }
    if (rb >= 0) {
        mb = a.stats[2 * (int64_t)rb];
        lb = a.stats[2 * (int64_t)rb + 1];
    }
    const float c2 = a.scale * 1.44269504088896341f;
    auto segment = [&](int sb, int se, float m, float l) {
        const float m2 = m * 1.44269504088896341f, il = BWD ? 0.f : 1.f / l;
        for (int e0 = sb; e0 < se; e0 += 4 * CSR_WAVE) {
            float x[4], y[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int e = e0 + u * CSR_WAVE + lane;
                x[u] = (e < se) ? __builtin_nontemporal_load(a.scores + e) : 0.f;
                if constexpr (BWD) y[u] = (e < se) ? __builtin_nontemporal_load(a.grad + e) : 0.f;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int e = e0 + u * CSR_WAVE + lane;
                if (e < se) {
                    if constexpr (BWD)
                        a.probs[e] = a.scale * x[u] * (y[u] - l);
                    else
                        a.probs[e] = __builtin_amdgcn_exp2f(x[u] * c2 - m2) * il;
                }
            }
        }
    };
    uint64_t todo = __ballot(ra >= 0);
    while (todo) {
        const int j = __builtin_ctzll(todo);
        todo &= todo - 1;
        segment(__shfl(a0, j, CSR_WAVE), __shfl(a1, j, CSR_WAVE), __shfl(ma, j, CSR_WAVE), __shfl(la, j, CSR_WAVE));
    }
    todo = __ballot(rb >= 0);
    while (todo) {
        const int j = __builtin_ctzll(todo);
        todo &= todo - 1;
        segment(__shfl(b0, j, CSR_WAVE), __shfl(b1, j, CSR_WAVE), __shfl(mb, j, CSR_WAVE), __shfl(lb, j, CSR_WAVE));
    }
}

}  // namespace csrk
