// Randomised check of the library's host logic (problem and schedule checks,
// lane layouts, workspace layout, candidates, cost model, format plan,
// signature, cache log format), built with g++ and the address and
// undefined-behaviour sanitizers by tests/test_host_fuzz.py.  No GPU.
//
// Invariants checked on every accepted problem: the default schedule and
// every candidate pass the schedule check; workspace sizes are aligned and
// at least the head; estimates are finite and non-negative; the signature is
// a pure function of its inputs; the plan proposes 1 part or a power of two
// from 4 to 256 with a power-of-two (or zero) whole-row threshold; a cache
// line parses back to the schedule it was written from.  Malformed cache
// lines and arbitrary problem / schedule fields must be rejected without a
// crash.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <vector>
#include <string>

#include "../csr_sparse_attention_amd/csrc/host.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next()  // splitmix64
{
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static int64_t pick(const int64_t* v, int n) { return v[next() % n]; }

static int failures = 0;
#define CHECK(cond, ...)                                   \
    do {                                                   \
        if (!(cond)) {                                     \
            if (failures < 20) std::fprintf(stderr, __VA_ARGS__); \
            ++failures;                                    \
        }                                                  \
    } while (0)

static csr_problem_t random_problem()
{
    static const int64_t sizes[] = {-1, 0, 1, 2, 7, 64, 1000, 232965, 2449029, 1000000, (int64_t)1 << 31};
    static const int64_t widths[] = {-3, 0, 1, 2, 3, 4, 5, 8, 16, 32, 64, 100, 128, 512, 602, 1024, 4096, 4097};
    csr_problem_t p;
    std::memset(&p, 0, sizeof p);
    p.op = (int32_t)(next() % 10);  // includes invalid ops 0 and 9
    p.dtype = (int32_t)(next() % 3);
    p.n_rows = pick(sizes, 11);
    p.n_cols = pick(sizes, 11);
    p.nnz = (next() % 4 == 0) ? pick(sizes, 11) : (int64_t)(next() % 200000000);
    p.width = pick(widths, 18);
    static const int32_t hd[][2] = {{8, 64}, {1, 512}, {2, 8}, {4, 32}, {3, 16}, {8, 48}, {0, 0}, {16, 64}};
    const int h = (int)(next() % 8);
    p.heads = hd[h][0];
    p.head_dim = hd[h][1];
    if (p.op == CSR_OP_MHA && next() % 2) p.width = (int64_t)p.heads * p.head_dim;
    const int64_t lds[] = {p.width, p.width + 1, p.width + 4, p.width - 1, 0};
    p.ld_a = pick(lds, 5);
    p.ld_b = pick(lds, 5);
    p.ld_out = pick(lds, 5);
    p.ld_c = pick(lds, 5);
    auto ptr = [&]() -> void* {
        static const uintptr_t bases[] = {0, 0x1000, 0x1004, 0x1008, 0x100000, 0x100010};
        return reinterpret_cast<void*>(bases[next() % 6]);
    };
    p.row_ptr = static_cast<const int32_t*>(ptr());
    p.col_idx = static_cast<const int32_t*>(ptr());
    p.a = ptr();
    p.b = ptr();
    p.c = ptr();
    p.out = ptr();
    p.probs = (next() % 3 == 0) ? static_cast<float*>(ptr()) : nullptr;
    p.probs_stride = (int64_t)(next() % 4) - 1;
    const float scales[] = {1.f, 0.125f, -2.f, 0.f, INFINITY, NAN};
    p.scale = scales[next() % 6];
    if (next() % 2) {
        // mostly well-formed: the op's dtype, positive sizes, natural strides
        // and aligned operands, with any width
        p.op = 1 + (int32_t)(next() % 8);
        const bool lane_group = p.op == CSR_OP_SPMM || p.op == CSR_OP_SDDMM || p.op == CSR_OP_ATTENTION ||
                                p.op == CSR_OP_ATTENTION_QK;  // fp32 or bf16; CSR_OP_SPMM_SDDMM: fp32
        p.dtype = (p.op == CSR_OP_MHA || (lane_group && next() % 3 == 0)) ? CSR_DTYPE_BF16 : CSR_DTYPE_F32;
        p.n_rows = 1 + (int64_t)(next() % 3000000);
        p.n_cols = 1 + (int64_t)(next() % 3000000);
        p.nnz = (int64_t)(next() % 120000000);
        if (p.op == CSR_OP_MHA) {
            static const int32_t dims[] = {8, 16, 32, 64, 128, 256, 512};
            p.heads = 1 + (int32_t)(next() % 16);
            p.head_dim = dims[next() % 7];
            p.width = (int64_t)p.heads * p.head_dim;
        } else {
            p.width = 1 + (int64_t)(next() % (p.op == CSR_OP_ATTENTION_QK ? 1024 : 4096));
            if (p.dtype == CSR_DTYPE_BF16) p.width += p.width % 2;
        }
        p.ld_a = p.ld_b = p.ld_c = p.ld_out = p.width + (int64_t)(next() % 3);
        static const uintptr_t good[] = {0x100000, 0x100004, 0x100008, 0x100010};
        p.row_ptr = reinterpret_cast<const int32_t*>(good[next() % 4]);
        p.col_idx = reinterpret_cast<const int32_t*>(good[next() % 4]);
        p.a = reinterpret_cast<const void*>(good[next() % 4]);
        p.b = reinterpret_cast<const void*>(good[next() % 4]);
        p.c = reinterpret_cast<const void*>(good[next() % 4]);
        p.out = reinterpret_cast<void*>(good[next() % 4]);
        p.probs = (p.op == CSR_OP_ATTENTION || p.op == CSR_OP_ATTENTION_QK) && next() % 2
                      ? reinterpret_cast<float*>(good[next() % 4]) : nullptr;
        p.probs_stride = 1;
        p.scale = 0.125f;
        if (p.op == CSR_OP_SPMM_SDDMM) p.out2 = reinterpret_cast<float*>(good[next() % 4]);
    }
    p.a_idx = (next() % 4 == 0) ? static_cast<const int32_t*>(ptr()) : nullptr;
    if (next() % 4 == 0) p.out2 = static_cast<float*>(ptr());
    p.out2_idx = (next() % 4 == 0) ? static_cast<const int32_t*>(ptr()) : nullptr;
    return p;
}

static void random_hist(int64_t* h, const csr_problem_t& p)
{
    std::memset(h, 0, sizeof(int64_t) * csrh::kHistInts);
    if (p.n_rows <= 0) return;
    int64_t rows_left = p.n_rows, nnz_left = p.nnz > 0 ? p.nnz : 0;
    for (int b = 0; b < 33 && rows_left > 0; ++b) {
        const int64_t c = (b == 32) ? rows_left : (int64_t)(next() % (uint64_t)(rows_left + 1));
        h[b] = c;
        rows_left -= c;
        if (b > 0 && c > 0) {
            const int64_t lo = (int64_t)1 << (b - 1);
            const int64_t s = std::min(nnz_left, c * lo);
            h[33 + b] = s;
            nnz_left -= s;
            h[66] = std::max(h[66], lo);
        }
    }
}

int main(int argc, char** argv)
{
    const int iters = argc > 1 ? std::atoi(argv[1]) : 100000;
    csrh::DeviceInfo dev;
    dev.cu_count = 256;
    dev.arch = 950;
    int accepted = 0, planned = 0, parsed = 0;
    for (int it = 0; it < iters; ++it) {
        csr_problem_t p = random_problem();
        std::string why;
        const bool need_ptrs = next() % 2;
        const int rc = csrh::check_problem(p, need_ptrs, &why);
        int64_t hist[csrh::kHistInts];
        random_hist(hist, p);
        if (rc == CSR_OK) {
            ++accepted;
            CHECK(!p.a_idx || ((p.op == CSR_OP_SPMM || p.op == CSR_OP_SPMM_SDDMM) && ((uintptr_t)p.a_idx % 4) == 0 &&
                               (!need_ptrs || p.nnz == 0 || p.a)),
                  "value index accepted for op %d\n", p.op);
            CHECK((!p.out2 && !p.out2_idx) ||
                      (p.op == CSR_OP_SPMM_SDDMM && ((uintptr_t)p.out2 % 4) == 0 && ((uintptr_t)p.out2_idx % 4) == 0),
                  "second output accepted for op %d\n", p.op);
            CHECK(p.op != CSR_OP_SPMM_SDDMM ||
                      (p.dtype == CSR_DTYPE_F32 && (!need_ptrs || p.nnz == 0 || (p.c && p.out2))),
                  "SpMM + SDDMM accepted without fp32 operands, U or z\n");
            const csr_schedule_t d = csrh::default_schedule(p);
            CHECK(csrh::check_schedule(p, d, &why) == CSR_OK, "default schedule rejected (op %d F %lld): %s\n",
                  p.op, (long long)p.width, why.c_str());
            const size_t wb = csrh::workspace_bytes(p, d);
            CHECK(wb >= csrh::kHeadBytes && wb % csrh::kAlign == 0, "bad workspace size %zu\n", wb);
            const auto cands = csrh::candidates(p, (next() % 2) ? hist : nullptr);
            CHECK(!cands.empty() && std::memcmp(&cands[0], &d, sizeof d) == 0, "first candidate is not the default\n");
            for (const auto& c : cands) {
                CHECK(csrh::check_schedule(p, c, &why) == CSR_OK, "candidate rejected (op %d map %d): %s\n", p.op,
                      c.mapping, why.c_str());
                const double e = csrh::estimate(p, c, hist, dev);
                CHECK(std::isfinite(e) && e >= 0.0, "estimate %g\n", e);
                const size_t w = csrh::workspace_bytes(p, c);
                CHECK(w >= csrh::kHeadBytes && w % csrh::kAlign == 0, "bad candidate workspace %zu\n", w);
            }
            {  // the probe subset: at most k distinct candidates, ascending, the best estimate among them,
               // and one of each mapping when k allows
                std::vector<double> est;
                for (const auto& c : cands) est.push_back(csrh::estimate(p, c, hist, dev));
                const int k = 1 + (int)(next() % 8);
                const std::vector<size_t> sub = csrh::probe_subset(cands, est, k);
                size_t best = 0;
                for (size_t i = 1; i < est.size(); ++i)
                    if (est[i] < est[best]) best = i;
                bool ok = (int)sub.size() == std::min<int>(k, (int)cands.size()), has_best = false;
                for (size_t i = 0; i < sub.size(); ++i) {
                    ok = ok && sub[i] < cands.size() && (i == 0 || sub[i] > sub[i - 1]);
                    has_best = has_best || est[sub[i]] == est[best];
                }
                std::vector<std::pair<int, int>> kinds, got;
                for (const auto& c : cands)
                    if (std::find(kinds.begin(), kinds.end(), std::make_pair(c.mapping, c.flags)) == kinds.end())
                        kinds.push_back({c.mapping, c.flags});
                for (size_t i : sub)
                    if (std::find(got.begin(), got.end(), std::make_pair(cands[i].mapping, cands[i].flags)) == got.end())
                        got.push_back({cands[i].mapping, cands[i].flags});
                const bool diverse = (int)got.size() >= std::min<int>(k, (int)kinds.size());
                CHECK(ok && has_best && diverse, "probe subset k %d of %zu: size %zu best %d diverse %d\n", k,
                      cands.size(), sub.size(), (int)has_best, (int)diverse);
            }
            const uint64_t s1 = csrh::signature(p, hist, dev), s2 = csrh::signature(p, hist, dev);
            CHECK(s1 == s2, "signature not deterministic\n");
            int P = -1, T = -1;
            csrh::hybrid_plan(p, (next() % 2) ? hist : nullptr, &P, &T);
            const bool p_ok = P == 1 || (P >= 4 && P <= 256 && (P & (P - 1)) == 0);
            const bool t_ok = T == 0 || (T > 0 && (T & (T - 1)) == 0);
            CHECK(p_ok && t_ok && (P > 1 || T == 0), "plan P %d T %d\n", P, T);
            if (P > 1) ++planned;
            // the cache line round trip
            const double us = (double)(next() % 100000) / 7.0;
            const std::string line = csrh::format_cache_line(s1, d, us);
            uint64_t sig = 0;
            csr_schedule_t back;
            double us2 = 0;
            CHECK(csrh::parse_cache_line(line, &sig, &back, &us2) && sig == s1 && std::memcmp(&back, &d, sizeof d) == 0,
                  "cache line round trip: %s\n", line.c_str());
            // truncated and corrupted lines are rejected or parse to a valid schedule, never crash
            std::string bad = line.substr(0, next() % (line.size() + 1));
            if (!bad.empty() && next() % 2) bad[next() % bad.size()] = (char)(32 + next() % 95);
            if (csrh::parse_cache_line(bad, &sig, &back, &us2)) ++parsed;
        }
        // arbitrary schedule fields: checked without a crash
        csr_schedule_t s;
        std::memset(&s, 0, sizeof s);
        s.version = (int32_t)(next() % 3);
        s.op = (int32_t)(next() % 10);
        s.mapping = (int32_t)(next() % 5);
        s.vec = (int32_t)(next() % 10);
        s.group_lanes = (int32_t)(1 << (next() % 8)) - (int32_t)(next() % 2);
        s.passes = (int32_t)(next() % 20);
        s.chunk_items = (int32_t)((next() % 2) ? 256 << (next() % 4) : next() % 5000);
        s.long_row = (int32_t)(next() % 300) - 10;
        s.flags = (int32_t)(next() % 8 == 0 ? 1 + next() % 3 : 0);
        if (rc == CSR_OK && csrh::check_schedule(p, s, &why) == CSR_OK) {
            const size_t w = csrh::workspace_bytes(p, s);
            CHECK(w >= csrh::kHeadBytes && w % csrh::kAlign == 0, "bad workspace for an accepted schedule\n");
        }
    }
    // the plan memory bound on the format's segment count: a random pattern,
    // its degree histogram, the segments the construction makes (one per
    // nonempty row kept whole, else one per distinct (row, column part)),
    // never above segment_bound
    int64_t seg_checks = 0;
    for (int it = 0; it < iters / 50; ++it) {
        const int64_t n_rows = 1 + (int64_t)(next() % 300), n_cols = 1 + (int64_t)(next() % 5000);
        std::vector<int64_t> deg(n_rows);
        int64_t nnz = 0;
        for (auto& d : deg) {
            const int kind = (int)(next() % 4);
            d = kind == 0 ? 0 : (kind == 1 ? (int64_t)(next() % 8) : (int64_t)(next() % (uint64_t)(n_cols + 1)));
            nnz += d;
        }
        int64_t h[csrh::kHistInts] = {0};
        for (int64_t d : deg) {
            int b = 0;
            while (b < 32 && ((int64_t)1 << b) <= d) ++b;  // d in [2^(b-1), 2^b)
            h[b] += 1;
            h[33 + b] += d;
            h[66] = std::max(h[66], d);
        }
        csr_problem_t p;
        std::memset(&p, 0, sizeof p);
        p.op = CSR_OP_SPMM;
        p.n_rows = n_rows;
        p.n_cols = n_cols;
        p.nnz = nnz;
        p.width = 1;
        const int P = 2 << (next() % 8);
        const int T = (next() % 3 == 0) ? 0 : 1 << (next() % 12);
        const int64_t part_cols = (n_cols + P - 1) / P;
        int64_t segs = 0;
        std::vector<char> seen(P);
        for (int64_t r = 0; r < n_rows; ++r) {
            if (deg[r] == 0) continue;
            if (deg[r] < T) {
                ++segs;
                continue;
            }
            std::fill(seen.begin(), seen.end(), 0);
            for (int64_t k = 0; k < deg[r]; ++k) {
                const int64_t part = std::min<int64_t>((int64_t)(next() % (uint64_t)n_cols) / part_cols, P - 1);
                if (!seen[part]) {
                    seen[part] = 1;
                    ++segs;
                }
            }
        }
        const int64_t bound = csrh::segment_bound(p, h, P, T), loose = csrh::segment_bound(p, nullptr, P, T);
        CHECK(segs <= bound && bound <= loose, "segments %lld above the bound %lld (loose %lld) P %d T %d\n",
              (long long)segs, (long long)bound, (long long)loose, P, T);
        ++seg_checks;
    }
    // plan log lines (plain, format, degree classes) round trip; the degree
    // classes' shape agrees with a row-by-row count of a random pattern
    int64_t bucket_checks = 0;
    for (int it = 0; it < iters / 50; ++it) {
        csrh::PlanChoice c;
        const int kind = (int)(next() % 3);
        c.parts = kind == 0 ? 1 : (kind == 1 ? 2 << (next() % 7) : 0);
        c.whole_below = kind == 2 ? 2 << (next() % 6) : (int)(next() % 3) * 64;
        c.sched = csrh::default_schedule([] {
            csr_problem_t q;
            std::memset(&q, 0, sizeof q);
            q.op = CSR_OP_SPMM;
            q.width = 32;
            q.ld_b = q.ld_out = 32;
            q.b = q.out = reinterpret_cast<void*>(0x1000);
            return q;
        }());
        const uint64_t sg = next();
        const std::string line = csrh::format_plan_line(sg, c, 12.5);
        uint64_t sg2 = 0;
        csrh::PlanChoice c2;
        double us = 0;
        CHECK(csrh::parse_plan_line(line, &sg2, &c2, &us) && sg2 == sg && c2.parts == c.parts &&
                  c2.whole_below == c.whole_below && std::memcmp(&c2.sched, &c.sched, sizeof c.sched) == 0,
              "plan line round trip: %s", line.c_str());
        // a degree-class line for SDDMM or with a threshold that is no power of two is refused
        csrh::PlanChoice bad = c;
        bad.parts = 0;
        bad.whole_below = 3 + 2 * (int)(next() % 10);
        CHECK(!csrh::parse_plan_line(csrh::format_plan_line(sg, bad, 1.0), &sg2, &c2, &us), "bad class line parsed\n");

        const int64_t n_rows = 1 + (int64_t)(next() % 400);
        std::vector<int64_t> deg(n_rows);
        int64_t nnz = 0;
        int64_t h[csrh::kHistInts] = {0};
        for (auto& d : deg) {
            d = (next() % 3 == 0) ? (int64_t)(next() % 200) : (int64_t)(next() % 9);
            nnz += d;
            int b = 0;
            while (b < 32 && ((int64_t)1 << b) <= d) ++b;
            h[b] += 1;
            h[33 + b] += d;
            h[66] = std::max(h[66], d);
        }
        csr_problem_t p;
        std::memset(&p, 0, sizeof p);
        p.op = CSR_OP_SPMM;
        p.n_rows = n_rows;
        p.n_cols = 1000;
        p.nnz = nnz;
        p.width = 4;
        const int E = 2 << (next() % 6);
        const csrh::BucketShape sh = csrh::bucket_shape(p, h, E);
        int64_t n_short = 0, slots = 0, nnz_long = 0, per_class[CSR_BUCKET_MAX_CLASSES] = {0};
        for (int64_t d : deg) {
            if (d >= 1 && d < E) {
                int c = 0;
                while (((int64_t)2 << c) <= d) ++c;  // 2^c <= d < 2^(c+1)
                ++per_class[c];
                ++n_short;
                slots += ((int64_t)2 << c) - 1;
            } else {
                nnz_long += d;
            }
        }
        bool same = sh.n_short == n_short && sh.n_slots == slots && sh.nnz_long == nnz_long &&
                    sh.nnz_short + sh.nnz_long == nnz && (1 << sh.n_classes) == E;
        int64_t row0 = 0, base = 0;
        for (int c = 0; c < sh.n_classes; ++c) {
            same = same && sh.class_rows[c] == per_class[c] && sh.class_row0[c] == row0 && sh.class_base[c] == base;
            row0 += per_class[c];
            base += per_class[c] * (((int64_t)2 << c) - 1);
        }
        const csrh::BucketLayout L = csrh::bucket_layout(p, sh);
        same = same && L.total >= (size_t)(n_rows * 4 + 3 * slots * 4 + (n_rows + 1) * 4 + 3 * nnz_long * 4) &&
               L.slot_col % 256 == 0 && L.long_val % 256 == 0;
        CHECK(same, "degree classes E %d: n_short %lld/%lld slots %lld/%lld nnz_long %lld/%lld\n", E,
              (long long)sh.n_short, (long long)n_short, (long long)sh.n_slots, (long long)slots,
              (long long)sh.nnz_long, (long long)nnz_long);
        for (int e2 : csrh::plan_buckets(p, h))
            CHECK(e2 == 8 || e2 == 32, "plan_buckets offered %d\n", e2);
        ++bucket_checks;
    }
    std::printf("degree-class checks %lld\n", (long long)bucket_checks);
    std::printf("iterations %d accepted problems %d planned formats %d corrupted lines parsed %d segment bounds %lld "
                "failures %d\n", iters, accepted, planned, parsed, (long long)seg_checks, failures);
    return failures ? 1 : 0;
}
