// C ABI of the library (declared in include/csrsa.h): contexts, argument
// checks, schedule execution, the auto-select path (degree histogram,
// signature, cache, cost model, micro-probes, guarded fallback) and the
// persistent cache log.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <fstream>
#include <functional>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/csrsa.h"
#include "host.h"
#include "launch.h"

struct CacheEntry {
    csr_schedule_t sched;
    double probe_us;
    bool persisted;
};

struct PlanEntry {
    csrh::PlanChoice choice;
    double probe_us;
    bool persisted;
};

struct csr_context_s {
    std::mutex mu;
    int device = -1;  // -1: host-only context (cache and host logic only)
    csrh::DeviceInfo dev;
    uint32_t flags = 0;
    std::string cache_path;
    std::map<uint64_t, CacheEntry> cache;
    std::map<uint64_t, PlanEntry> plans;  // planned products: layout and schedule chosen together
    int64_t skipped_lines = 0;
    int64_t io_errors = 0;
    int64_t* pinned = nullptr;  // 4 KiB pinned host buffer
    hipEvent_t ev0 = nullptr, ev1 = nullptr;
    std::string last_error;
    void* scratch = nullptr;        // this device's copy of the allocation-free scratch array
    hipError_t scratch_err = hipSuccess;
};

// Scratch memory of the allocation-free entry point (csr_spmm_noalloc): a
// file-scope device array, one copy per GPU, held until the process ends.
// Host code never uses the name itself (on the host it is only a stand-in,
// not a device address): the address of each device's copy comes from
// hipGetSymbolAddress, once per device, and is what kernels receive.
static __device__ __align__(256) unsigned char scratch[CSR_NOALLOC_SCRATCH_BYTES];

namespace {

// Address of each device's copy of `scratch`, looked up once per device with
// that device current.
std::mutex g_scratch_mu;
void* g_scratch_ptr[256] = {};

hipError_t scratch_address(int device, void** out)
{
    if (device < 0 || device >= 256) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[device]) {
        void* ptr = nullptr;
        hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));  // the current device is `device`
        if (e != hipSuccess) return e;
        if (!ptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[device] = ptr;
    }
    *out = g_scratch_ptr[device];
    return hipSuccess;
}

struct DeviceGuard {
    int prev = -1;
    bool changed = false;
    explicit DeviceGuard(int dev)
    {
        if (dev < 0) return;
        if (hipGetDevice(&prev) == hipSuccess && prev != dev) {
            changed = hipSetDevice(dev) == hipSuccess;
        }
    }
    ~DeviceGuard()
    {
        if (changed) (void)hipSetDevice(prev);
    }
};

// The context's lock for the whole of a call that may record an error (none
// for a NULL context): the checks, the error message and the work of one call
// are serialised with the other calls on the context.
struct CtxLock {
    std::unique_lock<std::mutex> lk;
    explicit CtxLock(csr_context_t ctx)
    {
        if (ctx) lk = std::unique_lock<std::mutex>(ctx->mu);
    }
};

int set_err(csr_context_t ctx, int code, const std::string& msg)
{
    if (ctx) ctx->last_error = msg;
    return code;
}

int hip_err(csr_context_t ctx, hipError_t e, const char* what)
{
    return set_err(ctx, CSR_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

#define CSR_HIP(ctx, call)                                   \
    do {                                                     \
        hipError_t e_ = (call);                              \
        if (e_ != hipSuccess) return hip_err(ctx, e_, #call); \
    } while (0)

// Appends one line; if the log ends in a partial line (an interrupted
// writer), a newline is written first so that the new line stays intact.
bool append_line(const std::string& path, const std::string& line)
{
    bool need_nl = false;
    if (FILE* r = std::fopen(path.c_str(), "rb")) {
        if (std::fseek(r, -1, SEEK_END) == 0) need_nl = std::fgetc(r) != '\n';
        std::fclose(r);
    }
    FILE* f = std::fopen(path.c_str(), "a");
    if (!f) return false;
    bool ok = true;
    if (need_nl) ok = std::fputc('\n', f) != EOF;
    ok = ok && std::fwrite(line.data(), 1, line.size(), f) == line.size();
    return (std::fclose(f) == 0) && ok;
}

void load_cache(csr_context_t ctx)
{
    std::ifstream in(ctx->cache_path);
    if (!in) return;  // a missing log is an empty cache
    std::string line;
    while (std::getline(in, line)) {
        if (line.empty() || line[0] == '#') continue;
        uint64_t sig;
        csr_schedule_t s;
        csrh::PlanChoice c;
        double us;
        if (csrh::parse_cache_line(line, &sig, &s, &us)) {
            ctx->cache[sig] = CacheEntry{s, us, true};  // a later line for a signature replaces an earlier one
        } else if (csrh::parse_plan_line(line, &sig, &c, &us)) {
            ctx->plans[sig] = PlanEntry{c, us, true};
        } else {
            ++ctx->skipped_lines;
        }
    }
}

int store_entry(csr_context_t ctx, uint64_t sig, const csr_schedule_t& s, double us)
{
    ctx->cache[sig] = CacheEntry{s, us, false};
    if (ctx->cache_path.empty()) {
        ctx->cache[sig].persisted = true;
        return CSR_OK;
    }
    if (append_line(ctx->cache_path, csrh::format_cache_line(sig, s, us))) {
        ctx->cache[sig].persisted = true;
        return CSR_OK;
    }
    ++ctx->io_errors;
    return set_err(ctx, CSR_ERR_CACHE_IO, "cannot append to the cache log " + ctx->cache_path);
}

int store_plan(csr_context_t ctx, uint64_t sig, const csrh::PlanChoice& c, double us)
{
    ctx->plans[sig] = PlanEntry{c, us, false};
    if (ctx->cache_path.empty()) {
        ctx->plans[sig].persisted = true;
        return CSR_OK;
    }
    if (append_line(ctx->cache_path, csrh::format_plan_line(sig, c, us))) {
        ctx->plans[sig].persisted = true;
        return CSR_OK;
    }
    ++ctx->io_errors;
    return set_err(ctx, CSR_ERR_CACHE_IO, "cannot append to the cache log " + ctx->cache_path);
}

bool env_flag(const char* name)
{
    const char* v = std::getenv(name);
    return v && *v && std::strcmp(v, "0") != 0;
}

int env_int(const char* name, int dflt)
{
    const char* v = std::getenv(name);
    if (!v || !*v) return dflt;
    return std::atoi(v);
}

// ---------------------------------------------------------------------------
// Execution of one schedule
// ---------------------------------------------------------------------------

// Index maps of an SDDMM over the column-part segment format (see csrk::Fp32Args)
struct RowMaps {
    const int32_t* u_row;
    const int32_t* out_idx;
    int32_t stream_y;  // SpMM: output rows stored non-temporally (the format's partial rows)
};

int run_schedule(csr_context_t ctx, const csr_problem_t& p, const csr_schedule_t& s, hipStream_t st,
                 const RowMaps* maps = nullptr)
{
    char* ws = static_cast<char*>(p.workspace);
    if (ctx->flags & CSR_CTX_VALIDATE) {
        int64_t* bad = reinterpret_cast<int64_t*>(ws);
        // the row softmax and its backward have no columns (col_idx is not read)
        const bool rows_only = p.op == CSR_OP_ROW_SOFTMAX || p.op == CSR_OP_SOFTMAX_BWD;
        CSR_HIP(ctx, csrk::launch_validate(p.row_ptr, rows_only ? nullptr : p.col_idx, p.n_rows, p.n_cols, p.nnz, bad,
                                           st));
        if (p.a_idx) CSR_HIP(ctx, csrk::launch_validate_index(p.a_idx, p.nnz, p.nnz, bad, st));
        if (p.out2_idx) CSR_HIP(ctx, csrk::launch_validate_index(p.out2_idx, p.nnz, p.nnz, bad, st));
        CSR_HIP(ctx, hipMemcpyAsync(ctx->pinned, bad, sizeof(int64_t), hipMemcpyDeviceToHost, st));
        CSR_HIP(ctx, hipStreamSynchronize(st));
        if (ctx->pinned[0] != 0)
            return set_err(ctx, CSR_ERR_INVALID_CSR, (p.a_idx || p.out2_idx)
                                                         ? "row_ptr / col_idx / the entry indexes fail CSR validation"
                                                         : "row_ptr / col_idx fail CSR validation");
    }
    if (p.n_rows == 0) return CSR_OK;
    if (p.op == CSR_OP_SDDMM && p.nnz == 0) return CSR_OK;

    const csrh::WsLayout L = csrh::ws_layout(p, s);
    int32_t* coords = reinterpret_cast<int32_t*>(ws + L.coords);
    if (s.mapping != CSR_MAP_ROWGROUP) {
        int32_t* bounds = L.bounds ? reinterpret_cast<int32_t*>(ws + L.bounds) : nullptr;
        CSR_HIP(ctx, csrk::launch_merge_path(p.row_ptr, p.n_rows, p.nnz, s.chunk_items, L.n_chunks, coords, st, bounds));
    }

    if (p.op == CSR_OP_ROW_SOFTMAX || p.op == CSR_OP_SOFTMAX_BWD) {
        if (p.nnz == 0) return CSR_OK;
        csrk::SoftmaxArgs a{};
        a.row_ptr = p.row_ptr;
        a.n_rows = p.n_rows;
        a.scores = static_cast<const float*>(p.a);
        a.grad = static_cast<const float*>(p.b);
        a.scale = p.scale;
        a.probs = static_cast<float*>(p.out);
        a.W = s.group_lanes;
        a.long_row = (s.group_lanes == 64) ? 0 : s.long_row;
        a.part = coords;
        a.bounds = L.bounds ? reinterpret_cast<const int32_t*>(ws + L.bounds) : nullptr;
        a.n_chunks = L.n_chunks;
        a.carry_row = reinterpret_cast<int32_t*>(ws + L.carry_row);
        a.carry_ml = reinterpret_cast<float*>(ws + L.carry_ml);
        a.stats = reinterpret_cast<float*>(ws + L.carry_val);
        if (p.op == CSR_OP_SOFTMAX_BWD)
            CSR_HIP(ctx, csrk::launch_row_softmax_backward(s.chunk_items, a, st));
        else
            CSR_HIP(ctx, csrk::launch_row_softmax(s.mapping, s.chunk_items, a, st));
        return CSR_OK;
    }
    if (p.op == CSR_OP_MHA) {
        csrk::MhaArgs a{};
        a.row_ptr = p.row_ptr;
        a.col_idx = p.col_idx;
        a.n_rows = p.n_rows;
        a.Q = static_cast<const uint16_t*>(p.a);
        a.K = static_cast<const uint16_t*>(p.b);
        a.V = static_cast<const uint16_t*>(p.c);
        a.H = p.heads;
        a.Dh = p.head_dim;
        a.scale = p.scale;
        a.out = static_cast<float*>(p.out);
        a.part = coords;
        a.n_chunks = L.n_chunks;
        a.carry_row = reinterpret_cast<int32_t*>(ws + L.carry_row);
        a.carry_ml = reinterpret_cast<float*>(ws + L.carry_ml);
        a.carry_val = reinterpret_cast<float*>(ws + L.carry_val);
        a.probs = p.probs;
        const int lph = p.head_dim / 8;
        CSR_HIP(ctx, csrk::launch_mha(s.mapping, lph, s.chunk_items, a, st));
        if (s.mapping != CSR_MAP_ROWGROUP) CSR_HIP(ctx, csrk::launch_mha_fixup(lph, a, st));
        return CSR_OK;
    }

    csrk::Fp32Args a{};
    a.row_ptr = p.row_ptr;
    a.col_idx = p.col_idx;
    a.n_rows = p.n_rows;
    a.F = (int32_t)p.width;
    a.W = s.group_lanes;
    a.scale = p.scale;
    a.long_row = s.long_row;
    a.part = coords;
    a.n_chunks = L.n_chunks;
    a.carry_row = reinterpret_cast<int32_t*>(ws + L.carry_row);
    a.carry_ml = reinterpret_cast<float*>(ws + L.carry_ml);
    a.carry_val = reinterpret_cast<float*>(ws + L.carry_val);
    a.stream_y = maps ? maps->stream_y : 0;
    const bool bf = p.dtype == CSR_DTYPE_BF16;
    if (p.op == CSR_OP_ATTENTION_QK) {
        a.U = p.a;
        a.ldu = p.ld_a;
        a.X = p.b;
        a.ldx = p.ld_b;
        a.V = p.c;
        a.ldv = p.ld_c;
        a.Y = static_cast<float*>(p.out);
        a.ldy = p.ld_out;
        a.probs = p.probs;
        a.probs_stride = p.probs_stride > 0 ? p.probs_stride : 1;
    }
    if (p.op == CSR_OP_SPMM_SDDMM) {
        a.ev = static_cast<const float*>(p.a);
        a.ev_idx = p.a_idx;
        a.X = p.b;
        a.ldx = p.ld_b;
        a.U = p.c;
        a.ldu = p.ld_c;
        a.Y = static_cast<float*>(p.out);
        a.ldy = p.ld_out;
        a.Z = p.out2;
        a.out_idx = p.out2_idx;
        CSR_HIP(ctx, csrk::launch_dual(s.mapping, s.vec, s.passes, s.chunk_items, a, st));
        // split rows: the SpMM's fix-up (the same carry layout)
        if (s.mapping != CSR_MAP_ROWGROUP) CSR_HIP(ctx, csrk::launch_spmm_fixup(s.vec, s.passes, a, st));
        return CSR_OK;
    }
    if (p.op == CSR_OP_SDDMM) {
        if (maps) {
            a.u_row = maps->u_row;
            a.out_idx = maps->out_idx;
        }
        a.U = p.a;
        a.ldu = p.ld_a;
        a.X = p.b;
        a.ldx = p.ld_b;
        a.Y = static_cast<float*>(p.out);
        CSR_HIP(ctx, bf ? csrk::launch_sddmm_bf16(s.mapping, s.vec, s.passes, s.chunk_items, a, st)
                        : csrk::launch_sddmm(s.mapping, s.vec, s.passes, s.chunk_items, a, st));
        return CSR_OK;
    }
    if (p.op != CSR_OP_ATTENTION_QK) {
        a.ev = static_cast<const float*>(p.a);
        if (p.op == CSR_OP_SPMM) a.ev_idx = p.a_idx;
        a.X = p.b;
        a.ldx = p.ld_b;
        a.Y = static_cast<float*>(p.out);
        a.ldy = p.ld_out;
        a.probs = p.probs;
        a.probs_stride = p.probs_stride > 0 ? p.probs_stride : 1;
    }
    // the fix-up reads fp32 pieces and writes fp32 rows: over bf16 operands it
    // takes the widest fp32 lane layout the width and the output allow
    csrk::Fp32Args fa = a;
    int fvec = s.vec, fnv = s.passes;
    if (bf && s.mapping != CSR_MAP_ROWGROUP) {
        fvec = 4;
        while (fvec > 1 && (p.width % fvec || p.ld_out % fvec || (uintptr_t)p.out % (4 * fvec))) fvec /= 2;
        int W = 0;
        if (!csrh::natural_layout(p.width, fvec, &W, &fnv))
            return set_err(ctx, CSR_ERR_SHAPE, "no fp32 layout for the fix-up of this width");
        fa.W = W;
    }
    if (p.op == CSR_OP_SPMM && (s.flags & CSR_SCHED_WIDE)) {
        CSR_HIP(ctx, csrk::launch_spmm_wide(s.passes, a, st));
    } else if (p.op == CSR_OP_SPMM) {
        CSR_HIP(ctx, bf ? csrk::launch_spmm_bf16(s.mapping, s.vec, s.passes, s.chunk_items, a, st)
                        : csrk::launch_spmm(s.mapping, s.vec, s.passes, s.chunk_items, a, st));
        if (s.mapping != CSR_MAP_ROWGROUP) CSR_HIP(ctx, csrk::launch_spmm_fixup(fvec, fnv, fa, st));
    } else if (p.op == CSR_OP_ATTENTION_QK) {
        CSR_HIP(ctx, bf ? csrk::launch_attention_qk_bf16(s.mapping, s.vec, s.passes, s.chunk_items, a, st)
                        : csrk::launch_attention_qk(s.mapping, s.vec, s.passes, s.chunk_items, a, st));
        if (s.mapping != CSR_MAP_ROWGROUP) CSR_HIP(ctx, csrk::launch_attention_qk_fixup(fvec, fnv, fa, st));
    } else {
        CSR_HIP(ctx, bf ? csrk::launch_attention_bf16(s.mapping, s.vec, s.passes, s.chunk_items, a, st)
                        : csrk::launch_attention(s.mapping, s.vec, s.passes, s.chunk_items, a, st));
        if (s.mapping != CSR_MAP_ROWGROUP) CSR_HIP(ctx, csrk::launch_attention_fixup(fvec, fnv, fa, st));
    }
    return CSR_OK;
}

size_t auto_workspace(const csr_problem_t& p)
{
    size_t need = csrh::kHeadBytes;
    for (const auto& c : csrh::candidates(p, nullptr)) need = std::max(need, csrh::workspace_bytes(p, c));
    csr_schedule_t rg = csrh::default_schedule(p);
    rg.mapping = CSR_MAP_ROWGROUP;
    rg.chunk_items = rg.long_row = 0;
    return std::max(need, csrh::workspace_bytes(p, rg));
}

int check_workspace(csr_context_t ctx, const csr_problem_t& p, size_t need)
{
    if (need > 0 && !p.workspace) return set_err(ctx, CSR_ERR_WORKSPACE, "workspace is NULL");
    if ((uintptr_t)p.workspace % csrh::kAlign) return set_err(ctx, CSR_ERR_ALIGN, "workspace must be 256-byte aligned");
    if (p.workspace_bytes < need)
        return set_err(ctx, CSR_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need) + " bytes");
    return CSR_OK;
}

int histogram(csr_context_t ctx, const csr_problem_t& p, hipStream_t st, int64_t* out)
{
    int64_t* dev = static_cast<int64_t*>(p.workspace);
    CSR_HIP(ctx, csrk::launch_degree_hist(p.row_ptr, p.n_rows, dev, st));
    CSR_HIP(ctx, hipMemcpyAsync(ctx->pinned, dev, csrh::kHistInts * sizeof(int64_t), hipMemcpyDeviceToHost, st));
    CSR_HIP(ctx, hipStreamSynchronize(st));
    std::memcpy(out, ctx->pinned, csrh::kHistInts * sizeof(int64_t));
    return CSR_OK;
}

// One timed run of schedule s on p (milliseconds), or a negative value if it failed.
double timed_run(csr_context_t ctx, const csr_problem_t& p, const csr_schedule_t& s, hipStream_t st,
                 const RowMaps* maps)
{
    if (env_flag("CSRSA_FAIL_PROBE")) return -1.0;
    if (!ctx->ev0) {
        if (hipEventCreate(&ctx->ev0) != hipSuccess || hipEventCreate(&ctx->ev1) != hipSuccess) return -1.0;
    }
    if (hipEventRecord(ctx->ev0, st) != hipSuccess) return -1.0;
    if (run_schedule(ctx, p, s, st, maps) != CSR_OK) return -1.0;
    if (hipEventRecord(ctx->ev1, st) != hipSuccess) return -1.0;
    if (hipEventSynchronize(ctx->ev1) != hipSuccess) return -1.0;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, ctx->ev0, ctx->ev1) != hipSuccess) return -1.0;
    return ms;
}

// Micro-probes: median run time (ms) of every candidate, or a negative
// value for a candidate that failed.  The GPU is first warmed up on the
// first candidate (clocks ramp up from idle), then the candidates are timed
// in interleaved rounds so that slow drifts (clocks, temperature) bias none
// of them; the number of runs per round adapts to the kernel's duration.
// One timed run of run() (milliseconds), or a negative value if it failed.
double timed_fn(csr_context_t ctx, const std::function<int()>& run, hipStream_t st)
{
    if (env_flag("CSRSA_FAIL_PROBE")) return -1.0;
    if (!ctx->ev0) {
        if (hipEventCreate(&ctx->ev0) != hipSuccess || hipEventCreate(&ctx->ev1) != hipSuccess) return -1.0;
    }
    if (hipEventRecord(ctx->ev0, st) != hipSuccess) return -1.0;
    if (run() != CSR_OK) return -1.0;
    if (hipEventRecord(ctx->ev1, st) != hipSuccess) return -1.0;
    if (hipEventSynchronize(ctx->ev1) != hipSuccess) return -1.0;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, ctx->ev0, ctx->ev1) != hipSuccess) return -1.0;
    return ms;
}

// Micro-probes of n alternatives run(0) .. run(n - 1), as probe_all does for
// schedules: warm-up on the first, one untimed run each, then interleaved
// timed rounds; the median per alternative, negative for one that failed.
std::vector<double> probe_runs(csr_context_t ctx, size_t n, const std::function<int(size_t)>& run, hipStream_t st)
{
    std::vector<double> med(n, -1.0);
    if (n == 0) return med;
    std::vector<std::vector<double>> t(n);
    std::vector<bool> failed(n, false);
    double warm = 0.0, last = -1.0;
    for (int k = 0; k < 20 && warm < 20.0; ++k) {
        last = timed_fn(ctx, [&] { return run(0); }, st);
        if (last < 0) break;
        warm += last;
    }
    const int reps = std::max(1, env_int("CSRSA_PROBE_REPS", 0));
    const int per_round = env_int("CSRSA_PROBE_REPS", 0) > 0 ? 1
                          : (last > 0 ? std::max(1, std::min(3, (int)(10.0 / last))) : 1);
    const int rounds = env_int("CSRSA_PROBE_REPS", 0) > 0 ? reps : 3;
    for (size_t i = 0; i < n; ++i)
        if (timed_fn(ctx, [&] { return run(i); }, st) < 0) failed[i] = true;
    for (int r = 0; r < rounds; ++r) {
        for (size_t i = 0; i < n; ++i) {
            if (failed[i]) continue;
            for (int k = 0; k < per_round; ++k) {
                const double ms = timed_fn(ctx, [&] { return run(i); }, st);
                if (ms < 0) {
                    failed[i] = true;
                    break;
                }
                t[i].push_back(ms);
            }
        }
    }
    for (size_t i = 0; i < n; ++i) {
        if (failed[i] || t[i].empty()) continue;
        std::sort(t[i].begin(), t[i].end());
        med[i] = t[i][t[i].size() / 2];
    }
    return med;
}

std::vector<double> probe_all(csr_context_t ctx, const csr_problem_t& p, const std::vector<csr_schedule_t>& cand,
                              const std::vector<size_t>& which, hipStream_t st, const RowMaps* maps)
{
    std::vector<double> med(cand.size(), -1.0);
    std::vector<std::vector<double>> t(cand.size());
    std::vector<bool> failed(cand.size(), false);
    double warm = 0.0, last = -1.0;
    for (int k = 0; k < 20 && warm < 20.0; ++k) {
        last = timed_run(ctx, p, cand[which[0]], st, maps);
        if (last < 0) break;
        warm += last;
    }
    const int reps = std::max(1, env_int("CSRSA_PROBE_REPS", 0));
    const int per_round = env_int("CSRSA_PROBE_REPS", 0) > 0 ? 1
                          : (last > 0 ? std::max(1, std::min(3, (int)(10.0 / last))) : 1);
    const int rounds = env_int("CSRSA_PROBE_REPS", 0) > 0 ? reps : 3;
    for (size_t i : which) {  // one untimed run each (code loading, caches)
        if (timed_run(ctx, p, cand[i], st, maps) < 0) failed[i] = true;
    }
    for (int r = 0; r < rounds; ++r) {
        for (size_t i : which) {
            if (failed[i]) continue;
            for (int k = 0; k < per_round; ++k) {
                const double ms = timed_run(ctx, p, cand[i], st, maps);
                if (ms < 0) {
                    failed[i] = true;
                    break;
                }
                t[i].push_back(ms);
            }
        }
    }
    for (size_t i : which) {
        if (failed[i] || t[i].empty()) continue;
        std::sort(t[i].begin(), t[i].end());
        med[i] = t[i][t[i].size() / 2];
    }
    return med;
}

int select_locked(csr_context_t ctx, const csr_problem_t& p, uint32_t mode, csr_schedule_t* out, uint64_t* sig_out,
                  const RowMaps* maps = nullptr)
{
    std::string why;
    const bool need_ptrs = (mode == CSR_SELECT_AUTO || mode == CSR_SELECT_FORCE_PROBE);
    int rc = csrh::check_problem(p, need_ptrs, &why);
    if (rc != CSR_OK) return set_err(ctx, rc, why);
    if (!p.row_ptr) return set_err(ctx, CSR_ERR_NULL, "row_ptr is NULL");
    if (ctx->device < 0) return set_err(ctx, CSR_ERR_DEVICE, "host-only context");
    rc = check_workspace(ctx, p, need_ptrs ? auto_workspace(p) : csrh::kHeadBytes);
    if (rc != CSR_OK) return rc;
    hipStream_t st = static_cast<hipStream_t>(p.stream);

    int64_t hist[csrh::kHistInts];
    rc = histogram(ctx, p, st, hist);
    if (rc != CSR_OK) return rc;
    const uint64_t sig = csrh::signature(p, hist, ctx->dev);
    if (sig_out) *sig_out = sig;

    if (mode == CSR_SELECT_AUTO || mode == CSR_SELECT_REPLAY_ONLY) {
        auto it = ctx->cache.find(sig);
        if (it != ctx->cache.end() && csrh::check_schedule(p, it->second.sched, nullptr) == CSR_OK) {
            *out = it->second.sched;
            return CSR_OK;
        }
        if (mode == CSR_SELECT_REPLAY_ONLY) return set_err(ctx, CSR_ERR_NO_CACHE_ENTRY, "no cached schedule for this input");
    }

    std::vector<csr_schedule_t> cand = csrh::candidates(p, hist);
    // rank by the cost model; probe the best few
    std::vector<std::pair<double, size_t>> order;
    for (size_t i = 0; i < cand.size(); ++i) order.push_back({csrh::estimate(p, cand[i], hist, ctx->dev), i});
    std::stable_sort(order.begin(), order.end(),
                     [](const std::pair<double, size_t>& x, const std::pair<double, size_t>& y) { return x.first < y.first; });
    // an in-place row softmax (or backward) cannot be probed: every probe
    // would overwrite its own input
    const bool in_place = (p.op == CSR_OP_ROW_SOFTMAX || p.op == CSR_OP_SOFTMAX_BWD) && p.out &&
                          (p.a == p.out || p.b == p.out);
    if (mode == CSR_SELECT_ESTIMATE || (ctx->flags & CSR_CTX_NO_PROBE) || in_place) {
        *out = cand[order[0].second];
        if (mode != CSR_SELECT_ESTIMATE && !in_place) store_entry(ctx, sig, *out, 0.0);
        return CSR_OK;
    }
    const int max_probe = std::max(1, env_int("CSRSA_PROBE_CANDIDATES", 6));
    std::vector<double> est(cand.size());
    for (const auto& o : order) est[o.second] = o.first;
    const std::vector<size_t> probe_set = csrh::probe_subset(cand, est, max_probe);  // ascending: ties go low
    const std::vector<double> med = probe_all(ctx, p, cand, probe_set, st, maps);
    double best = -1.0;
    size_t best_i = 0;
    for (size_t i : probe_set) {
        const double t = med[i];
        if (t < 0) continue;  // guardrail: a failing candidate is never chosen
        if (best < 0 || t < best * 0.99) {  // within 1 %: the lower candidate index wins
            best = t;
            best_i = i;
        }
    }
    best *= 1000.0;  // microseconds in the cache log
    if (best < 0) {
        // every probe failed: fall back to the default schedule
        (void)hipGetLastError();
        *out = csrh::default_schedule(p);
        return CSR_OK;
    }
    *out = cand[best_i];
    (void)store_entry(ctx, sig, *out, best);  // a log write failure keeps the entry in memory
    return CSR_OK;
}

// Shared body of the four operation calls.
int op_call(csr_context_t ctx, csr_problem_t& p, const csr_schedule_t* sched)
{
    if (!ctx) return CSR_ERR_NULL;
    try {
        std::lock_guard<std::mutex> lk(ctx->mu);
        ctx->last_error.clear();
        if (ctx->device < 0) return set_err(ctx, CSR_ERR_DEVICE, "host-only context");
        std::string why;
        int rc = csrh::check_problem(p, true, &why);
        if (rc != CSR_OK) return set_err(ctx, rc, why);
        DeviceGuard g(ctx->device);
        csr_schedule_t s;
        if (sched) {
            rc = csrh::check_schedule(p, *sched, &why);
            if (rc != CSR_OK) return set_err(ctx, rc, why);
            rc = check_workspace(ctx, p, csrh::workspace_bytes(p, *sched));
            if (rc != CSR_OK) return rc;
            s = *sched;
        } else {
            rc = select_locked(ctx, p, CSR_SELECT_AUTO, &s, nullptr);
            if (rc != CSR_OK) return rc;
        }
        return run_schedule(ctx, p, s, static_cast<hipStream_t>(p.stream));
    } catch (...) {
        return set_err(ctx, CSR_ERR_INTERNAL, "internal error");
    }
}

csr_problem_t blank_problem()
{
    csr_problem_t p;
    std::memset(&p, 0, sizeof p);
    p.scale = 1.0f;
    return p;
}

}  // namespace

extern "C" {

const char* csr_status_string(int status)
{
    switch (status) {
    case CSR_OK: return "ok";
    case CSR_ERR_NULL: return "null pointer";
    case CSR_ERR_SHAPE: return "invalid or unsupported shape";
    case CSR_ERR_DTYPE: return "unsupported dtype";
    case CSR_ERR_ALIGN: return "misaligned pointer or leading dimension";
    case CSR_ERR_WORKSPACE: return "workspace missing or too small";
    case CSR_ERR_INVALID_CSR: return "CSR validation failed";
    case CSR_ERR_SCHEDULE: return "schedule invalid for this problem";
    case CSR_ERR_NO_CACHE_ENTRY: return "no cached schedule";
    case CSR_ERR_CACHE_IO: return "cache file I/O error";
    case CSR_ERR_HIP: return "HIP runtime error";
    case CSR_ERR_DEVICE: return "no usable gfx950 device";
    case CSR_ERR_INTERNAL: return "internal error";
    default: return "unknown status";
    }
}

const char* csr_last_error(csr_context_t ctx) { return ctx ? ctx->last_error.c_str() : ""; }

int csr_context_create(csr_context_t* out, int device, const char* cache_path, uint32_t flags)
{
    if (!out) return CSR_ERR_NULL;
    *out = nullptr;
    csr_context_t ctx = nullptr;
    try {
        ctx = new csr_context_s();
        ctx->flags = flags;
        ctx->device = device;
        if (cache_path) ctx->cache_path = cache_path;
        if (device >= 0) {
            hipDeviceProp_t prop;
            if (hipGetDeviceProperties(&prop, device) != hipSuccess) {
                delete ctx;
                return CSR_ERR_DEVICE;
            }
            if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
                delete ctx;
                return CSR_ERR_DEVICE;
            }
            ctx->dev.cu_count = prop.multiProcessorCount;
            ctx->dev.arch = 950;
            DeviceGuard g(device);
            if (hipHostMalloc(reinterpret_cast<void**>(&ctx->pinned), 4096, hipHostMallocDefault) != hipSuccess) {
                delete ctx;
                return CSR_ERR_HIP;
            }
            // with the device current: its copy of the allocation-free scratch
            // array (a failure only disables csr_spmm_noalloc)
            ctx->scratch_err = scratch_address(device, &ctx->scratch);
        } else {
            ctx->pinned = static_cast<int64_t*>(std::calloc(512, sizeof(int64_t)));
        }
        if (!ctx->cache_path.empty()) load_cache(ctx);
    } catch (...) {
        delete ctx;
        return CSR_ERR_INTERNAL;
    }
    *out = ctx;
    return CSR_OK;
}

int csr_context_destroy(csr_context_t ctx)
{
    if (!ctx) return CSR_OK;
    int rc = csr_cache_flush(ctx);
    if (ctx->device >= 0) {
        DeviceGuard g(ctx->device);
        if (ctx->ev0) (void)hipEventDestroy(ctx->ev0);
        if (ctx->ev1) (void)hipEventDestroy(ctx->ev1);
        if (ctx->pinned) (void)hipHostFree(ctx->pinned);
    } else {
        std::free(ctx->pinned);
    }
    delete ctx;
    return rc;
}

int csr_spmm(csr_context_t ctx, int64_t n_rows, int64_t n_cols, int64_t nnz, const int32_t* row_ptr,
             const int32_t* col_idx, const float* vals, const void* X, int32_t x_dtype, int64_t F, int64_t ldx,
             float* Y, int64_t ldy, const csr_schedule_t* sched, void* workspace, size_t ws_bytes, void* stream)
{
    csr_problem_t p = blank_problem();
    p.op = CSR_OP_SPMM;
    p.dtype = x_dtype;
    p.n_rows = n_rows;
    p.n_cols = n_cols;
    p.nnz = nnz;
    p.width = F;
    p.ld_b = ldx;
    p.ld_out = ldy;
    p.row_ptr = row_ptr;
    p.col_idx = col_idx;
    p.a = vals;
    p.b = X;
    p.out = Y;
    p.workspace = workspace;
    p.workspace_bytes = ws_bytes;
    p.stream = stream;
    return op_call(ctx, p, sched);
}

int csr_spmm_perm(csr_context_t ctx, int64_t n_rows, int64_t n_cols, int64_t nnz, const int32_t* row_ptr,
                  const int32_t* col_idx, const float* vals, const int32_t* val_idx, const void* X, int32_t x_dtype,
                  int64_t F, int64_t ldx, float* Y, int64_t ldy, const csr_schedule_t* sched, void* workspace,
                  size_t ws_bytes, void* stream)
{
    if (!ctx) return CSR_ERR_NULL;
    if (nnz > 0 && (!vals || !val_idx)) {
        std::lock_guard<std::mutex> lk(ctx->mu);
        return set_err(ctx, CSR_ERR_NULL, "vals and val_idx must not be NULL");
    }
    csr_problem_t p = blank_problem();
    p.op = CSR_OP_SPMM;
    p.dtype = x_dtype;
    p.n_rows = n_rows;
    p.n_cols = n_cols;
    p.nnz = nnz;
    p.width = F;
    p.ld_b = ldx;
    p.ld_out = ldy;
    p.row_ptr = row_ptr;
    p.col_idx = col_idx;
    p.a = vals;
    p.a_idx = val_idx;
    p.b = X;
    p.out = Y;
    p.workspace = workspace;
    p.workspace_bytes = ws_bytes;
    p.stream = stream;
    return op_call(ctx, p, sched);
}

int csr_spmm_sddmm(csr_context_t ctx, int64_t n_rows, int64_t n_cols, int64_t nnz, const int32_t* row_ptr,
                   const int32_t* col_idx, const float* vals, const int32_t* val_idx, const float* X, int64_t F,
                   int64_t ldx, const float* U, int64_t ldu, float* Y, int64_t ldy, float* z, const int32_t* z_idx,
                   const csr_schedule_t* sched, void* workspace, size_t ws_bytes, void* stream)
{
    if (!ctx) return CSR_ERR_NULL;
    if (nnz > 0 && val_idx && !vals) {
        std::lock_guard<std::mutex> lk(ctx->mu);
        return set_err(ctx, CSR_ERR_NULL, "val_idx needs vals");
    }
    csr_problem_t p = blank_problem();
    p.op = CSR_OP_SPMM_SDDMM;
    p.dtype = CSR_DTYPE_F32;
    p.n_rows = n_rows;
    p.n_cols = n_cols;
    p.nnz = nnz;
    p.width = F;
    p.ld_b = ldx;
    p.ld_c = ldu;
    p.ld_out = ldy;
    p.row_ptr = row_ptr;
    p.col_idx = col_idx;
    p.a = vals;
    p.a_idx = val_idx;
    p.b = X;
    p.c = U;
    p.out = Y;
    p.out2 = z;
    p.out2_idx = z_idx;
    p.workspace = workspace;
    p.workspace_bytes = ws_bytes;
    p.stream = stream;
    return op_call(ctx, p, sched);
}

int csr_spmm_noalloc(csr_context_t ctx, int64_t n_rows, int64_t n_cols, int64_t nnz, const int32_t* row_ptr,
                     const int32_t* col_idx, const float* vals, const void* X, int32_t x_dtype, int64_t F,
                     int64_t ldx, float* Y, int64_t ldy, const csr_schedule_t* sched, void* stream)
{
    if (!ctx) return CSR_ERR_NULL;
    try {
        std::lock_guard<std::mutex> lk(ctx->mu);
        ctx->last_error.clear();
        if (ctx->device < 0) return set_err(ctx, CSR_ERR_DEVICE, "host-only context");
        if (!sched) return set_err(ctx, CSR_ERR_NULL, "an explicit schedule is required (select one beforehand)");
        if (ctx->scratch_err != hipSuccess || !ctx->scratch)
            return hip_err(ctx, ctx->scratch_err != hipSuccess ? ctx->scratch_err : hipErrorInvalidSymbol,
                           "scratch array address");
        csr_problem_t p = blank_problem();
        p.op = CSR_OP_SPMM;
        p.dtype = x_dtype;
        p.n_rows = n_rows;
        p.n_cols = n_cols;
        p.nnz = nnz;
        p.width = F;
        p.ld_b = ldx;
        p.ld_out = ldy;
        p.row_ptr = row_ptr;
        p.col_idx = col_idx;
        p.a = vals;
        p.b = X;
        p.out = Y;
        p.stream = stream;
        std::string why;
        int rc = csrh::check_problem(p, true, &why);
        if (rc != CSR_OK) return set_err(ctx, rc, why);
        rc = csrh::check_schedule(p, *sched, &why);
        if (rc != CSR_OK) return set_err(ctx, rc, why);
        const size_t need = csrh::workspace_bytes(p, *sched);
        if (need > (size_t)CSR_NOALLOC_SCRATCH_BYTES)
            return set_err(ctx, CSR_ERR_WORKSPACE, "the problem needs " + std::to_string(need) +
                                                       " bytes of scratch, more than the array's " +
                                                       std::to_string((size_t)CSR_NOALLOC_SCRATCH_BYTES));
        p.workspace = ctx->scratch;
        p.workspace_bytes = CSR_NOALLOC_SCRATCH_BYTES;
        DeviceGuard g(ctx->device);
        return run_schedule(ctx, p, *sched, static_cast<hipStream_t>(stream));
    } catch (...) {
        return set_err(ctx, CSR_ERR_INTERNAL, "internal error");
    }
}

int csr_sddmm(csr_context_t ctx, int64_t n_rows, int64_t n_cols, int64_t nnz, const int32_t* row_ptr,
              const int32_t* col_idx, const void* U, int64_t ldu, const void* V, int64_t ldv, int32_t dtype,
              int64_t K, float* out, const csr_schedule_t* sched, void* workspace, size_t ws_bytes, void* stream)
{
    csr_problem_t p = blank_problem();
    p.op = CSR_OP_SDDMM;
    p.dtype = dtype;
    p.n_rows = n_rows;
    p.n_cols = n_cols;
    p.nnz = nnz;
    p.width = K;
    p.ld_a = ldu;
    p.ld_b = ldv;
    p.row_ptr = row_ptr;
    p.col_idx = col_idx;
    p.a = U;
    p.b = V;
    p.out = out;
    p.workspace = workspace;
    p.workspace_bytes = ws_bytes;
    p.stream = stream;
    return op_call(ctx, p, sched);
}

// The one-head problem of head h: column views of Q, K, V, out and probs; for
// given scores (CSR_OP_ATTENTION), head h's row of the head-major scores.
static csr_problem_t head_view(const csr_problem_t& p, int32_t h, int64_t head_dim, size_t esize)
{
    csr_problem_t q = p;
    const int64_t off = (int64_t)h * head_dim;
    if (p.op == CSR_OP_ATTENTION)
        q.a = p.a ? static_cast<const float*>(p.a) + (int64_t)h * p.nnz : nullptr;
    else
        q.a = static_cast<const char*>(p.a) + off * esize;
    q.b = p.b ? static_cast<const char*>(p.b) + off * esize : nullptr;
    q.c = p.c ? static_cast<const char*>(p.c) + off * esize : nullptr;
    q.out = static_cast<float*>(p.out) + off;
    q.probs = p.probs ? p.probs + h : nullptr;
    return q;
}

// Runs the heads of an attention (from queries and keys, or from given
// scores) as one-head problems
// (ctx locked, device current).  One schedule serves every head: given, or
// selected on the head whose views allow the narrowest lane accesses (the
// lowest head index among equals), and checked against every head before
// anything is launched.
static int attention_heads(csr_context_t ctx, const csr_problem_t& p, int32_t heads, int64_t head_dim, size_t esize,
                           const csr_schedule_t* sched)
{
    std::string why;
    int h_sel = 0, v_sel = 1 << 30;
    for (int32_t h = 0; h < heads; ++h) {
        const csr_problem_t q = head_view(p, h, head_dim, esize);
        int rc = csrh::check_problem(q, true, &why);
        if (rc != CSR_OK) return set_err(ctx, rc, why);
        const int v = csrh::max_vec(q);
        if (v < v_sel) {
            v_sel = v;
            h_sel = h;
        }
    }
    const csr_problem_t qs = head_view(p, h_sel, head_dim, esize);
    csr_schedule_t s;
    if (sched) {
        s = *sched;
    } else {
        int rc = select_locked(ctx, qs, CSR_SELECT_AUTO, &s, nullptr);
        if (rc != CSR_OK) return rc;
    }
    for (int32_t h = 0; h < heads; ++h) {
        int rc = csrh::check_schedule(head_view(p, h, head_dim, esize), s, &why);
        if (rc != CSR_OK) return set_err(ctx, rc, why);
    }
    int rc = check_workspace(ctx, qs, csrh::workspace_bytes(qs, s));
    if (rc != CSR_OK) return rc;
    for (int32_t h = 0; h < heads; ++h) {
        rc = run_schedule(ctx, head_view(p, h, head_dim, esize), s, static_cast<hipStream_t>(p.stream));
        if (rc != CSR_OK) return rc;
    }
    return CSR_OK;
}

static bool aligned16(const void* p) { return ((uintptr_t)p % 16) == 0; }

int csr_attention(csr_context_t ctx, int64_t n_rows, int64_t n_cols, int64_t nnz, const int32_t* row_ptr,
                  const int32_t* col_idx, const float* edge_scores, const void* Q, const void* K,
                  const void* node_value, int32_t dtype, int32_t heads, int64_t head_dim, int64_t ldv, float scale,
                  float* out, int64_t ldo, float* probs_out, const csr_schedule_t* sched, void* workspace,
                  size_t ws_bytes, void* stream)
{
    csr_problem_t p = blank_problem();
    p.dtype = dtype;
    p.n_rows = n_rows;
    p.n_cols = n_cols;
    p.nnz = nnz;
    p.row_ptr = row_ptr;
    p.col_idx = col_idx;
    p.scale = scale;
    p.out = out;
    p.probs = probs_out;
    p.workspace = workspace;
    p.workspace_bytes = ws_bytes;
    p.stream = stream;
    if (edge_scores || (!Q && !K)) {
        // scores given (the trace page's operation); edge_scores may be NULL
        // only when there are no entries
        p.op = CSR_OP_ATTENTION;
        p.width = head_dim;
        p.ld_b = ldv;
        p.ld_out = ldo;
        p.a = edge_scores;
        p.b = node_value;
        if (heads == 1) {
            p.probs_stride = 1;
            return op_call(ctx, p, sched);
        }
        // several heads: head-major scores [heads, nnz], each head a one-head
        // problem on column views of node_value and out
        if (!ctx) return CSR_ERR_NULL;
        try {
            std::lock_guard<std::mutex> lk(ctx->mu);
            ctx->last_error.clear();
            if (ctx->device < 0) return set_err(ctx, CSR_ERR_DEVICE, "host-only context");
            if (heads < 1 || head_dim < 1) return set_err(ctx, CSR_ERR_SHAPE, "heads and head_dim must be >= 1");
            const int64_t width = (int64_t)heads * head_dim;
            if (ldv < width || ldo < width) return set_err(ctx, CSR_ERR_SHAPE, "ldv and ldo must be >= heads * head_dim");
            if (nnz > 0 && (!edge_scores || !node_value)) return set_err(ctx, CSR_ERR_NULL, "edge_scores or node_value is NULL");
            p.probs_stride = heads;
            DeviceGuard g(ctx->device);
            return attention_heads(ctx, p, heads, head_dim, dtype == CSR_DTYPE_BF16 ? 2 : 4, sched);
        } catch (...) {
            return set_err(ctx, CSR_ERR_INTERNAL, "internal error");
        }
    }
    if (!ctx) return CSR_ERR_NULL;
    const int64_t width = (int64_t)heads * head_dim;
    const bool mha = dtype == CSR_DTYPE_BF16 && heads >= 1 && head_dim >= 8 && head_dim <= 512 &&
                     (head_dim & (head_dim - 1)) == 0 && width <= 512 && ldv == width && ldo == width &&
                     aligned16(Q) && aligned16(K) && aligned16(node_value) && aligned16(out);
    if (mha) {
        // the multi-head kernel: every head of a row in one wavefront
        p.op = CSR_OP_MHA;
        p.heads = heads;
        p.head_dim = (int32_t)head_dim;
        p.width = width;
        p.a = Q;
        p.b = K;
        p.c = node_value;
        return op_call(ctx, p, sched);
    }
    try {
        std::lock_guard<std::mutex> lk(ctx->mu);
        ctx->last_error.clear();
        if (ctx->device < 0) return set_err(ctx, CSR_ERR_DEVICE, "host-only context");
        if (heads < 1 || head_dim < 1) return set_err(ctx, CSR_ERR_SHAPE, "heads and head_dim must be >= 1");
        if (!Q || !K || (nnz > 0 && !node_value)) return set_err(ctx, CSR_ERR_NULL, "Q, K or node_value is NULL");
        if (ldv < width || ldo < width) return set_err(ctx, CSR_ERR_SHAPE, "ldv and ldo must be >= heads * head_dim");
        p.op = CSR_OP_ATTENTION_QK;
        p.width = head_dim;
        p.ld_a = p.ld_b = width;
        p.ld_c = ldv;
        p.ld_out = ldo;
        p.a = Q;
        p.b = K;
        p.c = node_value;
        p.probs_stride = heads;
        DeviceGuard g(ctx->device);
        return attention_heads(ctx, p, heads, head_dim, dtype == CSR_DTYPE_BF16 ? 2 : 4, sched);
    } catch (...) {
        return set_err(ctx, CSR_ERR_INTERNAL, "internal error");
    }
}

int csr_mha_attention(csr_context_t ctx, int64_t n_rows, int64_t n_cols, int64_t nnz, const int32_t* row_ptr,
                      const int32_t* col_idx, const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                      int32_t heads, int32_t head_dim, float scale, float* out, float* probs_out,
                      const csr_schedule_t* sched, void* workspace, size_t ws_bytes, void* stream)
{
    csr_problem_t p = blank_problem();
    p.op = CSR_OP_MHA;
    p.dtype = CSR_DTYPE_BF16;
    p.n_rows = n_rows;
    p.n_cols = n_cols;
    p.nnz = nnz;
    p.heads = heads;
    p.head_dim = head_dim;
    p.width = (int64_t)heads * head_dim;
    p.row_ptr = row_ptr;
    p.col_idx = col_idx;
    p.a = Q;
    p.b = K;
    p.c = V;
    p.out = out;
    p.probs = probs_out;
    p.scale = scale;
    p.workspace = workspace;
    p.workspace_bytes = ws_bytes;
    p.stream = stream;
    return op_call(ctx, p, sched);
}

int csr_row_softmax(csr_context_t ctx, int64_t n_rows, int64_t nnz, const int32_t* row_ptr, const float* scores,
                    float scale, float* probs, const csr_schedule_t* sched, void* workspace, size_t ws_bytes,
                    void* stream)
{
    csr_problem_t p = blank_problem();
    p.op = CSR_OP_ROW_SOFTMAX;
    p.dtype = CSR_DTYPE_F32;
    p.n_rows = n_rows;
    p.n_cols = 0;
    p.nnz = nnz;
    p.width = 1;
    p.row_ptr = row_ptr;
    p.a = scores;
    p.out = probs;
    p.scale = scale;
    p.workspace = workspace;
    p.workspace_bytes = ws_bytes;
    p.stream = stream;
    return op_call(ctx, p, sched);
}

int csr_row_softmax_backward(csr_context_t ctx, int64_t n_rows, int64_t nnz, const int32_t* row_ptr,
                             const float* probs, const float* grad_probs, float scale, float* grad_scores,
                             const csr_schedule_t* sched, void* workspace, size_t ws_bytes, void* stream)
{
    csr_problem_t p = blank_problem();
    p.op = CSR_OP_SOFTMAX_BWD;
    p.dtype = CSR_DTYPE_F32;
    p.n_rows = n_rows;
    p.n_cols = 0;
    p.nnz = nnz;
    p.width = 1;
    p.row_ptr = row_ptr;
    p.a = probs;
    p.b = grad_probs;
    p.out = grad_scores;
    p.scale = scale;
    p.workspace = workspace;
    p.workspace_bytes = ws_bytes;
    p.stream = stream;
    return op_call(ctx, p, sched);
}

static int transpose_args(int64_t n_rows, int64_t n_cols, int64_t nnz)
{
    const int64_t lim = (int64_t)1 << 31;
    if (n_rows < 0 || n_cols < 0 || nnz < 0) return CSR_ERR_SHAPE;
    if (n_rows >= lim - 1 || n_cols >= lim - 1 || nnz >= lim) return CSR_ERR_SHAPE;
    if (nnz > 0 && (n_rows == 0 || n_cols == 0)) return CSR_ERR_SHAPE;
    return CSR_OK;
}

int csr_transpose_workspace_size(csr_context_t ctx, int64_t n_rows, int64_t n_cols, int64_t nnz, size_t* bytes)
{
    if (!ctx || !bytes) return CSR_ERR_NULL;
    std::lock_guard<std::mutex> lk(ctx->mu);
    const int rc = transpose_args(n_rows, n_cols, nnz);
    if (rc != CSR_OK) return set_err(ctx, rc, "bad sizes");
    if (ctx->device < 0) return set_err(ctx, CSR_ERR_DEVICE, "host-only context");
    DeviceGuard g(ctx->device);
    hipError_t e = csrk::transpose_workspace(n_cols, nnz, bytes);
    if (e != hipSuccess) return hip_err(ctx, e, "transpose workspace");
    return CSR_OK;
}

int csr_transpose(csr_context_t ctx, int64_t n_rows, int64_t n_cols, int64_t nnz, const int32_t* row_ptr,
                  const int32_t* col_idx, int32_t* t_row_ptr, int32_t* t_col_idx, int32_t* t_perm,
                  void* workspace, size_t ws_bytes, void* stream)
{
    if (!ctx || !row_ptr || !t_row_ptr) return CSR_ERR_NULL;
    if (nnz > 0 && (!col_idx || !t_col_idx || !t_perm || !workspace)) return CSR_ERR_NULL;
    std::lock_guard<std::mutex> lk(ctx->mu);
    const int rc = transpose_args(n_rows, n_cols, nnz);
    if (rc != CSR_OK) return set_err(ctx, rc, "bad sizes");
    try {
        ctx->last_error.clear();
        if (ctx->device < 0) return set_err(ctx, CSR_ERR_DEVICE, "host-only context");
        DeviceGuard g(ctx->device);
        size_t need = 0;
        CSR_HIP(ctx, csrk::transpose_workspace(n_cols, nnz, &need));
        if (ws_bytes < need) return set_err(ctx, CSR_ERR_WORKSPACE, "workspace too small for the transpose");
        hipStream_t st = static_cast<hipStream_t>(stream);
        if ((ctx->flags & CSR_CTX_VALIDATE) && nnz > 0) {
            int64_t* bad = reinterpret_cast<int64_t*>(workspace);
            CSR_HIP(ctx, csrk::launch_validate(row_ptr, col_idx, n_rows, n_cols, nnz, bad, st));
            CSR_HIP(ctx, hipMemcpyAsync(ctx->pinned, bad, sizeof(int64_t), hipMemcpyDeviceToHost, st));
            CSR_HIP(ctx, hipStreamSynchronize(st));
            if (ctx->pinned[0] != 0) return set_err(ctx, CSR_ERR_INVALID_CSR, "row_ptr / col_idx fail CSR validation");
        }
        CSR_HIP(ctx, csrk::launch_transpose(row_ptr, col_idx, n_rows, n_cols, nnz, t_row_ptr, t_col_idx, t_perm,
                                            workspace, ws_bytes, st));
        return CSR_OK;
    } catch (...) {
        return set_err(ctx, CSR_ERR_INTERNAL, "internal error");
    }
}

int csr_gather_values(csr_context_t ctx, int64_t n, const int32_t* perm, const float* src, float* dst, void* stream)
{
    if (!ctx) return CSR_ERR_NULL;
    std::lock_guard<std::mutex> lk(ctx->mu);
    if (n < 0 || n >= ((int64_t)1 << 31)) return set_err(ctx, CSR_ERR_SHAPE, "bad size");
    if (n > 0 && (!perm || !src || !dst)) return CSR_ERR_NULL;
    if (n > 0 && src == dst) return set_err(ctx, CSR_ERR_SHAPE, "src and dst must not alias");
    if (((uintptr_t)perm | (uintptr_t)src | (uintptr_t)dst) % 4)
        return set_err(ctx, CSR_ERR_ALIGN, "the arrays must be 4-byte aligned");
    if (ctx->device < 0) return set_err(ctx, CSR_ERR_DEVICE, "host-only context");
    DeviceGuard g(ctx->device);
    CSR_HIP(ctx, csrk::launch_gather_values(perm, src, dst, n, static_cast<hipStream_t>(stream)));
    return CSR_OK;
}

int csr_inverse_permutation(csr_context_t ctx, int64_t n, const int32_t* perm, int32_t* inv, void* stream)
{
    if (!ctx) return CSR_ERR_NULL;
    std::lock_guard<std::mutex> lk(ctx->mu);
    if (n < 0 || n >= ((int64_t)1 << 31)) return set_err(ctx, CSR_ERR_SHAPE, "bad size");
    if (n > 0 && (!perm || !inv)) return CSR_ERR_NULL;
    if (n > 0 && (const void*)perm == (const void*)inv) return set_err(ctx, CSR_ERR_SHAPE, "perm and inv must not alias");
    if (ctx->device < 0) return set_err(ctx, CSR_ERR_DEVICE, "host-only context");
    DeviceGuard g(ctx->device);
    CSR_HIP(ctx, csrk::launch_invert(perm, inv, n, static_cast<hipStream_t>(stream)));
    return CSR_OK;
}

static bool perm_size_ok(int64_t n) { return n >= 0 && n < ((int64_t)1 << 31); }

int csr_permutation_plan_workspace_size(csr_context_t ctx, int64_t n, size_t* bytes)
{
    if (!ctx || !bytes) return CSR_ERR_NULL;
    std::lock_guard<std::mutex> lk(ctx->mu);
    if (!perm_size_ok(n)) return set_err(ctx, CSR_ERR_SHAPE, "bad size");
    if (ctx->device < 0) return set_err(ctx, CSR_ERR_DEVICE, "host-only context");
    DeviceGuard g(ctx->device);
    CSR_HIP(ctx, csrk::permutation_plan_workspace(n, bytes));
    return CSR_OK;
}

int csr_permutation_plan(csr_context_t ctx, int64_t n, const int32_t* q, int32_t window_log2, int32_t* q1,
                         int32_t* pos, void* workspace, size_t ws_bytes, void* stream)
{
    if (!ctx) return CSR_ERR_NULL;
    std::lock_guard<std::mutex> lk(ctx->mu);
    if (!perm_size_ok(n) || window_log2 < 8 || window_log2 > 30) return set_err(ctx, CSR_ERR_SHAPE, "bad size or window");
    if (n > 0 && (!q || !q1 || !pos || !workspace)) return CSR_ERR_NULL;
    if (n > 0 && ((const void*)q == (const void*)q1 || (const void*)q == (const void*)pos || q1 == pos))
        return set_err(ctx, CSR_ERR_SHAPE, "q, q1 and pos must not alias");
    if (ctx->device < 0) return set_err(ctx, CSR_ERR_DEVICE, "host-only context");
    DeviceGuard g(ctx->device);
    size_t need = 0;
    CSR_HIP(ctx, csrk::permutation_plan_workspace(n, &need));
    if (ws_bytes < need || (uintptr_t)workspace % csrh::kAlign)
        return set_err(ctx, CSR_ERR_WORKSPACE, "workspace too small (or not 256-byte aligned) for the plan");
    CSR_HIP(ctx, csrk::launch_permutation_plan(q, n, window_log2, q1, pos, workspace, ws_bytes,
                                               static_cast<hipStream_t>(stream)));
    return CSR_OK;
}

int csr_permute_values(csr_context_t ctx, int64_t n, const int32_t* q1, const int32_t* pos, const float* src,
                       float* tmp, float* dst, void* stream)
{
    if (!ctx) return CSR_ERR_NULL;
    std::lock_guard<std::mutex> lk(ctx->mu);
    if (!perm_size_ok(n)) return set_err(ctx, CSR_ERR_SHAPE, "bad size");
    if (n > 0 && (!q1 || !pos || !src || !tmp || !dst)) return CSR_ERR_NULL;
    if (n > 0 && (src == tmp || src == dst || tmp == dst))
        return set_err(ctx, CSR_ERR_SHAPE, "src, tmp and dst must not alias");
    if (((uintptr_t)q1 | (uintptr_t)pos | (uintptr_t)src | (uintptr_t)tmp | (uintptr_t)dst) % 4)
        return set_err(ctx, CSR_ERR_ALIGN, "the arrays must be 4-byte aligned");
    if (ctx->device < 0) return set_err(ctx, CSR_ERR_DEVICE, "host-only context");
    DeviceGuard g(ctx->device);
    CSR_HIP(ctx, csrk::launch_permute(q1, pos, src, tmp, dst, n, static_cast<hipStream_t>(stream)));
    return CSR_OK;
}

// ---------------------------------------------------------------------------
// Column-part segment format
// ---------------------------------------------------------------------------

static bool valid_parts(int32_t parts)
{
    return parts >= 1 && parts <= 256 && (parts & (parts - 1)) == 0;
}

int csr_hybrid_capacity(int64_t n_rows, int64_t nnz, int32_t parts, int64_t* seg_cap)
{
    if (!seg_cap) return CSR_ERR_NULL;
    const int64_t lim = (int64_t)1 << 31;
    if (n_rows < 0 || nnz < 0 || n_rows >= lim - 1 || nnz >= lim || !valid_parts(parts)) return CSR_ERR_SHAPE;
    *seg_cap = std::min(nnz, n_rows * (int64_t)parts);
    return CSR_OK;
}

int csr_hybrid_build_workspace_size(csr_context_t ctx, int64_t n_rows, int64_t nnz, int32_t parts, size_t* bytes)
{
    if (!ctx || !bytes) return CSR_ERR_NULL;
    std::lock_guard<std::mutex> lk(ctx->mu);
    int64_t cap = 0;
    if (csr_hybrid_capacity(n_rows, nnz, parts, &cap) != CSR_OK) return set_err(ctx, CSR_ERR_SHAPE, "bad sizes or parts");
    if (ctx->device < 0) return set_err(ctx, CSR_ERR_DEVICE, "host-only context");
    DeviceGuard g(ctx->device);
    hipError_t e = csrk::hybrid_build_workspace(n_rows, nnz, parts, bytes);
    if (e != hipSuccess) return hip_err(ctx, e, "hybrid build workspace");
    return CSR_OK;
}

// Checks a format description: sizes, parts, capacity and arrays, and for a
// built format the segment count and part width it records.
static int check_hybrid(csr_context_t ctx, const csr_hybrid_t* h, bool built)
{
    if (!h) return CSR_ERR_NULL;
    int rc = transpose_args(h->n_rows, h->n_cols, h->nnz);
    if (rc != CSR_OK) return set_err(ctx, rc, "bad format sizes");
    if (!valid_parts(h->parts)) return set_err(ctx, CSR_ERR_SHAPE, "parts must be a power of two from 1 to 256");
    if (h->whole_below < 0 || h->reserved_ != 0) return set_err(ctx, CSR_ERR_SHAPE, "whole_below < 0 or reserved != 0");
    int64_t cap = 0;
    (void)csr_hybrid_capacity(h->n_rows, h->nnz, h->parts, &cap);
    // a build needs room for the worst case; a built format for its own segments
    if (!built && h->seg_cap < cap)
        return set_err(ctx, CSR_ERR_WORKSPACE, "segment capacity below min(nnz, n_rows * parts)");
    if (!h->seg_ptr || !h->row_seg_ptr) return set_err(ctx, CSR_ERR_NULL, "seg_ptr / row_seg_ptr is NULL");
    if (h->nnz > 0 && (!h->perm || !h->col_idx || !h->seg_row || !h->row_seg))
        return set_err(ctx, CSR_ERR_NULL, "a format array is NULL");
    if (built) {
        const int64_t pc = h->n_cols > 0 ? (h->n_cols + h->parts - 1) / h->parts : 1;
        if (h->part_cols != pc || h->n_seg < 0 || h->n_seg > cap || h->n_seg > h->seg_cap ||
            (h->nnz > 0) != (h->n_seg > 0))
            return set_err(ctx, CSR_ERR_SHAPE, "the format is not built (part_cols / n_seg)");
    }
    return CSR_OK;
}

// Builds the format of (row_ptr, col_idx) into h's arrays (ctx locked, device
// current).  h->seg_cap need only hold the segments this input has: the
// count is read back after the sort and checked before any segment array is
// written.  Synchronous.
static int build_format(csr_context_t ctx, const int32_t* row_ptr, const int32_t* col_idx, csr_hybrid_t* h,
                        void* workspace, size_t ws_bytes, hipStream_t st)
{
    size_t need = 0;
    CSR_HIP(ctx, csrk::hybrid_build_workspace(h->n_rows, h->nnz, h->parts, &need));
    if (ws_bytes < need || !workspace || (uintptr_t)workspace % csrh::kAlign)
        return set_err(ctx, CSR_ERR_WORKSPACE, "workspace too small (or not 256-byte aligned) for the build");
    const int32_t part_cols = h->n_cols > 0 ? (int32_t)((h->n_cols + h->parts - 1) / h->parts) : 1;
    int64_t n_seg = 0;
    if (h->nnz > 0) {
        int32_t* count = reinterpret_cast<int32_t*>(ctx->pinned);
        CSR_HIP(ctx, csrk::launch_hybrid_build_sort(row_ptr, col_idx, h->n_rows, h->nnz, h->parts, part_cols,
                                                    h->whole_below, h->perm, h->col_idx, workspace, ws_bytes, count,
                                                    st));
        CSR_HIP(ctx, hipStreamSynchronize(st));
        n_seg = count[0];
        if (n_seg < 1 || n_seg > h->seg_cap) return set_err(ctx, CSR_ERR_INTERNAL, "segment count out of range");
    }
    CSR_HIP(ctx, csrk::launch_hybrid_build_segments(h->n_rows, h->nnz, h->parts, n_seg, h->seg_ptr, h->seg_row,
                                                    h->row_seg_ptr, h->row_seg, workspace, st));
    h->n_seg = n_seg;
    h->part_cols = part_cols;
    return CSR_OK;
}

int csr_hybrid_build(csr_context_t ctx, const int32_t* row_ptr, const int32_t* col_idx, csr_hybrid_t* h,
                     void* workspace, size_t ws_bytes, void* stream)
{
    if (!ctx || !row_ptr || !h) return CSR_ERR_NULL;
    std::lock_guard<std::mutex> lk(ctx->mu);
    ctx->last_error.clear();
    int rc = check_hybrid(ctx, h, false);
    if (rc != CSR_OK) return rc;
    if (!workspace || (h->nnz > 0 && !col_idx)) return CSR_ERR_NULL;
    try {
        if (ctx->device < 0) return set_err(ctx, CSR_ERR_DEVICE, "host-only context");
        DeviceGuard g(ctx->device);
        size_t need = 0;
        CSR_HIP(ctx, csrk::hybrid_build_workspace(h->n_rows, h->nnz, h->parts, &need));
        if (ws_bytes < need || (uintptr_t)workspace % csrh::kAlign)
            return set_err(ctx, CSR_ERR_WORKSPACE, "workspace too small (or not 256-byte aligned) for the build");
        hipStream_t st = static_cast<hipStream_t>(stream);
        if ((ctx->flags & CSR_CTX_VALIDATE) && h->nnz > 0) {
            int64_t* bad = reinterpret_cast<int64_t*>(workspace);
            CSR_HIP(ctx, csrk::launch_validate(row_ptr, col_idx, h->n_rows, h->n_cols, h->nnz, bad, st));
            CSR_HIP(ctx, hipMemcpyAsync(ctx->pinned, bad, sizeof(int64_t), hipMemcpyDeviceToHost, st));
            CSR_HIP(ctx, hipStreamSynchronize(st));
            if (ctx->pinned[0] != 0) return set_err(ctx, CSR_ERR_INVALID_CSR, "row_ptr / col_idx fail CSR validation");
        }
        return build_format(ctx, row_ptr, col_idx, h, workspace, ws_bytes, st);
    } catch (...) {
        return set_err(ctx, CSR_ERR_INTERNAL, "internal error");
    }
}

// The product over the format as a plain problem on the segment pattern
static csr_problem_t hybrid_problem(const csr_hybrid_t* h, int32_t op, int64_t width, int32_t dtype)
{
    csr_problem_t p = blank_problem();
    p.op = op;
    p.dtype = dtype;
    p.n_rows = h->n_seg;
    p.n_cols = h->n_cols;
    p.nnz = h->nnz;
    p.width = width;
    p.ld_a = p.ld_b = p.ld_out = width;
    p.row_ptr = h->seg_ptr;
    p.col_idx = h->col_idx;
    return p;
}

// workspace of the segment product (schedule sched, or any the selector picks)
static int hybrid_inner_bytes(csr_context_t ctx, const csr_problem_t& p, const csr_schedule_t* sched, size_t* bytes)
{
    std::string why;
    int rc = csrh::check_problem(p, false, &why);
    if (rc != CSR_OK) return set_err(ctx, rc, why);
    size_t need = auto_workspace(p);
    if (sched) {
        rc = csrh::check_schedule(p, *sched, &why);
        if (rc != CSR_OK) return set_err(ctx, rc, why);
        need = std::max(need, csrh::workspace_bytes(p, *sched));
    }
    *bytes = (need + csrh::kAlign - 1) / csrh::kAlign * csrh::kAlign;
    return CSR_OK;
}

int csr_hybrid_workspace_size(csr_context_t ctx, const csr_hybrid_t* h, int32_t op, int64_t width, int32_t dtype,
                              const csr_schedule_t* sched, size_t* bytes)
{
    if (!bytes) return CSR_ERR_NULL;
    CtxLock lk(ctx);
    int rc = check_hybrid(ctx, h, true);
    if (rc != CSR_OK) return rc;
    if (op != CSR_OP_SPMM && op != CSR_OP_SDDMM) return set_err(ctx, CSR_ERR_SHAPE, "the format serves SpMM and SDDMM");
    csr_problem_t p = hybrid_problem(h, op, width, dtype);
    size_t inner = 0;
    rc = hybrid_inner_bytes(ctx, p, sched, &inner);
    if (rc != CSR_OK) return rc;
    *bytes = inner + (op == CSR_OP_SPMM ? (size_t)h->n_seg * width * 4 : 0);
    return CSR_OK;
}

// The segment product of a call over the format: the plain problem on the
// segment pattern with the caller's operands, its workspace (SpMM: followed
// by the segments' partial rows) and, for SDDMM, the index maps.
struct HybridCall {
    csr_problem_t p;
    RowMaps maps;
    float* part_rows;  // SpMM only
};

static int hybrid_call(csr_context_t ctx, const csr_hybrid_t* h, int32_t op, int64_t width, int32_t dtype,
                       const void* a, int64_t lda, const void* b, int64_t ldb, const csr_schedule_t* sched,
                       void* workspace, size_t ws_bytes, void* stream, float* sddmm_out, HybridCall* c)
{
    int rc = check_hybrid(ctx, h, true);
    if (rc != CSR_OK) return rc;
    if (op != CSR_OP_SPMM && op != CSR_OP_SDDMM) return set_err(ctx, CSR_ERR_SHAPE, "the format serves SpMM and SDDMM");
    c->p = hybrid_problem(h, op, width, dtype);
    c->p.a = a;
    c->p.b = b;
    c->p.ld_b = ldb;
    c->maps = RowMaps{nullptr, nullptr, 1};  // SpMM: the partial rows are read only by the sum
    c->part_rows = nullptr;
    if (op == CSR_OP_SDDMM) {
        c->p.ld_a = lda;
        c->p.out = sddmm_out;
        c->maps = RowMaps{h->seg_row, h->perm, 0};
    }
    size_t inner = 0;
    rc = hybrid_inner_bytes(ctx, c->p, sched, &inner);
    if (rc != CSR_OK) return rc;
    const size_t need = inner + (op == CSR_OP_SPMM ? (size_t)h->n_seg * width * 4 : 0);
    if (!workspace || (uintptr_t)workspace % csrh::kAlign)
        return set_err(ctx, CSR_ERR_WORKSPACE, "workspace is NULL or not 256-byte aligned");
    if (ws_bytes < need) return set_err(ctx, CSR_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need));
    if (op == CSR_OP_SPMM) {
        c->part_rows = reinterpret_cast<float*>(static_cast<char*>(workspace) + inner);
        c->p.out = c->part_rows;
        c->p.ld_out = width;
    }
    c->p.workspace = workspace;
    c->p.workspace_bytes = op == CSR_OP_SPMM ? inner : ws_bytes;
    c->p.stream = stream;
    std::string why;
    rc = csrh::check_problem(c->p, true, &why);
    if (rc != CSR_OK) return set_err(ctx, rc, why);
    return CSR_OK;
}

// Runs a prepared call (ctx locked, device current): the segment product
// with sched or the selected schedule, then (SpMM) the sum of the partial rows.
static int hybrid_run(csr_context_t ctx, const csr_hybrid_t* h, const HybridCall& c, const csr_schedule_t* sched,
                      float* Y, int64_t ldy)
{
    hipStream_t st = static_cast<hipStream_t>(c.p.stream);
    const RowMaps* maps = &c.maps;
    if (h->n_seg > 0) {
        csr_schedule_t s;
        if (sched) {
            s = *sched;
        } else {
            int rc = select_locked(ctx, c.p, CSR_SELECT_AUTO, &s, nullptr, maps);
            if (rc != CSR_OK) return rc;
        }
        int rc = run_schedule(ctx, c.p, s, st, maps);
        if (rc != CSR_OK) return rc;
    }
    if (c.p.op == CSR_OP_SPMM) {
        // lane layout of the sum: the widest access that F, ldy and Y allow
        // (the partial rows are 256-byte aligned with leading dimension F)
        const int64_t F = c.p.width;
        int vec = 4, W = 0, nv = 0;
        while (vec > 1 && (F % vec || ldy % vec || (uintptr_t)Y % (4 * vec) || !csrh::natural_layout(F, vec, &W, &nv)))
            vec /= 2;
        if (vec == 1 && !csrh::natural_layout(F, 1, &W, &nv)) return set_err(ctx, CSR_ERR_SHAPE, "width too large");
        CSR_HIP(ctx, csrk::launch_hybrid_reduce(vec, nv, W, Y, ldy, c.part_rows, (int32_t)F, h->row_seg_ptr, h->row_seg,
                                                h->n_rows, st));
    }
    return CSR_OK;
}

int csr_hybrid_spmm(csr_context_t ctx, const csr_hybrid_t* h, const float* vals, const void* X, int32_t x_dtype,
                    int64_t F, int64_t ldx, float* Y, int64_t ldy, const csr_schedule_t* sched, void* workspace,
                    size_t ws_bytes, void* stream)
{
    if (!ctx || !X || !Y) return CSR_ERR_NULL;
    std::lock_guard<std::mutex> lk(ctx->mu);
    ctx->last_error.clear();
    if (F < 1 || ldy < F || ldy >= ((int64_t)1 << 30)) return set_err(ctx, CSR_ERR_SHAPE, "bad width or ldy");
    try {
        HybridCall c;
        int rc = hybrid_call(ctx, h, CSR_OP_SPMM, F, x_dtype, vals, 0, X, ldx, sched, workspace, ws_bytes, stream,
                             nullptr, &c);
        if (rc != CSR_OK) return rc;
        if (ctx->device < 0) return set_err(ctx, CSR_ERR_DEVICE, "host-only context");
        DeviceGuard g(ctx->device);
        return hybrid_run(ctx, h, c, sched, Y, ldy);
    } catch (...) {
        return set_err(ctx, CSR_ERR_INTERNAL, "internal error");
    }
}

int csr_hybrid_sddmm(csr_context_t ctx, const csr_hybrid_t* h, const void* U, int64_t ldu, const void* V,
                     int64_t ldv, int32_t dtype, int64_t K, float* out, const csr_schedule_t* sched, void* workspace,
                     size_t ws_bytes, void* stream)
{
    if (!ctx) return CSR_ERR_NULL;
    try {
        std::lock_guard<std::mutex> lk(ctx->mu);
        ctx->last_error.clear();
        HybridCall c;
        int rc = hybrid_call(ctx, h, CSR_OP_SDDMM, K, dtype, U, ldu, V, ldv, sched, workspace, ws_bytes, stream, out,
                             &c);
        if (rc != CSR_OK) return rc;
        if (ctx->device < 0) return set_err(ctx, CSR_ERR_DEVICE, "host-only context");
        DeviceGuard g(ctx->device);
        return hybrid_run(ctx, h, c, sched, nullptr, 0);
    } catch (...) {
        return set_err(ctx, CSR_ERR_INTERNAL, "internal error");
    }
}

int csr_hybrid_select(csr_context_t ctx, const csr_hybrid_t* h, const csr_problem_t* call, uint32_t mode,
                      csr_schedule_t* out, uint64_t* signature)
{
    if (!ctx || !call || !out) return CSR_ERR_NULL;
    std::lock_guard<std::mutex> lk(ctx->mu);
    ctx->last_error.clear();
    if (mode > CSR_SELECT_ESTIMATE) return set_err(ctx, CSR_ERR_SHAPE, "unknown selection mode");
    try {
        HybridCall c;
        int rc = hybrid_call(ctx, h, call->op, call->width, call->dtype, call->a, call->ld_a, call->b, call->ld_b,
                             nullptr, call->workspace, call->workspace_bytes, call->stream,
                             static_cast<float*>(call->out), &c);
        if (rc != CSR_OK) return rc;
        if (ctx->device < 0) return set_err(ctx, CSR_ERR_DEVICE, "host-only context");
        DeviceGuard g(ctx->device);
        if (h->n_seg == 0) {  // nothing to run: the default schedule
            *out = csrh::default_schedule(c.p);
            if (signature) *signature = 0;
            return CSR_OK;
        }
        return select_locked(ctx, c.p, mode, out, signature, &c.maps);
    } catch (...) {
        return set_err(ctx, CSR_ERR_INTERNAL, "internal error");
    }
}

// ---------------------------------------------------------------------------
// Planned products
// ---------------------------------------------------------------------------

static size_t up256(size_t v) { return (v + csrh::kAlign - 1) / csrh::kAlign * csrh::kAlign; }

// Plan memory of a format with room for cap segments: perm, col_idx, seg_ptr,
// seg_row, row_seg_ptr, row_seg, then (SpMM) the values in format order.
struct PlanLayout {
    size_t perm, col, seg_ptr, seg_row, row_seg_ptr, row_seg, vals, total;
};

static PlanLayout plan_layout(const csr_problem_t& p, int64_t cap)
{
    PlanLayout L{};
    L.perm = 0;
    L.col = L.perm + up256((size_t)p.nnz * 4);
    L.seg_ptr = L.col + up256((size_t)p.nnz * 4);
    L.seg_row = L.seg_ptr + up256((size_t)(cap + 1) * 4);
    L.row_seg_ptr = L.seg_row + up256((size_t)cap * 4);
    L.row_seg = L.row_seg_ptr + up256((size_t)(p.n_rows + 1) * 4);
    L.vals = L.row_seg + up256((size_t)cap * 4);
    L.total = L.vals + (p.op == CSR_OP_SPMM ? up256((size_t)p.nnz * 4) : 0);
    return L;
}

// The format description of (P, T) with its arrays in plan memory.
static csr_hybrid_t plan_format(const csr_problem_t& p, int P, int T, int64_t cap, void* mem, float** vals)
{
    const PlanLayout L = plan_layout(p, cap);
    char* m = static_cast<char*>(mem);
    csr_hybrid_t h;
    std::memset(&h, 0, sizeof h);
    h.n_rows = p.n_rows;
    h.n_cols = p.n_cols;
    h.nnz = p.nnz;
    h.parts = P;
    h.whole_below = T;
    h.seg_cap = cap;
    h.perm = reinterpret_cast<int32_t*>(m + L.perm);
    h.col_idx = reinterpret_cast<int32_t*>(m + L.col);
    h.seg_ptr = reinterpret_cast<int32_t*>(m + L.seg_ptr);
    h.seg_row = reinterpret_cast<int32_t*>(m + L.seg_row);
    h.row_seg_ptr = reinterpret_cast<int32_t*>(m + L.row_seg_ptr);
    h.row_seg = reinterpret_cast<int32_t*>(m + L.row_seg);
    if (vals) *vals = p.op == CSR_OP_SPMM ? reinterpret_cast<float*>(m + L.vals) : nullptr;
    return h;
}

// The long rows' CSR of degree classes bk as a problem with p's operands.
static csr_problem_t bucket_long_problem(const csr_problem_t& p, const csr_bucket_t& bk, const float* long_val)
{
    csr_problem_t q = p;
    q.nnz = bk.nnz_long;
    q.row_ptr = bk.long_row_ptr;
    q.col_idx = bk.long_col;
    q.a = long_val;
    q.a_idx = nullptr;
    return q;
}

// The packed rows' SpMM for p (X = p.b, Y = p.out), in the natural lane
// layout of the width at the widest access the operands allow.
static int bucket_launch(csr_context_t ctx, const csr_problem_t& p, const csr_bucket_t& bk, const float* slot_val,
                         hipStream_t st)
{
    if (bk.n_short == 0) return CSR_OK;
    const int vec = csrh::max_vec(p);
    int W = 0, nv = 0;
    if (vec < 1 || !csrh::natural_layout(p.width, vec, &W, &nv))
        return set_err(ctx, CSR_ERR_SHAPE, "no lane layout for the packed rows at this width");
    constexpr int64_t kBlock = 256;  // threads per workgroup of the kernels
    csrk::BucketArgs a{};
    a.rows = bk.rows;
    a.slot_col = bk.slot_col;
    a.slot_val = slot_val;
    a.n_classes = bk.n_classes;
    a.F = (int32_t)p.width;
    a.W = W;
    int64_t blocks = 0, base = 0, row0 = 0;
    for (int c = 0; c < bk.n_classes; ++c) {
        a.cls_rows[c] = bk.class_rows[c];
        a.cls_base[c] = base;
        a.cls_row0[c] = row0;
        a.cls_block0[c] = blocks;
        base += bk.class_rows[c] * ((2 << c) - 1);
        row0 += bk.class_rows[c];
        blocks += (bk.class_rows[c] * W + kBlock - 1) / kBlock;
    }
    a.cls_block0[bk.n_classes] = blocks;
    if (base != bk.n_slots || row0 != bk.n_short) return set_err(ctx, CSR_ERR_SHAPE, "inconsistent degree classes");
    a.X = p.b;
    a.ldx = p.ld_b;
    a.Y = static_cast<float*>(p.out);
    a.ldy = p.ld_out;
    CSR_HIP(ctx, csrk::launch_bucket_spmm(p.dtype == CSR_DTYPE_BF16, vec, nv, a, st));
    return CSR_OK;
}

// The whole product over degree classes: the long rows' CSR with schedule s
// (it writes every row of Y, the packed ones as zeros), then the packed rows.
static int bucket_run(csr_context_t ctx, const csr_problem_t& p, const csr_bucket_t& bk, const csr_schedule_t& s,
                      const float* slot_val, const float* long_val, hipStream_t st)
{
    int rc = run_schedule(ctx, bucket_long_problem(p, bk, long_val), s, st);
    if (rc != CSR_OK) return rc;
    return bucket_launch(ctx, p, bk, slot_val, st);
}

// Plan memory and workspace of one layout of p (parts 1 plain, 0 degree
// classes of short threshold T, else the format (parts, T)).
static void layout_sizes(const csr_problem_t& p, const int64_t* hist, int P, int T, size_t* plan_bytes,
                         size_t* ws_bytes)
{
    size_t mem = csrh::kAlign, ws = up256(auto_workspace(p));
    if (P == 0) {
        const csrh::BucketShape sh = csrh::bucket_shape(p, hist, T);
        mem = std::max(mem, csrh::bucket_layout(p, sh).total);
        size_t build = 0;
        (void)csrk::bucket_build_workspace(p.n_rows, p.nnz, &build);
        csr_problem_t q = p;  // the long rows' product
        q.nnz = sh.nnz_long;
        q.row_ptr = nullptr;
        const size_t inner = up256(auto_workspace(q)) + up256((size_t)sh.n_slots * 4) +
                             up256((size_t)sh.nnz_long * 4);
        ws = std::max(ws, std::max(up256(build), inner));
    } else if (P > 1) {
        const int64_t cap = csrh::segment_bound(p, hist, P, T);
        mem = std::max(mem, plan_layout(p, cap).total);
        size_t build = 0;
        (void)csrk::hybrid_build_workspace(p.n_rows, p.nnz, P, &build);
        csr_problem_t q = p;  // the product on at most cap segments
        q.n_rows = cap;
        q.row_ptr = nullptr;
        q.ld_out = p.width;
        if (p.op == CSR_OP_SPMM) q.out = reinterpret_cast<void*>(csrh::kAlign);  // partial rows, 256-byte aligned
        const size_t inner = up256(auto_workspace(q)) +
                             (p.op == CSR_OP_SPMM ? up256((size_t)cap * p.width * 4) + up256((size_t)p.nnz * 4) : 0);
        ws = std::max(ws, std::max(up256(build), inner));
    }
    *plan_bytes = mem;
    *ws_bytes = ws;
}

// Plan memory and workspace for every layout a plan of p may probe.
static void plan_sizes(const csr_problem_t& p, const int64_t* hist, size_t* plan_bytes, size_t* ws_bytes)
{
    size_t mem = 0, ws = 0;
    layout_sizes(p, hist, 1, 0, &mem, &ws);
    auto take = [&](int P, int T) {
        size_t m = 0, w = 0;
        layout_sizes(p, hist, P, T, &m, &w);
        mem = std::max(mem, m);
        ws = std::max(ws, w);
    };
    for (int E : csrh::plan_buckets(p, hist)) take(0, E);
    for (const auto& f : csrh::plan_formats(p, hist)) take(f.first, f.second);
    *plan_bytes = mem;
    *ws_bytes = ws;
}

// Whether (parts, whole_below) names a layout a plan of p can take.
static bool layout_ok(const csr_problem_t& p, int P, int T)
{
    if (P == 1) return true;
    if (P == 0) return p.op == CSR_OP_SPMM && T >= 2 && T <= (1 << CSR_BUCKET_MAX_CLASSES) && (T & (T - 1)) == 0;
    return P >= 2 && P <= 256 && (P & (P - 1)) == 0 && T >= 0;
}

static int check_plan_problem(csr_context_t ctx, const csr_problem_t& p, bool need_ptrs)
{
    if (p.op != CSR_OP_SPMM && p.op != CSR_OP_SDDMM) return set_err(ctx, CSR_ERR_SHAPE, "plans serve SpMM and SDDMM");
    if (p.a_idx) return set_err(ctx, CSR_ERR_SHAPE, "plans take the values in entry order (no value index)");
    std::string why;
    int rc = csrh::check_problem(p, need_ptrs, &why);
    if (rc != CSR_OK) return set_err(ctx, rc, why);
    if (!p.row_ptr) return set_err(ctx, CSR_ERR_NULL, "row_ptr is NULL");
    if (ctx->device < 0) return set_err(ctx, CSR_ERR_DEVICE, "host-only context");
    return CSR_OK;
}

int csr_plan_size(csr_context_t ctx, const csr_problem_t* p, size_t* plan_bytes, size_t* workspace_bytes)
{
    if (!ctx || !p || !plan_bytes || !workspace_bytes) return CSR_ERR_NULL;
    try {
        std::lock_guard<std::mutex> lk(ctx->mu);
        ctx->last_error.clear();
        int rc = check_plan_problem(ctx, *p, false);
        if (rc != CSR_OK) return rc;
        rc = check_workspace(ctx, *p, csrh::kHeadBytes);
        if (rc != CSR_OK) return rc;
        DeviceGuard g(ctx->device);
        int64_t hist[csrh::kHistInts];
        rc = histogram(ctx, *p, static_cast<hipStream_t>(p->stream), hist);
        if (rc != CSR_OK) return rc;
        plan_sizes(*p, hist, plan_bytes, workspace_bytes);
        return CSR_OK;
    } catch (...) {
        return set_err(ctx, CSR_ERR_INTERNAL, "internal error");
    }
}

namespace {

// A plan under construction: the problem, its histogram and the format last
// built into the plan memory.
struct PlanBuild {
    csr_context_t ctx;
    const csr_problem_t& p;
    const int64_t* hist;
    void* mem;
    hipStream_t st;
    int built_P = -1, built_T = -1;  // the layout in the plan memory: parts (0: degree classes), threshold
    csr_hybrid_t h{};
    float* hv = nullptr;  // SpMM: the plan's values in format order
    csr_bucket_t bk{};    // degree classes, when built

    PlanBuild(csr_context_t c, const csr_problem_t& pr, const int64_t* hi, void* m)
        : ctx(c), p(pr), hist(hi), mem(m), st(static_cast<hipStream_t>(pr.stream))
    {
    }

    // builds the format (P, T) into the plan memory (kept if already there)
    // and moves the values into its order (ones when p has none)
    int build(int P, int T)
    {
        if (P == built_P && T == built_T) return CSR_OK;
        built_P = -1;
        h = plan_format(p, P, T, csrh::segment_bound(p, hist, P, T), mem, &hv);
        int rc = build_format(ctx, p.row_ptr, p.col_idx, &h, p.workspace, p.workspace_bytes, st);
        if (rc != CSR_OK) return rc;
        if (hv) {
            if (p.a)
                CSR_HIP(ctx, csrk::launch_gather_values(h.perm, static_cast<const float*>(p.a), hv, p.nnz, st));
            else
                CSR_HIP(ctx, csrk::launch_fill_f32(hv, p.nnz, 1.f, st));
        }
        built_P = P;
        built_T = T;
        return CSR_OK;
    }

    // builds the degree classes of short threshold E into the plan memory
    // (kept if already there), with the values in slot and long-row order
    int build_bucket(int E)
    {
        if (built_P == 0 && built_T == E) return CSR_OK;
        built_P = -1;
        const csrh::BucketShape sh = csrh::bucket_shape(p, hist, E);
        const csrh::BucketLayout L = csrh::bucket_layout(p, sh);
        char* m = static_cast<char*>(mem);
        std::memset(&bk, 0, sizeof bk);
        bk.short_below = E;
        bk.n_classes = sh.n_classes;
        bk.n_short = sh.n_short;
        bk.n_slots = sh.n_slots;
        bk.nnz_long = sh.nnz_long;
        for (int c = 0; c < CSR_BUCKET_MAX_CLASSES; ++c) bk.class_rows[c] = sh.class_rows[c];
        bk.rows = reinterpret_cast<int32_t*>(m + L.rows);
        bk.slot_col = reinterpret_cast<int32_t*>(m + L.slot_col);
        bk.slot_pos = reinterpret_cast<int32_t*>(m + L.slot_pos);
        bk.slot_val = reinterpret_cast<float*>(m + L.slot_val);
        bk.long_row_ptr = reinterpret_cast<int32_t*>(m + L.long_row_ptr);
        bk.long_col = reinterpret_cast<int32_t*>(m + L.long_col);
        bk.long_pos = reinterpret_cast<int32_t*>(m + L.long_pos);
        bk.long_val = reinterpret_cast<float*>(m + L.long_val);
        CSR_HIP(ctx, csrk::launch_bucket_build(p.row_ptr, p.col_idx, p.n_rows, p.nnz, E, sh.n_classes, sh.class_rows,
                                               sh.class_base, sh.class_row0, bk.rows, bk.slot_col, bk.slot_pos,
                                               bk.long_row_ptr, bk.long_col, bk.long_pos, p.workspace,
                                               p.workspace_bytes, st));
        const float* v = static_cast<const float*>(p.a);  // NULL: ones
        CSR_HIP(ctx, csrk::launch_gather_or_zero(bk.slot_pos, v, bk.slot_val, bk.n_slots, st));
        CSR_HIP(ctx, csrk::launch_gather_or_zero(bk.long_pos, v, bk.long_val, bk.nnz_long, st));
        built_P = 0;
        built_T = E;
        return CSR_OK;
    }

    // the built degree classes' long rows as a problem, and the whole product
    csr_problem_t long_problem() const { return bucket_long_problem(p, bk, bk.long_val); }
    int run_bucket(const csr_schedule_t& s) { return bucket_run(ctx, p, bk, s, bk.slot_val, bk.long_val, st); }

    // the call over the built format with p's operands
    int call(HybridCall* c, const csr_schedule_t* sched)
    {
        const void* a = p.op == CSR_OP_SPMM ? static_cast<const void*>(hv) : p.a;
        return hybrid_call(ctx, &h, p.op, p.width, p.dtype, a, p.ld_a, p.b, p.ld_b, sched, p.workspace,
                           p.workspace_bytes, p.stream, static_cast<float*>(p.out), c);
    }

    int run(const HybridCall& c, const csr_schedule_t& s)
    {
        return hybrid_run(ctx, &h, c, &s, static_cast<float*>(p.out), p.ld_out);
    }
};

struct PlanOption {
    int P, T;
    csr_schedule_t s;
    double ms;
};

// The cost model's choice: the format's plan (or the plain pattern), with the
// estimated best schedule of the product.
int estimate_plan(PlanBuild& b, csrh::PlanChoice* out)
{
    int P = 1, T = 0;
    csrh::hybrid_plan(b.p, b.hist, &P, &T);
    out->parts = 1;
    out->whole_below = 0;
    auto best_of = [&](const csr_problem_t& q, const int64_t* hq) {
        const std::vector<csr_schedule_t> cand = csrh::candidates(q, hq);
        size_t bi = 0;
        double bt = 0;
        for (size_t i = 0; i < cand.size(); ++i) {
            const double t = csrh::estimate(q, cand[i], hq, b.ctx->dev);
            if (i == 0 || t < bt) {
                bt = t;
                bi = i;
            }
        }
        return cand[bi];
    };
    if (P > 1 && b.build(P, T) == CSR_OK) {
        HybridCall c;
        if (b.call(&c, nullptr) == CSR_OK) {
            int64_t hs[csrh::kHistInts];
            if (histogram(b.ctx, c.p, b.st, hs) == CSR_OK) {
                out->parts = P;
                out->whole_below = T;
                out->sched = best_of(c.p, hs);
                return CSR_OK;
            }
        }
    }
    b.ctx->last_error.clear();
    out->sched = best_of(b.p, b.hist);
    return CSR_OK;
}

// Micro-probes the plain pattern's best schedules and, for each candidate
// format, its product's best schedules (the whole call: segment product and
// the sum of the partial rows); returns the fastest option (within 1 %, the
// earlier one: plain first, then the formats in order) and its median time.
int probe_plan(PlanBuild& b, csrh::PlanChoice* out, double* ms)
{
    const int max_probe = std::max(1, env_int("CSRSA_PROBE_CANDIDATES", 6));
    auto top = [&](const csr_problem_t& q, const int64_t* hq, int k) {
        const std::vector<csr_schedule_t> cand = csrh::candidates(q, hq);
        std::vector<double> est(cand.size());
        for (size_t i = 0; i < cand.size(); ++i) est[i] = csrh::estimate(q, cand[i], hq, b.ctx->dev);
        std::vector<csr_schedule_t> r;
        for (size_t i : csrh::probe_subset(cand, est, k)) r.push_back(cand[i]);
        return r;
    };
    // first round: the plain pattern's best few schedules and, per format,
    // its best few (one of each mapping first)
    std::vector<PlanOption> opts;
    {
        const std::vector<csr_schedule_t> cand = top(b.p, b.hist, max_probe);
        const std::vector<double> t =
            probe_runs(b.ctx, cand.size(), [&](size_t i) { return run_schedule(b.ctx, b.p, cand[i], b.st); }, b.st);
        for (size_t i = 0; i < cand.size(); ++i) opts.push_back({1, 0, cand[i], t[i]});
    }
    const int per_format = std::max(1, (max_probe + 1) / 2);
    for (const auto& f : csrh::plan_formats(b.p, b.hist)) {
        if (b.build(f.first, f.second) != CSR_OK) continue;  // a format that cannot be built is not a candidate
        HybridCall c;
        if (b.call(&c, nullptr) != CSR_OK) continue;
        int64_t hs[csrh::kHistInts];
        if (histogram(b.ctx, c.p, b.st, hs) != CSR_OK) continue;
        const std::vector<csr_schedule_t> cand = top(c.p, hs, per_format);
        const std::vector<double> t = probe_runs(b.ctx, cand.size(), [&](size_t i) { return b.run(c, cand[i]); }, b.st);
        for (size_t i = 0; i < cand.size(); ++i) opts.push_back({f.first, f.second, cand[i], t[i]});
    }
    // degree classes: the long rows' best few schedules, each timed with the packed rows
    for (int E : csrh::plan_buckets(b.p, b.hist)) {
        if (b.build_bucket(E) != CSR_OK) continue;
        const csr_problem_t q = b.long_problem();
        int64_t hs[csrh::kHistInts];
        if (histogram(b.ctx, q, b.st, hs) != CSR_OK) continue;
        const std::vector<csr_schedule_t> cand = top(q, hs, per_format);
        const std::vector<double> t = probe_runs(b.ctx, cand.size(), [&](size_t i) { return b.run_bucket(cand[i]); }, b.st);
        for (size_t i = 0; i < cand.size(); ++i) opts.push_back({0, E, cand[i], t[i]});
    }
    // second round: the winning format's wider set of schedules, timed
    // together (those of the first round again among them, so that the
    // comparison is within one batch)
    {
        int wi = -1;
        for (size_t i = 0; i < opts.size(); ++i)
            if (opts[i].ms >= 0 && (wi < 0 || opts[i].ms < opts[wi].ms * 0.99)) wi = (int)i;
        if (wi >= 0 && opts[wi].P != 1 && max_probe > per_format) {
            const int P = opts[wi].P, T = opts[wi].T;
            HybridCall c;
            int64_t hs[csrh::kHistInts];
            const bool ok = P == 0 ? (b.build_bucket(T) == CSR_OK && histogram(b.ctx, b.long_problem(), b.st, hs) == CSR_OK)
                                   : (b.build(P, T) == CSR_OK && b.call(&c, nullptr) == CSR_OK &&
                                      histogram(b.ctx, c.p, b.st, hs) == CSR_OK);
            if (ok) {
                const std::vector<csr_schedule_t> cand = top(P == 0 ? b.long_problem() : c.p, hs, max_probe);
                const std::vector<double> t = probe_runs(
                    b.ctx, cand.size(), [&](size_t i) { return P == 0 ? b.run_bucket(cand[i]) : b.run(c, cand[i]); },
                    b.st);
                // the other layouts' times came from another batch: scale
                // them by the winner's ratio between the two batches
                double ratio = 1.0;
                for (size_t i = 0; i < cand.size(); ++i)
                    if (t[i] > 0 && std::memcmp(&cand[i], &opts[wi].s, sizeof(csr_schedule_t)) == 0)
                        ratio = t[i] / opts[wi].ms;
                // the winning format's options replace its first-round ones,
                // in the same place (plain first, then the formats in order:
                // the order that decides ties)
                std::vector<PlanOption> merged;
                bool placed = false;
                for (const auto& o : opts) {
                    if (o.P == P && o.T == T) {
                        if (!placed)
                            for (size_t i = 0; i < cand.size(); ++i) merged.push_back({P, T, cand[i], t[i]});
                        placed = true;
                        continue;
                    }
                    merged.push_back(o);
                    if (merged.back().ms >= 0) merged.back().ms *= ratio;
                }
                opts.swap(merged);
            }
        }
    }
    b.ctx->last_error.clear();
    (void)hipGetLastError();
    if (env_flag("CSRSA_PLAN_TRACE")) {  // every probed option on stderr, one line each
        for (const auto& o : opts)
            std::fprintf(stderr, "csrsa plan probe op=%d F=%lld parts=%d whole=%d map=%d vec=%d w=%d nv=%d chunk=%d "
                                 "long=%d flags=%d ms=%.4f\n",
                         b.p.op, (long long)b.p.width, o.P, o.T, o.s.mapping, o.s.vec, o.s.group_lanes, o.s.passes,
                         o.s.chunk_items, o.s.long_row, o.s.flags, o.ms);
    }
    double best = -1.0;
    size_t bi = 0;
    for (size_t i = 0; i < opts.size(); ++i) {
        if (opts[i].ms < 0) continue;  // guardrail: a failing option is never chosen
        if (best < 0 || opts[i].ms < best * 0.99) {
            best = opts[i].ms;
            bi = i;
        }
    }
    if (best < 0) {  // every probe failed: the plain pattern, default schedule
        out->parts = 1;
        out->whole_below = 0;
        out->sched = csrh::default_schedule(b.p);
        *ms = 0.0;
        return CSR_OK;
    }
    out->parts = opts[bi].P;
    out->whole_below = opts[bi].T;
    out->sched = opts[bi].s;
    *ms = best;
    return CSR_OK;
}

// Fills *plan for choice c (building its format when it has one).
int materialize_plan(PlanBuild& b, const csrh::PlanChoice& c, uint64_t sig, double ms, csr_plan_t* plan)
{
    std::string why;
    csr_plan_t r;
    std::memset(&r, 0, sizeof r);
    r.version = CSR_PLAN_VERSION;
    r.op = b.p.op;
    r.dtype = b.p.dtype;
    r.parts = c.parts;
    r.whole_below = c.whole_below;
    r.n_rows = b.p.n_rows;
    r.n_cols = b.p.n_cols;
    r.nnz = b.p.nnz;
    r.width = b.p.width;
    r.signature = sig;
    r.sched = c.sched;
    r.row_ptr = b.p.row_ptr;
    r.col_idx = b.p.col_idx;
    r.probe_ms = ms;
    if (c.parts == 1) {
        int rc = csrh::check_schedule(b.p, c.sched, &why);
        if (rc != CSR_OK) return set_err(b.ctx, rc, why);
        r.vals = b.p.op == CSR_OP_SPMM ? const_cast<float*>(static_cast<const float*>(b.p.a)) : nullptr;
        r.workspace_bytes = up256(csrh::workspace_bytes(b.p, c.sched));
    } else if (c.parts == 0) {
        if (b.p.op != CSR_OP_SPMM) return set_err(b.ctx, CSR_ERR_SHAPE, "degree classes serve SpMM");
        int rc = b.build_bucket(c.whole_below);
        if (rc != CSR_OK) return rc;
        const csr_problem_t q = b.long_problem();
        rc = csrh::check_schedule(q, c.sched, &why);
        if (rc != CSR_OK) return set_err(b.ctx, rc, why);
        r.bkt = b.bk;
        // the long rows' product, then room for the values of a call that
        // passes its own (moved into slot and long-row order there)
        r.workspace_bytes = up256(csrh::workspace_bytes(q, c.sched)) + up256((size_t)b.bk.n_slots * 4) +
                            up256((size_t)b.bk.nnz_long * 4);
    } else {
        int rc = b.build(c.parts, c.whole_below);
        if (rc != CSR_OK) return rc;
        HybridCall hc;
        rc = b.call(&hc, &c.sched);
        if (rc != CSR_OK) return rc;
        r.fmt = b.h;
        r.vals = b.hv;
        size_t inner = 0;
        rc = hybrid_inner_bytes(b.ctx, hc.p, &c.sched, &inner);
        if (rc != CSR_OK) return rc;
        // SpMM: the partial rows, then room for the values of a call that
        // passes its own (moved into format order there, for that call only)
        r.workspace_bytes = inner + (b.p.op == CSR_OP_SPMM ? up256((size_t)b.h.n_seg * b.p.width * 4) +
                                                                  up256((size_t)b.p.nnz * 4)
                                                            : 0);
    }
    *plan = r;
    return CSR_OK;
}

int check_plan(csr_context_t ctx, const csr_plan_t* plan, int op)
{
    if (!plan) return CSR_ERR_NULL;
    if (plan->version != CSR_PLAN_VERSION || plan->op != op)
        return set_err(ctx, CSR_ERR_SHAPE, "not a plan of this operation and library version");
    if (plan->parts == 0) {
        if (plan->op != CSR_OP_SPMM || plan->bkt.short_below != plan->whole_below || plan->bkt.n_classes < 1 ||
            plan->bkt.n_classes > CSR_BUCKET_MAX_CLASSES)
            return set_err(ctx, CSR_ERR_SHAPE, "the plan's degree classes do not match it");
    } else if (plan->parts != 1 && plan->fmt.parts != plan->parts) {
        return set_err(ctx, CSR_ERR_SHAPE, "the plan's format does not match its parts");
    }
    if (ctx->device < 0) return set_err(ctx, CSR_ERR_DEVICE, "host-only context");
    return CSR_OK;
}

}  // namespace

int csr_plan_create(csr_context_t ctx, const csr_problem_t* pp, uint32_t mode, void* plan_mem, size_t plan_bytes,
                    csr_plan_t* plan)
{
    if (!ctx || !pp || !plan) return CSR_ERR_NULL;
    try {
        std::lock_guard<std::mutex> lk(ctx->mu);
        ctx->last_error.clear();
        if (mode > CSR_SELECT_ESTIMATE) return set_err(ctx, CSR_ERR_SHAPE, "unknown selection mode");
        const csr_problem_t& p = *pp;
        int rc = check_plan_problem(ctx, p, true);
        if (rc != CSR_OK) return rc;
        rc = check_workspace(ctx, p, csrh::kHeadBytes);
        if (rc != CSR_OK) return rc;
        DeviceGuard g(ctx->device);
        hipStream_t st = static_cast<hipStream_t>(p.stream);
        int64_t hist[csrh::kHistInts];
        rc = histogram(ctx, p, st, hist);
        if (rc != CSR_OK) return rc;
        size_t need_mem = 0, need_ws = 0;
        plan_sizes(p, hist, &need_mem, &need_ws);
        if (!plan_mem || plan_bytes < need_mem || (uintptr_t)plan_mem % csrh::kAlign)
            return set_err(ctx, CSR_ERR_WORKSPACE, "plan memory NULL, unaligned or below " + std::to_string(need_mem) +
                                                       " bytes");
        rc = check_workspace(ctx, p, need_ws);
        if (rc != CSR_OK) return rc;
        const uint64_t sig = csrh::plan_signature(p, hist, ctx->dev);
        PlanBuild b(ctx, p, hist, plan_mem);
        csrh::PlanChoice c;
        double ms = 0.0;
        bool have = false;
        if (mode == CSR_SELECT_AUTO || mode == CSR_SELECT_REPLAY_ONLY) {
            auto it = ctx->plans.find(sig);
            if (it != ctx->plans.end()) {
                c = it->second.choice;
                have = true;
            } else if (mode == CSR_SELECT_REPLAY_ONLY) {
                return set_err(ctx, CSR_ERR_NO_CACHE_ENTRY, "no cached plan for this input");
            }
        }
        if (!have) {
            if (mode == CSR_SELECT_ESTIMATE || (ctx->flags & CSR_CTX_NO_PROBE)) {
                rc = estimate_plan(b, &c);
                if (rc != CSR_OK) return rc;
                if (mode != CSR_SELECT_ESTIMATE) (void)store_plan(ctx, sig, c, 0.0);
            } else {
                rc = probe_plan(b, &c, &ms);
                if (rc != CSR_OK) return rc;
                (void)store_plan(ctx, sig, c, ms * 1000.0);  // a log write failure keeps the entry in memory
            }
        }
        rc = materialize_plan(b, c, sig, ms, plan);
        if (rc == CSR_OK) ctx->last_error.clear();
        return rc;
    } catch (...) {
        return set_err(ctx, CSR_ERR_INTERNAL, "internal error");
    }
}

int csr_plan_layout_size(csr_context_t ctx, const csr_problem_t* p, int32_t parts, int32_t whole_below,
                         size_t* plan_bytes, size_t* workspace_bytes)
{
    if (!ctx || !p || !plan_bytes || !workspace_bytes) return CSR_ERR_NULL;
    try {
        std::lock_guard<std::mutex> lk(ctx->mu);
        ctx->last_error.clear();
        int rc = check_plan_problem(ctx, *p, false);
        if (rc != CSR_OK) return rc;
        if (!layout_ok(*p, parts, whole_below)) return set_err(ctx, CSR_ERR_SHAPE, "no such layout for this problem");
        rc = check_workspace(ctx, *p, csrh::kHeadBytes);
        if (rc != CSR_OK) return rc;
        DeviceGuard g(ctx->device);
        int64_t hist[csrh::kHistInts];
        rc = histogram(ctx, *p, static_cast<hipStream_t>(p->stream), hist);
        if (rc != CSR_OK) return rc;
        layout_sizes(*p, hist, parts, whole_below, plan_bytes, workspace_bytes);
        return CSR_OK;
    } catch (...) {
        return set_err(ctx, CSR_ERR_INTERNAL, "internal error");
    }
}

int csr_plan_build(csr_context_t ctx, const csr_problem_t* pp, int32_t parts, int32_t whole_below,
                   const csr_schedule_t* sched, void* plan_mem, size_t plan_bytes, csr_plan_t* plan)
{
    if (!ctx || !pp || !plan) return CSR_ERR_NULL;
    try {
        std::lock_guard<std::mutex> lk(ctx->mu);
        ctx->last_error.clear();
        const csr_problem_t& p = *pp;
        int rc = check_plan_problem(ctx, p, true);
        if (rc != CSR_OK) return rc;
        if (!layout_ok(p, parts, whole_below)) return set_err(ctx, CSR_ERR_SHAPE, "no such layout for this problem");
        rc = check_workspace(ctx, p, csrh::kHeadBytes);
        if (rc != CSR_OK) return rc;
        DeviceGuard g(ctx->device);
        hipStream_t st = static_cast<hipStream_t>(p.stream);
        int64_t hist[csrh::kHistInts];
        rc = histogram(ctx, p, st, hist);
        if (rc != CSR_OK) return rc;
        size_t need_mem = 0, need_ws = 0;
        layout_sizes(p, hist, parts, whole_below, &need_mem, &need_ws);
        if (!plan_mem || plan_bytes < need_mem || (uintptr_t)plan_mem % csrh::kAlign)
            return set_err(ctx, CSR_ERR_WORKSPACE, "plan memory NULL, unaligned or below " + std::to_string(need_mem) +
                                                       " bytes");
        rc = check_workspace(ctx, p, need_ws);
        if (rc != CSR_OK) return rc;
        PlanBuild b(ctx, p, hist, plan_mem);
        csrh::PlanChoice c;
        c.parts = parts;
        c.whole_below = parts == 1 ? 0 : whole_below;
        if (sched) {
            c.sched = *sched;
        } else if (parts == 1) {
            rc = select_locked(ctx, p, CSR_SELECT_AUTO, &c.sched, nullptr, nullptr);
        } else if (parts == 0) {
            rc = b.build_bucket(whole_below);
            if (rc == CSR_OK) rc = select_locked(ctx, b.long_problem(), CSR_SELECT_AUTO, &c.sched, nullptr, nullptr);
        } else {
            rc = b.build(parts, whole_below);
            HybridCall hc;
            if (rc == CSR_OK) rc = b.call(&hc, nullptr);
            if (rc == CSR_OK) rc = select_locked(ctx, hc.p, CSR_SELECT_AUTO, &c.sched, nullptr, &hc.maps);
        }
        if (rc != CSR_OK) return rc;
        rc = materialize_plan(b, c, csrh::plan_signature(p, hist, ctx->dev), 0.0, plan);
        if (rc == CSR_OK) ctx->last_error.clear();
        return rc;
    } catch (...) {
        return set_err(ctx, CSR_ERR_INTERNAL, "internal error");
    }
}

int csr_plan_spmm(csr_context_t ctx, const csr_plan_t* plan, const float* vals, const void* X, int64_t ldx, float* Y,
                  int64_t ldy, void* workspace, size_t ws_bytes, void* stream)
{
    if (!ctx || !plan || !X || !Y) return CSR_ERR_NULL;
    try {
        std::lock_guard<std::mutex> lk(ctx->mu);
        ctx->last_error.clear();
        int rc = check_plan(ctx, plan, CSR_OP_SPMM);
        if (rc != CSR_OK) return rc;
        DeviceGuard g(ctx->device);
        hipStream_t st = static_cast<hipStream_t>(stream);
        std::string why;
        if (plan->parts == 1) {
            csr_problem_t p = blank_problem();
            p.op = CSR_OP_SPMM;
            p.dtype = plan->dtype;
            p.n_rows = plan->n_rows;
            p.n_cols = plan->n_cols;
            p.nnz = plan->nnz;
            p.width = plan->width;
            p.ld_b = ldx;
            p.ld_out = ldy;
            p.row_ptr = plan->row_ptr;
            p.col_idx = plan->col_idx;
            p.a = vals ? vals : plan->vals;
            p.b = X;
            p.out = Y;
            p.workspace = workspace;
            p.workspace_bytes = ws_bytes;
            p.stream = stream;
            rc = csrh::check_problem(p, true, &why);
            if (rc != CSR_OK) return set_err(ctx, rc, why);
            rc = csrh::check_schedule(p, plan->sched, &why);
            if (rc != CSR_OK) return set_err(ctx, rc, why);
            rc = check_workspace(ctx, p, csrh::workspace_bytes(p, plan->sched));
            if (rc != CSR_OK) return rc;
            return run_schedule(ctx, p, plan->sched, st);
        }
        if (plan->parts == 0) {
            const csr_bucket_t& bk = plan->bkt;
            csr_problem_t p = blank_problem();
            p.op = CSR_OP_SPMM;
            p.dtype = plan->dtype;
            p.n_rows = plan->n_rows;
            p.n_cols = plan->n_cols;
            p.nnz = plan->nnz;
            p.width = plan->width;
            p.ld_b = ldx;
            p.ld_out = ldy;
            p.row_ptr = plan->row_ptr;
            p.col_idx = plan->col_idx;
            p.a = bk.long_val;
            p.b = X;
            p.out = Y;
            p.workspace = workspace;
            p.workspace_bytes = ws_bytes;
            p.stream = stream;
            rc = csrh::check_problem(p, true, &why);
            if (rc != CSR_OK) return set_err(ctx, rc, why);
            const size_t tail = up256((size_t)bk.n_slots * 4) + up256((size_t)bk.nnz_long * 4);
            if (!workspace || ws_bytes < plan->workspace_bytes || plan->workspace_bytes < tail ||
                (uintptr_t)workspace % csrh::kAlign)
                return set_err(ctx, CSR_ERR_WORKSPACE, "workspace NULL, unaligned or below the plan's workspace_bytes");
            p.workspace_bytes = plan->workspace_bytes - tail;
            const csr_problem_t q = bucket_long_problem(p, bk, bk.long_val);
            rc = csrh::check_schedule(q, plan->sched, &why);
            if (rc != CSR_OK) return set_err(ctx, rc, why);
            rc = check_workspace(ctx, q, csrh::workspace_bytes(q, plan->sched));
            if (rc != CSR_OK) return rc;
            // this call's own values go into slot and long-row order at the end of the workspace
            const float* sv = bk.slot_val;
            const float* lv = bk.long_val;
            if (vals) {
                char* t = static_cast<char*>(workspace) + plan->workspace_bytes - tail;
                float* s2 = reinterpret_cast<float*>(t);
                float* l2 = reinterpret_cast<float*>(t + up256((size_t)bk.n_slots * 4));
                CSR_HIP(ctx, csrk::launch_gather_or_zero(bk.slot_pos, vals, s2, bk.n_slots, st));
                CSR_HIP(ctx, csrk::launch_gather_or_zero(bk.long_pos, vals, l2, bk.nnz_long, st));
                sv = s2;
                lv = l2;
            }
            return bucket_run(ctx, p, bk, plan->sched, sv, lv, st);
        }
        if (plan->width < 1 || ldy < plan->width || ldy >= ((int64_t)1 << 30))
            return set_err(ctx, CSR_ERR_SHAPE, "bad width or ldy");
        if (!plan->vals) return set_err(ctx, CSR_ERR_NULL, "the plan has no value array");
        if (!workspace || ws_bytes < plan->workspace_bytes || (uintptr_t)workspace % csrh::kAlign)
            return set_err(ctx, CSR_ERR_WORKSPACE, "workspace NULL, unaligned or below the plan's workspace_bytes");
        // this call's own values go into format order at the end of the workspace
        const float* fv = plan->vals;
        if (vals) {
            float* tmp = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan->workspace_bytes -
                                                  up256((size_t)plan->nnz * 4));
            CSR_HIP(ctx, csrk::launch_gather_values(plan->fmt.perm, vals, tmp, plan->nnz, st));
            fv = tmp;
        }
        HybridCall c;
        rc = hybrid_call(ctx, &plan->fmt, CSR_OP_SPMM, plan->width, plan->dtype, fv, 0, X, ldx, &plan->sched,
                         workspace, plan->workspace_bytes - up256((size_t)plan->nnz * 4), stream, nullptr, &c);
        if (rc != CSR_OK) return rc;
        return hybrid_run(ctx, &plan->fmt, c, &plan->sched, Y, ldy);
    } catch (...) {
        return set_err(ctx, CSR_ERR_INTERNAL, "internal error");
    }
}

int csr_plan_sddmm(csr_context_t ctx, const csr_plan_t* plan, const void* U, int64_t ldu, const void* V, int64_t ldv,
                   float* out, void* workspace, size_t ws_bytes, void* stream)
{
    if (!ctx || !plan) return CSR_ERR_NULL;
    try {
        std::lock_guard<std::mutex> lk(ctx->mu);
        ctx->last_error.clear();
        int rc = check_plan(ctx, plan, CSR_OP_SDDMM);
        if (rc != CSR_OK) return rc;
        DeviceGuard g(ctx->device);
        hipStream_t st = static_cast<hipStream_t>(stream);
        std::string why;
        if (plan->parts == 1) {
            csr_problem_t p = blank_problem();
            p.op = CSR_OP_SDDMM;
            p.dtype = plan->dtype;
            p.n_rows = plan->n_rows;
            p.n_cols = plan->n_cols;
            p.nnz = plan->nnz;
            p.width = plan->width;
            p.ld_a = ldu;
            p.ld_b = ldv;
            p.row_ptr = plan->row_ptr;
            p.col_idx = plan->col_idx;
            p.a = U;
            p.b = V;
            p.out = out;
            p.workspace = workspace;
            p.workspace_bytes = ws_bytes;
            p.stream = stream;
            rc = csrh::check_problem(p, true, &why);
            if (rc != CSR_OK) return set_err(ctx, rc, why);
            rc = csrh::check_schedule(p, plan->sched, &why);
            if (rc != CSR_OK) return set_err(ctx, rc, why);
            rc = check_workspace(ctx, p, csrh::workspace_bytes(p, plan->sched));
            if (rc != CSR_OK) return rc;
            return run_schedule(ctx, p, plan->sched, st);
        }
        HybridCall c;
        rc = hybrid_call(ctx, &plan->fmt, CSR_OP_SDDMM, plan->width, plan->dtype, U, ldu, V, ldv, &plan->sched,
                         workspace, ws_bytes, stream, out, &c);
        if (rc != CSR_OK) return rc;
        return hybrid_run(ctx, &plan->fmt, c, &plan->sched, nullptr, 0);
    } catch (...) {
        return set_err(ctx, CSR_ERR_INTERNAL, "internal error");
    }
}

int csr_select(csr_context_t ctx, const csr_problem_t* p, uint32_t mode, csr_schedule_t* out, uint64_t* signature)
{
    if (!ctx || !p || !out) return CSR_ERR_NULL;
    std::lock_guard<std::mutex> lk(ctx->mu);
    ctx->last_error.clear();
    if (mode > CSR_SELECT_ESTIMATE) return set_err(ctx, CSR_ERR_SHAPE, "unknown selection mode");
    try {
        DeviceGuard g(ctx->device);
        return select_locked(ctx, *p, mode, out, signature);
    } catch (...) {
        return set_err(ctx, CSR_ERR_INTERNAL, "internal error");
    }
}

int csr_default_schedule(csr_context_t ctx, const csr_problem_t* p, csr_schedule_t* out)
{
    if (!p || !out) return CSR_ERR_NULL;
    CtxLock lk(ctx);
    std::string why;
    int rc = csrh::check_problem(*p, false, &why);
    if (rc != CSR_OK) return set_err(ctx, rc, why);
    *out = csrh::default_schedule(*p);
    return CSR_OK;
}

int csr_hybrid_parts(csr_context_t ctx, const csr_problem_t* p, const int64_t* histogram, int32_t* parts)
{
    return csr_hybrid_plan(ctx, p, histogram, parts, nullptr);
}

int csr_hybrid_plan(csr_context_t ctx, const csr_problem_t* p, const int64_t* histogram, int32_t* parts,
                    int32_t* whole_below)
{
    if (!p || !parts) return CSR_ERR_NULL;
    CtxLock lk(ctx);
    std::string why;
    int rc = csrh::check_problem(*p, false, &why);
    if (rc != CSR_OK) return set_err(ctx, rc, why);
    int P = 1, T = 0;
    csrh::hybrid_plan(*p, histogram, &P, &T);
    *parts = P;
    if (whole_below) *whole_below = T;
    return CSR_OK;
}

int csr_candidates(csr_context_t ctx, const csr_problem_t* p, const int64_t* histogram, csr_schedule_t* out,
                   int32_t max, int32_t* n)
{
    if (!p || !n || (max > 0 && !out)) return CSR_ERR_NULL;
    CtxLock lk(ctx);
    std::string why;
    int rc = csrh::check_problem(*p, false, &why);
    if (rc != CSR_OK) return set_err(ctx, rc, why);
    const std::vector<csr_schedule_t> c = csrh::candidates(*p, histogram);
    *n = (int32_t)c.size();
    for (int32_t i = 0; i < max && i < (int32_t)c.size(); ++i) out[i] = c[i];
    return CSR_OK;
}

int csr_workspace_size(csr_context_t ctx, const csr_problem_t* p, const csr_schedule_t* sched, size_t* bytes)
{
    if (!p || !bytes) return CSR_ERR_NULL;
    CtxLock lk(ctx);
    std::string why;
    int rc = csrh::check_problem(*p, false, &why);
    if (rc != CSR_OK) return set_err(ctx, rc, why);
    if (sched) {
        rc = csrh::check_schedule(*p, *sched, &why);
        if (rc != CSR_OK) return set_err(ctx, rc, why);
        *bytes = csrh::workspace_bytes(*p, *sched);
    } else {
        *bytes = auto_workspace(*p);
    }
    return CSR_OK;
}

int csr_cache_flush(csr_context_t ctx)
{
    if (!ctx) return CSR_ERR_NULL;
    std::lock_guard<std::mutex> lk(ctx->mu);
    if (ctx->cache_path.empty()) return CSR_OK;
    int rc = CSR_OK;
    for (auto& kv : ctx->cache) {
        if (kv.second.persisted) continue;
        if (append_line(ctx->cache_path, csrh::format_cache_line(kv.first, kv.second.sched, kv.second.probe_us)))
            kv.second.persisted = true;
        else
            rc = CSR_ERR_CACHE_IO;
    }
    for (auto& kv : ctx->plans) {
        if (kv.second.persisted) continue;
        if (append_line(ctx->cache_path, csrh::format_plan_line(kv.first, kv.second.choice, kv.second.probe_us)))
            kv.second.persisted = true;
        else
            rc = CSR_ERR_CACHE_IO;
    }
    return rc;
}

int csr_cache_info(csr_context_t ctx, int64_t* entries, int64_t* skipped_lines, int64_t* io_errors)
{
    if (!ctx) return CSR_ERR_NULL;
    std::lock_guard<std::mutex> lk(ctx->mu);
    if (entries) *entries = (int64_t)(ctx->cache.size() + ctx->plans.size());
    if (skipped_lines) *skipped_lines = ctx->skipped_lines;
    if (io_errors) *io_errors = ctx->io_errors;
    return CSR_OK;
}

int csr_cache_lookup(csr_context_t ctx, uint64_t signature, csr_schedule_t* out)
{
    if (!ctx || !out) return CSR_ERR_NULL;
    std::lock_guard<std::mutex> lk(ctx->mu);
    auto it = ctx->cache.find(signature);
    if (it == ctx->cache.end()) return CSR_ERR_NO_CACHE_ENTRY;
    *out = it->second.sched;
    return CSR_OK;
}

int csr_cache_store(csr_context_t ctx, uint64_t signature, const csr_schedule_t* sched)
{
    if (!ctx || !sched) return CSR_ERR_NULL;
    std::lock_guard<std::mutex> lk(ctx->mu);
    if (sched->version != CSR_SCHEDULE_VERSION || sched->op < CSR_OP_SPMM || sched->op > CSR_OP_SPMM_SDDMM)
        return set_err(ctx, CSR_ERR_SCHEDULE, "not a schedule of this library version");
    return store_entry(ctx, signature, *sched, 0.0);
}

int csr_degree_histogram(csr_context_t ctx, int64_t n_rows, const int32_t* row_ptr, int64_t* out_host,
                         void* workspace, size_t ws_bytes, void* stream)
{
    if (!ctx || !row_ptr || !out_host) return CSR_ERR_NULL;
    try {
        std::lock_guard<std::mutex> lk(ctx->mu);
        if (ctx->device < 0) return set_err(ctx, CSR_ERR_DEVICE, "host-only context");
        if (n_rows < 0 || n_rows >= ((int64_t)1 << 31) - 1) return set_err(ctx, CSR_ERR_SHAPE, "bad n_rows");
        csr_problem_t p = blank_problem();
        p.n_rows = n_rows;
        p.row_ptr = row_ptr;
        p.workspace = workspace;
        p.workspace_bytes = ws_bytes;
        int rc = check_workspace(ctx, p, csrh::kHeadBytes);
        if (rc != CSR_OK) return rc;
        DeviceGuard g(ctx->device);
        return histogram(ctx, p, static_cast<hipStream_t>(stream), out_host);
    } catch (...) {
        return set_err(ctx, CSR_ERR_INTERNAL, "internal error");
    }
}

int csr_merge_path_partition(csr_context_t ctx, int64_t n_rows, int64_t nnz, const int32_t* row_ptr,
                             int32_t items_per_chunk, int32_t* coords, void* stream)
{
    if (!ctx || !row_ptr || !coords) return CSR_ERR_NULL;
    std::lock_guard<std::mutex> lk(ctx->mu);
    if (ctx->device < 0) return set_err(ctx, CSR_ERR_DEVICE, "host-only context");
    const int64_t lim = (int64_t)1 << 31;
    if (n_rows < 0 || nnz < 0 || n_rows >= lim - 1 || nnz >= lim || items_per_chunk < 1)
        return set_err(ctx, CSR_ERR_SHAPE, "bad sizes");
    DeviceGuard g(ctx->device);
    const int64_t total = n_rows + nnz;
    int64_t nc = (total + items_per_chunk - 1) / items_per_chunk;
    if (nc < 1) nc = 1;
    CSR_HIP(ctx, csrk::launch_merge_path(row_ptr, n_rows, nnz, items_per_chunk, nc, coords,
                                         static_cast<hipStream_t>(stream)));
    return CSR_OK;
}

int csr_signature(csr_context_t ctx, const csr_problem_t* p, const int64_t* histogram, uint64_t* signature)
{
    if (!p || !histogram || !signature) return CSR_ERR_NULL;
    csrh::DeviceInfo dev;
    if (ctx) dev = ctx->dev;
    *signature = csrh::signature(*p, histogram, dev);
    return CSR_OK;
}

}  // extern "C"
