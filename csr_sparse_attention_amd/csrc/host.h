// Host-side runtime: problem checks, lane layouts, workspace layout, schedule
// validation, signature and cost model.  Nothing here touches the GPU, so the
// selector logic can be exercised on a machine without one.
#pragma once

#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/csrsa.h"

namespace csrh {

constexpr int kLibVersion = 1;
constexpr int kHistInts = 67;    // counts[33], sums[33], max degree
constexpr size_t kAlign = 256;   // workspace region alignment
constexpr size_t kHeadBytes = 1024;  // workspace head: histogram / validation scratch

struct DeviceInfo {
    int cu_count = 0;   // 0 for a host-only context
    int arch = 0;       // 950 for gfx950, 0 unknown
};

// Largest fp32 vector width (1, 2, 4) that the operands' alignment allows.
int max_vec_f32(const csr_problem_t& p);
// Largest bf16 vector width (2, 4, 8; 0 if none) that the operands allow.
int max_vec_bf16(const csr_problem_t& p);
// The widest lane access for p's element type.
int max_vec(const csr_problem_t& p);

// Checks the shape, dtype and pointer fields of p for its op.  need_ptrs:
// operand pointers must be non-null.  Returns CSR_OK or an error code and a
// message in *why.
int check_problem(const csr_problem_t& p, bool need_ptrs, std::string* why);

// The natural lane layout of a row of `width` fp32 values read `vec` at a
// time: W = lanes per group, nv = passes.  Returns false if unsupported.
bool natural_layout(int64_t width, int vec, int* W, int* nv);

// Validates schedule s against problem p (CSR_OK or CSR_ERR_SCHEDULE + why).
int check_schedule(const csr_problem_t& p, const csr_schedule_t& s, std::string* why);

// Bytes of workspace needed by schedule s (s must be valid for p).
size_t workspace_bytes(const csr_problem_t& p, const csr_schedule_t& s);

// Merge-path chunk count for items_per_chunk.
int64_t n_chunks_for(const csr_problem_t& p, int items_per_chunk);

// Workspace regions of a merge-path schedule.
struct WsLayout {
    size_t coords, carry_row, carry_ml, carry_val, bounds, total;
    int64_t n_chunks;
};
WsLayout ws_layout(const csr_problem_t& p, const csr_schedule_t& s);

// The safe default schedule (the guardrail's fallback).
csr_schedule_t default_schedule(const csr_problem_t& p);

// Candidate schedules for the auto path, in fixed priority order (the first
// is the default).  hist may be null (no degree information).
std::vector<csr_schedule_t> candidates(const csr_problem_t& p, const int64_t* hist);

// Cost-model estimate (arbitrary time units, lower is better) of schedule s
// on problem p with degree histogram hist.
double estimate(const csr_problem_t& p, const csr_schedule_t& s, const int64_t* hist, const DeviceInfo& dev);

// The candidates to micro-probe, at most k of them: the best-estimated
// candidate of each mapping first (the cost model ranks schedules of one
// mapping more reliably than it ranks mappings against each other), then the
// rest in estimate order.  Returned as indices into cand, ascending.
std::vector<size_t> probe_subset(const std::vector<csr_schedule_t>& cand, const std::vector<double>& est, int k);

// FNV-1a 64 signature of (problem shape, alignment class, histogram, device).
uint64_t signature(const csr_problem_t& p, const int64_t* hist, const DeviceInfo& dev);

// Column parts and whole-row threshold of the column-part segment format
// expected to be fastest for problem p (parts 1: the plain CSR path); see
// hybrid_plan in host.cpp.
void hybrid_plan(const csr_problem_t& p, const int64_t* hist, int* parts, int* whole_below);
int hybrid_parts(const csr_problem_t& p, const int64_t* hist);

// Cache log line format.
std::string format_cache_line(uint64_t sig, const csr_schedule_t& s, double probe_us);
bool parse_cache_line(const std::string& line, uint64_t* sig, csr_schedule_t* s, double* probe_us);

// Planned products (a CSR matrix prepared for one SpMM / SDDMM): the joint
// choice of layout (plain CSR, the column-part segment format with its
// parts and whole-row threshold, or the degree classes with their short
// threshold) and of the product's schedule.
struct PlanChoice {
    int parts = 1;        // 1: the plain pattern; 0: degree classes
    int whole_below = 0;  // the format's whole-row threshold, or the classes' short threshold
    csr_schedule_t sched{};
};

// Signature of a planned problem: the plain signature's fields under a
// marker of its own, so plans and plain schedules never share a key.
uint64_t plan_signature(const csr_problem_t& p, const int64_t* hist, const DeviceInfo& dev);

// Upper bound of the segment count of the format with P parts and rows under
// T entries kept whole, from the degree histogram: a whole row is one
// segment, a split row of degree d at most min(d, P).
int64_t segment_bound(const csr_problem_t& p, const int64_t* hist, int P, int T);

// The formats a plan probes beside the plain pattern: the cost model's
// choice, half and twice its parts, and its parts with every row split; with
// the plain pattern chosen by the model, 4 and 16 parts when one part of the
// gathered operand would still hold at least 2 MiB.  (parts, whole_below) pairs.
std::vector<std::pair<int, int>> plan_formats(const csr_problem_t& p, const int64_t* hist);

// Degree classes with short threshold E (a power of two, 2 .. 64): the shape
// from the degree histogram (class c = bucket c of the histogram, degrees
// [2^(c-1), 2^c), padded to 2^c - 1 slots).
struct BucketShape {
    int E = 0, n_classes = 0;
    int64_t class_rows[CSR_BUCKET_MAX_CLASSES] = {0};
    int64_t class_base[CSR_BUCKET_MAX_CLASSES] = {0};  // first slot of each class
    int64_t class_row0[CSR_BUCKET_MAX_CLASSES] = {0};  // first packed row of each class
    int64_t n_short = 0, n_slots = 0, nnz_short = 0, nnz_long = 0;
};
BucketShape bucket_shape(const csr_problem_t& p, const int64_t* hist, int E);

// Plan memory of the degree classes: rows, slot columns, slot entries, slot
// values, the long rows' row_ptr, columns, entries and values (byte offsets).
struct BucketLayout {
    size_t rows, slot_col, slot_pos, slot_val, long_row_ptr, long_col, long_pos, long_val, total;
};
BucketLayout bucket_layout(const csr_problem_t& p, const BucketShape& b);

// The short thresholds a plan of p weighs (SpMM only): 8 and 32 where at
// least a quarter of the rows are nonempty and shorter, those rows hold at
// least a tenth of the entries (the long rows' product dominates otherwise),
// and padding stays under one slot per entry.
std::vector<int> plan_buckets(const csr_problem_t& p, const int64_t* hist);

std::string format_plan_line(uint64_t sig, const PlanChoice& c, double probe_us);
bool parse_plan_line(const std::string& line, uint64_t* sig, PlanChoice* c, double* probe_us);

}  // namespace csrh
