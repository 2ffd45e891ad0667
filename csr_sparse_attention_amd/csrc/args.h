// Kernel argument blocks (plain data, passed by value as kernel arguments).
#pragma once

#include <stdint.h>

namespace csrk {

struct Fp32Args {
    const int32_t* row_ptr;
    const int32_t* col_idx;
    int64_t n_rows;
    const float* ev;   // per-entry input: SpMM values (may be null = 1) or attention scores
    const void* U;     // SDDMM row operand (fp32 or bf16, as the gathered operand)
    int64_t ldu;
    const void* X;     // gathered operand: SpMM X, attention node_value, SDDMM V (fp32 or bf16)
    int64_t ldx;
    float* Y;          // output rows (SpMM, attention) or per-entry output (SDDMM)
    int64_t ldy;
    int32_t F;         // feature width (K for SDDMM)
    int32_t W;         // lanes per group, power of two
    float scale;       // attention score scale
    int32_t long_row;  // merge path: whole-wave threshold
    const int32_t* part;  // merge path: (x, y) per chunk boundary
    int64_t n_chunks;
    int32_t* carry_row;   // [2 n_chunks]: row of slot A / slot B, -1 if empty
    float* carry_ml;      // [2 n_chunks][2]: attention piece (max, sum of exp)
    float* carry_val;     // [2 n_chunks][F]
    // SDDMM on the column-part segment format: U row of each pattern row
    // (its segment's row) and output slot of each entry (its original
    // position); null = the row / entry itself
    const int32_t* u_row;
    const int32_t* out_idx;
    int32_t stream_y;  // SpMM output rows by non-temporal stores (partial rows of the format)
    // attention from queries and keys: U = Q (ldu), X = K (ldx), V = values (ldv)
    const void* V;
    int64_t ldv;
    // attention: the probabilities of the entries (null = not wanted), entry e
    // at probs[e * probs_stride]
    float* probs;
    int64_t probs_stride;
    // SpMM: entry e's value is ev[ev_idx[e]] (null: ev[e])
    const int32_t* ev_idx;
    // SpMM + SDDMM on one pattern (Op::Dual): U the row operand (ldu), Y the
    // SpMM's rows, Z the SDDMM's per-entry output, written at Z[out_idx[e]]
    // (null: Z[e])
    float* Z;
};

// SpMM over the packed short rows of the degree classes (class c = 0 .. 5
// holds rows of 2^c .. 2^(c+1) - 1 entries, 2^(c+1) - 1 slots each, slot j of
// its row i at slot index base[c] + j * rows[c] + i)
struct BucketArgs {
    const int32_t* rows;      // packed rows, class by class
    const int32_t* slot_col;  // -1: padding
    const float* slot_val;
    int32_t n_classes;
    int32_t F;
    int32_t W;                // lanes per row group
    int32_t pad_;
    int64_t cls_rows[6];
    int64_t cls_base[6];
    int64_t cls_row0[6];
    int64_t cls_block0[7];    // first workgroup of each class; [n_classes] = the grid
    const void* X;
    int64_t ldx;
    float* Y;
    int64_t ldy;
};

struct MhaArgs {
    const int32_t* row_ptr;
    const int32_t* col_idx;
    int64_t n_rows;
    const uint16_t* Q;
    const uint16_t* K;
    const uint16_t* V;
    int32_t H, Dh;
    float scale;
    float* out;
    const int32_t* part;
    int64_t n_chunks;
    int32_t* carry_row;  // [2 n_chunks]
    float* carry_ml;     // [2 n_chunks][H][2]
    float* carry_val;    // [2 n_chunks][H * Dh]
    float* probs;        // [nnz][H] probabilities of the entries per head, or null
};

struct SoftmaxArgs {
    const int32_t* row_ptr;
    int64_t n_rows;
    const float* scores;  // [nnz] (the backward: the probabilities p)
    const float* grad;    // [nnz] the backward's incoming gradient g, else unused
    float scale;
    float* probs;         // [nnz]
    int32_t W;            // lanes per group for short rows
    int32_t long_row;     // whole-wave threshold
    const int32_t* part;
    const int32_t* bounds;  // [n_chunks + 1][2]: entry range of the row at each chunk boundary
    int64_t n_chunks;
    int32_t* carry_row;   // [2 n_chunks]
    float* carry_ml;      // [2 n_chunks][2]
    float* stats;         // [n_rows][2]: row maximum, sum of exponentials
};

}  // namespace csrk
