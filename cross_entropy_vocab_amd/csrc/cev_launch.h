// cev_launch.h -- host-side launchers between the C ABI (api.cpp) and the
// kernels.  Arguments arrive validated; each launcher only enqueues work and
// returns the hipError_t of the launch.  Internal to libcevocab.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cevocab.h"

namespace cev {

// Everything a forward sweep needs for one call.  Row selection: when rowlist
// is non-null the block index b maps to row rowlist[b] for b < *nlist (the
// compacted sparse-supervision path); otherwise block b is row b.
struct SweepArgs {
    const void *logits;
    int64_t rows;
    int64_t vocab;
    int64_t row_stride;        // elements
    const int64_t *labels;     // single-target sweeps
    const int64_t *indices;    // top-K sweeps: [rows, K]
    int64_t K;
    int64_t index_row_stride;
    int64_t ignore_index;
    const uint8_t *row_mask;
    const int64_t *rowlist;    // rows to sweep (compacted), or null for every row
    const int64_t *nlist;
    int64_t *out_list;         // every-row sweeps only: if set, compaction workgroups
    int64_t *out_count;        //   appended to the grid write the valid rows here
    int swizzle;               // every-row sweeps: block b takes row swizzle_row(b)
    int64_t splits;            // workgroups per row (1 = whole rows); needs partials
    void *partials;            // [rows * splits] SplitPartial, device scratch
    double temperature;
    double label_smoothing;    // eps in [0, 1]; ce_forward only
    float c;                   // log2(e) / T, rounded to fp32
    float inv_t;               // 1 / T, rounded to fp32
    float *logp;               // [rows] or [rows, K]
    float *q;                  // top-K: [rows, K] 1 - p at each gathered index, or null
    float *loss;
    float *entropy;
    int64_t *argmax;
    cev_saved *saved;
    int32_t *status;
};

// Statistics of one part of a row split over several workgroups.
struct SplitPartial {
    float m;                   // largest non-target stored logit of the part, -inf if none
    int32_t pad;
    int64_t arg;               // lowest non-target column holding m (INT64_MAX if none)
    double s;                  // sum of e^{(z - b)/T}, b = max(m, -FLT_MAX)
    double h;                  // sum of e^{(z - b)/T} (b - z)/T
    double zs;                 // sum of the part's non-target stored values
};

// Launch shape for a row of nvec 16-byte vectors.  512 threads x 2 vectors
// was the fastest shape measured on MI355X for 152064-wide bf16 rows (6.7 TB/s
// of the ~7.0 TB/s streaming-read ceiling); on 32768-wide bf16 rows (4096
// vectors) 256 x 2 beat it, 50 against 55-58 us for 4096 rows, as more rows
// in flight hide each row's closing step.  256 x 4 is not offered: the
// compiler gives that instantiation over 256 registers per lane (one wave per
// SIMD), and it measured at half the rate.
struct Shape {
    int block, U;
};

inline Shape pick_shape(int64_t nvec)
{
    if (nvec >= 8192)
        return {512, 2};
    if (nvec >= 4096)
        return {256, 2};
    if (nvec >= 4 * 128 * 4)
        return {128, 4};
    return {64, 4};
}

// Workgroups per row for the split forward: enough workgroups to fill the
// chip when rows are few (< 128), each part at least 2048 16-byte vectors.
int64_t sweep_splits(int64_t rows, int64_t vocab, int dtype);

struct CompactArgs {
    int64_t rows;
    int64_t vocab;
    const int64_t *labels;
    int64_t ignore_index;
    const uint8_t *row_mask;
    int64_t *rowlist;          // out [rows]
    int64_t *nlist;            // out [1]
    float *logp;
    float *loss;
    float *entropy;
    int64_t *argmax;
    cev_saved *saved;
    int32_t *status;
};

struct BackwardArgs {
    const void *logits;
    int64_t rows;
    int64_t vocab;             // columns held here (a shard's width for the vocab-parallel form)
    int64_t row_stride;
    int64_t col_offset;        // global column of element 0 (0 unless vocab-parallel)
    int64_t vocab_total;       // full vocabulary width: label range and eps / V
    const int64_t *labels;
    int64_t ignore_index;
    const uint8_t *row_mask;
    const float *g;
    const cev_saved *saved;
    void *dlogits;
    int64_t d_row_stride;
    double temperature;
    double label_smoothing;    // eps in [0, 1]
    float c;                   // log2(e) / T
    float inv_t;               // 1 / T
    float eps;                 // label_smoothing as fp32
    float eps_over_v;          // label_smoothing / vocab_total, rounded once to fp32
    int32_t *status;
};

// Top-K backward (gradient of sum_k g_k log p_{i_k}).
constexpr int kMaxTopK = 1024;
struct TopkBackwardArgs {
    const void *logits;
    int64_t rows;
    int64_t vocab;
    int64_t row_stride;
    const int64_t *indices;    // [rows, K], row stride index_row_stride
    int64_t K;
    int64_t index_row_stride;
    int64_t ignore_index;
    const uint8_t *row_mask;
    const float *g;            // [rows, K] dense
    const cev_saved *saved;    // from sls_topk_forward: m_z, log2 d
    const float *q;            // [rows, K] from sls_topk_forward: 1 - p at each index
    void *dlogits;
    int64_t d_row_stride;
    float c;                   // log2(e) / T
    float inv_t;               // 1 / T
    int32_t *status;
};

hipError_t launch_topk_backward(int dtype, const TopkBackwardArgs &a, hipStream_t stream);
// The lane-held tile form (K <= 64, rows of whole aligned 16-byte vectors), for
// tuning harnesses; hipErrorInvalidValue where it does not apply.
hipError_t launch_topk_backward_tile_cfg(int dtype, const TopkBackwardArgs &a, int block, int U,
                                         hipStream_t stream);

// Vocab-parallel shard sweep: one partial record per row over one shard.
struct ShardArgs {
    const void *logits;
    int64_t rows;
    int64_t vocab;             // the shard's width
    int64_t row_stride;
    int64_t col_offset;
    int64_t vocab_total;
    const int64_t *labels;
    int64_t ignore_index;
    const uint8_t *row_mask;
    float c;                   // log2(e) / T
    float inv_t;               // 1 / T
    cev_vocab_partial *partials;
    int32_t *status;
};

// Merge of P shards' partial records, then the closing step.
struct MergeArgs {
    const cev_vocab_partial *partials;  // [parts][rows]
    int64_t parts;
    int64_t rows;
    int64_t vocab;             // full width
    const int64_t *labels;
    int64_t ignore_index;
    const uint8_t *row_mask;
    double temperature;
    double label_smoothing;
    float *loss;
    float *logp;
    float *entropy;
    int64_t *argmax;
    cev_saved *saved;
    int32_t *status;
};

hipError_t launch_shard_sweep(int dtype, const ShardArgs &a, bool want_entropy, bool want_zsum,
                              hipStream_t stream);
hipError_t launch_vocab_merge(const MergeArgs &a, hipStream_t stream);

// Linear cross-entropy: logits = hidden x head^T on the matrix cores.
struct LceArgs {
    const unsigned short *hidden;   // [rows, ldh] bf16
    int64_t rows;
    int64_t hidden_dim;             // multiple of 64
    int64_t ldh;                    // multiple of 8
    const unsigned short *weight;   // head [vocab, ldw] bf16
    int64_t vocab;
    int64_t ldw;                    // multiple of 8
    const int64_t *labels;
    int64_t ignore_index;
    const uint8_t *row_mask;
    double temperature;
    double label_smoothing;
    float c;                        // log2(e) / T
    float inv_t;                    // 1 / T
    int64_t splits;                 // vocab splits (workgroups per row block)
    cev_vocab_partial *partials;    // forward: [splits][rows]
    const float *g;                 // backward: [rows]
    const cev_saved *saved;         // backward: [rows]
    unsigned short *dlogits;        // backward: [dl_rows, ldd] bf16 scratch
    int64_t ldd;                    // multiple of 64, >= vocab
    int64_t dl_rows;                // rows of dlogits written (>= rows; rows past rows are zero)
    float *logits_out;              // forward: if set, the fp32 logits [rows, ldl] are stored here
    const float *logits_in;         // backward: if set, dlogits come from these stored logits
    int64_t ldl;                    // row stride of the stored logits, a multiple of 4, >= vocab
    int32_t *status;
};

int64_t lce_splits(int64_t rows, int64_t vocab);
int64_t lce_dl_stride(int64_t vocab);
hipError_t launch_lce_forward(const LceArgs &a, bool want_entropy, bool want_zsum,
                              hipStream_t stream);
size_t lce_backward_workspace(int64_t rows, int64_t hidden_dim, int64_t vocab);
hipError_t launch_lce_backward(const LceArgs &a, void *workspace, float *dhidden,
                               int64_t dhidden_stride, float *dweight, int64_t dweight_stride,
                               hipStream_t stream);

// Generalized JSD / KL between a student and a teacher row (one workgroup
// per row).
struct JsdArgs {
    const void *student;
    const void *teacher;
    int64_t rows;
    int64_t vocab;
    int64_t s_stride;          // elements
    int64_t t_stride;
    const int64_t *labels;     // nullable: label == ignore_index masks the row
    int64_t ignore_index;
    const uint8_t *row_mask;
    double beta;               // in [0, 1]
    float c;                   // log2(e) / T
    float inv_t;               // 1 / T
    float *loss;               // forward
    cev_jsd_saved *saved;      // forward
    const cev_jsd_saved *saved_in;   // backward
    const float *g;            // backward
    void *dstudent;            // backward
    int64_t d_stride;
    int vec;                   // every row of every operand 16-byte aligned: vector path
    int32_t *status;
};

hipError_t launch_jsd_forward(int dtype, const JsdArgs &a, hipStream_t stream);
hipError_t launch_jsd_backward(int dtype, const JsdArgs &a, hipStream_t stream);
hipError_t launch_jsd_tiles_cfg(int dtype, const JsdArgs &a, int block, int U, hipStream_t stream);

// Forward + backward in one call, one workgroup per row (rows 16-byte aligned).
struct FusedArgs {
    const void *logits;
    int64_t rows;
    int64_t vocab;
    int64_t row_stride;        // elements; rows start 16-byte aligned
    const int64_t *labels;
    int64_t ignore_index;
    const uint8_t *row_mask;
    const float *g;
    double temperature;
    double label_smoothing;    // eps in [0, 1]
    float c;                   // log2(e) / T
    float inv_t;               // 1 / T
    float *loss;
    float *logp;
    float *entropy;
    int64_t *argmax;
    cev_saved *saved;
    void *dlogits;
    int64_t d_row_stride;      // elements; rows start 16-byte aligned
    int32_t *status;
};

hipError_t launch_fused(int dtype, const FusedArgs &a, bool want_entropy, hipStream_t stream);

hipError_t launch_sls_sweep(int dtype, const SweepArgs &a, bool want_entropy, bool want_argmax,
                            hipStream_t stream);
hipError_t launch_topk_sweep(int dtype, const SweepArgs &a, hipStream_t stream);
hipError_t launch_compact(const CompactArgs &a, hipStream_t stream);
hipError_t launch_backward(int dtype, const BackwardArgs &a, hipStream_t stream);

// Explicit launch configurations (workgroup size, 16-byte vectors per thread
// per step, and for the backward the steps per workgroup, 0 = a whole row,
// and the tile order: 0 row order, 1 rows from the last, 2 XCD-contiguous).
// The entry points above pick one of these; tuning harnesses call them directly.
hipError_t launch_sls_sweep_cfg(int dtype, const SweepArgs &a, bool want_entropy,
                                bool want_argmax, int block, int U, hipStream_t stream);
hipError_t launch_sls_sweep_lds_cfg(int dtype, const SweepArgs &a, bool want_entropy,
                                    bool want_argmax, int block, int U, size_t lds,
                                    hipStream_t stream);
hipError_t launch_backward_cfg(int dtype, const BackwardArgs &a, int block, int U, int iters,
                               int order, int store_nt, hipStream_t stream);
hipError_t launch_backward_tile_cfg(int dtype, const BackwardArgs &a, int block, int U, int store_nt,
                                    hipStream_t stream);
hipError_t launch_topk_sweep_cfg(int dtype, const SweepArgs &a, int block, int U, hipStream_t stream);
hipError_t launch_topk_backward_cfg(int dtype, const TopkBackwardArgs &a, int block, int U,
                                    hipStream_t stream);

} // namespace cev
