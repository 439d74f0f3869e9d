/*
 * cevocab.h -- collapse-safe selective log-softmax and cross-entropy over a
 * [rows, vocab] logit matrix, forward and analytic backward, for AMD Instinct
 * MI355X (gfx950).  C ABI of libcevocab.so.
 *
 * Pages cited below:
 *   [swift-10337]  ms-swift PR #10337, "perf(rlhf): chunk selective_log_softmax
 *                  instead of looping per token"
 *   [swift-10353]  ms-swift PR #10353, custom SFT loss (sparse supervision and
 *                  the analytic chunked backward)
 *   [liger-1555]   Liger-Kernel PR #1555, "Fix softmax collapse in CE, GRPO,
 *                  KL/JSD and softmax", with the unsloth-zoo commit #2080 that
 *                  the page quotes ([unsloth-2080])
 *
 * Notation, per row r: z_j the stored logit, T > 0 the temperature,
 * x_j = z_j / T, t = labels[r].  A row is VALID when row_mask is NULL or
 * row_mask[r] != 0, t != ignore_index, and 0 <= t < vocab.  A label outside
 * [0, vocab) that is not ignore_index makes the row ignored and ORs
 * CEV_STATUS_BAD_LABEL into *status.
 *
 * Conventions shared by every entry point
 *   Memory    Every array argument is a device pointer owned by the caller.
 *             The library never allocates, frees, keeps a pointer, or
 *             synchronizes.  All work is enqueued on `stream` (NULL = the
 *             default stream) and is asynchronous: buffers must stay alive
 *             until the stream reaches that point.
 *   Layout    logits is row-major with `row_stride` ELEMENTS between row
 *             starts (row_stride >= vocab) and unit column stride.  The base
 *             pointer must be aligned to the element size.  Rows whose start
 *             is 16-byte aligned take the vector path; others a peeled head.
 *   Dtypes    CEV_F32 (IEEE binary32) or CEV_BF16 (upper half of binary32),
 *             widened to fp32 exactly.  Accumulation is fp32; every per-row
 *             closing step (log, softplus, sigmoid, entropy) is fp64.
 *   Errors    The return value is CEV_OK or a negative CEV_E* code.  Argument
 *             errors are detected on the host BEFORE anything is enqueued and
 *             have no side effects.  rows == 0 is a successful no-op.  A failed
 *             kernel launch returns CEV_ELAUNCH.  Data errors inside arrays
 *             (a bad label or index) do not fail the call: the affected rows
 *             or entries are treated as ignored and a CEV_STATUS_* bit is ORed
 *             into *status, if status is non-NULL; the caller reads it after
 *             its own synchronization.  *status is never cleared by the library.
 *   Outputs   Ignored rows get log p = loss = entropy = 0 and argmax = -1
 *             ([swift-10353], PR information: ignored labels get zero upstream
 *             weight and losses are scattered back to the per-token shape).
 *             Every log p written is <= 0 ([unsloth-2080], Summary: the log-prob
 *             must never come out positive).
 *   Determinism  Fixed reduction order, no floating-point atomics: repeated
 *             calls with the same arguments give bit-identical results.  The
 *             functions hold no state and may be called concurrently on
 *             different streams with disjoint outputs.
 */
#ifndef CEVOCAB_H
#define CEVOCAB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;
typedef struct ihipStream_t *cev_stream_t; /* the same handle as hipStream_t */

enum cev_dtype { CEV_F32 = 0, CEV_BF16 = 1 };

enum cev_error {
    CEV_OK = 0,
    CEV_ENULL = -1,        /* a required pointer is NULL */
    CEV_ESHAPE = -2,       /* rows outside [0, 2^22], vocab outside [1, 2^30), K outside
                              [1, 1024], or a size overflows */
    CEV_ESTRIDE = -3,      /* a row stride smaller than the row */
    CEV_EALIGN = -4,       /* a pointer not aligned to its element size */
    CEV_EDTYPE = -5,       /* unknown dtype */
    CEV_ETEMP = -6,        /* temperature not finite or not > 0 */
    CEV_EWORKSPACE = -7,   /* workspace too small */
    CEV_EALIAS = -8,       /* an output overlaps an input it is computed from */
    CEV_ELAUNCH = -9,      /* the HIP runtime refused a launch */
    CEV_ESMOOTH = -10,     /* label_smoothing not finite or outside [0, 1] */
    CEV_EBETA = -11,       /* jsd beta not finite or outside [0, 1] */
    CEV_ESCRATCH = -12     /* ce_forward_noalloc: the call needs more than the static scratch,
                              or the scratch's device address could not be looked up */
};

/* Bits ORed into the optional device status word. */
#define CEV_STATUS_BAD_LABEL 1u /* a label outside [0, vocab) and != ignore_index */
#define CEV_STATUS_BAD_INDEX 2u /* a gathered index outside [0, vocab) and != ignore_index */
#define CEV_STATUS_BAD_PARTS 4u /* ce_vocab_merge: the partial records of a valid row do not
                                   all mark it valid, or not exactly one holds its label */

/* Per-row record written by ce_forward and read by ce_backward: 16 bytes,
 * 16-byte aligned.  m_z is the exact largest stored logit of the row,
 * log2_d = log2 sum_j exp((z_j - m_z)/T), q = 1 - p_t computed as sigmoid(u)
 * (never by subtraction), flags bit 0 = row valid.  ([liger-1555], Summary,
 * GRPO bullet: the forward keeps an accurate log p rather than only lse, and
 * the backward rebuilds the normaliser from it.) */
typedef struct cev_saved {
    float m_z;
    float log2_d;
    float q;
    int32_t flags;
} cev_saved;

/*
 * sls_forward -- selective log-softmax at the label ([swift-10337], PR
 * information: gather(log_softmax(logits / T), labels) with temperature and
 * row_mask), in the collapse-safe form of [liger-1555] (Summary, CE bullet):
 *   u = log sum_{j != t} e^{x_j - m_o} + m_o - x_t,  m_o = max_{j != t} x_j,
 *   logp[r] = -softplus(u)   (never positive; exact 0 only when V = 1).
 *
 *   logits        [rows, row_stride] fp32 or bf16 (dtype), read only
 *   labels        [rows] int64
 *   ignore_index  label value meaning "ignored" (conventionally -100)
 *   temperature   T > 0, finite; x = z / T
 *   row_mask      [rows] uint8 or NULL; 0 = row ignored
 *   logp          [rows] fp32 out, required
 *   entropy       [rows] fp32 out or NULL: H = -sum_j p_j log p_j, summed as
 *                 non-negative terms ([unsloth-2080], Summary: entropy takes
 *                 log s from the target-excluded term)
 *   argmax        [rows] int64 out or NULL: lowest j with z_j = max_k z_k,
 *                 compared on the stored values; -1 for ignored rows
 *   status        device int32 or NULL (see Errors)
 */
int sls_forward(const void *logits, int64_t rows, int64_t vocab, int64_t row_stride, int dtype,
                const int64_t *labels, int64_t ignore_index, double temperature,
                const uint8_t *row_mask, float *logp, float *entropy, int64_t *argmax,
                int32_t *status, cev_stream_t stream);

/*
 * sls_topk_forward -- selective log-softmax at K gathered indices per row
 * ([swift-10337], PR information: top-K indices are supported), each in the
 * collapse-safe form logp[r,k] = -softplus(u_k), u_k = log sum_{j != i_k}
 * e^{x_j - M} + M - x_{i_k}, where the sum over the columns outside the
 * gathered set comes from one sweep and the other gathered columns are added
 * to it (nothing is subtracted, so a peaked gathered column keeps its tiny
 * complement).
 *
 *   indices       [rows, K] int64 with row stride index_row_stride (>= K)
 *   logp          [rows, K] fp32 out, dense.  An index equal to ignore_index
 *                 gives 0; an index outside [0, vocab) gives 0 and sets
 *                 CEV_STATUS_BAD_INDEX; a masked row gives K zeros.
 *   q             [rows, K] fp32 out or NULL: 1 - p at each index, computed as
 *                 sigmoid(u_k) (0 where logp is 0 by the rules above)
 *   saved         [rows] cev_saved out or NULL, 16-byte aligned: m_z and
 *                 log2_d of the row for sls_topk_backward (q and the target
 *                 are not used there; flags bit 0 = row not masked)
 *   Other arguments as sls_forward.
 */
int sls_topk_forward(const void *logits, int64_t rows, int64_t vocab, int64_t row_stride,
                     int dtype, const int64_t *indices, int64_t K, int64_t index_row_stride,
                     int64_t ignore_index, double temperature, const uint8_t *row_mask,
                     float *logp, float *q, void *saved, int32_t *status, cev_stream_t stream);

/*
 * sls_topk_backward -- gradient of sum_k g[r,k] logp[r,k] with respect to the
 * stored logits, for the top-K gather of sls_topk_forward ([swift-10337], PR
 * information: gradients flow through the top-K indices), with the 1/T of
 * x = z/T applied:
 *   dlogits[r, j] = (1/T) (G_j - Gs p_j),
 * Gs = sum of g[r,k] over the entries with a valid index, G_j = the sum of
 * g[r,k] over the entries whose index is j (repeated indices add).  A gathered
 * column is formed as (G_j q_j - p_j (Gs - G_j)) / T from the forward's q, so
 * a peaked column keeps its small value without cancellation; every other
 * column is -(Gs/T) p_j.  Entries with an ignored or out-of-range index add
 * nothing (the latter also set CEV_STATUS_BAD_INDEX); masked rows get an
 * all-zero row.
 *
 *   indices, K, index_row_stride, row_mask   as passed to sls_topk_forward
 *   g             [rows, K] fp32, dense: upstream gradient of logp[r, k]
 *   saved, q      the sls_topk_forward outputs for the same arguments
 *   dlogits       [rows, dlogits_row_stride] out, as ce_backward
 */
int sls_topk_backward(const void *logits, int64_t rows, int64_t vocab, int64_t row_stride,
                      int dtype, const int64_t *indices, int64_t K, int64_t index_row_stride,
                      int64_t ignore_index, double temperature, const uint8_t *row_mask,
                      const float *g, const void *saved, const float *q, void *dlogits,
                      int64_t dlogits_row_stride, int32_t *status, cev_stream_t stream);

/*
 * ce_forward -- per-row cross-entropy forward with sparse-supervision
 * compaction ([swift-10353], PR information: supervised rows are selected
 * before the cross-entropy, losses scattered back to the per-token shape).
 * On the device it (1) compacts the valid rows into an ascending list and a
 * count, and writes the zero outputs of every ignored row, then (2) sweeps
 * only the listed rows.  No host synchronization happens in between.
 *
 *   label_smoothing  eps in [0, 1] ([unsloth-2080], Summary: smoothing kept in
 *                 the collapse-safe target term): loss = (1 - eps)(-log p_t)
 *                 + (eps/V) sum_j (-log p_j); 0 gives the plain loss
 *   loss          [rows] fp32 out, required: softplus(u) = -log p_t (with
 *                 smoothing as above), 0 at holes
 *   saved         [rows] cev_saved out, required, 16-byte aligned: the record
 *                 ce_backward needs
 *   logp, entropy, argmax   as sls_forward, each optional (NULL)
 *   valid_rows    [rows] int64 out or NULL: the first *n_valid entries are the
 *                 valid rows in ascending order; the rest are left untouched
 *   n_valid       device int64 out or NULL: the number of valid rows
 *   workspace     device scratch, or NULL.  With fewer than 16 rows and long
 *                 rows, each row is split over several workgroups whose partial
 *                 (max, sum) records are merged in a fixed order afterwards; this
 *                 needs workspace_bytes >= cev_workspace_size(rows, vocab, dtype)
 *                 and a 32-byte aligned workspace, else whole rows are swept
 *                 (same results up to rounding, lower occupancy).  When
 *                 valid_rows or n_valid is NULL the workspace also holds them and
 *                 must be at least (rows + 1) * 8 bytes, 8-byte aligned;
 *                 when both are NULL it may be NULL too, and then every row
 *                 is swept in place with no list (same results).
 *                 The workspace is overwritten; calls that share one race.
 */
int ce_forward(const void *logits, int64_t rows, int64_t vocab, int64_t row_stride, int dtype,
               const int64_t *labels, int64_t ignore_index, double temperature,
               double label_smoothing, const uint8_t *row_mask, float *loss, void *saved, float *logp, float *entropy,
               int64_t *argmax, int64_t *valid_rows, int64_t *n_valid, void *workspace,
               size_t workspace_bytes, int32_t *status, cev_stream_t stream);

/*
 * ce_forward_noalloc -- ce_forward without a workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  Same arguments, outputs,
 * errors and results as ce_forward (bit for bit); the workspace lives in a
 * static device array of cev_noalloc_scratch_bytes() bytes (4 MiB) that each
 * GPU holds until the process ends.  A call whose cev_workspace_size(rows,
 * vocab, dtype) exceeds it (more than 524287 rows) returns CEV_ESCRATCH
 * before anything is enqueued.  The first call on each device looks up the array's
 * device address (hipGetSymbolAddress, no allocation); a caller that captures
 * graphs makes one ordinary call on that device first.  Every call on a GPU
 * shares that GPU's array: calls that overlap on one GPU (different streams,
 * or host threads) race and must be serialized by the caller.  Nothing is
 * allocated, freed or synchronized.
 */
int ce_forward_noalloc(const void *logits, int64_t rows, int64_t vocab, int64_t row_stride,
                       int dtype, const int64_t *labels, int64_t ignore_index, double temperature,
                       double label_smoothing, const uint8_t *row_mask, float *loss, void *saved,
                       float *logp, float *entropy, int64_t *argmax, int64_t *valid_rows,
                       int64_t *n_valid, int32_t *status, cev_stream_t stream);

/* Size in bytes of the static scratch that ce_forward_noalloc uses per GPU. */
size_t cev_noalloc_scratch_bytes(void);

/*
 * ce_backward -- analytic gradient of the per-row loss with respect to the
 * stored logits, one pass over each valid row ([swift-10353], PR information:
 * g * softmax(logits) - g * one_hot(labels), ignored labels get zero weight,
 * written into a separate gradient buffer), with the 1/T of x = z/T applied,
 * and the target column taken as -(g/T) q, q = s_others / d = 1 - p_t
 * ([liger-1555], Summary: dx_y = -sum_others / d), so each row sums to zero:
 *   dlogits[r, j] = (g[r]/T) p_j  (j != t),   dlogits[r, t] = -(g[r]/T) q_r.
 * With label smoothing eps every column also gets -(g[r]/T) eps/V and the
 * target +(g[r]/T) eps.  Ignored rows get an all-zero row.  The output dtype is the logits dtype;
 * bf16 is rounded to nearest even from fp32.
 *
 *   g             [rows] fp32: upstream gradient of loss[r] (for a caller that
 *                 differentiates log p instead, pass g = -dL/dlogp)
 *   saved         [rows] cev_saved from ce_forward with identical arguments
 *                 (label_smoothing included)
 *   dlogits       [rows, dlogits_row_stride] out, same dtype as logits; must
 *                 not overlap logits (CEV_EALIAS); columns >= vocab untouched
 */
int ce_backward(const void *logits, int64_t rows, int64_t vocab, int64_t row_stride, int dtype,
                const int64_t *labels, int64_t ignore_index, double temperature,
                double label_smoothing, const uint8_t *row_mask, const float *g, const void *saved, void *dlogits,
                int64_t dlogits_row_stride, int32_t *status, cev_stream_t stream);

/*
 * ce_fused -- ce_forward and ce_backward in one call, for an upstream weight g
 * that is known before the forward (token weights, a mean over rows).  When
 * every row of logits and dlogits starts 16-byte aligned, one workgroup per row
 * sweeps the row, closes it in fp64 and then writes (g/T)(softmax - onehot),
 * keeping part of the row on chip between the two passes (43% of a
 * 152064-wide bf16 row) and reading the rest again at once: 4.73 GB of
 * algorithmic traffic for the 8192 x 152064 bf16 step instead of the two
 * calls' 6.98 GB.  This realises the
 * gradient-in-the-forward idea of the unsloth-zoo #2079 Summary quoted on the
 * Liger-Kernel PR #1555 page for a plain logit matrix.  Otherwise it runs
 * ce_forward then ce_backward.  Outputs and their meaning are those of
 * ce_forward (loss, saved, logp, entropy, argmax, valid_rows, n_valid) and
 * ce_backward (dlogits); g, dlogits and dlogits_row_stride as in ce_backward.
 * valid_rows / n_valid are computed only when requested; a missing one of the
 * pair takes (rows + 1) * 8 bytes of workspace, and the two-pass fallback uses
 * the workspace as ce_forward does.
 */
int ce_fused(const void *logits, int64_t rows, int64_t vocab, int64_t row_stride, int dtype,
             const int64_t *labels, int64_t ignore_index, double temperature,
             double label_smoothing, const uint8_t *row_mask, const float *g, float *loss, void *saved, float *logp,
             float *entropy, int64_t *argmax, void *dlogits, int64_t dlogits_row_stride,
             int64_t *valid_rows, int64_t *n_valid, void *workspace, size_t workspace_bytes,
             int32_t *status, cev_stream_t stream);

/*
 * Vocab-parallel (tensor-parallel) logits: the columns of each row are split
 * over P shards, each held by one rank.  The target-excluded sums of every
 * shard are combined in one exchange step, as the Liger-Kernel PR #1555 page
 * (Summary, CE bullet) does for vocab-parallel cross-entropy: both sums
 * reduced together.  Per call on each rank:
 *   1. ce_vocab_shard_forward on the rank's columns -> one partial record
 *      per row;
 *   2. an all-gather of the records (48 B per row per shard) by the caller
 *      (RCCL), into [P][rows] order of ascending column ranges;
 *   3. ce_vocab_merge on every rank -> the same loss, log p, entropy, argmax
 *      and saved record that ce_forward gives for the whole row;
 *   4. ce_vocab_shard_backward on the rank's columns.
 * The merge is fixed-order and fp64, so every rank gets bit-identical outputs.
 */

/* One shard's statistics of one row (written by ce_vocab_shard_forward,
 * merged by ce_vocab_merge); 48 bytes, 8-byte aligned. */
typedef struct cev_vocab_partial {
    float m;       /* largest non-target stored logit of the shard, -inf if none */
    float zt;      /* the stored target logit if the shard holds the label, else 0 */
    int64_t arg;   /* lowest global column holding m, INT64_MAX if none */
    double s;      /* sum over the shard's non-target columns of e^{(z - B)/T},
                      B = max(m, -FLT_MAX) */
    double h;      /* sum of e^{(z - B)/T} (B - z)/T (0 unless CEV_PART_ENTROPY) */
    double zs;     /* sum of the non-target stored values (0 unless CEV_PART_VALUE_SUM) */
    int32_t flags; /* bit 0: row valid; bit 1: this shard holds the label */
    int32_t pad;
} cev_vocab_partial;

#define CEV_PART_ENTROPY 1u   /* also sum the entropy term (needed for entropy) */
#define CEV_PART_VALUE_SUM 2u /* also sum the values (needed for label smoothing) */

/*
 * ce_vocab_shard_forward -- the forward sweep of ce_forward over one shard:
 * columns [col_offset, col_offset + shard_vocab) of a vocab-wide row.
 *
 *   logits        [rows, row_stride] the shard's columns only (element 0 of a
 *                 row is global column col_offset); shard_vocab <= row_stride
 *   col_offset, vocab   0 <= col_offset, col_offset + shard_vocab <= vocab;
 *                 labels are global columns in [0, vocab)
 *   what          CEV_PART_* bits
 *   partials      [rows] cev_vocab_partial out, 8-byte aligned.  Invalid rows
 *                 (same rule as ce_forward) get flags = 0.
 *   Other arguments as sls_forward.
 */
int ce_vocab_shard_forward(const void *logits, int64_t rows, int64_t shard_vocab,
                           int64_t row_stride, int dtype, int64_t col_offset, int64_t vocab,
                           const int64_t *labels, int64_t ignore_index, double temperature,
                           const uint8_t *row_mask, unsigned what, void *partials,
                           int32_t *status, cev_stream_t stream);

/*
 * ce_vocab_merge -- merge P shards' partial records of every row in a fixed
 * order (shard 0 first), in fp64: the common base is the largest m, each sum
 * is rescaled by e^{(B_p - B)/T} (the partial/combine rule of the
 * unsloth-zoo #2080 Summary quoted on the Liger-Kernel PR #1555 page), the
 * argmax is the lowest column holding the largest value, and the target logit
 * comes from the one shard holding the label.  Then the closing step of
 * ce_forward.
 *
 *   partials      [parts][rows] cev_vocab_partial, shard p's records at
 *                 partials + p * rows; 1 <= parts <= 4096
 *   vocab         the full vocabulary width (for labels and smoothing)
 *   loss, saved   required, as ce_forward; logp, entropy, argmax optional.
 *                 entropy needs records made with CEV_PART_ENTROPY, and
 *                 label_smoothing != 0 needs CEV_PART_VALUE_SUM.
 *   A valid row whose records disagree (a shard marks it invalid, or not
 *   exactly one shard holds its label) gets the ignored-row outputs and ORs
 *   CEV_STATUS_BAD_PARTS into *status.
 */
int ce_vocab_merge(const void *partials, int64_t parts, int64_t rows, int64_t vocab,
                   const int64_t *labels, int64_t ignore_index, double temperature,
                   double label_smoothing, const uint8_t *row_mask, float *loss, void *saved,
                   float *logp, float *entropy, int64_t *argmax, int32_t *status,
                   cev_stream_t stream);

/*
 * ce_vocab_shard_backward -- ce_backward over one shard's columns, from the
 * merged saved record: (g/T)(p_j - eps/V) at every column of the shard, and
 * (g/T)(eps - eps/V - q) at the label if the shard holds it.  Arguments as
 * ce_backward, plus col_offset and vocab as in ce_vocab_shard_forward
 * (logits and dlogits hold the shard's columns only).
 */
int ce_vocab_shard_backward(const void *logits, int64_t rows, int64_t shard_vocab,
                            int64_t row_stride, int dtype, int64_t col_offset, int64_t vocab,
                            const int64_t *labels, int64_t ignore_index, double temperature,
                            double label_smoothing, const uint8_t *row_mask, const float *g,
                            const void *saved, void *dlogits, int64_t dlogits_row_stride,
                            int32_t *status, cev_stream_t stream);

/*
 * Linear cross-entropy: logits = hidden x head^T, formed tile by tile on the
 * bf16 matrix cores and consumed in registers, so the [rows, vocab] logits
 * never reach HBM (the fused linear CE / log-prob setting of [unsloth-2080]
 * Summary, whose Speed section measures a frozen 2560 x 151936 head).  The
 * logits are the fp32 accumulations of bf16 products; everything after them
 * is the collapse-safe cross-entropy of ce_forward / ce_backward.
 *
 *   hidden        [rows, hidden_stride] bf16, hidden_dim a multiple of 64 in
 *                 [64, 65536], hidden_stride >= hidden_dim a multiple of 8,
 *                 16-byte aligned
 *   weight        the head, [vocab, weight_stride] bf16 (row j = class j),
 *                 same rules; no bias
 *   workspace     device scratch of at least lce_workspace_size(rows,
 *                 hidden_dim, vocab) bytes, 16-byte aligned; overwritten,
 *                 calls that share one race
 *   labels, ignore_index, temperature, label_smoothing, row_mask, status
 *                 as ce_forward
 */

/* lce_forward -- loss, log p, entropy, argmax and the saved record of every
 * row, as ce_forward computes them from the logits hidden x head^T (argmax:
 * lowest column of the largest fp32 logit).  loss and saved are required;
 * logp, entropy and argmax may be NULL.
 *   logits, logits_stride   NULL (the logits are never stored), or a
 *                 caller-owned fp32 [rows, logits_stride] buffer (stride >=
 *                 vocab, a multiple of 4, 16-byte aligned, overlapping no
 *                 other argument) that receives z = hidden x head^T (before
 *                 the temperature) for every row, masked ones included;
 *                 columns past vocab are left as they were.  Memory traded
 *                 for the backward's recomputation (see lce_backward).
 *                 CEV_ESTRIDE / CEV_EALIGN for a bad stride / alignment,
 *                 CEV_EALIAS if it overlaps hidden, head or the workspace. */
int lce_forward(const void *hidden, int64_t rows, int64_t hidden_dim, int64_t hidden_stride,
                const void *weight, int64_t vocab, int64_t weight_stride, const int64_t *labels,
                int64_t ignore_index, double temperature, double label_smoothing,
                const uint8_t *row_mask, float *loss, void *saved, float *logp, float *entropy,
                int64_t *argmax, float *logits, int64_t logits_stride, void *workspace,
                size_t workspace_bytes, int32_t *status, cev_stream_t stream);

/* lce_backward -- with dlogits = ce_backward's gradient of the per-row loss
 * weighted by g (from the saved record and the logits, recomputed from
 * hidden and head, or read from `logits` when the forward stored them there:
 * the same fp32 values, so the same dlogits bit for bit):
 *   dhidden = dlogits x head   [rows, dhidden_stride] fp32, required
 *   dweight = dlogits^T x hidden   [vocab, dweight_stride] fp32, or NULL for a
 *             frozen head
 * Both strides >= hidden_dim.  dlogits is kept in the workspace in bf16
 * (rounded to nearest even), the operand the two products read.  `logits`
 * (NULL to recompute) is checked as in lce_forward and must not overlap
 * dhidden, dweight or the workspace (CEV_EALIAS). */
int lce_backward(const void *hidden, int64_t rows, int64_t hidden_dim, int64_t hidden_stride,
                 const void *weight, int64_t vocab, int64_t weight_stride,
                 const int64_t *labels, int64_t ignore_index, double temperature,
                 double label_smoothing, const uint8_t *row_mask, const float *g,
                 const void *saved, const float *logits, int64_t logits_stride, float *dhidden,
                 int64_t dhidden_stride, float *dweight, int64_t dweight_stride, void *workspace,
                 size_t workspace_bytes, int32_t *status, cev_stream_t stream);

/* Bytes of workspace lce_forward and lce_backward need (0 for invalid
 * arguments). */
size_t lce_workspace_size(int64_t rows, int64_t hidden_dim, int64_t vocab);

/* ---------------------------------------------------------------------------
 * Generalized Jensen-Shannon divergence between a student and a teacher logit
 * row, with the KL divergences at its ends (the generalized JSD of the
 * unsloth-zoo #2079 Summary quoted on the Liger-Kernel PR #1555 page): with
 * P_s = softmax(student / T), P_t = softmax(teacher / T),
 *   beta = 0      KL(P_t || P_s)   (forward KL)
 *   beta = 1      KL(P_s || P_t)   (reverse KL)
 *   0 < beta < 1  beta KL(P_t || M) + (1 - beta) KL(P_s || M),
 *                 M = beta P_t + (1 - beta) P_s
 * per row, no reduction; the teacher is not differentiated.  Log-softmax is
 * based at each row's argmax (log p there is -log1p of the others' sum) and
 * the gradient entry at the student's argmax is minus the sum of the others
 * (Liger-Kernel PR #1555, Summary, "fused KL / JSD" bullet), so rows peaked far
 * beyond the fp32 softmax collapse keep an accurate, zero-sum gradient.
 *
 *   student, teacher  [rows, *_stride] in dtype (both CEV_F32 or both
 *                     CEV_BF16), element-aligned, read only; when every row
 *                     of every operand starts 16-byte aligned the kernels
 *                     use 16-byte vector accesses, otherwise scalar ones
 *   labels            [rows] int64 or NULL: a row whose label equals
 *                     ignore_index is masked (any other value is fine)
 *   row_mask          [rows] u8 or NULL: 0 masks the row
 *   temperature       finite, > 0 (CEV_ETEMP); beta in [0, 1] (CEV_EBETA)
 * Masked rows get loss 0, an invalid saved record and an all-zero gradient.
 * Deterministic: fixed reduction order, no float atomics.
 */

/* Per-row record of jsd_forward, read by jsd_backward: 48 bytes. */
typedef struct cev_jsd_saved {
    float ms;      /* largest stored student logit */
    float ls0;     /* log1p(sum over the student's other columns of e^{(z - ms)/T}) */
    float mt;      /* largest stored teacher logit */
    float lt0;     /* the same for the teacher */
    float k;       /* the loss at beta = 1; in between sum P_s log2(P_s / M) (base 2); 0 at beta = 0 */
    float garg;    /* the gradient entry at the student's argmax per unit of g/T (minus
                      the fp64 sum of the others), when flags bit 1 is set */
    int32_t arg;   /* the student's argmax column (first occurrence), -1 if masked */
    int32_t flags; /* bit 0: row valid; bit 1: garg holds */
    float dl;      /* ls0 - lt0 formed in fp64, then rounded */
    float pad[3];
} cev_jsd_saved;

/* jsd_forward -- loss [rows] fp32 and saved [rows] x 48 bytes (16-byte
 * aligned), both required. */
int jsd_forward(const void *student, const void *teacher, int64_t rows, int64_t vocab,
                int64_t student_stride, int64_t teacher_stride, int dtype,
                const int64_t *labels, int64_t ignore_index, double temperature, double beta,
                const uint8_t *row_mask, float *loss, void *saved, int32_t *status,
                cev_stream_t stream);

/* jsd_backward -- dstudent [rows, dstudent_stride] in dtype (must not overlap
 * either input) = g[r] times the gradient of row r's
 * loss with respect to the student logits; bf16 is rounded to nearest even
 * from fp32, the argmax entry from the fp64 sum of the others.  saved from
 * jsd_forward with the same arguments. */
int jsd_backward(const void *student, const void *teacher, int64_t rows, int64_t vocab,
                 int64_t student_stride, int64_t teacher_stride, int dtype,
                 const int64_t *labels, int64_t ignore_index, double temperature, double beta,
                 const uint8_t *row_mask, const float *g, const void *saved, void *dstudent,
                 int64_t dstudent_stride, int32_t *status, cev_stream_t stream);

/* Bytes of workspace that let ce_forward hold the compacted row list and
 * count and, for few rows, the split-row partial records (0 for invalid
 * arguments). */
size_t cev_workspace_size(int64_t rows, int64_t vocab, int dtype);

/* Static text for a CEV_* return code. */
const char *cev_status_string(int code);

/* Library version as major * 10000 + minor * 100 + patch. */
int cev_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CEVOCAB_H */
