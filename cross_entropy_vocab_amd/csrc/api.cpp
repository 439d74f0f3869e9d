// api.cpp -- the C ABI of libcevocab.so: argument validation on the host, then
// kernel launches on the caller's stream.  Nothing here allocates, frees or
// synchronizes.  Entry points and their semantics are declared in cevocab.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <initializer_list>

#include "cev_launch.h"
#include "cevocab.h"

namespace {

using cev::BackwardArgs;
using cev::CompactArgs;
using cev::SweepArgs;

constexpr int64_t kMaxRows = 1 << 22;         // one workgroup per row; the grid stays < 2^32 work-items
constexpr int64_t kMaxVocab = INT32_MAX / 2;  // step codes are 32-bit
constexpr int64_t kMaxK = 1024;               // gathered indices per row held in LDS
constexpr int64_t kMaxParts = 4096;           // shards merged by ce_vocab_merge

int elem_size(int dtype) { return dtype == CEV_F32 ? 4 : 2; }

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

hipStream_t to_hip(cev_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

// Checks shared by every entry point.  On success *done is set when rows == 0
// (nothing to enqueue).
int check_common(const void *logits, int64_t rows, int64_t vocab, int64_t row_stride, int dtype,
                 double temperature, bool *done)
{
    *done = false;
    if (dtype != CEV_F32 && dtype != CEV_BF16)
        return CEV_EDTYPE;
    if (!(std::isfinite(temperature) && temperature > 0.0))
        return CEV_ETEMP;
    if (rows < 0 || vocab < 1 || rows > kMaxRows || vocab > kMaxVocab)
        return CEV_ESHAPE;
    if (row_stride < vocab)
        return CEV_ESTRIDE;
    if (rows == 0) {
        *done = true;
        return CEV_OK;
    }
    if (row_stride > INT64_MAX / 4 / rows)
        return CEV_ESHAPE;
    if (!logits)
        return CEV_ENULL;
    if (!aligned(logits, (uintptr_t)elem_size(dtype)))
        return CEV_EALIGN;
    // The per-row closing step works from fp32 copies of log2(e)/T and 1/T;
    // both must be finite and non-zero.
    const double c = 1.4426950408889634074 / temperature;
    if (!(c < 3.0e38 && c > 1.0e-37) || !(1.0 / temperature < 3.0e38))
        return CEV_ETEMP;
    return CEV_OK;
}

void fill_temperature(SweepArgs &a, double temperature)
{
    a.temperature = temperature;
    a.c = (float)(1.4426950408889634074 / temperature);
    a.inv_t = (float)(1.0 / temperature);
}

int launch_status(hipError_t e) { return e == hipSuccess ? CEV_OK : CEV_ELAUNCH; }

bool smoothing_ok(double eps) { return std::isfinite(eps) && eps >= 0.0 && eps <= 1.0; }

// dlogits must not overlap logits (the kernels read a row after other
// workgroups may have written theirs).
bool overlaps(const void *logits, int64_t row_stride, const void *dlogits, int64_t d_row_stride,
              int64_t rows, int64_t vocab, int es)
{
    const uintptr_t l0 = (uintptr_t)logits, l1 = l0 + (uintptr_t)(((rows - 1) * row_stride + vocab) * es);
    const uintptr_t d0 = (uintptr_t)dlogits, d1 = d0 + (uintptr_t)(((rows - 1) * d_row_stride + vocab) * es);
    return l0 < d1 && d0 < l1;
}

} // namespace

extern "C" {

int sls_forward(const void *logits, int64_t rows, int64_t vocab, int64_t row_stride, int dtype,
                const int64_t *labels, int64_t ignore_index, double temperature,
                const uint8_t *row_mask, float *logp, float *entropy, int64_t *argmax,
                int32_t *status, cev_stream_t stream)
{
    bool done;
    int rc = check_common(logits, rows, vocab, row_stride, dtype, temperature, &done);
    if (rc != CEV_OK || done)
        return rc;
    if (!labels || !logp)
        return CEV_ENULL;
    if (!aligned(labels, 8) || !aligned(logp, 4) || !aligned(entropy, 4) || !aligned(argmax, 8) ||
        !aligned(status, 4))
        return CEV_EALIGN;
    SweepArgs a{};
    a.logits = logits;
    a.rows = rows;
    a.vocab = vocab;
    a.row_stride = row_stride;
    a.labels = labels;
    a.ignore_index = ignore_index;
    a.row_mask = row_mask;
    a.splits = 1;
    a.swizzle = 1;
    fill_temperature(a, temperature);
    a.logp = logp;
    a.entropy = entropy;
    a.argmax = argmax;
    a.status = status;
    return launch_status(cev::launch_sls_sweep(dtype, a, entropy != nullptr, argmax != nullptr,
                                               to_hip(stream)));
}

int sls_topk_forward(const void *logits, int64_t rows, int64_t vocab, int64_t row_stride,
                     int dtype, const int64_t *indices, int64_t K, int64_t index_row_stride,
                     int64_t ignore_index, double temperature, const uint8_t *row_mask,
                     float *logp, float *q, void *saved, int32_t *status, cev_stream_t stream)
{
    if (K < 1 || K > kMaxK)
        return CEV_ESHAPE;
    if (index_row_stride < K)
        return CEV_ESTRIDE;
    bool done;
    int rc = check_common(logits, rows, vocab, row_stride, dtype, temperature, &done);
    if (rc != CEV_OK || done)
        return rc;
    if (!indices || !logp)
        return CEV_ENULL;
    if (!aligned(indices, 8) || !aligned(logp, 4) || !aligned(q, 4) || !aligned(saved, 16) ||
        !aligned(status, 4))
        return CEV_EALIGN;
    SweepArgs a{};
    a.logits = logits;
    a.rows = rows;
    a.vocab = vocab;
    a.row_stride = row_stride;
    a.indices = indices;
    a.K = K;
    a.index_row_stride = index_row_stride;
    a.splits = 1;
    a.ignore_index = ignore_index;
    a.row_mask = row_mask;
    fill_temperature(a, temperature);
    a.logp = logp;
    a.q = q;
    a.saved = static_cast<cev_saved *>(saved);
    a.status = status;
    return launch_status(cev::launch_topk_sweep(dtype, a, to_hip(stream)));
}

int sls_topk_backward(const void *logits, int64_t rows, int64_t vocab, int64_t row_stride,
                      int dtype, const int64_t *indices, int64_t K, int64_t index_row_stride,
                      int64_t ignore_index, double temperature, const uint8_t *row_mask,
                      const float *g, const void *saved, const float *q, void *dlogits,
                      int64_t dlogits_row_stride, int32_t *status, cev_stream_t stream)
{
    if (K < 1 || K > kMaxK)
        return CEV_ESHAPE;
    if (index_row_stride < K)
        return CEV_ESTRIDE;
    bool done;
    int rc = check_common(logits, rows, vocab, row_stride, dtype, temperature, &done);
    if (rc != CEV_OK || done)
        return rc;
    if (dlogits_row_stride < vocab)
        return CEV_ESTRIDE;
    if (dlogits_row_stride > INT64_MAX / 4 / rows || index_row_stride > INT64_MAX / 8 / rows)
        return CEV_ESHAPE;
    if (!indices || !g || !saved || !q || !dlogits)
        return CEV_ENULL;
    const int es = elem_size(dtype);
    if (!aligned(indices, 8) || !aligned(g, 4) || !aligned(saved, 16) || !aligned(q, 4) ||
        !aligned(dlogits, (uintptr_t)es) || !aligned(status, 4))
        return CEV_EALIGN;
    if (overlaps(logits, row_stride, dlogits, dlogits_row_stride, rows, vocab, es))
        return CEV_EALIAS;
    cev::TopkBackwardArgs a{};
    a.logits = logits;
    a.rows = rows;
    a.vocab = vocab;
    a.row_stride = row_stride;
    a.indices = indices;
    a.K = K;
    a.index_row_stride = index_row_stride;
    a.ignore_index = ignore_index;
    a.row_mask = row_mask;
    a.g = g;
    a.saved = static_cast<const cev_saved *>(saved);
    a.q = q;
    a.dlogits = dlogits;
    a.d_row_stride = dlogits_row_stride;
    a.c = (float)(1.4426950408889634074 / temperature);
    a.inv_t = (float)(1.0 / temperature);
    a.status = status;
    return launch_status(cev::launch_topk_backward(dtype, a, to_hip(stream)));
}

// Workspace of ce_forward: the compacted row list and its count, then (for
// few rows) the partial records of the split sweep, 32-byte aligned.
static size_t list_bytes(int64_t rows) { return (size_t)(rows + 1) * sizeof(int64_t); }

static size_t partial_offset(int64_t rows) { return (list_bytes(rows) + 31) & ~(size_t)31; }

size_t cev_workspace_size(int64_t rows, int64_t vocab, int dtype)
{
    if (rows < 0 || vocab < 1 || (dtype != CEV_F32 && dtype != CEV_BF16))
        return 0;
    const int64_t sp = cev::sweep_splits(rows, vocab, dtype);
    if (sp <= 1)
        return list_bytes(rows);
    return partial_offset(rows) + (size_t)rows * (size_t)sp * sizeof(cev::SplitPartial);
}

int ce_forward(const void *logits, int64_t rows, int64_t vocab, int64_t row_stride, int dtype,
               const int64_t *labels, int64_t ignore_index, double temperature,
               double label_smoothing, const uint8_t *row_mask, float *loss, void *saved,
               float *logp, float *entropy, int64_t *argmax, int64_t *valid_rows,
               int64_t *n_valid, void *workspace, size_t workspace_bytes, int32_t *status,
               cev_stream_t stream)
{
    bool done;
    int rc = check_common(logits, rows, vocab, row_stride, dtype, temperature, &done);
    if (rc != CEV_OK)
        return rc;
    if (!smoothing_ok(label_smoothing))
        return CEV_ESMOOTH;
    if (done)
        return rc;
    if (!labels || !loss || !saved)
        return CEV_ENULL;
    if (!aligned(labels, 8) || !aligned(loss, 4) || !aligned(saved, 16) || !aligned(logp, 4) ||
        !aligned(entropy, 4) || !aligned(argmax, 8) || !aligned(valid_rows, 8) ||
        !aligned(n_valid, 8) || !aligned(status, 4))
        return CEV_EALIGN;
    int64_t *list = valid_rows;
    int64_t *count = n_valid;
    // With neither list output asked for and no workspace there is no list:
    // every row is swept in place (ignored rows exit at once).
    const bool no_list = !valid_rows && !n_valid && !workspace;
    if ((!list || !count) && !no_list) {
        if (!workspace)
            return CEV_ENULL;
        if (!aligned(workspace, 8))
            return CEV_EALIGN;
        if (workspace_bytes < list_bytes(rows))
            return CEV_EWORKSPACE;
        int64_t *ws = static_cast<int64_t *>(workspace);
        if (!list)
            list = ws;
        if (!count)
            count = ws + rows;
    }
    // Few rows: split each row over several workgroups when the workspace
    // holds the partial records; otherwise sweep whole rows.
    int64_t splits = cev::sweep_splits(rows, vocab, dtype);
    void *partials = nullptr;
    if (splits > 1 && workspace && aligned(workspace, 32) &&
        workspace_bytes >= cev_workspace_size(rows, vocab, dtype))
        partials = static_cast<char *>(workspace) + partial_offset(rows);
    else
        splits = 1;

    // Whole rows: every row is swept in place, ignored rows exiting at once,
    // with the compaction in workgroups appended to the same launch (one
    // launch instead of two); rows are rotated within groups of 8 by a hash
    // so that a periodic mask cannot leave some XCDs idle.  On 8192 x 152064
    // bf16 rows that measured 340 against 344 us (compaction launch, then the
    // listed rows) with a random 10% mask, 337 against 342 us with every 10th
    // row ignored and 328 against 337 us with every 8th; in row order without
    // the rotation those two took 356 and 349 us.  Split rows (few of them)
    // compact first and sweep the listed parts.
    const bool in_place = no_list || splits == 1;
    SweepArgs a{};
    a.logits = logits;
    a.rows = rows;
    a.vocab = vocab;
    a.row_stride = row_stride;
    a.labels = labels;
    a.ignore_index = ignore_index;
    a.row_mask = row_mask;
    if (in_place) {
        a.out_list = list;
        a.out_count = count;
        a.swizzle = 1;
    } else {
        CompactArgs ca{};
        ca.rows = rows;
        ca.vocab = vocab;
        ca.labels = labels;
        ca.ignore_index = ignore_index;
        ca.row_mask = row_mask;
        ca.rowlist = list;
        ca.nlist = count;
        ca.logp = logp;
        ca.loss = loss;
        ca.entropy = entropy;
        ca.argmax = argmax;
        ca.saved = static_cast<cev_saved *>(saved);
        ca.status = status;
        hipError_t e = cev::launch_compact(ca, to_hip(stream));
        if (e != hipSuccess)
            return CEV_ELAUNCH;
        a.rowlist = list;
        a.nlist = count;
    }
    a.splits = splits;
    a.partials = partials;
    fill_temperature(a, temperature);
    a.label_smoothing = label_smoothing;
    a.logp = logp;
    a.loss = loss;
    a.entropy = entropy;
    a.argmax = argmax;
    a.saved = static_cast<cev_saved *>(saved);
    a.status = status;
    return launch_status(cev::launch_sls_sweep(dtype, a, entropy != nullptr, argmax != nullptr,
                                               to_hip(stream)));
}

int ce_backward(const void *logits, int64_t rows, int64_t vocab, int64_t row_stride, int dtype,
                const int64_t *labels, int64_t ignore_index, double temperature,
                double label_smoothing, const uint8_t *row_mask, const float *g,
                const void *saved, void *dlogits, int64_t dlogits_row_stride, int32_t *status,
                cev_stream_t stream)
{
    bool done;
    int rc = check_common(logits, rows, vocab, row_stride, dtype, temperature, &done);
    if (rc != CEV_OK)
        return rc;
    if (!smoothing_ok(label_smoothing))
        return CEV_ESMOOTH;
    if (done)
        return rc;
    if (dlogits_row_stride < vocab)
        return CEV_ESTRIDE;
    if (dlogits_row_stride > INT64_MAX / 4 / rows)
        return CEV_ESHAPE;
    if (!labels || !g || !saved || !dlogits)
        return CEV_ENULL;
    const int es = elem_size(dtype);
    if (!aligned(labels, 8) || !aligned(g, 4) || !aligned(saved, 16) ||
        !aligned(dlogits, (uintptr_t)es) || !aligned(status, 4))
        return CEV_EALIGN;
    if (overlaps(logits, row_stride, dlogits, dlogits_row_stride, rows, vocab, es))
        return CEV_EALIAS;
    BackwardArgs a{};
    a.logits = logits;
    a.rows = rows;
    a.vocab = vocab;
    a.row_stride = row_stride;
    a.col_offset = 0;
    a.vocab_total = vocab;
    a.labels = labels;
    a.ignore_index = ignore_index;
    a.row_mask = row_mask;
    a.g = g;
    a.saved = static_cast<const cev_saved *>(saved);
    a.dlogits = dlogits;
    a.d_row_stride = dlogits_row_stride;
    a.temperature = temperature;
    a.label_smoothing = label_smoothing;
    a.c = (float)(1.4426950408889634074 / temperature);
    a.inv_t = (float)(1.0 / temperature);
    a.eps = (float)label_smoothing;
    a.eps_over_v = (float)(label_smoothing / (double)vocab);
    a.status = status;
    return launch_status(cev::launch_backward(dtype, a, to_hip(stream)));
}

int ce_fused(const void *logits, int64_t rows, int64_t vocab, int64_t row_stride, int dtype,
             const int64_t *labels, int64_t ignore_index, double temperature,
             double label_smoothing, const uint8_t *row_mask, const float *g, float *loss,
             void *saved, float *logp, float *entropy, int64_t *argmax, void *dlogits,
             int64_t dlogits_row_stride, int64_t *valid_rows, int64_t *n_valid, void *workspace,
             size_t workspace_bytes, int32_t *status, cev_stream_t stream)
{
    bool done;
    int rc = check_common(logits, rows, vocab, row_stride, dtype, temperature, &done);
    if (rc != CEV_OK)
        return rc;
    if (!smoothing_ok(label_smoothing))
        return CEV_ESMOOTH;
    if (done)
        return rc;
    if (dlogits_row_stride < vocab)
        return CEV_ESTRIDE;
    if (dlogits_row_stride > INT64_MAX / 4 / rows)
        return CEV_ESHAPE;
    if (!labels || !g || !loss || !saved || !dlogits)
        return CEV_ENULL;
    const int es = elem_size(dtype);
    if (!aligned(labels, 8) || !aligned(g, 4) || !aligned(loss, 4) || !aligned(saved, 16) ||
        !aligned(logp, 4) || !aligned(entropy, 4) || !aligned(argmax, 8) ||
        !aligned(valid_rows, 8) || !aligned(n_valid, 8) || !aligned(dlogits, (uintptr_t)es) ||
        !aligned(status, 4))
        return CEV_EALIGN;
    if (overlaps(logits, row_stride, dlogits, dlogits_row_stride, rows, vocab, es))
        return CEV_EALIAS;
    const bool want_list = valid_rows || n_valid;
    if (want_list && (!valid_rows || !n_valid)) {
        if (!workspace)
            return CEV_ENULL;
        if (!aligned(workspace, 8))
            return CEV_EALIGN;
        if (workspace_bytes < list_bytes(rows))
            return CEV_EWORKSPACE;
    }

    // One workgroup per row for both passes when every row of both matrices
    // starts 16-byte aligned; otherwise ce_forward then ce_backward.
    const bool aligned_rows = aligned(logits, 16) && aligned(dlogits, 16) &&
                              (row_stride * es) % 16 == 0 && (dlogits_row_stride * es) % 16 == 0;
    if (!aligned_rows) {
        rc = ce_forward(logits, rows, vocab, row_stride, dtype, labels, ignore_index, temperature,
                        label_smoothing, row_mask, loss, saved, logp, entropy, argmax,
                        valid_rows, n_valid, workspace, workspace_bytes, status, stream);
        if (rc != CEV_OK)
            return rc;
        return ce_backward(logits, rows, vocab, row_stride, dtype, labels, ignore_index,
                           temperature, label_smoothing, row_mask, g, saved, dlogits,
                           dlogits_row_stride, status, stream);
    }
    if (want_list) {
        int64_t *list = valid_rows ? valid_rows : static_cast<int64_t *>(workspace);
        int64_t *count = n_valid ? n_valid : static_cast<int64_t *>(workspace) + rows;
        CompactArgs ca{};
        ca.rows = rows;
        ca.vocab = vocab;
        ca.labels = labels;
        ca.ignore_index = ignore_index;
        ca.row_mask = row_mask;
        ca.rowlist = list;
        ca.nlist = count;
        ca.logp = logp;
        ca.loss = loss;
        ca.entropy = entropy;
        ca.argmax = argmax;
        ca.saved = static_cast<cev_saved *>(saved);
        ca.status = status;
        if (cev::launch_compact(ca, to_hip(stream)) != hipSuccess)
            return CEV_ELAUNCH;
    }
    cev::FusedArgs fa{};
    fa.logits = logits;
    fa.rows = rows;
    fa.vocab = vocab;
    fa.row_stride = row_stride;
    fa.labels = labels;
    fa.ignore_index = ignore_index;
    fa.row_mask = row_mask;
    fa.g = g;
    fa.temperature = temperature;
    fa.label_smoothing = label_smoothing;
    fa.c = (float)(1.4426950408889634074 / temperature);
    fa.inv_t = (float)(1.0 / temperature);
    fa.loss = loss;
    fa.logp = logp;
    fa.entropy = entropy;
    fa.argmax = argmax;
    fa.saved = static_cast<cev_saved *>(saved);
    fa.dlogits = dlogits;
    fa.d_row_stride = dlogits_row_stride;
    fa.status = status;
    return launch_status(cev::launch_fused(dtype, fa, entropy != nullptr, to_hip(stream)));
}

// Checks of a shard's column range [col_offset, col_offset + shard_vocab) of a
// vocab-wide row.
static int check_shard(int64_t shard_vocab, int64_t col_offset, int64_t vocab)
{
    if (vocab < 1 || vocab > kMaxVocab || col_offset < 0 || shard_vocab > vocab ||
        col_offset > vocab - shard_vocab)
        return CEV_ESHAPE;
    return CEV_OK;
}

int ce_vocab_shard_forward(const void *logits, int64_t rows, int64_t shard_vocab,
                           int64_t row_stride, int dtype, int64_t col_offset, int64_t vocab,
                           const int64_t *labels, int64_t ignore_index, double temperature,
                           const uint8_t *row_mask, unsigned what, void *partials,
                           int32_t *status, cev_stream_t stream)
{
    bool done;
    int rc = check_common(logits, rows, shard_vocab, row_stride, dtype, temperature, &done);
    if (rc != CEV_OK)
        return rc;
    if ((rc = check_shard(shard_vocab, col_offset, vocab)) != CEV_OK)
        return rc;
    if (done)
        return CEV_OK;
    if (!labels || !partials)
        return CEV_ENULL;
    if (!aligned(labels, 8) || !aligned(partials, 8) || !aligned(status, 4))
        return CEV_EALIGN;
    cev::ShardArgs a{};
    a.logits = logits;
    a.rows = rows;
    a.vocab = shard_vocab;
    a.row_stride = row_stride;
    a.col_offset = col_offset;
    a.vocab_total = vocab;
    a.labels = labels;
    a.ignore_index = ignore_index;
    a.row_mask = row_mask;
    a.c = (float)(1.4426950408889634074 / temperature);
    a.inv_t = (float)(1.0 / temperature);
    a.partials = static_cast<cev_vocab_partial *>(partials);
    a.status = status;
    return launch_status(cev::launch_shard_sweep(dtype, a, (what & CEV_PART_ENTROPY) != 0,
                                                 (what & CEV_PART_VALUE_SUM) != 0,
                                                 to_hip(stream)));
}

int ce_vocab_merge(const void *partials, int64_t parts, int64_t rows, int64_t vocab,
                   const int64_t *labels, int64_t ignore_index, double temperature,
                   double label_smoothing, const uint8_t *row_mask, float *loss, void *saved,
                   float *logp, float *entropy, int64_t *argmax, int32_t *status,
                   cev_stream_t stream)
{
    if (!(std::isfinite(temperature) && temperature > 0.0))
        return CEV_ETEMP;
    if (!smoothing_ok(label_smoothing))
        return CEV_ESMOOTH;
    if (parts < 1 || parts > kMaxParts || rows < 0 || rows > kMaxRows || vocab < 1 ||
        vocab > kMaxVocab)
        return CEV_ESHAPE;
    if (rows == 0)
        return CEV_OK;
    if (!partials || !labels || !loss || !saved)
        return CEV_ENULL;
    if (!aligned(partials, 8) || !aligned(labels, 8) || !aligned(loss, 4) ||
        !aligned(saved, 16) || !aligned(logp, 4) || !aligned(entropy, 4) ||
        !aligned(argmax, 8) || !aligned(status, 4))
        return CEV_EALIGN;
    cev::MergeArgs a{};
    a.partials = static_cast<const cev_vocab_partial *>(partials);
    a.parts = parts;
    a.rows = rows;
    a.vocab = vocab;
    a.labels = labels;
    a.ignore_index = ignore_index;
    a.row_mask = row_mask;
    a.temperature = temperature;
    a.label_smoothing = label_smoothing;
    a.loss = loss;
    a.logp = logp;
    a.entropy = entropy;
    a.argmax = argmax;
    a.saved = static_cast<cev_saved *>(saved);
    a.status = status;
    return launch_status(cev::launch_vocab_merge(a, to_hip(stream)));
}

int ce_vocab_shard_backward(const void *logits, int64_t rows, int64_t shard_vocab,
                            int64_t row_stride, int dtype, int64_t col_offset, int64_t vocab,
                            const int64_t *labels, int64_t ignore_index, double temperature,
                            double label_smoothing, const uint8_t *row_mask, const float *g,
                            const void *saved, void *dlogits, int64_t dlogits_row_stride,
                            int32_t *status, cev_stream_t stream)
{
    bool done;
    int rc = check_common(logits, rows, shard_vocab, row_stride, dtype, temperature, &done);
    if (rc != CEV_OK)
        return rc;
    if ((rc = check_shard(shard_vocab, col_offset, vocab)) != CEV_OK)
        return rc;
    if (!smoothing_ok(label_smoothing))
        return CEV_ESMOOTH;
    if (done)
        return CEV_OK;
    if (dlogits_row_stride < shard_vocab)
        return CEV_ESTRIDE;
    if (dlogits_row_stride > INT64_MAX / 4 / rows)
        return CEV_ESHAPE;
    if (!labels || !g || !saved || !dlogits)
        return CEV_ENULL;
    const int es = elem_size(dtype);
    if (!aligned(labels, 8) || !aligned(g, 4) || !aligned(saved, 16) ||
        !aligned(dlogits, (uintptr_t)es) || !aligned(status, 4))
        return CEV_EALIGN;
    if (overlaps(logits, row_stride, dlogits, dlogits_row_stride, rows, shard_vocab, es))
        return CEV_EALIAS;
    BackwardArgs a{};
    a.logits = logits;
    a.rows = rows;
    a.vocab = shard_vocab;
    a.row_stride = row_stride;
    a.col_offset = col_offset;
    a.vocab_total = vocab;
    a.labels = labels;
    a.ignore_index = ignore_index;
    a.row_mask = row_mask;
    a.g = g;
    a.saved = static_cast<const cev_saved *>(saved);
    a.dlogits = dlogits;
    a.d_row_stride = dlogits_row_stride;
    a.temperature = temperature;
    a.label_smoothing = label_smoothing;
    a.c = (float)(1.4426950408889634074 / temperature);
    a.inv_t = (float)(1.0 / temperature);
    a.eps = (float)label_smoothing;
    a.eps_over_v = (float)(label_smoothing / (double)vocab);
    a.status = status;
    return launch_status(cev::launch_backward(dtype, a, to_hip(stream)));
}

// Shapes of the linear cross-entropy: bf16 hidden [rows, hs] and head
// [vocab, ws], hidden_dim a multiple of 64, strides multiples of 8.
static int check_lce(const void *hidden, int64_t rows, int64_t hd, int64_t hs, const void *weight,
                     int64_t vocab, int64_t ws, double temperature, double eps, bool *done)
{
    *done = false;
    if (!(std::isfinite(temperature) && temperature > 0.0))
        return CEV_ETEMP;
    if (!smoothing_ok(eps))
        return CEV_ESMOOTH;
    if (rows < 0 || rows > kMaxRows || vocab < 1 || vocab > kMaxVocab || hd < 64 ||
        hd > 65536 || hd % 64 != 0)
        return CEV_ESHAPE;
    if (hs < hd || ws < hd || hs % 8 != 0 || ws % 8 != 0)
        return CEV_ESTRIDE;
    if (rows == 0) {
        *done = true;
        return CEV_OK;
    }
    if (!hidden || !weight)
        return CEV_ENULL;
    if (!aligned(hidden, 16) || !aligned(weight, 16))
        return CEV_EALIGN;
    const double c = 1.4426950408889634074 / temperature;
    if (!(c < 3.0e38 && c > 1.0e-37) || !(1.0 / temperature < 3.0e38))
        return CEV_ETEMP;
    return CEV_OK;
}

size_t lce_workspace_size(int64_t rows, int64_t hidden_dim, int64_t vocab)
{
    if (rows < 0 || rows > kMaxRows || vocab < 1 || vocab > kMaxVocab || hidden_dim < 64 ||
        hidden_dim % 64 != 0)
        return 0;
    const size_t fwd = (size_t)cev::lce_splits(rows, vocab) * (size_t)rows * sizeof(cev_vocab_partial);
    const size_t bwd = cev::lce_backward_workspace(rows, hidden_dim, vocab);
    return fwd > bwd ? fwd : bwd;
}

static cev::LceArgs lce_args(const void *hidden, int64_t rows, int64_t hd, int64_t hs,
                             const void *weight, int64_t vocab, int64_t ws, const int64_t *labels,
                             int64_t ignore_index, double temperature, double eps,
                             const uint8_t *row_mask, int32_t *status)
{
    cev::LceArgs a{};
    a.hidden = static_cast<const unsigned short *>(hidden);
    a.rows = rows;
    a.hidden_dim = hd;
    a.ldh = hs;
    a.weight = static_cast<const unsigned short *>(weight);
    a.vocab = vocab;
    a.ldw = ws;
    a.labels = labels;
    a.ignore_index = ignore_index;
    a.row_mask = row_mask;
    a.temperature = temperature;
    a.label_smoothing = eps;
    a.c = (float)(1.4426950408889634074 / temperature);
    a.inv_t = (float)(1.0 / temperature);
    a.splits = cev::lce_splits(rows, vocab);
    a.ldd = cev::lce_dl_stride(vocab);
    a.status = status;
    return a;
}

// Bytes [b, e) that a row-major matrix of `rows` rows of `cols` elements
// (row stride `stride`, `es` bytes each) touches; empty for a NULL pointer.
struct Span {
    uintptr_t b, e;
};
static Span span(const void *p, int64_t rows, int64_t cols, int64_t stride, int64_t es)
{
    if (!p || rows <= 0 || cols <= 0)
        return Span{0, 0};
    const uintptr_t b = (uintptr_t)p;
    return Span{b, b + (uintptr_t)(((rows - 1) * stride + cols) * es)};
}

// Optional stored fp32 logits [rows, logits_stride]: the stride covers the
// vocabulary and keeps rows 16-byte aligned, and the buffer overlaps none of
// the other arguments' memory (`others`).
static int check_lce_logits(const float *logits, int64_t logits_stride, int64_t rows,
                            int64_t vocab, std::initializer_list<Span> others)
{
    if (!logits)
        return CEV_OK;
    if (logits_stride < vocab || logits_stride % 4 != 0)
        return CEV_ESTRIDE;
    if (!aligned(logits, 16))
        return CEV_EALIGN;
    const Span z = span(logits, rows, vocab, logits_stride, 4);
    for (const Span &o : others)
        if (o.b < z.e && z.b < o.e)
            return CEV_EALIAS;
    return CEV_OK;
}

int lce_forward(const void *hidden, int64_t rows, int64_t hidden_dim, int64_t hidden_stride,
                const void *weight, int64_t vocab, int64_t weight_stride, const int64_t *labels,
                int64_t ignore_index, double temperature, double label_smoothing,
                const uint8_t *row_mask, float *loss, void *saved, float *logp, float *entropy,
                int64_t *argmax, float *logits, int64_t logits_stride, void *workspace,
                size_t workspace_bytes, int32_t *status, cev_stream_t stream)
{
    bool done;
    int rc = check_lce(hidden, rows, hidden_dim, hidden_stride, weight, vocab, weight_stride,
                       temperature, label_smoothing, &done);
    if (rc != CEV_OK || done)
        return rc;
    if (!labels || !loss || !saved || !workspace)
        return CEV_ENULL;
    if (!aligned(labels, 8) || !aligned(loss, 4) || !aligned(saved, 16) || !aligned(logp, 4) ||
        !aligned(entropy, 4) || !aligned(argmax, 8) || !aligned(workspace, 16) ||
        !aligned(status, 4))
        return CEV_EALIGN;
    if ((rc = check_lce_logits(logits, logits_stride, rows, vocab,
                               {span(hidden, rows, hidden_dim, hidden_stride, 2),
                                span(weight, vocab, hidden_dim, weight_stride, 2),
                                span(workspace, 1, (int64_t)workspace_bytes, 0, 1)})) != CEV_OK)
        return rc;
    if (workspace_bytes < lce_workspace_size(rows, hidden_dim, vocab))
        return CEV_EWORKSPACE;
    cev::LceArgs a = lce_args(hidden, rows, hidden_dim, hidden_stride, weight, vocab,
                              weight_stride, labels, ignore_index, temperature, label_smoothing,
                              row_mask, status);
    a.partials = static_cast<cev_vocab_partial *>(workspace);
    a.logits_out = logits;
    a.ldl = logits ? logits_stride : 0;
    hipError_t e = cev::launch_lce_forward(a, entropy != nullptr, label_smoothing != 0.0,
                                           to_hip(stream));
    if (e != hipSuccess)
        return CEV_ELAUNCH;
    cev::MergeArgs m{};
    m.partials = a.partials;
    m.parts = a.splits;
    m.rows = rows;
    m.vocab = vocab;
    m.labels = labels;
    m.ignore_index = ignore_index;
    m.row_mask = row_mask;
    m.temperature = temperature;
    m.label_smoothing = label_smoothing;
    m.loss = loss;
    m.logp = logp;
    m.entropy = entropy;
    m.argmax = argmax;
    m.saved = static_cast<cev_saved *>(saved);
    m.status = status;
    return launch_status(cev::launch_vocab_merge(m, to_hip(stream)));
}

int lce_backward(const void *hidden, int64_t rows, int64_t hidden_dim, int64_t hidden_stride,
                 const void *weight, int64_t vocab, int64_t weight_stride,
                 const int64_t *labels, int64_t ignore_index, double temperature,
                 double label_smoothing, const uint8_t *row_mask, const float *g,
                 const void *saved, const float *logits, int64_t logits_stride, float *dhidden,
                 int64_t dhidden_stride, float *dweight, int64_t dweight_stride, void *workspace,
                 size_t workspace_bytes, int32_t *status, cev_stream_t stream)
{
    bool done;
    int rc = check_lce(hidden, rows, hidden_dim, hidden_stride, weight, vocab, weight_stride,
                       temperature, label_smoothing, &done);
    if (rc != CEV_OK || done)
        return rc;
    if (dhidden_stride < hidden_dim || (dweight && dweight_stride < hidden_dim))
        return CEV_ESTRIDE;
    if (!labels || !g || !saved || !dhidden || !workspace)
        return CEV_ENULL;
    if (!aligned(labels, 8) || !aligned(g, 4) || !aligned(saved, 16) || !aligned(dhidden, 4) ||
        !aligned(dweight, 4) || !aligned(workspace, 16) || !aligned(status, 4))
        return CEV_EALIGN;
    if ((rc = check_lce_logits(logits, logits_stride, rows, vocab,
                               {span(dhidden, rows, hidden_dim, dhidden_stride, 4),
                                span(dweight, vocab, hidden_dim, dweight_stride, 4),
                                span(workspace, 1, (int64_t)workspace_bytes, 0, 1)})) != CEV_OK)
        return rc;
    if (workspace_bytes < lce_workspace_size(rows, hidden_dim, vocab))
        return CEV_EWORKSPACE;
    cev::LceArgs a = lce_args(hidden, rows, hidden_dim, hidden_stride, weight, vocab,
                              weight_stride, labels, ignore_index, temperature, label_smoothing,
                              row_mask, status);
    a.g = g;
    a.saved = static_cast<const cev_saved *>(saved);
    a.logits_in = logits;
    a.ldl = logits ? logits_stride : 0;
    return launch_status(cev::launch_lce_backward(a, workspace, dhidden, dhidden_stride,
                                                  dweight, dweight_stride, to_hip(stream)));
}

// Checks shared by the two JSD entry points.
static int check_jsd(const void *student, const void *teacher, int64_t rows, int64_t vocab,
                     int64_t s_stride, int64_t t_stride, int dtype, double temperature,
                     double beta, bool *done)
{
    int rc = check_common(student, rows, vocab, s_stride, dtype, temperature, done);
    if (rc != CEV_OK)
        return rc;
    if (!(std::isfinite(beta) && beta >= 0.0 && beta <= 1.0))
        return CEV_EBETA;
    if (t_stride < vocab)
        return CEV_ESTRIDE;
    if (*done)
        return CEV_OK;
    if (t_stride > INT64_MAX / 4 / rows)
        return CEV_ESHAPE;
    if (!teacher)
        return CEV_ENULL;
    if (!aligned(teacher, (uintptr_t)elem_size(dtype)))
        return CEV_EALIGN;
    return CEV_OK;
}

// Every row of the matrix starts 16 bytes aligned.
static bool rows16(const void *p, int64_t stride, int es)
{
    return aligned(p, 16) && (stride * es) % 16 == 0;
}

static cev::JsdArgs jsd_args(const void *student, const void *teacher, int64_t rows,
                             int64_t vocab, int64_t s_stride, int64_t t_stride,
                             const int64_t *labels, int64_t ignore_index, double temperature,
                             double beta, const uint8_t *row_mask, int32_t *status)
{
    cev::JsdArgs a{};
    a.student = student;
    a.teacher = teacher;
    a.rows = rows;
    a.vocab = vocab;
    a.s_stride = s_stride;
    a.t_stride = t_stride;
    a.labels = labels;
    a.ignore_index = ignore_index;
    a.row_mask = row_mask;
    a.beta = beta;
    a.c = (float)(1.4426950408889634074 / temperature);
    a.inv_t = (float)(1.0 / temperature);
    a.status = status;
    return a;
}

int jsd_forward(const void *student, const void *teacher, int64_t rows, int64_t vocab,
                int64_t student_stride, int64_t teacher_stride, int dtype,
                const int64_t *labels, int64_t ignore_index, double temperature, double beta,
                const uint8_t *row_mask, float *loss, void *saved, int32_t *status,
                cev_stream_t stream)
{
    bool done;
    int rc = check_jsd(student, teacher, rows, vocab, student_stride, teacher_stride, dtype,
                       temperature, beta, &done);
    if (rc != CEV_OK || done)
        return rc;
    if (!loss || !saved)
        return CEV_ENULL;
    if (!aligned(labels, 8) || !aligned(loss, 4) || !aligned(saved, 16) || !aligned(status, 4))
        return CEV_EALIGN;
    cev::JsdArgs a = jsd_args(student, teacher, rows, vocab, student_stride, teacher_stride,
                              labels, ignore_index, temperature, beta, row_mask, status);
    const int es = elem_size(dtype);
    a.vec = rows16(student, student_stride, es) && rows16(teacher, teacher_stride, es);
    a.loss = loss;
    a.saved = static_cast<cev_jsd_saved *>(saved);
    return launch_status(cev::launch_jsd_forward(dtype, a, to_hip(stream)));
}

int jsd_backward(const void *student, const void *teacher, int64_t rows, int64_t vocab,
                 int64_t student_stride, int64_t teacher_stride, int dtype,
                 const int64_t *labels, int64_t ignore_index, double temperature, double beta,
                 const uint8_t *row_mask, const float *g, const void *saved, void *dstudent,
                 int64_t dstudent_stride, int32_t *status, cev_stream_t stream)
{
    bool done;
    int rc = check_jsd(student, teacher, rows, vocab, student_stride, teacher_stride, dtype,
                       temperature, beta, &done);
    if (rc != CEV_OK)
        return rc;
    if (dstudent_stride < vocab)
        return CEV_ESTRIDE;
    if (done)
        return CEV_OK;
    if (!g || !saved || !dstudent)
        return CEV_ENULL;
    const int es = elem_size(dtype);
    if (!aligned(labels, 8) || !aligned(g, 4) || !aligned(saved, 16) || !aligned(status, 4) ||
        !aligned(dstudent, (uintptr_t)es))
        return CEV_EALIGN;
    if (overlaps(student, student_stride, dstudent, dstudent_stride, rows, vocab, es) ||
        overlaps(teacher, teacher_stride, dstudent, dstudent_stride, rows, vocab, es))
        return CEV_EALIAS;
    cev::JsdArgs a = jsd_args(student, teacher, rows, vocab, student_stride, teacher_stride,
                              labels, ignore_index, temperature, beta, row_mask, status);
    a.vec = rows16(student, student_stride, es) && rows16(teacher, teacher_stride, es) &&
            rows16(dstudent, dstudent_stride, es);
    a.g = g;
    a.saved_in = static_cast<const cev_jsd_saved *>(saved);
    a.dstudent = dstudent;
    a.d_stride = dstudent_stride;
    return launch_status(cev::launch_jsd_backward(dtype, a, to_hip(stream)));
}

const char *cev_status_string(int code)
{
    switch (code) {
    case CEV_OK: return "ok";
    case CEV_ENULL: return "a required pointer is NULL";
    case CEV_ESHAPE: return "invalid shape: rows < 0, vocab < 1, K outside [1, 1024], or a size overflows";
    case CEV_ESTRIDE: return "a row stride is smaller than the row";
    case CEV_EALIGN: return "a pointer is not aligned to its element size";
    case CEV_EDTYPE: return "unknown dtype (expected CEV_F32 or CEV_BF16)";
    case CEV_ETEMP: return "temperature must be finite and > 0";
    case CEV_EWORKSPACE: return "workspace smaller than cev_workspace_size(rows)";
    case CEV_EALIAS: return "an output overlaps an input it is computed from";
    case CEV_ELAUNCH: return "kernel launch failed";
    case CEV_ESMOOTH: return "label_smoothing must be finite and in [0, 1]";
    case CEV_EBETA: return "beta must be finite and in [0, 1]";
    case CEV_ESCRATCH: return "ce_forward_noalloc: the call needs more workspace than the static "
                              "scratch holds, or its device address could not be looked up";
    default: return "unknown error code";
    }
}

int cev_version(void) { return 210; }

} // extern "C"
