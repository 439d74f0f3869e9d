/*
 * oracle_cev.c -- fp64 CPU oracle for row-wise selective log-softmax and
 * cross-entropy over a [rows, vocab] logit matrix.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load this file's library. The product path
 * (the HIP library) never links, calls or reads it, and this file shares no
 * code, header or constant with that path.
 *
 * Everything is the plain definition in double precision, written in the
 * collapse-safe arrangement that the Liger-Kernel PR #1555 page ("Fix softmax
 * collapse in CE, GRPO, KL/JSD and softmax", Details) uses for its own fp64
 * reference: the loss is softplus(lse over the non-target classes - x_target),
 * because plain fp64 cross-entropy itself reads 0 once the target leads by more
 * than about 36.7.  No blocking, fusion or reordering beyond that: one row at a
 * time, one column at a time.
 *
 * Notation (per row r): z_j the stored logit (fp32, or bf16 widened exactly),
 * T the temperature, x_j = z_j / T, t the label.
 *
 * A row is valid when its mask byte is non-zero (or there is no mask), its
 * label differs from ignore_index and lies in [0, V).  A label outside [0, V)
 * that is not ignore_index sets ORACLE_BAD_LABEL in the returned status and the
 * row is treated as ignored.  Ignored rows produce zero outputs and argmax -1
 * (ms-swift PR #10353, PR information: zero upstream weights for ignored labels,
 * losses scattered back to the per-token shape).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_BAD_LABEL 1
#define ORACLE_BAD_INDEX 2

/* Widen one stored element to double.  dtype 0 = fp32, 1 = bf16 (the upper
 * 16 bits of an IEEE binary32), 2 = fp64 (logits formed in double, as the
 * product of a hidden state and a head), so the widening is exact in all
 * cases. */
static double load_z(const void *row, int dtype, int64_t j)
{
    if (dtype == 2)
        return ((const double *)row)[j];
    if (dtype == 0)
        return (double)((const float *)row)[j];
    uint32_t w = (uint32_t)((const uint16_t *)row)[j] << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

static const void *row_ptr(const void *logits, int dtype, int64_t row_stride, int64_t r)
{
    size_t esz = dtype == 2 ? 8 : (dtype == 0 ? 4 : 2);
    return (const char *)logits + (size_t)r * (size_t)row_stride * esz;
}

/* softplus(u) = log(1 + e^u), written as max(u,0) + log1p(e^-|u|) so that it
 * neither overflows for large u nor loses e^u for very negative u. */
static double softplus(double u)
{
    if (u == -INFINITY)
        return 0.0;
    return fmax(u, 0.0) + log1p(exp(-fabs(u)));
}

/* sigmoid(u) = 1 / (1 + e^-u); for u < 0 as e^u / (1 + e^u) to keep e^u. */
static double sigmoid(double u)
{
    if (u < 0.0) {
        double e = exp(u);
        return e / (1.0 + e);
    }
    return 1.0 / (1.0 + exp(-u));
}

static int row_valid(int64_t label, int64_t V, int64_t ignore_index, const uint8_t *row_mask,
                     int64_t r, int *status)
{
    if (row_mask && row_mask[r] == 0)
        return 0;
    if (label == ignore_index)
        return 0;
    if (label < 0 || label >= V) {
        *status |= ORACLE_BAD_LABEL;
        return 0;
    }
    return 1;
}

/* Stable list of the valid rows in ascending order; returns their count.
 * (ms-swift PR #10353, PR information: supervised rows are selected before the
 * cross-entropy and the losses are scattered back afterwards.) */
int64_t oracle_valid_rows(const int64_t *labels, const uint8_t *row_mask, int64_t rows,
                          int64_t vocab, int64_t ignore_index, int64_t *out, int32_t *status)
{
    int st = 0;
    int64_t n = 0;
    for (int64_t r = 0; r < rows; ++r)
        if (row_valid(labels[r], vocab, ignore_index, row_mask, r, &st))
            out[n++] = r;
    if (status)
        *status |= st;
    return n;
}

/* log sum_{j != excl} exp(x_j), x_j = z_j / T, shifted by the maximum of the
 * terms it sums.  Returns -inf for an empty sum. */
static double lse_excluding(const void *row, int dtype, int64_t V, double T, int64_t excl)
{
    double m = -INFINITY;
    for (int64_t j = 0; j < V; ++j)
        if (j != excl) {
            double x = load_z(row, dtype, j) / T;
            if (x > m)
                m = x;
        }
    if (m == -INFINITY)
        return -INFINITY;
    double s = 0.0;
    for (int64_t j = 0; j < V; ++j)
        if (j != excl)
            s += exp(load_z(row, dtype, j) / T - m);
    return m + log(s);
}

/*
 * Per-row forward for rows [r0, r1): log p_t, loss, entropy, argmax and
 * q = 1 - p_t.  Any output pointer may be NULL.  Outputs are indexed by the
 * absolute row r.
 *
 *  - loss = -log p_t = softplus(u), u = lse_{j != t}(x) - x_t
 *    (Liger PR #1555, Summary, CE/FLCE bullet: loss from the sum without the
 *    target; Details: the fp64 reference form softplus(lse_others - x_y));
 *    with label smoothing eps (the unsloth-zoo #2080 Summary quoted on the
 *    Liger page keeps smoothing in the collapse-safe target term):
 *    loss = (1 - eps)(-log p_t) + (eps / V) sum_j (-log p_j).
 *  - q = 1 - p_t = sigmoid(u) = s_others / d (same bullet: dx_y = -sum_others/d).
 *  - entropy H = -sum_j p_j log p_j, with log p_t = -loss and, for j != t,
 *    log p_j = x_j - lse, lse = x_t + loss.
 *  - argmax = lowest j with z_j = max_k z_k, compared on the stored values.
 */
int oracle_ce_rows(const void *logits, int64_t rows, int64_t vocab, int64_t row_stride, int dtype,
                   const int64_t *labels, int64_t ignore_index, double T, double eps,
                   const uint8_t *row_mask, int64_t r0, int64_t r1, double *logp, double *loss,
                   double *entropy, int64_t *argmax, double *q)
{
    int st = 0;
    (void)rows;
    for (int64_t r = r0; r < r1; ++r) {
        const void *row = row_ptr(logits, dtype, row_stride, r);
        int64_t t = labels[r];
        if (!row_valid(t, vocab, ignore_index, row_mask, r, &st)) {
            if (logp) logp[r] = 0.0;
            if (loss) loss[r] = 0.0;
            if (entropy) entropy[r] = 0.0;
            if (argmax) argmax[r] = -1;
            if (q) q[r] = 0.0;
            continue;
        }
        double xt = load_z(row, dtype, t) / T;
        double u = lse_excluding(row, dtype, vocab, T, t) - xt;
        double l = softplus(u);
        if (logp) logp[r] = -l;
        if (loss) {
            /* label smoothing: (1 - eps) (-log p_t) + eps * mean_j (-log p_j),
             * with -log p_j = lse - x_j and lse = x_t + l */
            double ls = 0.0;
            if (eps != 0.0) {
                double lse = xt + l;
                for (int64_t j = 0; j < vocab; ++j)
                    ls += lse - load_z(row, dtype, j) / T;
                ls /= (double)vocab;
            }
            loss[r] = (1.0 - eps) * l + eps * ls;
        }
        if (q) q[r] = sigmoid(u);
        if (entropy) {
            double lse = xt + l;
            double h = exp(-l) * l;
            for (int64_t j = 0; j < vocab; ++j)
                if (j != t) {
                    double x = load_z(row, dtype, j) / T;
                    h += exp(x - lse) * (lse - x);
                }
            entropy[r] = h;
        }
        if (argmax) {
            int64_t a = 0;
            double best = load_z(row, dtype, 0);
            for (int64_t j = 1; j < vocab; ++j) {
                double z = load_z(row, dtype, j);
                if (z > best) {
                    best = z;
                    a = j;
                }
            }
            argmax[r] = a;
        }
    }
    return st;
}

/*
 * Gradient rows [r0, r1) of the per-row loss with respect to the stored logits:
 * dl_j = (g_r / T) (p_j - (1 - eps) [j == t] - eps / V), with the target
 * column taken as (g_r / T)(-q + eps - eps / V), q = 1 - p_t = sigmoid(u), so
 * no 1 - p_t is ever formed by subtraction (ms-swift PR #10353, PR information: backward as
 * g*softmax - g*one_hot with zero weight for ignored labels; Liger PR #1555,
 * Summary: dx_y = -sum_others/d).  out has (r1 - r0) rows of vocab doubles;
 * ignored rows are all zero.
 */
int oracle_ce_grad_rows(const void *logits, int64_t rows, int64_t vocab, int64_t row_stride,
                        int dtype, const int64_t *labels, int64_t ignore_index, double T,
                        double eps, const uint8_t *row_mask, const double *g, int64_t r0,
                        int64_t r1, double *out)
{
    int st = 0;
    (void)rows;
    for (int64_t r = r0; r < r1; ++r) {
        const void *row = row_ptr(logits, dtype, row_stride, r);
        double *o = out + (size_t)(r - r0) * (size_t)vocab;
        int64_t t = labels[r];
        if (!row_valid(t, vocab, ignore_index, row_mask, r, &st)) {
            for (int64_t j = 0; j < vocab; ++j)
                o[j] = 0.0;
            continue;
        }
        double xt = load_z(row, dtype, t) / T;
        double u = lse_excluding(row, dtype, vocab, T, t) - xt;
        double lse = xt + softplus(u);
        double w = g[r] / T;
        double ev = eps / (double)vocab;
        for (int64_t j = 0; j < vocab; ++j)
            o[j] = j == t ? w * (-sigmoid(u) + eps - ev)
                          : w * (exp(load_z(row, dtype, j) / T - lse) - ev);
    }
    return st;
}

/*
 * Selective log-softmax at K gathered indices per row (ms-swift PR #10337,
 * PR information: gather(log_softmax(logits / T), index) with top-K indices,
 * temperature and row_mask), in the same collapse-safe form as the single
 * target: log p_k = -softplus(lse_{j != i_k}(x) - x_{i_k}).
 * idx is [rows, K] with row stride idx_stride; logp_out is [rows, K] dense.
 * An entry equal to ignore_index, and every entry of a masked row, gives 0.
 * An entry outside [0, V) gives 0 and sets ORACLE_BAD_INDEX.  q_out (nullable,
 * [rows, K]) receives 1 - p at each gathered index as sigmoid(u), 0 for
 * entries that give 0.
 */
int oracle_topk_rows(const void *logits, int64_t rows, int64_t vocab, int64_t row_stride, int dtype,
                     const int64_t *idx, int64_t K, int64_t idx_stride, int64_t ignore_index,
                     double T, const uint8_t *row_mask, int64_t r0, int64_t r1, double *logp_out,
                     double *q_out)
{
    int st = 0;
    (void)rows;
    for (int64_t r = r0; r < r1; ++r) {
        const void *row = row_ptr(logits, dtype, row_stride, r);
        for (int64_t k = 0; k < K; ++k) {
            int64_t i = idx[r * idx_stride + k];
            double v = 0.0, qk = 0.0;
            if (row_mask && row_mask[r] == 0) {
                v = 0.0;
            } else if (i == ignore_index) {
                v = 0.0;
            } else if (i < 0 || i >= vocab) {
                st |= ORACLE_BAD_INDEX;
                v = 0.0;
            } else {
                double xi = load_z(row, dtype, i) / T;
                double u = lse_excluding(row, dtype, vocab, T, i) - xi;
                v = -softplus(u);
                qk = sigmoid(u);
            }
            if (q_out)
                q_out[r * K + k] = qk;
            logp_out[r * K + k] = v;
        }
    }
    return st;
}

/*
 * Gradient rows [r0, r1) of L = sum_k g[r, k] log p_{i_k} (the top-K
 * selective log-softmax) with respect to the stored logits:
 * dL/dz_j = (1/T) sum_k g_k ([j = i_k] - p_j).  At a gathered column j the
 * two terms combine to (1/T)(G_j (1 - p_j) - p_j (Gs - G_j)), G_j the sum of
 * the g_k gathered at j, Gs the sum over all valid entries; 1 - p_j is taken
 * as sigmoid(lse_{m != j}(x) - x_j), never by subtraction (the same
 * collapse-safe rule as the single target).  Ignored or out-of-range entries
 * contribute nothing; masked rows are zero.  g is [rows, K] dense; out has
 * (r1 - r0) rows of vocab doubles.
 */
int oracle_topk_grad_rows(const void *logits, int64_t rows, int64_t vocab, int64_t row_stride,
                          int dtype, const int64_t *idx, int64_t K, int64_t idx_stride,
                          int64_t ignore_index, double T, const uint8_t *row_mask,
                          const double *g, int64_t r0, int64_t r1, double *out)
{
    int st = 0;
    (void)rows;
    for (int64_t r = r0; r < r1; ++r) {
        const void *row = row_ptr(logits, dtype, row_stride, r);
        double *o = out + (size_t)(r - r0) * (size_t)vocab;
        for (int64_t j = 0; j < vocab; ++j)
            o[j] = 0.0;
        if (row_mask && row_mask[r] == 0)
            continue;
        double gs = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            int64_t i = idx[r * idx_stride + k];
            if (i == ignore_index)
                continue;
            if (i < 0 || i >= vocab) {
                st |= ORACLE_BAD_INDEX;
                continue;
            }
            gs += g[r * K + k];
        }
        double lse = lse_excluding(row, dtype, vocab, T, -1);
        for (int64_t j = 0; j < vocab; ++j)
            o[j] = -(gs / T) * exp(load_z(row, dtype, j) / T - lse);
        for (int64_t k = 0; k < K; ++k) {
            int64_t i = idx[r * idx_stride + k];
            if (i == ignore_index || i < 0 || i >= vocab)
                continue;
            int first = 1;
            for (int64_t k2 = 0; k2 < k; ++k2)
                if (idx[r * idx_stride + k2] == i)
                    first = 0;
            if (!first)
                continue;
            double gj = 0.0;
            for (int64_t k2 = k; k2 < K; ++k2)
                if (idx[r * idx_stride + k2] == i)
                    gj += g[r * K + k2];
            double xi = load_z(row, dtype, i) / T;
            double qj = sigmoid(lse_excluding(row, dtype, vocab, T, i) - xi);
            double pj = exp(xi - lse);
            o[i] = (gj * qj - pj * (gs - gj)) / T;
        }
    }
    return st;
}
