// sweep.hip -- forward vocab sweeps for gfx950: one workgroup per row, one HBM
// pass over the row, target-excluded online softmax statistics in fp32, and a
// per-row closing step in fp64.
//
// The form follows Liger-Kernel PR #1555 ("Fix softmax collapse in CE, GRPO,
// KL/JSD and softmax"), Summary, CE/FLCE bullet: the first pass accumulates the
// sum WITHOUT the target, and the loss is softplus(log(sum_others) + m - x_t),
// so e^0 = 1 is never added to e^{-margin}.  Unlike the pages' Triton kernels
// (which skip the target's whole block and re-read it afterwards, per the
// unsloth-zoo #2080 Summary quoted there), the sweep here excludes the target
// per 16-byte vector: a wave-uniform range test per step, with a per-element
// mask only in the one step that holds the target.  The sum is based at m_o,
// the largest NON-target logit, so it is >= 1 and cannot underflow to zero
// even when every other term is below the fp32 normal range.
#include "cev_compact.h"
#include "cev_device.h"
#include "cev_launch.h"
#include "cev_rowclose.h"
#include "cev_sweep_row.h"

namespace cev {
namespace {


// Per-row closing step (cev_rowclose.h) with the sweep's outputs; zt is the
// stored target logit.
template <bool WANT_H, bool WANT_ARG>
__device__ void close_row(const SweepArgs &a, int64_t r, float zt, int64_t t, float M, double S,
                          double Hs, double Zs, int64_t a_o)
{
    RowOutputs o;
    o.logp = a.logp;
    o.loss = a.loss;
    o.entropy = WANT_H ? a.entropy : nullptr;
    o.argmax = WANT_ARG ? a.argmax : nullptr;
    o.saved = a.saved;
    close_row_fp64(o, r, zt, t, M, S, Hs, a_o, a.temperature, Zs, a.label_smoothing, a.vocab);
}

// Row of block b in a swizzled every-row sweep.  Workgroup b runs on XCD
// b % 8; within each whole group of 8 blocks the rows are rotated by a hash
// of the group index (Fibonacci hashing, the top 3 bits of g * 2^32/phi), so
// that the rows a periodic mask ignores (every 2nd ... 100th) land on all
// XCDs about equally -- in row order every 10th row would fall on 4 of the 8
// -- while each group still covers 8 neighbouring rows.
__device__ __forceinline__ int64_t swizzle_row(int64_t b, int64_t rows)
{
    if (b >= (rows & ~(int64_t)7))
        return b;
    const uint32_t rot = ((uint32_t)((uint64_t)b >> 3) * 0x9E3779B1u) >> 29;
    return (b & ~(int64_t)7) | ((b + rot) & 7);
}

// ------------------------------------------------------------------------
// Single-target sweep: sls_forward and the sweep stage of ce_forward.  With
// SPLIT, `a.splits` workgroups share one row (block b * splits + p takes part
// p of compacted row b) and each writes a partial record for k_merge instead
// of closing the row.  Otherwise block b takes row b (rotated within groups
// of 8 when a.swizzle is set; ignored rows only write their zero outputs);
// with a.out_list set, the blocks after the
// last row compact the valid rows into it (they are dispatched last, so the
// compaction overlaps the final rows' sweeps and costs no launch of its own).
template <int DT, int BLOCK, int U, bool WANT_H, bool WANT_ARG, bool SPLIT, bool WANT_Z>
__global__ __launch_bounds__(BLOCK) void k_sls_sweep(SweepArgs a)
{
    constexpr int ES = Elem<DT>::kSize, W = BLOCK / kWave;
    __shared__ float sh_f[W];
    __shared__ double sh_d[3 * W];
    __shared__ int64_t sh_i[W];
    __shared__ int sh_c[W];
    const int tid = threadIdx.x;

    if constexpr (!SPLIT) {
        if (a.out_list && (int64_t)blockIdx.x >= a.rows) {
            CompactTile c;
            c.labels = a.labels;
            c.row_mask = a.row_mask;
            c.ignore_index = a.ignore_index;
            c.vocab = a.vocab;
            c.rows = a.rows;
            c.tile = compact_tile_rows(a.rows, BLOCK);
            c.ntiles = (a.rows + c.tile - 1) / c.tile;
            c.list = a.out_list;
            c.count = a.out_count;
            compact_tile<BLOCK>(c, (int64_t)blockIdx.x - a.rows, sh_c);
            return;
        }
    }

    int64_t b = blockIdx.x, part = 0, parts = 1;
    int64_t r;
    if constexpr (SPLIT) {
        // compacted rows (all valid), `splits` workgroups per row
        parts = a.splits;
        b = blockIdx.x / parts;
        part = blockIdx.x % parts;
        if (b >= load_uniform(a.nlist))
            return;
        r = load_uniform(a.rowlist + b);
    } else {
        r = a.swizzle ? swizzle_row(b, a.rows) : b;
    }
    const int64_t V = a.vocab;
    const char *rowp = static_cast<const char *>(a.logits) + (size_t)r * (size_t)a.row_stride * ES;
    const int64_t t = load_uniform(a.labels + r);
    if constexpr (!SPLIT) {
        const bool masked = a.row_mask && mask_byte(a.row_mask, r) == 0;
        const bool ignored = masked || t == a.ignore_index;
        const bool bad = !ignored && (t < 0 || t >= V);
        if (ignored || bad) {
            if (tid == 0) {
                if (a.logp)
                    a.logp[r] = 0.0f;
                if (a.loss)
                    a.loss[r] = 0.0f;
                if (a.entropy)
                    a.entropy[r] = 0.0f;
                if (a.argmax)
                    a.argmax[r] = -1;
                if (a.saved) {
                    cev_saved z;
                    z.m_z = 0.0f;
                    z.log2_d = 0.0f;
                    z.q = 0.0f;
                    z.flags = 0;
                    a.saved[r] = z;
                }
                if (bad && a.status)
                    atomicOr(a.status, (int32_t)CEV_STATUS_BAD_LABEL);
            }
            return;
        }
    }

    // Issuing the first step before the label and mask are known was measured
    // (8192 x 152064 bf16, 10% masked: 336-338 against 335 us; no gain where
    // no row is ignored): the dropped loads of ignored rows cost more than the
    // label's round trip, which the other rows in flight already hide.
    const RowStats rs = sweep_row<DT, BLOCK, U, WANT_H, WANT_ARG, true, WANT_Z, !SPLIT>(
        rowp, V, t, part, parts, a.c, a.inv_t, sh_f, sh_d, sh_i);
    const float M = rs.M;
    const double S = rs.S, Hs = rs.Hs, Zs = rs.Zs;
    const int64_t a_o = rs.a_o;

    if (tid == 0) {
        if constexpr (SPLIT) {
            SplitPartial pr;
            pr.m = M;
            pr.pad = 0;
            pr.arg = a_o;
            pr.s = S;
            pr.h = Hs;
            pr.zs = Zs;
            static_cast<SplitPartial *>(a.partials)[b * parts + part] = pr;
        } else {
            close_row<WANT_H, WANT_ARG>(a, r, rs.zt, t, M, S, Hs, Zs, a_o);
        }
    }
}

// Merge of a row's split partials (fixed order, fp64), then the closing step,
// by one wave: lane l reads parts l, l + 64, ...  Part p holds, over its
// columns, the largest non-target logit m_p, its lowest column, the sum S_p
// based at B_p = max(m_p, -FLT_MAX) and the entropy term H_p at the same
// base; moving to the common base B multiplies both by e^{(B_p - B)/T} and
// adds (B - B_p)/T * S_p to H_p (the partial/combine rescaling of the
// unsloth-zoo #2080 Summary quoted on the Liger-Kernel PR #1555 page).
template <int DT, bool WANT_H, bool WANT_ARG>
__device__ __forceinline__ void merge_close(const SweepArgs &a, int64_t r, const SplitPartial *pp,
                                            int parts, int lane)
{
    float m = -INFINITY;
    for (int p = lane; p < parts; p += kWave)
        m = fmaxf(m, pp[p].m);
    const float M = wave_max(m);
    const float B = fmaxf(M, -FLT_MAX);
    const double T = a.temperature;
    double S = 0.0, H = 0.0, Z = 0.0;
    int64_t arg = INT64_MAX;
    for (int p = lane; p < parts; p += kWave) {
        const SplitPartial pr = pp[p];
        Z += pr.zs;
        if (pr.s > 0.0) {
            const double bp = (double)fmaxf(pr.m, -FLT_MAX);
            const double f = exp((bp - (double)B) / T);
            S += pr.s * f;
            if constexpr (WANT_H)
                H += f * (pr.h + ((double)B - bp) / T * pr.s);
        }
        if (pr.m == M && pr.arg < arg)
            arg = pr.arg;
    }
    S = wave_sum(S);
    Z = wave_sum(Z);
    if constexpr (WANT_H)
        H = wave_sum(H);
    if constexpr (WANT_ARG)
        arg = wave_min(arg);
    if (lane == 0) {
        const char *rowp = static_cast<const char *>(a.logits) +
                           (size_t)r * (size_t)a.row_stride * Elem<DT>::kSize;
        const int64_t t = a.labels[r];
        close_row<WANT_H, WANT_ARG>(a, r, load_elem<DT>(rowp, t), t, M, S, H, Z, arg);
    }
}

// The split-row merge as its own launch: one wave per compacted row.
template <int DT, bool WANT_H, bool WANT_ARG>
__global__ __launch_bounds__(256) void k_merge(SweepArgs a)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t b = (int64_t)blockIdx.x * (256 / kWave) + threadIdx.x / kWave;
    if (b >= *a.nlist)
        return;
    merge_close<DT, WANT_H, WANT_ARG>(a, a.rowlist[b], static_cast<const SplitPartial *>(a.partials) +
                                                          b * a.splits, (int)a.splits, lane);
}

// ------------------------------------------------------------------------
// Top-K sweep: the sum runs over the columns outside the gathered set; each
// gathered column's complement is that sum plus the other gathered terms.

// One gathered index's closing step in fp64: s = the sum of the other columns'
// terms based at B, zk the index's stored value.  log p = -softplus(u) and
// q = 1 - p = sigmoid(u), u = log s + (B - zk)/T, both from one e^{-|u|}.
// Kept out of line: inlined into the per-index loop, its fp64 constants were
// hoisted into vector registers that stayed live across the whole kernel.
__device__ __noinline__ void topk_close(double s, double B, double zk, double T, float *logp,
                                        float *q)
{
    const double u = s > 0.0 ? log(s) + (B - zk) / T : -INFINITY;
    const double e = exp(-fabs(u));
    *logp = (float)(-(fmax(u, 0.0) + log1p(e)));
    if (q)
        *q = (float)((u < 0.0 ? e : 1.0) / (1.0 + e));
}
// Masks gathered column x in a wave step whose first column is lo: a column
// at offset d sits in lane (d / VE) % 64, vector d / (64 VE) of the lane,
// element d % VE.
template <int DT, int U>
__device__ __forceinline__ void mask_gathered(float (&v)[U * Elem<DT>::kVE], int64_t x, int64_t lo,
                                              int lane)
{
    constexpr int VE = Elem<DT>::kVE;
    const int64_t d = x - lo;
    if (x >= 0 && (uint64_t)d < (uint64_t)((int64_t)kWave * U * VE)) {
        const int dd = (int)d;
        if (((dd / VE) & (kWave - 1)) == lane) {
            const int i = (dd / (kWave * VE)) * VE + dd % VE;
#pragma unroll
            for (int j = 0; j < U * VE; ++j)
                if (j == i)
                    v[j] = -INFINITY;
        }
    }
}

// SMALLK (K <= 64): every wave holds the K gathered columns in its lanes
// (lane k: column k, -1 if ignored or out of range), read straight from the
// index row, so the sweep starts one round trip after the row does and needs
// no LDS for its exclusion tests; the gathered values are loaded while the
// sweep runs and only the closing step reads them.  Otherwise the columns go
// through LDS first.
template <int DT, int BLOCK, int U, bool SMALLK>
__global__ __launch_bounds__(BLOCK) void k_topk_sweep(SweepArgs a)
{
    constexpr int VE = Elem<DT>::kVE, ES = Elem<DT>::kSize, W = BLOCK / kWave;
    constexpr int64_t CH = (int64_t)kWave * U;
    __shared__ float sh_f[2 * W];
    __shared__ double sh_d[W];
    // Dynamic LDS sized by K: the gathered columns, their values and terms,
    // and first-occurrence flags (K <= 1024, checked on the host).
    extern __shared__ __align__(16) unsigned char xlds[];
    int64_t *xcol = reinterpret_cast<int64_t *>(xlds);
    double *xterm = reinterpret_cast<double *>(xcol + a.K);
    float *xz = reinterpret_cast<float *>(xterm + a.K);
    unsigned char *xfirst = reinterpret_cast<unsigned char *>(xz + a.K);
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int64_t r = blockIdx.x;
    const int64_t V = a.vocab;
    const int K = (int)a.K;
    float *out = a.logp + (size_t)r * (size_t)K;

    float *qout = a.q ? a.q + (size_t)r * (size_t)K : nullptr;
    if (a.row_mask && mask_byte(a.row_mask, r) == 0) {
        for (int k = tid; k < K; k += BLOCK) {
            out[k] = 0.0f;
            if (qout)
                qout[k] = 0.0f;
        }
        if (a.saved && tid == 0) {
            cev_saved z;
            z.m_z = 0.0f;
            z.log2_d = 0.0f;
            z.q = 0.0f;
            z.flags = 0;
            a.saved[r] = z;
        }
        return;
    }
    const char *rowp = static_cast<const char *>(a.logits) + (size_t)r * (size_t)a.row_stride * ES;
    const int64_t *irow = a.indices + (size_t)r * (size_t)a.index_row_stride;
    // The wave's first step of the row goes out before the gathered indices
    // are read, so the stream is in flight during that round trip.
    const RowGeom g = row_geom<DT, U>(rowp, V, 0, 1);
    const u32x4 *vp = reinterpret_cast<const u32x4 *>(rowp + (size_t)g.ahead * ES);
    u32x4 cur[U], nxt[U];
    if (wave < g.nfull) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            cur[u] = load16_stream(vp + (int64_t)wave * CH + u * kWave + lane);
    }

    int64_t mycol = -1;   // SMALLK: this lane's gathered column
    float myz = -INFINITY;
    if constexpr (SMALLK) {
        if (lane < K) {
            const int64_t i = irow[lane];
            const bool ok = i != a.ignore_index && i >= 0 && i < V;
            if (wave == 0 && i != a.ignore_index && !ok && a.status)
                atomicOr(a.status, (int32_t)CEV_STATUS_BAD_INDEX);
            mycol = ok ? i : -1;
            if (ok)
                myz = load_elem<DT>(rowp, i);   // used after the sweep
        }
    } else {
        bool bad = false;
        for (int k = tid; k < K; k += BLOCK) {
            const int64_t i = irow[k];
            const bool ok = i != a.ignore_index && i >= 0 && i < V;
            bad |= (i != a.ignore_index && !ok);
            xcol[k] = ok ? i : -1;
            xz[k] = ok ? load_elem<DT>(rowp, i) : -INFINITY;
        }
        if (bad && a.status)
            atomicOr(a.status, (int32_t)CEV_STATUS_BAD_INDEX);
        __syncthreads();
        for (int k = tid; k < K; k += BLOCK) {
            bool first = xcol[k] >= 0;
            for (int k2 = 0; k2 < k && first; ++k2)
                first = xcol[k2] != xcol[k];
            xfirst[k] = first;
        }
        __syncthreads();
    }

    const float c = a.c;
    LaneState st{-INFINITY, 0.0f, 0.0f, 0.0f, 0.0f, -1};

    // Whether column col is gathered (per lane; the lanes' columns may differ).
    auto excluded = [&](int64_t col) {
        bool x = false;
        for (int k = 0; k < K; ++k)
            x |= (SMALLK ? lane_value(mycol, k) : xcol[k]) == col;
        return x;
    };

    if (tid < g.head) {
        float v[1] = {excluded(tid) ? -INFINITY : load_elem<DT>(rowp, tid)};
        fold<DT, 1, false, false, true>(st, v, 0, c);
    }
    {
        // Lane l holds the wave step that gathered column l falls in (-1 if
        // none), so each step's test is one compare and a ballot.
        int my_step = -1;
        if constexpr (SMALLK) {
            if (mycol >= g.ahead && mycol < g.ahead + g.nfull * CH * VE)
                my_step = (int)((mycol - g.ahead) / (CH * VE));
        }
        int64_t k = wave;
        for (; k < g.nfull; k += W) {
            const int64_t kn = k + W;
            if (kn < g.nfull) {
#pragma unroll
                for (int u = 0; u < U; ++u)
                    nxt[u] = load16_stream(vp + kn * CH + u * kWave + lane);
            }
            float v[U * VE];
            unpack_step<DT, U>(cur, v);
            const int64_t lo = g.ahead + k * CH * VE;
            bool any;
            if constexpr (SMALLK) {
                uint64_t hits = __ballot(my_step == (int)k);
                any = hits != 0;
                while (hits) {
                    const int k2 = __builtin_ctzll(hits);
                    hits &= hits - 1;
                    mask_gathered<DT, U>(v, lane_value(mycol, k2), lo, lane);
                }
            } else {
                any = false;
                for (int kk = 0; kk < K; kk += kWave) {
                    const int64_t x = kk + lane < K ? xcol[kk + lane] : -1;
                    any |= __any(x >= 0 && (uint64_t)(x - lo) < (uint64_t)(CH * VE)) != 0;
                }
                if (any)
                    for (int k2 = 0; k2 < K; ++k2)
                        mask_gathered<DT, U>(v, xcol[k2], lo, lane);
            }
            if (any)
                fold<DT, U * VE, false, false, true>(st, v, 0, c);
            else
                fold<DT, U * VE, false, false, false>(st, v, 0, c);
#pragma unroll
            for (int u = 0; u < U; ++u)
                cur[u] = nxt[u];
        }
    }
    for (int64_t j = g.nfull * CH + tid; j < g.nvec; j += BLOCK) {
        float v[VE];
        unpack16<DT>(load16_stream(vp + j), v);
#pragma unroll
        for (int e = 0; e < VE; ++e)
            if (excluded(g.ahead + j * VE + e))
                v[e] = -INFINITY;
        fold<DT, VE, false, false, true>(st, v, 0, c);
    }
    if (g.tail0 + tid < g.tail1) {
        const int64_t col = g.tail0 + tid;
        float v[1] = {excluded(col) ? -INFINITY : load_elem<DT>(rowp, col)};
        fold<DT, 1, false, false, true>(st, v, 0, c);
    }

    const double T = a.temperature;
    if constexpr (SMALLK) {
        // The maxima over the swept and the gathered columns in one exchange;
        // then wave 0's lane k closes index k from registers.
        float mx[2] = {st.m, myz};
        block_max_n<BLOCK, 2>(mx, sh_f);
        const float M = mx[0];
        const float Mall = fmaxf(mx[1], M);
        const float B = fmaxf(M, -FLT_MAX);
        const float bl = fmaxf(st.m, -FLT_MAX);
        const float f = exp2_hw((bl - B) * c);
        const double S = block_sum<BLOCK>((double)(st.s - st.comp) * (double)f, sh_d);
        if (wave != 0)
            return;
        const float Ball = fmaxf(Mall, -FLT_MAX);
        const double s_rest = S > 0.0 ? S * exp(((double)B - (double)Ball) / T) : 0.0;
        // This lane's column counts once in the others' sums when it is the
        // first occurrence of its column.
        bool first = mycol >= 0;
        for (int k2 = 0; k2 < K; ++k2)
            first = first && !(k2 < lane && lane_value(mycol, k2) == mycol);
        const double term = first ? exp(((double)myz - (double)Ball) / T) : 0.0;
        double s_mine = s_rest, d = s_rest;   // sum over the others; over all columns
        for (int k2 = 0; k2 < K; ++k2) {
            const double tk = lane_value(term, k2);
            d += tk;
            if (lane_value(mycol, k2) != mycol)
                s_mine += tk;
        }
        if (lane < K) {
            if (mycol < 0) {
                out[lane] = 0.0f;
                if (qout)
                    qout[lane] = 0.0f;
            } else {
                topk_close(s_mine, (double)Ball, (double)myz, T, out + lane,
                           qout ? qout + lane : nullptr);
            }
        }
        if (a.saved && lane == 0) {
            // The row's normaliser over all columns, for the top-K backward:
            // d = sum_j e^{(z_j - m_z)/T} with m_z the exact row maximum.
            cev_saved sv;
            sv.m_z = Mall;
            sv.log2_d = (float)(log(d) * kLog2e);
            sv.q = 0.0f;
            sv.flags = 1;
            a.saved[r] = sv;
        }
        return;
    }

    const float M = block_max<BLOCK>(st.m, sh_f);
    const float B = fmaxf(M, -FLT_MAX);
    const float bl = fmaxf(st.m, -FLT_MAX);
    const float f = exp2_hw((bl - B) * c);
    const double S = block_sum<BLOCK>((double)(st.s - st.comp) * (double)f, sh_d);
    float gm = -INFINITY;
    for (int k = tid; k < K; k += BLOCK)
        gm = fmaxf(gm, xz[k]);
    const float Mall = fmaxf(block_max<BLOCK>(gm, sh_f), M);
    const float Ball = fmaxf(Mall, -FLT_MAX);
    const double s_rest = S > 0.0 ? S * exp(((double)B - (double)Ball) / T) : 0.0;
    // Each gathered column's term e^{(z - Ball)/T}, computed once (in
    // parallel over the indices) and summed below in index order by every
    // index that needs it.
    for (int k = tid; k < K; k += BLOCK)
        xterm[k] = xfirst[k] ? exp(((double)xz[k] - (double)Ball) / T) : 0.0;
    __syncthreads();
    for (int k = tid; k < K; k += BLOCK) {
        if (xcol[k] < 0) {
            out[k] = 0.0f;
            if (qout)
                qout[k] = 0.0f;
            continue;
        }
        double s = s_rest;
        for (int k2 = 0; k2 < K; ++k2)
            if (xfirst[k2] && xcol[k2] != xcol[k])
                s += xterm[k2];
        topk_close(s, (double)Ball, (double)xz[k], T, out + k, qout ? qout + k : nullptr);
    }
    if (a.saved && tid == 0) {
        // The row's normaliser over all columns, for the top-K backward:
        // d = sum_j e^{(z_j - m_z)/T} with m_z the exact row maximum.
        double d = s_rest;
        for (int k2 = 0; k2 < K; ++k2)
            if (xfirst[k2])
                d += xterm[k2];
        cev_saved sv;
        sv.m_z = Mall;
        sv.log2_d = (float)(log(d) * kLog2e);
        sv.q = 0.0f;
        sv.flags = 1;
        a.saved[r] = sv;
    }
}

// lds: dynamic LDS reserved per workgroup (unused by the kernel), which caps
// how many workgroups a CU holds at once.
template <int DT, int BLOCK, int U, bool SPLIT, bool WANT_Z>
void launch_sls_z(const SweepArgs &a, bool want_h, bool want_arg, hipStream_t s, size_t lds = 0)
{
    int64_t extra = 0;   // compaction workgroups of an every-row sweep
    if (!SPLIT && !a.rowlist && a.out_list)
        extra = (a.rows + compact_tile_rows(a.rows, BLOCK) - 1) / compact_tile_rows(a.rows, BLOCK);
    dim3 grid((unsigned)(a.rows * (SPLIT ? a.splits : 1) + extra)), block(BLOCK);
    if (want_h && want_arg)
        hipLaunchKernelGGL((k_sls_sweep<DT, BLOCK, U, true, true, SPLIT, WANT_Z>), grid, block, lds, s, a);
    else if (want_h)
        hipLaunchKernelGGL((k_sls_sweep<DT, BLOCK, U, true, false, SPLIT, WANT_Z>), grid, block, lds, s, a);
    else if (want_arg)
        hipLaunchKernelGGL((k_sls_sweep<DT, BLOCK, U, false, true, SPLIT, WANT_Z>), grid, block, lds, s, a);
    else
        hipLaunchKernelGGL((k_sls_sweep<DT, BLOCK, U, false, false, SPLIT, WANT_Z>), grid, block, lds, s, a);
}

// The running sum of the stored values is taken only when label smoothing
// needs it.
template <int DT, int BLOCK, int U, bool SPLIT>
hipError_t launch_sls_t(const SweepArgs &a, bool want_h, bool want_arg, hipStream_t s,
                        size_t lds = 0)
{
    if (a.label_smoothing != 0.0)
        launch_sls_z<DT, BLOCK, U, SPLIT, true>(a, want_h, want_arg, s, lds);
    else
        launch_sls_z<DT, BLOCK, U, SPLIT, false>(a, want_h, want_arg, s, lds);
    return hipGetLastError();
}

template <int DT> hipError_t launch_merge_t(const SweepArgs &a, bool want_h, bool want_arg, hipStream_t s)
{
    dim3 grid((unsigned)((a.rows + 3) / 4)), block(256);
    if (want_h && want_arg)
        hipLaunchKernelGGL((k_merge<DT, true, true>), grid, block, 0, s, a);
    else if (want_h)
        hipLaunchKernelGGL((k_merge<DT, true, false>), grid, block, 0, s, a);
    else if (want_arg)
        hipLaunchKernelGGL((k_merge<DT, false, true>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((k_merge<DT, false, false>), grid, block, 0, s, a);
    return hipGetLastError();
}

} // namespace

// Launch configuration, exposed for tuning harnesses.
hipError_t launch_sls_sweep_cfg(int dtype, const SweepArgs &a, bool want_h, bool want_arg,
                                int block, int U, hipStream_t s)
{
#define CEV_SLS_CASE(B, UU)                                                                     \
    if (block == B && U == UU)                                                                  \
        return dtype == CEV_BF16 ? launch_sls_t<CEV_BF16, B, UU, false>(a, want_h, want_arg, s) \
                                 : launch_sls_t<CEV_F32, B, UU, false>(a, want_h, want_arg, s);
    CEV_SLS_CASE(64, 4)
    CEV_SLS_CASE(128, 4)
    CEV_SLS_CASE(256, 2)
    CEV_SLS_CASE(256, 4)
    CEV_SLS_CASE(512, 2)
    CEV_SLS_CASE(512, 4)
#undef CEV_SLS_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_sls_sweep_lds_cfg(int dtype, const SweepArgs &a, bool want_h, bool want_arg,
                                    int block, int U, size_t lds, hipStream_t s)
{
#define CEV_SLSL_CASE(B, UU)                                                                    \
    if (block == B && U == UU)                                                                  \
        return dtype == CEV_BF16 ? launch_sls_t<CEV_BF16, B, UU, false>(a, want_h, want_arg, s, lds) \
                                 : launch_sls_t<CEV_F32, B, UU, false>(a, want_h, want_arg, s, lds);
    CEV_SLSL_CASE(256, 2)
    CEV_SLSL_CASE(512, 2)
    CEV_SLSL_CASE(512, 4)
#undef CEV_SLSL_CASE
    return hipErrorInvalidValue;
}

int64_t sweep_splits(int64_t rows, int64_t vocab, int dtype)
{
    // Measured on MI355X (152064-wide bf16 rows, sweep + merge against the
    // whole-row sweep): splitting wins at 8 rows (14.5 against 16.6 us), breaks
    // even at 32 and loses from 64 rows up (64: 24.8 against 20.6 us), where
    // the whole-row workgroups already cover the chip's memory channels.
    constexpr int64_t kMaxSplitRows = 16;
    constexpr int64_t kTargetBlocks = 2048;  // 8 workgroups per CU on 256 CUs
    constexpr int64_t kMinPartVectors = 2048;
    constexpr int64_t kMaxSplits = 256;
    if (rows <= 0 || rows >= kMaxSplitRows)
        return 1;
    const int64_t nvec = vocab / (dtype == CEV_BF16 ? 8 : 4);
    int64_t sp = (kTargetBlocks + rows - 1) / rows;
    const int64_t by_size = nvec / kMinPartVectors;
    sp = sp < by_size ? sp : by_size;
    sp = sp < kMaxSplits ? sp : kMaxSplits;
    return sp >= 2 ? sp : 1;
}

hipError_t launch_sls_sweep(int dtype, const SweepArgs &a, bool want_h, bool want_arg,
                            hipStream_t s)
{
    if (a.splits > 1 && a.partials && a.rowlist) {
        // 512 x 2 per part: 14.5 us at 8 rows against 15.1 (256 x 4) and 15.9
        // (128 x 4).
        hipError_t e = dtype == CEV_BF16 ? launch_sls_t<CEV_BF16, 512, 2, true>(a, want_h, want_arg, s)
                                         : launch_sls_t<CEV_F32, 512, 2, true>(a, want_h, want_arg, s);
        if (e != hipSuccess)
            return e;
        return dtype == CEV_BF16 ? launch_merge_t<CEV_BF16>(a, want_h, want_arg, s)
                                 : launch_merge_t<CEV_F32>(a, want_h, want_arg, s);
    }
    if (a.rowlist)
        return hipErrorInvalidValue; // a row list comes only with split rows
    Shape sh = pick_shape(a.vocab / (dtype == CEV_BF16 ? 8 : 4));
    // Long rows: 512 x 4 where it still holds seven or eight waves per SIMD
    // (fp32; bf16 without the entropy term, 73 VGPRs), 512 x 2 for bf16 with
    // the entropy term (81 VGPRs at 512 x 4).  Same-process A/B against
    // 512 x 2: grpo forward 328.6 against 332.2 us, peaked fp32 with entropy
    // 187.3 against 191.0 us, peaked bf16 with entropy 105.7 against 103.1 us.
    if (sh.block == 512 && sh.U == 2 && (dtype == CEV_F32 || !want_h))
        sh.U = 4;
    return launch_sls_sweep_cfg(dtype, a, want_h, want_arg, sh.block, sh.U, s);
}

hipError_t launch_topk_sweep_cfg(int dtype, const SweepArgs &a, int block, int U, hipStream_t s)
{
    dim3 grid((unsigned)a.rows);
    const size_t lds = (size_t)a.K * (sizeof(int64_t) + sizeof(double) + sizeof(float) + 1);
#define CEV_TOPK_CASE(B, UU)                                                                    \
    if (block == B && U == UU) {                                                                \
        if (a.K <= kWave) {                                                                     \
            if (dtype == CEV_BF16)                                                              \
                hipLaunchKernelGGL((k_topk_sweep<CEV_BF16, B, UU, true>), grid, dim3(B), lds, s, a); \
            else                                                                                \
                hipLaunchKernelGGL((k_topk_sweep<CEV_F32, B, UU, true>), grid, dim3(B), lds, s, a); \
        } else {                                                                                \
            if (dtype == CEV_BF16)                                                              \
                hipLaunchKernelGGL((k_topk_sweep<CEV_BF16, B, UU, false>), grid, dim3(B), lds, s, a); \
            else                                                                                \
                hipLaunchKernelGGL((k_topk_sweep<CEV_F32, B, UU, false>), grid, dim3(B), lds, s, a); \
        }                                                                                       \
        return hipGetLastError();                                                               \
    }
    CEV_TOPK_CASE(256, 2)
    CEV_TOPK_CASE(512, 2)
#undef CEV_TOPK_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_topk_sweep(int dtype, const SweepArgs &a, hipStream_t s)
{
    // 256 x 2: on 4096 x 32768 bf16 rows with K = 8, 62 us against 81-82 us
    // for 256 x 4 and 512 x 2 and 68 us for 128 x 4 (LDS-held indices); 52 us
    // with the indices held in lanes (K <= 64).
    return launch_topk_sweep_cfg(dtype, a, 256, 2, s);
}

} // namespace cev
