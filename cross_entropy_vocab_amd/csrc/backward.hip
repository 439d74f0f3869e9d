// backward.hip -- analytic backward sweep for gfx950: one pass that reads each
// valid row once and writes dlogits once, in the logits dtype.
//
// dlogits[r, j] = (g_r / T) p_j for j != t and -(g_r / T) q_r at the target
// (label smoothing eps, unsloth-zoo #2080 Summary on the Liger page:
// (g/T)(p_j - eps/V), and (g/T)(eps - eps/V - q) at the target),
// where q_r = s_others / d = 1 - p_t comes from the forward's saved record
// (Liger-Kernel PR #1555, Summary: dx_y = -sum_others / d; ms-swift PR #10353,
// PR information: g * softmax - g * one_hot with zero weight for ignored
// labels).  p_j = 2^((z_j - m_z) c - log2 d) is rebuilt from the record; the
// factor |g/T| is folded into the exponent (so a small p_j times a large g
// cannot lose a subnormal product) and the sign of g is applied to the bits.
#include "cev_device.h"
#include "cev_launch.h"

namespace cev {
namespace {

struct RowConst {
    float mz;      // exact row maximum of the stored logits
    float kexp;    // log2 d - log2 |g / T|
    float ev;      // |g / T| eps / V, the label-smoothing share of every column
    float tval;    // -|g / T| (q - eps + eps / V), the target entry before the sign
    unsigned sgn;  // 0x80000000 when g < 0 (or is -0)
    bool valid;
};

template <int DT>
__device__ __forceinline__ void grad_vec(const float (&z)[Elem<DT>::kVE], float (&o)[Elem<DT>::kVE],
                                         const RowConst &rc, float c, int64_t col0, int64_t t)
{
    constexpr int VE = Elem<DT>::kVE;
#pragma unroll
    for (int e = 0; e < VE; ++e)
        o[e] = exp2_hw(fmaf(z[e] - rc.mz, c, -rc.kexp)) - rc.ev;
    if ((uint64_t)(t - col0) < (uint64_t)VE) {
#pragma unroll
        for (int e = 0; e < VE; ++e)
            if (col0 + e == t)
                o[e] = rc.tval;
    }
}

template <int DT> __device__ __forceinline__ u32x4 pack_vec(const float (&o)[Elem<DT>::kVE], unsigned sgn)
{
    u32x4 w;
    if constexpr (DT == CEV_F32) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[i] = __float_as_uint(o[i]) ^ sgn;
    } else {
        const unsigned s2 = sgn | (sgn >> 16);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[i] = pack_bf16x2(o[2 * i], o[2 * i + 1]) ^ s2;
    }
    return w;
}

template <int DT> __device__ __forceinline__ void store_elem(char *rowp, int64_t col, float v, unsigned sgn)
{
    if constexpr (DT == CEV_F32)
        __builtin_nontemporal_store(__uint_as_float(__float_as_uint(v) ^ sgn),
                                    reinterpret_cast<float *>(rowp) + col);
    else
        __builtin_nontemporal_store((unsigned short)(to_bf16(v) ^ (sgn >> 16)),
                                    reinterpret_cast<unsigned short *>(rowp) + col);
}

template <int DT>
__device__ __forceinline__ float grad_scalar(float z, const RowConst &rc, float c, int64_t col, int64_t t)
{
    return col == t ? rc.tval : exp2_hw(fmaf(z - rc.mz, c, -rc.kexp)) - rc.ev;
}

// blockIdx.x = row * slices + slice; slice sl covers the row's 16-byte vectors
// [sl * per, (sl + 1) * per) (slice 0 also the head columns, the last slice
// the tail columns).  With per = BLOCK * U every thread moves exactly U
// vectors: short-lived workgroups spread over all channels, which measured
// faster on MI355X than long per-row loops for this read-plus-write stream.
// SHARD: the row holds global columns [col_offset, col_offset + vocab) of a
// vocab_total-wide row (vocab-parallel form); otherwise the whole row.
template <int DT, int BLOCK, int U, bool SHARD, bool SNT>
__global__ __launch_bounds__(BLOCK) void k_backward(BackwardArgs a, int slices, int64_t per,
                                                    int order)
{
    constexpr int VE = Elem<DT>::kVE, ES = Elem<DT>::kSize;
    const int tid = threadIdx.x;
    // order 0: tiles in row order; 1: rows from the last; 2: XCD-contiguous.
    // Workgroup b runs on XCD b % 8, so order 2 gives each XCD a contiguous
    // eighth of the tiles (a row's tiles then share one L2 for its record):
    // 744 against 750-751 us on the 8192 x 152064 bf16 backward.
    int64_t bid = blockIdx.x;
    if (order == 2) {
        const int64_t total = a.rows * slices, g8 = (total + 7) / 8;
        bid = (bid % 8) * g8 + bid / 8;
        if (bid >= total)
            return;
    }
    const int64_t rb = bid / slices;
    const int64_t r = order == 1 ? a.rows - 1 - rb : rb;
    const int sl = (int)(bid % slices);
    const int64_t V = a.vocab;
    // Every per-row input is loaded up front (independent scalar loads, issued
    // together), and the row's first step of logits goes out as soon as the
    // saved record says the forward read this row: one short round trip
    // before the stream starts instead of a chain of dependent loads.
    const cev_saved sv = a.saved[r];
    const int64_t tg = load_uniform(a.labels + r);
    const float graw = load_uniform(a.g + r);

    const char *lrow = static_cast<const char *>(a.logits) + (size_t)r * (size_t)a.row_stride * ES;
    char *drow = static_cast<char *>(a.dlogits) + (size_t)r * (size_t)a.d_row_stride * ES;
    const bool vec_ok = (((uintptr_t)lrow ^ (uintptr_t)drow) & 15u) == 0;
    int64_t head = (int64_t)(((16u - ((unsigned)(uintptr_t)lrow & 15u)) & 15u) / ES);
    head = head < V ? head : V;
    const int64_t nvec = (V - head) / VE;
    const int64_t tail0 = head + nvec * VE;
    const u32x4 *lvp = reinterpret_cast<const u32x4 *>(lrow + head * ES);
    u32x4 *dvp = reinterpret_cast<u32x4 *>(drow + head * ES);
    const int64_t v0 = (int64_t)sl * per;
    const int64_t v1 = v0 + per < nvec ? v0 + per : nvec;
    const int64_t base0 = v0 + tid;

    u32x4 w[U];
    if (vec_ok && (sv.flags & 1)) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = base0 + (int64_t)u * BLOCK;
            if (j < v1)
                w[u] = load16_stream(lvp + j);
        }
    }

    const bool masked = a.row_mask && mask_byte(a.row_mask, r) == 0;
    const bool ignored = masked || tg == a.ignore_index;
    const int64_t VT = SHARD ? a.vocab_total : V;
    const bool bad = !ignored && (tg < 0 || tg >= VT);
    // The target's column here; outside [0, V) when another shard holds it.
    const int64_t t = SHARD ? tg - a.col_offset : tg;
    if (bad && sl == 0 && tid == 0 && a.status)
        atomicOr(a.status, (int32_t)CEV_STATUS_BAD_LABEL);

    // Per-row constants in fp32: |g/T| enters through log2 (one v_log_f32),
    // about 1e-7 absolute in the exponent, i.e. ~1e-7 relative in dlogits.
    RowConst rc;
    rc.valid = !ignored && !bad && (sv.flags & 1);
    rc.mz = sv.m_z;
    rc.sgn = 0u;
    rc.kexp = 0.0f;
    rc.ev = 0.0f;
    rc.tval = 0.0f;
    if (rc.valid) {
        const float gp = graw * a.inv_t;
        const float ag = fabsf(gp);
        const float eps = a.eps;
        const float epv = a.eps_over_v;
        rc.sgn = __float_as_uint(gp) & 0x80000000u;
        rc.kexp = sv.log2_d - __log2f(ag);
        rc.ev = ag * epv;
        rc.tval = -(ag * ((sv.q - eps) + epv));
    }
    const float c = a.c;

    if (!vec_ok) {
        // Source and destination rows disagree modulo 16 bytes: element path.
        const int64_t c0 = V * sl / slices, c1 = V * (sl + 1) / slices;
        for (int64_t col = c0 + tid; col < c1; col += BLOCK) {
            const float v = rc.valid ? grad_scalar<DT>(load_elem<DT>(lrow, col), rc, c, col, t) : 0.0f;
            store_elem<DT>(drow, col, v, rc.sgn);
        }
        return;
    }

    if (sl == 0 && tid < head) {
        const float v = rc.valid ? grad_scalar<DT>(load_elem<DT>(lrow, tid), rc, c, tid, t) : 0.0f;
        store_elem<DT>(drow, tid, v, rc.sgn);
    }
    if (sl == slices - 1 && tail0 + tid < V) {
        const int64_t col = tail0 + tid;
        const float v = rc.valid ? grad_scalar<DT>(load_elem<DT>(lrow, col), rc, c, col, t) : 0.0f;
        store_elem<DT>(drow, col, v, rc.sgn);
    }

    if (!rc.valid) {
        const u32x4 zero = {0u, 0u, 0u, 0u};
        for (int64_t j = base0; j < v1; j += BLOCK)
            store16<SNT>(zero, dvp + j);
        return;
    }
    for (int64_t base = base0; base < v1; base += (int64_t)BLOCK * U) {
        if (base != base0) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t j = base + (int64_t)u * BLOCK;
                if (j < v1)
                    w[u] = load16_stream(lvp + j);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = base + (int64_t)u * BLOCK;
            if (j < v1) {
                float z[VE], o[VE];
                unpack16<DT>(w[u], z);
                grad_vec<DT>(z, o, rc, c, head + j * VE, t);
                store16<SNT>(pack_vec<DT>(o, rc.sgn), dvp + j);
            }
        }
    }
}

// ------------------------------------------------------------------------
// One-shot tiles for calls whose rows all start 16-byte aligned in both
// matrices and hold a whole number of 16-byte vectors (no head or tail
// columns), with the values that decide the tile's first load passed as
// leading scalar kernel arguments.  Those arrive in SGPRs when the wave
// starts (kernel-argument preloading on gfx950), so the saved record is the
// only load in front of the tile's stream: one scalar round trip instead of
// two (the argument block, then the record).  The remaining inputs (labels,
// g, mask, constants) are loaded while the logits are in flight.
//
// Tiles are numbered in row order; workgroup b runs on XCD b % 8 and takes
// tile (b % 8) * g8 + b / 8, so each XCD sweeps a contiguous eighth of the
// matrix (a row's tiles then share one L2 for its record).  The row of tile
// n is n / slices, computed as (n * mul) >> shift from host-side constants
// (exact for n < 2^31).
template <int DT, int BLOCK, int U, bool SHARD, bool SNT>
__global__ __launch_bounds__(BLOCK) void k_backward_tile(const cev_saved *saved, const char *logits,
                                                         uint64_t row_bytes, uint64_t mul,
                                                         uint32_t shift, uint32_t slices,
                                                         uint32_t g8, uint32_t total, BackwardArgs a)
{
    constexpr int VE = Elem<DT>::kVE;
    constexpr uint32_t per = (uint32_t)BLOCK * U;
    const int tid = threadIdx.x;
    const uint32_t bid = (blockIdx.x % 8) * g8 + blockIdx.x / 8;
    if (bid >= total)
        return;
    const uint32_t r = (uint32_t)(((uint64_t)bid * mul) >> shift);
    const uint32_t sl = bid - r * slices;
    const u32x4 rec = load_uniform(reinterpret_cast<const u32x4 *>(saved + r));
    const uint32_t v0 = sl * per;
    const u32x4 *lvp = reinterpret_cast<const u32x4 *>(logits + (size_t)r * row_bytes) + v0;
    const int64_t nvec = a.vocab / VE;
    const uint32_t nv = (uint32_t)(nvec - v0 < (int64_t)per ? nvec - v0 : per);
    u32x4 w[U];
    if (rec[3] & 1u) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t j = (uint32_t)(u * BLOCK + tid);
            if (j < nv)
                w[u] = load16_stream(lvp + j);
        }
    }
    const int64_t tg = load_uniform(a.labels + r);
    const float graw = load_uniform(a.g + r);
    const bool masked = a.row_mask && mask_byte(a.row_mask, r) == 0;
    const bool ignored = masked || tg == a.ignore_index;
    const int64_t VT = SHARD ? a.vocab_total : a.vocab;
    const bool bad = !ignored && (tg < 0 || tg >= VT);
    if (bad && sl == 0 && tid == 0 && a.status)
        atomicOr(a.status, (int32_t)CEV_STATUS_BAD_LABEL);
    // The target column relative to the tile's first column (outside the
    // tile, or the shard, when another holds it).
    const int64_t t = (SHARD ? tg - a.col_offset : tg) - (int64_t)v0 * VE;
    RowConst rc;
    rc.valid = !ignored && !bad && (rec[3] & 1u);
    rc.mz = __uint_as_float(rec[0]);
    rc.sgn = 0u;
    rc.kexp = 0.0f;
    rc.ev = 0.0f;
    rc.tval = 0.0f;
    if (rc.valid) {
        const float gp = graw * a.inv_t;
        const float ag = fabsf(gp);
        rc.sgn = __float_as_uint(gp) & 0x80000000u;
        rc.kexp = __uint_as_float(rec[1]) - __log2f(ag);
        rc.ev = ag * a.eps_over_v;
        rc.tval = -(ag * ((__uint_as_float(rec[2]) - a.eps) + a.eps_over_v));
    }
    u32x4 *dvp = reinterpret_cast<u32x4 *>(static_cast<char *>(a.dlogits) +
                                           (size_t)r * (size_t)a.d_row_stride * Elem<DT>::kSize) + v0;
    if (!rc.valid) {
        const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t j = (uint32_t)(u * BLOCK + tid);
            if (j < nv)
                store16<SNT>(zero, dvp + j);
        }
        return;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t j = (uint32_t)(u * BLOCK + tid);
        if (j < nv) {
            float z[VE], o[VE];
            unpack16<DT>(w[u], z);
            grad_vec<DT>(z, o, rc, a.c, (int64_t)j * VE, t);
            store16<SNT>(pack_vec<DT>(o, rc.sgn), dvp + j);
        }
    }
}

// ------------------------------------------------------------------------
// Top-K backward: gradient of sum_k g_k log p_{i_k} with respect to the
// logits (ms-swift PR #10337, PR information: gradients through top-K
// indices), dL/dz_j = (1/T) sum_k g_k ([j = i_k] - p_j).  Every column gets
// -(Gs/T) p_j, Gs = sum of the valid g_k (|Gs/T| folded into the exponent);
// a gathered column j gets (G_j q_j - p_j (Gs - G_j)) / T instead, G_j the sum
// of the g_k gathered at j and q_j = 1 - p_j from the forward as sigmoid(u),
// so the peaked case never forms 1 - p_j by subtraction.  Same one-shot slices
// as k_backward; each workgroup first lists the gathered columns that fall in
// its slice.
template <int DT, int BLOCK, int U>
__global__ __launch_bounds__(BLOCK) void k_topk_backward(TopkBackwardArgs a, int slices, int64_t per)
{
    constexpr int VE = Elem<DT>::kVE, ES = Elem<DT>::kSize, W = BLOCK / kWave;
    // Dynamic LDS, K entries each: the row's indices, its g, and the list of
    // gathered columns this slice writes (first index k of each, and the two
    // per-column terms).
    extern __shared__ __align__(16) unsigned char lds[];
    const int K = (int)a.K;
    int64_t *sidx = reinterpret_cast<int64_t *>(lds);
    float *sg = reinterpret_cast<float *>(sidx + K);
    int *lk = reinterpret_cast<int *>(sg + K);
    float *la = reinterpret_cast<float *>(lk + K);
    float *lb = la + K;
    __shared__ double sh_d[W];
    __shared__ int ln;
    __shared__ int sbad;
    const int tid = threadIdx.x;
    const int64_t r = blockIdx.x / slices;
    const int sl = blockIdx.x % slices;
    const int64_t V = a.vocab;
    const char *lrow = static_cast<const char *>(a.logits) + (size_t)r * (size_t)a.row_stride * ES;
    char *drow = static_cast<char *>(a.dlogits) + (size_t)r * (size_t)a.d_row_stride * ES;
    const bool scalar_path = (((uintptr_t)lrow ^ (uintptr_t)drow) & 15u) != 0;
    int64_t head = (int64_t)(((16u - ((unsigned)(uintptr_t)lrow & 15u)) & 15u) / ES);
    head = head < V ? head : V;
    const int64_t nvec = (V - head) / VE;
    const int64_t tail0 = head + nvec * VE;
    const int64_t v0 = (int64_t)sl * per;
    const int64_t v1 = v0 + per < nvec ? v0 + per : nvec;
    // Does this workgroup write column `col`?
    auto owns = [&](int64_t col) {
        if (scalar_path)
            return col >= V * sl / slices && col < V * (sl + 1) / slices;
        if (col < head)
            return sl == 0;
        if (col >= tail0)
            return sl == slices - 1;
        const int64_t j = (col - head) / VE;
        return j >= v0 && j < v1;
    };
    const cev_saved sv = a.saved[r];
    // The slice's first step goes out as soon as the record says the row was
    // read, before the gathered indices and g are processed.
    const u32x4 *lvp = reinterpret_cast<const u32x4 *>(lrow + head * ES);
    const int64_t base0 = v0 + tid;
    u32x4 w[U];
    if (!scalar_path && (sv.flags & 1)) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = base0 + (int64_t)u * BLOCK;
            if (j < v1)
                w[u] = load16_stream(lvp + j);
        }
    }
    const bool masked = (a.row_mask && mask_byte(a.row_mask, r) == 0) || !(sv.flags & 1);
    const int64_t *idx = a.indices + (size_t)r * (size_t)a.index_row_stride;
    const float *gk = a.g + (size_t)r * (size_t)K;
    const float *qk = a.q + (size_t)r * (size_t)K;

    if (tid == 0) {
        ln = 0;
        sbad = 0;
    }
    __syncthreads();
    // Gs = sum of the g_k at valid indices (fp64, fixed order per thread and
    // across the block, so every slice of the row gets the same value).
    double gpart = 0.0;
    for (int k = tid; k < K; k += BLOCK) {
        const int64_t i = idx[k];
        sidx[k] = i;
        const float g = gk[k];
        sg[k] = g;
        if (i == a.ignore_index)
            continue;
        if (i < 0 || i >= V) {
            sbad = 1;
            continue;
        }
        gpart += (double)g;
    }
    const float gs = (float)block_sum<BLOCK>(gpart, sh_d); // block_sum synchronises
    if (tid == 0 && sbad && sl == 0 && a.status && !masked)
        atomicOr(a.status, (int32_t)CEV_STATUS_BAD_INDEX);
    if (!masked) {
        for (int k = tid; k < K; k += BLOCK) {
            const int64_t i = sidx[k];
            if (i == a.ignore_index || i < 0 || i >= V || !owns(i))
                continue;
            bool first = true;
            for (int k2 = 0; k2 < k && first; ++k2)
                first = sidx[k2] != i;
            if (!first)
                continue;
            double gj = 0.0;
            for (int k2 = k; k2 < K; ++k2)
                if (sidx[k2] == i)
                    gj += (double)sg[k2];
            const int n = atomicAdd(&ln, 1);
            lk[n] = k;
            la[n] = (float)(gj * (double)qk[k] * (double)a.inv_t);
            lb[n] = (float)(((double)gs - gj) * (double)a.inv_t);
        }
    }
    __syncthreads();
    const int L = ln;
    const float mz = sv.m_z, l2d = sv.log2_d, c = a.c;
    const float gsT = gs * a.inv_t;
    const float kexp = l2d - __log2f(fabsf(gsT));
    // Every column but the gathered ones is -(Gs/T) p_j: the sign applied to
    // the bits is the opposite of Gs's.  Gathered values carry their own sign
    // and are pre-flipped so that the same XOR leaves them as computed.
    const unsigned sgn = (__float_as_uint(gsT) & 0x80000000u) ^ 0x80000000u;
    auto gathered = [&](float z, int n) {
        const float p = exp2_hw(fmaf(z - mz, c, -l2d));
        return __uint_as_float(__float_as_uint(la[n] - p * lb[n]) ^ sgn);
    };
    auto value = [&](float z, int64_t col) {
        float o = exp2_hw(fmaf(z - mz, c, -kexp));
        for (int n = 0; n < L; ++n)
            if (sidx[lk[n]] == col)
                o = gathered(z, n);
        return o;
    };

    if (scalar_path) {
        const int64_t c0 = V * sl / slices, c1 = V * (sl + 1) / slices;
        for (int64_t col = c0 + tid; col < c1; col += BLOCK) {
            const float v = masked ? 0.0f : value(load_elem<DT>(lrow, col), col);
            store_elem<DT>(drow, col, v, masked ? 0u : sgn);
        }
        return;
    }
    u32x4 *dvp = reinterpret_cast<u32x4 *>(drow + head * ES);
    if (sl == 0 && tid < head) {
        const float v = masked ? 0.0f : value(load_elem<DT>(lrow, tid), tid);
        store_elem<DT>(drow, tid, v, masked ? 0u : sgn);
    }
    if (sl == slices - 1 && tail0 + tid < V) {
        const int64_t col = tail0 + tid;
        const float v = masked ? 0.0f : value(load_elem<DT>(lrow, col), col);
        store_elem<DT>(drow, col, v, masked ? 0u : sgn);
    }
    if (masked) {
        const u32x4 zero = {0u, 0u, 0u, 0u};
        for (int64_t j = base0; j < v1; j += BLOCK)
            store16_stream(zero, dvp + j);
        return;
    }
    for (int64_t base = base0; base < v1; base += (int64_t)BLOCK * U) {
        if (base != base0) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t j = base + (int64_t)u * BLOCK;
                if (j < v1)
                    w[u] = load16_stream(lvp + j);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = base + (int64_t)u * BLOCK;
            if (j < v1) {
                float z[VE], o[VE];
                unpack16<DT>(w[u], z);
#pragma unroll
                for (int e = 0; e < VE; ++e)
                    o[e] = exp2_hw(fmaf(z[e] - mz, c, -kexp));
                const int64_t col0 = head + j * VE;
                for (int n = 0; n < L; ++n) {
                    const int64_t d = sidx[lk[n]] - col0;
                    if ((uint64_t)d < (uint64_t)VE) {
#pragma unroll
                        for (int e = 0; e < VE; ++e)
                            if (e == d)
                                o[e] = gathered(z[e], n);
                    }
                }
                store16_stream(pack_vec<DT>(o, sgn), dvp + j);
            }
        }
    }
}

// The top-K backward for K <= 64 on rows of whole 16-byte vectors: one-shot
// tiles of BLOCK * U vectors in row order (tile n of row n / slices, the
// division by multiply-shift), the saved record read first and the tile's
// loads issued as soon as it marks the row as read.  Every wave holds the K
// entries in its lanes (lane k: index k, its g and q), forms Gs and, for the
// first occurrence of each gathered column, G_j and the two terms of that
// column from the lanes with v_readlane, in the same order as the general
// kernel; no LDS and no barrier.  A gathered column is applied by the lane
// that holds its vector.
template <int DT, int BLOCK, int U>
__global__ __launch_bounds__(BLOCK) void k_topk_backward_tile(const cev_saved *saved, const char *logits,
                                                              uint64_t row_bytes, uint64_t mul,
                                                              uint32_t shift, uint32_t slices,
                                                              uint32_t total, TopkBackwardArgs a)
{
    constexpr int VE = Elem<DT>::kVE;
    constexpr uint32_t per = (uint32_t)BLOCK * U;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const uint32_t bid = blockIdx.x;
    if (bid >= total)
        return;
    const uint32_t r = (uint32_t)(((uint64_t)bid * mul) >> shift);
    const uint32_t sl = bid - r * slices;
    const u32x4 rec = load_uniform(reinterpret_cast<const u32x4 *>(saved + r));
    const uint32_t v0 = sl * per;
    const u32x4 *lvp = reinterpret_cast<const u32x4 *>(logits + (size_t)r * row_bytes) + v0;
    const int64_t V = a.vocab;
    const int64_t nvec = V / VE;
    const uint32_t nv = (uint32_t)(nvec - v0 < (int64_t)per ? nvec - v0 : per);
    u32x4 w[U];
    if (rec[3] & 1u) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t j = (uint32_t)(u * BLOCK + tid);
            if (j < nv)
                w[u] = load16_stream(lvp + j);
        }
    }
    const bool masked = (a.row_mask && mask_byte(a.row_mask, r) == 0) || !(rec[3] & 1u);
    const int K = (int)a.K;
    int64_t col = -1;
    float g = 0.0f, q = 0.0f;
    bool bad = false;
    if (lane < K) {
        const int64_t i = a.indices[(size_t)r * (size_t)a.index_row_stride + lane];
        g = a.g[(size_t)r * (size_t)K + lane];
        q = a.q[(size_t)r * (size_t)K + lane];
        const bool ok = i != a.ignore_index && i >= 0 && i < V;
        bad = i != a.ignore_index && !ok;
        col = ok ? i : -1;
    }
    if (sl == 0 && wave == 0 && !masked && __any(bad) && lane == 0 && a.status)
        atomicOr(a.status, (int32_t)CEV_STATUS_BAD_INDEX);
    // Gs: the valid g_k summed in fp64 (the same value in every lane and tile).
    const float gs = (float)wave_sum(col >= 0 ? (double)g : 0.0);
    // This lane's column: first occurrence, and G_j over its later duplicates.
    bool first = col >= 0;
    double gj = 0.0;
    for (int k2 = 0; k2 < K; ++k2) {
        const int64_t c2 = lane_value(col, k2);
        if (c2 == col) {
            if (k2 < lane)
                first = false;
            else
                gj += (double)lane_value(g, k2);
        }
    }
    const float la = first ? (float)(gj * (double)q * (double)a.inv_t) : 0.0f;
    const float lb = first ? (float)(((double)gs - gj) * (double)a.inv_t) : 0.0f;
    // The tile-relative vector of this lane's column, if the tile writes it.
    const int64_t jj = first ? col / VE - (int64_t)v0 : -1;
    const bool mine = jj >= 0 && jj < (int64_t)nv;

    u32x4 *dvp = reinterpret_cast<u32x4 *>(static_cast<char *>(a.dlogits) +
                                           (size_t)r * (size_t)a.d_row_stride * Elem<DT>::kSize) + v0;
    if (masked) {
        const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t j = (uint32_t)(u * BLOCK + tid);
            if (j < nv)
                store16_stream(zero, dvp + j);
        }
        return;
    }
    const float mz = __uint_as_float(rec[0]), l2d = __uint_as_float(rec[1]), c = a.c;
    const float gsT = gs * a.inv_t;
    const float kexp = l2d - __log2f(fabsf(gsT));
    // Every column but the gathered ones is -(Gs/T) p_j: the sign applied to
    // the bits is the opposite of Gs's; gathered values are pre-flipped.
    const unsigned sgn = (__float_as_uint(gsT) & 0x80000000u) ^ 0x80000000u;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t j = (uint32_t)(u * BLOCK + tid);
        float z[VE], o[VE];
        unpack16<DT>(w[u], z);
#pragma unroll
        for (int e = 0; e < VE; ++e)
            o[e] = exp2_hw(fmaf(z[e] - mz, c, -kexp));
        // gathered columns in this wave's vectors of step u
        uint64_t hits = __ballot(mine && jj / BLOCK == u && (jj % BLOCK) / kWave == wave);
        while (hits) {
            const int k2 = __builtin_ctzll(hits);
            hits &= hits - 1;
            const int64_t c2 = lane_value(col, k2);
            if ((int64_t)((c2 / VE - (int64_t)v0) % kWave) == lane) {
                const float a2 = lane_value(la, k2), b2 = lane_value(lb, k2);
                const int e2 = (int)(c2 % VE);
#pragma unroll
                for (int e = 0; e < VE; ++e)
                    if (e == e2) {
                        const float p = exp2_hw(fmaf(z[e] - mz, c, -l2d));
                        o[e] = __uint_as_float(__float_as_uint(a2 - p * b2) ^ sgn);
                    }
            }
        }
        if (j < nv)
            store16_stream(pack_vec<DT>(o, sgn), dvp + j);
    }
}

template <int DT, int BLOCK, int U, bool SHARD, bool SNT>
hipError_t launch_bwd_t(const BackwardArgs &a, int iters, int order, hipStream_t s)
{
    // iters wave-steps of BLOCK * U vectors per workgroup; 0 = a whole row.
    const int64_t nvec = a.vocab / Elem<DT>::kVE;
    int64_t per = iters > 0 ? (int64_t)BLOCK * U * iters : (nvec > 0 ? nvec : 1);
    if (per < 1)
        per = 1;
    int64_t slices = (nvec + per - 1) / per;
    slices = slices < 1 ? 1 : slices;
    // The flat grid must stay below 2^32 work-items: widen the slices if not.
    while ((uint64_t)a.rows * (uint64_t)slices * BLOCK > 0xFFFFFFFFull && slices > 1) {
        per *= 2;
        slices = (nvec + per - 1) / per;
    }
    const int64_t total = a.rows * slices;
    dim3 grid((unsigned)(order == 2 ? (total + 7) / 8 * 8 : total)), block(BLOCK);
    hipLaunchKernelGGL((k_backward<DT, BLOCK, U, SHARD, SNT>), grid, block, 0, s, a, (int)slices, per,
                       order);
    return hipGetLastError();
}

// Multiply-shift division by d: for n < 2^31, n / d == (n * mul) >> shift
// with shift = 32 + ceil(log2 d) and mul = ceil(2^shift / d).
struct DivMagic {
    uint64_t mul;
    uint32_t shift;
};

inline DivMagic div_magic(uint32_t d)
{
    uint32_t l = 0;
    while (((uint64_t)1 << l) < d)
        ++l;
    DivMagic m;
    m.shift = 32 + l;
    m.mul = (uint64_t)((((unsigned __int128)1 << m.shift) + d - 1) / d);
    return m;
}

template <int DT, int BLOCK, int U, bool SHARD, bool SNT>
hipError_t launch_bwd_tile_t(const BackwardArgs &a, hipStream_t s)
{
    const int64_t nvec = a.vocab / Elem<DT>::kVE;
    const int64_t per = (int64_t)BLOCK * U;
    const int64_t slices = (nvec + per - 1) / per;
    const int64_t total = a.rows * slices;   // < 2^31, checked by the caller
    const uint32_t g8 = (uint32_t)((total + 7) / 8);
    const DivMagic dm = div_magic((uint32_t)slices);
    const uint64_t row_bytes = (uint64_t)a.row_stride * Elem<DT>::kSize;
    hipLaunchKernelGGL((k_backward_tile<DT, BLOCK, U, SHARD, SNT>), dim3(g8 * 8), dim3(BLOCK), 0, s,
                       a.saved, static_cast<const char *>(a.logits), row_bytes, dm.mul, dm.shift,
                       (uint32_t)slices, g8, (uint32_t)total, a);
    return hipGetLastError();
}

// Tiles of `per` 16-byte vectors over every row.
inline int64_t tile_count(const BackwardArgs &a, int es, int64_t per)
{
    const int64_t nvec = a.vocab * es / 16;
    return a.rows * ((nvec + per - 1) / per);
}

// Whether every row of both matrices starts 16-byte aligned and holds whole
// 16-byte vectors (the one-shot tile form's precondition).
inline bool tile_form_ok(const BackwardArgs &a, int es)
{
    return ((uintptr_t)a.logits & 15u) == 0 && ((uintptr_t)a.dlogits & 15u) == 0 &&
           (a.row_stride * es) % 16 == 0 && (a.d_row_stride * es) % 16 == 0 && (a.vocab * es) % 16 == 0;
}

} // namespace

// Launch configuration, exposed for tuning harnesses.
hipError_t launch_backward_cfg(int dtype, const BackwardArgs &a, int block, int U, int iters,
                               int order, int store_nt, hipStream_t s)
{
    if (a.col_offset != 0 || a.vocab_total != a.vocab)
        return hipErrorInvalidValue; // whole rows only
#define CEV_BWD_CASE(B, UU, NT)                                                                     \
    if (block == B && U == UU && (store_nt != 0) == NT)                                             \
        return dtype == CEV_BF16 ? launch_bwd_t<CEV_BF16, B, UU, false, NT>(a, iters, order, s)     \
                                 : launch_bwd_t<CEV_F32, B, UU, false, NT>(a, iters, order, s);
    CEV_BWD_CASE(64, 1, false)
    CEV_BWD_CASE(64, 1, true)
    CEV_BWD_CASE(64, 2, false)
    CEV_BWD_CASE(64, 2, true)
    CEV_BWD_CASE(64, 4, false)
    CEV_BWD_CASE(64, 4, true)
    CEV_BWD_CASE(128, 1, false)
    CEV_BWD_CASE(128, 1, true)
    CEV_BWD_CASE(128, 2, false)
    CEV_BWD_CASE(128, 2, true)
    CEV_BWD_CASE(128, 4, false)
    CEV_BWD_CASE(128, 4, true)
    CEV_BWD_CASE(256, 1, false)
    CEV_BWD_CASE(256, 1, true)
    CEV_BWD_CASE(256, 2, false)
    CEV_BWD_CASE(256, 2, true)
    CEV_BWD_CASE(256, 4, false)
    CEV_BWD_CASE(256, 4, true)
    CEV_BWD_CASE(512, 1, false)
#undef CEV_BWD_CASE
    return hipErrorInvalidValue;
}

// One-shot tile form with preloaded arguments, for tuning harnesses (rows
// 16-byte aligned in both matrices, whole vectors; checked here).
hipError_t launch_backward_tile_cfg(int dtype, const BackwardArgs &a, int block, int U, int store_nt,
                                    hipStream_t s)
{
    const int es = dtype == CEV_BF16 ? 2 : 4;
    if (!tile_form_ok(a, es) || tile_count(a, es, (int64_t)block * U) >= ((int64_t)1 << 31) ||
        a.col_offset != 0 || a.vocab_total != a.vocab)
        return hipErrorInvalidValue;
#define CEV_BWT_CASE(B, UU, NT)                                                                     \
    if (block == B && U == UU && (store_nt != 0) == NT)                                             \
        return dtype == CEV_BF16 ? launch_bwd_tile_t<CEV_BF16, B, UU, false, NT>(a, s)              \
                                 : launch_bwd_tile_t<CEV_F32, B, UU, false, NT>(a, s);
    CEV_BWT_CASE(64, 4, true)
    CEV_BWT_CASE(128, 1, true)
    CEV_BWT_CASE(128, 2, true)
    CEV_BWT_CASE(128, 2, false)
    CEV_BWT_CASE(128, 4, true)
    CEV_BWT_CASE(256, 1, true)
    CEV_BWT_CASE(256, 1, false)
    CEV_BWT_CASE(256, 2, true)
    CEV_BWT_CASE(256, 2, false)
    CEV_BWT_CASE(512, 1, true)
    CEV_BWT_CASE(512, 1, false)
#undef CEV_BWT_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_backward(int dtype, const BackwardArgs &a, hipStream_t s)
{
    const bool shard = a.col_offset != 0 || a.vocab_total != a.vocab;
    // Rows 16-byte aligned in both matrices: one-shot 4 KB tiles of 256
    // threads x 1 vector with preloaded arguments (on the 8192 x 152064 bf16
    // backward 688 us against 706 us for the general kernel's 128 x 2 tiles,
    // and 689-731 us for 128 x 1, 128 x 2, 256 x 2, 512 x 1, 64 x 4 and
    // 128 x 4).  A vocab shard gets its own instantiation (and kernel name in
    // traces).
    const int es = dtype == CEV_BF16 ? 2 : 4;
    if (tile_form_ok(a, es) && tile_count(a, es, 256) < ((int64_t)1 << 31)) {
        if (dtype == CEV_BF16)
            return shard ? launch_bwd_tile_t<CEV_BF16, 256, 1, true, true>(a, s)
                         : launch_bwd_tile_t<CEV_BF16, 256, 1, false, true>(a, s);
        return shard ? launch_bwd_tile_t<CEV_F32, 256, 1, true, true>(a, s)
                     : launch_bwd_tile_t<CEV_F32, 256, 1, false, true>(a, s);
    }
    // Otherwise the general kernel (head and tail columns, rows whose two
    // matrices disagree modulo 16 bytes): 4 KB workgroups of 128 threads x 2
    // vectors with nontemporal stores, 753-758 us against 781-821 us for
    // 256 x 4 on the same backward, the best of 20 shapes (64-256 threads,
    // 1-4 vectors, 1-3 steps, either store policy).
    if (shard)
        return dtype == CEV_BF16 ? launch_bwd_t<CEV_BF16, 128, 2, true, true>(a, 1, 2, s)
                                 : launch_bwd_t<CEV_F32, 128, 2, true, true>(a, 1, 2, s);
    return launch_backward_cfg(dtype, a, 128, 2, 1, 2, 1, s);
}

template <int DT, int B, int UU>
void launch_topk_bwd_t(const TopkBackwardArgs &a, hipStream_t s)
{
    const int64_t nvec = a.vocab / Elem<DT>::kVE;
    int64_t per = (int64_t)B * UU;
    int64_t slices = (nvec + per - 1) / per;
    slices = slices < 1 ? 1 : slices;
    while ((uint64_t)a.rows * (uint64_t)slices * B > 0xFFFFFFFFull && slices > 1) {
        per *= 2;
        slices = (nvec + per - 1) / per;
    }
    const size_t lds = (size_t)a.K * (sizeof(int64_t) + 4 * sizeof(float));
    hipLaunchKernelGGL((k_topk_backward<DT, B, UU>), dim3((unsigned)(a.rows * slices)), dim3(B), lds,
                       s, a, (int)slices, per);
}

hipError_t launch_topk_backward_cfg(int dtype, const TopkBackwardArgs &a, int block, int U,
                                    hipStream_t s)
{
#define CEV_TKB_CASE(B, UU)                                                                     \
    if (block == B && U == UU) {                                                                \
        if (dtype == CEV_BF16)                                                                  \
            launch_topk_bwd_t<CEV_BF16, B, UU>(a, s);                                           \
        else                                                                                    \
            launch_topk_bwd_t<CEV_F32, B, UU>(a, s);                                            \
        return hipGetLastError();                                                               \
    }
    CEV_TKB_CASE(128, 2)
    CEV_TKB_CASE(256, 1)
    CEV_TKB_CASE(256, 2)
    CEV_TKB_CASE(256, 4)
#undef CEV_TKB_CASE
    return hipErrorInvalidValue;
}

template <int DT, int B, int UU>
hipError_t launch_topk_bwd_tile_t(const TopkBackwardArgs &a, hipStream_t s)
{
    const int64_t nvec = a.vocab / Elem<DT>::kVE;
    const int64_t per = (int64_t)B * UU;
    const int64_t slices = (nvec + per - 1) / per;
    const int64_t total = a.rows * slices;   // < 2^31, checked by the caller
    const DivMagic dm = div_magic((uint32_t)slices);
    hipLaunchKernelGGL((k_topk_backward_tile<DT, B, UU>), dim3((unsigned)total), dim3(B), 0, s,
                       a.saved, static_cast<const char *>(a.logits),
                       (uint64_t)a.row_stride * Elem<DT>::kSize, dm.mul, dm.shift, (uint32_t)slices,
                       (uint32_t)total, a);
    return hipGetLastError();
}

// Whether the lane-held form applies: K <= 64 and every row of both matrices
// starting 16-byte aligned with whole 16-byte vectors.
inline bool topk_tile_ok(const TopkBackwardArgs &a, int es)
{
    const int64_t per = 256;   // the smallest tile launched
    return a.K <= kWave && ((uintptr_t)a.logits & 15u) == 0 && ((uintptr_t)a.dlogits & 15u) == 0 &&
           (a.row_stride * es) % 16 == 0 && (a.d_row_stride * es) % 16 == 0 &&
           (a.vocab * es) % 16 == 0 &&
           a.rows * ((a.vocab * es / 16 + per - 1) / per) < ((int64_t)1 << 31);
}

hipError_t launch_topk_backward_tile_cfg(int dtype, const TopkBackwardArgs &a, int block, int U,
                                         hipStream_t s)
{
    if (!topk_tile_ok(a, dtype == CEV_BF16 ? 2 : 4))
        return hipErrorInvalidValue;
#define CEV_TKT_CASE(B, UU)                                                                     \
    if (block == B && U == UU)                                                                  \
        return dtype == CEV_BF16 ? launch_topk_bwd_tile_t<CEV_BF16, B, UU>(a, s)                \
                                 : launch_topk_bwd_tile_t<CEV_F32, B, UU>(a, s);
    CEV_TKT_CASE(256, 1)
    CEV_TKT_CASE(256, 2)
    CEV_TKT_CASE(256, 4)
#undef CEV_TKT_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_topk_backward(int dtype, const TopkBackwardArgs &a, hipStream_t s)
{
    if (topk_tile_ok(a, dtype == CEV_BF16 ? 2 : 4))
        return launch_topk_backward_tile_cfg(dtype, a, 256, 2, s);
    return launch_topk_backward_cfg(dtype, a, 256, 4, s);
}

} // namespace cev
