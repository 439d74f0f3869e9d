// backward.hip -- analytic backward sweep for gfx950: one pass that reads each
// valid row once and writes dlogits once, in the logits dtype.
//
// dlogits[r, j] = (g_r / T) p_j for j != t and -(g_r / T) q_r at the target,
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
    float tval;    // -|g / T| q, the target entry before the sign
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
        o[e] = exp2_hw(fmaf(z[e] - rc.mz, c, -rc.kexp));
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
    return col == t ? rc.tval : exp2_hw(fmaf(z - rc.mz, c, -rc.kexp));
}

// blockIdx.x = row * slices + slice; slice sl covers the row's 16-byte vectors
// [sl * per, (sl + 1) * per) (slice 0 also the head columns, the last slice
// the tail columns).  With per = BLOCK * U every thread moves exactly U
// vectors: short-lived workgroups spread over all channels, which measured
// faster on MI355X than long per-row loops for this read-plus-write stream.
template <int DT, int BLOCK, int U>
__global__ __launch_bounds__(BLOCK) void k_backward(BackwardArgs a, int slices, int64_t per,
                                                    int reverse)
{
    constexpr int VE = Elem<DT>::kVE, ES = Elem<DT>::kSize;
    const int tid = threadIdx.x;
    const int64_t rb = blockIdx.x / slices;
    const int64_t r = reverse ? a.rows - 1 - rb : rb;
    const int sl = blockIdx.x % slices;
    const int64_t V = a.vocab;
    const int64_t t = a.labels[r];
    const bool masked = a.row_mask && a.row_mask[r] == 0;
    const bool ignored = masked || t == a.ignore_index;
    const bool bad = !ignored && (t < 0 || t >= V);
    const cev_saved sv = a.saved[r];
    if (bad && sl == 0 && tid == 0 && a.status)
        atomicOr(a.status, (int32_t)CEV_STATUS_BAD_LABEL);

    // Per-row constants in fp32: |g/T| enters through log2 (one v_log_f32),
    // about 1e-7 absolute in the exponent, i.e. ~1e-7 relative in dlogits.
    RowConst rc;
    rc.valid = !ignored && !bad && (sv.flags & 1);
    rc.mz = sv.m_z;
    rc.sgn = 0u;
    rc.kexp = 0.0f;
    rc.tval = 0.0f;
    if (rc.valid) {
        const float gp = a.g[r] * a.inv_t;
        const float ag = fabsf(gp);
        rc.sgn = __float_as_uint(gp) & 0x80000000u;
        rc.kexp = sv.log2_d - __log2f(ag);
        rc.tval = -(ag * sv.q);
    }
    const float c = a.c;

    const char *lrow = static_cast<const char *>(a.logits) + (size_t)r * (size_t)a.row_stride * ES;
    char *drow = static_cast<char *>(a.dlogits) + (size_t)r * (size_t)a.d_row_stride * ES;

    if ((((uintptr_t)lrow ^ (uintptr_t)drow) & 15u) != 0) {
        // Source and destination rows disagree modulo 16 bytes: element path.
        const int64_t c0 = V * sl / slices, c1 = V * (sl + 1) / slices;
        for (int64_t col = c0 + tid; col < c1; col += BLOCK) {
            const float v = rc.valid ? grad_scalar<DT>(load_elem<DT>(lrow, col), rc, c, col, t) : 0.0f;
            store_elem<DT>(drow, col, v, rc.sgn);
        }
        return;
    }

    int64_t head = (int64_t)(((16u - ((unsigned)(uintptr_t)lrow & 15u)) & 15u) / ES);
    head = head < V ? head : V;
    const int64_t nvec = (V - head) / VE;
    const int64_t tail0 = head + nvec * VE;
    const u32x4 *lvp = reinterpret_cast<const u32x4 *>(lrow + head * ES);
    u32x4 *dvp = reinterpret_cast<u32x4 *>(drow + head * ES);
    const int64_t v0 = (int64_t)sl * per;
    const int64_t v1 = v0 + per < nvec ? v0 + per : nvec;

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
        for (int64_t j = v0 + tid; j < v1; j += BLOCK)
            store16_stream(zero, dvp + j);
        return;
    }
    for (int64_t base = v0 + tid; base < v1; base += (int64_t)BLOCK * U) {
        u32x4 w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = base + (int64_t)u * BLOCK;
            if (j < v1)
                w[u] = load16_stream(lvp + j);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = base + (int64_t)u * BLOCK;
            if (j < v1) {
                float z[VE], o[VE];
                unpack16<DT>(w[u], z);
                grad_vec<DT>(z, o, rc, c, head + j * VE, t);
                store16_stream(pack_vec<DT>(o, rc.sgn), dvp + j);
            }
        }
    }
}

template <int DT, int BLOCK, int U>
hipError_t launch_bwd_t(const BackwardArgs &a, int iters, int reverse, hipStream_t s)
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
    dim3 grid((unsigned)(a.rows * slices)), block(BLOCK);
    hipLaunchKernelGGL((k_backward<DT, BLOCK, U>), grid, block, 0, s, a, (int)slices, per,
                       reverse);
    return hipGetLastError();
}

} // namespace

// Launch configuration, exposed for tuning harnesses.
hipError_t launch_backward_cfg(int dtype, const BackwardArgs &a, int block, int U, int iters,
                               int reverse, hipStream_t s)
{
#define CEV_BWD_CASE(B, UU)                                                                     \
    if (block == B && U == UU)                                                                  \
        return dtype == CEV_BF16 ? launch_bwd_t<CEV_BF16, B, UU>(a, iters, reverse, s)          \
                                 : launch_bwd_t<CEV_F32, B, UU>(a, iters, reverse, s);
    CEV_BWD_CASE(256, 2)
    CEV_BWD_CASE(256, 4)
    CEV_BWD_CASE(256, 8)
    CEV_BWD_CASE(512, 2)
    CEV_BWD_CASE(512, 4)
#undef CEV_BWD_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_backward(int dtype, const BackwardArgs &a, hipStream_t s)
{
    return launch_backward_cfg(dtype, a, 256, 4, 1, 0, s);
}

} // namespace cev
