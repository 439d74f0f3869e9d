// fused.hip -- per-row cross-entropy forward and analytic backward in one call,
// each row fetched from HBM about once, for an upstream weight g that is known
// before the forward (token weights, mean reduction).
//
// One workgroup per row sweeps the row for the target-excluded statistics
// with caching loads (Liger-Kernel PR #1555, Summary, CE bullet: the sum
// without the target), closes it in fp64, and right away re-reads the same
// row -- the few hundred rows in flight (~80-160 MB) fit the 256 MB Infinity
// Cache, which serves much of the re-read -- to write (g/T)(p_j - [j = t])
// with the target column -(g/T) q (ms-swift PR #10353, PR information:
// g * softmax - g * one_hot; Liger PR #1555: dx_y = -sum_others/d).  Label
// smoothing eps (unsloth-zoo #2080 Summary, on the Liger page) takes eps/V off
// every column, giving (g/T)(p_j - eps/V) and (g/T)(eps - eps/V - q) at t.
// Several workgroups per CU overlap one row's arithmetic with other rows'
// memory traffic.  (Holding a whole 152064-wide bf16 row in registers instead
// was measured slower, 1.42 ms against 0.98 ms for 8192 rows: a CU can then
// hold only one row, and its load, arithmetic and store phases cannot
// overlap.)
#include "cev_device.h"
#include "cev_launch.h"
#include "cev_rowclose.h"
#include "cev_sweep_row.h"

namespace cev {
namespace {

// Replace element `e` of a VE-wide vector (runtime index) by `x`.
template <int VE> __device__ __forceinline__ void set_elem(float (&v)[VE], int e, float x)
{
#pragma unroll
    for (int k = 0; k < VE; ++k)
        if (k == e)
            v[k] = x;
}

// Pass 1 is the streaming forward sweep of the row with plain (caching) loads
// (NT1 = false; streaming loads there make pass 2 miss the cache: 1.36 ms
// against 0.98 ms); pass 2, by the same workgroup right after the row is
// closed, re-reads the row and writes dlogits, last vectors first (DESC).
template <int DT, int BLOCK, int U, bool WANT_H, bool NT1, bool DESC, bool WANT_Z = false>
__global__ __launch_bounds__(BLOCK) void k_fused_stream(FusedArgs a)
{
    constexpr int VE = Elem<DT>::kVE, ES = Elem<DT>::kSize, W = BLOCK / kWave;
    constexpr int U2 = 4;
    __shared__ float sh_f[W];
    __shared__ double sh_d[3 * W];
    __shared__ int64_t sh_i[W];
    __shared__ float sh_bc[4];
    __shared__ unsigned sh_sgn;
    const int tid = threadIdx.x;
    const int64_t r = blockIdx.x;
    const int64_t V = a.vocab;
    const int64_t t = a.labels[r];
    const bool masked = a.row_mask && a.row_mask[r] == 0;
    const bool ignored = masked || t == a.ignore_index;
    const bool bad = !ignored && (t < 0 || t >= V);
    const char *lrow = static_cast<const char *>(a.logits) + (size_t)r * (size_t)a.row_stride * ES;
    char *drow = static_cast<char *>(a.dlogits) + (size_t)r * (size_t)a.d_row_stride * ES;
    // Rows start 16-byte aligned here (checked on the host).
    const u32x4 *lvp = reinterpret_cast<const u32x4 *>(lrow);
    u32x4 *dvp = reinterpret_cast<u32x4 *>(drow);
    const int64_t nvec = V / VE;
    const int64_t tail0 = nvec * VE;

    if (ignored || bad) {
        const u32x4 zero = {0u, 0u, 0u, 0u};
        for (int64_t j = tid; j < nvec; j += BLOCK)
            store16_stream(zero, dvp + j);
        if (tail0 + tid < V) {
            if constexpr (DT == CEV_F32)
                reinterpret_cast<float *>(drow)[tail0 + tid] = 0.0f;
            else
                reinterpret_cast<unsigned short *>(drow)[tail0 + tid] = 0;
        }
        if (tid == 0) {
            if (a.loss)
                a.loss[r] = 0.0f;
            if (a.logp)
                a.logp[r] = 0.0f;
            if (a.entropy)
                a.entropy[r] = 0.0f;
            if (a.argmax)
                a.argmax[r] = -1;
            cev_saved z;
            z.m_z = 0.0f;
            z.log2_d = 0.0f;
            z.q = 0.0f;
            z.flags = 0;
            a.saved[r] = z;
            if (bad && a.status)
                atomicOr(a.status, (int32_t)CEV_STATUS_BAD_LABEL);
        }
        return;
    }

    const RowStats rs = sweep_row<DT, BLOCK, U, WANT_H, true, NT1, WANT_Z>(
        lrow, V, t, 0, 1, a.c, a.inv_t, sh_f, sh_d, sh_i);
    if (tid == 0) {
        RowOutputs o;
        o.logp = a.logp;
        o.loss = a.loss;
        o.entropy = WANT_H ? a.entropy : nullptr;
        o.argmax = a.argmax;
        o.saved = a.saved;
        const cev_saved sv = close_row_fp64(o, r, load_elem<DT>(lrow, t), t, rs.M, rs.S, rs.Hs,
                                            rs.a_o, a.temperature, rs.Zs, a.label_smoothing, V);
        const float gp = a.g[r] * a.inv_t;
        const float ag = fabsf(gp);
        const float eps = (float)a.label_smoothing;
        const float epv = (float)(a.label_smoothing / (double)V);
        sh_bc[0] = sv.m_z;
        sh_bc[1] = sv.log2_d - __log2f(ag);
        sh_bc[2] = -(ag * ((sv.q - eps) + epv));
        sh_bc[3] = ag * epv;
        sh_sgn = __float_as_uint(gp) & 0x80000000u;
    }
    __syncthreads();
    const float mz = sh_bc[0], kexp = sh_bc[1], tval = sh_bc[2], ev = sh_bc[3], c = a.c;
    const unsigned sgn = sh_sgn;

    // Pass 2, last vectors first: the most recently read part of the row is
    // the likeliest still to sit in this XCD's L2.
    const int64_t nstep = (nvec + (int64_t)BLOCK * U2 - 1) / ((int64_t)BLOCK * U2);
    for (int64_t it = 0; it < nstep; ++it) {
        const int64_t st = DESC ? nstep - 1 - it : it;
        const int64_t base = st * (int64_t)BLOCK * U2 + tid;
        u32x4 w[U2];
#pragma unroll
        for (int u = 0; u < U2; ++u) {
            const int64_t j = base + (int64_t)u * BLOCK;
            if (j < nvec)
                w[u] = load16_stream(lvp + j);
        }
#pragma unroll
        for (int u = 0; u < U2; ++u) {
            const int64_t j = base + (int64_t)u * BLOCK;
            if (j < nvec) {
                float v[VE], o[VE];
                unpack16<DT>(w[u], v);
#pragma unroll
                for (int k = 0; k < VE; ++k)
                    o[k] = exp2_hw(fmaf(v[k] - mz, c, -kexp)) - ev;
                if ((uint64_t)(t - j * VE) < (uint64_t)VE)
                    set_elem<VE>(o, (int)(t - j * VE), tval);
                u32x4 out;
                if constexpr (DT == CEV_F32) {
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        out[k] = __float_as_uint(o[k]) ^ sgn;
                } else {
                    const unsigned s2 = sgn | (sgn >> 16);
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        out[k] = pack_bf16x2(o[2 * k], o[2 * k + 1]) ^ s2;
                }
                store16_stream(out, dvp + j);
            }
        }
    }
    if (tail0 + tid < V) {
        const int64_t col = tail0 + tid;
        const float z = load_elem<DT>(lrow, col);
        const float o = col == t ? tval : exp2_hw(fmaf(z - mz, c, -kexp)) - ev;
        if constexpr (DT == CEV_F32)
            reinterpret_cast<float *>(drow)[col] = __uint_as_float(__float_as_uint(o) ^ sgn);
        else
            reinterpret_cast<unsigned short *>(drow)[col] = (unsigned short)(to_bf16(o) ^ (sgn >> 16));
    }
}

// 512 threads, 4 vectors per thread per pass-1 step, pass 2 from the row's end:
// the fastest shape measured on MI355X for 152064-wide bf16 rows (976 us for
// 8192 rows against 1021-1151 us for the other shapes tried).
template <int DT, bool NT1> hipError_t launch_stream_t(const FusedArgs &a, bool want_h, hipStream_t s)
{
    dim3 grid((unsigned)a.rows), block(512);
    const bool z = a.label_smoothing != 0.0;
    if (want_h && z)
        hipLaunchKernelGGL((k_fused_stream<DT, 512, 4, true, NT1, true, true>), grid, block, 0, s, a);
    else if (want_h)
        hipLaunchKernelGGL((k_fused_stream<DT, 512, 4, true, NT1, true>), grid, block, 0, s, a);
    else if (z)
        hipLaunchKernelGGL((k_fused_stream<DT, 512, 4, false, NT1, true, true>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((k_fused_stream<DT, 512, 4, false, NT1, true>), grid, block, 0, s, a);
    return hipGetLastError();
}

} // namespace

// Tuning: workgroup size, vectors per step in pass 1, pass-2 order, and extra
// dynamic LDS per workgroup (which caps how many rows a CU holds at once).
hipError_t launch_fused_stream_cfg(int dtype, const FusedArgs &a, int block, int U, bool desc,
                                   size_t lds_bytes, hipStream_t s)
{
    if (a.label_smoothing != 0.0)
        return hipErrorInvalidValue; // the tuning shapes carry no label-smoothing sum
    dim3 grid((unsigned)a.rows);
#define CEV_FS_CASE(B, UU, D)                                                                   \
    if (block == B && U == UU && desc == D) {                                                   \
        if (dtype == CEV_BF16)                                                                  \
            hipLaunchKernelGGL((k_fused_stream<CEV_BF16, B, UU, false, false, D>), grid,        \
                               dim3(B), lds_bytes, s, a);                                       \
        else                                                                                    \
            hipLaunchKernelGGL((k_fused_stream<CEV_F32, B, UU, false, false, D>), grid,         \
                               dim3(B), lds_bytes, s, a);                                       \
        return hipGetLastError();                                                               \
    }
    CEV_FS_CASE(512, 2, true)
    CEV_FS_CASE(512, 2, false)
    CEV_FS_CASE(256, 4, true)
    CEV_FS_CASE(256, 4, false)
    CEV_FS_CASE(1024, 2, true)
    CEV_FS_CASE(512, 4, true)
#undef CEV_FS_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_fused(int dtype, const FusedArgs &a, bool want_h, hipStream_t s)
{
    return dtype == CEV_BF16 ? launch_stream_t<CEV_BF16, false>(a, want_h, s)
                             : launch_stream_t<CEV_F32, false>(a, want_h, s);
}

} // namespace cev
