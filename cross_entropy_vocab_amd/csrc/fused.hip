// fused.hip -- per-row cross-entropy forward and analytic backward in one call
// and one HBM read of each row, for an upstream weight g that is known before
// the forward (token weights, mean reduction).  Two forms:
//
//  * k_fused_stream (used): one workgroup sweeps its row for the statistics
//    with caching loads, closes it, and right away re-reads the same row --
//    now in the Infinity Cache -- to write dlogits (below).
//  * k_fused (kept for rows that fit, measured slower on 152064-wide rows):
//    the row held in registers, described here.
//  Each workgroup of 512 threads keeps an entire row
// in registers (a 152064-wide bf16 row is 304 KB of a CU's 512 KB register
// file; 512 threads, two waves per SIMD, up to 256 registers each), so the
// logits are read once and dlogits written once: 4 bytes of HBM traffic per
// bf16 element instead of the 6 of a separate forward and backward.
//
// With the row resident the exact maximum is known before any exponential, so
// the target-excluded sum needs no online rescaling: pass A takes the maximum
// over the non-target columns, pass B sums e^{(z - B)/T} at that base, the row
// is closed in fp64 (Liger-Kernel PR #1555, Summary, CE bullet: the sum without
// the target and dx_y = -sum_others/d), and pass C rebuilds each p_j from the
// registers and writes (g/T)(p_j - [j = t]) (ms-swift PR #10353, PR
// information: the chunked backward as g * softmax - g * one_hot).
#include "cev_device.h"
#include "cev_launch.h"
#include "cev_rowclose.h"
#include "cev_sweep_row.h"

namespace cev {
namespace {

constexpr int kFusedBlock = 512;

// An empty asm that claims to modify every resident register: each pass then
// re-widens the packed row instead of keeping widened copies alive across
// passes (for bf16 those copies would double the registers the row needs).
template <int NV> __device__ __forceinline__ void fence_row(u32x4 (&w)[NV])
{
#pragma unroll
    for (int i = 0; i < NV; ++i)
        asm volatile("" : "+v"(w[i]));
}

// Per-vector ordering points: a pass handles one resident vector at a time
// (its inputs are fenced just before use, its accumulators just after), so the
// scheduler cannot widen many vectors at once and exhaust the register file.
__device__ __forceinline__ void fence_vec(u32x4 &w) { asm volatile("" : "+v"(w)); }
__device__ __forceinline__ void fence_acc(float &x) { asm volatile("" : "+v"(x)); }

// Replace element `e` of a VE-wide vector (runtime index) by `x`.
template <int VE> __device__ __forceinline__ void set_elem(float (&v)[VE], int e, float x)
{
#pragma unroll
    for (int k = 0; k < VE; ++k)
        if (k == e)
            v[k] = x;
}

// One workgroup per row r = blockIdx.x.  Thread tid holds the row's 16-byte
// vectors tid + i * 512, i < NV (coalesced for every i), and one of the fewer
// than VE tail columns.  Rows start 16-byte aligned (checked on the host); all
// in-row indices fit 32 bits (vocab < 2^30).
template <int DT, int NV, bool WANT_H>
__global__ __launch_bounds__(kFusedBlock) void k_fused(FusedArgs a)
{
    constexpr int VE = Elem<DT>::kVE, ES = Elem<DT>::kSize, W = kFusedBlock / kWave;
    __shared__ float sh_f[W];
    __shared__ double sh_d[W];
    __shared__ int64_t sh_i[W];
    __shared__ float sh_zt;
    __shared__ float sh_bc[3];
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
    const u32x4 *lvp = reinterpret_cast<const u32x4 *>(lrow);
    u32x4 *dvp = reinterpret_cast<u32x4 *>(drow);
    const int nvec = (int)(V / VE);
    const int tail0 = nvec * VE;
    const bool has_tail = tail0 + tid < V;

    if (ignored || bad) {
        const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int j = tid + i * kFusedBlock;
            if (j < nvec)
                store16_stream(zero, dvp + j);
        }
        if (has_tail) {
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

    // The whole row, one load per register vector, all in flight at once.  The
    // index is clamped instead of branched on, so the loads issue back to back
    // (the host guarantees nvec >= 512); only the last, partly filled register
    // column holds duplicates, and the passes mask those.
    u32x4 w[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int j = tid + i * kFusedBlock;
        w[i] = load16_stream(lvp + (j < nvec ? j : nvec - 1));
    }
    const float ztail = has_tail ? load_elem<DT>(lrow, tail0 + tid) : -INFINITY;

    // Where the target sits: vector jt = t / VE of thread jt % 512, register
    // jt / 512, element t % VE; or tail column t - tail0.
    const int t32 = (int)t;
    const bool t_tail = t32 >= tail0;
    const int jt = t32 / VE;
    const int it = t_tail ? -1 : jt / kFusedBlock;
    const bool t_mine = !t_tail && tid == jt % kFusedBlock;
    const int et = t32 % VE;
    const bool t_tail_mine = t_tail && tail0 + tid == t32;

    // Pass A: the exact largest non-target value.
    fence_row<NV>(w);
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        fence_vec(w[i]);
        float v[VE];
        unpack16<DT>(w[i], v);
        if (i == it && t_mine) {
            float zt = 0.0f;
#pragma unroll
            for (int k = 0; k < VE; ++k)
                zt = k == et ? v[k] : zt;
            sh_zt = zt;
            set_elem<VE>(v, et, -INFINITY);
        }
        if ((i + 1) * kFusedBlock > nvec && tid + i * kFusedBlock >= nvec) {
#pragma unroll
            for (int k = 0; k < VE; ++k)
                v[k] = -INFINITY;
        }
#pragma unroll
        for (int k = 0; k < VE; ++k)
            m = fmaxf(m, v[k]);
        fence_acc(m);
    }
    if (has_tail) {
        if (t_tail_mine)
            sh_zt = ztail;
        else
            m = fmaxf(m, ztail);
    }
    const float lane_m = m;
    const float M = block_max<kFusedBlock>(m, sh_f);
    const float B = fmaxf(M, -FLT_MAX);
    const float c = a.c, inv_t = a.inv_t;

    // Pass B: target-excluded sum (and entropy term) at the common base B.
    fence_row<NV>(w);
    float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    float h = 0.0f;
    const float nb = fminf(-B * c, kBig);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        fence_vec(w[i]);
        float v[VE];
        unpack16<DT>(w[i], v);
        float e[VE];
#pragma unroll
        for (int k = 0; k < VE; ++k) {
            if constexpr (DT == CEV_F32)
                e[k] = exp2_hw((v[k] - B) * c);
            else
                e[k] = exp2_hw(fmaf(v[k], c, nb));
        }
        if (i == it && t_mine)
            set_elem<VE>(e, et, 0.0f);
        if ((i + 1) * kFusedBlock > nvec && tid + i * kFusedBlock >= nvec) {
#pragma unroll
            for (int k = 0; k < VE; ++k)
                e[k] = 0.0f;
        }
#pragma unroll
        for (int k = 0; k < VE; ++k)
            s[k & 3] += e[k];
        if constexpr (WANT_H) {
#pragma unroll
            for (int k = 0; k < VE; ++k)
                h = fmaf(e[k], (B - v[k]) * inv_t, h);
            fence_acc(h);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k)
            fence_acc(s[k]);
    }
    if (has_tail && !t_tail_mine) {
        const float e = exp2_hw((ztail - B) * c);
        s[0] += e;
        if constexpr (WANT_H)
            h = fmaf(e, (B - ztail) * inv_t, h);
    }
    const double S = block_sum<kFusedBlock>((double)((s[0] + s[1]) + (s[2] + s[3])), sh_d);
    double Hs = 0.0;
    if constexpr (WANT_H)
        Hs = block_sum<kFusedBlock>((double)h, sh_d);

    // Lowest non-target column holding M, from the registers.
    int64_t a_o = INT64_MAX;
    if (a.argmax) {
        int mine = INT32_MAX;
        if (M != -INFINITY && lane_m == M) {
            // Rare: only lanes that hold the row maximum scan their registers.
            fence_row<NV>(w);
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int j = tid + i * kFusedBlock;
                if (j < nvec && mine == INT32_MAX) {
                    float v[VE];
                    unpack16<DT>(w[i], v);
#pragma unroll
                    for (int k = 0; k < VE; ++k)
                        if (mine == INT32_MAX && v[k] == M && j * VE + k != t32)
                            mine = j * VE + k;
                }
            }
            if (mine == INT32_MAX && has_tail && !t_tail_mine && ztail == M)
                mine = tail0 + tid;
        }
        a_o = block_min<kFusedBlock>(mine == INT32_MAX ? INT64_MAX : (int64_t)mine, sh_i);
    }

    if (tid == 0) {
        RowOutputs o;
        o.logp = a.logp;
        o.loss = a.loss;
        o.entropy = WANT_H ? a.entropy : nullptr;
        o.argmax = a.argmax;
        o.saved = a.saved;
        const cev_saved sv = close_row_fp64(o, r, sh_zt, t, M, S, Hs, a_o, a.temperature);
        // Backward constants: |g/T| folded into the exponent, sign on the bits.
        const float gp = a.g[r] * inv_t;
        const float ag = fabsf(gp);
        sh_bc[0] = sv.m_z;
        sh_bc[1] = sv.log2_d - __log2f(ag);
        sh_bc[2] = -(ag * sv.q);
        sh_sgn = __float_as_uint(gp) & 0x80000000u;
    }
    __syncthreads();
    const float mz = sh_bc[0], kexp = sh_bc[1], tval = sh_bc[2];
    const unsigned sgn = sh_sgn;

    // Pass C: dlogits from the registers.
    fence_row<NV>(w);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int j = tid + i * kFusedBlock;
        fence_vec(w[i]);
        float v[VE], o[VE];
        unpack16<DT>(w[i], v);
#pragma unroll
        for (int k = 0; k < VE; ++k)
            o[k] = exp2_hw(fmaf(v[k] - mz, c, -kexp));
        if (i == it && t_mine)
            set_elem<VE>(o, et, tval);
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
        if ((i + 1) * kFusedBlock <= nvec || j < nvec)
            store16_stream(out, dvp + j);
    }
    if (has_tail) {
        const float o = t_tail_mine ? tval : exp2_hw(fmaf(ztail - mz, c, -kexp));
        if constexpr (DT == CEV_F32)
            reinterpret_cast<float *>(drow)[tail0 + tid] = __uint_as_float(__float_as_uint(o) ^ sgn);
        else
            reinterpret_cast<unsigned short *>(drow)[tail0 + tid] =
                (unsigned short)(to_bf16(o) ^ (sgn >> 16));
    }
}

// Cache-resident two-pass form: pass 1 is the streaming forward sweep of the
// row with plain (caching) loads, and pass 2, by the same workgroup right
// after the row is closed, re-reads the row -- which the few hundred rows in
// flight (~80-160 MB) leave in the 256 MB Infinity Cache -- and writes
// dlogits.  Several workgroups per CU overlap one row's arithmetic with other
// rows' memory traffic, which the register-resident form cannot.
template <int DT, int BLOCK, int U, bool WANT_H, bool NT1, bool DESC>
__global__ __launch_bounds__(BLOCK) void k_fused_stream(FusedArgs a)
{
    constexpr int VE = Elem<DT>::kVE, ES = Elem<DT>::kSize, W = BLOCK / kWave;
    constexpr int U2 = 4;
    __shared__ float sh_f[W];
    __shared__ double sh_d[W];
    __shared__ int64_t sh_i[W];
    __shared__ float sh_bc[3];
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

    const RowStats rs = sweep_row<DT, BLOCK, U, WANT_H, true, NT1>(lrow, V, t, 0, 1, a.c, a.inv_t,
                                                                     sh_f, sh_d, sh_i);
    if (tid == 0) {
        RowOutputs o;
        o.logp = a.logp;
        o.loss = a.loss;
        o.entropy = WANT_H ? a.entropy : nullptr;
        o.argmax = a.argmax;
        o.saved = a.saved;
        const cev_saved sv = close_row_fp64(o, r, load_elem<DT>(lrow, t), t, rs.M, rs.S, rs.Hs,
                                            rs.a_o, a.temperature);
        const float gp = a.g[r] * a.inv_t;
        const float ag = fabsf(gp);
        sh_bc[0] = sv.m_z;
        sh_bc[1] = sv.log2_d - __log2f(ag);
        sh_bc[2] = -(ag * sv.q);
        sh_sgn = __float_as_uint(gp) & 0x80000000u;
    }
    __syncthreads();
    const float mz = sh_bc[0], kexp = sh_bc[1], tval = sh_bc[2], c = a.c;
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
                    o[k] = exp2_hw(fmaf(v[k] - mz, c, -kexp));
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
        const float o = col == t ? tval : exp2_hw(fmaf(z - mz, c, -kexp));
        if constexpr (DT == CEV_F32)
            reinterpret_cast<float *>(drow)[col] = __uint_as_float(__float_as_uint(o) ^ sgn);
        else
            reinterpret_cast<unsigned short *>(drow)[col] = (unsigned short)(to_bf16(o) ^ (sgn >> 16));
    }
}

template <int DT, int NV> hipError_t launch_fused_nv(const FusedArgs &a, bool want_h, hipStream_t s)
{
    dim3 grid((unsigned)a.rows), block(kFusedBlock);
    if (want_h)
        hipLaunchKernelGGL((k_fused<DT, NV, true>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((k_fused<DT, NV, false>), grid, block, 0, s, a);
    return hipGetLastError();
}

template <int DT> hipError_t launch_fused_t(const FusedArgs &a, int nv, bool want_h, hipStream_t s)
{
    switch (nv) {
    case 8: return launch_fused_nv<DT, 8>(a, want_h, s);
    case 16: return launch_fused_nv<DT, 16>(a, want_h, s);
    case 24: return launch_fused_nv<DT, 24>(a, want_h, s);
    case 32: return launch_fused_nv<DT, 32>(a, want_h, s);
    case 40: return launch_fused_nv<DT, 40>(a, want_h, s);
    default: return launch_fused_nv<DT, 48>(a, want_h, s);
    }
}

// 512 threads, 4 vectors per thread per pass-1 step, pass 2 from the row's end:
// the fastest shape measured on MI355X for 152064-wide bf16 rows (976 us for
// 8192 rows against 1021-1151 us for the other shapes tried).
template <int DT, bool NT1> hipError_t launch_stream_t(const FusedArgs &a, bool want_h, hipStream_t s)
{
    dim3 grid((unsigned)a.rows), block(512);
    if (want_h)
        hipLaunchKernelGGL((k_fused_stream<DT, 512, 4, true, NT1, true>), grid, block, 0, s, a);
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

int fused_vectors_per_thread(int64_t vocab, int dtype)
{
    const int64_t nvec = vocab / (dtype == CEV_BF16 ? 8 : 4);
    const int64_t per = (nvec + kFusedBlock - 1) / kFusedBlock;
    const int64_t nv = ((per + 7) / 8) * 8;
    if (nv > kMaxFusedVectors)
        return 0;
    return (int)(nv < 8 ? 8 : nv);
}

// variant 1: register-resident rows; 2: cache-resident two-pass rows (pass 1
// with plain loads); 3: the same with streaming loads in pass 1.
hipError_t launch_fused_cfg(int dtype, const FusedArgs &a, bool want_h, int variant, hipStream_t s)
{
    if (variant == 1) {
        const int nv = fused_vectors_per_thread(a.vocab, dtype);
        if (nv == 0)
            return hipErrorInvalidValue;
        return dtype == CEV_BF16 ? launch_fused_t<CEV_BF16>(a, nv, want_h, s)
                                 : launch_fused_t<CEV_F32>(a, nv, want_h, s);
    }
    if (variant == 3)
        return dtype == CEV_BF16 ? launch_stream_t<CEV_BF16, true>(a, want_h, s)
                                 : launch_stream_t<CEV_F32, true>(a, want_h, s);
    return dtype == CEV_BF16 ? launch_stream_t<CEV_BF16, false>(a, want_h, s)
                             : launch_stream_t<CEV_F32, false>(a, want_h, s);
}

hipError_t launch_fused(int dtype, const FusedArgs &a, bool want_h, hipStream_t s)
{
    return launch_fused_cfg(dtype, a, want_h, 2, s);
}

} // namespace cev
