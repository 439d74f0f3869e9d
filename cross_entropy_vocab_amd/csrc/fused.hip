// fused.hip -- per-row cross-entropy forward and analytic backward in one call,
// each row fetched from HBM about once, for an upstream weight g that is known
// before the forward (token weights, mean reduction).
//
// One workgroup per row sweeps the row for the target-excluded statistics
// (Liger-Kernel PR #1555, Summary, CE bullet: the sum without the target),
// closes it in fp64, and then writes (g/T)(p_j - [j = t]) with the target
// column -(g/T) q (ms-swift PR #10353, PR information: g * softmax -
// g * one_hot; Liger PR #1555: dx_y = -sum_others/d).  Label smoothing eps
// (unsloth-zoo #2080 Summary, on the Liger page) takes eps/V off every column,
// giving (g/T)(p_j - eps/V) and (g/T)(eps - eps/V - q) at t.  Part of each row
// stays on chip (registers and LDS) between the two passes; the rest is read
// again, from the caches where it is still there.  Two rows per CU overlap
// one row's arithmetic with the other's memory traffic.  (Holding a whole
// 152064-wide bf16 row on chip would leave room for one row per CU, and with
// it no overlap: 1.42 ms against 0.98 ms for 8192 rows, measured.)
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

// The row's fp64 closing step (one lane, once per row) and the constants of
// the second pass, published in LDS.
__device__ __forceinline__ void fused_close(const FusedArgs &a, int64_t r, float zt, int64_t t,
                                            float M, double S, double Hs, int64_t a_o, double Zs,
                                            bool want_h, float *sh_bc, unsigned *sh_sgn)
{
    RowOutputs o;
    o.logp = a.logp;
    o.loss = a.loss;
    o.entropy = want_h ? a.entropy : nullptr;
    o.argmax = a.argmax;
    o.saved = a.saved;
    const cev_saved sv = close_row_fp64(o, r, zt, t, M, S, Hs, a_o, a.temperature, Zs,
                                        a.label_smoothing, a.vocab);
    const float gp = a.g[r] * a.inv_t;
    const float ag = fabsf(gp);
    const float eps = (float)a.label_smoothing;
    const float epv = (float)(a.label_smoothing / (double)a.vocab);
    sh_bc[0] = sv.m_z;
    sh_bc[1] = sv.log2_d - __log2f(ag);
    sh_bc[2] = -(ag * ((sv.q - eps) + epv));
    sh_bc[3] = ag * epv;
    *sh_sgn = __float_as_uint(gp) & 0x80000000u;
}

// One workgroup of 512 threads per row, two rows per CU (at most 128 VGPRs,
// 64 KB of LDS each), so that one row's arithmetic overlaps the other's
// memory traffic.  Each wave sweeps its wave steps of U vectors per lane in
// row order (step k of the row's wave steps is wave k mod 8's).  The vectors
// of its first S steps stay in registers and those of the next SL steps in
// LDS (each lane its own) until the second pass, which re-reads only the
// rest of the row: of a 152064-wide bf16 row's 148 wave steps, the 64 that
// are each wave's first 8 (43% of the row) never leave the CU between the
// passes.  Registers set the split (held_steps): more held steps spill.
// Wave steps held in registers, per form: as many as fit in 128 VGPRs
// beside the sweep's own registers with few or no spills (fp32 steps carry
// half the columns of bf16 ones but unpack into as many registers).
constexpr int held_steps(int dt, bool want_h, bool want_z)
{
    return dt == CEV_F32 ? (want_h && want_z ? 4 : want_h || want_z ? 5 : 6)
                         : (want_h || want_z ? 3 : 4);
}

template <int DT, bool WANT_H, bool WANT_Z>
__global__ __launch_bounds__(512, 4) void k_fused_hold(FusedArgs a)
{
    constexpr int BLOCK = 512, U = 2, S = held_steps(DT, WANT_H, WANT_Z), SL = 4;
    constexpr int VE = Elem<DT>::kVE, ES = Elem<DT>::kSize, W = BLOCK / kWave;
    constexpr int64_t CH = (int64_t)kWave * U;
    __shared__ float sh_f[W];
    __shared__ double sh_d[3 * W];
    __shared__ int64_t sh_i[W];
    __shared__ float sh_bc[4];
    __shared__ unsigned sh_sgn;
    // steps S .. S + SL - 1 of each wave, held in LDS (each lane its own vectors)
    __shared__ u32x4 sh_hold[SL][W][U][kWave];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
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
    const RowGeom g = row_geom<DT, U>(lrow, V, 0, 1);   // ahead = 0: aligned rows
    const int64_t nvec = g.nvec, nfull = g.nfull, tail0 = g.tail0;

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

    // Pass 1.  The register-held steps' loads go out at once, the LDS-held
    // steps' one step ahead (all nontemporal: those parts are not read
    // again); the other steps stream with caching loads, one step ahead, for
    // the second pass to find in cache.  Vector indices are 32-bit (a row
    // holds fewer than 2^31 vectors).
    u32x4 hold[S][U];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int64_t k = wave + (int64_t)s * W;
        if (k < nfull) {
#pragma unroll
            for (int u = 0; u < U; ++u)
                hold[s][u] = load16_stream(lvp + (unsigned)(k * CH + u * kWave + lane));
        }
    }
    const float c = a.c;
    LaneState st{-INFINITY, 0.0f, 0.0f, 0.0f, 0.0f, -1};
    auto fold_step = [&](const u32x4(&w)[U], int64_t k) {
        float v[U * VE];
        unpack_step<DT, U>(w, v);
        const int64_t lo = k * CH * VE;
        if ((uint64_t)(t - lo) < (uint64_t)(CH * VE)) {
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int e = 0; e < VE; ++e)
                    if ((k * CH + u * kWave + lane) * VE + e == t)
                        v[u * VE + e] = -INFINITY;
            fold<DT, U * VE, WANT_H, true, true, WANT_Z>(st, v, 16 + (int)k, c);
        } else {
            fold<DT, U * VE, WANT_H, true, false, WANT_Z>(st, v, 16 + (int)k, c);
        }
    };
    // steps S .. S + SL - 1 (kept in LDS: nontemporal loads), then the rest
    // (caching loads, re-read in the second pass)
    constexpr int SH = S + SL;
    int64_t k = wave + (int64_t)S * W;
    u32x4 cur[U], nxt[U];
    if (k < nfull) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            cur[u] = load16_stream(lvp + (unsigned)(k * CH + u * kWave + lane));
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int64_t ks = wave + (int64_t)s * W;
        if (ks < nfull)
            fold_step(hold[s], ks);
    }
    for (int sl = 0; sl < SL && k < nfull; ++sl, k += W) {
        const int64_t kn = k + W;
        if (kn < nfull) {
#pragma unroll
            for (int u = 0; u < U; ++u)
                nxt[u] = load16_stream(lvp + (unsigned)(kn * CH + u * kWave + lane));
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            sh_hold[sl][wave][u][lane] = cur[u];
        fold_step(cur, k);
#pragma unroll
        for (int u = 0; u < U; ++u)
            cur[u] = nxt[u];
    }
    for (; k < nfull; k += W) {
        const int64_t kn = k + W;
        if (kn < nfull) {
#pragma unroll
            for (int u = 0; u < U; ++u)
                nxt[u] = lvp[(unsigned)(kn * CH + u * kWave + lane)];
        }
        fold_step(cur, k);
#pragma unroll
        for (int u = 0; u < U; ++u)
            cur[u] = nxt[u];
    }
    for (int64_t j = nfull * CH + tid; j < nvec; j += BLOCK) {
        float v[VE];
        unpack16<DT>(lvp[j], v);
#pragma unroll
        for (int e = 0; e < VE; ++e)
            if (j * VE + e == t)
                v[e] = -INFINITY;
        fold<DT, VE, WANT_H, true, true, WANT_Z>(st, v, 16 + (int)(nfull + (j - nfull * CH)), c);
    }
    if (tail0 + tid < V) {
        const int64_t col = tail0 + tid;
        float v[1] = {col == t ? -INFINITY : load_elem<DT>(lrow, col)};
        fold<DT, 1, WANT_H, true, true, WANT_Z>(st, v, 16 + (int)(nfull + g.nrem + tid), c);
    }

    // Combine the lanes as the streaming sweep does.
    const float M = block_max<BLOCK>(st.m, sh_f);
    const Rescan<DT, U> rsc = rescan_issue<DT, U>(lrow, g, st.best, M != -INFINITY && st.m == M);
    {
        const float B = fmaxf(M, -FLT_MAX);
        const float bl = fmaxf(st.m, -FLT_MAX);
        const float f = exp2_hw((bl - B) * c);
        const float sl = st.s - st.comp;
        constexpr int NS = 1 + (WANT_H ? 1 : 0) + (WANT_Z ? 1 : 0);
        double sums[NS];
        sums[0] = (double)sl * (double)f;
        if constexpr (WANT_H)
            sums[1] = (double)f * (double)fmaf(fminf(B - bl, kBig), sl, st.h);
        if constexpr (WANT_Z)
            sums[NS - 1] = (double)st.zs;
        block_sum_n<BLOCK, NS>(sums, sh_d);
        const int64_t a_o = block_min<BLOCK>(rescan_finish<DT, U>(rsc, M, t), sh_i);
        if (tid == 0) {
            const double Hs = WANT_H ? sums[1] * (double)a.inv_t : 0.0;
            const double Zs = WANT_Z ? sums[NS - 1] : 0.0;
            fused_close(a, r, load_elem<DT>(lrow, t), t, M, sums[0], Hs, a_o, Zs, WANT_H, sh_bc,
                        &sh_sgn);
        }
    }
    __syncthreads();
    const float mz = sh_bc[0], kexp = sh_bc[1], tval = sh_bc[2], ev = sh_bc[3];
    const unsigned sgn = sh_sgn;

    // Pass 2: the held steps from registers, the rest re-read (the row's
    // end, the most recently read, first).
    auto grad_store = [&](const u32x4 &wv, unsigned j) {
        float v[VE], o[VE];
        unpack16<DT>(wv, v);
#pragma unroll
        for (int e = 0; e < VE; ++e)
            o[e] = exp2_hw(fmaf(v[e] - mz, c, -kexp)) - ev;
        if ((uint64_t)(t - (int64_t)j * VE) < (uint64_t)VE)
            set_elem<VE>(o, (int)(t - (int64_t)j * VE), tval);
        u32x4 out;
        if constexpr (DT == CEV_F32) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                out[e] = __float_as_uint(o[e]) ^ sgn;
        } else {
            const unsigned s2 = sgn | (sgn >> 16);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                out[e] = pack_bf16x2(o[2 * e], o[2 * e + 1]) ^ s2;
        }
        store16_stream(out, dvp + j);
    };
    for (int64_t j = nfull * CH + tid; j < nvec; j += BLOCK)
        grad_store(load16_stream(lvp + j), (unsigned)j);
    if (tail0 + tid < V) {
        const int64_t col = tail0 + tid;
        const float z = load_elem<DT>(lrow, col);
        const float o = col == t ? tval : exp2_hw(fmaf(z - mz, c, -kexp)) - ev;
        if constexpr (DT == CEV_F32)
            reinterpret_cast<float *>(drow)[col] = __uint_as_float(__float_as_uint(o) ^ sgn);
        else
            reinterpret_cast<unsigned short *>(drow)[col] = (unsigned short)(to_bf16(o) ^ (sgn >> 16));
    }
    // the wave's streamed steps, last first; the first step's loads are in
    // flight while the held steps are written
    const int64_t kfirst = wave + (int64_t)SH * W;
    int64_t k2 = nfull > kfirst ? wave + ((nfull - 1 - wave) / W) * W : -1;
    if (k2 >= kfirst) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            cur[u] = load16_stream(lvp + (unsigned)(k2 * CH + u * kWave + lane));
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int64_t ks = wave + (int64_t)s * W;
        if (ks < nfull) {
#pragma unroll
            for (int u = 0; u < U; ++u)
                grad_store(hold[s][u], (unsigned)(ks * CH + u * kWave + lane));
        }
    }
    for (int sl = 0; sl < SL; ++sl) {
        const int64_t ks = wave + (int64_t)(S + sl) * W;
        if (ks < nfull) {
#pragma unroll
            for (int u = 0; u < U; ++u)
                grad_store(sh_hold[sl][wave][u][lane], (unsigned)(ks * CH + u * kWave + lane));
        }
    }
    for (; k2 >= kfirst; k2 -= W) {
        const int64_t kn = k2 - W;
        if (kn >= kfirst) {
#pragma unroll
            for (int u = 0; u < U; ++u)
                nxt[u] = load16_stream(lvp + (unsigned)(kn * CH + u * kWave + lane));
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            grad_store(cur[u], (unsigned)(k2 * CH + u * kWave + lane));
#pragma unroll
        for (int u = 0; u < U; ++u)
            cur[u] = nxt[u];
    }
}

template <int DT> hipError_t launch_t(const FusedArgs &a, bool want_h, hipStream_t s)
{
    dim3 grid((unsigned)a.rows), block(512);
    const bool z = a.label_smoothing != 0.0;
    if (want_h && z)
        hipLaunchKernelGGL((k_fused_hold<DT, true, true>), grid, block, 0, s, a);
    else if (want_h)
        hipLaunchKernelGGL((k_fused_hold<DT, true, false>), grid, block, 0, s, a);
    else if (z)
        hipLaunchKernelGGL((k_fused_hold<DT, false, true>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((k_fused_hold<DT, false, false>), grid, block, 0, s, a);
    return hipGetLastError();
}

} // namespace

hipError_t launch_fused(int dtype, const FusedArgs &a, bool want_h, hipStream_t s)
{
    return dtype == CEV_BF16 ? launch_t<CEV_BF16>(a, want_h, s) : launch_t<CEV_F32>(a, want_h, s);
}

} // namespace cev
