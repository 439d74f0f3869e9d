// cev_sweep_row.h -- the streaming vocab sweep over one row (or one part of
// a row): target-excluded online softmax statistics in fp32 per lane, then
// combined over the workgroup.  Shared by the forward sweeps and the fused
// forward+backward.  Internal to libcevocab.so.
#pragma once

#include "cev_device.h"

namespace cev {

constexpr float kBig = 3.0e38f;

// Running statistics of one lane over the (non-excluded) columns it has seen.
struct LaneState {
    float m;    // exact largest stored value seen, -inf if none
    float s;    // sum of 2^((z - b) c), b = max(m, -FLT_MAX), c = log2(e)/T
    float comp; // Kahan compensation: the true sum is about s - comp
    float h;    // sum of 2^((z - b) c) (b - z), for the entropy (1/T applied at the end)
    float zs;   // plain sum of the stored values (label smoothing only)
    int best;   // code of the first step in which m was reached
};

template <int N> __device__ __forceinline__ float tree_sum(float (&e)[N])
{
#pragma unroll
    for (int w = 1; w < N; w *= 2)
#pragma unroll
        for (int i = 0; i + w < N; i += 2 * w)
            e[i] += e[i + w];
    return e[0];
}

// Fold one step of N values into the lane state.  Excluded columns arrive as
// -inf; MAYBE_INF selects the guarded entropy term for such steps.  WANT_Z
// also sums the stored values.  The entropy term is kept in units of the
// stored values (one subtract and one FMA per column) and scaled by 1/T once
// per lane when the workgroup combines.
template <int DT, int N, bool WANT_H, bool WANT_ARG, bool MAYBE_INF, bool WANT_Z = false>
__device__ __forceinline__ void fold(LaneState &st, float (&v)[N], int code, float c)
{
    float sm = v[0];
#pragma unroll
    for (int i = 1; i < N; ++i)
        sm = fmaxf(sm, v[i]);
    if constexpr (WANT_ARG)
        st.best = sm > st.m ? code : st.best;
    const float mnew = fmaxf(st.m, sm);
    const float bold = fmaxf(st.m, -FLT_MAX);
    const float bnew = fmaxf(mnew, -FLT_MAX);
    // Rescale to the new base; f == 1 exactly when the maximum did not move.
    const float f = exp2_hw((bold - bnew) * c);
    if constexpr (WANT_H)
        st.h = f * fmaf(fminf(bnew - bold, kBig), st.s, st.h);
    st.s *= f;
    st.comp *= f;
    st.m = mnew;

    // The exponentials 8 at a time: the pairwise tree over N values is the
    // tree over the 8-value chunks' trees, and the entropy term is a running
    // chain, so the result is the same as over all N at once while only one
    // chunk's exponentials are live (fewer registers, more waves per SIMD).
    constexpr int C = N < 8 ? N : 8, NC = N / C;
    const float nb = fminf(-bnew * c, kBig);
    float part[NC], zpart[NC];
    float ph = 0.0f;
#pragma unroll
    for (int q = 0; q < NC; ++q) {
        float e[C];
#pragma unroll
        for (int i = 0; i < C; ++i) {
            if constexpr (DT == CEV_F32)
                // (z - b) first: exact for the terms near the maximum that dominate.
                e[i] = exp2_hw((v[q * C + i] - bnew) * c);
            else
                e[i] = exp2_hw(fmaf(v[q * C + i], c, nb));
        }
        if constexpr (WANT_H) {
#pragma unroll
            for (int i = 0; i < C; ++i) {
                float d = bnew - v[q * C + i];
                if constexpr (MAYBE_INF)
                    d = fminf(d, kBig);
                ph = fmaf(e[i], d, ph);
            }
        }
        if constexpr (WANT_Z) {
            // sum of the stored values (excluded columns count 0)
            float zv[C];
#pragma unroll
            for (int i = 0; i < C; ++i)
                zv[i] = MAYBE_INF ? (v[q * C + i] == -INFINITY ? 0.0f : v[q * C + i]) : v[q * C + i];
            zpart[q] = tree_sum(zv);
        }
        part[q] = tree_sum(e);
    }
    if constexpr (WANT_H)
        st.h += ph;
    if constexpr (WANT_Z)
        st.zs += tree_sum(zpart);
    const float ps = tree_sum(part);
    const float y = ps - st.comp;
    const float tsum = st.s + y;
    st.comp = (tsum - st.s) - y;
    st.s = tsum;
}

template <int DT, int U>
__device__ __forceinline__ void unpack_step(const u32x4 (&w)[U], float (&v)[U * Elem<DT>::kVE])
{
    constexpr int VE = Elem<DT>::kVE;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float t[VE];
        unpack16<DT>(w[u], t);
#pragma unroll
        for (int e = 0; e < VE; ++e)
            v[u * VE + e] = t[e];
    }
}

// Geometry of the column range one workgroup sweeps.  A row is `ahead` scalar
// columns up to its first 16-byte boundary, then 16-byte vectors, then fewer
// than VE scalar columns.  A workgroup takes vectors [vbeg, vbeg + nvec) of
// that row (nfull wave steps of CH vectors, then nrem single vectors), plus the
// head columns [0, head) if it owns the row's start and the tail columns
// [tail0, tail1) if it owns the row's end.
struct RowGeom {
    int head;
    int64_t ahead;            // the row's head length (column of vector 0)
    int64_t vbeg, nvec, nfull, nrem;
    int64_t tail0, tail1;
};

// Split the row into `parts` ranges of whole vectors; part `p` of them.
template <int DT, int U>
__device__ __forceinline__ RowGeom row_geom(const char *rowp, int64_t V, int64_t p, int64_t parts)
{
    constexpr int VE = Elem<DT>::kVE, ES = Elem<DT>::kSize;
    constexpr int64_t CH = (int64_t)kWave * U;
    RowGeom g;
    int64_t h = (int64_t)(((16u - ((unsigned)(uintptr_t)rowp & 15u)) & 15u) / ES);
    g.ahead = h < V ? h : V;
    const int64_t nv = (V - g.ahead) / VE;
    if (parts == 1) {
        // whole rows: no 64-bit divisions in front of the first load
        g.vbeg = 0;
        g.nvec = nv;
    } else {
        g.vbeg = nv * p / parts;
        g.nvec = nv * (p + 1) / parts - g.vbeg;
    }
    g.nfull = g.nvec / CH;
    g.nrem = g.nvec - g.nfull * CH;
    g.head = p == 0 ? (int)g.ahead : 0;
    g.tail0 = g.ahead + nv * VE;
    g.tail1 = p == parts - 1 ? V : g.tail0;
    return g;
}

// Codes name the step where a lane's maximum first appeared, so that the
// argmax can be found by re-reading that one step:
//   [0, 16)                         head column
//   16 + k                          wave step (chunk) k of the range
//   16 + nfull + i                  remainder vector vbeg + nfull*CH + i
//   16 + nfull + nrem + i           tail column tail0 + i
// The argmax re-read, in two halves so that its loads are in flight while
// the workgroup reduces its sums: rescan_issue loads the vectors of the step
// named by `code` (the one where this lane first saw its maximum M; a lane
// whose maximum is not M loads nothing), rescan_finish finds the lowest
// column there holding M, the target excepted.
template <int DT, int U> struct Rescan {
    u32x4 w[U];
    int64_t col0;   // first column of w[0]; vector u starts 64 u vectors later
    int kind;       // 0 nothing, 1 a head column, 2 a wave step, 3 one vector, 4 a tail column
    int64_t col;    // kinds 1 and 4: the column itself
};

template <int DT, int U>
__device__ __forceinline__ Rescan<DT, U> rescan_issue(const char *rowp, const RowGeom &g, int code,
                                                      bool mine)
{
    constexpr int VE = Elem<DT>::kVE;
    constexpr int64_t CH = (int64_t)kWave * U;
    const int lane = threadIdx.x & (kWave - 1);
    const u32x4 *vp = reinterpret_cast<const u32x4 *>(rowp + (size_t)g.ahead * Elem<DT>::kSize);
    Rescan<DT, U> r;
    r.kind = 0;
    r.col0 = 0;
    r.col = 0;
    if (!mine)
        return r;
    if (code < 16) {
        r.kind = 1;
        r.col = code;
        return r;
    }
    int64_t c2 = code - 16;
    if (c2 < g.nfull) {
        const int64_t j0 = g.vbeg + c2 * CH + lane;
#pragma unroll
        for (int u = 0; u < U; ++u)
            r.w[u] = load16_stream(vp + j0 + u * kWave);
        r.kind = 2;
        r.col0 = g.ahead + j0 * VE;
        return r;
    }
    c2 -= g.nfull;
    if (c2 < g.nrem) {
        const int64_t j = g.vbeg + g.nfull * CH + c2;
        r.w[0] = load16_stream(vp + j);
        r.kind = 3;
        r.col0 = g.ahead + j * VE;
        return r;
    }
    c2 -= g.nrem;
    r.kind = 4;
    r.col = g.tail0 + c2;
    return r;
}

// Lowest column of one 16-byte vector (first column col0) holding M, the
// target column t excepted; INT64_MAX if none.
template <int DT>
__device__ __forceinline__ int64_t scan_vec(const u32x4 &w, int64_t col0, float M, int64_t t)
{
    constexpr int VE = Elem<DT>::kVE;
    float v[VE];
    unpack16<DT>(w, v);
    const int64_t dt = t - col0;
    const int te = (dt >= 0 && dt < VE) ? (int)dt : -1;
    int first = VE;
#pragma unroll
    for (int e = VE - 1; e >= 0; --e)
        if (v[e] == M && e != te)
            first = e;
    return first < VE ? col0 + first : INT64_MAX;
}

template <int DT, int U>
__device__ __forceinline__ int64_t rescan_finish(const Rescan<DT, U> &r, float M, int64_t t)
{
    constexpr int VE = Elem<DT>::kVE;
    if (r.kind == 0)
        return INT64_MAX;
    if (r.kind == 1 || r.kind == 4)
        return r.col;
    if (r.kind == 3)
        return scan_vec<DT>(r.w[0], r.col0, M, t);
    int64_t found = INT64_MAX;
#pragma unroll
    for (int u = U - 1; u >= 0; --u) {
        const int64_t f = scan_vec<DT>(r.w[u], r.col0 + (int64_t)u * kWave * VE, M, t);
        found = f != INT64_MAX ? f : found;
    }
    return found;
}


// Loads for a sweep: streaming (nontemporal) when the row is read once, plain
// when a second pass over the same row follows and should find it in cache.
template <bool NT> __device__ __forceinline__ u32x4 load16(const u32x4 *p)
{
    if constexpr (NT)
        return load16_stream(p);
    else
        return *p;
}

struct RowStats {
    float M;       // largest non-target stored value of the range (-inf if none)
    double S;      // sum over the range of e^{(z - B)/T}, B = max(M, -FLT_MAX)
    double Hs;     // sum of e^{(z - B)/T} (B - z)/T (entropy only)
    double Zs;     // sum of the non-target stored values of the range (WANT_Z)
    int64_t a_o;   // lowest non-target column holding M (argmax only)
    float zt;      // the stored target logit (WANT_ZT only)
};

// The first wave step of a sweep: the row's geometry and this wave's first
// vectors, whose loads depend only on the row's address.  Issued before the
// row's label is known, so that the stream is in flight during that load.
template <int DT, int U> struct SweepStart {
    RowGeom g;
    u32x4 cur[U];
};

template <int DT, int U, bool NT>
__device__ __forceinline__ SweepStart<DT, U> sweep_start(const char *rowp, int64_t V, int64_t part,
                                                        int64_t parts)
{
    constexpr int ES = Elem<DT>::kSize;
    constexpr int64_t CH = (int64_t)kWave * U;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    SweepStart<DT, U> s0;
    s0.g = row_geom<DT, U>(rowp, V, part, parts);
    const u32x4 *vp = reinterpret_cast<const u32x4 *>(rowp + (size_t)s0.g.ahead * ES) + s0.g.vbeg;
    if (wave < s0.g.nfull) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            s0.cur[u] = load16<NT>(vp + (int64_t)wave * CH + u * kWave + lane);
    }
    return s0;
}

// Sweep part `part` of `parts` of a row with one workgroup: per lane, fold the
// range's columns (the target column t excluded) into (max, Kahan sum, entropy
// term, first step of the max), then combine the lanes: the exact maximum
// first, one rescale per lane to the common base, fp64 sums; the argmax comes
// from re-reading the one step where each maximal lane first saw the maximum.
// Every thread of the workgroup returns the same statistics.  s0 holds the
// range's geometry and the wave's first step (sweep_start); sh_d holds
// 3 * BLOCK / 64 doubles.
template <int DT, int BLOCK, int U, bool WANT_H, bool WANT_ARG, bool NT, bool WANT_Z = false,
          bool WANT_ZT = false>
__device__ __forceinline__ RowStats sweep_row_from(const char *rowp, int64_t t, const SweepStart<DT, U> &s0,
                                                   float c, float inv_t, float *sh_f, double *sh_d,
                                                   int64_t *sh_i)
{
    constexpr int VE = Elem<DT>::kVE, ES = Elem<DT>::kSize, W = BLOCK / kWave;
    constexpr int64_t CH = (int64_t)kWave * U;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const RowGeom &g = s0.g;
    const u32x4 *vp = reinterpret_cast<const u32x4 *>(rowp + (size_t)g.ahead * ES) + g.vbeg;
    const int64_t col_v = g.ahead + g.vbeg * VE;   // first column of the range's vectors
    LaneState st{-INFINITY, 0.0f, 0.0f, 0.0f, 0.0f, -1};

    int64_t k = wave;
    u32x4 cur[U], nxt[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
        cur[u] = s0.cur[u];
    // The closing step's target logit, loaded after the first step so that
    // waiting for that step never waits for it (column 0 when the range holds
    // no target, t < 0; the value is then unused).
    float zt = 0.0f;
    if constexpr (WANT_ZT)
        zt = load_elem<DT>(rowp, t >= 0 ? t : 0);

    if (tid < g.head) {
        float v[1] = {tid == t ? -INFINITY : load_elem<DT>(rowp, tid)};
        fold<DT, 1, WANT_H, WANT_ARG, true, WANT_Z>(st, v, tid, c);
    }

    // Full wave steps, interleaved over the waves, one step of loads in flight
    // ahead of the arithmetic.
    {
        for (; k < g.nfull; k += W) {
            const int64_t kn = k + W;
            if (kn < g.nfull) {
#pragma unroll
                for (int u = 0; u < U; ++u)
                    nxt[u] = load16<NT>(vp + kn * CH + u * kWave + lane);
            }
            float v[U * VE];
            unpack_step<DT, U>(cur, v);
            const int64_t lo = col_v + k * CH * VE;
            const bool has_t = (uint64_t)(t - lo) < (uint64_t)(CH * VE);
            if (has_t) {
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int e = 0; e < VE; ++e)
                        if (col_v + (k * CH + u * kWave + lane) * VE + e == t)
                            v[u * VE + e] = -INFINITY;
            }
            if (has_t)
                fold<DT, U * VE, WANT_H, WANT_ARG, true, WANT_Z>(st, v, 16 + (int)k, c);
            else
                fold<DT, U * VE, WANT_H, WANT_ARG, false, WANT_Z>(st, v, 16 + (int)k, c);
#pragma unroll
            for (int u = 0; u < U; ++u)
                cur[u] = nxt[u];
        }
    }

    for (int64_t j = g.nfull * CH + tid; j < g.nvec; j += BLOCK) {
        float v[VE];
        unpack16<DT>(load16<NT>(vp + j), v);
#pragma unroll
        for (int e = 0; e < VE; ++e)
            if (col_v + j * VE + e == t)
                v[e] = -INFINITY;
        fold<DT, VE, WANT_H, WANT_ARG, true, WANT_Z>(st, v, 16 + (int)(g.nfull + (j - g.nfull * CH)), c);
    }
    if (g.tail0 + tid < g.tail1) {
        const int64_t col = g.tail0 + tid;
        float v[1] = {col == t ? -INFINITY : load_elem<DT>(rowp, col)};
        fold<DT, 1, WANT_H, WANT_ARG, true, WANT_Z>(st, v, 16 + (int)(g.nfull + g.nrem + tid), c);
    }

    // Combine the lanes: exact maximum first, then each lane rescales its own
    // sum once to the common base and the sums are added in fp64 (one LDS
    // exchange for all of them).  The argmax re-read goes out as soon as the
    // row's maximum is known, from the lanes that hold it.  (Issuing it after
    // the wave's maximum instead, from every wave, measured slower.)
    const float M = block_max<BLOCK>(st.m, sh_f);
    Rescan<DT, U> rsc;
    if constexpr (WANT_ARG)
        rsc = rescan_issue<DT, U>(rowp, g, st.best, M != -INFINITY && st.m == M);
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
    const double S = sums[0];
    double Hs = 0.0;
    if constexpr (WANT_H)
        Hs = sums[1] * (double)inv_t;
    double Zs = 0.0;
    if constexpr (WANT_Z)
        Zs = sums[NS - 1];
    int64_t a_o = INT64_MAX;
    if constexpr (WANT_ARG)
        a_o = block_min<BLOCK>(rescan_finish<DT, U>(rsc, M, t), sh_i);

    return RowStats{M, S, Hs, Zs, a_o, zt};
}

template <int DT, int BLOCK, int U, bool WANT_H, bool WANT_ARG, bool NT, bool WANT_Z = false,
          bool WANT_ZT = false>
__device__ __forceinline__ RowStats sweep_row(const char *rowp, int64_t V, int64_t t, int64_t part, int64_t parts,
                              float c, float inv_t, float *sh_f, double *sh_d, int64_t *sh_i)
{
    const SweepStart<DT, U> s0 = sweep_start<DT, U, NT>(rowp, V, part, parts);
    return sweep_row_from<DT, BLOCK, U, WANT_H, WANT_ARG, NT, WANT_Z, WANT_ZT>(rowp, t, s0, c, inv_t,
                                                                               sh_f, sh_d, sh_i);
}

} // namespace cev
