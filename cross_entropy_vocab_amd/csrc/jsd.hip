// jsd.hip -- collapse-safe generalized Jensen-Shannon divergence between a
// student and a teacher logit row, with the forward and reverse KL at its two
// ends (the generalized JSD of the unsloth-zoo #2079 Summary quoted on the
// Liger-Kernel PR #1555 page: logits divided by T, log-softmax of both rows,
// beta = 0 forward KL, beta = 1 reverse KL, the mixture in between), and its
// gradient with respect to the student logits, the entry at the student's
// argmax taken as minus the sum of the others (Liger-Kernel PR #1555,
// Summary, "fused KL / JSD" bullet).
//
// Per valid row, with x = z_student / T, y = z_teacher / T:
//   ls_j = (x_j - x_a) - log1p(S_s),  S_s = sum_{j != a} e^(x_j - x_a)
//   (a = first argmax; the same for the teacher), so log p at the argmax is
//   -log1p(S), not a difference of two nearly equal numbers;
//   delta_j = lt_j - ls_j;
//   beta = 0: loss = sum pt delta,              d_j = (ps_j - pt_j) / T
//   beta = 1: loss = -sum ps delta,             d_j = ps_j (-delta_j - loss) / T
//   else:     r = ls - lm, q = lt - lm as functions of delta (log1p / expm1
//             of a non-positive exponent), K = sum ps r,
//             loss = beta sum pt q + (1 - beta) K, d_j = (1 - beta) ps_j (r_j - K) / T
// all times the row's upstream gradient g.
//
//   k_jsd_forward   one workgroup per row.  Pass 1 reads both rows once
//                   and keeps, per lane, each row's maximum, its first column
//                   and the sum of the other columns at that maximum (fp64):
//                   when the maximum moves, the old maximum's own term 1 joins
//                   the rescaled sum, so the argmax is excluded without a
//                   second sweep.  At the two KL ends the loss is accumulated
//                   in the same pass against the running maxima (KlAcc); in
//                   between, pass 2 re-reads both rows and sums the loss terms
//                   in fp64.  Writes the loss and a 48-byte record per row,
//                   which at beta < 1 also holds the student-argmax entry of
//                   the gradient (minus the fp64 sum of the others) unless
//                   the row is so peaked that those sums lose terms below the
//                   fp32 range that matter.
//   k_jsd_bwd_tiles one-shot slices of 8192 columns (beta < 1, 16-byte
//                   aligned rows): every entry elementwise, the argmax entry
//                   from the record; rows without it are left to
//   k_jsd_backward  one workgroup per row (beta = 1, unaligned rows, or the
//                   rows above): one read of both rows, one write of the
//                   gradient, the argmax entry written last from the row's
//                   own sum.
#include "cev_device.h"
#include "cev_launch.h"

namespace cev {
namespace {

constexpr int kJB = 256;   // threads per row

// Largest value m seen, its first column, and the sum over the other columns
// seen of 2^((z - m) c).
struct MaxSum {
    float m;
    int col;
    double s;
};

__device__ __forceinline__ MaxSum ms_empty() { return MaxSum{-INFINITY, INT32_MAX, 0.0}; }

// Merge two states: the larger maximum wins (then the lower column); the
// loser's maximum element becomes one of the others.
__device__ __forceinline__ MaxSum ms_merge(MaxSum a, MaxSum b, float c)
{
    if (b.m > a.m || (b.m == a.m && b.col < a.col)) {
        const MaxSum t = a;
        a = b;
        b = t;
    }
    if (b.m == -INFINITY)
        return a;
    if (b.m == a.m)
        a.s += b.s + 1.0;
    else
        a.s += (b.s + 1.0) * (double)exp2_hw((b.m - a.m) * c);
    return a;
}

// The sweeps keep the running maximum wave-uniform: every lane of a wave holds
// the same m and col (the largest value the wave has seen and its first
// column) and its own share s of the sum over the other columns; lane 0 also
// holds the terms of earlier maxima.  A step moves m only when some lane sees
// a larger value -- a scalar branch taken about ln(steps) times per row --
// and otherwise adds its terms with no per-column test.  The loops are
// wave-convergent: in a step where some lanes have no column (MASK), those
// lanes add nothing.

// Largest of n values (-inf for a lane without a column).
template <int N>
__device__ __forceinline__ float vec_max(const float (&v)[N])
{
    float m = v[0];
#pragma unroll
    for (int i = 1; i < N; ++i)
        m = fmaxf(m, v[i]);
    return m;
}

// Move the wave's maximum to m2 = the largest value of this step (larger than
// st.m), at its lowest column: every lane's share is scaled by
// f = 2^((m - m2) c) and lane 0 adds the old maximum's own term f.  Returns
// the index of m2's column among this lane's n values, or -1.
template <int N>
__device__ __forceinline__ int wm_move(MaxSum &st, const float (&v)[N], float vm, int col0,
                                       float c, bool lane0)
{
    const float m2 = wave_max(fmaxf(vm, st.m));
    int64_t mine = INT32_MAX;
    if (vm == m2) {
#pragma unroll
        for (int i = N - 1; i >= 0; --i)
            if (v[i] == m2)
                mine = col0 + i;
    }
    const int c2 = (int)wave_min(mine);
    if (st.m != -INFINITY) {
        const double f = (double)exp2_hw((st.m - m2) * c);
        st.s = st.s * f + (lane0 ? f : 0.0);
    }
    st.m = m2;
    st.col = c2;
    const int e = c2 - col0;
    return (e >= 0 && e < N) ? e : -1;
}

// One step of a sweep over one row: n values from column col0.
template <bool MASK, int N>
__device__ __forceinline__ void ms_step(MaxSum &st, const float (&v)[N], int col0, float c,
                                        bool lane0, bool valid)
{
    float vm = vec_max(v);
    if (MASK && !valid)
        vm = -INFINITY;
    int ex = -1;
    const bool rise = __any(vm > st.m);
    if (rise)
        ex = wm_move(st, v, vm, col0, c, lane0);
    if (MASK && !valid)
        return;
    float acc = 0.0f;
    if (rise) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const float t = exp2_hw((v[i] - st.m) * c);
            acc += i == ex ? 0.0f : t;
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i)
            acc += exp2_hw((v[i] - st.m) * c);
    }
    st.s += (double)acc;
}

// The row's state from the waves' states: the lanes of a wave share m and
// col, so their shares add; waves merge through LDS.
template <int BLOCK>
__device__ __forceinline__ MaxSum ms_block(MaxSum st, float c, MaxSum *sh)
{
    st.s = wave_sum(st.s);
    const int w = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0)
        sh[w] = st;
    __syncthreads();
    MaxSum r = sh[0];
#pragma unroll
    for (int i = 1; i < BLOCK / kWave; ++i)
        r = ms_merge(r, sh[i], c);
    __syncthreads();
    return r;
}

// Single-pass loss of the two KL ends.  P is the row whose probabilities
// weight the loss (the teacher for beta = 0, the student for beta = 1), Q the
// other; A = sum_j w_j [(zP_j - mP) - (zQ_j - mQ)] with w_j = e^((zP_j - mP)/T)
// against the running maxima mP, mQ, so that at the end
//   loss = A / (T W) +- (log1p(S_s) - log1p(S_t)),  W = sum_j w_j = 1 + S_P.
// When mQ rises by d every bracket grows by d: A += d W.  When mP rises by d
// every weight shrinks by e^(-d/T) and every bracket by d:
// A = e^(-d/T) (A - d W).  The column of each row's own maximum contributes
// exactly 0 to its bracket, so a peaked row loses nothing to cancellation.
// Each lane holds its share of A; W's share is the lane's s (plus the
// maximum's own term 1 in lane 0).
struct KlAcc {
    double a;
};

// The terms of n columns; EX: column ep of P and eq of Q (the maxima, when
// they moved in this step) are left out of the sums.  The weight
// 2^((zP - mP) c) of each column serves both P's sum and A.
template <bool EX, int N>
__device__ __forceinline__ void kl_terms(KlAcc &k, MaxSum &sp, MaxSum &sq, const float (&xp)[N],
                                         const float (&xq)[N], float c, int ep, int eq)
{
    float accp = 0.0f, accq = 0.0f, acca = 0.0f;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const float ap = xp[i] - sp.m, aq = xq[i] - sq.m;
        const float wp = exp2_hw(ap * c), wq = exp2_hw(aq * c);
        accp += (EX && i == ep) ? 0.0f : wp;
        accq += (EX && i == eq) ? 0.0f : wq;
        acca = fmaf(wp, ap - aq, acca);
        // one column's chain at a time: the other waves on the SIMD hide its
        // latency, and the live registers stay within 8 waves per SIMD
        __builtin_amdgcn_sched_barrier(0);
    }
    sp.s += (double)accp;
    sq.s += (double)accq;
    k.a += (double)acca;
}

// One step of the single pass: n values of P and Q from column col0.
template <bool MASK, int N>
__device__ __forceinline__ void kl_step(KlAcc &k, MaxSum &sp, MaxSum &sq, const float (&xp)[N],
                                        const float (&xq)[N], int col0, float c, bool lane0,
                                        bool valid)
{
    float vp = vec_max(xp), vq = vec_max(xq);
    if (MASK && !valid) {
        vp = -INFINITY;
        vq = -INFINITY;
    }
    int ep = -1, eq = -1;
    const bool rq = __any(vq > sq.m), rp = __any(vp > sp.m);
    if (rq) {
        // (the shifts are differences of two floats, exact in fp64)
        const float mq0 = sq.m;
        eq = wm_move(sq, xq, vq, col0, c, lane0);
        if (mq0 != -INFINITY && sp.m != -INFINITY)
            k.a += ((double)sq.m - (double)mq0) * (sp.s + (lane0 ? 1.0 : 0.0));
    }
    if (rp) {
        const float mp0 = sp.m;
        const double w0 = sp.s + (lane0 ? 1.0 : 0.0);
        ep = wm_move(sp, xp, vp, col0, c, lane0);
        if (mp0 != -INFINITY)
            k.a = (double)exp2_hw((mp0 - sp.m) * c) * (k.a - ((double)sp.m - (double)mp0) * w0);
    }
    if (MASK && !valid)
        return;
    if (rq || rp)
        kl_terms<true>(k, sp, sq, xp, xq, c, ep, eq);
    else
        kl_terms<false>(k, sp, sq, xp, xq, c, -1, -1);
}

// Merge lane b's (P, Q, A) into lane a's: both A are brought to the merged
// maxima first.
__device__ __forceinline__ void kl_merge(KlAcc &ka, MaxSum &pa, MaxSum &qa, KlAcc kb, MaxSum pb,
                                         MaxSum qb, float c)
{
    const float Mp = fmaxf(pa.m, pb.m), Mq = fmaxf(qa.m, qb.m);
    double A = 0.0;
    if (pa.m != -INFINITY)
        A += (double)exp2_hw((pa.m - Mp) * c) *
             (ka.a + (((double)Mq - qa.m) - ((double)Mp - pa.m)) * (pa.s + 1.0));
    if (pb.m != -INFINITY)
        A += (double)exp2_hw((pb.m - Mp) * c) *
             (kb.a + (((double)Mq - qb.m) - ((double)Mp - pb.m)) * (pb.s + 1.0));
    ka.a = A;
    pa = ms_merge(pa, pb, c);
    qa = ms_merge(qa, qb, c);
}

template <int BLOCK>
__device__ __forceinline__ void kl_block(KlAcc &k, MaxSum &sp, MaxSum &sq, float c,
                                         MaxSum *shp, MaxSum *shq, double *sha)
{
    sp.s = wave_sum(sp.s);
    sq.s = wave_sum(sq.s);
    k.a = wave_sum(k.a);
    const int w = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) {
        shp[w] = sp;
        shq[w] = sq;
        sha[w] = k.a;
    }
    __syncthreads();
    sp = shp[0];
    sq = shq[0];
    k.a = sha[0];
#pragma unroll
    for (int i = 1; i < BLOCK / kWave; ++i)
        kl_merge(k, sp, sq, KlAcc{sha[i]}, shp[i], shq[i], c);
    __syncthreads();
}

// Per-row constants of pass 2 and of the backward.
constexpr float kLog2e = 1.4426950408889634f, kLn2 = 0.6931471805599453f;
constexpr double kLn2d = 0.69314718055994530942;

struct JsdRow {
    float ms, mt;          // stored maxima
    float ls2, lt2;        // log1p(S_s), log1p(S_t) in log2 units
    float dl0;             // log1p(S_s) - log1p(S_t), rounded once from fp64
    float dl2;             // the same in log2 units
    float lt2b;            // lt2 - log2(beta): beta pt = 2^((zt - mt) c - lt2b)
};

// l2b = log2(beta) as a float (0 where beta * pt is not needed).
__device__ __forceinline__ JsdRow jsd_row(float ms, float ls0, float mt, float lt0, float dl0,
                                          float l2b = 0.0f)
{
    const float lt2 = lt0 * kLog2e;
    return JsdRow{ms, mt, ls0 * kLog2e, lt2, dl0, dl0 * kLog2e, lt2 - l2b};
}

// The mixture's gaps in log2 units, r2 = (ls - lm)/ln2 and q2 = (lt - lm)/ln2,
// from d2 = (lt - ls)/ln2:
// beta e^lt + (1 - beta) e^ls = e^ls (1 + beta (e^delta - 1))
//                             = e^lt (1 + (1 - beta) (e^-delta - 1)),
// with the exponent never positive.  Hardware exp2 / log2 suffice: the gaps
// then err by a few 1e-7 absolute, the size of the error the
// log-probabilities they are built from already carry, and d2 = 0 gives
// exactly 0.  Forward and backward form r2 by these same fp32 steps, so a
// column's gap rounds the same in both.
//
// With w the weight of the larger probability's term (beta where d2 <= 0,
// else 1 - beta) and c = 1 - w, the argument of the log is w e + c: one FMA
// of two non-negative terms, good to fp32 precision relative to itself even
// where it is as small as c (beta = 1e-6 with e near 0, where 1 + w (e - 1)
// would lose both c, to w's rounding, and e, to the rounding of e - 1).  The
// fp32 pair (beta, 1 - beta) is chosen so that it sums to exactly 1 in fp32,
// so e = 1 gives exactly 1 and d2 = 0 a zero gap.
struct MixW {
    float b, b1;   // beta and 1 - beta in fp32, b + b1 == 1 exactly in fp32
};

__device__ __forceinline__ MixW mix_w(double beta)
{
    float b = (float)beta, b1 = (float)(1.0 - beta);
    // the rounding errors of the pair are below 4.5e-8, so moving the larger
    // by one ulp (6e-8) towards the deficit always reaches a sum of 1
    const float sum = b + b1;
    if (sum != 1.0f) {
        float &big = b >= b1 ? b : b1;
        // (both are positive and finite: one ulp is one step of the bits)
        big = __uint_as_float(__float_as_uint(big) + (sum > 1.0f ? 0xFFFFFFFFu : 1u));
    }
    return MixW{b, b1};
}

__device__ __forceinline__ void mix_gaps2(float d2, const MixW &mw, float &r2, float &q2)
{
    const float e = exp2_hw(-fabsf(d2));
    const bool lo = d2 <= 0.0f;
    const float w = lo ? mw.b : mw.b1, c = lo ? mw.b1 : mw.b;
    const float g2 = -__builtin_amdgcn_logf(fmaf(w, e, c));
    r2 = g2 - fmaxf(d2, 0.0f);
    q2 = g2 + fminf(d2, 0.0f);
}

template <int DT>
__device__ __forceinline__ void load_vec(const char *row, int64_t v, float (&out)[Elem<DT>::kVE],
                                         bool stream)
{
    const u32x4 *p = reinterpret_cast<const u32x4 *>(row) + v;
    const u32x4 w = stream ? load16_stream(p) : *p;
    unpack16<DT>(w, out);
}

template <int DT> __device__ __forceinline__ u32x4 load_raw(const char *row, int64_t v, bool stream)
{
    const u32x4 *p = reinterpret_cast<const u32x4 *>(row) + v;
    return stream ? load16_stream(p) : *p;
}

template <bool B> struct Flag {
    static constexpr bool value = B;
};

// Visit the 16-byte vectors tid, tid + kJB, ... < nv of both rows in a
// wave-convergent loop (every thread takes the same number of steps), with
// the next pair's loads issued before the current pair's arithmetic.
// f(xs, xt, col0, Flag<MASK>, valid): MASK only in the last step, where a
// thread past the end has valid = false and undefined values.
template <int DT, bool STREAM, class F>
__device__ __forceinline__ void sweep_pairs(const char *rs, const char *rt, int64_t nv, int tid,
                                            F &&f)
{
    constexpr int VE = Elem<DT>::kVE;
    const int64_t steps = (nv + kJB - 1) / kJB;
    int64_t v = tid;
    u32x4 cs = {0u, 0u, 0u, 0u}, ct = cs;
    if (steps > 0 && v < nv) {
        cs = load_raw<DT>(rs, v, STREAM);
        ct = load_raw<DT>(rt, v, STREAM);
    }
    for (int64_t k = 0; k + 1 < steps; ++k) {   // every thread has a vector
        const int64_t vn = v + kJB;
        u32x4 ns = cs, nt = ct;
        if (vn < nv) {
            ns = load_raw<DT>(rs, vn, STREAM);
            nt = load_raw<DT>(rt, vn, STREAM);
        }
        float xs[VE], xt[VE];
        unpack16<DT>(cs, xs);
        unpack16<DT>(ct, xt);
        f(xs, xt, (int)(v * VE), Flag<false>{}, true);
        cs = ns;
        ct = nt;
        v = vn;
    }
    if (steps > 0) {   // the last step, outside the loop
        float xs[VE], xt[VE];
        unpack16<DT>(cs, xs);
        unpack16<DT>(ct, xt);
        f(xs, xt, (int)(v * VE), Flag<true>{}, v < nv);
    }
}

template <int DT> __device__ __forceinline__ float load_one(const char *row, int64_t j)
{
    if constexpr (DT == CEV_F32)
        return reinterpret_cast<const float *>(row)[j];
    else
        return bf16_lo(reinterpret_cast<const unsigned short *>(row)[j]);
}

// Columns j0 .. V-1 one at a time, in the same wave-convergent form.
template <int DT, class F>
__device__ __forceinline__ void sweep_tail(const char *rs, const char *rt, int64_t j0, int64_t V,
                                           int tid, F &&f)
{
    for (int64_t b = j0; b < V; b += kJB) {
        const int64_t j = b + tid;
        const bool valid = j < V;
        const float xs[1] = {valid ? load_one<DT>(rs, j) : 0.0f};
        const float xt[1] = {valid ? load_one<DT>(rt, j) : 0.0f};
        f(xs, xt, (int)j, Flag<true>{}, valid);
    }
}

// The mixture's loss terms of n columns, in log2 units: adds sum beta pt q2
// to L, sum ps r2 to K and G3 = sum ps (r2 - ra2), ra2 the gap at the
// student's argmax.
template <int N>
__device__ __forceinline__ void mix_terms(const float (&zs)[N], const float (&zt)[N],
                                          const JsdRow &rc, float c, const MixW &mw, float ra2,
                                          double &L, double &K, double &G3)
{
    float l = 0.0f, k = 0.0f, k3 = 0.0f;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const float as = zs[i] - rc.ms, at = zt[i] - rc.mt;
        const float ps = exp2_hw(fmaf(as, c, -rc.ls2));
        const float ptb = exp2_hw(fmaf(at, c, -rc.lt2b));   // beta pt
        float r2, q2;
        mix_gaps2(fmaf(at - as, c, rc.dl2), mw, r2, q2);
        l = fmaf(ptb, q2, l);
        k = fmaf(ps, r2, k);
        k3 = fmaf(ps, r2 - ra2, k3);
    }
    L += (double)l;
    K += (double)k;
    G3 += (double)k3;
}

// ------------------------------------------------------------------ forward
// The forward's fp32 terms (e^((z - m)/T) in the sums of the others, the
// probabilities in pass 2) are lost below 2^-126.
// The argmax entry it forms from them is kept only when the student's mass
// off its argmax, g0, is at least V 2^-80: the V dropped terms then move it by
// under 2^-46 of g0 (for mixture gaps r up to 10^6 in size, under 2^-26),
// far inside the error of the terms themselves.
__device__ __forceinline__ bool garg_usable(double g0, int64_t V)
{
    return g0 >= (double)V * 0x1p-80;
}

template <int DT, int MODE>
__global__ __launch_bounds__(kJB) __attribute__((amdgpu_waves_per_eu(8, 8))) void k_jsd_forward(JsdArgs a)
{
    constexpr int VE = Elem<DT>::kVE, ES = Elem<DT>::kSize;
    __shared__ MaxSum sh_ms[kJB / kWave];
    __shared__ double sh_d[kJB / kWave];
    const int tid = threadIdx.x;
    const int64_t r = blockIdx.x;
    const bool masked = (a.row_mask && a.row_mask[r] == 0) ||
                        (a.labels && a.labels[r] == a.ignore_index);
    cev_jsd_saved *sv = a.saved + r;
    if (masked) {
        if (tid == 0) {
            a.loss[r] = 0.0f;
            cev_jsd_saved rec{};
            rec.arg = -1;
            *sv = rec;
        }
        return;
    }
    const char *rs = static_cast<const char *>(a.student) + (size_t)r * (size_t)a.s_stride * ES;
    const char *rt = static_cast<const char *>(a.teacher) + (size_t)r * (size_t)a.t_stride * ES;
    const int64_t V = a.vocab, nv = a.vec ? V / VE : 0;   // rows not 16-byte aligned: scalar
    const float c = a.c, inv_t = a.inv_t;
    const bool lane0 = (tid & (kWave - 1)) == 0;

    MaxSum ss = ms_empty(), st = ms_empty();
    if constexpr (MODE != 2) {
        // the KL ends: one pass (P = teacher at beta = 0, student at beta = 1)
        __shared__ MaxSum sh_q[kJB / kWave];
        __shared__ double sh_a[kJB / kWave];
        MaxSum &sp = MODE == 0 ? st : ss, &sq = MODE == 0 ? ss : st;
        KlAcc k{0.0};
        const auto step = [&](const auto &xs, const auto &xt, int col0, auto mask, bool valid) {
            if constexpr (MODE == 0)
                kl_step<decltype(mask)::value>(k, sp, sq, xt, xs, col0, c, lane0, valid);
            else
                kl_step<decltype(mask)::value>(k, sp, sq, xs, xt, col0, c, lane0, valid);
        };
        sweep_pairs<DT, true>(rs, rt, nv, tid, step);
        sweep_tail<DT>(rs, rt, nv * VE, V, tid, step);
        kl_block<kJB>(k, sp, sq, c, sh_ms, sh_q, sh_a);
        if (tid == 0) {
            const double ls0d = log1p(ss.s), lt0d = log1p(st.s);
            const double W = sp.s + 1.0, dl = ls0d - lt0d;
            const double loss = k.a / W * (double)inv_t + (MODE == 0 ? dl : -dl);
            a.loss[r] = (float)loss;
            // beta = 0: the argmax entry is sum_{j != a} pt_j - sum_{j != a} ps_j, both
            // sums formed without cancellation (the teacher's from its own maximum
            // sum when its argmax is the same column, else as 1 - pt_a < 1/2)
            double garg = 0.0;
            if constexpr (MODE == 0) {
                const double g0 = ss.s / (1.0 + ss.s);
                double gt;
                if (ss.col == st.col) {
                    gt = st.s / (1.0 + st.s);
                } else {
                    const double lta = ((double)load_one<DT>(rt, ss.col) - (double)st.m) *
                                           (double)inv_t - lt0d;
                    gt = -expm1(lta);
                }
                garg = gt - g0;
            }
            cev_jsd_saved rec{};
            rec.ms = ss.m;
            rec.ls0 = (float)ls0d;
            rec.mt = st.m;
            rec.lt0 = (float)lt0d;
            rec.k = MODE == 1 ? (float)loss : 0.0f;
            rec.garg = (float)garg;
            rec.arg = ss.col;
            rec.flags = (MODE == 0 && garg_usable(ss.s / (1.0 + ss.s), V)) ? 3 : 1;
            rec.dl = (float)dl;
            *sv = rec;
        }
        return;
    }

    // pass 1: maxima, argmaxes, sums of the others
    const auto step1 = [&](const auto &xs, const auto &xt, int col0, auto mask, bool valid) {
        ms_step<decltype(mask)::value>(ss, xs, col0, c, lane0, valid);
        ms_step<decltype(mask)::value>(st, xt, col0, c, lane0, valid);
    };
    sweep_pairs<DT, false>(rs, rt, nv, tid, step1);
    sweep_tail<DT>(rs, rt, nv * VE, V, tid, step1);
    ss = ms_block<kJB>(ss, c, sh_ms);
    st = ms_block<kJB>(st, c, sh_ms);
    const double ls0d = log1p(ss.s), lt0d = log1p(st.s);
    const float ls0 = (float)ls0d, lt0 = (float)lt0d, dl0 = (float)(ls0d - lt0d);
    const JsdRow rc = jsd_row(ss.m, ls0, st.m, lt0, dl0, (float)log2(a.beta));

    // the mixture gap at the student's argmax, in the same fp32 steps as the
    // terms: with K = sum_j ps_j r_j, sum_{j != a} ps_j (r_j - K) equals
    // ps_a sum_j ps_j (r_j - r_a), in which every column whose gap rounds to
    // r_a's (all of them on a saturated row) contributes exactly 0
    const MixW mw = mix_w(a.beta);
    float ra2, qa2;
    {
        const float at = load_one<DT>(rt, ss.col) - rc.mt, as = 0.0f;
        mix_gaps2(fmaf(at - as, c, rc.dl2), mw, ra2, qa2);
    }

    // pass 2: the loss terms (log2 units)
    double L = 0.0, K = 0.0, G3 = 0.0;
    sweep_pairs<DT, true>(rs, rt, nv, tid, [&](const float (&xs)[VE], const float (&xt)[VE],
                                               int, auto, bool valid) {
        if (valid)
            mix_terms(xs, xt, rc, c, mw, ra2, L, K, G3);
    });
    for (int64_t j = nv * VE + tid; j < V; j += kJB) {
        const float xs[1] = {load_one<DT>(rs, j)}, xt[1] = {load_one<DT>(rt, j)};
        mix_terms(xs, xt, rc, c, mw, ra2, L, K, G3);
    }
    L = block_sum<kJB>(L, sh_d);
    K = block_sum<kJB>(K, sh_d);
    G3 = block_sum<kJB>(G3, sh_d);
    if (tid == 0) {
        const double beta = a.beta;
        const double loss = kLn2d * (L + (1.0 - beta) * K);
        // the argmax entry: -(1 - beta) ps_a G3 (G3 in log2 units)
        const double g0 = ss.s / (1.0 + ss.s);
        a.loss[r] = (float)loss;
        cev_jsd_saved rec{};
        rec.ms = ss.m;
        rec.ls0 = ls0;
        rec.mt = st.m;
        rec.lt0 = lt0;
        rec.k = (float)K;   // log2 units
        rec.garg = (float)(-(1.0 - beta) * kLn2d * G3 / (1.0 + ss.s));
        rec.arg = ss.col;
        rec.flags = garg_usable(g0, V) ? 3 : 1;
        rec.dl = dl0;
        *sv = rec;
    }
}

// ----------------------------------------------------------------- backward
// The row's weight |g| (1 - beta) / T (|g| / T at the ends) is folded into the
// exponents as log2 of it (es = ls2 - log2 w, et = lt2 - log2 w), and where
// the probability is then multiplied by a factor (beta > 0: up to a few
// hundred) it is formed 2^24 too large and scaled back exactly after the
// product, so an entry is flushed to zero only when it is itself below the
// fp32 normal range; the sign of g is applied to the bits (beta = 0) or to
// the scale 2^-24.  EXCL: the student's argmax column gets 0 and the entries
// are summed into sum (the per-row kernel); otherwise every column is written
// as computed and the caller replaces the argmax one.
constexpr float kPreInv = 1.0f / 16777216.0f;   // 2^-24: undoes the 2^24 carried in the exponent
template <int MODE, bool EXCL, int N>
__device__ __forceinline__ void grad_terms(const float (&zs)[N], const float (&zt)[N],
                                           const JsdRow &rc, float es, float et, float c,
                                           float inv_t, const MixW &mw, float kk, unsigned sgn,
                                           int col0, int arg, float (&out)[N], double &sum)
{
    // the scale back from 2^24 (times ln 2 for the mixture, whose gaps are in
    // log2 units), carrying the sign of g
    const float post = __uint_as_float(__float_as_uint(MODE == 2 ? kLn2 * kPreInv : kPreInv) ^ sgn);
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const float as = zs[i] - rc.ms, at = zt[i] - rc.mt;
        const float pw = exp2_hw(fmaf(as, c, -es));
        float d;
        if constexpr (MODE == 0) {
            d = pw - exp2_hw(fmaf(at, c, -et));
            d = __uint_as_float(__float_as_uint(d) ^ sgn);
        } else if constexpr (MODE == 1) {
            const float delta = fmaf(at - as, inv_t, rc.dl0);   // lt - ls
            d = (pw * (-delta - kk)) * post;
        } else {
            float r2, q2;   // kk: K in log2 units
            mix_gaps2(fmaf(at - as, c, rc.dl2), mw, r2, q2);
            d = (pw * (r2 - kk)) * post;
        }
        if constexpr (EXCL) {
            if (col0 + i == arg)
                d = 0.0f;
            acc += d;
        }
        out[i] = d;
    }
    if constexpr (EXCL)
        sum += (double)acc;
}

template <int DT> __device__ __forceinline__ void store_vec(char *row, int64_t v, const float *d)
{
    u32x4 o;
    if constexpr (DT == CEV_F32) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            o[i] = __float_as_uint(d[i]);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            o[i] = pack_bf16x2(d[2 * i], d[2 * i + 1]);
    }
    store16_stream(o, reinterpret_cast<u32x4 *>(row) + v);
}

template <int DT> __device__ __forceinline__ void store_one(char *row, int64_t j, float d)
{
    if constexpr (DT == CEV_F32)
        reinterpret_cast<float *>(row)[j] = d;
    else
        reinterpret_cast<unsigned short *>(row)[j] = to_bf16(d);
}

// REST: after k_jsd_bwd_tiles, only the valid rows whose record has no
// argmax entry.
template <int DT, int MODE, int BB = kJB, bool REST = false>
__global__ __launch_bounds__(BB) void k_jsd_backward(JsdArgs a)
{
    constexpr int VE = Elem<DT>::kVE, ES = Elem<DT>::kSize;
    __shared__ double sh_d[BB / kWave];
    const int tid = threadIdx.x;
    const int64_t r = blockIdx.x;
    const int64_t V = a.vocab, nv = a.vec ? V / VE : 0;
    char *rd = static_cast<char *>(a.dstudent) + (size_t)r * (size_t)a.d_stride * ES;
    const bool masked = (a.row_mask && a.row_mask[r] == 0) ||
                        (a.labels && a.labels[r] == a.ignore_index);
    const cev_jsd_saved sv = a.saved_in[r];
    if (REST && (masked || (sv.flags & 3) != 1))
        return;
    if (masked || !(sv.flags & 1)) {   // no record from the forward: a zero row
        const float z[VE] = {};
        for (int64_t v = tid; v < nv; v += BB)
            store_vec<DT>(rd, v, z);
        for (int64_t j = nv * VE + tid; j < V; j += BB)
            store_one<DT>(rd, j, 0.0f);
        return;
    }
    const char *rs = static_cast<const char *>(a.student) + (size_t)r * (size_t)a.s_stride * ES;
    const char *rt = static_cast<const char *>(a.teacher) + (size_t)r * (size_t)a.t_stride * ES;
    const float c = a.c, inv_t = a.inv_t;
    const JsdRow rc = jsd_row(sv.ms, sv.ls0, sv.mt, sv.lt0, sv.dl);
    const float gr = a.g[r];
    const float wabs = fabsf(gr) * inv_t * (MODE == 2 ? (float)(1.0 - a.beta) : 1.0f);
    const float lw = __log2f(wabs);                  // -inf for g = 0: every entry 0
    const float es = rc.ls2 - lw - (MODE == 0 ? 0.0f : 24.0f), et = rc.lt2 - lw;
    const unsigned sgn = __float_as_uint(gr) & 0x80000000u;
    const MixW mw = mix_w(a.beta);
    double sum = 0.0;
    for (int64_t v = tid; v < nv; v += BB) {
        float xs[VE], xt[VE], d[VE];
        load_vec<DT>(rs, v, xs, true);
        load_vec<DT>(rt, v, xt, true);
        grad_terms<MODE, true>(xs, xt, rc, es, et, c, inv_t, mw, sv.k, sgn, (int)(v * VE),
                               sv.arg, d, sum);
        store_vec<DT>(rd, v, d);
    }
    for (int64_t j = nv * VE + tid; j < V; j += BB) {
        const float xs[1] = {load_one<DT>(rs, j)}, xt[1] = {load_one<DT>(rt, j)};
        float d[1];
        grad_terms<MODE, true>(xs, xt, rc, es, et, c, inv_t, mw, sv.k, sgn, (int)j, sv.arg, d,
                               sum);
        store_one<DT>(rd, j, d[0]);
    }
    sum = block_sum<BB>(sum, sh_d);   // ends with a barrier: every store above is done
    if (tid == 0)
        store_one<DT>(rd, sv.arg, (float)(-sum));
}

// One-shot slices (beta < 1, every row 16-byte aligned): workgroup b handles
// vectors [per sl, per (sl + 1)) of row b / slices, plus the row's tail
// columns in its last slice; the argmax entry comes from the record.  The
// row's inputs are read through the scalar cache and the slice's first step
// of both rows goes out as soon as the record says the tile path owns the
// row, before the other per-row checks resolve.
template <int DT, int MODE, int TB, int TU>
__global__ __launch_bounds__(TB) void k_jsd_bwd_tiles(JsdArgs a, int slices, int64_t per)
{
    constexpr int VE = Elem<DT>::kVE, ES = Elem<DT>::kSize;
    const int tid = threadIdx.x;
    const int64_t r = blockIdx.x / slices;
    const int sl = (int)(blockIdx.x % slices);
    const int64_t V = a.vocab, nv = V / VE;
    const int64_t v0 = (int64_t)sl * per, v1 = v0 + per < nv ? v0 + per : nv;
    char *rd = static_cast<char *>(a.dstudent) + (size_t)r * (size_t)a.d_stride * ES;
    u32x4 *dvp = reinterpret_cast<u32x4 *>(rd);
    const cev_jsd_saved sv = a.saved_in[r];
    const float gr = load_uniform(a.g + r);
    const int64_t lab = a.labels ? load_uniform(a.labels + r) : 0;
    const char *rs = static_cast<const char *>(a.student) + (size_t)r * (size_t)a.s_stride * ES;
    const char *rt = static_cast<const char *>(a.teacher) + (size_t)r * (size_t)a.t_stride * ES;
    const int64_t base0 = v0 + tid;
    float xs[TU][VE], xt[TU][VE];
    if ((sv.flags & 3) == 3) {
#pragma unroll
        for (int u = 0; u < TU; ++u) {
            const int64_t j = base0 + (int64_t)u * TB;
            if (j < v1) {
                load_vec<DT>(rs, j, xs[u], true);
                load_vec<DT>(rt, j, xt[u], true);
            }
        }
    }
    const bool masked = (a.row_mask && mask_byte(a.row_mask, r) == 0) ||
                        (a.labels && lab == a.ignore_index);
    if (!masked && (sv.flags & 3) == 1)
        return;   // valid, no argmax entry in the record: the per-row kernel's
    if (masked || !(sv.flags & 1)) {
        const u32x4 zero = {0u, 0u, 0u, 0u};
        for (int64_t j = base0; j < v1; j += TB)
            store16_stream(zero, dvp + j);
        if (sl == slices - 1 && nv * VE + tid < V)
            store_one<DT>(rd, nv * VE + tid, 0.0f);
        return;
    }
    const float c = a.c, inv_t = a.inv_t;
    const JsdRow rc = jsd_row(sv.ms, sv.ls0, sv.mt, sv.lt0, sv.dl);
    const float wabs = fabsf(gr) * inv_t * (MODE == 2 ? (float)(1.0 - a.beta) : 1.0f);
    const float lw = __log2f(wabs);
    const float es = rc.ls2 - lw - (MODE == 0 ? 0.0f : 24.0f), et = rc.lt2 - lw;
    const unsigned sgn = __float_as_uint(gr) & 0x80000000u;
    const MixW mw = mix_w(a.beta);
    const float darg = gr * inv_t * sv.garg;
    double unused = 0.0;
    for (int64_t base = base0; base < v1; base += (int64_t)TB * TU) {
        if (base != base0) {
#pragma unroll
            for (int u = 0; u < TU; ++u) {
                const int64_t j = base + (int64_t)u * TB;
                if (j < v1) {
                    load_vec<DT>(rs, j, xs[u], true);
                    load_vec<DT>(rt, j, xt[u], true);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < TU; ++u) {
            const int64_t j = base + (int64_t)u * TB;
            if (j < v1) {
                float d[VE];
                const int col0 = (int)(j * VE);
                grad_terms<MODE, false>(xs[u], xt[u], rc, es, et, c, inv_t, mw, sv.k, sgn,
                                        col0, sv.arg, d, unused);
                store_vec<DT>(rd, j, d);
                // the one lane holding the argmax column overwrites it (a later
                // store of the same work-item to the same address)
                if ((unsigned)(sv.arg - col0) < (unsigned)VE)
                    store_one<DT>(rd, sv.arg, darg);
            }
        }
    }
    if (sl == slices - 1 && nv * VE + tid < V) {
        const int64_t j = nv * VE + tid;
        const float xs1[1] = {load_one<DT>(rs, j)}, xt1[1] = {load_one<DT>(rt, j)};
        float d[1];
        grad_terms<MODE, false>(xs1, xt1, rc, es, et, c, inv_t, mw, sv.k, sgn, (int)j, sv.arg,
                                d, unused);
        store_one<DT>(rd, j, j == sv.arg ? darg : d[0]);
    }
}

template <int DT, int MODE, int TB, int TU>
void launch_tiles_t(const JsdArgs &a, hipStream_t s)
{
    const int64_t nv = a.vocab / Elem<DT>::kVE;
    int64_t per = (int64_t)TB * TU;
    int64_t slices = nv > 0 ? (nv + per - 1) / per : 1;
    while ((uint64_t)a.rows * (uint64_t)slices * TB > 0xFFFFFFFFull && slices > 1) {
        per *= 2;
        slices = (nv + per - 1) / per;
    }
    hipLaunchKernelGGL((k_jsd_bwd_tiles<DT, MODE, TB, TU>), dim3((unsigned)(a.rows * slices)),
                       dim3(TB), 0, s, a, (int)slices, per);
}

template <int DT>
void launch_fwd_t(const JsdArgs &a, int mode, hipStream_t s)
{
    const dim3 grid((unsigned)a.rows), block(kJB);
    if (mode == 0)
        hipLaunchKernelGGL((k_jsd_forward<DT, 0>), grid, block, 0, s, a);
    else if (mode == 1)
        hipLaunchKernelGGL((k_jsd_forward<DT, 1>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((k_jsd_forward<DT, 2>), grid, block, 0, s, a);
}

template <int DT>
void launch_bwd_t(const JsdArgs &a, int mode, hipStream_t s)
{
    if (mode != 1 && a.vec) {
        const dim3 grid((unsigned)a.rows), block(kJB);
        // Tile shapes measured on 2048 x 151936 bf16 rows: 256 threads x 2
        // vectors at beta = 0 (271 us against 299 us for 256 x 4), 256 x 1 in
        // between (274 against 295 us).
        if (mode == 0) {
            launch_tiles_t<DT, 0, 256, 2>(a, s);
            hipLaunchKernelGGL((k_jsd_backward<DT, 0, kJB, true>), grid, block, 0, s, a);
        } else {
            launch_tiles_t<DT, 2, 256, 1>(a, s);
            hipLaunchKernelGGL((k_jsd_backward<DT, 2, kJB, true>), grid, block, 0, s, a);
        }
        return;
    }
    const dim3 grid((unsigned)a.rows), block(kJB);
    if (mode == 0)
        hipLaunchKernelGGL((k_jsd_backward<DT, 0>), grid, block, 0, s, a);
    else if (mode == 1)
        hipLaunchKernelGGL((k_jsd_backward<DT, 1>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((k_jsd_backward<DT, 2>), grid, block, 0, s, a);
}

int jsd_mode(double beta) { return beta == 0.0 ? 0 : beta == 1.0 ? 1 : 2; }

} // namespace

// Tuning: the beta < 1 tile backward alone with an explicit shape (rows
// 16-byte aligned; the rows without an argmax entry are not written).
hipError_t launch_jsd_tiles_cfg(int dtype, const JsdArgs &a, int block, int U, hipStream_t s)
{
    const int mode = jsd_mode(a.beta);
    if (mode == 1 || !a.vec)
        return hipErrorInvalidValue;
#define CEV_JT_CASE(B, UU)                                                                      \
    if (block == B && U == UU) {                                                                \
        if (dtype == CEV_BF16)                                                                  \
            mode == 0 ? launch_tiles_t<CEV_BF16, 0, B, UU>(a, s) : launch_tiles_t<CEV_BF16, 2, B, UU>(a, s); \
        else                                                                                    \
            mode == 0 ? launch_tiles_t<CEV_F32, 0, B, UU>(a, s) : launch_tiles_t<CEV_F32, 2, B, UU>(a, s);   \
        return hipGetLastError();                                                               \
    }
    CEV_JT_CASE(128, 1)
    CEV_JT_CASE(128, 2)
    CEV_JT_CASE(256, 1)
    CEV_JT_CASE(256, 2)
    CEV_JT_CASE(256, 4)
    CEV_JT_CASE(64, 2)
#undef CEV_JT_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_jsd_forward(int dtype, const JsdArgs &a, hipStream_t s)
{
    if (dtype == CEV_BF16)
        launch_fwd_t<CEV_BF16>(a, jsd_mode(a.beta), s);
    else
        launch_fwd_t<CEV_F32>(a, jsd_mode(a.beta), s);
    return hipGetLastError();
}

hipError_t launch_jsd_backward(int dtype, const JsdArgs &a, hipStream_t s)
{
    if (dtype == CEV_BF16)
        launch_bwd_t<CEV_BF16>(a, jsd_mode(a.beta), s);
    else
        launch_bwd_t<CEV_F32>(a, jsd_mode(a.beta), s);
    return hipGetLastError();
}

} // namespace cev
