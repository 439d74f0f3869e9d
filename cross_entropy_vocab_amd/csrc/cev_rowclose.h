// cev_rowclose.h -- the per-row closing step shared by the forward sweeps and
// the fused forward+backward: everything after the vocab reduction, in fp64,
// from exact inputs.  Internal to libcevocab.so.
#pragma once

#include "cev_device.h"

namespace cev {

constexpr double kLog2e = 1.4426950408889634074;

struct RowOutputs {
    float *logp;      // each may be null
    float *loss;
    float *entropy;
    int64_t *argmax;
    cev_saved *saved;
};

// Inputs: the stored target logit zt (column t), the largest non-target logit
// M (sum base B = max(M, -FLT_MAX)), S = sum_{j != t} e^{(z_j - B)/T},
// Hs = sum_{j != t} e^{(z_j - B)/T} (B - z_j)/T, Zs = sum_{j != t} z_j, the
// lowest non-target column holding M, T, the label smoothing eps and V.  With
// u = log S + (B - z_t)/T (the collapse-safe form of the Liger-Kernel PR #1555
// Summary, CE bullet):
//   nll = softplus(u) = -log p_t,   q = 1 - p_t = sigmoid(u),
//   lse = z_t/T + nll,   H = p_t nll + q (lse - B/T) + e^{B/T - lse} Hs,
//   loss = (1 - eps) nll + eps (lse - (Zs + z_t) / (T V)),
// every entropy term non-negative; log p = -nll is never smoothed.  Returns
// the saved record (also written to o.saved when that is non-null).
__device__ inline cev_saved close_row_fp64(const RowOutputs &o, int64_t r, float zt, int64_t t,
                                           float M, double S, double Hs, int64_t a_o, double T,
                                           double Zs = 0.0, double eps = 0.0, int64_t V = 1)
{
    const float B = fmaxf(M, -FLT_MAX);
    const double u = S > 0.0 ? log(S) + ((double)B - (double)zt) / T : -INFINITY;
    // softplus(u) and sigmoid(u) share e = e^{-|u|} (one fp64 exp instead of
    // two; the same values as the separate forms, bit for bit).
    const double e = exp(-fabs(u));
    const double loss = fmax(u, 0.0) + log1p(e);
    const double q = (u < 0.0 ? e : 1.0) / (1.0 + e);
    const double lse = (double)zt / T + loss;
    if (o.logp)
        o.logp[r] = (float)(-loss);
    if (o.loss) {
        const double smooth = eps != 0.0 ? lse - (Zs + (double)zt) / (T * (double)V) : 0.0;
        o.loss[r] = (float)((1.0 - eps) * loss + eps * smooth);
    }
    if (o.entropy) {
        double H = 0.0;
        if (S > 0.0)
            H = exp(-loss) * loss + q * (lse - (double)B / T) + exp((double)B / T - lse) * Hs;
        o.entropy[r] = (float)H;
    }
    if (o.argmax)
        o.argmax[r] = (zt > M || (zt == M && t < a_o)) ? t : a_o;
    const float mz = fmaxf(zt, M);
    cev_saved sv;
    sv.m_z = mz;
    sv.log2_d = (float)((lse - (double)mz / T) * kLog2e);
    sv.q = (float)q;
    sv.flags = 1;
    if (o.saved)
        o.saved[r] = sv;
    return sv;
}

} // namespace cev
