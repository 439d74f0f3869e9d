// shard.hip -- vocab-parallel (tensor-parallel) form of the forward: each
// rank sweeps its own columns of every row into a partial record, the records
// of all ranks are gathered, and a fixed-order fp64 merge produces the
// outputs of the whole row.  Liger-Kernel PR #1555, Summary, CE bullet:
// vocab-parallel cross-entropy reduces its two sums in one exchange; the merge
// rescales each part's sum by its own base (the partial/combine rule of the
// unsloth-zoo #2080 Summary quoted on the same page).
#include "cev_device.h"
#include "cev_launch.h"
#include "cev_rowclose.h"
#include "cev_sweep_row.h"

namespace cev {
namespace {

// One workgroup per row: the target-excluded sweep over the shard's columns.
// The label is a global column; when another shard holds it, nothing here is
// excluded (t = -1 matches no column).
template <int DT, int BLOCK, int U, bool WANT_H, bool WANT_Z>
__global__ __launch_bounds__(BLOCK) void k_shard_sweep(ShardArgs a)
{
    constexpr int ES = Elem<DT>::kSize, W = BLOCK / kWave;
    __shared__ float sh_f[W];
    __shared__ double sh_d[3 * W];
    __shared__ int64_t sh_i[W];
    const int tid = threadIdx.x;
    const int64_t r = blockIdx.x;
    const int64_t tg = load_uniform(a.labels + r);
    const bool masked = a.row_mask && mask_byte(a.row_mask, r) == 0;
    const bool ignored = masked || tg == a.ignore_index;
    const bool bad = !ignored && (tg < 0 || tg >= a.vocab_total);
    if (ignored || bad) {
        if (tid == 0) {
            cev_vocab_partial p;
            p.m = -INFINITY;
            p.zt = 0.0f;
            p.arg = INT64_MAX;
            p.s = 0.0;
            p.h = 0.0;
            p.zs = 0.0;
            p.flags = 0;
            p.pad = 0;
            a.partials[r] = p;
            if (bad && a.status)
                atomicOr(a.status, (int32_t)CEV_STATUS_BAD_LABEL);
        }
        return;
    }
    const int64_t tl = tg - a.col_offset;
    const bool owns = tl >= 0 && tl < a.vocab;
    const char *rowp = static_cast<const char *>(a.logits) + (size_t)r * (size_t)a.row_stride * ES;
    // The shard's target logit, when it holds the label, is loaded with the
    // sweep's first step (column 0 stands in otherwise, unused).
    const RowStats rs = sweep_row<DT, BLOCK, U, WANT_H, true, true, WANT_Z, true>(
        rowp, a.vocab, owns ? tl : -1, 0, 1, a.c, a.inv_t, sh_f, sh_d, sh_i);
    if (tid == 0) {
        cev_vocab_partial p;
        p.m = rs.M;
        p.zt = owns ? rs.zt : 0.0f;
        p.arg = rs.a_o == INT64_MAX ? INT64_MAX : rs.a_o + a.col_offset;
        p.s = rs.S;
        p.h = rs.Hs;
        p.zs = rs.Zs;
        p.flags = 1 | (owns ? 2 : 0);
        p.pad = 0;
        a.partials[r] = p;
    }
}

template <int DT, int BLOCK, int U>
void launch_shard_t(const ShardArgs &a, bool want_h, bool want_z, hipStream_t s)
{
    dim3 grid((unsigned)a.rows), block(BLOCK);
    if (want_h && want_z)
        hipLaunchKernelGGL((k_shard_sweep<DT, BLOCK, U, true, true>), grid, block, 0, s, a);
    else if (want_h)
        hipLaunchKernelGGL((k_shard_sweep<DT, BLOCK, U, true, false>), grid, block, 0, s, a);
    else if (want_z)
        hipLaunchKernelGGL((k_shard_sweep<DT, BLOCK, U, false, true>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((k_shard_sweep<DT, BLOCK, U, false, false>), grid, block, 0, s, a);
}

// One thread per row; the shards' records are merged one after another in
// shard order, so every rank that merges the same records gets the same bits.
// (Measured on MI355X for 8192 rows x 8 shards: 6.8 us, against 14.2 us with
// one wave per row and the shards spread over its lanes: here neighbouring
// threads read neighbouring records, and every lane runs a closing step.)
constexpr int kMergeBlock = 64;

__global__ __launch_bounds__(kMergeBlock) void k_vocab_merge(MergeArgs a)
{
    const int64_t r = (int64_t)blockIdx.x * kMergeBlock + threadIdx.x;
    if (r >= a.rows)
        return;
    const int64_t t = a.labels[r];
    const bool masked = a.row_mask && a.row_mask[r] == 0;
    const bool ignored = masked || t == a.ignore_index;
    const bool bad = !ignored && (t < 0 || t >= a.vocab);
    auto write_ignored = [&](unsigned st) {
        if (a.logp)
            a.logp[r] = 0.0f;
        a.loss[r] = 0.0f;
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
        if (st && a.status)
            atomicOr(a.status, (int32_t)st);
    };
    if (ignored || bad) {
        write_ignored(bad ? CEV_STATUS_BAD_LABEL : 0u);
        return;
    }

    const int64_t parts = a.parts;
    const cev_vocab_partial *pp = a.partials + r;
    float M = -INFINITY, zt = 0.0f;
    int owners = 0, invalid = 0;
    for (int64_t p = 0; p < parts; ++p) {
        const cev_vocab_partial &pr = pp[(size_t)p * (size_t)a.rows];
        M = fmaxf(M, pr.m);
        invalid += (pr.flags & 1) ? 0 : 1;
        if (pr.flags & 2) {
            ++owners;
            zt = pr.zt;
        }
    }
    if (owners != 1 || invalid != 0) {
        write_ignored(CEV_STATUS_BAD_PARTS);
        return;
    }
    const float B = fmaxf(M, -FLT_MAX);
    const double T = a.temperature;
    double S = 0.0, H = 0.0, Z = 0.0;
    int64_t arg = INT64_MAX;
    for (int64_t p = 0; p < parts; ++p) {
        const cev_vocab_partial &pr = pp[(size_t)p * (size_t)a.rows];
        Z += pr.zs;
        if (pr.s > 0.0) {
            const double bp = (double)fmaxf(pr.m, -FLT_MAX);
            const double f = exp((bp - (double)B) / T);
            S += pr.s * f;
            H += f * (pr.h + ((double)B - bp) / T * pr.s);
        }
        if (pr.m == M && pr.arg < arg)
            arg = pr.arg;
    }
    RowOutputs o;
    o.logp = a.logp;
    o.loss = a.loss;
    o.entropy = a.entropy;
    o.argmax = a.argmax;
    o.saved = a.saved;
    close_row_fp64(o, r, zt, t, M, S, H, arg, T, Z, a.label_smoothing, a.vocab);
}

} // namespace

hipError_t launch_shard_sweep(int dtype, const ShardArgs &a, bool want_h, bool want_z,
                              hipStream_t s)
{
    const Shape sh = pick_shape(a.vocab / (dtype == CEV_BF16 ? 8 : 4));
#define CEV_SHARD_CASE(B, UU)                                                                   \
    if (sh.block == B && sh.U == UU) {                                                          \
        if (dtype == CEV_BF16)                                                                  \
            launch_shard_t<CEV_BF16, B, UU>(a, want_h, want_z, s);                              \
        else                                                                                    \
            launch_shard_t<CEV_F32, B, UU>(a, want_h, want_z, s);                               \
        return hipGetLastError();                                                               \
    }
    CEV_SHARD_CASE(64, 4)
    CEV_SHARD_CASE(128, 4)
    CEV_SHARD_CASE(256, 2)
    CEV_SHARD_CASE(512, 2)
#undef CEV_SHARD_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_vocab_merge(const MergeArgs &a, hipStream_t s)
{
    dim3 grid((unsigned)((a.rows + kMergeBlock - 1) / kMergeBlock)), block(kMergeBlock);
    hipLaunchKernelGGL(k_vocab_merge, grid, block, 0, s, a);
    return hipGetLastError();
}

} // namespace cev
