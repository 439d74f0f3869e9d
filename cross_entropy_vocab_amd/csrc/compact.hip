// compact.hip -- stable device-side compaction of the valid rows, the first
// stage of ce_forward (ms-swift PR #10353, PR information: supervised rows are
// selected after label alignment and before the cross-entropy, and the losses
// are scattered back to the per-token shape).  The count stays on the device,
// so unlike the page's valid-index detection no host synchronization is
// needed; the sweep that follows launches one workgroup per row and the
// surplus workgroups exit on reading the count.
//
// One workgroup of 1024 threads walks the rows in tiles of 8192 (8 rows per
// thread), takes an exclusive prefix sum of the per-thread valid counts, and
// writes the row numbers in ascending order.  It also writes the zero outputs
// of every ignored row, which the sweep never visits.
#include "cev_device.h"
#include "cev_launch.h"

namespace cev {
namespace {

constexpr int kCompactBlock = 1024;
constexpr int kRowsPerThread = 8;

__device__ __forceinline__ int wave_inclusive_scan(int v)
{
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int w = __shfl_up(v, o);
        if (lane >= o)
            v += w;
    }
    return v;
}

__global__ __launch_bounds__(kCompactBlock) void k_compact(CompactArgs a)
{
    constexpr int W = kCompactBlock / kWave;
    __shared__ int wave_tot[W];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    int64_t carry = 0;
    bool bad_seen = false;
    for (int64_t base = 0; base < a.rows; base += (int64_t)kCompactBlock * kRowsPerThread) {
        const int64_t r0 = base + (int64_t)tid * kRowsPerThread;
        unsigned valid_bits = 0;
        int cnt = 0;
#pragma unroll
        for (int i = 0; i < kRowsPerThread; ++i) {
            const int64_t r = r0 + i;
            if (r >= a.rows)
                break;
            const int64_t t = a.labels[r];
            const bool masked = a.row_mask && a.row_mask[r] == 0;
            const bool ignored = masked || t == a.ignore_index;
            const bool bad = !ignored && (t < 0 || t >= a.vocab);
            bad_seen |= bad;
            if (!ignored && !bad) {
                valid_bits |= 1u << i;
                ++cnt;
            } else {
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
            }
        }
        const int incl = wave_inclusive_scan(cnt);
        if (lane == kWave - 1)
            wave_tot[wave] = incl;
        __syncthreads();
        int before = 0, total = 0;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const int x = wave_tot[w];
            before += w < wave ? x : 0;
            total += x;
        }
        int64_t off = carry + before + (incl - cnt);
#pragma unroll
        for (int i = 0; i < kRowsPerThread; ++i)
            if (valid_bits & (1u << i))
                a.rowlist[off++] = r0 + i;
        carry += total;
        __syncthreads(); // wave_tot is rewritten by the next tile
    }
    if (bad_seen && a.status)
        atomicOr(a.status, (int32_t)CEV_STATUS_BAD_LABEL);
    if (tid == 0)
        *a.nlist = carry;
}

} // namespace

hipError_t launch_compact(const CompactArgs &a, hipStream_t s)
{
    hipLaunchKernelGGL(k_compact, dim3(1), dim3(kCompactBlock), 0, s, a);
    return hipGetLastError();
}

} // namespace cev
