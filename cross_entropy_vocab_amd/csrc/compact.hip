// compact.hip -- stable device-side compaction of the valid rows, the first
// stage of ce_forward (ms-swift PR #10353, PR information: supervised rows are
// selected after label alignment and before the cross-entropy, and the losses
// are scattered back to the per-token shape).  The count stays on the device,
// so unlike the page's valid-index detection no host synchronization is
// needed; the sweep that follows launches one workgroup per row and the
// surplus workgroups exit on reading the count.
//
// Up to 64 workgroups of 1024 threads each own a tile of consecutive rows.  A
// workgroup first counts the valid rows of all earlier tiles itself (a
// redundant read of at most 9 bytes per earlier row, which is cheaper than a
// second launch or a grid-wide wait), then ranks its own rows with wave
// ballots and writes them in ascending order.  It also writes the zero
// outputs of every ignored row in its tile, which the sweep never visits.
#include "cev_device.h"
#include "cev_launch.h"

namespace cev {
namespace {

constexpr int kCompactBlock = 1024;
constexpr int kMaxCompactBlocks = 64;

__device__ __forceinline__ bool row_is_valid(const CompactArgs &a, int64_t r, bool *bad)
{
    const int64_t t = a.labels[r];
    const bool masked = a.row_mask && a.row_mask[r] == 0;
    const bool ignored = masked || t == a.ignore_index;
    *bad = !ignored && (t < 0 || t >= a.vocab);
    return !ignored && !*bad;
}

__global__ __launch_bounds__(kCompactBlock) void k_compact(CompactArgs a, int64_t tile)
{
    constexpr int W = kCompactBlock / kWave;
    __shared__ int wave_cnt[W];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int64_t t0 = (int64_t)blockIdx.x * tile;
    const int64_t t1 = t0 + tile < a.rows ? t0 + tile : a.rows;

    // Valid rows before this tile.
    int cnt = 0;
#pragma unroll 8
    for (int64_t r = tid; r < t0; r += kCompactBlock) {
        bool bad;
        cnt += row_is_valid(a, r, &bad) ? 1 : 0;
    }
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1)
        cnt += __shfl_xor(cnt, o);
    if (lane == 0)
        wave_cnt[wave] = cnt;
    __syncthreads();
    int64_t before = 0;
#pragma unroll
    for (int w = 0; w < W; ++w)
        before += wave_cnt[w];
    __syncthreads();

    bool bad_seen = false;
    for (int64_t base = t0; base < t1; base += kCompactBlock) {
        const int64_t r = base + tid;
        bool bad = false;
        const bool in = r < t1;
        const bool valid = in && row_is_valid(a, r, &bad);
        bad_seen |= bad;
        if (in && !valid) {
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
        const unsigned long long m = __ballot(valid);
        const int below = __popcll(m & ((1ull << lane) - 1ull));
        if (lane == 0)
            wave_cnt[wave] = __popcll(m);
        __syncthreads();
        int64_t off = before, total = 0;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const int x = wave_cnt[w];
            off += w < wave ? x : 0;
            total += x;
        }
        if (valid)
            a.rowlist[off + below] = r;
        before += total;
        __syncthreads(); // wave_cnt is rewritten by the next sub-tile
    }
    if (bad_seen && a.status)
        atomicOr(a.status, (int32_t)CEV_STATUS_BAD_LABEL);
    if (blockIdx.x == gridDim.x - 1 && tid == 0)
        *a.nlist = before;
}

} // namespace

hipError_t launch_compact(const CompactArgs &a, hipStream_t s)
{
    // Tiles of whole 1024-row sub-tiles, at most 64 workgroups.
    const int64_t sub = (a.rows + kCompactBlock - 1) / kCompactBlock;
    const int64_t per = (sub + kMaxCompactBlocks - 1) / kMaxCompactBlocks;
    const int64_t tile = per * kCompactBlock;
    const int64_t blocks = (a.rows + tile - 1) / tile;
    hipLaunchKernelGGL(k_compact, dim3((unsigned)blocks), dim3(kCompactBlock), 0, s, a, tile);
    return hipGetLastError();
}

} // namespace cev
