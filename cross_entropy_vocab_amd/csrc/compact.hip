// compact.hip -- stable device-side compaction of the valid rows, the first
// stage of ce_forward (ms-swift PR #10353, PR information: supervised rows are
// selected after label alignment and before the cross-entropy, and the losses
// are scattered back to the per-token shape).  The count stays on the device,
// so unlike the page's valid-index detection no host synchronization is
// needed; the sweep that follows launches one workgroup per row and the
// surplus workgroups exit on reading the count.
//
// Up to 64 workgroups of 1024 threads each own a tile of consecutive rows
// (compact_tile in cev_compact.h) and also write the zero outputs of every
// ignored row in their tile, which the sweep never visits.  This stand-alone
// form serves the split-row sweep; whole-row sweeps run the same tiles in
// workgroups appended to the sweep launch.
#include "cev_compact.h"
#include "cev_device.h"
#include "cev_launch.h"

namespace cev {
namespace {

constexpr int kCompactBlock = 1024;

__global__ __launch_bounds__(kCompactBlock) void k_compact(CompactArgs a, CompactTile c)
{
    __shared__ int wave_cnt[kCompactBlock / kWave];
    const bool bad_seen = compact_tile<kCompactBlock>(c, blockIdx.x, wave_cnt);
    // Zero outputs of the tile's ignored rows, which the sweep never visits.
    const int64_t t0 = (int64_t)blockIdx.x * c.tile;
    const int64_t t1 = t0 + c.tile < c.rows ? t0 + c.tile : c.rows;
    for (int64_t r = t0 + threadIdx.x; r < t1; r += kCompactBlock) {
        bool bad;
        if (!gate_row(c.labels, c.row_mask, c.ignore_index, c.vocab, r, &bad)) {
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
    if (bad_seen && a.status)
        atomicOr(a.status, (int32_t)CEV_STATUS_BAD_LABEL);
}

} // namespace

hipError_t launch_compact(const CompactArgs &a, hipStream_t s)
{
    CompactTile c;
    c.labels = a.labels;
    c.row_mask = a.row_mask;
    c.ignore_index = a.ignore_index;
    c.vocab = a.vocab;
    c.rows = a.rows;
    c.tile = compact_tile_rows(a.rows, kCompactBlock);
    c.ntiles = (a.rows + c.tile - 1) / c.tile;
    c.list = a.rowlist;
    c.count = a.nlist;
    hipLaunchKernelGGL(k_compact, dim3((unsigned)c.ntiles), dim3(kCompactBlock), 0, s, a, c);
    return hipGetLastError();
}

} // namespace cev
