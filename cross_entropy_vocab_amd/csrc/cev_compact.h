// cev_compact.h -- stable compaction of the valid rows of one tile: the
// ascending list of rows whose label is neither ignore_index nor out of range
// and whose mask byte (if any) is nonzero (ms-swift PR #10353, PR information:
// supervised rows are picked after label alignment and before the loss, and
// the losses go back to the per-token positions).  Shared by k_compact and by
// the compaction workgroups that ce_forward appends to its sweep launch.
// Internal to libcevocab.so.
#pragma once

#include "cev_device.h"

namespace cev {

struct CompactTile {
    const int64_t *labels;
    const uint8_t *row_mask;   // may be null
    int64_t ignore_index;
    int64_t vocab;
    int64_t rows;
    int64_t tile;              // rows per tile, a multiple of the workgroup size
    int64_t ntiles;
    int64_t *list;             // out: the valid rows in ascending order
    int64_t *count;            // out: their number (written by the last tile)
};

__device__ __forceinline__ bool gate_row(const int64_t *labels, const uint8_t *row_mask,
                                         int64_t ignore_index, int64_t vocab, int64_t r, bool *bad)
{
    const int64_t t = labels[r];
    const bool masked = row_mask && row_mask[r] == 0;
    const bool ignored = masked || t == ignore_index;
    *bad = !ignored && (t < 0 || t >= vocab);
    return !ignored && !*bad;
}

// One workgroup writes the list entries of tile `ti`.  It first counts the
// valid rows of all earlier tiles itself (a redundant read of at most 9 bytes
// per earlier row, cheaper than a second launch or a grid-wide wait), then
// ranks its own rows with wave ballots, BLOCK rows at a time.  wave_cnt is
// LDS for BLOCK / 64 ints.  Returns whether the tile holds a bad label.
template <int BLOCK>
__device__ __forceinline__ bool compact_tile(const CompactTile &c, int64_t ti, int *wave_cnt)
{
    constexpr int W = BLOCK / kWave;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int64_t t0 = ti * c.tile;
    const int64_t t1 = t0 + c.tile < c.rows ? t0 + c.tile : c.rows;

    int cnt = 0;
#pragma unroll 8
    for (int64_t r = tid; r < t0; r += BLOCK) {
        bool bad;
        cnt += gate_row(c.labels, c.row_mask, c.ignore_index, c.vocab, r, &bad) ? 1 : 0;
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
    for (int64_t base = t0; base < t1; base += BLOCK) {
        const int64_t r = base + tid;
        bool bad = false;
        const bool valid = r < t1 && gate_row(c.labels, c.row_mask, c.ignore_index, c.vocab, r, &bad);
        bad_seen |= bad;
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
            c.list[off + below] = r;
        before += total;
        __syncthreads(); // wave_cnt is rewritten by the next sub-tile
    }
    if (ti == c.ntiles - 1 && tid == 0)
        *c.count = before;
    return bad_seen;
}

// Tiles of whole BLOCK-row sub-tiles, at most kMaxCompactTiles of them.
constexpr int64_t kMaxCompactTiles = 64;
__host__ __device__ inline int64_t compact_tile_rows(int64_t rows, int block)
{
    const int64_t sub = (rows + block - 1) / block;
    const int64_t per = (sub + kMaxCompactTiles - 1) / kMaxCompactTiles;
    return per * block;
}

} // namespace cev
