// lce.hip -- linear cross-entropy: logits = hidden x head^T computed tile by
// tile on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16) and consumed in
// registers, so the [rows, vocab] logits need not reach HBM (the fused linear CE
// / log-prob setting of the unsloth-zoo #2080 Summary quoted on the
// Liger-Kernel PR #1555 page).
//
//   forward   k_lce_fwd: each workgroup owns 256 rows and one vocab split; per
//             256-column tile it runs the K loop over the hidden size, then
//             folds the tile into target-excluded softmax statistics: every
//             lane forms its terms at the row's running maximum, and one
//             reduce-scatter over the 32 lanes that hold a row slot hands
//             each slot's sum to the lane that keeps that row's running
//             state (entropy and value sums alike, when asked); the tile's
//             maximum and its first column are reduced only for a slot where
//             some value exceeds the running maximum.  At the end of its
//             split each row gets one cev_vocab_partial record, and
//             k_vocab_merge closes the rows exactly as for vocab-parallel
//             logits.
//   backward  k_lce_dl recomputes each logit tile and writes
//             dlogits = (g/T)(softmax - onehot) in bf16 (the per-element
//             formula of k_backward, from the saved record); when the
//             forward also stored the fp32 logits (an option that trades
//             R x V x 4 bytes of memory for the recomputation),
//             k_lce_dl_stored forms the same dlogits from them instead.
//             k_lce_gemm then forms dhidden = dlogits x head with the head
//             read as stored (its MFMA fragments formed by transposing LDS
//             reads) and, for a trainable head, dhead = dlogits^T x hidden
//             with both read as stored too.
//
// Tiles: 8 waves in a 4 x 2 grid (two per SIMD), each wave 64 x 128 of C as
// 2 x 4 blocks of 32 x 32; K steps of 64, copied from global memory straight
// into a double-buffered LDS tile of 2 x 64 KB (LDS-DMA).  A 256 x 256 workgroup tile needs
// 64 KB of operands per 256 x 256 x 64 MACs, half the traffic per MAC of a
// 128 x 256 tile, and the second wave on each SIMD covers the first's loads
// and barriers; the LDS-fragment + MFMA loop alone runs at 88% of the bf16
// peak on MI355X.  Fragment layout of the 32x32x16 bf16 MFMA on gfx950 (checked on the
// device): lane l supplies A[l % 32][8 (l / 32) .. +8] and B[same k][l % 32];
// accumulator element v of lane l is C[8 (v / 4) + 4 (l / 32) + v % 4][l % 32].
// In the logit products the B rows are staged permuted so that the four
// 32-column blocks of a wave interleave: lane l of block nb holds output column
// 4 (l % 32) + nb of the wave's 128, so each lane owns four adjacent columns
// of every row it holds (8-byte stores of dlogits).
#include "cev_device.h"
#include "cev_launch.h"

namespace cev {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kLT = 512;                         // threads per workgroup (8 waves)
constexpr int kBM = 256, kBN = 256, kBK = 64;    // workgroup tile
constexpr int kTM = 2, kTN = 4;                  // 32 x 32 blocks per wave (64 x 128)
constexpr int kChunks = kBM * kBK / 8 / kLT;     // 16-byte copies per thread per operand
constexpr float kBigL = 3.0e38f;

struct GemmSmem {
    unsigned short a[2][kBM * kBK];
    unsigned short b[2][kBN * kBK];
};

// Element (row, k) of a staged tile.  Rows are 128 bytes (eight 16-byte
// chunks, the 32 banks once); chunk c of row r is stored at position
// c ^ (r & 7), so the 16-byte fragment reads of 8 consecutive rows at one chunk
// and the staging writes of one row's 8 chunks each touch every bank once.
__device__ __forceinline__ int lds_at(int row, int k)
{
    return row * kBK + ((((k >> 3) ^ row) & 7) << 3) + (k & 7);
}

// Tile row q of a B tile holds matrix row perm_b(q): within each half of 128,
// q = 32 nb + i takes row 4 i + nb.
__device__ __forceinline__ int perm_b(int q)
{
    return (q & 128) | ((q & 31) << 2) | ((q >> 5) & 3);
}

// LDS byte address of a shared-memory pointer.
__device__ __forceinline__ unsigned lds_u32(const unsigned short *lds)
{
    return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) unsigned short *)lds;
}

// Rows [r0, r0 + 256) x k [k0, k0 + 64) of a K-contiguous bf16 matrix
// X[row * ld + k] copied from global memory straight into the LDS tile `lds`
// (global_load_lds_dwordx4: each lane's 16 bytes land at M0 + 16 * lane, with
// no VGPR or LDS-store instruction in between).  Wave w's instruction i fills
// the 64 chunks [512 i + 64 w, +64) of the tile, so each lane fetches the
// chunk that the swizzled layout keeps at its position: tile row q = p / 8,
// logical chunk (p % 8) ^ (q % 8), from matrix row r0 + q (r0 + perm_b(q) for
// a B tile); rows past `rows` re-read the last row (their results are never
// used).  The copies complete in order with the other vector-memory
// operations of the wave, so dma_wait() (vmcnt 0) followed by a barrier
// makes the whole tile visible to every wave.  M0 is set in the same asm
// statement, one wait state before its use.
template <bool PERM>
__device__ __forceinline__ void dma_tile(const unsigned short *X, int64_t ld, int64_t rows,
                                         int64_t r0, int64_t k0, unsigned short *lds, int tid)
{
    const int lane = tid & 63, w = tid >> 6;
    const unsigned base = lds_u32(lds);
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
        const int p = kLT * i + 64 * w + lane;
        const int q = p >> 3;
        const int lc = (p & 7) ^ (q & 7);
        const int mr = PERM ? perm_b(q) : q;
        const int64_t gr = r0 + mr < rows ? r0 + mr : rows - 1;
        const unsigned short *src = X + gr * ld + k0 + lc * 8;
        const unsigned m0 =
            __builtin_amdgcn_readfirstlane(base + (unsigned)(kLT * i + 64 * w) * 16u);
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                     :: "s"(m0), "v"(src) : "memory");
    }
}

// Wait for this wave's tile copies (and its other vector-memory operations).
__device__ __forceinline__ void dma_wait()
{
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int NBLK>
__device__ __forceinline__ void frag_load_kn(const unsigned short *lt, bf16x8 (&f)[NBLK], int ks,
                                             int c0, int lane);

// Fragments of K sub-step ks (16 deep) for this wave: A rows wm*64 + 32 mb +
// (lane % 32), B rows wn*128 + 32 nb + (lane % 32), k = 16 ks + 8 (lane / 32);
// an operand staged K rows x 256 columns (AKN / BKN) goes through
// frag_load_kn instead.

template <bool AKN, bool BKN>
__device__ __forceinline__ void frag_load(const unsigned short *la, const unsigned short *lb,
                                          bf16x8 (&af)[kTM], bf16x8 (&bf)[kTN], int ks, int wm,
                                          int wn, int lane)
{
    const int kk = ks * 16 + (lane >> 5) * 8;
    if constexpr (AKN) {
        frag_load_kn<kTM>(la, af, ks, wm * 64, lane);
    } else {
#pragma unroll
        for (int mb = 0; mb < kTM; ++mb)
            af[mb] = *reinterpret_cast<const bf16x8 *>(
                la + lds_at(wm * 64 + mb * 32 + (lane & 31), kk));
    }
    if constexpr (BKN) {
        frag_load_kn<kTN>(lb, bf, ks, wn * 128, lane);
    } else {
#pragma unroll
        for (int nb = 0; nb < kTN; ++nb)
            bf[nb] = *reinterpret_cast<const bf16x8 *>(
                lb + lds_at(wn * 128 + nb * 32 + (lane & 31), kk));
    }
}

// The same copies with a uniform base: a lane's byte offset from a tile's
// origin does not depend on the K step (nor, up to a uniform row offset, on the
// chunk i), so each copy takes the origin in SGPRs and the lane's offset as a
// 32-bit VGPR (global_load_lds_dwordx4 v, s[..]); the K loops then keep one
// VGPR per operand instead of eight 64-bit addresses.  Used when the tile lies
// inside the matrix and the offsets fit 32 bits (leading dimension < 2^24).
// The asm waits 5 states before the copy in case the base was just moved into
// SGPRs by a vector instruction.
__device__ __forceinline__ void dma_copy_s(const unsigned short *base, unsigned voff, unsigned m0)
{
    // (readfirstlane returns int: each half goes through unsigned, so that the
    // low half is not sign-extended into the high one)
    const uint64_t b = (uint64_t)(uintptr_t)base;
    const uint64_t hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(b >> 32));
    const uint64_t lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)b);
    const uint64_t sb = (hi << 32) | lo;
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(m0), "v"(voff), "s"(sb) : "memory");
}

constexpr int64_t kFastLd = 1 << 24;

// Uniform row offset of chunk i of a K-contiguous tile (row q = 64 i + x of
// the tile, x the lane's row within a chunk; for a B tile, perm_b(q) =
// 128 (i / 2) + 2 (i % 2) + 4 (x % 32) + x / 32).
template <bool PERM> __device__ __forceinline__ int chunk_row(int i)
{
    return PERM ? 128 * (i >> 1) + 2 * (i & 1) : 64 * i;
}

// The lane's byte offset within a K-contiguous tile (see dma_tile).
template <bool PERM> __device__ __forceinline__ unsigned dma_voff(int64_t ld, int tid)
{
    const int lane = tid & 63, w = tid >> 6;
    const int x = 8 * w + (lane >> 3);
    const int lc = (lane & 7) ^ ((lane >> 3) & 7);
    const int row = PERM ? 4 * (x & 31) + (x >> 5) : x;
    return (unsigned)(((int64_t)row * ld + lc * 8) * 2);
}

template <bool PERM>
__device__ __forceinline__ void dma_tile_s(const unsigned short *X, int64_t ld, int64_t r0,
                                           int64_t k0, unsigned voff, unsigned short *lds,
                                           int tid)
{
    const unsigned base = lds_u32(lds) + (unsigned)(tid >> 6) * 1024u;
#pragma unroll
    for (int i = 0; i < kChunks; ++i)
        dma_copy_s(X + (r0 + chunk_row<PERM>(i)) * ld + k0, voff,
                   __builtin_amdgcn_readfirstlane(base + (unsigned)i * (kLT * 16)));
}

// B tiles of an N-contiguous operand X[k * ld + n] (the head as stored, for
// dhidden = dlogits x head) are staged as they lie: 64 K rows of 256 columns,
// 512 bytes each, and the MFMA fragments are formed by gfx950's transposing
// LDS reads.  Chunk c (16 bytes) of row k is stored at position c ^ 4 kn_swz(k):
// one transposing read touches rows {r, r+1, r+2, r+3, r+8, .., r+11} (r a
// multiple of 4) at four adjacent chunks, which the swizzle spreads over eight
// distinct groups of four chunks.
__device__ __forceinline__ int kn_swz(int k) { return (k & 3) | (((k >> 3) & 1) << 2); }

// Rows [k0, k0 + 64) x columns [n0, n0 + 256) of X into the LDS tile, by
// LDS-DMA as in dma_tile: position p holds row p / 32, chunk (p % 32) ^
// 4 kn_swz(row).  Rows past kr re-read row kr - 1 and columns past nc the
// last chunk of the row (the matching A columns are zero, or the output
// columns are never stored).
__device__ __forceinline__ void dma_tile_kn(const unsigned short *X, int64_t ld, int64_t kr,
                                            int64_t nc, int64_t k0, int64_t n0,
                                            unsigned short *lds, int tid)
{
    const int lane = tid & 63, w = tid >> 6;
    const unsigned base = lds_u32(lds);
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
        const int p = kLT * i + 64 * w + lane;
        const int k = p >> 5;
        const int lc = (p & 31) ^ (4 * kn_swz(k));
        const int64_t gk = k0 + k < kr ? k0 + k : kr - 1;
        const int64_t gn = n0 + lc * 8 < nc ? n0 + lc * 8 : nc - 8;
        const unsigned short *src = X + gk * ld + gn;
        const unsigned m0 =
            __builtin_amdgcn_readfirstlane(base + (unsigned)(kLT * i + 64 * w) * 16u);
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                     :: "s"(m0), "v"(src) : "memory");
    }
}

// The lane's byte offset within an N-contiguous tile: row 2 w + lane / 32 of
// each 16-row chunk, chunk (lane % 32) ^ 4 kn_swz(row) (the same for every
// chunk i), whose columns past nc re-read the row's last chunk.
__device__ __forceinline__ unsigned dma_voff_kn(int64_t ld, int64_t n0, int64_t nc, int tid)
{
    const int lane = tid & 63, w = tid >> 6;
    const int k = 2 * w + (lane >> 5);
    const int lc = (lane & 31) ^ (4 * kn_swz(k));
    const int64_t gn = n0 + lc * 8 < nc ? lc * 8 : nc - 8 - n0;
    return (unsigned)(((int64_t)k * ld + gn) * 2);
}

__device__ __forceinline__ void dma_tile_kn_s(const unsigned short *X, int64_t ld, int64_t k0,
                                              int64_t n0, unsigned voff, unsigned short *lds,
                                              int tid)
{
    const unsigned base = lds_u32(lds) + (unsigned)(tid >> 6) * 1024u;
#pragma unroll
    for (int i = 0; i < kChunks; ++i)
        dma_copy_s(X + (k0 + 16 * i) * ld + n0, voff,
                   __builtin_amdgcn_readfirstlane(base + (unsigned)i * (kLT * 16)));
}

// Fragments of K sub-step ks from a tile staged K rows x 256 columns (an
// N-contiguous B, or an M-contiguous A): nblk blocks of 32 columns from column
// c0.  ds_read_b64_tr_b16 works on groups of 16 lanes: lane i of a group reads
// 4 consecutive values, and lane j receives value j % 4 of the reads of lanes
// j / 4, j / 4 + 4, j / 4 + 8, j / 4 + 12 (checked on the device).  Lane i
// reads row k + i / 4 at columns 4 (i % 4) .. +3, so lane j gets column j of
// rows k .. k + 3: two reads give the 8 K values of one column that the
// 32x32x16 MFMA takes from a lane (column l % 32, K 8 (l / 32) .. +8), for A
// as for B.
template <int NBLK>
__device__ __forceinline__ void frag_load_kn(const unsigned short *lt, bf16x8 (&f)[NBLK], int ks,
                                             int c0, int lane)
{
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4s lds_v4s;
    const int g = lane >> 4, i = lane & 15;
#pragma unroll
    for (int nb = 0; nb < NBLK; ++nb) {
        const int col = c0 + nb * 32 + 16 * (g & 1) + 4 * (i & 3);
        v4s h[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int k = ks * 16 + 8 * (g >> 1) + 4 * t + (i >> 2);
            const int e = k * kBN + ((((col >> 3) ^ (4 * kn_swz(k))) & 31) << 3) + (col & 7);
            h[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_v4s *)(const_cast<unsigned short *>(lt) + e));
        }
        const short v8 __attribute__((ext_vector_type(8))) = {h[0][0], h[0][1], h[0][2], h[0][3],
                                                              h[1][0], h[1][1], h[1][2], h[1][3]};
        __builtin_memcpy(&f[nb], &v8, 16);
    }
}

template <bool B> struct Flag {
    static constexpr bool value = B;
};

// One K step of 64 from LDS: 4 sub-steps of 16, 8 MFMAs each per wave, with
// the fragments of sub-step ks + 1 read while the MFMAs of sub-step ks issue
// (one MFMA, one LDS read, in turn).  issue() runs once the first sub-step's
// reads are out: the caller starts the next K step's tile copies there.
struct NoIssue {
    __device__ void operator()() const {}
};

template <bool AKN = false, bool BKN = false, class F = NoIssue>
__device__ __forceinline__ void mma_stage(const unsigned short *la, const unsigned short *lb,
                                          f32x16 (&acc)[kTM][kTN], int wm, int wn, int lane,
                                          F &&issue = NoIssue{})
{
    bf16x8 af[2][kTM], bf[2][kTN];
    auto frags = [&](int ks, bf16x8 (&a)[kTM], bf16x8 (&b)[kTN]) {
        frag_load<AKN, BKN>(la, lb, a, b, ks, wm, wn, lane);
    };
    frags(0, af[0], bf[0]);
    issue();
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
        if (ks + 1 < kBK / 16)
            frags(ks + 1, af[(ks + 1) & 1], bf[(ks + 1) & 1]);
#pragma unroll
        for (int mb = 0; mb < kTM; ++mb)
#pragma unroll
            for (int nb = 0; nb < kTN; ++nb)
                acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    af[ks & 1][mb], bf[ks & 1][nb], acc[mb][nb], 0, 0, 0);
        if (ks + 1 < kBK / 16) {
            // scheduling groups (mask 0x008: MFMA, 0x100: LDS read)
#pragma unroll
            for (int q = 0; q < kTM + kTN; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, kTM * kTN - (kTM + kTN), 0);
        }
    }
}

__device__ __forceinline__ void zero_acc(f32x16 (&acc)[kTM][kTN])
{
#pragma unroll
    for (int mb = 0; mb < kTM; ++mb)
#pragma unroll
        for (int nb = 0; nb < kTN; ++nb)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[mb][nb][v] = 0.0f;
}

// The K loop over every (N tile, K step) pair of one workgroup, with the next
// pair's tile copies in flight during the current pair's MFMAs; after the
// last K step of a tile, epi(tile, acc) consumes the accumulators.  A: rows
// [row0, row0 + 256) of XA; B: 256-row tiles [t_begin, t_end) of XB (staged
// permuted, see perm_b); nk K steps of 64.  Each step ends with dma_wait and a
// barrier: the next buffer is then complete and the current one free.
//
// The last step of a tile is peeled so that the epilogue runs while the next
// tile's first copies are in flight.  Copying straight into LDS (instead of
// through registers and LDS stores) took the forward from 6.8 to 6.3-6.5 ms and
// the dlogits and gradient products by 3-5% on MI355X at 8192 x 2560 x 151936,
// with bit-identical results.
template <class Epi>
__device__ __forceinline__ void gemm_tiles(GemmSmem &sm, const unsigned short *XA, int64_t lda,
                                           int64_t rowsA, int64_t row0, const unsigned short *XB,
                                           int64_t ldb, int64_t rowsB, int64_t nk,
                                           int64_t t_begin, int64_t t_end, Epi &&epi)
{
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 1, wn = w & 1;   // 4 x 2 waves
    if (t_end <= t_begin || nk <= 0)
        return;
    f32x16 acc[kTM][kTN];
    zero_acc(acc);
    const bool fast_a = row0 + kBM <= rowsA && lda < kFastLd, ld_b = ldb < kFastLd;
    const unsigned voff_a = dma_voff<false>(lda, tid), voff_b = dma_voff<true>(ldb, tid);
    auto copy = [&](int64_t b0, int64_t k0, int to) {
        if (fast_a)
            dma_tile_s<false>(XA, lda, row0, k0, voff_a, sm.a[to], tid);
        else
            dma_tile<false>(XA, lda, rowsA, row0, k0, sm.a[to], tid);
        if (ld_b && b0 + kBN <= rowsB)
            dma_tile_s<true>(XB, ldb, b0, k0, voff_b, sm.b[to], tid);
        else
            dma_tile<true>(XB, ldb, rowsB, b0, k0, sm.b[to], tid);
    };
    copy(t_begin * kBN, 0, 0);
    dma_wait();
    __syncthreads();
    int buf = 0;
    for (int64_t tile = t_begin; tile < t_end; ++tile) {
        const int64_t b0 = tile * kBN;
        for (int64_t kt = 1; kt < nk; ++kt) {
            mma_stage(sm.a[buf], sm.b[buf], acc, wm, wn, lane,
                      [&] { copy(b0, kt * kBK, buf ^ 1); });
            dma_wait();
            __syncthreads();
            buf ^= 1;
        }
        const bool more = tile + 1 < t_end;
        if (more)
            copy(b0 + kBN, 0, buf ^ 1);
        mma_stage(sm.a[buf], sm.b[buf], acc, wm, wn, lane);
        epi(tile, acc);
        zero_acc(acc);
        dma_wait();
        __syncthreads();
        buf ^= 1;
    }
}

// One output tile of a long contraction (the gradient products): the same
// K step as gemm_tiles in one branch-free loop (the last step copies its own
// K range again, unused), accumulators returned to the caller.  Measured on
// MI355X for the dhidden shape: 12% faster than running it through gemm_tiles.
// Each operand is K-contiguous (A: rowsA rows from row0; B: rowsB rows from
// col0, staged permuted) or, with AKN / BKN, stored as K rows of contiguous
// M / N values (kA / kB rows, at least mA / nB of them readable per row;
// output rows row0 + 0..255 and columns col0 + 0..255).
template <bool AKN = false, bool BKN = false>
__device__ __forceinline__ void gemm_one_tile(GemmSmem &sm, const unsigned short *XA,
                                              int64_t lda, int64_t rowsA, int64_t row0,
                                              const unsigned short *XB, int64_t ldb,
                                              int64_t rowsB, int64_t col0, int64_t nk,
                                              f32x16 (&acc)[kTM][kTN], int64_t mA = 0,
                                              int64_t nB = 0)
{
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 1, wn = w & 1;
    zero_acc(acc);
    if (nk <= 0)
        return;
    const bool fast_a = AKN ? lda < kFastLd : (row0 + kBM <= rowsA && lda < kFastLd);
    const bool fast_b = BKN ? ldb < kFastLd : (col0 + kBN <= rowsB && ldb < kFastLd);
    const unsigned voff_a = AKN ? dma_voff_kn(lda, row0, mA, tid) : dma_voff<false>(lda, tid);
    const unsigned voff_b = BKN ? dma_voff_kn(ldb, col0, nB, tid) : dma_voff<true>(ldb, tid);
    auto copy = [&](int64_t kstep, int to) {
        const int64_t k0 = kstep * kBK;
        if constexpr (AKN) {
            if (fast_a && k0 + kBK <= rowsA)
                dma_tile_kn_s(XA, lda, k0, row0, voff_a, sm.a[to], tid);
            else
                dma_tile_kn(XA, lda, rowsA, mA, k0, row0, sm.a[to], tid);
        } else {
            if (fast_a)
                dma_tile_s<false>(XA, lda, row0, k0, voff_a, sm.a[to], tid);
            else
                dma_tile<false>(XA, lda, rowsA, row0, k0, sm.a[to], tid);
        }
        if constexpr (BKN) {
            if (fast_b && k0 + kBK <= rowsB)
                dma_tile_kn_s(XB, ldb, k0, col0, voff_b, sm.b[to], tid);
            else
                dma_tile_kn(XB, ldb, rowsB, nB, k0, col0, sm.b[to], tid);
        } else {
            if (fast_b)
                dma_tile_s<true>(XB, ldb, col0, k0, voff_b, sm.b[to], tid);
            else
                dma_tile<true>(XB, ldb, rowsB, col0, k0, sm.b[to], tid);
        }
    };
    copy(0, 0);
    dma_wait();
    __syncthreads();
    int buf = 0;
    for (int64_t it = 0; it < nk; ++it) {
        const int64_t nx = it + 1 < nk ? it + 1 : it;
        mma_stage<AKN, BKN>(sm.a[buf], sm.b[buf], acc, wm, wn, lane, [&] { copy(nx, buf ^ 1); });
        dma_wait();
        __syncthreads();
        buf ^= 1;
    }
}

// Local row (0..255) of accumulator element v of block mb for this lane.
__device__ __forceinline__ int acc_row(int wm, int mb, int v, int lane)
{
    return wm * 64 + mb * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}

// Reductions over the 32 lanes that hold one row (lane bits 0-4), without the
// LDS crossbar: DPP swaps lanes within each quad (quad_perm [1,0,3,2] and
// [2,3,0,1]), then quad with quad (row_half_mirror: lane i of 8 reads 7 - i)
// and eight with eight (row_mirror: lane i of 16 reads 15 - i); the two
// 16-lane rows of each half-wave are combined by v_permlane16_swap, which
// hands each row the other's values.  Every lane ends with the result.
template <int CTRL> __device__ __forceinline__ int dpp(int x)
{
    return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}
template <int CTRL> __device__ __forceinline__ float dpp(float x)
{
    return __int_as_float(dpp<CTRL>(__float_as_int(x)));
}
constexpr int kQuadSwap1 = 0xB1, kQuadSwap2 = 0x4E, kHalfMirror = 0x141, kMirror = 0x140;

template <class T, class Op> __device__ __forceinline__ T row_reduce(T x, Op op)
{
    x = op(x, dpp<kQuadSwap1>(x));
    x = op(x, dpp<kQuadSwap2>(x));
    x = op(x, dpp<kHalfMirror>(x));
    x = op(x, dpp<kMirror>(x));
    unsigned u;
    __builtin_memcpy(&u, &x, 4);
    const auto sw = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    T a, b;
    const unsigned ua = sw[0], ub = sw[1];
    __builtin_memcpy(&a, &ua, 4);
    __builtin_memcpy(&b, &ub, 4);
    return op(a, b);
}
__device__ __forceinline__ float row_max(float x)
{
    return row_reduce(x, [](float p, float q) { return fmaxf(p, q); });
}
__device__ __forceinline__ int row_min(int x)
{
    return row_reduce(x, [](int p, int q) { return min(p, q); });
}

// Reduce-scatter over the 32 lanes of each half-wave: x[k] holds this lane's
// share of row slot k (k < 32); on return lane l holds op over the 32 lanes
// of its half of slot l % 32.  Five exchange stages halve the slots a lane
// carries: lane bit 4 by v_permlane16_swap, which hands the lane pair
// (l, l + 16) of x[k] and x[k + 16] in one instruction (the lane in the
// lower row keeps slot k, the upper one slot k + 16); lane bits 3, 2, 1, 0 by
// DPP (row rotate by 8, half-row mirror, quad swaps), each lane sending the
// half of its slots that its partner keeps.  31 combines in all, against 32
// five-step broadcast reductions.
template <int CTRL, class T> __device__ __forceinline__ T dpp_t(T x)
{
    unsigned u;
    __builtin_memcpy(&u, &x, 4);
    u = (unsigned)__builtin_amdgcn_update_dpp(0, (int)u, CTRL, 0xF, 0xF, false);
    T r;
    __builtin_memcpy(&r, &u, 4);
    return r;
}

template <int CTRL, int N, class T, class Op>
__device__ __forceinline__ void rs_stage(T (&x)[32], bool upper, Op op)
{
#pragma unroll
    for (int j = 0; j < N; ++j) {
        const T send = upper ? x[j] : x[j + N];
        const T keep = upper ? x[j + N] : x[j];
        x[j] = op(keep, dpp_t<CTRL>(send));
    }
}

template <class T, class Op> __device__ __forceinline__ T reduce_scatter32(T (&x)[32], int lane, Op op)
{
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        unsigned a, b;
        __builtin_memcpy(&a, &x[k], 4);
        __builtin_memcpy(&b, &x[k + 16], 4);
        const auto sw = __builtin_amdgcn_permlane16_swap(a, b, false, false);
        T p, q;
        const unsigned u0 = sw[0], u1 = sw[1];
        __builtin_memcpy(&p, &u0, 4);
        __builtin_memcpy(&q, &u1, 4);
        x[k] = op(p, q);
    }
    rs_stage<0x128, 8>(x, (lane & 8) != 0, op);    // row_ror:8, partner l ^ 8
    rs_stage<kHalfMirror, 4>(x, (lane & 4) != 0, op);
    rs_stage<kQuadSwap2, 2>(x, (lane & 2) != 0, op);
    rs_stage<kQuadSwap1, 1>(x, (lane & 1) != 0, op);
    return x[0];
}

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup b on XCD
// b % 8), each with its own L2.  The forward and dlogits grids are renumbered
// so that the workgroups one XCD runs together form a contiguous run of
// (row block, split) pairs: 256 workgroups of 32 row blocks x 8 splits give
// each XCD 4 row blocks x 8 splits, whose hidden slices stay in its L2 while
// the head streams through, instead of every row block on every XCD.
__device__ __forceinline__ int64_t xcd_order(int64_t b, int64_t grid)
{
    return grid % 8 == 0 ? (b % 8) * (grid / 8) + b / 8 : b;
}

// The lane index as a value the compiler cannot see through.  Epilogues run
// once per tile inside the tile loop; their per-row addresses only depend on
// the lane and the row block, so the compiler would otherwise hoist all 32 of
// them above the K loop and keep them live through it (64 VGPRs).
__device__ __forceinline__ int opaque_lane()
{
    int l = (int)(threadIdx.x & 63);
    asm volatile("" : "+v"(l));
    return l;
}

// First output column of the four this lane holds in a wave's 128 columns.
__device__ __forceinline__ int64_t lane_col(int64_t tile, int wn, int lane)
{
    return tile * kBN + wn * 128 + 4 * (lane & 31);
}

// Running target-excluded statistics of one row over the columns seen so far:
// maximum m, sum s of 2^((z - b) c) at b = max(m, -FLT_MAX), entropy term h at
// the same base, value sum zs, first column of the maximum.
struct RowState {
    float m, s, h, zs;
    int arg;
};

// ------------------------------------------------------------------ forward
template <bool WANT_H, bool WANT_Z, bool STORE>
__global__ __launch_bounds__(kLT) void k_lce_fwd(LceArgs a)
{
    __shared__ GemmSmem sm;
    __shared__ int s_lab[kBM];
    __shared__ float s_zt[kBM];
    __shared__ int s_own[kBM];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 1, wn = w & 1;
    const int64_t S = a.splits;
    const int64_t vb = xcd_order(blockIdx.x, gridDim.x);
    const int64_t rb = vb / S, sp = vb % S;
    const int64_t row0 = rb * kBM;
    const int64_t V = a.vocab;
    const int64_t ntiles = (V + kBN - 1) / kBN;
    const int64_t t0 = ntiles * sp / S, t1 = ntiles * (sp + 1) / S;
    if (tid < kBM) {
        const int64_t r = row0 + tid;
        int lab = -1;
        if (r < a.rows) {
            const int64_t t = a.labels[r];
            const bool masked = a.row_mask && a.row_mask[r] == 0;
            if (!masked && t != a.ignore_index && t >= 0 && t < V)
                lab = (int)t;
        }
        s_lab[tid] = lab;
        s_zt[tid] = 0.0f;
        s_own[tid] = 0;
    }
    __syncthreads();

    const float c = a.c, inv_t = a.inv_t;
    // Row slot k = mb * 16 + v of a lane is accumulator row v of block mb: in
    // half h of the wave it is row acc_row(wm, mb, v, lane), and lane
    // h * 32 + k keeps that row's running state.  Every lane of the half also
    // needs each slot's running maximum, which the owners publish in s_mr
    // after each tile.
    RowState st = RowState{-INFINITY, 0.0f, 0.0f, 0.0f, INT32_MAX};
    __shared__ __align__(16) float s_mr[kLT / kWave][kWave];
    s_mr[w][lane] = -INFINITY;
    // the label of row wm * 64 + lane: which tiles hold a target for this wave
    const int mylab = s_lab[wm * 64 + lane];
    // every row of this wave's 64 lies below rows (no per-row check on stores)
    const bool all_rows = row0 + wm * 64 + 64 <= a.rows;

    // One tile: MASK (wave-uniform, rare) when some of this wave's columns
    // lie past V or hold the target of one of its rows; those columns count
    // as -inf, and the lane holding a target records z_t.
    auto tile_body = [&](int64_t tile, f32x16(&acc)[kTM][kTN], auto mask) {
        constexpr bool MASK = decltype(mask)::value;
        const int el = opaque_lane();
        const int64_t c0 = lane_col(tile, wn, el);
        // stored logits: this lane's rows are row0 + rb0 + k (k below)
        const int rb0 = wm * 64 + 4 * (el >> 5);
        float *lrow0 = STORE ? a.logits_out + (row0 + rb0) * a.ldl + c0 : nullptr;
        // the row stride as a value the compiler cannot hoist: the 32 products
        // k * ldl are then formed per tile on the scalar unit instead of being
        // kept live through the K loop
        int64_t ldl = a.ldl;
        if constexpr (STORE)
            asm volatile("" : "+s"(ldl));
        // Each slot's terms at the running maximum; where some lane of the
        // wave sees a larger value (wave-uniform branch, about ln(tiles) times
        // per row), at the tile's maximum instead, whose value and first
        // column the slot's owner picks up.
        const int half = el >> 5;
        float mr[32];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const float4 m4 = *reinterpret_cast<const float4 *>(&s_mr[w][half * 32 + 4 * q]);
            mr[4 * q] = m4.x;
            mr[4 * q + 1] = m4.y;
            mr[4 * q + 2] = m4.z;
            mr[4 * q + 3] = m4.w;
        }
        float ts[32], th[32], tz[32];
        float own_tm = -INFINITY;
        int own_arg = INT32_MAX;
#pragma unroll
        for (int mb = 0; mb < kTM; ++mb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int k = mb * 16 + v;
                float x[kTN];
#pragma unroll
                for (int nb = 0; nb < kTN; ++nb)
                    x[nb] = acc[mb][nb][v];
                if constexpr (STORE) {
                    // the raw logits of this lane's four columns, one 16-byte
                    // store at the tile's lane address plus k rows
                    const int k = mb * 32 + 8 * (v / 4) + v % 4;
                    float *dst = lrow0 + (int64_t)k * ldl;
                    if constexpr (!MASK) {
                        if (all_rows || row0 + rb0 + k < a.rows)
                            *reinterpret_cast<float4 *>(dst) = make_float4(x[0], x[1], x[2], x[3]);
                    } else if (row0 + rb0 + k < a.rows) {
                        if (c0 + kTN <= V) {
                            *reinterpret_cast<float4 *>(dst) = make_float4(x[0], x[1], x[2], x[3]);
                        } else {
#pragma unroll
                            for (int nb = 0; nb < kTN; ++nb)
                                if (c0 + nb < V)
                                    dst[nb] = x[nb];
                        }
                    }
                }
                if constexpr (MASK) {
                    const int rl = acc_row(wm, mb, v, el);
                    const int64_t d = (int64_t)s_lab[rl] - c0;
#pragma unroll
                    for (int nb = 0; nb < kTN; ++nb) {
                        if (d == nb) {
                            s_zt[rl] = x[nb];
                            s_own[rl] = 1;
                        }
                        if (d == nb || c0 + nb >= V)
                            x[nb] = -INFINITY;
                    }
                }
                const float lm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
                float b = mr[k];
                if (__any(lm > b)) {
                    const float tm = row_max(lm);
                    int cand = INT32_MAX;
#pragma unroll
                    for (int nb = kTN - 1; nb >= 0; --nb)
                        if (x[nb] == tm)
                            cand = (int)(c0 + nb);
                    const int targ = row_min(tm != -INFINITY ? cand : INT32_MAX);
                    if ((el & 31) == k) {
                        own_tm = tm;
                        own_arg = targ;
                    }
                    b = fmaxf(b, tm);
                }
                const float base = fmaxf(b, -FLT_MAX);
                float ls = 0.0f, lh = 0.0f, lz = 0.0f;
#pragma unroll
                for (int nb = 0; nb < kTN; ++nb) {
                    const float e = exp2_hw((x[nb] - base) * c);
                    ls += e;
                    if constexpr (WANT_H)
                        lh = fmaf(e, fminf((base - x[nb]) * inv_t, kBigL), lh);
                    if constexpr (WANT_Z)
                        lz += x[nb] == -INFINITY ? 0.0f : x[nb];
                }
                ts[k] = ls;
                th[k] = lh;
                tz[k] = lz;
            }
        const auto add = [](float p, float q) { return p + q; };
        const float tsum = reduce_scatter32(ts, el, add);
        float hsum = 0.0f, zsum = 0.0f;
        if constexpr (WANT_H)
            hsum = reduce_scatter32(th, el, add);
        if constexpr (WANT_Z)
            zsum = reduce_scatter32(tz, el, add);
        // merge into the owner's state: the tile's terms are at base
        // max(running max, tile max)
        if (own_tm > st.m) {
            const float bo = fmaxf(st.m, -FLT_MAX), bn = fmaxf(own_tm, -FLT_MAX);
            const float fo = exp2_hw((bo - bn) * c);
            if constexpr (WANT_H)
                st.h = fo * fmaf(fminf((bn - bo) * inv_t, kBigL), st.s, st.h) + hsum;
            st.s = st.s * fo + tsum;
            st.m = own_tm;
            st.arg = own_arg;
        } else {
            st.s += tsum;
            if constexpr (WANT_H)
                st.h += hsum;
        }
        if constexpr (WANT_Z)
            st.zs += zsum;
        s_mr[w][el] = st.m;
    };
    auto epi = [&](int64_t tile, f32x16(&acc)[kTM][kTN]) {
        const int64_t cw = tile * kBN + wn * 128;   // this wave's first column
        const bool tail = cw + 128 > V;
        const bool hit = __any(mylab >= cw && mylab < cw + 128);
        if (tail || hit)
            tile_body(tile, acc, Flag<true>{});
        else
            tile_body(tile, acc, Flag<false>{});
    };
    gemm_tiles(sm, a.hidden, a.ldh, a.rows, row0, a.weight, a.ldw, V, a.hidden_dim / kBK, t0, t1,
               epi);

    // The two waves along N hold the two column halves of each row: combine
    // them through LDS (the operand tiles are done).
    struct RowPart {
        float m;
        int arg;
        double s, h, z;
    };
    RowPart *part = reinterpret_cast<RowPart *>(&sm);   // [2][kBM]
    {
        const int ri = lane & 31;
        RowPart p;
        p.m = st.m;
        p.arg = st.arg;
        p.s = (double)st.s;
        p.h = (double)st.h;
        p.z = (double)st.zs;
        part[wn * kBM + acc_row(wm, ri >> 4, ri & 15, lane)] = p;
    }
    __syncthreads();
    const int64_t r = row0 + tid;
    if (tid < kBM && r < a.rows) {
        const RowPart pp[2] = {part[tid], part[kBM + tid]};
        const float M = fmaxf(pp[0].m, pp[1].m);
        const double B = (double)fmaxf(M, -FLT_MAX);
        double S2 = 0.0, H2 = 0.0;
        int am = INT32_MAX;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            if (pp[q].s > 0.0) {
                const double bp = (double)fmaxf(pp[q].m, -FLT_MAX);
                const double f = exp((bp - B) / a.temperature);
                S2 += pp[q].s * f;
                H2 += f * (pp[q].h + (B - bp) / a.temperature * pp[q].s);
            }
            if (pp[q].m == M && M != -INFINITY)
                am = min(am, pp[q].arg);
        }
        cev_vocab_partial out;
        out.m = M;
        out.zt = s_zt[tid];
        out.arg = am == INT32_MAX ? INT64_MAX : (int64_t)am;
        out.s = S2;
        out.h = H2;
        out.zs = pp[0].z + pp[1].z;
        out.flags = (s_lab[tid] >= 0 ? 1 : 0) | (s_own[tid] ? 2 : 0);
        out.pad = 0;
        a.partials[sp * a.rows + r] = out;
    }
}

// ----------------------------------------------------------------- backward
// dlogits tile by tile: (g/T) p_j - (g/T) eps/V, the target -(g/T)(q - eps +
// eps/V); p_j = 2^((z_j - m_z) c - log2 d) from the saved record with |g/T|
// folded into the exponent, the sign of g applied to the bits, bf16 by RNE.
// Columns [V, ldd) of the dlogits rows are written as zeros.
struct __align__(16) DlRow {
    float mz, kexp, ev, tv;
};

// The constants of row r (label and sign bit of g through lab, sgn); rows
// that are masked, ignored, past `rows` or not read by the forward give
// kexp = inf, so every entry of theirs comes out as 0.
__device__ __forceinline__ DlRow dl_row(const LceArgs &a, int64_t r, int &lab, unsigned &sgn)
{
    const int64_t V = a.vocab;
    lab = -1;
    sgn = 0u;
    DlRow rc{0.0f, INFINITY, 0.0f, 0.0f};
    if (r < a.rows) {
        const int64_t t = a.labels[r];
        const bool masked = a.row_mask && a.row_mask[r] == 0;
        const cev_saved sv = a.saved[r];
        if (!masked && t != a.ignore_index && t >= 0 && t < V && (sv.flags & 1)) {
            const float gp = a.g[r] * a.inv_t;
            const float ag = fabsf(gp);
            const float eps = (float)a.label_smoothing;
            const float epv = (float)(a.label_smoothing / (double)V);
            lab = (int)t;
            rc.mz = sv.m_z;
            rc.kexp = sv.log2_d - __log2f(ag);
            rc.ev = ag * epv;
            rc.tv = -(ag * ((sv.q - eps) + epv));
            sgn = __float_as_uint(gp) & 0x80000000u;
        }
    }
    return rc;
}

// SMOOTH: label smoothing is on (eps/V comes off every column; without it
// that term is zero and skipped).
template <bool SMOOTH>
__global__ __launch_bounds__(kLT) void k_lce_dl(LceArgs a)
{
    __shared__ GemmSmem sm;
    // per row: {m_z, kexp, eps/V term, sign bit of g} and {label, target value}
    __shared__ float4 s_rc[kBM];
    __shared__ int2 s_lt[kBM];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 1, wn = w & 1;
    const int64_t S = a.splits;
    const int64_t vb = xcd_order(blockIdx.x, gridDim.x);
    const int64_t rb = vb / S, sp = vb % S;
    const int64_t row0 = rb * kBM;
    const int64_t V = a.vocab, ldd = a.ldd;
    const int64_t ntiles = (V + kBN - 1) / kBN;
    const int64_t t0 = ntiles * sp / S, t1 = ntiles * (sp + 1) / S;

    if (tid < kBM) {
        int lab;
        unsigned sgn;
        const DlRow rc = dl_row(a, row0 + tid, lab, sgn);
        s_rc[tid] = make_float4(rc.mz, rc.kexp, rc.ev, __uint_as_float(sgn));
        s_lt[tid] = make_int2(lab, (int)__float_as_uint(rc.tv));
    }
    __syncthreads();
    const float c = a.c;
    // dl_rows is a multiple of 64: a wave's 64 rows are all below it or none is
    const bool wave_rows = row0 + wm * 64 < a.dl_rows;

    // the label of row wm * 64 + lane: which tiles hold a target for this wave
    const int mylab = s_lt[wm * 64 + lane].x;

    // Each lane writes its four adjacent columns of a row as one 8-byte store
    // (ldd is a multiple of 64, so a group of four is wholly inside or past it).
    // The lane's 32 rows are wm * 64 + 4 * half + k for k = 32 mb + 8 (v / 4) +
    // v % 4, so one 64-bit address per tile plus a wave-uniform k * ldd per row.
    // MASK (wave-uniform, rare): some of this wave's columns lie past V or
    // hold the target of one of its rows.
    auto tile_body = [&](int64_t tile, f32x16(&acc)[kTM][kTN], auto mask) {
        constexpr bool MASK = decltype(mask)::value;
        const int el = opaque_lane();
        const int64_t c0 = lane_col(tile, wn, el);
        if (c0 >= ldd)
            return;
        const int half = el >> 5;
        const int rb0 = wm * 64 + 4 * half;
        unsigned short *lbase = a.dlogits + (row0 + rb0) * ldd + c0;
#pragma unroll
        for (int mb = 0; mb < kTM; ++mb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int k = mb * 32 + 8 * (v / 4) + v % 4;
                const float4 rc = s_rc[rb0 + k];
                const unsigned sgn = __float_as_uint(rc.w);
                float o[kTN];
#pragma unroll
                for (int nb = 0; nb < kTN; ++nb) {
                    float e = exp2_hw(fmaf(acc[mb][nb][v] - rc.x, c, -rc.y));
                    if constexpr (SMOOTH)
                        e -= rc.z;
                    if constexpr (MASK) {
                        const int64_t col = c0 + nb;
                        const int2 lt = s_lt[rb0 + k];
                        if (col == lt.x)
                            e = __int_as_float(lt.y);
                        if (col >= V)
                            e = 0.0f;
                    }
                    o[nb] = __uint_as_float(__float_as_uint(e) ^ sgn);
                }
                uint2 pk;
                pk.x = pack_bf16x2(o[0], o[1]);
                pk.y = pack_bf16x2(o[2], o[3]);
                *reinterpret_cast<uint2 *>(lbase + (int64_t)k * ldd) = pk;
            }
    };
    auto epi = [&](int64_t tile, f32x16(&acc)[kTM][kTN]) {
        if (!wave_rows)   // rows at or past dl_rows: nothing to write
            return;
        const int64_t cw = tile * kBN + wn * 128;   // this wave's first column
        const bool tail = cw + 128 > V;
        const bool hit = __any(mylab >= cw && mylab < cw + 128);
        if (tail || hit)
            tile_body(tile, acc, Flag<true>{});
        else
            tile_body(tile, acc, Flag<false>{});
    };
    gemm_tiles(sm, a.hidden, a.ldh, a.rows, row0, a.weight, a.ldw, V, a.hidden_dim / kBK, t0, t1,
               epi);
}

// dlogits from logits the forward stored (fp32, [rows, ldl]): the per-element
// steps of k_lce_dl's epilogue on the same fp32 values, so the dlogits are
// bit-identical to the recomputing path.  One workgroup per row and chunk of
// kDlsCols columns (4 per thread and step, 16-byte loads, 8-byte stores);
// rows in [rows, dl_rows) and columns in [vocab, ldd) are written as zeros.
constexpr int kDlsT = 256, kDlsU = 4, kDlsCols = kDlsT * 4 * kDlsU;

__global__ __launch_bounds__(kDlsT) void k_lce_dl_stored(LceArgs a, int64_t chunks)
{
    const int64_t r = blockIdx.x / chunks, ch = blockIdx.x % chunks;
    const int64_t V = a.vocab, ldd = a.ldd;
    // The saved record's valid flag first, then every load of the chunk:
    // only rows the forward read have logits worth loading (masked, ignored
    // and padding rows come out as zeros), and the row's other constants
    // arrive while those loads are in flight.
    const bool have = r < a.rows && (a.saved[r].flags & 1);
    const float *lrow = a.logits_in + (have ? r : 0) * a.ldl;
    float z[kDlsU][4];
#pragma unroll
    for (int u = 0; u < kDlsU; ++u) {
        const int64_t col = ch * kDlsCols + (int64_t)(u * kDlsT + threadIdx.x) * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            z[u][i] = 0.0f;
        if (have && col < ldd) {
            if (col + 4 <= V) {
                const float4 q = *reinterpret_cast<const float4 *>(lrow + col);
                z[u][0] = q.x;
                z[u][1] = q.y;
                z[u][2] = q.z;
                z[u][3] = q.w;
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (col + i < V)
                        z[u][i] = lrow[col + i];
            }
        }
    }
    int lab;
    unsigned sgn;
    const DlRow rc = dl_row(a, r, lab, sgn);
    const float c = a.c;
    unsigned short *drow = a.dlogits + r * ldd;
#pragma unroll
    for (int u = 0; u < kDlsU; ++u) {
        const int64_t col = ch * kDlsCols + (int64_t)(u * kDlsT + threadIdx.x) * 4;
        if (col >= ldd)
            continue;
        float o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float e = exp2_hw(fmaf(z[u][i] - rc.mz, c, -rc.kexp)) - rc.ev;
            if (col + i == lab)
                e = rc.tv;
            if (col + i >= V)
                e = 0.0f;
            o[i] = __uint_as_float(__float_as_uint(e) ^ sgn);
        }
        uint2 pk;
        pk.x = pack_bf16x2(o[0], o[1]);
        pk.y = pack_bf16x2(o[2], o[3]);
        *reinterpret_cast<uint2 *>(drow + col) = pk;
    }
}

// C[M, N] (fp32, row stride ldc) = sum_k A[m][k] B[n][k], A and B
// K-contiguous, N a multiple of 4; one 256 x 256 tile per workgroup (M tiles
// fastest).  Split along K: workgroup split s covers K steps
// [nk s / splits, nk (s + 1) / splits) of 64 and writes its partial product to
// C + s * cstride (reduced afterwards in split order).  vec4: C and ldc allow
// 16-byte stores.  AKN: A is stored as ka K rows of contiguous M values
// (A[k * lda + m], am of them readable per row); BKN: B likewise
// (B[k * ldb + n], kb rows), and each lane then holds one column of each
// 32-column block (4-byte stores, 32 adjacent columns per half-wave).
template <bool AKN, bool BKN>
__global__ __launch_bounds__(kLT) void k_lce_gemm(const unsigned short *XA, int64_t lda,
                                                 int64_t M, const unsigned short *XB,
                                                 int64_t ldb, int64_t N, int64_t nk,
                                                 int64_t splits, float *C, int64_t ldc,
                                                 int64_t cstride, int vec4, int64_t ka,
                                                 int64_t am, int64_t kb)
{
    __shared__ GemmSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 1, wn = w & 1;
    const int64_t mt = (M + kBM - 1) / kBM;
    const int64_t tiles = mt * ((N + kBN - 1) / kBN);
    const int64_t sp = blockIdx.x / tiles, t = blockIdx.x % tiles;
    const int64_t row0 = (t % mt) * kBM, nt = t / mt;
    const int64_t k0 = nk * sp / splits, k1 = nk * (sp + 1) / splits;
    float *Cs = C + sp * cstride;
    f32x16 acc[kTM][kTN];
    const unsigned short *A0 = AKN ? XA + k0 * kBK * lda : XA + k0 * kBK;
    const unsigned short *B0 = BKN ? XB + k0 * kBK * ldb : XB + k0 * kBK;
    gemm_one_tile<AKN, BKN>(sm, A0, lda, AKN ? ka - k0 * kBK : M, row0, B0, ldb,
                            BKN ? kb - k0 * kBK : N, nt * kBN, k1 - k0, acc, am, N);
    if constexpr (BKN) {
        const int64_t cb = nt * kBN + wn * 128 + (lane & 31);
#pragma unroll
        for (int mb = 0; mb < kTM; ++mb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t r = row0 + acc_row(wm, mb, v, lane);
                if (r >= M)
                    continue;
                float *dst = Cs + r * ldc;
#pragma unroll
                for (int nb = 0; nb < kTN; ++nb)
                    if (cb + 32 * nb < N)
                        dst[cb + 32 * nb] = acc[mb][nb][v];
            }
        return;
    }
    const int64_t c0 = lane_col(nt, wn, lane);
    if (c0 >= N)
        return;
#pragma unroll
    for (int mb = 0; mb < kTM; ++mb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int64_t r = row0 + acc_row(wm, mb, v, lane);
            if (r >= M)
                continue;
            float *dst = Cs + r * ldc + c0;
            if (vec4) {
                *reinterpret_cast<float4 *>(dst) =
                    make_float4(acc[mb][0][v], acc[mb][1][v], acc[mb][2][v], acc[mb][3][v]);
            } else {
#pragma unroll
                for (int nb = 0; nb < kTN; ++nb)
                    dst[nb] = acc[mb][nb][v];
            }
        }
}

// out[r][c] = sum over s in order of P[s][r][c] (P rows of N floats, N a
// multiple of 4); four columns per thread.
__global__ __launch_bounds__(256) void k_splitk_reduce(const float *P, int64_t splits,
                                                      int64_t M, int64_t N, float *out,
                                                      int64_t ldo)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t nq = N / 4;
    if (i >= M * nq)
        return;
    const int64_t r = i / nq, c = (i % nq) * 4;
    float4 acc = *reinterpret_cast<const float4 *>(P + r * N + c);
    for (int64_t s = 1; s < splits; ++s) {
        const float4 p = *reinterpret_cast<const float4 *>(P + (s * M + r) * N + c);
        acc.x += p.x;
        acc.y += p.y;
        acc.z += p.z;
        acc.w += p.w;
    }
    float *dst = out + r * ldo + c;
    dst[0] = acc.x;
    dst[1] = acc.y;
    dst[2] = acc.z;
    dst[3] = acc.w;
}

int64_t round64(int64_t x) { return (x + 63) / 64 * 64; }
size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// K splits for a product of `tiles` output tiles with nk K steps: the fewest
// splits that minimise the number of full-chip rounds per split (a grid of
// tiles x S workgroups on 256 compute units, one workgroup each), keeping at
// least 16 K steps per split and S partial products within max_by_room.
int64_t gemm_splits(int64_t tiles, int64_t nk, size_t max_by_room)
{
    constexpr int64_t kCUs = 256;
    int64_t best = 1;
    double best_t = (double)((tiles + kCUs - 1) / kCUs);
    for (int64_t s = 2; s <= 16 && (size_t)s <= max_by_room && nk / s >= 16; ++s) {
        const double t = (double)((tiles * s + kCUs - 1) / kCUs) / (double)s;
        if (t < best_t - 1e-9) {
            best = s;
            best_t = t;
        }
    }
    return best;
}

} // namespace

int64_t lce_splits(int64_t rows, int64_t vocab)
{
    // A multiple of 8 vocab splits, enough for 256 workgroups (one per CU).
    const int64_t ntiles = (vocab + kBN - 1) / kBN;
    const int64_t nrb = (rows + kBM - 1) / kBM;
    int64_t s = 8;
    while (s * nrb < 256 && s < 64)
        s *= 2;
    return s <= ntiles ? s : ntiles;
}

int64_t lce_dl_stride(int64_t vocab) { return round64(vocab); }

template <bool STORE>
void launch_lce_fwd_t(const LceArgs &a, bool want_h, bool want_z, hipStream_t s)
{
    const int64_t nrb = (a.rows + kBM - 1) / kBM;
    dim3 grid((unsigned)(nrb * a.splits)), block(kLT);
    if (want_h && want_z)
        hipLaunchKernelGGL((k_lce_fwd<true, true, STORE>), grid, block, 0, s, a);
    else if (want_h)
        hipLaunchKernelGGL((k_lce_fwd<true, false, STORE>), grid, block, 0, s, a);
    else if (want_z)
        hipLaunchKernelGGL((k_lce_fwd<false, true, STORE>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((k_lce_fwd<false, false, STORE>), grid, block, 0, s, a);
}

hipError_t launch_lce_forward(const LceArgs &a, bool want_h, bool want_z, hipStream_t s)
{
    if (a.logits_out)
        launch_lce_fwd_t<true>(a, want_h, want_z, s);
    else
        launch_lce_fwd_t<false>(a, want_h, want_z, s);
    return hipGetLastError();
}

// Backward workspace: dlogits [round64(R), round64(V)] (zero past row R and
// column V) and room for up to kMaxSplitK fp32 partial products of dhidden.
constexpr int64_t kMaxSplitK = 8;

size_t lce_backward_workspace(int64_t rows, int64_t hidden_dim, int64_t vocab)
{
    const size_t vp = (size_t)round64(vocab), rp = (size_t)round64(rows);
    return align256(rp * vp * 2) + align256((size_t)kMaxSplitK * rows * hidden_dim * 4);
}

hipError_t launch_lce_backward(const LceArgs &a, void *workspace, float *dhidden, int64_t ldo,
                               float *dweight, int64_t ldw_out, hipStream_t s)
{
    const int64_t R = a.rows, H = a.hidden_dim, V = a.vocab;
    const int64_t vp = round64(V), rp = round64(R);
    char *ws = static_cast<char *>(workspace);
    unsigned short *dl = reinterpret_cast<unsigned short *>(ws);
    ws += align256((size_t)rp * vp * 2);
    float *part = reinterpret_cast<float *>(ws);

    LceArgs b = a;
    b.dlogits = dl;
    b.ldd = vp;
    b.dl_rows = rp;
    const int64_t nrb = (R + kBM - 1) / kBM;
    if (a.logits_in) {
        const int64_t chunks = (vp + kDlsCols - 1) / kDlsCols;
        hipLaunchKernelGGL(k_lce_dl_stored, dim3((unsigned)(rp * chunks)), dim3(kDlsT), 0, s, b,
                           chunks);
    } else {
        if (a.label_smoothing != 0.0)
            hipLaunchKernelGGL(k_lce_dl<true>, dim3((unsigned)(nrb * b.splits)), dim3(kLT), 0, s,
                               b);
        else
            hipLaunchKernelGGL(k_lce_dl<false>, dim3((unsigned)(nrb * b.splits)), dim3(kLT), 0,
                               s, b);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    // dhidden[R, H] = dlogits[R, V] x head[V, H]: dlogits runs along the
    // vocab, the head is read as stored (its K rows past V re-read row V - 1
    // against zero dlogits columns).  Few output tiles and a long contraction:
    // split along K so the grid fills the chip.
    const int64_t tiles = nrb * ((H + kBN - 1) / kBN);
    const int64_t S = gemm_splits(tiles, vp / kBK, (size_t)kMaxSplitK);
    if (S > 1) {
        hipLaunchKernelGGL((k_lce_gemm<false, true>), dim3((unsigned)(tiles * S)), dim3(kLT), 0,
                           s, dl, vp, R, a.weight, a.ldw, H, vp / kBK, S, part, H, R * H, 0,
                           (int64_t)0, (int64_t)0, V);
        const int64_t n = R * (H / 4);
        hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                           part, S, R, H, dhidden, ldo);
    } else {
        hipLaunchKernelGGL((k_lce_gemm<false, true>), dim3((unsigned)tiles), dim3(kLT), 0, s, dl,
                           vp, R, a.weight, a.ldw, H, vp / kBK, (int64_t)1, dhidden, ldo,
                           (int64_t)0, 0, (int64_t)0, (int64_t)0, V);
    }
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    // dhead[V, H] = dlogits^T x hidden, both read as stored: K runs over the
    // rows (dlogits' rows past R are zero, hidden's re-read row R - 1).
    if (dweight) {
        const int64_t wtiles = ((V + kBM - 1) / kBM) * ((H + kBN - 1) / kBN);
        hipLaunchKernelGGL((k_lce_gemm<true, true>), dim3((unsigned)wtiles), dim3(kLT), 0, s, dl,
                           vp, V, a.hidden, a.ldh, H, rp / kBK, (int64_t)1, dweight, ldw_out,
                           (int64_t)0, 0, rp, vp, R);
        e = hipGetLastError();
    }
    return e;
}

} // namespace cev
