// cev_device.h -- device-side building blocks shared by the gfx950 kernels:
// 16-byte loads/stores, bf16 widening and rounding, exp2, wave and block
// reductions.  Internal to libcevocab.so.
#pragma once

#include <hip/hip_runtime.h>
#include <float.h>
#include <stdint.h>

#include "cevocab.h"

namespace cev {

constexpr int kWave = 64;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Elements per 16-byte vector and bytes per element for each storage dtype.
template <int DT> struct Elem;
template <> struct Elem<CEV_F32> {
    static constexpr int kVE = 4;
    static constexpr int kSize = 4;
};
template <> struct Elem<CEV_BF16> {
    static constexpr int kVE = 8;
    static constexpr int kSize = 2;
};

// Streaming 16-byte load: each logit is read once per pass, so keep it out of
// the caches' way (measured on MI355X: ~7.0 TB/s for nontemporal 16-byte reads
// against ~5.5-6.0 TB/s for plain ones).
__device__ __forceinline__ u32x4 load16_stream(const u32x4 *p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void store16_stream(u32x4 v, u32x4 *p) { __builtin_nontemporal_store(v, p); }
// 16-byte store, nontemporal (NT) or with the default cache policy.  A plain
// store lets the L2 gather a wave's lines before they go out; in a mixed
// read-plus-write stream that measured faster than nontemporal stores.
template <bool NT> __device__ __forceinline__ void store16(u32x4 v, u32x4 *p)
{
    if constexpr (NT)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

// Workgroup-uniform read of a kernel input that no thread writes during the
// launch, through the scalar cache: the pointer is cast to the constant
// address space, so the compiler emits a scalar load even in kernels that
// also store to memory (where it would otherwise fall back to a vector load,
// whose latency behind a streaming sweep is microseconds).
template <class T> __device__ __forceinline__ T load_uniform(const T *p)
{
    return *(const __attribute__((address_space(4))) T *)p;
}

// Row r's mask byte, read as the aligned 4-byte word that holds it so that the
// load can be a scalar one.  The word lies in the same page as the byte, so
// the wider read cannot fault; the other three bytes are ignored.
__device__ __forceinline__ unsigned mask_byte(const uint8_t *m, int64_t r)
{
    const uintptr_t p = (uintptr_t)(m + r);
    const unsigned w = load_uniform(reinterpret_cast<const unsigned *>(p & ~(uintptr_t)3));
    return (w >> (8u * (unsigned)(p & 3u))) & 0xffu;
}

// bf16 -> fp32 is exact: the bf16 bits are the upper half of the fp32 word.
__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// Widen one 16-byte vector into VE floats, in column order.
template <int DT> __device__ __forceinline__ void unpack16(const u32x4 &w, float *out)
{
    if constexpr (DT == CEV_F32) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            out[i] = __uint_as_float(w[i]);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = bf16_lo(w[i]);
            out[2 * i + 1] = bf16_hi(w[i]);
        }
    }
}

// One element at column col of a row that starts at rowp.
template <int DT> __device__ __forceinline__ float load_elem(const char *rowp, int64_t col)
{
    if constexpr (DT == CEV_F32)
        return __builtin_nontemporal_load(reinterpret_cast<const float *>(rowp) + col);
    else
        return __uint_as_float((unsigned)__builtin_nontemporal_load(
                                   reinterpret_cast<const unsigned short *>(rowp) + col)
                               << 16);
}

// Two fp32 values rounded to bf16 (round to nearest even; v_cvt_pk_bf16_f32 on
// gfx950), packed low = a, high = b.
__device__ __forceinline__ unsigned pack_bf16x2(float a, float b)
{
    f32x2 f = {a, b};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ unsigned short to_bf16(float a) { return (unsigned short)(pack_bf16x2(a, 0.0f) & 0xffffu); }

// Hardware 2^x (v_exp_f32): -inf -> 0, very negative -> 0 or a subnormal.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- reductions
// Wave-wide reductions without the LDS crossbar (ds_bpermute costs an LDS
// round trip per step).  Six steps, each combining a lane with a partner that
// holds the same number of values: DPP inside each 16-lane row (quad_perm
// [1,0,3,2], quad_perm [2,3,0,1], then row_half_mirror, lane i of 8 reading
// 7 - i, and row_mirror, lane i of 16 reading 15 - i), then gfx950's
// v_permlane16_swap (row 2k with row 2k + 1) and v_permlane32_swap (the two
// half-waves).  Both lanes of a pair form op(a, b) of the same two values with
// a commutative op, so every lane ends with the same bits.
constexpr int kDppQuad1 = 0xB1, kDppQuad2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

template <int CTRL> __device__ __forceinline__ unsigned dpp_u32(unsigned x)
{
    return (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}

// A value of 4 or 8 bytes as 32-bit words, for the cross-lane moves.
template <class T> struct Words {
    static constexpr int N = sizeof(T) / 4;
    unsigned w[N];
};
template <class T> __device__ __forceinline__ Words<T> to_words(T x)
{
    Words<T> r;
    __builtin_memcpy(r.w, &x, sizeof(T));
    return r;
}
template <class T> __device__ __forceinline__ T from_words(const Words<T> &r)
{
    T x;
    __builtin_memcpy(&x, r.w, sizeof(T));
    return x;
}

template <int CTRL, class T> __device__ __forceinline__ T dpp_move(T x)
{
    Words<T> r = to_words(x);
#pragma unroll
    for (int i = 0; i < Words<T>::N; ++i)
        r.w[i] = dpp_u32<CTRL>(r.w[i]);
    return from_words<T>(r);
}

// op over the value pair that v_permlane{16,32}_swap hands each lane: the even
// row (lower half-wave) value first, the odd row (upper half) value second.
template <bool HALF, class T, class Op> __device__ __forceinline__ T swap_combine(T x, Op op)
{
    Words<T> a = to_words(x), b = a;
#pragma unroll
    for (int i = 0; i < Words<T>::N; ++i) {
        const auto sw = HALF ? __builtin_amdgcn_permlane32_swap(a.w[i], a.w[i], false, false)
                             : __builtin_amdgcn_permlane16_swap(a.w[i], a.w[i], false, false);
        a.w[i] = sw[0];
        b.w[i] = sw[1];
    }
    return op(from_words<T>(a), from_words<T>(b));
}

template <class T, class Op> __device__ __forceinline__ T wave_reduce(T x, Op op)
{
    x = op(x, dpp_move<kDppQuad1>(x));
    x = op(x, dpp_move<kDppQuad2>(x));
    x = op(x, dpp_move<kDppHalfMirror>(x));
    x = op(x, dpp_move<kDppMirror>(x));
    x = swap_combine<false>(x, op);
    return swap_combine<true>(x, op);
}

__device__ __forceinline__ float wave_max(float v)
{
    return wave_reduce(v, [](float p, float q) { return fmaxf(p, q); });
}

__device__ __forceinline__ double wave_sum(double v)
{
    return wave_reduce(v, [](double p, double q) { return p + q; });
}

__device__ __forceinline__ int64_t wave_min(int64_t v)
{
    return wave_reduce(v, [](int64_t p, int64_t q) { return q < p ? q : p; });
}

// A lane's value as a wave-uniform scalar (v_readlane).
__device__ __forceinline__ int64_t lane_value(int64_t v, int l)
{
    const uint64_t u = (uint64_t)v;
    const unsigned lo = __builtin_amdgcn_readlane((unsigned)u, l);
    const unsigned hi = __builtin_amdgcn_readlane((unsigned)(u >> 32), l);
    return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ float lane_value(float v, int l)
{
    return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), l));
}
__device__ __forceinline__ double lane_value(double v, int l)
{
    return __builtin_bit_cast(double, lane_value(__builtin_bit_cast(int64_t, v), l));
}

// Block-wide reductions; every thread gets the result.  `sh` is LDS scratch of
// BLOCK / 64 entries that the caller does not touch in between.  The combine
// order is fixed, so results are deterministic.
template <int BLOCK> __device__ __forceinline__ float block_max(float v, float *sh)
{
    constexpr int W = BLOCK / kWave;
    v = wave_max(v);
    if constexpr (W == 1)
        return v;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    if (lane == 0)
        sh[wave] = v;
    __syncthreads();
    float r = sh[0];
#pragma unroll
    for (int i = 1; i < W; ++i)
        r = fmaxf(r, sh[i]);
    __syncthreads();
    return r;
}

template <int BLOCK> __device__ __forceinline__ double block_sum(double v, double *sh)
{
    constexpr int W = BLOCK / kWave;
    v = wave_sum(v);
    if constexpr (W == 1)
        return v;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    if (lane == 0)
        sh[wave] = v;
    __syncthreads();
    double r = sh[0];
#pragma unroll
    for (int i = 1; i < W; ++i)
        r += sh[i];
    __syncthreads();
    return r;
}

// N maxima over the workgroup in one exchange (`sh`: N * BLOCK / 64 entries).
template <int BLOCK, int N> __device__ __forceinline__ void block_max_n(float (&v)[N], float *sh)
{
    constexpr int W = BLOCK / kWave;
#pragma unroll
    for (int i = 0; i < N; ++i)
        v[i] = wave_max(v[i]);
    if constexpr (W == 1)
        return;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    if (lane == 0) {
#pragma unroll
        for (int i = 0; i < N; ++i)
            sh[i * W + wave] = v[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < N; ++i) {
        float r = sh[i * W];
#pragma unroll
        for (int w = 1; w < W; ++w)
            r = fmaxf(r, sh[i * W + w]);
        v[i] = r;
    }
    __syncthreads();
}

// N sums over the workgroup in one exchange (`sh`: N * BLOCK / 64 entries);
// each is the same fixed-order sum block_sum forms.
template <int BLOCK, int N> __device__ __forceinline__ void block_sum_n(double (&v)[N], double *sh)
{
    constexpr int W = BLOCK / kWave;
#pragma unroll
    for (int i = 0; i < N; ++i)
        v[i] = wave_sum(v[i]);
    if constexpr (W == 1)
        return;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    if (lane == 0) {
#pragma unroll
        for (int i = 0; i < N; ++i)
            sh[i * W + wave] = v[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < N; ++i) {
        double r = sh[i * W];
#pragma unroll
        for (int w = 1; w < W; ++w)
            r += sh[i * W + w];
        v[i] = r;
    }
    __syncthreads();
}

template <int BLOCK> __device__ __forceinline__ int64_t block_min(int64_t v, int64_t *sh)
{
    constexpr int W = BLOCK / kWave;
    v = wave_min(v);
    if constexpr (W == 1)
        return v;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    if (lane == 0)
        sh[wave] = v;
    __syncthreads();
    int64_t r = sh[0];
#pragma unroll
    for (int i = 1; i < W; ++i)
        r = sh[i] < r ? sh[i] : r;
    __syncthreads();
    return r;
}

// ---------------------------------------------------------------- fp64 math
// softplus(u) = log(1 + e^u) = max(u, 0) + log1p(e^{-|u|}); 0 at u = -inf.
__device__ __forceinline__ double softplus64(double u)
{
    if (u == -INFINITY)
        return 0.0;
    return fmax(u, 0.0) + log1p(exp(-fabs(u)));
}

// sigmoid(u) = 1 / (1 + e^{-u}), as e^u / (1 + e^u) for u < 0.
__device__ __forceinline__ double sigmoid64(double u)
{
    if (u < 0.0) {
        double e = exp(u);
        return e / (1.0 + e);
    }
    return 1.0 / (1.0 + exp(-u));
}

} // namespace cev
