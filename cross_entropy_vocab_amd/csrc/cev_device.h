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
__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1)
        v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ double wave_sum(double v)
{
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1)
        v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ int64_t wave_min(int64_t v)
{
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
        int64_t w = __shfl_xor(v, o);
        v = w < v ? w : v;
    }
    return v;
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
