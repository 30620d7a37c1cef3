// Device helpers shared by the KDA kernels: bf16 conversion, the base-2
// exponential, the logistic function, state loads/stores and the chain's
// token segment.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_internal.h"

namespace kda {

constexpr float kLog2eF = 1.44269504088896341f;  // 1 / ln 2

__device__ __forceinline__ float bf16_to_f32(uint16_t bits)
{
    return __uint_as_float(static_cast<uint32_t>(bits) << 16);
}

// fp32 -> bf16 with round to nearest, ties to even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// 2^x on the hardware exponential unit (v_exp_f32).
__device__ __forceinline__ float exp2_f32(float x) { return __builtin_amdgcn_exp2f(x); }

// Logistic 1 / (1 + e^-x) = 1 / (1 + 2^(-x log2 e)): one exp2 and one
// reciprocal.  Large |x| saturates cleanly to 0 or 1 (2^+inf = inf, 1/inf = 0).
__device__ __forceinline__ float sigmoid_f32(float x)
{
    return __builtin_amdgcn_rcpf(1.0f + exp2_f32(-x * kLog2eF));
}

template <int KIND>
__device__ __forceinline__ float load_state(const void *base, int64_t idx)
{
    if constexpr (KIND == kStateBf16)
        return bf16_to_f32(static_cast<const uint16_t *>(base)[idx]);
    else if constexpr (KIND == kStateFp32)
        return static_cast<const float *>(base)[idx];
    else
        return 0.0f;
}

template <int KIND>
__device__ __forceinline__ void store_state(void *base, int64_t idx, float value)
{
    if constexpr (KIND == kStateBf16)
        static_cast<uint16_t *>(base)[idx] = f32_to_bf16_rne(value);
    else if constexpr (KIND == kStateFp32)
        static_cast<float *>(base)[idx] = value;
}

// Token range [*begin, *end) of sequence n and its batch row.  Packed
// segments are clamped into [0, T], so malformed offsets can never move an
// access outside the tensors.
__device__ __forceinline__ void chain_segment(const FwdParams &p, int64_t n, int64_t *begin,
                                              int64_t *end, int64_t *row)
{
    if (p.cu_seqlens) {
        int64_t lo = p.cu_seqlens[n], hi = p.cu_seqlens[n + 1];
        lo = lo < 0 ? 0 : (lo > p.T ? p.T : lo);
        hi = hi < lo ? lo : (hi > p.T ? p.T : hi);
        *begin = lo;
        *end = hi;
        *row = 0;
    } else {
        *begin = 0;
        *end = p.T;
        *row = n;
    }
}

}  // namespace kda
