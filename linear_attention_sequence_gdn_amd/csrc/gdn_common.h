// gdn_common.h -- device helpers shared by the gfx950 GDN kernels.
//
// Internal header of the HIP library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;     // head dim (d_k = d_v)
constexpr int kChunk = 64;  // tokens per chunk of the chunked prefill
constexpr int kMaxDecodeTokens = 4;  // tokens per sequence in one multi-token decode step

// ---- number formats --------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16 bits, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ uint32_t f32_to_bf16(float f)
{
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// two fp32 -> bf16 pair (lo in bits 15:0), one conversion instruction
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// ---- scalar activations -----------------------------------------------------

// 1 / (1 + e^-x) and x / (1 + e^-x) with the hardware reciprocal (about 1 ulp)
__device__ __forceinline__ float sigmoid_f(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }
__device__ __forceinline__ float silu_f(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }
// softplus(x) = max(x, 0) + log1p(exp(-|x|))
__device__ __forceinline__ float softplus_f(float x) { return fmaxf(x, 0.0f) + log1pf(__expf(-fabsf(x))); }

constexpr float kLog2e = 1.4426950408889634f;

// ---- wave reductions (wave64) ----------------------------------------------

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// ---- matrix cores ----------------------------------------------------------
// D(16x16, fp32) += A(16x32, fp16) * B(32x16, fp16).
// Lane l holds A row (l % 16) and B column (l % 16); its eight operand
// elements cover contraction indices kappa(l / 16, 0..7) of the 32-wide
// block, with the same assignment for A and B.  The kernels use
//   kappa(q, i) = 4q + i        for i < 4
//               = 16 + 4q + i-4 for i >= 4,
// which lets a lane build a B operand from the fp32 accumulator rows it
// already owns (accumulator lane l holds rows 4*(l/16)+0..3 of column l%16).
__device__ __forceinline__ f32x4 mfma16(half8 a, half8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ half8 pack_h8(f32x4 lo, f32x4 hi)
{
    half8 r;
    r[0] = (_Float16)lo[0]; r[1] = (_Float16)lo[1]; r[2] = (_Float16)lo[2]; r[3] = (_Float16)lo[3];
    r[4] = (_Float16)hi[0]; r[5] = (_Float16)hi[1]; r[6] = (_Float16)hi[2]; r[7] = (_Float16)hi[3];
    return r;
}

}  // namespace gdn
