// Register-resident epilogue functors for the fused linear layer.
//
// Each functor maps one fp32 GEMM result y = (X W^T)[m,n] + b[n] to the
// output value while it is still in registers, so the raw GEMM output never
// reaches HBM.  All math is binary32.
//
//   tail (a)  GELU(clamp(y * s, lo, hi))     page "Kimi-K2.6 l2_p53",
//             problem statement (scale, Hardtanh, GELU after the GEMM)
//   tail (c)  (y * sigmoid(y)) * s           page "Kimi-K2.6 l2_p59",
//             problem analysis (swish then scaling)
//   tail (b)  pooled windows go through gelu() then a scale and a max; the
//             pooling and the max are cross-lane steps done in the GEMM
//             kernel itself (page "Kimi-K2.6 l2_p98", steps 2-5 of its
//             reading of the reference model)
//
// GELU is the exact form x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2)); erff and
// expf are the ROCm device-library functions (correctly rounded to a few
// ulp), not fast approximations.
#pragma once

#include <hip/hip_runtime.h>

namespace lin_epi {

__device__ __forceinline__ float gelu_erf(float x)
{
    return 0.5f * x * (1.0f + erff(x * 0.70710678118654752440f));
}

struct TailParams {
    float scale;
    float lo;
    float hi;
};

// kind 0: the linear layer alone
struct TailNone {
    __device__ __forceinline__ static float apply(float y, const TailParams &) { return y; }
};

// kind 1: scale -> Hardtanh (inclusive clamp) -> GELU
struct TailScaleHardtanhGelu {
    __device__ __forceinline__ static float apply(float y, const TailParams &p)
    {
        float t = y * p.scale;
        t = fminf(fmaxf(t, p.lo), p.hi);
        return gelu_erf(t);
    }
};

// kind 3: swish -> scale.  For very negative y, expf(-y) overflows to +inf
// and the sigmoid becomes exactly 0, so the result is -0, never NaN.
struct TailSwishScale {
    __device__ __forceinline__ static float apply(float y, const TailParams &p)
    {
        const float sig = 1.0f / (1.0f + expf(-y));
        return (y * sig) * p.scale;
    }
};

}  // namespace lin_epi
