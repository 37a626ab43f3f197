// Software 2^x on the FMA units, FlashAttention-4's relief for the
// exponential unit ("Attention Is the Bottleneck", FlashAttention-4 section):
// x = n + f with n = rint(x) and |f| <= 1/2 (Cody and Waite's range
// reduction), 2^f by a degree-4 polynomial in Horner form, then 2^n by
// v_ldexp_f32.  The coefficients minimise the largest relative error on
// [-1/2, 1/2] (exp2_poly_fit.py writes them): 2.7e-6 in float32 Horner form.
// Arguments below -126, masked scores at -inf included, give exactly 0.
#pragma once

#include <hip/hip_runtime.h>

namespace xattn {

constexpr float kExp2C0 = 9.999992847e-01f;
constexpr float kExp2C1 = 6.931218505e-01f;
constexpr float kExp2C2 = 2.402474433e-01f;
constexpr float kExp2C3 = 5.591757968e-02f;
constexpr float kExp2C4 = 9.569989517e-03f;

__host__ __device__ __forceinline__ float soft_exp2(float x) {
    const float xc = fmaxf(x, -127.f);   // keeps n finite for -inf
    const float n = __builtin_rintf(xc);
    const float f = xc - n;
    float p = __builtin_fmaf(kExp2C4, f, kExp2C3);
    p = __builtin_fmaf(p, f, kExp2C2);
    p = __builtin_fmaf(p, f, kExp2C1);
    p = __builtin_fmaf(p, f, kExp2C0);
    const float r = __builtin_ldexpf(p, (int)n);
    return x < -126.f ? 0.f : r;
}

}  // namespace xattn
