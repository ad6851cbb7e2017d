// RoPE angle arithmetic shared by the device kernels.
//
// cos and sin of the rotation angle p * f, computed in fp32 registers from
// the frequency's speed in turns per position, g = f / (2 pi), split on the
// host into fp32 hi + lo (g ~= hi + lo).  The angle is reduced exactly in
// turns: p * hi is split into its rounded value and its exact FMA error, the
// integer turns are dropped, and the remaining fraction feeds a quadrant
// reduction and Taylor polynomials of degree 9 (sine) and 10 (cosine) on
// |y| <= pi/4.  No position x frequency table exists in memory.
#pragma once

#include <hip/hip_runtime.h>

namespace is {

__device__ __forceinline__ float2 sincos_of_turns(int p, float ghi, float glo) {
  // The reduction relies on each product being rounded where written:
  // contracting p*ghi into the later subtraction would count its rounding
  // error twice.
#pragma clang fp contract(off)
  const float pf = (float)p;                  // exact: p < 2^24
  const float t = pf * ghi;
  const float e = __builtin_fmaf(pf, ghi, -t);  // exact error of p*ghi
  const float r = (t - __builtin_rintf(t)) + __builtin_fmaf(pf, glo, e);  // turns
  const float x4 = r * 4.0f;                   // quarter turns, exact
  const float q = __builtin_rintf(x4);
  const float z = x4 - q;                      // exact, |z| <= 1/2
  // y = z * pi/2 with pi/2 split in two floats
  const float y = __builtin_fmaf(z, 1.57079637050628662109375f,
                                 z * -4.37113900018624283e-8f);
  const float y2 = y * y;
  // Taylor series of sin and cos about 0, truncated after y^9 and y^10
  // (remainders below 2e-9 on |y| <= pi/4).
  const float sp = __builtin_fmaf(y2, __builtin_fmaf(y2, __builtin_fmaf(y2,
                       2.75573192239858907e-6f, -1.98412698412698413e-4f),
                       8.33333333333333333e-3f), -1.66666666666666667e-1f);
  const float sy = __builtin_fmaf(y * y2, sp, y);
  const float cp = __builtin_fmaf(y2, __builtin_fmaf(y2, __builtin_fmaf(y2,
                       __builtin_fmaf(y2, -2.75573192239858907e-7f,
                                      2.48015873015873016e-5f),
                       -1.38888888888888889e-3f), 4.16666666666666667e-2f), -0.5f);
  const float cy = __builtin_fmaf(y2, cp, 1.0f);
  const int quadrant = ((int)q) & 3;
  float c, s;
  if (quadrant == 0) { c = cy; s = sy; }
  else if (quadrant == 1) { c = -sy; s = cy; }
  else if (quadrant == 2) { c = -cy; s = -sy; }
  else { c = sy; s = -cy; }
  return make_float2(c, s);
}

}  // namespace is
