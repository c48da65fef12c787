// float64 2^y for the sampling and acceptance kernels of librva (gfx950).
//
// A branch-free Taylor evaluation, and a faster table-driven variant for bulk use.  Both stay
// within a few ulp of 2^y, far inside the 1e-9 (relative to the total mass) band within which
// a draw's bin may depend on rounding.
#pragma once

#include <hip/hip_runtime.h>

namespace rva {

// Taylor coefficients ln(2)^k / k! of 2^f, k = 0..13, correctly rounded.  They travel in
// the kernel arguments (scalar registers), so the FMAs take them as scalar operands instead of
// rebuilding 64-bit literals in vector registers at every use.
struct Exp2Poly {
  double c[14];
};
constexpr Exp2Poly kExp2Taylor = {{
    0x1.0000000000000p+0,  0x1.62e42fefa39efp-1,  0x1.ebfbdff82c58fp-3,  0x1.c6b08d704a0c0p-5,
    0x1.3b2ab6fba4e77p-7,  0x1.5d87fe78a6731p-10, 0x1.430912f86c787p-13, 0x1.ffcbfc588b0c7p-17,
    0x1.62c0223a5c824p-20, 0x1.b5253d395e7c4p-24, 0x1.e4cf5158b8ecap-28, 0x1.e8cac7351bb25p-32,
    0x1.c3bd650fc2986p-36, 0x1.816193166d0f9p-40}};

// 2^y in float64 for y <= 0, without branches: y is clamped at -1100 (the result then
// underflows to 0; NaN from fully masked rows also lands there), n = rint(y) by the
// round-to-nearest of adding and removing 1.5 * 2^52 (whose low word is then n), f = y - n
// with |f| <= 1/2, 2^f from the Taylor series of exp(f ln 2) to degree 13 (truncation
// < 2e-16), scaled by 2^n.
__device__ __forceinline__ double exp2_f64(const Exp2Poly& P, double y) {
  constexpr double kShifter = 0x1.8p52;
  y = fmax(y, -1100.0);
  const double s = y + kShifter;
  const double n = s - kShifter;
  const double f = y - n;
  double p = P.c[13];
#pragma unroll
  for (int k = 12; k >= 0; --k) p = fma(p, f, P.c[k]);
  return ldexp(p, int(__double2loint(s)));
}
constexpr double kLog2eF64 = 1.4426950408889634074;
// e^(x - m) in float64 for float32 x <= m (x = -inf gives 0)
__device__ __forceinline__ double exp_shift_f64(const Exp2Poly& P, float x, float m) {
  return exp2_f64(P, (double(x) - double(m)) * kLog2eF64);
}

// Faster 2^y in float64 for the bulk of the draw: y = (256 n + j) / 256 + f with k = 256 n + j
// = rint(256 y) and |f| <= 1/512; 2^y = 2^n * tab[j] * 2^f, tab[j] = 2^(j/256) (built per
// workgroup in LDS by exp2_f64), 2^f from its Taylor series to degree 4 (truncation
// < 4e-17).  Relative error about 1.5 ulp.
__device__ __forceinline__ double exp2_tab(const Exp2Poly& P, const double* tab, double y) {
  constexpr double kShifter = 0x1.8p52;
  y = fmax(y, -1100.0);
  const double s = fma(y, 256.0, kShifter);  // y * 256 is exact; the add rounds it to k
  const double kd = s - kShifter;
  const int k = int(__double2loint(s));
  const double f = fma(kd, -1.0 / 256.0, y);
  double p = fma(P.c[4], f, P.c[3]);
  p = fma(p, f, P.c[2]);
  p = fma(p, f, P.c[1]);
  p = fma(p, f, 1.0);
  return ldexp(tab[k & 255] * p, k >> 8);
}
__device__ __forceinline__ double exp_shift_tab(const Exp2Poly& P, const double* tab, float x, float m) {
  return exp2_tab(P, tab, (double(x) - double(m)) * kLog2eF64);
}
// Fills tab[j] = 2^(j/256), j < 256 (the workgroup must have >= 256 threads; ends with a barrier).
__device__ __forceinline__ void fill_exp2_tab(const Exp2Poly& P, double* tab) {
  if (threadIdx.x < 256) tab[threadIdx.x] = exp2_f64(P, double(threadIdx.x) / 256.0);
  __syncthreads();
}

}  // namespace rva
