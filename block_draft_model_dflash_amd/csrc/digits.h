// Exact int8 digit splits of f32 rows (the Ozaki scheme: Ozaki, Ogita, Oishi, Rump, Numerical
// Algorithms 59, 2012; Ootomo, Ozaki, Yokota, IJHPCA 38, 2024), for dot products of key and
// query rows on the int8 matrix unit.
//
// A row r of f32 values with largest magnitude amax > 0 = m * 2^e (m in [0.5, 1)) is written as
//   r_d = 2^E * sum_{t < 7} D_t[d] * 128^-(t+1) + (remainder),   E = e + 1,
// every digit D_t in [-64, 64]: x = r_d * 2^-E has |x| < 1/2, and each step takes y = 128 * x
// (exact), D = round-to-nearest-even(y) (|y| <= 64), x = y - D (exact: the fraction of y, |x| <=
// 1/2).  Seven digits hold 49 bits below 2^E; an element loses bits only below 2^(E-50)
// (remainder at most 2^(E-50) in magnitude).  An all-zero row has E = 0 and zero digits.
//
// For two such rows, q . k = 2^(Eq+Ek) * 128^-2 * sum_{d <= 12} 128^-d * S_d with S_d the sum over
// the pairs t + u = d of the exact integer dot products D^q_t . D^k_u; keeping d <= 6 (28 pairs)
// drops at most 6 * 64^2 * 128^-9 * 128 dims of 2^(Eq+Ek) from d = 7 (less from the later
// ones): with |q|, |k| ~ 1 about 2^-35 worst case and 2^-42 typically, against the f64 sum's
// 2^-46.  Each S_d is exact in int32: |D^q D^k| <= 2^12, times 128 dims, times at most 7 pairs.
#pragma once
#include <hip/hip_runtime.h>

namespace dfl {

constexpr int DIG_T = 7;                       // digits per element
constexpr int DIG_ROW = DIG_T * 128;           // bytes of one 128-dim row's digits: [plane][dim]
// context rows in a call from which the default mode scores with digits (below them the f64
// kernel, with a workgroup per q head, is faster: on the 8B-shaped block with one sequence the
// two cross between 12288 and 16384 rows)
constexpr long DIG_AUTO_ROWS = 16384;

// the exponent E of a row from its largest magnitude
__device__ __forceinline__ int dig_exponent(float amax) {
  int e = 0;
  if (amax > 0.f) (void)frexpf(amax, &e);
  return amax > 0.f ? e + 1 : 0;
}

// the seven digits of v in a row of exponent E
__device__ __forceinline__ void dig_split(float v, int E, int (&d)[DIG_T]) {
  float x = ldexpf(v, -E);
#pragma unroll
  for (int t = 0; t < DIG_T; t++) {
    const float y = x * 128.f;
    const float r = rintf(y);
    d[t] = (int)r;
    x = y - r;
  }
}

}  // namespace dfl
