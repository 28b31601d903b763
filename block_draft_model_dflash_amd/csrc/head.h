// Device helpers shared by the q/k epilogue, the context append and the attention kernels: the
// f32 of a projection's f64 partial slices, and a head's RMSNorm + RoPE.
#pragma once
#include "common.h"
#include "lanes.h"

namespace dfl {

// f32 of the sum of S f64 partial slices of element (m, col): one rounding.  The slices are
// loaded together (they are independent) and added in slice order.
constexpr int MAX_SLICES = 16;
__device__ __forceinline__ float reduce_parts(const double* __restrict__ part, int S, int mstride, int m, size_t N,
                                              size_t col) {
  if (S == 1) return (float)part[(size_t)m * N + col];  // one slice: a plain load
  double v[MAX_SLICES];
#pragma unroll
  for (int s = 0; s < MAX_SLICES; s++) v[s] = s < S ? part[((size_t)s * mstride + m) * N + col] : 0.0;
  double o = v[0];
#pragma unroll
  for (int s = 1; s < MAX_SLICES; s++)
    if (s < S) o += v[s];
  return (float)o;
}

// Per-head RMSNorm then RoPE (cortiq-engine dflash.rs, Drafter::block / append: q_norm or k_norm
// over the head's hd values, s = 1/sqrt(f32(sum x^2 / hd) + eps), y = (x*s)*w, then the rotation
// of the pairs (d, d + hd/2) by the angle f32(pos) * inv_freq[d], an f32 product; a layer
// without rotary positions, Geometry::rotary false, keeps y).  One wave per
// (head, row): lane l holds dims l and l + hd/2 (hd <= 128), the pair the rotation mixes, so
// nothing crosses lanes but the sum of squares.  The angle's cosine and sine and the rotation are
// evaluated in f64 from the f32 y and rounded once.
__device__ __forceinline__ void head_norm_rope(float x0, float x1, int lane, int hd, const float* __restrict__ w,
                                               float eps, const float* __restrict__ inv_freq, long long pos,
                                               bool rope, float& o0, float& o1) {
  const int half = hd >> 1;
  const bool on = lane < half;
  double ss = on ? (double)x0 * (double)x0 + (double)x1 * (double)x1 : 0.0;
  ss = wave_sum_f64(ss);
  const float sc = 1.0f / sqrtf((float)(ss / (double)hd) + eps);
  if (!on) return;
  const float y0 = (x0 * sc) * w[lane], y1 = (x1 * sc) * w[lane + half];
  if (!rope) {
    o0 = y0;
    o1 = y1;
    return;
  }
  const float ang = (float)pos * inv_freq[lane];
  double sn, cs;
  sincos((double)ang, &sn, &cs);
  o0 = (float)((double)y0 * cs - (double)y1 * sn);
  o1 = (float)((double)y1 * cs + (double)y0 * sn);
}

}  // namespace dfl
