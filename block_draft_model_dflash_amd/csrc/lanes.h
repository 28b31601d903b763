// Cross-lane reductions of a 64-lane wave without LDS: DPP within each 16-lane row, then the
// gfx950 lane-half swaps across rows.  Every lane of the reduced group ends with the same value:
// within a row, neighbours, pairs of a quad, quads (half-row mirror) and half-rows (row mirror)
// are combined with their mirror images, and a+b == b+a, so mirrored partners hold equal
// results; across rows, v_permlane16_swap / v_permlane32_swap hand each lane its partner's
// value and both add (lower half) + (upper half) in that order.
#pragma once
#include <hip/hip_runtime.h>

namespace dfl {

template <int CTRL>
__device__ __forceinline__ unsigned dpp_u32(unsigned x) {
  return (unsigned)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(x)));
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const unsigned long long u = __builtin_bit_cast(unsigned long long, x);
  const unsigned lo = dpp_u32<CTRL>((unsigned)u), hi = dpp_u32<CTRL>((unsigned)(u >> 32));
  return __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
}
constexpr int DPP_XOR1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141;  // lane i <- 7 - i within each half-row
constexpr int DPP_MIRROR = 0x140;       // lane i <- 15 - i within each row

// the value of the lane in the other row of the pair (rows 0<->1, 2<->3): (lower, upper)
__device__ __forceinline__ void swap16_u32(unsigned x, unsigned& lo, unsigned& hi) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  // r[0] holds the even row's values in both rows of a pair, r[1] the odd row's
  lo = r[0];
  hi = r[1];
}
__device__ __forceinline__ void swap32_u32(unsigned x, unsigned& lo, unsigned& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  lo = r[0];  // lanes 0-31's values, in both halves
  hi = r[1];  // lanes 32-63's values, in both halves
}

__device__ __forceinline__ float row16_max_f32(float x) {
  x = fmaxf(x, dpp_f32<DPP_XOR1>(x));
  x = fmaxf(x, dpp_f32<DPP_XOR2>(x));
  x = fmaxf(x, dpp_f32<DPP_HALF_MIRROR>(x));
  return fmaxf(x, dpp_f32<DPP_MIRROR>(x));
}
// maximum over each 32-lane half (lanes 0-31, 32-63)
__device__ __forceinline__ float half32_max_f32(float x) {
  x = row16_max_f32(x);
  unsigned lo, hi;
  swap16_u32(__float_as_uint(x), lo, hi);
  return fmaxf(__uint_as_float(lo), __uint_as_float(hi));
}

// maximum over the whole wave
__device__ __forceinline__ float wave_max_f32(float x) {
  x = half32_max_f32(x);
  unsigned lo, hi;
  swap32_u32(__float_as_uint(x), lo, hi);
  return fmaxf(__uint_as_float(lo), __uint_as_float(hi));
}

__device__ __forceinline__ double row16_sum_f64(double x) {
  x += dpp_f64<DPP_XOR1>(x);
  x += dpp_f64<DPP_XOR2>(x);
  x += dpp_f64<DPP_HALF_MIRROR>(x);
  return x + dpp_f64<DPP_MIRROR>(x);
}
__device__ __forceinline__ double row16_max_f64(double x) {
  x = fmax(x, dpp_f64<DPP_XOR1>(x));
  x = fmax(x, dpp_f64<DPP_XOR2>(x));
  x = fmax(x, dpp_f64<DPP_HALF_MIRROR>(x));
  return fmax(x, dpp_f64<DPP_MIRROR>(x));
}

// (lower, upper) halves of a double across the row pair / wave half
__device__ __forceinline__ void swap16_f64(double x, double& lo, double& hi) {
  const unsigned long long u = __builtin_bit_cast(unsigned long long, x);
  unsigned l0, h0, l1, h1;
  swap16_u32((unsigned)u, l0, h0);
  swap16_u32((unsigned)(u >> 32), l1, h1);
  lo = __builtin_bit_cast(double, ((unsigned long long)l1 << 32) | l0);
  hi = __builtin_bit_cast(double, ((unsigned long long)h1 << 32) | h0);
}
__device__ __forceinline__ void swap32_f64(double x, double& lo, double& hi) {
  const unsigned long long u = __builtin_bit_cast(unsigned long long, x);
  unsigned l0, h0, l1, h1;
  swap32_u32((unsigned)u, l0, h0);
  swap32_u32((unsigned)(u >> 32), l1, h1);
  lo = __builtin_bit_cast(double, ((unsigned long long)l1 << 32) | l0);
  hi = __builtin_bit_cast(double, ((unsigned long long)h1 << 32) | h0);
}

// sum / max over the lanes l, l^16, l^32, l^48 (the four rows at one row position)
__device__ __forceinline__ double cross4_sum_f64(double x) {
  double lo, hi;
  swap16_f64(x, lo, hi);
  x = lo + hi;
  swap32_f64(x, lo, hi);
  return lo + hi;
}
__device__ __forceinline__ double cross4_max_f64(double x) {
  double lo, hi;
  swap16_f64(x, lo, hi);
  x = fmax(lo, hi);
  swap32_f64(x, lo, hi);
  return fmax(lo, hi);
}
__device__ __forceinline__ double wave_sum_f64(double x) { return cross4_sum_f64(row16_sum_f64(x)); }
__device__ __forceinline__ double wave_max_f64(double x) { return cross4_max_f64(row16_max_f64(x)); }

}  // namespace dfl

namespace dfl {

// A8_32 of one element whose 32-element group sits in one 32-lane half of the wave (cortiq-engine
// dflash_dev.rs, the per-group int8 activation quantizer): d = amax/127, q = round(y * 127/amax)
// clamped to +-127; an all-zero group gives q = 0, d = 0.  Lane 0 of the group writes d.
__device__ __forceinline__ void emit_a8(float y, size_t qi, int8_t* __restrict__ xq, float* __restrict__ dx, size_t di,
                                        int lane) {
  const float amax = half32_max_f32(fabsf(y));
  int8_t q = 0;
  float d = 0.f;
  if (amax > 0.f) {
    d = amax / 127.0f;
    const float inv = 127.0f / amax;
    float r = __builtin_rintf(y * inv);
    r = fminf(fmaxf(r, -127.f), 127.f);
    q = (int8_t)r;
  }
  xq[qi] = q;
  if ((lane & 31) == 0) dx[di] = d;
}

}  // namespace dfl

namespace dfl {

// Arg-max in the order (larger value first, smaller index first among equal values): the order a
// top-k list keeps.  Over distinct indices it is a strict total order, so every lane of the wave
// ends with the same winner.
__device__ __forceinline__ bool argmax_better(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}
template <int CTRL>
__device__ __forceinline__ void argmax_dpp(float& v, int& i) {
  const float ov = dpp_f32<CTRL>(v);
  const int oi = (int)dpp_u32<CTRL>((unsigned)i);
  if (argmax_better(ov, oi, v, i)) {
    v = ov;
    i = oi;
  }
}
__device__ __forceinline__ void argmax_pick(unsigned vl, unsigned vh, unsigned il, unsigned ih, float& v, int& i) {
  const bool h = argmax_better(__uint_as_float(vh), (int)ih, __uint_as_float(vl), (int)il);
  v = __uint_as_float(h ? vh : vl);
  i = (int)(h ? ih : il);
}
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  argmax_dpp<DPP_XOR1>(v, i);
  argmax_dpp<DPP_XOR2>(v, i);
  argmax_dpp<DPP_HALF_MIRROR>(v, i);
  argmax_dpp<DPP_MIRROR>(v, i);
  unsigned vl, vh, il, ih;
  swap16_u32(__float_as_uint(v), vl, vh);
  swap16_u32((unsigned)i, il, ih);
  argmax_pick(vl, vh, il, ih, v, i);
  swap32_u32(__float_as_uint(v), vl, vh);
  swap32_u32((unsigned)i, il, ih);
  argmax_pick(vl, vh, il, ih, v, i);
}

}  // namespace dfl

namespace dfl {

// Maximum of a 64-bit unsigned key over the wave (every lane ends with it).
template <int CTRL>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long x) {
  const unsigned lo = dpp_u32<CTRL>((unsigned)x), hi = dpp_u32<CTRL>((unsigned)(x >> 32));
  return ((unsigned long long)hi << 32) | lo;
}
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long x) {
  unsigned long long y;
  y = dpp_u64<DPP_XOR1>(x);
  x = y > x ? y : x;
  y = dpp_u64<DPP_XOR2>(x);
  x = y > x ? y : x;
  y = dpp_u64<DPP_HALF_MIRROR>(x);
  x = y > x ? y : x;
  y = dpp_u64<DPP_MIRROR>(x);
  x = y > x ? y : x;
  unsigned l0, h0, l1, h1;
  swap16_u32((unsigned)x, l0, h0);
  swap16_u32((unsigned)(x >> 32), l1, h1);
  unsigned long long a = ((unsigned long long)l1 << 32) | l0, b = ((unsigned long long)h1 << 32) | h0;
  x = a > b ? a : b;
  swap32_u32((unsigned)x, l0, h0);
  swap32_u32((unsigned)(x >> 32), l1, h1);
  a = ((unsigned long long)l1 << 32) | l0;
  b = ((unsigned long long)h1 << 32) | h0;
  return a > b ? a : b;
}

}  // namespace dfl
