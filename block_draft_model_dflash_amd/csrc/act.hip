// Row-wise producers of the next matrix's activations: split-K reduction, residual add,
// RMSNorm, SwiGLU, q/k-norm + RoPE (block rows and context append), and the A8_32 quantizer.
//
// Sources: cortiq-engine "dflash.rs" -- fn rms (mean of squares in f64, scale 1/sqrt(f32(ms)
// + eps) in f32, (x*s)*w), Drafter::rotate (half-split pairs, angle = f32(pos)*inv_freq),
// Drafter::mlp (g/(1+e^-g)*u), Drafter::block (h += o), Drafter::settle_rows (K and V of
// context rows); "gpu_wgpu/dflash_dev.rs" -- dflash_qk (q/k rms then rotation, one workgroup
// a head and row).  A8_32 (int8 per row and group of 32): amax, d = amax/127, inv = 127/amax,
// q = clamp(rint(x*inv)), all f32 and correctly rounded (hipcc keeps IEEE division/sqrt).
//
// Every value stored as f32 is the rounding of an f64 evaluation (matrix products arrive as
// f64 partial sums; SwiGLU and the rotation are evaluated in f64), so it is the correctly
// rounded f32 of its step; the f32 steps the pages fix (the RMSNorm scale and products, the
// RoPE angle, the quantizer) are done in f32 exactly as written.
#include "common.h"
#include "digits.h"
#include "lanes.h"
#include "head.h"

namespace dfl {

__device__ __forceinline__ double block_sum_f64(double v, double* red) {
  v = wave_sum_f64(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double t = 0.0;
  for (int i = 0; i < nw; i++) t += red[i];
  return t;
}

constexpr int ROW_THREADS = 1024;  // one workgroup per row, 16 waves

// v = resid + o; optional write-back; RMSNorm; then A8_32 (QUANT) or f32.  The dx element of
// (row m, group g) sits at g*dxg + m*dxm.  One workgroup per row (without a norm, k_act_cols
// below runs instead).  Each sweep takes four elements a thread, their loads issued together;
// the first sweep also loads its norm weights, so a row of up to 4096 waits on memory once
// before the sum of squares and not again after it.
template <bool QUANT>
__global__ __launch_bounds__(ROW_THREADS) void k_norm_act(const double* __restrict__ part,
                                                         const float* __restrict__ x, int S, int part_mstride,
                                                         const float* __restrict__ resid, float* __restrict__ h_out,
                                                         const float* __restrict__ w, float eps, int M, int N,
                                                         int8_t* __restrict__ xq, float* __restrict__ dx, int dxg,
                                                         int dxm, float* __restrict__ xf) {
  extern __shared__ float row[];  // N floats
  __shared__ double red[ROW_THREADS / 64];
  const int m = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  if (m >= M) {
    for (int i = tid; i < N; i += ROW_THREADS) {
      if (QUANT) {
        xq[(size_t)m * N + i] = 0;
        if ((lane & 31) == 0) dx[(size_t)(i >> 5) * dxg + (size_t)m * dxm] = 0.f;
      } else {
        xf[(size_t)m * N + i] = 0.f;
      }
    }
    return;
  }
  constexpr int U = 4, SWEEP = U * ROW_THREADS;
  double ss = 0.0;
  float w0[U];  // the first sweep's weights
  for (int i0 = tid; i0 < N; i0 += SWEEP) {
    float o[U], r[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int i = i0 + u * ROW_THREADS;
      o[u] = i < N ? (part ? reduce_parts(part, S, part_mstride, m, N, i) : x[(size_t)m * N + i]) : 0.f;
      r[u] = i < N && resid ? resid[(size_t)m * N + i] : 0.f;
      if (i0 == tid) w0[u] = i < N ? w[i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int i = i0 + u * ROW_THREADS;
      if (i >= N) break;
      const float v = resid ? r[u] + o[u] : o[u];
      if (h_out) h_out[(size_t)m * N + i] = v;
      row[i] = v;
      ss += (double)v * (double)v;
    }
  }
  ss = block_sum_f64(ss, red);
  const float sc = 1.0f / sqrtf((float)(ss / (double)N) + eps);
  for (int i0 = tid; i0 < N; i0 += SWEEP) {
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int i = i0 + u * ROW_THREADS;
      if (i >= N) break;
      const float t = row[i] * sc;
      const float y = t * (i0 == tid ? w0[u] : w[i]);
      if (QUANT)
        emit_a8(y, (size_t)m * N + i, xq, dx, (size_t)(i >> 5) * dxg + (size_t)m * dxm, lane);
      else
        xf[(size_t)m * N + i] = y;
    }
  }
}

// The same without a norm, where nothing crosses a row: one workgroup per (256 columns, row),
// so a few wide rows (the taps of an append) spread over the whole chip.  N % 32 == 0 when
// quantizing, so a 32-element group is all in or all out of range.
constexpr int ACT_COLS = 256;
template <bool QUANT>
__global__ __launch_bounds__(ACT_COLS) void k_act_cols(const double* __restrict__ part, const float* __restrict__ x,
                                                      int S, int part_mstride, const float* __restrict__ resid,
                                                      float* __restrict__ h_out, int M, int N, int8_t* __restrict__ xq,
                                                      float* __restrict__ dx, int dxg, int dxm,
                                                      float* __restrict__ xf) {
  const int m = blockIdx.y, lane = threadIdx.x & 63;
  const int i = blockIdx.x * ACT_COLS + threadIdx.x;
  const bool in = i < N;
  if (m >= M) {
    if (!in) return;
    if (QUANT) {
      xq[(size_t)m * N + i] = 0;
      if ((lane & 31) == 0) dx[(size_t)(i >> 5) * dxg + (size_t)m * dxm] = 0.f;
    } else {
      xf[(size_t)m * N + i] = 0.f;
    }
    return;
  }
  float v = 0.f;
  if (in) {
    const float o = part ? reduce_parts(part, S, part_mstride, m, N, i) : x[(size_t)m * N + i];
    v = resid ? resid[(size_t)m * N + i] + o : o;
    if (h_out) h_out[(size_t)m * N + i] = v;
  }
  if (QUANT) {
    if (in) emit_a8(v, (size_t)m * N + i, xq, dx, (size_t)(i >> 5) * dxg + (size_t)m * dxm, lane);
  } else if (in) {
    xf[(size_t)m * N + i] = v;
  }
}

template <bool NORM, bool QUANT>
static hipError_t norm_act_inst(const double* part, const float* x, int S, int part_mstride, const float* resid,
                                float* h_out, const float* w, float eps, int M, int grid, int N, int8_t* xq,
                                float* dx, int dxg, int dxm, float* xf, hipStream_t st) {
  if constexpr (!NORM) {
    hipLaunchKernelGGL((k_act_cols<QUANT>), dim3((N + ACT_COLS - 1) / ACT_COLS, grid), dim3(ACT_COLS), 0, st, part, x,
                       S, part_mstride, resid, h_out, M, N, xq, dx, dxg, dxm, xf);
  } else {
    const size_t lds = (size_t)N * 4;
    hipError_t e = allow_lds((const void*)k_norm_act<QUANT>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_norm_act<QUANT>), dim3(grid), dim3(ROW_THREADS), lds, st, part, x, S, part_mstride, resid,
                       h_out, w, eps, M, N, xq, dx, dxg, dxm, xf);
  }
  return hipGetLastError();
}

hipError_t launch_norm_act(const double* part, const float* x, int S, int part_mstride, const float* resid,
                           float* h_out, const float* w, float eps, int M, int Mpad, int N, bool quant, int8_t* xq,
                           float* dxT, float* xf, hipStream_t st) {
  if ((w && (size_t)N * 4 > 96 * 1024) || (quant && N % 32) || (!part && !x) || S > MAX_SLICES)
    return hipErrorInvalidValue;
  if (w && quant)
    return norm_act_inst<true, true>(part, x, S, part_mstride, resid, h_out, w, eps, M, Mpad, N, xq, dxT, Mpad, 1, xf,
                                     st);
  if (w)
    return norm_act_inst<true, false>(part, x, S, part_mstride, resid, h_out, w, eps, M, Mpad, N, xq, dxT, Mpad, 1, xf,
                                      st);
  if (quant)
    return norm_act_inst<false, true>(part, x, S, part_mstride, resid, h_out, w, eps, M, Mpad, N, xq, dxT, Mpad, 1, xf,
                                      st);
  return norm_act_inst<false, false>(part, x, S, part_mstride, resid, h_out, w, eps, M, Mpad, N, xq, dxT, Mpad, 1, xf,
                                     st);
}

// RMSNorm + A8_32 (or f32) of rows whose sum of squares arrives in pieces: one workgroup per
// (256 columns, row).  The pieces are added lane-strided then across the wave, the same order on
// every run; s = 1/sqrt(f32(sum/N) + eps) and (h*s)*w in f32.  Rows >= M are written as zeros.
// xc (optional) receives the f32 rows too (a row convolution's input).
constexpr int RMS_COLS = 256;
template <bool QUANT>
__global__ __launch_bounds__(RMS_COLS) void k_rms_act(const float* __restrict__ h, const double* __restrict__ ssq,
                                                      int nparts, const float* __restrict__ w, float eps, int M,
                                                      int Mpad, int N, int8_t* __restrict__ xq,
                                                      float* __restrict__ dxT, float* __restrict__ xf,
                                                      float* __restrict__ xc) {
  const int m = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const int i = blockIdx.x * RMS_COLS + tid;
  if (m >= M) {
    if (i < N) {
      if (QUANT) {
        xq[(size_t)m * N + i] = 0;
        if ((lane & 31) == 0) dxT[(size_t)(i >> 5) * Mpad + m] = 0.f;
      } else {
        xf[(size_t)m * N + i] = 0.f;
      }
      if (xc) xc[(size_t)m * N + i] = 0.f;
    }
    return;
  }
  // this column's value and weight travel while the row's scale is formed; every wave forms the
  // scale itself (the same loads and the same order of additions), so no wave waits for another
  const float hv = i < N ? h[(size_t)m * N + i] : 0.f, wv = i < N ? w[i] : 0.f;
  double t = 0.0;
  int p = lane;
  for (; p + 192 < nparts; p += 256) {  // four pieces per lane in flight at once
    const double v0 = ssq[(size_t)m * nparts + p], v1 = ssq[(size_t)m * nparts + p + 64];
    const double v2 = ssq[(size_t)m * nparts + p + 128], v3 = ssq[(size_t)m * nparts + p + 192];
    t += v0;
    t += v1;
    t += v2;
    t += v3;
  }
  for (; p < nparts; p += 64) t += ssq[(size_t)m * nparts + p];
  t = wave_sum_f64(t);
  if (i >= N) return;  // N is a multiple of 32: whole A8 groups leave together
  const float sc = 1.0f / sqrtf((float)(t / (double)N) + eps);
  const float y = (hv * sc) * wv;
  if (xc) xc[(size_t)m * N + i] = y;
  if (QUANT)
    emit_a8(y, (size_t)m * N + i, xq, dxT, (size_t)(i >> 5) * Mpad + m, lane);
  else
    xf[(size_t)m * N + i] = y;
}

hipError_t launch_rms_act(const float* h, const double* ssq, int nparts, const float* w, float eps, int M, int Mpad,
                          int N, bool quant, int8_t* xq, float* dxT, float* xf, hipStream_t st, float* xc) {
  if (N % 32 || M > Mpad || nparts < 1) return hipErrorInvalidValue;
  dim3 g((unsigned)((N + RMS_COLS - 1) / RMS_COLS), (unsigned)Mpad);
  if (quant)
    hipLaunchKernelGGL(k_rms_act<true>, g, dim3(RMS_COLS), 0, st, h, ssq, nparts, w, eps, M, Mpad, N, xq, dxT, xf,
                       xc);
  else
    hipLaunchKernelGGL(k_rms_act<false>, g, dim3(RMS_COLS), 0, st, h, ssq, nparts, w, eps, M, Mpad, N, xq, dxT, xf,
                       xc);
  return hipGetLastError();
}

// Row convolutions (cortiq-engine dflash.rs, Drafter::conv_in / Drafter::conv, and the device
// block's dflash_conv): y[r][i] = sum over o < min(kn, r + 1) of (base[stage][o][i] +
// d[r][stage][o][i / gs]) * x[r - o][i], r the row's index in its sequence's block (rows of
// different sequences never mix).  Evaluated in f64 (every product of two f32 sums is exact
// there) and rounded once.  One thread per (column, row), 256 columns a workgroup.
constexpr int CONV_COLS = 256;
__device__ __forceinline__ float row_conv_at(const float* __restrict__ x, const float* __restrict__ d,
                                             const float* __restrict__ base, int m, int i, int r, int N, int gs,
                                             int kn, int stage) {
  const int groups = N / gs, pr = 2 * kn * groups, g = i / gs;
  double acc = 0.0;
  for (int o = 0; o < kn && o <= r; o++) {
    const int so = stage * kn + o;
    const double k = (double)base[(size_t)so * N + i] + (double)d[(size_t)m * pr + (size_t)so * groups + g];
    acc += k * (double)x[(size_t)(m - o) * N + i];
  }
  return (float)acc;
}

// Stage 0 on the normed rows x, then A8_32 into xq/dxT (or f32 into xf); rows M..Mpad zero.
template <bool QUANT>
__global__ __launch_bounds__(CONV_COLS) void k_conv_in(const float* __restrict__ x, const float* __restrict__ d,
                                                       const float* __restrict__ base, int M, int Mpad, int B, int N,
                                                       int gs, int kn, int8_t* __restrict__ xq,
                                                       float* __restrict__ dxT, float* __restrict__ xf) {
  const int m = blockIdx.y, i = blockIdx.x * CONV_COLS + threadIdx.x, lane = threadIdx.x & 63;
  if (i >= N) return;  // N is a multiple of 32: whole A8 groups leave together
  const float y = m < M ? row_conv_at(x, d, base, m, i, m % B, N, gs, kn, 0) : 0.f;
  if (QUANT)
    emit_a8(y, (size_t)m * N + i, xq, dxT, (size_t)(i >> 5) * Mpad + m, lane);
  else
    xf[(size_t)m * N + i] = y;
}

// Stage 1 on the sub-layer's output o, added to the residual rows h (h = f32(h + f32(conv))),
// with the rows' sums of squares in 16-column pieces ssq[m*(N/16) + i/16], as the residual
// GEMM epilogue writes them.
__global__ __launch_bounds__(CONV_COLS) void k_conv_out(const float* __restrict__ o, const float* __restrict__ d,
                                                        const float* __restrict__ base, int B, int N, int gs, int kn,
                                                        float* __restrict__ h, double* __restrict__ ssq) {
  const int m = blockIdx.y, i = blockIdx.x * CONV_COLS + threadIdx.x, lane = threadIdx.x & 63;
  if (i >= N) return;  // N is a multiple of 32: whole 16-column pieces leave together
  const float y = row_conv_at(o, d, base, m, i, m % B, N, gs, kn, 1);
  const float hv = h[(size_t)m * N + i] + y;
  h[(size_t)m * N + i] = hv;
  const double sq = row16_sum_f64((double)hv * (double)hv);
  if ((lane & 15) == 0) ssq[(size_t)m * (N / 16) + (i >> 4)] = sq;
}

hipError_t launch_conv_in(const float* x, const float* d, const float* base, int M, int Mpad, int B, int N, int gs,
                          int kn, bool quant, int8_t* xq, float* dxT, float* xf, hipStream_t st) {
  if (N % 32 || M > Mpad || gs < 1 || N % gs || kn < 1 || B < 1) return hipErrorInvalidValue;
  dim3 g((unsigned)((N + CONV_COLS - 1) / CONV_COLS), (unsigned)Mpad);
  if (quant)
    hipLaunchKernelGGL(k_conv_in<true>, g, dim3(CONV_COLS), 0, st, x, d, base, M, Mpad, B, N, gs, kn, xq, dxT, xf);
  else
    hipLaunchKernelGGL(k_conv_in<false>, g, dim3(CONV_COLS), 0, st, x, d, base, M, Mpad, B, N, gs, kn, xq, dxT, xf);
  return hipGetLastError();
}

hipError_t launch_conv_out(const float* o, const float* d, const float* base, int M, int B, int N, int gs, int kn,
                           float* h, double* ssq, hipStream_t st) {
  if (N % 32 || gs < 1 || N % gs || kn < 1 || B < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_conv_out, dim3((unsigned)((N + CONV_COLS - 1) / CONV_COLS), (unsigned)M), dim3(CONV_COLS), 0,
                     st, o, d, base, B, N, gs, kn, h, ssq);
  return hipGetLastError();
}

// h = x and each row's sum of squares per 256 columns (f64, in a fixed order).
__global__ __launch_bounds__(RMS_COLS) void k_copy_ssq(const float* __restrict__ x, float* __restrict__ h, int N,
                                                       double* __restrict__ ssq) {
  __shared__ double red[RMS_COLS / 64];
  const int m = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = blockIdx.x * RMS_COLS + tid;
  double t = 0.0;
  if (i < N) {
    const float v = x[(size_t)m * N + i];
    h[(size_t)m * N + i] = v;
    t = (double)v * (double)v;
  }
  t = wave_sum_f64(t);
  if (lane == 0) red[wave] = t;
  __syncthreads();
  if (tid == 0) {
    double s = red[0];
    for (int k = 1; k < RMS_COLS / 64; k++) s += red[k];
    ssq[(size_t)m * gridDim.x + blockIdx.x] = s;
  }
}

hipError_t launch_copy_ssq(const float* x, float* h, int M, int N, double* ssq, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  dim3 g((unsigned)((N + RMS_COLS - 1) / RMS_COLS), (unsigned)M);
  hipLaunchKernelGGL(k_copy_ssq, g, dim3(RMS_COLS), 0, st, x, h, N, ssq);
  return hipGetLastError();
}

// A8_32 of plain rows with scales in row order [rows][cols/32] (a unit entry point).
hipError_t launch_quant_rows(const float* x, int rows, int cols, int8_t* q, float* d, hipStream_t st) {
  if (cols % 32) return hipErrorInvalidValue;
  return norm_act_inst<false, true>(nullptr, x, 1, rows, nullptr, nullptr, nullptr, 0.f, rows, rows, cols, q, d, 1,
                                    cols / 32, nullptr, st);
}

__global__ void k_transpose_scales(const float* __restrict__ d, int rows, int groups, int Mpad,
                                   float* __restrict__ dT) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= groups * Mpad) return;
  const int g = i / Mpad, m = i % Mpad;
  dT[i] = m < rows ? d[(size_t)m * groups + g] : 0.f;
}

hipError_t launch_transpose_scales(const float* d, int rows, int groups, int Mpad, float* dT, hipStream_t st) {
  const int n = groups * Mpad;
  hipLaunchKernelGGL(k_transpose_scales, dim3((n + 255) / 256), dim3(256), 0, st, d, rows, groups, Mpad, dT);
  return hipGetLastError();
}

// a = silu(g) * u with g, u the f32 products, evaluated in f64.  Gate and up share n-tiles
// pairwise: column (i/16)*32 + i%16 is gate row i, 16 further the up row i.  Grid
// (ceil(I/1024), Mpad).
template <bool QUANT>
__global__ __launch_bounds__(256) void k_swiglu_act(const double* __restrict__ part, int S, int M, int Mpad, int I,
                                                   int8_t* __restrict__ xq, float* __restrict__ dxT,
                                                   float* __restrict__ xf) {
  const int m = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const size_t N2 = 2 * (size_t)I;
  for (int it = 0; it < 4; it++) {
    const int i = blockIdx.x * 1024 + it * 256 + tid;
    if (i >= I) break;
    float a = 0.f;
    if (m < M) {
      const size_t gc = (size_t)(i >> 4) * 32 + (i & 15);
      const double g = reduce_parts(part, S, Mpad, m, N2, gc);
      const double u = reduce_parts(part, S, Mpad, m, N2, gc + 16);
      a = (float)(g / (1.0 + exp(-g)) * u);
    }
    if (QUANT)
      emit_a8(a, (size_t)m * I + i, xq, dxT, (size_t)(i >> 5) * Mpad + m, lane);
    else
      xf[(size_t)m * I + i] = a;
  }
}

hipError_t launch_swiglu_act(const double* part, int S, int M, int Mpad, int I, bool quant, int8_t* xq, float* dxT,
                             float* xf, hipStream_t st) {
  if (I % 32 || S > MAX_SLICES) return hipErrorInvalidValue;
  dim3 g((unsigned)((I + 1023) / 1024), (unsigned)Mpad);
  if (quant)
    hipLaunchKernelGGL(k_swiglu_act<true>, g, dim3(256), 0, st, part, S, M, Mpad, I, xq, dxT, xf);
  else
    hipLaunchKernelGGL(k_swiglu_act<false>, g, dim3(256), 0, st, part, S, M, Mpad, I, xq, dxT, xf);
  return hipGetLastError();
}

// Grid (nh + 2 kvh heads, M rows), one wave each.  Columns of the fused projection: q heads,
// then k heads, then v heads, hd each.
__global__ __launch_bounds__(64) void k_qkv_epilogue(const double* __restrict__ part, int S, int Mpad, int B,
                                                    SeqInfo si, int nh, int kvh, int hd,
                                                    const float* __restrict__ q_norm,
                                                    const float* __restrict__ k_norm,
                                                    const float* __restrict__ inv_freq, float eps, int rope,
                                                    float* __restrict__ q, float* __restrict__ k,
                                                    float* __restrict__ v, int8_t* __restrict__ qd,
                                                    int* __restrict__ qe) {
  const int head = blockIdx.x, m = blockIdx.y, lane = threadIdx.x, half = hd >> 1;
  const size_t N = (size_t)(nh + 2 * kvh) * hd;
  const size_t col = (size_t)head * hd + lane;
  if (head >= nh + kvh) {
    for (int d = lane; d < hd; d += 64)
      v[((size_t)m * kvh + (head - nh - kvh)) * hd + d] = reduce_parts(part, S, Mpad, m, N, (size_t)head * hd + d);
    return;
  }
  const bool on = lane < half;
  const float x0 = on ? reduce_parts(part, S, Mpad, m, N, col) : 0.f;
  const float x1 = on ? reduce_parts(part, S, Mpad, m, N, col + half) : 0.f;
  const long long pos = si.pos0[m / B] + (m % B);
  const bool isq = head < nh;
  float o0 = 0.f, o1 = 0.f;
  head_norm_rope(x0, x1, lane, hd, isq ? q_norm : k_norm, eps, inv_freq, pos, rope != 0, o0, o1);
  if (qd && isq) {  // head_dim 128: lane l holds dims l and l + 64
    const int E = dig_exponent(wave_max_f32(fmaxf(fabsf(o0), fabsf(o1))));
    int d0[DIG_T], d1[DIG_T];
    dig_split(o0, E, d0);
    dig_split(o1, E, d1);
    const size_t r = (size_t)m * nh + head;
    int8_t* row = qd + r * DIG_ROW;
#pragma unroll
    for (int t = 0; t < DIG_T; t++) {
      row[t * 128 + lane] = (int8_t)d0[t];
      row[t * 128 + 64 + lane] = (int8_t)d1[t];
    }
    if (lane == 0) qe[r] = E;
  }
  if (!on) return;
  float* dst = isq ? q + ((size_t)m * nh + head) * hd : k + ((size_t)m * kvh + (head - nh)) * hd;
  dst[lane] = o0;
  dst[lane + half] = o1;
}

hipError_t launch_qkv_epilogue(const double* part, int S, int Mpad, int M, int B, const SeqInfo& si, int nh, int kvh,
                               int hd, const float* q_norm, const float* k_norm, const float* inv_freq, float eps,
                               bool rope, float* q, float* k, float* v, int8_t* qd, int* qe, hipStream_t st) {
  if (hd > 128 || hd % 2 || S > MAX_SLICES || (qd && (hd != 128 || !qe))) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_qkv_epilogue, dim3(nh + 2 * kvh, M), dim3(64), 0, st, part, S, Mpad, B, si, nh, kvh, hd,
                     q_norm, k_norm, inv_freq, eps, (int)rope, q, k, v, qd, qe);
  return hipGetLastError();
}

// Context append: grid (layers * 2 * kvh, n), one wave each.  Columns of the all-layer K|V
// projection: layer l's k heads then its v heads.  Cache layout [L][max_seqs][kvh][max_ctx][hd],
// elements f32 or (an f16 cache) the f32 values rounded to f16, to nearest even.
template <typename CT>
__global__ __launch_bounds__(64) void k_kv_append(const double* __restrict__ part, int S, int Mpad, int layers,
                                                 int kvh, int hd, const float* __restrict__ k_norms,
                                                 const float* __restrict__ inv_freq, float eps,
                                                 unsigned long long rot_mask, long long pos0, int row0, int slot,
                                                 int max_seqs, int max_ctx, CT* __restrict__ kc,
                                                 CT* __restrict__ vc, int8_t* __restrict__ kd,
                                                 int* __restrict__ ke) {
  const int unit = blockIdx.x, i = blockIdx.y, lane = threadIdx.x, half = hd >> 1;
  const int l = unit / (2 * kvh), rem = unit % (2 * kvh), kind = rem / kvh, h = rem % kvh;
  const size_t kvd = (size_t)kvh * hd, N = (size_t)layers * 2 * kvd;
  const size_t col0 = ((size_t)l * 2 + kind) * kvd + (size_t)h * hd;
  const size_t dst = ((((size_t)l * max_seqs + slot) * kvh + h) * max_ctx + (size_t)(row0 + i)) * hd;
  if (kind == 1) {
    for (int d = lane; d < hd; d += 64) vc[dst + d] = (CT)reduce_parts(part, S, Mpad, i, N, col0 + d);
    return;
  }
  const bool on = lane < half;
  const float x0 = on ? reduce_parts(part, S, Mpad, i, N, col0 + lane) : 0.f;
  const float x1 = on ? reduce_parts(part, S, Mpad, i, N, col0 + lane + half) : 0.f;
  float o0 = 0.f, o1 = 0.f;
  const bool rope = l >= 64 || ((rot_mask >> l) & 1ull);
  head_norm_rope(x0, x1, lane, hd, k_norms + (size_t)l * hd, eps, inv_freq, pos0 + i, rope, o0, o1);
  if (kd) {  // head_dim 128: lane l holds dims l and l + 64; the digits of the values stored
    const float v0 = (float)(CT)o0, v1 = (float)(CT)o1;
    const int E = dig_exponent(wave_max_f32(fmaxf(fabsf(v0), fabsf(v1))));
    int d0[DIG_T], d1[DIG_T];
    dig_split(v0, E, d0);
    dig_split(v1, E, d1);
    const size_t r = (((size_t)l * max_seqs + slot) * kvh + h) * max_ctx + (size_t)(row0 + i);
    int8_t* row = kd + r * DIG_ROW;
#pragma unroll
    for (int t = 0; t < DIG_T; t++) {
      row[t * 128 + lane] = (int8_t)d0[t];
      row[t * 128 + 64 + lane] = (int8_t)d1[t];
    }
    if (lane == 0) ke[r] = E;
  }
  if (!on) return;
  kc[dst + lane] = (CT)o0;
  kc[dst + lane + half] = (CT)o1;
}

hipError_t launch_kv_append(const double* part, int S, int Mpad, int n, int layers, int kvh, int hd,
                            const float* k_norms, const float* inv_freq, float eps, unsigned long long rot_mask,
                            long long pos0, int row0, int slot, int max_seqs, int max_ctx, bool f16, void* kc,
                            void* vc, int8_t* kd, int* ke, hipStream_t st) {
  if (hd > 128 || hd % 2 || S > MAX_SLICES || (kd && (hd != 128 || !ke))) return hipErrorInvalidValue;
  if (f16)
    hipLaunchKernelGGL(k_kv_append<_Float16>, dim3(layers * 2 * kvh, n), dim3(64), 0, st, part, S, Mpad, layers, kvh,
                       hd, k_norms, inv_freq, eps, rot_mask, pos0, row0, slot, max_seqs, max_ctx, (_Float16*)kc,
                       (_Float16*)vc, kd, ke);
  else
    hipLaunchKernelGGL(k_kv_append<float>, dim3(layers * 2 * kvh, n), dim3(64), 0, st, part, S, Mpad, layers, kvh, hd,
                       k_norms, inv_freq, eps, rot_mask, pos0, row0, slot, max_seqs, max_ctx, (float*)kc, (float*)vc,
                       kd, ke);
  return hipGetLastError();
}

// Cache rows back to f32 (a read-back for checks): out[r][h][d] = cache[layer][seq][h][row0+r][d].
template <typename CT>
__global__ __launch_bounds__(128) void k_read_cache(const CT* __restrict__ cache, size_t layer_elems, int layer,
                                                    int seq, int row0, int kvh, int hd, int max_ctx,
                                                    float* __restrict__ out) {
  const int r = blockIdx.x, h = blockIdx.y;
  const CT* src = cache + (size_t)layer * layer_elems + (((size_t)seq * kvh + h) * max_ctx + row0 + r) * hd;
  for (int d = threadIdx.x; d < hd; d += blockDim.x) out[((size_t)r * kvh + h) * hd + d] = (float)src[d];
}

hipError_t launch_read_cache(const void* cache, bool f16, size_t layer_elems, int layer, int seq, int row0, int n,
                             int kvh, int hd, int max_ctx, float* out, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (f16)
    hipLaunchKernelGGL(k_read_cache<_Float16>, dim3(n, kvh), dim3(128), 0, st, (const _Float16*)cache, layer_elems,
                       layer, seq, row0, kvh, hd, max_ctx, out);
  else
    hipLaunchKernelGGL(k_read_cache<float>, dim3(n, kvh), dim3(128), 0, st, (const float*)cache, layer_elems, layer,
                       seq, row0, kvh, hd, max_ctx, out);
  return hipGetLastError();
}

}  // namespace dfl
