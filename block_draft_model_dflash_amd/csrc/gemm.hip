// Weight-streaming quantized GEMM for gfx950: y[m][n] = sum_g d_w[n][g] * d_x[m][g] * s_g[m][n],
// s_g = sum over the 32 columns of group g of q_w * q_x (exact int32), with the drafter's
// 4-bit (Q4_32) or 8-bit (Q8_32) weights and A8_32 activations (gpu_wgpu/dflash_dev.rs,
// Dev::q4 / Dev::q8: int8 activations per group of 32 against the quantized weights).
//
// The block has 16..128 activation rows and thousands of weight rows, so the weights are the
// stream: each wave owns one 16-row n-tile and walks its superblocks (common.h) front to back,
// issuing PF 128-bit loads ahead.  One v_mfma_i32_16x16x32_i8 covers exactly one group of 32
// for 16 rows x 16 columns, so the per-group rescale is applied to its integer result right
// away.  The int8 activation block and its scales are staged once per workgroup in LDS and
// shared by the workgroup's four waves; K is split across blockIdx.y when the weight has few
// n-tiles (partial sums [S][Mpad][N] are reduced by the consumer kernel, in slice order).
//
// The rescale accumulates in f64: d_w*d_x is exact in f64 and so is its product with a Q4 group
// sum, so each output is the f32 rounding of (nearly) the exact sum, the same value a plain f64
// evaluation gives.  Every product feeds an int8 quantizer downstream, and a value one ulp off
// there flips codes that the following layers amplify to percent-level differences in the
// logits; correctly rounded outputs keep two implementations on the same codes.
#include "common.h"

namespace dfl {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef double v2d __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float f16_to_f32(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xffffu));
}

template <int FMT>
struct Super;
template <>
struct Super<Q4> {
  uint4 c;
  uint2 s;
};
template <>
struct Super<Q8> {
  uint4 c0, c1;
  uint2 s;
};

__device__ __forceinline__ void super_load(const uint8_t* sb, int lane, Super<Q4>& r) {
  r.c = *(const uint4*)(sb + 16 * lane);
  r.s = *(const uint2*)(sb + SB_SCALES_Q4 + 8 * (lane & 15));
}
__device__ __forceinline__ void super_load(const uint8_t* sb, int lane, Super<Q8>& r) {
  r.c0 = *(const uint4*)(sb + 16 * lane);
  r.c1 = *(const uint4*)(sb + 1024 + 16 * lane);
  r.s = *(const uint2*)(sb + SB_SCALES_Q8 + 8 * (lane & 15));
}

// The same through a buffer resource covering one wave's superblocks: a superblock past the
// resource's end reads as zeros and costs no memory traffic, so a load ring needs no branches.
constexpr int RSRC_WORD3 = 0x00020000;  // raw (untyped) buffer access, gfx9-family encoding
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wave_rsrc(const uint8_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, bytes, RSRC_WORD3);
}
__device__ __forceinline__ void super_load(__amdgpu_buffer_rsrc_t rs, int off, int lane, Super<Q4>& r) {
  r.c = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16 * lane, 0, 0));
  r.s = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, off + SB_SCALES_Q4 + 8 * (lane & 15), 0, 0));
}
__device__ __forceinline__ void super_load(__amdgpu_buffer_rsrc_t rs, int off, int lane, Super<Q8>& r) {
  r.c0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16 * lane, 0, 0));
  r.c1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 1024 + 16 * lane, 0, 0));
  r.s = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, off + SB_SCALES_Q8 + 8 * (lane & 15), 0, 0));
}

__device__ __forceinline__ uint32_t pick(uint4 v, int j) { return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w; }

// B operand of group j: 8 signed bytes, columns k0..k0+7 of the lane's row.  Q4 gives 16*q.
__device__ __forceinline__ long b_operand(const Super<Q4>& r, int j) {
  const uint32_t w = pick(r.c, j);
  const uint32_t lo = (w << 4) & 0xF0F0F0F0u, hi = w & 0xF0F0F0F0u;
  return (long)(((unsigned long)hi << 32) | lo);
}
__device__ __forceinline__ long b_operand(const Super<Q8>& r, int j) {
  const uint4 v = j < 2 ? r.c0 : r.c1;
  const uint32_t lo = (j & 1) ? v.z : v.x, hi = (j & 1) ? v.w : v.y;
  return (long)(((unsigned long)hi << 32) | lo);
}
template <int FMT>
__device__ __forceinline__ float w_scale(const Super<FMT>& r, int j) {
  const uint32_t w = j < 2 ? r.s.x : r.s.y;
  return f16_to_f32(w >> (16 * (j & 1)));
}

// superblocks in flight per wave (a register ring): deep for the block's few rows, shallower
// when the accumulators of many row tiles take the registers
constexpr int PF = 8;
template <int MT>
struct Ring {
  static constexpr int depth = MT <= 2 ? 8 : MT <= 4 ? 4 : 2;
};
// LDS budget of one workgroup's activation chunk (int8 rows and their scales): two
// workgroups fit a 160 KB CU
constexpr size_t LDS_BUDGET = 76 * 1024;

template <int FMT, int MT, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void k_gemm_q(const uint8_t* __restrict__ W, int N, int K,
                                                      const int8_t* __restrict__ xq,
                                                      const float* __restrict__ dxT, int kbps, int kcb,
                                                      void* __restrict__ out, int direct, int out_ld, int m_store) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int MR = MT * 16;
  constexpr int SBB = FMT == Q4 ? SB_Q4 : SB_Q8;
  constexpr int NT = 64 * WAVES;
  const int ASTR = kcb * 128 + 16;  // padded LDS row: rows land 4 banks apart
  int8_t* A = (int8_t*)smem;
  float* DX = (float*)(smem + MR * ASTR);  // [kcb*4 groups][MR] activation scales (exact in f64)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ntile = blockIdx.x * WAVES + wave;
  const bool active = ntile < (N >> 4);
  const int KB = K >> 7;
  const int kb0 = blockIdx.y * kbps;
  const int kb1 = min(kb0 + kbps, KB);
  const uint8_t* wt = W + (size_t)ntile * KB * SBB;
  const int quarter = lane >> 4, row16 = lane & 15;

  double acc[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; mt++)
#pragma unroll
    for (int r = 0; r < 4; r++) acc[mt][r] = 0.0;

  constexpr int RD = Ring<MT>::depth;
  Super<FMT> r[RD];
  for (int c0 = kb0; c0 < kb1; c0 += kcb) {
    const int c1 = min(c0 + kcb, kb1);
    const int ncols = (c1 - c0) * 128;
    if (c0 != kb0) __syncthreads();  // the previous chunk's LDS reads are done
    // the weights' ring is filled first, so their HBM latency overlaps the activations' staging
    const __amdgpu_buffer_rsrc_t rs = wave_rsrc(wt, active ? c1 * SBB : 0);
#pragma unroll
    for (int p = 0; p < RD; p++) super_load(rs, (c0 + p) * SBB, lane, r[p]);
    const int v16 = ncols >> 4;
    for (int i = tid; i < MR * v16; i += NT) {
      const int rr = i / v16, c = i - rr * v16;
      *(uint4*)(A + rr * ASTR + c * 16) = *(const uint4*)(xq + (size_t)rr * K + (size_t)c0 * 128 + c * 16);
    }
    const int ng = ncols >> 5;
    const float* dsrc = dxT + (size_t)c0 * 4 * MR;
    for (int i = tid; i < ng * MR; i += NT) DX[i] = dsrc[i];
    __syncthreads();
    if (!active) continue;
    for (int kb = c0; kb < c1; kb += RD) {
#pragma unroll
      for (int p = 0; p < RD; p++) {
        if (kb + p < c1) {
          const int kk = kb + p - c0;
#pragma unroll MT <= 2 ? 4 : 1
          for (int j = 0; j < 4; j++) {
            const long b = b_operand(r[p], j);
            const double dw = (double)w_scale<FMT>(r[p], j);
            const int col = kk * 128 + 32 * j + 8 * quarter;
#pragma unroll
            for (int mt = 0; mt < MT; mt++) {
              const long a = *(const long*)(A + (mt * 16 + row16) * ASTR + col);
              const v4i sm = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, b, (v4i){0, 0, 0, 0}, 0, 0, 0);
              const v4f dx = *(const v4f*)(DX + (kk * 4 + j) * MR + mt * 16 + 4 * quarter);
              acc[mt][0] = __builtin_fma((double)sm[0], dw * (double)dx[0], acc[mt][0]);
              acc[mt][1] = __builtin_fma((double)sm[1], dw * (double)dx[1], acc[mt][1]);
              acc[mt][2] = __builtin_fma((double)sm[2], dw * (double)dx[2], acc[mt][2]);
              acc[mt][3] = __builtin_fma((double)sm[3], dw * (double)dx[3], acc[mt][3]);
            }
          }
        }
        // refill the slot with the superblock RD ahead (zeros, no traffic, past the chunk)
        super_load(rs, (kb + p + RD) * SBB, lane, r[p]);
      }
    }
  }
  if (!active) return;
  const double post = FMT == Q4 ? 0.0625 : 1.0;  // Q4 codes entered the MFMA as 16*q
  const int n = ntile * 16 + row16;
#pragma unroll
  for (int mt = 0; mt < MT; mt++) {
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int m = mt * 16 + 4 * quarter + r;
      const double v = acc[mt][r] * post;
      if (direct) {
        if (m < m_store) ((float*)out)[(size_t)m * out_ld + n] = (float)v;
      } else {
        ((double*)out)[((size_t)blockIdx.y * MR + m) * N + n] = v;
      }
    }
  }
}

// The integer accumulators of the same tiles: sums[m][n][g] for every group (Q4 shifted back).
template <int FMT>
__global__ __launch_bounds__(256) void k_group_sums(const uint8_t* __restrict__ W, int N, int K,
                                                   const int8_t* __restrict__ xq, int Mpad, int M,
                                                   int32_t* __restrict__ sums) {
  constexpr int SBB = FMT == Q4 ? SB_Q4 : SB_Q8;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ntile = blockIdx.x * 4 + wave;
  if (ntile >= (N >> 4)) return;
  const int KB = K >> 7, G = K >> 5, kb = blockIdx.y;
  const int quarter = lane >> 4, row16 = lane & 15;
  Super<FMT> r;
  super_load(W + ((size_t)ntile * KB + kb) * SBB, lane, r);
  for (int j = 0; j < 4; j++) {
    const long b = b_operand(r, j);
    const int g = 4 * kb + j;
    for (int mt = 0; mt < Mpad / 16; mt++) {
      const long a = *(const long*)(xq + (size_t)(mt * 16 + row16) * K + 32 * g + 8 * quarter);
      const v4i s = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, b, (v4i){0, 0, 0, 0}, 0, 0, 0);
      for (int i = 0; i < 4; i++) {
        const int m = mt * 16 + 4 * quarter + i;
        const int n = ntile * 16 + row16;
        if (m < M) sums[((size_t)m * N + n) * G + g] = FMT == Q4 ? (s[i] >> 4) : s[i];
      }
    }
  }
}

static int ceil_div(int a, int b) { return (a + b - 1) / b; }

int normalize_splits(int K, int s) {
  const int KB = K / 128;
  if (s < 1) s = 1;
  if (s > KB) s = KB;
  if (s > 16) s = 16;  // the consumers add at most 16 slices
  const int kbps = ceil_div(KB, s);
  return ceil_div(KB, kbps);
}

int choose_splits(int N, int K, int Mpad) {
  (void)Mpad;
  const int tiles = N / 16, KB = K / 128;
  // A product with thousands of n-tiles streams its weights without splitting K; a smaller one
  // gives each wave about PF superblocks, so all of its loads are in flight from the start.
  if (tiles >= 4096) return 1;
  // at least ~2048 waves (eight per CU), and at most 16 superblocks per wave
  const int by_waves = ceil_div(2048, tiles), by_depth = ceil_div(KB, 2 * PF);
  return normalize_splits(K, by_waves > by_depth ? by_waves : by_depth);
}

template <int FMT, int MT>
static hipError_t gemm_inst(const void* W, int N, int K, const int8_t* xq, const float* dxT, int splits, void* out,
                            bool direct, int out_ld, int m_store, hipStream_t st) {
  constexpr int WAVES = 4;  // n-tiles sharing one LDS copy of the activations
  const int KB = K / 128;
  const int kbps = ceil_div(KB, splits);
  // per 128-column block: MT*16 rows of 128 codes + 4 groups x MT*16 f32 scales; row padding
  size_t budget = max_dynamic_lds();
  if (budget > LDS_BUDGET) budget = LDS_BUDGET;
  int kcb_max = (int)((budget - (size_t)256 * MT) / ((size_t)2304 * MT));
  if (kcb_max < 1) kcb_max = 1;
  const int kcb = kbps < kcb_max ? kbps : kcb_max;
  const size_t lds = (size_t)MT * 16 * (kcb * 128 + 16) + (size_t)kcb * 4 * MT * 16 * 4;
  hipError_t e = allow_lds((const void*)k_gemm_q<FMT, MT, WAVES>, lds);
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)ceil_div(N / 16, WAVES), (unsigned)ceil_div(KB, kbps));
  hipLaunchKernelGGL((k_gemm_q<FMT, MT, WAVES>), grid, dim3(64 * WAVES), lds, st, (const uint8_t*)W, N, K, xq, dxT,
                     kbps, kcb, out, direct ? 1 : 0, out_ld, m_store);
  return hipGetLastError();
}

template <int FMT>
static hipError_t gemm_fmt(const void* W, int N, int K, const int8_t* xq, const float* dxT, int Mpad, int splits,
                           void* out, bool direct, int out_ld, int m_store, hipStream_t st) {
  switch (Mpad / 16) {
    case 1: return gemm_inst<FMT, 1>(W, N, K, xq, dxT, splits, out, direct, out_ld, m_store, st);
    case 2: return gemm_inst<FMT, 2>(W, N, K, xq, dxT, splits, out, direct, out_ld, m_store, st);
    case 3: return gemm_inst<FMT, 3>(W, N, K, xq, dxT, splits, out, direct, out_ld, m_store, st);
    case 4: return gemm_inst<FMT, 4>(W, N, K, xq, dxT, splits, out, direct, out_ld, m_store, st);
    case 5: return gemm_inst<FMT, 5>(W, N, K, xq, dxT, splits, out, direct, out_ld, m_store, st);
    case 6: return gemm_inst<FMT, 6>(W, N, K, xq, dxT, splits, out, direct, out_ld, m_store, st);
    case 7: return gemm_inst<FMT, 7>(W, N, K, xq, dxT, splits, out, direct, out_ld, m_store, st);
    case 8: return gemm_inst<FMT, 8>(W, N, K, xq, dxT, splits, out, direct, out_ld, m_store, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_q(int fmt, const void* W, int N, int K, const int8_t* xq, const float* dxT, int Mpad,
                         int splits, void* out, bool direct, int out_ld, int m_store, hipStream_t st) {
  if (N % 16 || K % 128 || Mpad % 16 || Mpad < 16 || Mpad > 128) return hipErrorInvalidValue;
  splits = normalize_splits(K, splits);
  if (direct && splits != 1) return hipErrorInvalidValue;
  if (fmt == Q4) return gemm_fmt<Q4>(W, N, K, xq, dxT, Mpad, splits, out, direct, out_ld, m_store, st);
  if (fmt == Q8) return gemm_fmt<Q8>(W, N, K, xq, dxT, Mpad, splits, out, direct, out_ld, m_store, st);
  return hipErrorInvalidValue;
}

hipError_t launch_group_sums(int fmt, const void* W, int N, int K, const int8_t* xq, int Mpad, int M,
                             int32_t* sums, hipStream_t st) {
  if (N % 16 || K % 128 || Mpad % 16 || Mpad < 16 || Mpad > 128) return hipErrorInvalidValue;
  dim3 grid((unsigned)ceil_div(N / 16, 4), (unsigned)(K / 128));
  if (fmt == Q4)
    hipLaunchKernelGGL(k_group_sums<Q4>, grid, dim3(256), 0, st, (const uint8_t*)W, N, K, xq, Mpad, M, sums);
  else if (fmt == Q8)
    hipLaunchKernelGGL(k_group_sums<Q8>, grid, dim3(256), 0, st, (const uint8_t*)W, N, K, xq, Mpad, M, sums);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// f32 matrices (the unquantized drafter): one wave per output row, lanes across K, products
// and sums in f64 (f32 x f32 is exact in f64), one rounding at the end.
__global__ __launch_bounds__(256) void k_gemm_f32(const float* __restrict__ W, int N, int K,
                                                 const float* __restrict__ x, int Mpad, int M,
                                                 void* __restrict__ out, int direct, int out_ld, int m_store) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = blockIdx.x * 4 + wave;
  if (n >= N) return;
  const float* w = W + (size_t)n * K;
  for (int m = 0; m < Mpad; m++) {
    double acc = 0.0;
    if (m < M)
      for (int k = lane; k < K; k += 64) acc = __builtin_fma((double)w[k], (double)x[(size_t)m * K + k], acc);
    for (int o = 32; o; o >>= 1) acc += __shfl_xor(acc, o);
    if (lane == 0) {
      if (direct) {
        if (m < m_store) ((float*)out)[(size_t)m * out_ld + n] = (float)acc;
      } else {
        ((double*)out)[(size_t)m * N + n] = acc;
      }
    }
  }
}

hipError_t launch_gemm_f32(const float* W, int N, int K, const float* x, int Mpad, int M, void* out, bool direct,
                           int out_ld, int m_store, hipStream_t st) {
  hipLaunchKernelGGL(k_gemm_f32, dim3((unsigned)ceil_div(N, 4)), dim3(256), 0, st, W, N, K, x, Mpad, M, out,
                     direct ? 1 : 0, out_ld, m_store);
  return hipGetLastError();
}

}  // namespace dfl
