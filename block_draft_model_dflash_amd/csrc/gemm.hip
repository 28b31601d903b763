// Weight-streaming quantized GEMM for gfx950: y[m][n] = sum_g d_w[n][g] * d_x[m][g] * s_g[m][n],
// s_g = sum over the 32 columns of group g of q_w * q_x (exact int32), with the drafter's
// 4-bit (Q4_32) or 8-bit (Q8_32) weights and A8_32 activations (gpu_wgpu/dflash_dev.rs,
// Dev::q4 / Dev::q8: int8 activations per group of 32 against the quantized weights).
//
// The block has 16..128 activation rows and thousands of weight rows, so the weights are the
// stream: each wave owns one 16-row n-tile (and a share of its k-blocks) and walks its
// superblocks (common.h) front to back with a ring of loads in flight.  One
// v_mfma_i32_16x16x32_i8 covers exactly one group of 32 for 16 rows x 16 columns, so the
// per-group rescale is applied to its integer result right away.  The int8 activation block and
// its scales are staged in LDS and shared by the workgroup's waves.  A product with few n-tiles
// splits K over the waves of one workgroup, which add their sums in LDS; the epilogue (the
// residual add with the row's sum of squares, with or without a row convolution's second stage,
// or SwiGLU with its A8 quantizer) runs in the same kernel, so no partial sums travel through
// memory.
//
// The rescale accumulates in f64: d_w*d_x is exact in f64 and so is its product with a Q4 group
// sum, so each output is the f32 rounding of (nearly) the exact sum, the same value a plain f64
// evaluation gives.  Every product feeds an int8 quantizer downstream, and a value one ulp off
// there flips codes that the following layers amplify to percent-level differences in the
// logits; correctly rounded outputs keep two implementations on the same codes.
#include <type_traits>

#include "common.h"
#include "lanes.h"

namespace dfl {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef double v2d __attribute__((ext_vector_type(2)));
typedef double v4d __attribute__((ext_vector_type(4)));

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
// `off` (the superblock's byte offset) is the same for the whole wave and goes in the scalar
// offset; only the lane's position within the superblock is a vector offset.
__device__ __forceinline__ void super_load(__amdgpu_buffer_rsrc_t rs, int off, int lane, Super<Q4>& r) {
  r.c = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * lane, off, 0));
  r.s = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, SB_SCALES_Q4 + 8 * (lane & 15), off, 0));
}
__device__ __forceinline__ void super_load(__amdgpu_buffer_rsrc_t rs, int off, int lane, Super<Q8>& r) {
  r.c0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * lane, off, 0));
  r.c1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, 1024 + 16 * lane, off, 0));
  r.s = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, SB_SCALES_Q8 + 8 * (lane & 15), off, 0));
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

// Element type of the staged activation scales: f64 when eight n-tiles share them.
template <int NTW>
struct DxType {
  using T = float;
  using V = v4f;
};
template <>
struct DxType<8> {
  using T = double;
  using V = v4d;
};

// Register ring depth (superblocks in flight per wave) and the k-blocks one turn of the ring
// covers across the workgroup's k-waves: about 32/MT k-blocks, so one turn's activations fit the
// LDS chunk.
template <int MT, int KW>
struct Ring {
  static constexpr int raw = 32 / MT / KW;
  static constexpr int depth = raw < 1 ? 1 : raw > 8 ? 8 : raw;
  static constexpr int step = depth * KW;
};

// The four groups of superblock r against k-block kk of the staged activations: one
// v_mfma_i32_16x16x32_i8 per group and m-tile, its exact int32 sums rescaled by d_w * d_x in f64.
template <int FMT, int MT, int NTW>
__device__ __forceinline__ void superblock_mfma(const Super<FMT>& r, const int8_t* A, int ASTR,
                                                const typename DxType<NTW>::T* DX, int MR, int kk, int quarter,
                                                int row16, double (&acc)[MT][4]) {
#pragma unroll MT <= 2 ? 4 : 1
  for (int j = 0; j < 4; j++) {
    const long b = b_operand(r, j);
    const double dw = (double)w_scale<FMT>(r, j);
    const int col = kk * 128 + 32 * j + 8 * quarter;
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
      const long a = *(const long*)(A + (mt * 16 + row16) * ASTR + col);
      const v4i sm = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, b, (v4i){0, 0, 0, 0}, 0, 0, 0);
      const auto dx = *(const typename DxType<NTW>::V*)(DX + (kk * 4 + j) * MR + mt * 16 + 4 * quarter);
      acc[mt][0] = __builtin_fma((double)sm[0], dw * (double)dx[0], acc[mt][0]);
      acc[mt][1] = __builtin_fma((double)sm[1], dw * (double)dx[1], acc[mt][1]);
      acc[mt][2] = __builtin_fma((double)sm[2], dw * (double)dx[2], acc[mt][2]);
      acc[mt][3] = __builtin_fma((double)sm[3], dw * (double)dx[3], acc[mt][3]);
    }
  }
}

// The end of a workgroup's product: the k-waves' sums, then the epilogue.  Every wave leaves its
// partials in LDS and k-wave s % KW adds slot s's in wave order (the same order on every run)
// and finishes it.  Output slot s = 4*mt + q of the accumulators is rows m0 + 16*mt + 4*quarter +
// q, column row16 of n-tile ntile.
template <int FMT, int MT, int NTW, int KW, bool CONV>
__device__ __forceinline__ void gemm_finish(double (&acc)[MT][4], const float (&hres)[MT][4], uint8_t* smem,
                                            const GemmOut& o, int N, int m0, int nb, int ntile, bool active,
                                            int nt, int kw) {
  constexpr int MR = MT * 16, NT = 64 * NTW * KW;
  const int tid = threadIdx.x, lane = tid & 63, quarter = lane >> 4, row16 = lane & 15, Mpad = o.Mpad;
  // output slot s = 4*mt + q of the accumulators (rows m0 + 16*mt + 4*quarter + q, column
  // row16 of the n-tile) is finished by k-wave s % KW
  auto mine = [&](int s) { return KW == 1 || s % KW == kw; };
  if (KW > 1) {
    __syncthreads();
    double* red = (double*)smem;
    if (active)
#pragma unroll
      for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int q = 0; q < 4; q++) red[(((kw * NTW + nt) * MT + mt) * 4 + q) * 64 + lane] = acc[mt][q];
    __syncthreads();
    if (active)
#pragma unroll
      for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int q = 0; q < 4; q++)
          if (mine(4 * mt + q)) {
            double v = red[((nt * MT + mt) * 4 + q) * 64 + lane];
            for (int k = 1; k < KW; k++) v += red[(((k * NTW + nt) * MT + mt) * 4 + q) * 64 + lane];
            acc[mt][q] = v;
          }
  }
  const double post = FMT == Q4 ? 0.0625 : 1.0;  // Q4 codes entered the MFMA as 16*q
  const int n = ntile * 16 + row16;

  if (o.epi == EPI_SWIGLU) {
    // NTW = 4g: each group of four n-tiles gate(2b), up(2b), gate(2b+1), up(2b+1) (b = nb*NTW/4 +
    // group) gives the 32 columns 32b.. of a = silu(gate) * up, one A8 group per row
    constexpr int WC = NTW * 16, AC = NTW * 8;  // product columns and a columns of the workgroup
    __syncthreads();
    float* G = (float*)smem;  // [MR][WC]: the tiles' f32 products
    if (active)
#pragma unroll
      for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int q = 0; q < 4; q++)
          if (mine(4 * mt + q)) G[(mt * 16 + 4 * quarter + q) * WC + nt * 16 + row16] = (float)(acc[mt][q] * post);
    __syncthreads();
    const int I = N >> 1;
    for (int i = tid; i < MR * AC; i += NT) {
      const int ml = i / AC, j = i % AC, m = m0 + ml;
      if (m >= Mpad) break;  // whole 32-lane groups leave together (AC is a multiple of 32)
      const int jj = j & 31;
      const int gc = (j >> 5) * 64 + (jj >> 4) * 32 + (jj & 15);
      const double g = G[ml * WC + gc], u = G[ml * WC + gc + 16];
      const float a = (float)(g / (1.0 + exp(-g)) * u);
      const int c = nb * AC + j;
      if (o.xq)
        emit_a8(a, (size_t)m * I + c, o.xq, o.dxT, (size_t)(c >> 5) * Mpad + m, lane);
      else
        o.xf[(size_t)m * I + c] = a;
    }
    return;
  }
  if (CONV) {  // EPI_CONV (its own instances, so the other epilogues carry none of this)
    // the row convolution's stage 1 needs the rows before each row, which sit in other lanes
    // and waves: the workgroup's f32 tile goes through LDS first (rows of a block never cross
    // the row group, checked at launch), then one thread per (row, column) adds its convolved
    // value to h; 16 consecutive threads hold one n-tile's 16 columns of a row for the sums of
    // squares
    constexpr int WC = NTW * 16;
    __syncthreads();
    float* Y = (float*)smem;  // [MR][WC]
    if (active)
#pragma unroll
      for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int q = 0; q < 4; q++)
          if (mine(4 * mt + q)) Y[(mt * 16 + 4 * quarter + q) * WC + nt * 16 + row16] = (float)(acc[mt][q] * post);
    __syncthreads();
    const int groups = N / o.cgs, pr = 2 * o.ckn * groups;
    for (int i = tid; i < MR * WC; i += NT) {
      const int ml = i / WC, cc = i % WC, m = m0 + ml, nn = nb * WC + cc;
      if (m >= Mpad) break;  // rows in order: the rest are past Mpad too (whole 16-lane groups)
      double sq = 0.0;
      if (m < o.M && nn < N) {
        const int r = m % o.cB, g = nn / o.cgs;
        double c = 0.0;
        for (int k = 0; k < o.ckn && k <= r; k++) {
          const int so = o.ckn + k;  // stage 1
          const double kk = (double)o.cbase[(size_t)so * N + nn] + (double)o.cd[(size_t)m * pr + (size_t)so * groups + g];
          c += kk * (double)Y[(ml - k) * WC + cc];
        }
        const float hv = o.h[(size_t)m * N + nn] + (float)c;
        o.h[(size_t)m * N + nn] = hv;
        sq = (double)hv * (double)hv;
      }
      sq = row16_sum_f64(sq);
      if ((lane & 15) == 0 && nn < N) o.ssq[(size_t)m * (N >> 4) + (nn >> 4)] = sq;
    }
    return;
  }
  if (!active) return;
#pragma unroll
  for (int mt = 0; mt < MT; mt++) {
#pragma unroll
    for (int q = 0; q < 4; q++) {
      if (!mine(4 * mt + q)) continue;
      const int m = m0 + mt * 16 + 4 * quarter + q;
      const double v = acc[mt][q] * post;
      if (o.epi == EPI_F64) {
        if (m < Mpad) ((double*)o.y)[(size_t)m * N + n] = v;
      } else if (o.epi == EPI_F32) {
        if (m < o.m_store) ((float*)o.y)[(size_t)m * o.ld + n] = (float)v;
      } else {  // EPI_RESID: h += f32(v), and the tile's share of each row's sum of squares
        double sq = 0.0;
        if (m < o.M) {
          const float hv = hres[mt][q] + (float)v;
          o.h[(size_t)m * N + n] = hv;
          sq = (double)hv * (double)hv;
        }
        sq = row16_sum_f64(sq);
        if (row16 == 0 && m < Mpad) o.ssq[(size_t)m * (N >> 4) + ntile] = sq;
      }
    }
  }
}

// One workgroup: NTW n-tiles x KW k-waves.  Wave (nt, kw) streams the superblocks kb = kw,
// kw + KW, ... of n-tile blockIdx.x*NTW + nt through its register ring; the activations of a
// chunk of kcb k-blocks (a multiple of the ring's step, so the ring runs on across chunks) are
// staged in LDS and shared by all waves.  The k-waves' f64 sums are then added in wave order
// through LDS (the same order on every run) and wave kw = 0 applies the epilogue.
//
// TURNS > 0: every chunk holds exactly TURNS ring turns (the last one may run past the tile,
// where the slots read zeros), so the ring is straight-line code and the compiler counts the
// loads in flight exactly; TURNS = 0 is the same with a runtime loop (shapes smaller than one
// full chunk).
template <int FMT, int MT, int NTW, int KW, int TURNS, bool CONV>
__global__ __launch_bounds__(64 * NTW * KW) void k_gemm_q(const uint8_t* __restrict__ W, int N, int K,
                                                         const int8_t* __restrict__ xq,
                                                         const float* __restrict__ dxT, int kcb, int RG,
                                                         GemmOut o) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int MR = MT * 16;
  constexpr int SBB = FMT == Q4 ? SB_Q4 : SB_Q8;
  constexpr int NT = 64 * NTW * KW;
  constexpr int RD = Ring<MT, KW>::depth, STEP = Ring<MT, KW>::step;
  const int ASTR = kcb * 128 + 16;  // padded LDS row: rows land 4 banks apart
  int8_t* A = (int8_t*)smem;
  // [kcb*4 groups][MR] activation scales; a workgroup of eight n-tiles keeps them as f64, so the
  // conversion is done once at staging instead of once per n-tile in the loop
  using DxT = typename DxType<NTW>::T;
  DxT* DX = (DxT*)(smem + MR * ASTR);
  // the wave index is uniform across the wave: saying so keeps the weight tile's buffer
  // resource in scalar registers (no per-lane descriptor loop around each load)
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nt = wave % NTW, kw = wave / NTW;
  // blockIdx.x = n-block * RG + row group: the row groups of one n-block are neighbours in the
  // grid, so they ask for the same weights at about the same time (this layout runs more than
  // one row group only for a row convolution's epilogue over more than 16 rows)
  const int rg = blockIdx.x % RG, nb = blockIdx.x / RG, m0 = rg * MR;
  const int ntile = nb * NTW + nt;
  const bool active = ntile < (N >> 4);
  const int KB = K >> 7, Mpad = o.Mpad;
  const uint8_t* wt = W + (size_t)(active ? ntile : 0) * KB * SBB;
  const int quarter = lane >> 4, row16 = lane & 15;

  double acc[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; mt++)
#pragma unroll
    for (int r = 0; r < 4; r++) acc[mt][r] = 0.0;

  // activations come through buffer resources that end at row Mpad (and at the last scale), so
  // every staging load is unconditional: a row past the end reads as zeros, and a lane whose
  // slot lies past the chunk loads something it then does not store
  const __amdgpu_buffer_rsrc_t xr = wave_rsrc((const uint8_t*)xq, Mpad * K);
  const __amdgpu_buffer_rsrc_t dr = wave_rsrc((const uint8_t*)dxT, (K >> 5) * Mpad * 4);
  constexpr int SB = 8;  // 16-byte activation pieces (and scales) each thread has in flight
  uint4 av[SB];
  float dv[SB];
  auto stage_load = [&](int c0, int c1, int i0) {
    const int v16 = (c1 - c0) * 8;  // 16-byte pieces of a staged row
#pragma unroll
    for (int b = 0; b < SB; b++) {
      const int i = i0 + b * NT, rr = i / v16, c = i - rr * v16;
      av[b] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, (m0 + rr) * K + c0 * 128 + c * 16, 0, 0));
    }
#pragma unroll
    for (int b = 0; b < SB; b++) {  // scales of group c0*4 + g, row m0 + m ([group][Mpad])
      const int i = i0 + b * NT, g = i / MR, m = i - g * MR;
      dv[b] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(dr, ((c0 * 4 + g) * Mpad + m0 + m) * 4, 0, 0));
    }
  };
  // the stores are unconditional too (a conditional store would pull its load down next to it):
  // a slot past the chunk writes row 0's padding or the scale array's spare word, never read
  auto stage_store = [&](int c0, int c1, int i0) {
    const int v16 = (c1 - c0) * 8, nv = MR * v16, nd = (c1 - c0) * 4 * MR;
#pragma unroll
    for (int b = 0; b < SB; b++) {
      const int i = i0 + b * NT, rr = i / v16, c = i - rr * v16;
      *(uint4*)(A + (i < nv ? rr * ASTR + c * 16 : kcb * 128)) = av[b];
    }
#pragma unroll
    for (int b = 0; b < SB; b++) {  // a scale of a row past Mpad belongs to the next group: 0
      const int i = i0 + b * NT, m = i % MR;
      DX[i < nd ? i : kcb * 4 * MR] = (DxT)(m0 + m < Mpad ? dv[b] : 0.f);
    }
  };

  // the first chunk's activations are requested before the weights: loads return in order, so
  // the staging then waits for them alone while the weights keep arriving
  stage_load(0, min(kcb, KB), tid);
  __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the weights'

  // the ring is filled before the activations are stored, so the weights' HBM latency overlaps
  // the staging; a superblock past the tile reads as zeros and costs nothing
  const __amdgpu_buffer_rsrc_t rs = wave_rsrc(wt, active ? KB * SBB : 0);
  Super<FMT> r[RD];
#pragma unroll
  for (int p = 0; p < RD; p++) super_load(rs, (kw + p * KW) * SBB, lane, r[p]);
  __builtin_amdgcn_sched_barrier(0);

  // the residual rows the epilogue adds to (needed only at the end), loaded without a branch
  // (a branch around them would make every later wait count them as possibly missing): rows
  // past M, and every row of another epilogue or of a tile past N, read as zeros
  const __amdgpu_buffer_rsrc_t hr = wave_rsrc((const uint8_t*)o.h, o.epi == EPI_RESID && active ? o.M * N * 4 : 0);
  float hres[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; mt++)
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int m = m0 + mt * 16 + 4 * quarter + q;
      hres[mt][q] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(hr, (m * N + ntile * 16 + row16) * 4, 0, 0));
    }

  // the ring turns over the staged chunk [c0, c1).  No branch in the ring: a chunk before the
  // last holds whole ring turns (kcb is a multiple of STEP), so a slot past c1 only occurs past
  // the tile's end, where it holds zeros and adds exactly 0 (its LDS reads are clamped into the
  // staged range, which holds finite values)
  auto chunk = [&](int c0, int c1) {
    constexpr int UNROLL = TURNS > 0 ? TURNS : 1;
    const int turns = TURNS > 0 ? TURNS : (c1 - c0 - kw + STEP - 1) / STEP;
#pragma unroll UNROLL
    for (int t = 0; t < turns; t++) {
      const int kb = c0 + kw + t * STEP;
#pragma unroll
      for (int p = 0; p < RD; p++) {
        const int kbp = kb + p * KW;
        superblock_mfma<FMT, MT, NTW>(r[p], A, ASTR, DX, MR, min(kbp, c1 - 1) - c0, quarter, row16, acc);
        // refill the slot with this wave's superblock one ring turn ahead
        super_load(rs, (kbp + STEP) * SBB, lane, r[p]);
      }
    }
  };

  // the first chunk, its first batch of activations already on the way (straight-line code, so
  // the stores wait for those loads alone)
  {
    const int c1 = min(kcb, KB);
    stage_store(0, c1, tid);
    for (int i0 = tid + NT * SB; i0 < MR * c1 * 8; i0 += NT * SB) {
      stage_load(0, c1, i0);
      stage_store(0, c1, i0);
    }
    __syncthreads();
    if (active) chunk(0, c1);
  }
  for (int c0 = kcb; c0 < KB; c0 += kcb) {
    const int c1 = min(c0 + kcb, KB);
    __syncthreads();  // the previous chunk's LDS reads are done
    for (int i0 = tid; i0 < MR * (c1 - c0) * 8; i0 += NT * SB) {
      stage_load(c0, c1, i0);
      stage_store(c0, c1, i0);
    }
    __syncthreads();
    if (active) chunk(c0, c1);
  }

  gemm_finish<FMT, MT, NTW, KW, CONV>(acc, hres, smem, o, N, m0, nb, ntile, active, nt, kw);
}

// 16 rows, K split over the eight waves of a workgroup (the products with few n-tiles), with
// every wave staging only its own activations.  Wave kw uses k-blocks kw, kw + 8, ... and
// nothing else, so the workgroup never copies all 16 x K codes into LDS behind a barrier: each
// ring slot carries a superblock's weights together with its k-block's 16 activation rows
// (32 bytes per lane, four lanes a row, coalesced) and their 64 scales, and the wave passes the
// activations through its own LDS buffer into the MFMA's operand layout right before use (a
// wave's LDS accesses take effect in order, so it needs no barrier).  The arithmetic and its
// order are k_gemm_q's with one m-tile, one n-tile and eight k-waves: both give the same bits.
template <int FMT>
struct KsSlot {
  Super<FMT> w;
  uint4 a0, a1;  // row lane / 4, bytes 32 * (lane % 4) .. +32 of the k-block
  float d;       // scale of group lane / 16, row lane % 16
};
constexpr int KS_WAVES = 8, KS_RD = 4, KS_XSTR = 144;  // 16 waves or deeper rings measured slower
constexpr int KS_BUF = 16 * KS_XSTR + 64 * 4;  // a wave's LDS: 16 rows of codes, 64 scales
// TURNS > 0: every wave runs exactly TURNS ring turns (K a multiple of the turn's 32 k-blocks, or
// one turn for smaller K), as straight-line code, so the compiler counts the loads in flight
// exactly and a slot waits only for its own; in a runtime loop it waits for every load at the
// top of each turn, which drains the ring.  TURNS = 0: the runtime loop (other K).
template <int FMT, int TURNS>
__global__ __launch_bounds__(64 * KS_WAVES) void k_gemm_ks(const uint8_t* __restrict__ W, int N, int K,
                                                          const int8_t* __restrict__ xq,
                                                          const float* __restrict__ dxT, GemmOut o) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int SBB = FMT == Q4 ? SB_Q4 : SB_Q8;
  const int tid = threadIdx.x, lane = tid & 63, kw = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int quarter = lane >> 4, row16 = lane & 15;
  const int ntile = blockIdx.x;  // the grid has exactly N/16 workgroups, and Mpad is 16
  const int KB = K >> 7;
  uint8_t* X = smem + kw * KS_BUF;
  float* DX = (float*)(X + 16 * KS_XSTR);
  // superblocks past the tile read as zeros (weights and scales: every product is 0); the
  // activations of such a slot come from the tile's last k-block, finite values
  const __amdgpu_buffer_rsrc_t rs = wave_rsrc(W + (size_t)ntile * KB * SBB, KB * SBB);
  const __amdgpu_buffer_rsrc_t xr = wave_rsrc((const uint8_t*)xq, 16 * K);
  const __amdgpu_buffer_rsrc_t dr = wave_rsrc((const uint8_t*)dxT, (K >> 5) * 16 * 4);
  const int arow = lane >> 2, apart = lane & 3;
  auto load = [&](int kb, KsSlot<FMT>& s) {
    const int kc = min(kb, KB - 1);
    s.a0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, arow * K + kc * 128 + 32 * apart, 0, 0));
    s.a1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, arow * K + kc * 128 + 32 * apart + 16, 0, 0));
    s.d = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(dr, (kc * 64 + lane) * 4, 0, 0));
    super_load(rs, kb * SBB, lane, s.w);
  };
  KsSlot<FMT> r[KS_RD];
#pragma unroll
  for (int p = 0; p < KS_RD; p++) load(kw + p * KS_WAVES, r[p]);
  // the residual rows the epilogue adds to (needed only at the end)
  const __amdgpu_buffer_rsrc_t hr = wave_rsrc((const uint8_t*)o.h, o.epi == EPI_RESID ? o.M * N * 4 : 0);
  float hres[1][4];
#pragma unroll
  for (int q = 0; q < 4; q++)
    hres[0][q] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(hr, ((4 * quarter + q) * N + ntile * 16 + row16) * 4, 0, 0));

  double acc[1][4] = {{0.0, 0.0, 0.0, 0.0}};
  constexpr int STEP = KS_RD * KS_WAVES;
  const int turns = TURNS > 0 ? TURNS : (KB - kw + STEP - 1) / STEP;
  constexpr int UNROLL = TURNS > 0 ? TURNS : 1;
#pragma unroll UNROLL
  for (int t = 0; t < turns; t++) {
#pragma unroll
    for (int p = 0; p < KS_RD; p++) {
      KsSlot<FMT>& s = r[p];
      *(uint4*)(X + arow * KS_XSTR + 32 * apart) = s.a0;
      *(uint4*)(X + arow * KS_XSTR + 32 * apart + 16) = s.a1;
      DX[lane] = s.d;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const long b = b_operand(s.w, j);
        const double dw = (double)w_scale<FMT>(s.w, j);
        const long a = *(const long*)(X + row16 * KS_XSTR + 32 * j + 8 * quarter);
        const v4i sm = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, b, (v4i){0, 0, 0, 0}, 0, 0, 0);
        const v4f dx = *(const v4f*)(DX + 16 * j + 4 * quarter);
        acc[0][0] = __builtin_fma((double)sm[0], dw * (double)dx[0], acc[0][0]);
        acc[0][1] = __builtin_fma((double)sm[1], dw * (double)dx[1], acc[0][1]);
        acc[0][2] = __builtin_fma((double)sm[2], dw * (double)dx[2], acc[0][2]);
        acc[0][3] = __builtin_fma((double)sm[3], dw * (double)dx[3], acc[0][3]);
      }
      // refill the slot one ring turn ahead (past the tile: zeros, no traffic); the barrier
      // keeps the refill here, where it has a whole turn to arrive (unrolled, the scheduler
      // would otherwise sink it next to its use)
      load(kw + (t + 1) * STEP + p * KS_WAVES, s);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  gemm_finish<FMT, 1, 1, KS_WAVES, false>(acc, hres, smem, o, N, 0, ntile, ntile, true, 0, kw);
}

template <int FMT, int TURNS>
static hipError_t gemm_ks_turns(const void* W, int N, int K, const int8_t* xq, const float* dxT, const GemmOut& o,
                                hipStream_t st) {
  size_t lds = (size_t)KS_WAVES * KS_BUF;
  const size_t red = (size_t)KS_WAVES * 4 * 64 * 8;  // every k-wave's partials (after the loop)
  if (red > lds) lds = red;
  const void* kern = (const void*)k_gemm_ks<FMT, TURNS>;
  hipError_t e = allow_lds(kern, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_gemm_ks<FMT, TURNS>), dim3((unsigned)(N / 16)), dim3(64 * KS_WAVES), lds, st,
                     (const uint8_t*)W, N, K, xq, dxT, o);
  return hipGetLastError();
}

// the turn count every wave shares, where it is one of the unrolled instances (K of 4096 and
// below, 8192, 12288, 16384, 20480), else the runtime loop
template <int FMT>
static hipError_t gemm_ks_inst(const void* W, int N, int K, const int8_t* xq, const float* dxT, const GemmOut& o,
                               hipStream_t st) {
  constexpr int STEP = KS_RD * KS_WAVES;
  const int KB = K >> 7;
  const int turns = KB <= STEP ? 1 : KB % STEP == 0 ? KB / STEP : 0;
  switch (turns) {
    case 1: return gemm_ks_turns<FMT, 1>(W, N, K, xq, dxT, o, st);
    case 2: return gemm_ks_turns<FMT, 2>(W, N, K, xq, dxT, o, st);
    case 3: return gemm_ks_turns<FMT, 3>(W, N, K, xq, dxT, o, st);
    case 4: return gemm_ks_turns<FMT, 4>(W, N, K, xq, dxT, o, st);
    case 5: return gemm_ks_turns<FMT, 5>(W, N, K, xq, dxT, o, st);
    default: return gemm_ks_turns<FMT, 0>(W, N, K, xq, dxT, o, st);
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

// ---- products of more than 16 rows (a batch of sequences, the context append) ----
//
// The weights are the MFMA's A operand and the activations its B operand, so lane l of a wave
// accumulates D[n][m] for the four n-rows 4*quarter .. +3 of its n-tile and the single
// activation row m = l % 16 of each m-tile.  The rescale of a group then needs one activation
// scale per lane and m-tile (the same for the lane's four n-rows) and four weight scales per
// lane (the same for every m-tile), converted once per superblock: each term costs one int->f64
// conversion, one product d_w * d_x and one fused multiply-add.  A workgroup serves MT m-tiles
// (all the rows of its row group), NTW n-tiles and KW k-waves; every weight superblock is read
// once per row group and used for all of its rows.  The activations come in chunks of KW
// k-blocks (one for each k-wave) through two LDS buffers: while the waves multiply chunk c, the
// loads of chunk c + 1 are in flight to registers, and they are stored to the other buffer
// before the barrier that closes the step; the activation scales are kept in LDS as f64.

// A superblock for this orientation: the lane's codes as in Super<FMT>, and the f16 scales of
// the lane's four n-rows (rows 4*quarter .. +3 of the tile, four groups each: 32 bytes).
template <int FMT>
struct SuperR;
template <>
struct SuperR<Q4> {
  uint4 c;
  uint4 s0, s1;
};
template <>
struct SuperR<Q8> {
  uint4 c0, c1;
  uint4 s0, s1;
};

__device__ __forceinline__ void super_load_r(__amdgpu_buffer_rsrc_t rs, int off, int lane, SuperR<Q4>& r) {
  r.c = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * lane, off, 0));
  const int so = SB_SCALES_Q4 + 32 * (lane >> 4);
  r.s0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, so, off, 0));
  r.s1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, so + 16, off, 0));
}
__device__ __forceinline__ void super_load_r(__amdgpu_buffer_rsrc_t rs, int off, int lane, SuperR<Q8>& r) {
  r.c0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * lane, off, 0));
  r.c1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, 1024 + 16 * lane, off, 0));
  const int so = SB_SCALES_Q8 + 32 * (lane >> 4);
  r.s0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, so, off, 0));
  r.s1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, so + 16, off, 0));
}
__device__ __forceinline__ long a_operand(const SuperR<Q4>& r, int j) {
  const uint32_t w = pick(r.c, j);
  const uint32_t lo = (w << 4) & 0xF0F0F0F0u, hi = w & 0xF0F0F0F0u;
  return (long)(((unsigned long)hi << 32) | lo);
}
__device__ __forceinline__ long a_operand(const SuperR<Q8>& r, int j) {
  const uint4 v = j < 2 ? r.c0 : r.c1;
  const uint32_t lo = (j & 1) ? v.z : v.x, hi = (j & 1) ? v.w : v.y;
  return (long)(((unsigned long)hi << 32) | lo);
}
// the scale of n-row 4*quarter + rr, group j, as f64 (f16 scales [row][group] in s0 | s1)
template <int FMT>
__device__ __forceinline__ double w_scale_r(const SuperR<FMT>& r, int rr, int j) {
  const int i = rr * 4 + j;  // 0..15
  const uint4 v = i < 8 ? r.s0 : r.s1;
  const uint32_t w = pick(v, (i & 7) >> 1);
  return (double)f16_to_f32(w >> (16 * (i & 1)));
}

constexpr int gcd2(int a, int b) { return b ? gcd2(b, a % b) : a; }
constexpr int lcm3(int a, int b, int c) { return a / gcd2(a, b) * b / gcd2(a / gcd2(a, b) * b, c) * c; }

constexpr int ROWS_XSTR = 144;  // LDS bytes per staged row of a k-block (128 + 16: rows 36 banks apart)

template <int MT, int KW>
struct RowsChunk {
  static constexpr int MR = MT * 16;
  static constexpr int XBYTES = KW * MR * ROWS_XSTR;               // codes [KW][MR][144]
  static constexpr int BYTES = XBYTES + KW * 4 * MR * 8;           // + scales [KW][4][MR] f64
  static constexpr int PIECES = (KW * MR * 8 + 511) / 512;          // 16-byte code pieces per thread
  static constexpr int SCALES = (KW * 4 * MR + 511) / 512;          // scales per thread
};

// (at most 128 registers: two workgroups a CU; only the Q8 product with two n-tiles x four k-waves
// needs the cap, and spills two registers outside its loop)
template <int FMT, int MT, int NTW, int KW>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void k_gemm_rows(const uint8_t* __restrict__ W, int N, int K,
                                                  const int8_t* __restrict__ xq, const float* __restrict__ dxT,
                                                  int RG, GemmOut o) {
  static_assert(NTW * KW == 8, "eight waves");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  using CH = RowsChunk<MT, KW>;
  constexpr int MR = CH::MR, NT = 512, RD = 3;  // RD: chunks of weights in flight per wave
  constexpr int SBB = FMT == Q4 ? SB_Q4 : SB_Q8;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nt = wave % NTW, kw = wave / NTW;
  // workgroups go round-robin over the eight XCDs (each with its own L2): the RG row groups of
  // an n-block get ids eight apart, so they run on one XCD and read its weights through one L2
  const int nb = (blockIdx.x / (8 * RG)) * 8 + blockIdx.x % 8, rg = (blockIdx.x / 8) % RG, m0 = rg * MR;
  if (nb * NTW >= (N >> 4)) return;  // the whole workgroup: padding of the last group of eight
  const int ntile = nb * NTW + nt;
  const bool active = ntile < (N >> 4);
  const int KB = K >> 7, NC = (KB + KW - 1) / KW, Mpad = o.Mpad;
  const int quarter = lane >> 4, col = lane & 15;

  // activations: rows past Mpad read as zeros through the resource; a k-block past K is clamped
  // to the last one (its weights read as zeros, so it adds exactly 0)
  const __amdgpu_buffer_rsrc_t xr = wave_rsrc((const uint8_t*)xq, Mpad * K);
  // NSET register sets of staged activations: chunk c's loads are issued NSET chunk steps
  // before the step that stores them (set c % NSET), so their latency is hidden behind that many
  // steps of work.  With 64-row workgroups, weights read cold (µs, 128 rows, one set / four):
  // head 556 / 527, gate|up 100 / 93, down 51 / 49; with 32-row ones (two workgroups a CU) one
  // set for four n-tiles and two for two measured the same as two sets for all.
  constexpr int NSET = MT >= 4 ? 4 : MT == 2 && NTW >= 4 ? 1 : 2;
  uint4 avs[NSET][CH::PIECES];
  float dvs[NSET][CH::SCALES];
  auto stage_load = [&](int c, uint4 (&av)[CH::PIECES], float (&dv)[CH::SCALES]) {
#pragma unroll
    for (int b = 0; b < CH::PIECES; b++) {
      const int i = tid + b * NT, w = i / (MR * 8), rem = i % (MR * 8), row = rem >> 3, pc = rem & 7;
      const int kb = min(c * KW + min(w, KW - 1), KB - 1);
      av[b] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, (m0 + row) * K + kb * 128 + pc * 16, 0, 0));
    }
#pragma unroll
    for (int b = 0; b < CH::SCALES; b++) {
      const int i = min(tid + b * NT, KW * 4 * MR - 1), w = i / (4 * MR), rem = i % (4 * MR), g = rem / MR, row = rem % MR;
      const int kb = min(c * KW + w, KB - 1);
      dv[b] = m0 + row < Mpad ? dxT[(size_t)(kb * 4 + g) * Mpad + m0 + row] : 0.f;
    }
  };
  auto stage_store = [&](int buf, const uint4 (&av)[CH::PIECES], const float (&dv)[CH::SCALES]) {
    uint8_t* X = smem + buf * CH::BYTES;
    double* DX = (double*)(X + CH::XBYTES);
#pragma unroll
    for (int b = 0; b < CH::PIECES; b++) {
      const int i = tid + b * NT, w = i / (MR * 8), rem = i % (MR * 8), row = rem >> 3, pc = rem & 7;
      if (i < KW * MR * 8) *(uint4*)(X + (w * MR + row) * ROWS_XSTR + pc * 16) = av[b];
    }
#pragma unroll
    for (int b = 0; b < CH::SCALES; b++) {
      const int i = tid + b * NT;
      if (i < KW * 4 * MR) DX[i] = (double)dv[b];
    }
  };

  // this wave's weights: one superblock per chunk (k-block c*KW + kw); past the tile: zeros
  const uint8_t* wt = W + (size_t)(active ? ntile : 0) * KB * SBB;
  const __amdgpu_buffer_rsrc_t rs = wave_rsrc(wt, active ? KB * SBB : 0);
  SuperR<FMT> ring[RD];

  double acc[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; mt++)
#pragma unroll
    for (int rr = 0; rr < 4; rr++) acc[mt][rr] = 0.0;

  auto compute = [&](int buf, const SuperR<FMT>& r) {
    const uint8_t* X = smem + buf * CH::BYTES + kw * MR * ROWS_XSTR;
    const double* DX = (const double*)(smem + buf * CH::BYTES + CH::XBYTES) + kw * 4 * MR;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const long a = a_operand(r, j);
      double dw[4];
#pragma unroll
      for (int rr = 0; rr < 4; rr++) dw[rr] = w_scale_r<FMT>(r, rr, j);
#pragma unroll
      for (int mt = 0; mt < MT; mt++) {
        const long b = *(const long*)(X + (mt * 16 + col) * ROWS_XSTR + 32 * j + 8 * quarter);
        const v4i sm = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, b, (v4i){0, 0, 0, 0}, 0, 0, 0);
        const double dx = DX[j * MR + mt * 16 + col];
#pragma unroll
        for (int rr = 0; rr < 4; rr++) acc[mt][rr] = __builtin_fma((double)sm[rr], dw[rr] * dx, acc[mt][rr]);
      }
    }
  };

  // chunk 0's activations first (loads return in order: the store then waits for them alone),
  // then the weights of the first RD chunks, then the activations of chunks 1 .. NSET
  stage_load(0, avs[0], dvs[0]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int p = 0; p < RD; p++) super_load_r(rs, (p * KW + kw) * SBB, lane, ring[p]);
  __builtin_amdgcn_sched_barrier(0);
  stage_store(0, avs[0], dvs[0]);
#pragma unroll
  for (int k = 1; k <= NSET; k++)
    if (NC > k) stage_load(k, avs[k % NSET], dvs[k % NSET]);
  __syncthreads();
  // step c: chunk c's products from LDS buffer c & 1; chunk c + 1 (loaded NSET steps ago) into
  // the other buffer, whose readers (chunk c - 1) passed the last barrier; chunk c + 1 + NSET's
  // loads into the register set just freed; chunk c + RD's weights into the ring slot just used.
  // U steps an iteration keep the buffer, the ring slot and the register set compile-time
  // indices.
  constexpr int U = lcm3(RD, NSET, 2);
  for (int c0 = 0; c0 < NC; c0 += U) {
#pragma unroll
    for (int p = 0; p < U; p++) {
      const int c = c0 + p;
      if (c >= NC) break;  // uniform
      const int sn = (p + 1) % NSET;
      if (active) compute(p & 1, ring[p % RD]);
      if (c + 1 < NC) stage_store((p + 1) & 1, avs[sn], dvs[sn]);
      if (c + 1 + NSET < NC) stage_load(c + 1 + NSET, avs[sn], dvs[sn]);
      super_load_r(rs, ((c + RD) * KW + kw) * SBB, lane, ring[p % RD]);
      __syncthreads();
    }
  }

  // the k-waves' sums through LDS, added in wave order by k-wave 0, which finishes the n-tile
  // (slot (mt, rr): row m0 + 16*mt + col, column 16*ntile + 4*quarter + rr)
  const bool fin = kw == 0;
  if (KW > 1) {
    double* red = (double*)smem;
    if (active)
#pragma unroll
      for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int rr = 0; rr < 4; rr++) red[(((kw * NTW + nt) * MT + mt) * 4 + rr) * 64 + lane] = acc[mt][rr];
    __syncthreads();
    if (fin && active)
#pragma unroll
      for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int rr = 0; rr < 4; rr++) {
          double v = red[((nt * MT + mt) * 4 + rr) * 64 + lane];
          for (int k = 1; k < KW; k++) v += red[(((k * NTW + nt) * MT + mt) * 4 + rr) * 64 + lane];
          acc[mt][rr] = v;
        }
  }
  const double post = FMT == Q4 ? 0.0625 : 1.0;  // Q4 codes entered the MFMA as 16*q
  const int n0 = ntile * 16 + 4 * quarter;       // the lane's first column

  if (o.epi == EPI_SWIGLU) {
    // NTW = 4g: each group of four n-tiles gate(2b), up(2b), gate(2b+1), up(2b+1) gives the 32
    // columns 32b.. of a = silu(gate) * up, one A8 group per row
    constexpr int WC = NTW * 16, AC = NTW * 8;
    __syncthreads();
    float* G = (float*)smem;  // [MR][WC]
    if (fin && active)
#pragma unroll
      for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int rr = 0; rr < 4; rr++) G[(mt * 16 + col) * WC + nt * 16 + 4 * quarter + rr] = (float)(acc[mt][rr] * post);
    __syncthreads();
    const int I = N >> 1;
    for (int i = tid; i < MR * AC; i += NT) {
      const int ml = i / AC, j = i % AC, m = m0 + ml;
      if (m >= Mpad) break;  // whole 32-lane groups leave together (AC is a multiple of 32)
      const int jj = j & 31;
      const int gc = (j >> 5) * 64 + (jj >> 4) * 32 + (jj & 15);
      const double g = G[ml * WC + gc], u = G[ml * WC + gc + 16];
      const float av2 = (float)(g / (1.0 + exp(-g)) * u);
      const int c = nb * AC + j;
      if (o.xq)
        emit_a8(av2, (size_t)m * I + c, o.xq, o.dxT, (size_t)(c >> 5) * Mpad + m, lane);
      else
        o.xf[(size_t)m * I + c] = av2;
    }
    return;
  }
  if (!fin || !active) return;
#pragma unroll
  for (int mt = 0; mt < MT; mt++) {
    const int m = m0 + mt * 16 + col;
    if (o.epi == EPI_F64) {
      if (m < Mpad)
#pragma unroll
        for (int rr = 0; rr < 4; rr++) ((double*)o.y)[(size_t)m * N + n0 + rr] = acc[mt][rr] * post;
    } else if (o.epi == EPI_F32) {
      if (m < o.m_store)
#pragma unroll
        for (int rr = 0; rr < 4; rr++) ((float*)o.y)[(size_t)m * o.ld + n0 + rr] = (float)(acc[mt][rr] * post);
    } else {  // EPI_RESID: h += f32(v), and the n-tile's share of each row's sum of squares
      double sq = 0.0;
      if (m < o.M) {
#pragma unroll
        for (int rr = 0; rr < 4; rr++) {
          const float hv = o.h[(size_t)m * N + n0 + rr] + (float)(acc[mt][rr] * post);
          o.h[(size_t)m * N + n0 + rr] = hv;
          sq += (double)hv * (double)hv;
        }
      }
      sq = cross4_sum_f64(sq);  // the four quarters hold the n-tile's other columns of row m
      if (quarter == 0 && m < Mpad) o.ssq[(size_t)m * (N >> 4) + ntile] = sq;
    }
  }
}

template <int FMT, int MT, int NTW, int KW>
static hipError_t gemm_rows_inst(const void* W, int N, int K, const int8_t* xq, const float* dxT, const GemmOut& o,
                                 hipStream_t st) {
  using CH = RowsChunk<MT, KW>;
  size_t lds = 2 * (size_t)CH::BYTES;
  const size_t red = KW > 1 ? (size_t)KW * NTW * MT * 4 * 64 * 8 : 0;
  const size_t swg = (size_t)CH::MR * NTW * 16 * 4;
  if (red > lds) lds = red;
  if (swg > lds) lds = swg;
  if (lds > max_dynamic_lds()) return hipErrorInvalidValue;
  const void* kern = (const void*)k_gemm_rows<FMT, MT, NTW, KW>;
  hipError_t e = allow_lds(kern, lds);
  if (e != hipSuccess) return e;
  const int RG = (o.Mpad + CH::MR - 1) / CH::MR;
  const int nblocks = (N / 16 + NTW - 1) / NTW;
  dim3 grid((unsigned)((nblocks + 7) / 8 * 8 * RG));
  hipLaunchKernelGGL((k_gemm_rows<FMT, MT, NTW, KW>), grid, dim3(512), lds, st, (const uint8_t*)W, N, K, xq, dxT, RG,
                     o);
  return hipGetLastError();
}

// Shape of a product of more than 16 rows: 32 rows per workgroup; eight n-tiles x one k-wave
// where there are many n-tiles (and for SwiGLU, which needs whole groups of four), else two
// n-tiles x four k-waves so a product with few n-tiles still fills the chip.  At 32 rows the
// kernel stays within 128 registers, so two workgroups share a CU and one's start (its first
// weights) overlaps the other's stream; 64-row workgroups (one a CU) measured 6% slower on the
// batched forward, 16-row ones 8% slower.  Batched, per forward: eight n-tiles x one k-wave
// for the head 418 µs against 448 with four x two (gate|up the same); four x two for the
// others 159 / 122 / 276 µs (qkv, o, down) against 144 / 110 / 230 with two x four.
template <int FMT>
static hipError_t gemm_rows_fmt(const void* W, int N, int K, const int8_t* xq, const float* dxT, const GemmOut& o,
                                hipStream_t st) {
  const bool wide = o.epi == EPI_SWIGLU || N / 16 >= 2048;
  if (o.Mpad <= 16)
    return wide ? gemm_rows_inst<FMT, 1, 8, 1>(W, N, K, xq, dxT, o, st) : gemm_rows_inst<FMT, 1, 1, 8>(W, N, K, xq, dxT, o, st);
  return wide ? gemm_rows_inst<FMT, 2, 8, 1>(W, N, K, xq, dxT, o, st) : gemm_rows_inst<FMT, 2, 2, 4>(W, N, K, xq, dxT, o, st);
}

static int ceil_div(int a, int b) { return (a + b - 1) / b; }

// rows one workgroup takes: 16 for up to 16 rows; more rows are split into groups of 16 (or 32
// rows for products whose workgroups hold four n-tiles), each its own workgroup, so the
// activations a workgroup stages stay small and the weights are shared through the caches
static int gemm_mt(int Mpad, int layout) {
  if (Mpad <= 16) return 1;
  return layout == 1 ? 1 : 2;
}

int gemm_layout(int N, int Mpad, int epi) {
  // more than 16 rows already give a product with few n-tiles several workgroups per n-block
  // (one per row group): four n-tiles x two k-waves then beats splitting K eight ways
  if (Mpad > 16 && epi != EPI_SWIGLU && N / 16 < 2048) return 0;
  // 16 rows and many n-tiles (the head, gate|up): eight n-tiles a workgroup, one wave each,
  // stage the activations once for twice the weights
  if (Mpad <= 16 && N / 16 >= 1024) return 3;
  // thousands of n-tiles (the head, gate|up) stream without splitting K much; a product with
  // few n-tiles splits K over eight (four) waves so every CU has about eight waves in flight
  if (epi == EPI_SWIGLU) return 0;
  return N / 16 >= 2048 ? 2 : 1;
}

template <int FMT, int MT, int NTW, int KW>
static hipError_t gemm_inst(const void* W, int N, int K, const int8_t* xq, const float* dxT, const GemmOut& o,
                            hipStream_t st) {
  constexpr int MR = MT * 16, STEP = Ring<MT, KW>::step;
  // LDS of a chunk of kcb k-blocks: MR rows of kcb*128 codes (+16 B row padding) and kcb*4*MR
  // scales.  About 76 KB so two workgroups share a CU; a workgroup of eight n-tiles (one per CU
  // by its registers) may take 96 KB for its f64 scales
  constexpr size_t DXB = sizeof(typename DxType<NTW>::T);
  constexpr size_t BUDGET = (NTW == 8 ? 96 : 76) * 1024;
  constexpr size_t PER_KB = (size_t)MR * 128 + 4 * MR * DXB;
  constexpr int KCB_FULL = (int)((BUDGET - (size_t)MR * 16 - 16) / PER_KB) / STEP * STEP;
  constexpr int KCB = KCB_FULL < STEP ? STEP : KCB_FULL;
  const int KB = K / 128;
  const int kcb = KCB > KB ? KB : KCB;
  size_t lds = (size_t)MR * (kcb * 128 + 16) + ((size_t)kcb * 4 * MR + 1) * DXB;  // + the scales' spare slot
  const size_t red = KW > 1 ? (size_t)KW * NTW * MT * 4 * 64 * 8 : 0;  // every k-wave's partials
  const size_t swg = (size_t)MR * NTW * 16 * 4;
  if (red > lds) lds = red;
  if (swg > lds) lds = swg;
  if (lds > max_dynamic_lds()) return hipErrorInvalidValue;
  // whole chunks of whole ring turns take the unrolled kernel
  const bool unrolled = kcb == KCB && KCB % STEP == 0;
  const int RG = ceil_div(o.Mpad, MR);
  dim3 grid((unsigned)(ceil_div(N / 16, NTW) * RG));
  auto go = [&](auto conv) -> hipError_t {
    constexpr bool CV = decltype(conv)::value;
    const void* kern = unrolled ? (const void*)k_gemm_q<FMT, MT, NTW, KW, KCB / STEP, CV>
                                : (const void*)k_gemm_q<FMT, MT, NTW, KW, 0, CV>;
    hipError_t e = allow_lds(kern, lds);
    if (e != hipSuccess) return e;
    if (unrolled)
      hipLaunchKernelGGL((k_gemm_q<FMT, MT, NTW, KW, KCB / STEP, CV>), grid, dim3(64 * NTW * KW), lds, st,
                         (const uint8_t*)W, N, K, xq, dxT, kcb, RG, o);
    else
      hipLaunchKernelGGL((k_gemm_q<FMT, MT, NTW, KW, 0, CV>), grid, dim3(64 * NTW * KW), lds, st, (const uint8_t*)W,
                         N, K, xq, dxT, kcb, RG, o);
    return hipSuccess;
  };
  const hipError_t e = o.epi == EPI_CONV ? go(std::true_type()) : go(std::false_type());
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

template <int FMT, int MT>
static hipError_t gemm_mt_inst(int layout, const void* W, int N, int K, const int8_t* xq, const float* dxT,
                               const GemmOut& o, hipStream_t st) {
  if (layout == 0) return gemm_inst<FMT, MT, 4, 2>(W, N, K, xq, dxT, o, st);
  if (layout == 2) return gemm_inst<FMT, MT, 4, 1>(W, N, K, xq, dxT, o, st);
  if (layout == 3) return gemm_inst<FMT, MT, 8, 1>(W, N, K, xq, dxT, o, st);
  if constexpr (MT == 1)
    if (o.Mpad == 16 && o.epi != EPI_CONV) return gemm_ks_inst<FMT>(W, N, K, xq, dxT, o, st);
  if constexpr (MT <= 2)
    return gemm_inst<FMT, MT, 1, 8>(W, N, K, xq, dxT, o, st);
  else
    return gemm_inst<FMT, MT, 2, 4>(W, N, K, xq, dxT, o, st);
}

template <int FMT>
static hipError_t gemm_fmt(int layout, const void* W, int N, int K, const int8_t* xq, const float* dxT,
                           const GemmOut& o, hipStream_t st) {
  if (gemm_mt(o.Mpad, layout) == 1) return gemm_mt_inst<FMT, 1>(layout, W, N, K, xq, dxT, o, st);
  return gemm_mt_inst<FMT, 2>(layout, W, N, K, xq, dxT, o, st);
}

hipError_t launch_gemm_q(int fmt, const void* W, int N, int K, const int8_t* xq, const float* dxT, int layout,
                         const GemmOut& o, hipStream_t st) {
  if (N % 16 || K % 128 || o.Mpad % 16 || o.Mpad < 16 || o.Mpad > 128 || o.M > o.Mpad) return hipErrorInvalidValue;
  if (o.epi == EPI_SWIGLU && (N % 64 || (!o.xq && !o.xf) || (o.xq && !o.dxT))) return hipErrorInvalidValue;
  if ((o.epi == EPI_F64 || o.epi == EPI_F32) && !o.y) return hipErrorInvalidValue;
  if ((o.epi == EPI_RESID || o.epi == EPI_CONV) && (!o.h || !o.ssq)) return hipErrorInvalidValue;
  if (o.epi == EPI_CONV && (!o.cd || !o.cbase || o.cB < 1 || 16 % o.cB || o.cgs < 1 || N % o.cgs || o.ckn < 1))
    return hipErrorInvalidValue;  // a block's rows within every 16-row group
  // more than 16 rows: the row kernel (every weight superblock read once per 32 rows), unless a
  // specific layout is asked for or the epilogue is a row convolution's
  if ((layout < 0 && o.Mpad > 16 && o.epi != EPI_CONV) || layout == 8) {
    if (fmt == Q4) return gemm_rows_fmt<Q4>(W, N, K, xq, dxT, o, st);
    if (fmt == Q8) return gemm_rows_fmt<Q8>(W, N, K, xq, dxT, o, st);
    return hipErrorInvalidValue;
  }
  if (layout < 0) layout = gemm_layout(N, o.Mpad, o.epi);
  if (o.epi == EPI_SWIGLU && layout != 0 && layout != 3) layout = 0;  // whole groups of four n-tiles
  if (o.epi == EPI_SWIGLU && layout == 3 && N % 128) layout = 0;
  if (fmt == Q4) return gemm_fmt<Q4>(layout, W, N, K, xq, dxT, o, st);
  if (fmt == Q8) return gemm_fmt<Q8>(layout, W, N, K, xq, dxT, o, st);
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
