// Candidate selection on the device (cortiq-engine "dflash.rs": top_k and
// Drafter::select_with): each draft row's top candidates from its logits, then the greedy
// left-to-right re-scoring against the token chosen before it, so only the chosen tokens (not
// the logits) need to leave the GPU.
//
// Top-k order: larger value first, the earlier index first among equal values -- the order in
// which the pages' insertion list keeps its entries.  A row is cut into chunks of 4096; a
// workgroup finds a chunk's top T by T rounds of a workgroup-wide arg-max (each thread owns 16
// elements and a mask of those already taken), and a second kernel merges the chunks' lists the
// same way.  The re-scoring repeats the pages' f32 arithmetic term by term, in their order and
// without contraction, so its decisions are those of the reference evaluation.
#include "common.h"

namespace dfl {

constexpr int TK_THREADS = 256;
constexpr int TK_PER = 16;                       // elements each thread owns
constexpr int TK_CHUNK = TK_THREADS * TK_PER;   // elements of one chunk

__device__ __forceinline__ bool better(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

// T rounds of a workgroup arg-max over the (v[e], ix[e]) of every thread (ix < 0: empty).
// Round t's winner is written by thread 0 to out_v[t], out_i[t].
__device__ void block_top(const float (&v)[TK_PER], const int (&ix)[TK_PER], int T, float* out_v, int* out_i) {
  __shared__ float wv[2][TK_THREADS / 64];
  __shared__ int wi[2][TK_THREADS / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  unsigned taken = 0;
  for (int t = 0; t < T; t++) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int e = 0; e < TK_PER; e++)
      if (ix[e] >= 0 && !((taken >> e) & 1u) && better(v[e], ix[e], bv, bi)) {
        bv = v[e];
        bi = ix[e];
      }
#pragma unroll
    for (int o = 32; o; o >>= 1) {
      const float ov = __shfl_xor(bv, o);
      const int oi = __shfl_xor(bi, o);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    const int slot = t & 1;  // alternate buffers: one barrier per round
    if (lane == 0) {
      wv[slot][wave] = bv;
      wi[slot][wave] = bi;
    }
    __syncthreads();
    bv = wv[slot][0];
    bi = wi[slot][0];
#pragma unroll
    for (int w = 1; w < TK_THREADS / 64; w++)
      if (better(wv[slot][w], wi[slot][w], bv, bi)) {
        bv = wv[slot][w];
        bi = wi[slot][w];
      }
#pragma unroll
    for (int e = 0; e < TK_PER; e++)
      if (ix[e] == bi) taken |= 1u << e;
    if (tid == 0) {  // a round that found nothing (a short chunk) leaves index -1
      out_v[t] = bv;
      out_i[t] = bi == 0x7fffffff ? -1 : bi;
    }
  }
}

// Grid (chunks, rows): the top T of elements [c*4096, (c+1)*4096) of row r.
__global__ __launch_bounds__(TK_THREADS) void k_topk_chunk(const float* __restrict__ x, int width, int ld, int T,
                                                          float* __restrict__ pv, int* __restrict__ pi) {
  const int c = blockIdx.x, r = blockIdx.y, nch = gridDim.x, tid = threadIdx.x;
  float v[TK_PER];
  int ix[TK_PER];
#pragma unroll
  for (int e = 0; e < TK_PER; e++) {
    const int i = c * TK_CHUNK + e * TK_THREADS + tid;
    ix[e] = i < width ? i : -1;
    v[e] = i < width ? x[(size_t)r * ld + i] : -INFINITY;
  }
  const size_t o = ((size_t)r * nch + c) * T;
  block_top(v, ix, T, pv + o, pi + o);
}

// Grid (rows): the top T of a row from its chunks' lists (nch * T <= 4096 entries).
__global__ __launch_bounds__(TK_THREADS) void k_topk_merge(const float* __restrict__ pv, const int* __restrict__ pi,
                                                          int nch, int T, float* __restrict__ vals,
                                                          int* __restrict__ idx) {
  const int r = blockIdx.x, tid = threadIdx.x, n = nch * T;
  float v[TK_PER];
  int ix[TK_PER];
#pragma unroll
  for (int e = 0; e < TK_PER; e++) {
    const int j = e * TK_THREADS + tid;
    const bool ok = j < n && pi[(size_t)r * n + j] >= 0;
    ix[e] = ok ? pi[(size_t)r * n + j] : -1;
    v[e] = ok ? pv[(size_t)r * n + j] : -INFINITY;
  }
  block_top(v, ix, T, vals + (size_t)r * T, idx + (size_t)r * T);
}

hipError_t launch_top_k(const float* x, int rows, int width, int ld, int T, float* part_v, int* part_i, float* vals,
                        int* idx, hipStream_t st) {
  const int nch = (width + TK_CHUNK - 1) / TK_CHUNK;
  if (rows <= 0 || T < 1 || T > width || nch * T > TK_CHUNK) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_topk_chunk, dim3(nch, rows), dim3(TK_THREADS), 0, st, x, width, ld, T, part_v, part_i);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_topk_merge, dim3(rows), dim3(TK_THREADS), 0, st, part_v, part_i, nch, T, vals, idx);
  return hipGetLastError();
}

size_t top_k_scratch(int rows, int width, int T) {
  const size_t nch = (width + TK_CHUNK - 1) / TK_CHUNK;
  return 2 * ((rows * nch * T * 4 + 255) & ~(size_t)255);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// One workgroup: rows in order.  For row j: pc[r] = pred[prev][r] * hp[j][r]; candidate c's score
// is its logit + the f32 sum of pc[r] * succ[tok][r] from r = 0 upward (one thread a candidate);
// the first largest score wins and becomes prev.
constexpr int SEL_THREADS = 256;
__global__ __launch_bounds__(SEL_THREADS) void k_select(const float* __restrict__ cv, const int* __restrict__ ci,
                                                       int rows, int T, const float* __restrict__ hp, int rank,
                                                       const uint16_t* __restrict__ pred,
                                                       const uint16_t* __restrict__ succ, int anchor,
                                                       int* __restrict__ chosen, int* __restrict__ plain) {
#pragma clang fp contract(off)
  extern __shared__ float pc[];  // [rank]
  __shared__ float sc[64];
  __shared__ int prev_s;
  const int tid = threadIdx.x;
  if (tid == 0) prev_s = anchor;
  __syncthreads();
  for (int j = 0; j < rows; j++) {
    const int prev = prev_s;
    for (int r = tid; r < rank; r += SEL_THREADS)
      pc[r] = f16_bits_to_f32(pred[(size_t)prev * rank + r]) * hp[(size_t)j * rank + r];
    __syncthreads();
    if (tid < T) {
      const int tok = max(ci[(size_t)j * T + tid], 0);  // -1 only from non-finite logits: stay in bounds
      const uint16_t* s = succ + (size_t)tok * rank;
      float sum = 0.0f;
      for (int r = 0; r < rank; r++) {
        const float prod = pc[r] * f16_bits_to_f32(s[r]);  // rounded on its own (no contraction here)
        sum = sum + prod;
      }
      sc[tid] = cv[(size_t)j * T + tid] + sum;
    }
    __syncthreads();
    if (tid == 0) {
      float best = -INFINITY;
      int tok = max(ci[(size_t)j * T], 0);
      for (int c = 0; c < T; c++)
        if (sc[c] > best) {
          best = sc[c];
          tok = max(ci[(size_t)j * T + c], 0);
        }
      chosen[j] = tok;
      plain[j] = ci[(size_t)j * T];
      prev_s = tok;
    }
    __syncthreads();
  }
}

hipError_t launch_select(const float* cv, const int* ci, int rows, int T, const float* hp, int rank,
                         const uint16_t* pred, const uint16_t* succ, int anchor, int* chosen, int* plain,
                         hipStream_t st) {
  if (T < 1 || T > 64 || rank < 1 || (size_t)rank * 4 > 48 * 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_select, dim3(1), dim3(SEL_THREADS), (size_t)rank * 4, st, cv, ci, rows, T, hp, rank, pred, succ,
                     anchor, chosen, plain);
  return hipGetLastError();
}

}  // namespace dfl
