// Candidate selection on the device (cortiq-engine "dflash.rs": top_k and
// Drafter::select_with): each draft row's top candidates from its logits, then the greedy
// left-to-right re-scoring against the token chosen before it, so only the chosen tokens (not
// the logits) need to leave the GPU.
//
// Top-k order: larger value first, the earlier index first among equal values -- the order in
// which the pages' insertion list keeps its entries.  A row is cut into chunks of 4096; a
// workgroup finds a chunk's top T (each wave its own through a threshold and a sort across the
// lanes, then wave 0 over the waves' lists), and a second kernel merges the chunks' lists the
// same way.  Elements compare as 64-bit keys, so every step is exact.  The re-scoring repeats the pages' f32 arithmetic term by term, in their order and
// without contraction, so its decisions are those of the reference evaluation.
#include "common.h"
#include "lanes.h"

namespace dfl {

constexpr int TK_THREADS = 256;
constexpr int TK_PER = 16;                       // elements each thread owns
constexpr int TK_CHUNK = TK_THREADS * TK_PER;   // elements of one chunk

// An element as one 64-bit key whose unsigned order is the top-k order: the high word is the
// value's bits made monotone (-0 first made +0, so it ties with +0 as a float compare does), the
// low word 0xffffffff - index, so among equal values the earlier index is larger.  Key 0: empty.
__device__ __forceinline__ unsigned long long topk_key(float v, int i) {
  const unsigned b = __float_as_uint(v + 0.0f);
  const unsigned o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((unsigned long long)o << 32) | (0xffffffffu - (unsigned)i);
}
__device__ __forceinline__ void topk_decode(unsigned long long k, float& v, int& i) {
  const unsigned o = (unsigned)(k >> 32);
  v = k ? __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o) : -INFINITY;
  i = k ? (int)(0xffffffffu - (unsigned)k) : -1;
}

// T rounds of a wave-wide maximum over every lane's keys; the winner is cleared where it sits
// (indices are distinct), and round t's winner goes to out[t] (0: the round found nothing).
template <int PER>
__device__ __forceinline__ void wave_top(unsigned long long (&key)[PER], int T, unsigned long long* out) {
  const int lane = threadIdx.x & 63;
  for (int t = 0; t < T; t++) {
    unsigned long long best = 0;
#pragma unroll
    for (int e = 0; e < PER; e++) best = key[e] > best ? key[e] : best;
    best = wave_max_u64(best);
#pragma unroll
    for (int e = 0; e < PER; e++) key[e] = key[e] == best ? 0ull : key[e];
    if (lane == 0) out[t] = best;
  }
}

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int m) {
  const int lo = __shfl_xor((int)(unsigned)v, m), hi = __shfl_xor((int)(unsigned)(v >> 32), m);
  return ((unsigned long long)(unsigned)hi << 32) | (unsigned)lo;
}

// The wave's 64 keys (one a lane) sorted largest first across the lanes by a bitonic network:
// blocks of k lanes alternate direction, so each merge step sees a bitonic sequence; in the
// last (k = 64) every lower partner keeps the larger key.
__device__ __forceinline__ unsigned long long wave_sort_desc(unsigned long long v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1)
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const unsigned long long o = shfl_xor_u64(v, j);
      const bool keep_max = ((lane & j) == 0) == ((lane & k) == 0);
      v = keep_max ? (o > v ? o : v) : (o < v ? o : v);
    }
  return v;
}

// The wave's top T (T <= 64) through a threshold: the T-th largest of the lanes' maxima is at
// most the T-th largest key (those T maxima are T distinct keys), so the wave's top T are among
// the keys at least that large -- usually a few dozen.  Those are gathered (cand, 64 keys of
// LDS), sorted across the lanes, and the first T written to out[0..T).  More than 64 of them
// (many of the top keys in a few lanes), or T > 64: the rounds of wave_top instead.
template <int PER>
__device__ __forceinline__ void wave_top_fast(unsigned long long (&key)[PER], int T, unsigned long long* out,
                                              unsigned long long* cand) {
  const int lane = threadIdx.x & 63;
  if (T > 64) {
    wave_top<PER>(key, T, out);
    return;
  }
  unsigned long long m = 0;
#pragma unroll
  for (int e = 0; e < PER; e++) m = key[e] > m ? key[e] : m;
  const unsigned long long sm = wave_sort_desc(m);
  const unsigned th_lo = __builtin_amdgcn_readlane((unsigned)sm, T - 1);
  const unsigned th_hi = __builtin_amdgcn_readlane((unsigned)(sm >> 32), T - 1);
  const unsigned long long th = ((unsigned long long)th_hi << 32) | th_lo;
  int base = 0;
#pragma unroll
  for (int e = 0; e < PER; e++) {  // every nonempty key >= th gets a slot, in lane order
    const bool take = key[e] != 0ull && key[e] >= th;
    const unsigned long long bal = __builtin_amdgcn_ballot_w64(take);
    const int slot = base + (int)__builtin_amdgcn_mbcnt_hi((unsigned)(bal >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)bal, 0));
    if (take && slot < 64) cand[slot] = key[e];
    base += __builtin_popcountll(bal);
  }
  if (base > 64) {  // uniform: base is the same in every lane
    wave_top<PER>(key, T, out);
    return;
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");  // the lanes' stores before their loads
  const unsigned long long v = wave_sort_desc(lane < base ? cand[lane] : 0ull);
  if (lane < T) out[lane] = v;
}

// The top T of the keys of the whole workgroup: each wave finds its own top T, then wave 0
// finds the top T of those 4T keys (one sort when 4T <= 64).  Written by the first T lanes of
// wave 0 to out_v, out_i (index -1 where there are fewer than T elements).
__device__ void block_top(unsigned long long (&key)[TK_PER], int T, float* out_v, int* out_i) {
  constexpr int NW = TK_THREADS / 64;
  __shared__ unsigned long long lk[NW][64];
  __shared__ unsigned long long cand[NW][64];
  __shared__ unsigned long long ok[64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  wave_top_fast<TK_PER>(key, T, lk[wave], cand[wave]);
  __syncthreads();
  if (wave != 0) return;
  if (NW * T <= 64) {
    const int w = min(lane / T, NW - 1), t = lane % T;
    const unsigned long long v = wave_sort_desc(lane < NW * T ? lk[w][t] : 0ull);
    if (lane < T) topk_decode(v, out_v[lane], out_i[lane]);
    return;
  }
  unsigned long long ck[NW];
#pragma unroll
  for (int k = 0; k < NW; k++) {
    const int j = lane + 64 * k, w = min(j / T, NW - 1), t = j % T;
    ck[k] = j < NW * T ? lk[w][t] : 0ull;
  }
  wave_top<NW>(ck, T, ok);
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");  // lane 0's stores before the lanes' loads
  if (lane < T) topk_decode(ok[lane], out_v[lane], out_i[lane]);
}

// Grid (chunks, rows): the top T of elements [c*4096, (c+1)*4096) of row r.
__global__ __launch_bounds__(TK_THREADS) void k_topk_chunk(const float* __restrict__ x, int width, int ld, int T,
                                                          float* __restrict__ pv, int* __restrict__ pi) {
  const int c = blockIdx.x, r = blockIdx.y, nch = gridDim.x, tid = threadIdx.x;
  unsigned long long key[TK_PER];
#pragma unroll
  for (int e = 0; e < TK_PER; e++) {
    const int i = c * TK_CHUNK + e * TK_THREADS + tid;
    const float v = x[(size_t)r * ld + min(i, width - 1)];
    key[e] = i < width ? topk_key(v, i) : 0ull;
  }
  const size_t o = ((size_t)r * nch + c) * T;
  block_top(key, T, pv + o, pi + o);
}

// Grid (rows): the top T of a row from its chunks' lists (nch * T <= 4096 entries).
__global__ __launch_bounds__(TK_THREADS) void k_topk_merge(const float* __restrict__ pv, const int* __restrict__ pi,
                                                          int nch, int T, float* __restrict__ vals,
                                                          int* __restrict__ idx) {
  const int r = blockIdx.x, tid = threadIdx.x, n = nch * T;
  unsigned long long key[TK_PER];
#pragma unroll
  for (int e = 0; e < TK_PER; e++) {
    const int j = min(e * TK_THREADS + tid, n - 1);
    const int i = pi[(size_t)r * n + j];
    const float v = pv[(size_t)r * n + j];
    key[e] = e * TK_THREADS + tid < n && i >= 0 ? topk_key(v, i) : 0ull;
  }
  block_top(key, T, vals + (size_t)r * T, idx + (size_t)r * T);
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

bool top_k_fits(int width, int T) { return (long)((width + TK_CHUNK - 1) / TK_CHUNK) * T <= TK_CHUNK; }

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

// The same re-scoring computed for every predecessor a row can have, then a chain of look-ups.
// Row j's predecessor is the anchor (j = 0) or one of the T candidates of row j-1, so a
// workgroup per row forms the score of every (predecessor option p, candidate c) pair with the
// pages' arithmetic: pc = pred[p] * hp[j] (an f32 product per term), then candidate c's logit +
// the f32 sum of pc[r] * succ[c][r] from r = 0 upward.  One thread a pair, so the T*T sequential
// sums run side by side.  A single wave then walks the rows: the first largest score among
// scores[j][prev] names row j's choice, which is row j+1's predecessor option.
constexpr int SELP_THREADS = 256;
size_t select_par_lds_bytes(int T, int rank) {
  return (size_t)T * rank * 2 * 2 + (size_t)T * rank * 4 + (size_t)rank * 4 + (size_t)T * 8 * 2;
}
__global__ __launch_bounds__(SELP_THREADS) void k_select_scores(const float* __restrict__ cv,
                                                               const int* __restrict__ ci, int T,
                                                               const float* __restrict__ hp, int rank,
                                                               const uint16_t* __restrict__ pred,
                                                               const uint16_t* __restrict__ succ, int anchor,
                                                               float* __restrict__ scores) {
#pragma clang fp contract(off)
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int j = blockIdx.x, tid = threadIdx.x, np = j ? T : 1;
  uint16_t* PV = (uint16_t*)lds;                // [np][rank] predecessor rows
  uint16_t* SU = PV + (size_t)T * rank;         // [T][rank] successor rows
  float* PC = (float*)(SU + (size_t)T * rank);  // [np][rank]
  float* HP = PC + (size_t)T * rank;            // [rank]
  int* PT = (int*)(HP + rank);                  // [T] predecessor tokens
  int* ST = PT + T;                             // [T] candidate tokens
  if (tid < T) {
    PT[tid] = j ? max(ci[(j - 1) * T + tid], 0) : anchor;  // -1 only from non-finite logits
    ST[tid] = max(ci[j * T + tid], 0);
  }
  for (int r = tid; r < rank; r += SELP_THREADS) HP[r] = hp[(size_t)j * rank + r];
  __syncthreads();
  for (int e = tid; e < np * rank; e += SELP_THREADS) PV[e] = pred[(size_t)PT[e / rank] * rank + e % rank];
  for (int e = tid; e < T * rank; e += SELP_THREADS) SU[e] = succ[(size_t)ST[e / rank] * rank + e % rank];
  __syncthreads();
  for (int e = tid; e < np * rank; e += SELP_THREADS) PC[e] = f16_bits_to_f32(PV[e]) * HP[e % rank];
  __syncthreads();
  for (int e = tid; e < np * T; e += SELP_THREADS) {
    const int pp = e / T, c = e % T;
    const float* pc = PC + (size_t)pp * rank;
    const uint16_t* su = SU + (size_t)c * rank;
    float sum = 0.0f;
    for (int r = 0; r < rank; r++) {
      const float prod = pc[r] * f16_bits_to_f32(su[r]);  // rounded on its own (no contraction here)
      sum = sum + prod;
    }
    scores[((size_t)j * T + pp) * T + c] = cv[j * T + c] + sum;
  }
}

// One wave: row by row, the first largest of scores[j][prev][0..T) (prev: 0 for row 0, then the
// previous row's choice).  The scores are first copied to LDS when they fit (STAGE), so each
// step of the chain waits for LDS, not memory.
constexpr int CHAIN_THREADS = 256;
template <bool STAGE>
__global__ __launch_bounds__(CHAIN_THREADS) void k_select_chain(const float* __restrict__ scores,
                                                               const int* __restrict__ ci, int rows, int T,
                                                               int* __restrict__ chosen, int* __restrict__ plain) {
  extern __shared__ float sl[];
  __shared__ int cl[16 * 64];
  const int tid = threadIdx.x, lane = tid & 63;
  const float* S = scores;
  const int* C = ci;
  if (STAGE) {  // all threads copy, eight loads each in flight; the candidate lists too
    for (int e = tid; e < rows * T; e += CHAIN_THREADS) cl[e] = ci[e];
    C = cl;
    const int n = rows * T * T;
    for (int base = tid; base < n; base += CHAIN_THREADS * 8) {
      float v[8];
#pragma unroll
      for (int b = 0; b < 8; b++) v[b] = scores[min(base + b * CHAIN_THREADS, n - 1)];
#pragma unroll
      for (int b = 0; b < 8; b++)
        if (base + b * CHAIN_THREADS < n) sl[base + b * CHAIN_THREADS] = v[b];
    }
    __syncthreads();
    S = sl;
  }
  if (tid >= 64) return;
  int prev = 0;
  for (int j = 0; j < rows; j++) {
    const float sc0 = lane < T ? S[((size_t)j * T + prev) * T + lane] : -INFINITY;  // T <= 64
    float sc = sc0;
    int c = lane;  // lanes >= T hold -inf behind every candidate
    wave_argmax(sc, c);
    c = c < T ? c : 0;  // (only a NaN score could leave a lane past T on top)
    if (lane == 0) {
      chosen[j] = max(C[j * T + c], 0);
      plain[j] = C[j * T];
    }
    prev = c;
  }
}

size_t select_scratch(int rows, int T) { return (size_t)rows * T * T * 4; }

hipError_t launch_select(const float* cv, const int* ci, int rows, int T, const float* hp, int rank,
                         const uint16_t* pred, const uint16_t* succ, int anchor, int* chosen, int* plain,
                         float* scores, hipStream_t st) {
  if (T < 1 || T > 64 || rank < 1 || (size_t)rank * 4 > 48 * 1024) return hipErrorInvalidValue;
  const size_t lds = select_par_lds_bytes(T, rank);
  if (scores && lds <= max_dynamic_lds()) {
    hipError_t e = allow_lds((const void*)k_select_scores, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_select_scores, dim3(rows), dim3(SELP_THREADS), lds, st, cv, ci, T, hp, rank, pred, succ,
                       anchor, scores);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t sb = select_scratch(rows, T);
    if (sb <= 48 * 1024 && rows * T <= 16 * 64)
      hipLaunchKernelGGL(k_select_chain<true>, dim3(1), dim3(CHAIN_THREADS), sb, st, scores, ci, rows, T, chosen, plain);
    else
      hipLaunchKernelGGL(k_select_chain<false>, dim3(1), dim3(CHAIN_THREADS), 0, st, scores, ci, rows, T, chosen, plain);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_select, dim3(1), dim3(SEL_THREADS), (size_t)rank * 4, st, cv, ci, rows, T, hp, rank, pred, succ,
                     anchor, chosen, plain);
  return hipGetLastError();
}

}  // namespace dfl
