// Block-vs-context attention (cortiq-engine "dflash.rs", Drafter::block).  Query head j uses
// kv head j / rep.  Its key set is the layer's range [lo, hi) of context positions (the caller
// computes it) plus all of the block's own rows, with no causal mask among the block rows.  A
// windowed layer also hides, from block row r, the context positions below anchor + r + 1 - w.
// Scores are (q . k) * hd^-0.5, then a softmax over the key set and y = sum of p * v.
//
// The pages' device kernel (gpu_wgpu/dflash_dev.rs, dflash_attn) writes every score to a global
// scratch and re-reads it; here the context is split into chunks, each wave keeps a running
// (max, sum, acc) per query in registers (online softmax), and a merge combines the chunks.
// A workgroup serves one (sequence, kv head, chunk, q head of the group).  Its eight waves take
// the chunk's 16-key tiles in turn (wave w: tiles w, w + 8, ...), each straight from memory
// into registers with the next tile's keys and values in flight while the current one is
// computed, so the loop has no LDS staging and no barrier; the waves' (max, sum, acc) are then
// combined in LDS in wave order and written once.  The q heads sharing a kv head read the
// same tiles: their workgroups get ids 8 apart, which puts them on the same XCD (workgroups
// go round-robin over the eight), where the tiles come from one L2.  The chunks hold context
// rows only; the block's own 16 keys, a few thousand flops per (head, row), are scored by the
// merge, which then combines them with the chunks.  The 16 block rows of a head are the 16
// columns of v_mfma_f64_16x16x4f64 tiles:
//   S^T[key][q] = K . Q^T   (A = 16 keys, B = the head's queries)
//   Y^T[d][q]  += V^T . P^T (A = 16-dim slices of V, B = the probabilities, already in the
//                            accumulator layout of S^T)
// so the probabilities never leave registers.  Context K/V is f32 [slot][kvh][max_ctx][hd].
// Context K/V is f32 or, with an f16 cache, f16 [slot][kvh][max_ctx][hd]; either converts to f64
// exactly.
// Lane layout of the f64 16x16x4 MFMA: lane l gives A[l%16][l/16] and B[l/16][l%16] and holds
// D[l/16 + 4r][l%16] in accumulator slot r (rows interleaved, unlike the f32 16x16 forms).
//
// Scores, softmax and values are evaluated in f64 (the f32 keys, values and queries are exact
// in f64) and the output is rounded once to f32: it feeds an int8 quantizer, where a value one
// ulp off flips codes that the following layers amplify, so it has to be the correctly rounded
// result that any exact evaluation gives.
#include "common.h"
#include "digits.h"
#include "lanes.h"

namespace dfl {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef double v4d __attribute__((ext_vector_type(4)));

constexpr int ATTN_WAVES = 8;
constexpr int ATTN_THREADS = 64 * ATTN_WAVES;

// Chunks a sequence with n context rows takes (the block's own rows are the merge's part).
__device__ __forceinline__ int attn_chunks(int nctx, int ck) { return nctx > 0 ? (nctx + ck - 1) / ck : 0; }

// LDS of the combine: every wave's (max, sum, weight) per query and its acc, rows HD + 1 doubles
// apart, and one more (max, sum, weight) row for the common maximum
template <int HD>
constexpr size_t attn_comb_bytes() {
  return (size_t)ATTN_WAVES * 16 * (HD + 1) * 8 + (size_t)(ATTN_WAVES + 1) * 16 * 3 * 8;
}
// all of a workgroup's LDS: the combine, then the queries (16 rows of HD + 2 doubles)
template <int HD>
constexpr size_t attn_lds_bytes() {
  return attn_comb_bytes<HD>() + (size_t)16 * (HD + 2) * 8;
}

// Grid: ceil(tasks / 8) * 8 * rep workgroups for tasks (sequence, kv head, chunk) numbered
// t = (s * kvh + g) * maxn + c; id = (t / 8) * 8 * rep + h * 8 + t % 8 serves q head g*rep + h.
// Four cache elements of a row as loaded: f32 (16 bytes) or f16 (8 bytes, an f16 cache).
template <typename CT>
struct CacheVec;
template <>
struct CacheVec<float> {
  typedef float v4 __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ v4 load(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(v4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  }
};
template <>
struct CacheVec<_Float16> {
  typedef _Float16 v4 __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ v4 load(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(v4, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
  }
};

template <int HD, typename CT, bool WIN>
__global__ __launch_bounds__(ATTN_THREADS) void k_attn_partial(AttnShape a, SeqInfo si, int maxn,
                                                               const float* __restrict__ q,
                                                               const CT* __restrict__ kc,
                                                               const CT* __restrict__ vc,
                                                               double* __restrict__ part, double* __restrict__ ml) {
  constexpr int NI = HD / 16;  // 16-dim slices: k-steps of the scores, output tiles of the values
  constexpr int ND = HD / 64;  // 64-dim groups of a value row
  constexpr int HDP = HD + 1;  // LDS row of a wave's acc (odd, so the 16 query rows spread over banks)
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int rep = a.nh / a.kvh, per = 8 * rep;
  const int id = blockIdx.x, t = (id / per) * 8 + id % 8, h = (id % per) / 8;
  if (t >= si.n * a.kvh * maxn) return;  // the whole workgroup: padding of the last group of 8
  const int s = t / (a.kvh * maxn), g = (t / maxn) % a.kvh, c = t % maxn;
  const int nctx = si.nctx[s];
  if (c >= attn_chunks(nctx, a.ck)) return;  // the whole workgroup: this sequence has fewer chunks
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int quarter = lane >> 4, col = lane & 15;
  const int j = g * rep + h;
  const int k0 = c * a.ck, kend = min(nctx, k0 + a.ck);
  const int nt = (kend - k0 + 15) / 16;  // >= 1: every launched chunk holds context rows
  const CT* Kctx = kc + (((size_t)si.slot[s] * a.kvh + g) * a.max_ctx + si.ctx0[s]) * HD;
  const CT* Vctx = vc + (((size_t)si.slot[s] * a.kvh + g) * a.max_ctx + si.ctx0[s]) * HD;
  // under a window (WIN: some row of the call masks keys), query row col does not see the keys
  // before index mask0 + col: their scores become -1e300, so exp() gives them exactly 0 beside
  // any visible key; a chunk in which a row sees no key keeps the finite maximum -1e300, and the
  // merge weights it by exp(-1e300 - m) = 0
  const int kmin = si.mask0[s] + col;

  // the head's queries in LDS as f64 (converted once here, not once per tile; rows HD + 2
  // doubles apart, so the 16 rows of one read fall in different banks), the B operand of the
  // scores: q[row col][16*i4 + 4*quarter ..]
  constexpr int QS = HD + 2;
  double* Qs = (double*)(lds + attn_comb_bytes<HD>());
  for (int e = tid; e < 16 * HD / 4; e += ATTN_THREADS) {
    const int row = e / (HD / 4), c4 = e % (HD / 4);
    const int rr = min(row, a.B - 1);  // rows past B: a copy of the last (their results are not kept)
    const v4f qv = *(const v4f*)(q + ((size_t)(s * a.B + rr) * a.nh + j) * HD + 4 * c4);
    *(v4d*)(Qs + row * QS + 4 * c4) = (v4d){(double)qv[0], (double)qv[1], (double)qv[2], (double)qv[3]};
  }
  __syncthreads();
  double m_run = -INFINITY, l_run = 0.0;
  v4d acc[NI];
#pragma unroll
  for (int dt = 0; dt < NI; dt++) acc[dt] = (v4d){0.0, 0.0, 0.0, 0.0};

  // a tile's operands, loaded unconditionally (keys past the chunk are clamped to its last key:
  // their scores are masked, so their values are multiplied by 0):
  //   kr[i4]    = K[key0 + col][16*i4 + 4*quarter ..]           (A of the scores)
  //   vr[k][d4] = V[key0 + 4k + quarter][64*d4 + 4*col ..]      (A of the values, dims
  //               64*d4 + 4*col + e of output tile dt = 4*d4 + e)
  // (buffer loads: a plain load of read-only memory may be re-issued next to its use when
  // registers run short, which would take the next tile out of flight)
  typedef typename CacheVec<CT>::v4 v4c;
  constexpr int ES = (int)sizeof(CT);
  v4c kr[NI], vr[4][ND];
  const __amdgpu_buffer_rsrc_t kres = __builtin_amdgcn_make_buffer_rsrc((void*)Kctx, (short)0, kend * HD * ES, 0x00020000);
  const __amdgpu_buffer_rsrc_t vres = __builtin_amdgcn_make_buffer_rsrc((void*)Vctx, (short)0, kend * HD * ES, 0x00020000);
  auto load_k = [&](int i) {
    const int key = min(k0 + 16 * i + col, kend - 1);
#pragma unroll
    for (int i4 = 0; i4 < NI; i4++) kr[i4] = CacheVec<CT>::load(kres, (key * HD + 16 * i4 + 4 * quarter) * ES);
  };
  auto load_v = [&](int i) {
#pragma unroll
    for (int k = 0; k < 4; k++) {
      const int key = min(k0 + 16 * i + 4 * k + quarter, kend - 1);
#pragma unroll
      for (int d4 = 0; d4 < ND; d4++) vr[k][d4] = CacheVec<CT>::load(vres, (key * HD + 64 * d4 + 4 * col) * ES);
    }
  };
  const int last = nt - 1;
  // keys, then values, as in the loop (loads return in order: each wait then covers its own)
  load_k(min(w, last));
  __builtin_amdgcn_sched_barrier(0);
  load_v(min(w, last));
  __builtin_amdgcn_sched_barrier(0);
  for (int i = w; i < nt; i += ATTN_WAVES) {
    const int nvalid = min(16, kend - (k0 + 16 * i));  // keys of this tile
    v4d st0 = (v4d){0.0, 0.0, 0.0, 0.0}, st1 = st0;
#pragma unroll
    for (int i4 = 0; i4 < NI; i4++) {
      const v4d qv = *(const v4d*)(Qs + col * QS + 16 * i4 + 4 * quarter);
      st0 = __builtin_amdgcn_mfma_f64_16x16x4f64((double)kr[i4][0], qv[0], st0, 0, 0, 0);
      st1 = __builtin_amdgcn_mfma_f64_16x16x4f64((double)kr[i4][1], qv[1], st1, 0, 0, 0);
      st0 = __builtin_amdgcn_mfma_f64_16x16x4f64((double)kr[i4][2], qv[2], st0, 0, 0, 0);
      st1 = __builtin_amdgcn_mfma_f64_16x16x4f64((double)kr[i4][3], qv[3], st1, 0, 0, 0);
    }
    load_k(min(i + ATTN_WAVES, last));  // the next tile's keys travel during the softmax and values
    double p[4], mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int key = quarter + 4 * r;  // accumulator slot r holds key row quarter + 4r
      const double sc = (st0[r] + st1[r]) * (double)a.scale;
      p[r] = key < nvalid ? (!WIN || k0 + 16 * i + key >= kmin ? sc : -1e300) : -INFINITY;
      mx = fmax(mx, p[r]);
    }
    mx = cross4_max_f64(mx);  // the same query's slots in the other three lane rows
    const double m_new = fmax(m_run, mx);
    double ps = 0.0;
#pragma unroll
    for (int r = 0; r < 4; r++) {
      p[r] = exp(p[r] - m_new);
      ps += p[r];
    }
    ps = cross4_sum_f64(ps);
    // after the first tiles the running maxima rarely move; where none of the wave's does,
    // exp(m_run - m_new) is exactly 1, so the rescaling (an exact no-op then) is skipped
    if (__builtin_amdgcn_ballot_w64(m_new != m_run)) {
      const double corr = exp(m_run - m_new);
      l_run = l_run * corr + ps;
#pragma unroll
      for (int dt = 0; dt < NI; dt++) acc[dt] *= corr;
    } else {
      l_run = l_run + ps;
    }
    m_run = m_new;
    // step k pairs the probabilities of slot k with those keys' values; the NI output tiles are
    // independent, so consecutive MFMAs never wait on each other's result
#pragma unroll
    for (int k = 0; k < 4; k++) {
#pragma unroll
      for (int dt = 0; dt < NI; dt++)
        acc[dt] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)vr[k][dt >> 2][dt & 3], p[k], acc[dt], 0, 0, 0);
    }
    load_v(min(i + ATTN_WAVES, last));
  }

  // combine the waves in wave order: M = the largest maximum (wave 0 has tile 0, so M is
  // finite), e_w = exp(m_w - M) (0 for a wave without tiles), L = sum e_w l_w,
  // acc = sum e_w acc_w
  double* A = (double*)lds;                   // [wave][query][HDP]
  double* MLs = A + ATTN_WAVES * 16 * HDP;    // [wave][query]: m, l, then e (then M)
#pragma unroll
  for (int dt = 0; dt < NI; dt++)
#pragma unroll
    for (int r = 0; r < 4; r++)  // slot r of tile dt: dim 64*(dt/4) + 16r + 4*quarter + dt%4
      A[(w * 16 + col) * HDP + 64 * (dt >> 2) + 16 * r + 4 * quarter + (dt & 3)] = acc[dt][r];
  if (quarter == 0) {
    MLs[(w * 16 + col) * 3] = m_run;
    MLs[(w * 16 + col) * 3 + 1] = l_run;
  }
  __syncthreads();
  // one thread per (wave, query) takes that wave's weight, so the exps run side by side rather
  // than eight after another in one thread; M is kept in the row past the waves'
  if (tid < ATTN_WAVES * 16) {
    const int qr = tid & 15, v = tid >> 4;
    double M = -INFINITY;
    for (int u = 0; u < ATTN_WAVES; u++) M = fmax(M, MLs[(u * 16 + qr) * 3]);
    const double mv = MLs[(v * 16 + qr) * 3];
    MLs[(v * 16 + qr) * 3 + 2] = mv == -INFINITY ? 0.0 : exp(mv - M);
    if (v == 0) MLs[(ATTN_WAVES * 16 + qr) * 3] = M;
  }
  __syncthreads();
  if (tid < 16) {  // one thread per query: the sum, in wave order (the loop below reads only e)
    double L = 0.0;
    for (int v = 0; v < ATTN_WAVES; v++) L += MLs[(v * 16 + tid) * 3 + 1] * MLs[(v * 16 + tid) * 3 + 2];
    const size_t prow = ((((size_t)s * a.kvh + g) * a.maxch + c) * rep + h) * 16 + tid;
    if (tid < a.B) {
      ml[prow * 2] = MLs[(ATTN_WAVES * 16 + tid) * 3];
      ml[prow * 2 + 1] = L;
    }
  }
  for (int o = tid; o < 16 * HD; o += ATTN_THREADS) {
    const int qq = o / HD, d = o % HD;
    if (qq >= a.B) break;  // rows in order: the rest are past B too
    double y = 0.0;
#pragma unroll
    for (int v = 0; v < ATTN_WAVES; v++) y += A[(v * 16 + qq) * HDP + d] * MLs[(v * 16 + qq) * 3 + 2];
    const size_t prow = ((((size_t)s * a.kvh + g) * a.maxch + c) * rep + h) * 16 + qq;
    part[prow * HD + d] = y;
  }
}

// ---- the chunk partials with integer scores (head_dim 128, four q heads per kv head) ----
//
// The scores come from exact int8 digit splits (digits.h) of the queries (written by the q/k
// epilogue) and of the keys (written beside the cache by the append): q . k is 2^(Eq+Ek) *
// 128^-2 * sum_d 128^-d S_d over the diagonals d <= 6, each S_d an exact int32 sum of the digit
// pairs t + u = d, two v_mfma_i32_16x16x64_i8 per pair; the seven diagonals are combined in f64
// and scaled by hd^-0.5.  The softmax and the values stay f64, as in k_attn_partial, and the
// partials and their layout are the same, so the merge reads either.
//
// A workgroup serves one (sequence, kv head, chunk) with one wave per q head of the kv head, so
// each 16-key tile is read once for four heads: the key digits go from memory straight into LDS
// (buffer loads to LDS; 14 blocks of 1 KB, block 2u + hh holding plane u, dims 64hh + 16*quarter
// .. +16 of key col at lane position 16*quarter + col, the A operand's layout), the values are
// converted to f64 into LDS once, and the key exponents are kept there too.  The tiles are
// double-buffered: tile i + 1 lands while tile i is computed, and tile i + 2 is requested after
// the barrier that ends tile i.  A wave keeps its head's query digits in registers (the B
// operand) and runs every tile of the chunk, so its (max, sum, acc) is the chunk's partial.
constexpr int GQ_REP = 4, GQ_THREADS = 64 * GQ_REP;
constexpr int GQ_KD = 2 * DIG_T * 1024;           // one tile's key digits
constexpr int GQ_VS = 128 + 4;                    // LDS row of a value row, in doubles
constexpr int GQ_VB = 16 * GQ_VS * 8;             // one tile's values, bytes
constexpr int GQ_TILES = 2 * (GQ_KD + GQ_VB + 64);  // two buffers of digits, values, exponents
constexpr int GQ_STAGE = GQ_REP * 16 * 129 * 8;   // the partials' staging after the loop
constexpr size_t GQ_LDS = GQ_TILES > GQ_STAGE ? GQ_TILES : GQ_STAGE;

template <typename CT, bool WIN>
__global__ __launch_bounds__(GQ_THREADS, 2) void k_attn_gqa_dig(AttnShape a, SeqInfo si, int maxn,
                                                                const int8_t* __restrict__ qd,
                                                                const int* __restrict__ qe,
                                                                const CT* __restrict__ vc,
                                                                const int8_t* __restrict__ kd,
                                                                const int* __restrict__ ke,
                                                                double* __restrict__ part, double* __restrict__ ml) {
  constexpr int HD = 128, NI = HD / 16, ND = HD / 64;
  typedef int v4i __attribute__((ext_vector_type(4)));
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int task = blockIdx.x;
  if (task >= si.n * a.kvh * maxn) return;
  const int s = task / (a.kvh * maxn), g = (task / maxn) % a.kvh, c = task % maxn;
  const int nctx = si.nctx[s];
  if (c >= attn_chunks(nctx, a.ck)) return;  // the whole workgroup: this sequence has fewer chunks
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int quarter = lane >> 4, col = lane & 15;
  const int j = g * GQ_REP + w;
  const int k0 = c * a.ck, kend = min(nctx, k0 + a.ck);
  const int nt = (kend - k0 + 15) / 16;  // >= 1: every launched chunk holds context rows
  const size_t row0 = ((size_t)si.slot[s] * a.kvh + g) * a.max_ctx + si.ctx0[s];
  const CT* Vctx = vc + row0 * HD;
  const int kmin = si.mask0[s] + col;  // a window: query row col sees keys from here on

  // this head's query digits (rows past B: a copy of the last, whose results are not kept)
  v4i qdr[DIG_T][2];
  int eq;
  {
    const int rr = min(col, a.B - 1);
    const size_t qrow = (size_t)(s * a.B + rr) * a.nh + j;
    const int8_t* qp = qd + qrow * DIG_ROW + 16 * quarter;
#pragma unroll
    for (int t = 0; t < DIG_T; t++)
#pragma unroll
      for (int hh = 0; hh < 2; hh++) qdr[t][hh] = *(const v4i*)(qp + t * 128 + 64 * hh);
    eq = qe[qrow];
  }

  // tile buffers: [2][digits GQ_KD | values GQ_VB | exponents 16 ints]
  auto kbuf = [&](int b) { return lds + b * (GQ_KD + GQ_VB + 64); };
  typedef typename CacheVec<CT>::v4 v4c;
  constexpr int ES = (int)sizeof(CT);
  const __amdgpu_buffer_rsrc_t kdres = __builtin_amdgcn_make_buffer_rsrc((void*)(kd + row0 * DIG_ROW), (short)0, kend * DIG_ROW, 0x00020000);
  const __amdgpu_buffer_rsrc_t keres = __builtin_amdgcn_make_buffer_rsrc((void*)(ke + row0), (short)0, kend * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t vres = __builtin_amdgcn_make_buffer_rsrc((void*)Vctx, (short)0, kend * HD * ES, 0x00020000);
  v4c vl[2];
  int kel = 0;
  // tile i's loads: the digit blocks b = w, w + 4, .. (buffer loads to LDS), two 4-element
  // pieces of values per thread (registers), one exponent per thread of the first 16; keys past
  // the chunk clamped to its last key (masked below)
  auto gload = [&](int i) {
    uint8_t* B = kbuf(i & 1);
    const int keyk = min(k0 + 16 * i + col, kend - 1);
#pragma unroll
    for (int b = 0; b < 4; b++) {
      const int blk = w + 4 * b;
      if (blk < 2 * DIG_T)  // uniform
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kdres, (__attribute__((address_space(3))) void*)(B + blk * 1024), 16,
                                                 keyk * DIG_ROW + (blk >> 1) * 128 + 64 * (blk & 1) + 16 * quarter, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 2; u++) {
      const int p = tid + u * GQ_THREADS, row = p >> 5, c4 = p & 31;
      const int key = min(k0 + 16 * i + row, kend - 1);
      vl[u] = CacheVec<CT>::load(vres, (key * HD + 4 * c4) * ES);
    }
    if (tid < 16) kel = (int)__builtin_amdgcn_raw_buffer_load_b32(keres, min(k0 + 16 * i + tid, kend - 1) * 4, 0, 0);
  };
  auto lstore = [&](int i) {
    uint8_t* B = kbuf(i & 1);
    double* V = (double*)(B + GQ_KD);
#pragma unroll
    for (int u = 0; u < 2; u++) {
      const int p = tid + u * GQ_THREADS, row = p >> 5, c4 = p & 31;
      *(v4d*)(V + row * GQ_VS + 4 * c4) = (v4d){(double)vl[u][0], (double)vl[u][1], (double)vl[u][2], (double)vl[u][3]};
    }
    if (tid < 16) ((int*)(B + GQ_KD + GQ_VB))[tid] = kel;
  };
  // the loads to LDS are counted by vmcnt but not waited for by the compiler: every wave waits
  // for all of its loads before the barrier that publishes a tile (the memory clobber keeps the
  // LDS reads below it)
  auto publish = [&]() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  gload(0);
  lstore(0);
  if (nt > 1) gload(1);
  publish();

  double m_run = -INFINITY, l_run = 0.0;
  v4d acc[NI];
#pragma unroll
  for (int dt = 0; dt < NI; dt++) acc[dt] = (v4d){0.0, 0.0, 0.0, 0.0};
  for (int i = 0; i < nt; i++) {
    const uint8_t* B = kbuf(i & 1);
    const double* V = (const double*)(B + GQ_KD);
    const int* KE = (const int*)(B + GQ_KD + GQ_VB);
    const int nvalid = min(16, kend - (k0 + 16 * i));
    // the 28 digit pairs t + u <= 6, the pairs of one diagonal into one exact int32 sum
    v4i dacc[DIG_T];
#pragma unroll
    for (int d = 0; d < DIG_T; d++) dacc[d] = (v4i){0, 0, 0, 0};
#pragma unroll
    for (int hh = 0; hh < 2; hh++)
#pragma unroll
      for (int u = 0; u < DIG_T; u++) {
        const v4i kdv = *(const v4i*)(B + (2 * u + hh) * 1024 + lane * 16);
#pragma unroll
        for (int t = 0; t + u < DIG_T; t++)
          dacc[t + u] = __builtin_amdgcn_mfma_i32_16x16x64_i8(kdv, qdr[t][hh], dacc[t + u], 0, 0, 0);
      }
    // accumulator slot r: key 4*quarter + r, query col (int32 16x16 rows are contiguous)
    double p[4], mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int key = 4 * quarter + r;
      double S = (double)dacc[DIG_T - 1][r];
#pragma unroll
      for (int d = DIG_T - 2; d >= 0; d--) S = __builtin_fma(S, 0.0078125, (double)dacc[d][r]);
      const double sc = ldexp(S, eq + KE[key] - 14) * (double)a.scale;
      p[r] = key < nvalid ? (!WIN || k0 + 16 * i + key >= kmin ? sc : -1e300) : -INFINITY;
      mx = fmax(mx, p[r]);
    }
    mx = cross4_max_f64(mx);  // the same query's slots in the other three lane rows
    const double m_new = fmax(m_run, mx);
    double ps = 0.0;
#pragma unroll
    for (int r = 0; r < 4; r++) {
      p[r] = exp(p[r] - m_new);
      ps += p[r];
    }
    ps = cross4_sum_f64(ps);
    if (__builtin_amdgcn_ballot_w64(m_new != m_run)) {
      const double corr = exp(m_run - m_new);
      l_run = l_run * corr + ps;
#pragma unroll
      for (int dt = 0; dt < NI; dt++) acc[dt] *= corr;
    } else {
      l_run = l_run + ps;
    }
    m_run = m_new;
    // Y^T[d][q] += V^T . P^T: step k pairs slot k (key 4*quarter + k) with that key's values,
    // A = V[key][64*d4 + 4*col + e] for output tile 4*d4 + e
#pragma unroll
    for (int k = 0; k < 4; k++) {
#pragma unroll
      for (int d4 = 0; d4 < ND; d4++) {
        const v4d vv = *(const v4d*)(V + (4 * quarter + k) * GQ_VS + 64 * d4 + 4 * col);
#pragma unroll
        for (int e = 0; e < 4; e++)
          acc[4 * d4 + e] = __builtin_amdgcn_mfma_f64_16x16x4f64(vv[e], p[k], acc[4 * d4 + e], 0, 0, 0);
      }
    }
    // tile i + 1's values into its buffer (its digits landed during tile i), then the barrier
    // that ends tile i, then tile i + 2 into the buffer tile i leaves
    if (i + 1 < nt) lstore(i + 1);
    publish();
    if (i + 2 < nt) gload(i + 2);
  }

  // the partial through LDS (the buffers are free after the loop's last barrier, with no load
  // in flight), so the stores are whole rows: wave w's acc at [w][query][HD + 1]
  double* A = (double*)lds + (size_t)w * 16 * (HD + 1);
#pragma unroll
  for (int dt = 0; dt < NI; dt++)
#pragma unroll
    for (int r = 0; r < 4; r++)  // slot r of tile dt: dim 64*(dt/4) + 16r + 4*quarter + dt%4
      A[col * (HD + 1) + 64 * (dt >> 2) + 16 * r + 4 * quarter + (dt & 3)] = acc[dt][r];
  const size_t prow0 = ((((size_t)s * a.kvh + g) * a.maxch + c) * GQ_REP + w) * 16;
  if (quarter == 0 && col < a.B) {
    ml[(prow0 + col) * 2] = m_run;
    ml[(prow0 + col) * 2 + 1] = l_run;
  }
  for (int o = lane; o < 16 * HD; o += 64) {  // a wave's LDS accesses take effect in order
    const int qq = o / HD, d = o % HD;
    if (qq >= a.B) break;  // rows in order: the rest are past B too
    part[(prow0 + qq) * HD + d] = A[qq * (HD + 1) + d];
  }
}

// One workgroup per (q head, block row, sequence) finishes the row: it scores the block's own
// keys (f64 dot products of the f32 query and keys, then the same scale), takes the common
// maximum of those scores and of the chunks' maxima, and adds the block's values and the
// chunks' partial sums with weights exp(m - max) in a fixed order.  Every load (the chunk
// partials, the block's keys and values, the query) is issued before the first wait.
constexpr int MERGE_THREADS = 256;
template <int HD, bool QUANT, int MAXC>
__global__ __launch_bounds__(MERGE_THREADS) void k_attn_merge(AttnShape a, SeqInfo si, const float* __restrict__ q,
                                                              const float* __restrict__ kb,
                                                              const float* __restrict__ vb,
                                                              const double* __restrict__ part,
                                                              const double* __restrict__ ml, int Mpad,
                                                              int8_t* __restrict__ xq, float* __restrict__ dxT,
                                                              float* __restrict__ xf) {
  constexpr int NG = MERGE_THREADS / HD;       // chunk groups: thread (d, gi) adds chunks gi, gi+NG, ...
  constexpr int CPG = MAXC / NG;               // chunks per group at most (MAXC >= the call's chunks)
  constexpr int KSL = HD / 16;                 // dims per thread of a block score (16 threads a key)
  constexpr int VPG = 16 / NG;                 // block values per thread
  __shared__ double s_sc[16];                  // block scores
  __shared__ double s_e[16 + MAXC];            // weights: block keys, then chunks
  __shared__ double s_y[NG][HD];
  __shared__ double s_l;
  const int j = blockIdx.x, r = blockIdx.y, s = blockIdx.z, tid = threadIdx.x, lane = tid & 63;
  const int rep = a.nh / a.kvh, g = j / rep, hw = j % rep;
  const int nch = attn_chunks(si.nctx[s], a.ck);
  const int d = tid % HD, gi = tid / HD;
  const size_t base = ((size_t)s * a.kvh + g) * a.maxch * rep;
  auto row_of = [&](int c) { return (base + (size_t)c * rep + hw) * 16 + r; };
  const int m = s * a.B + r;

  // loads, all unconditional (indices clamped into range; what lies past the end is not used)
  // so they are in flight together; the launch picks MAXC just above the call's chunk count
  double accp[CPG];
  const int clast = nch > 0 ? nch - 1 : 0;
#pragma unroll
  for (int k = 0; k < CPG; k++) {
    const int c = min(gi + k * NG, clast);
    accp[k] = nch > 0 ? part[row_of(c) * HD + d] : 0.0;
  }
  const int key = tid >> 4, sl = tid & 15;
  const int keyc = min(key, a.B - 1);
  v4f qv[KSL / 4], kv[KSL / 4];
#pragma unroll
  for (int e = 0; e < KSL / 4; e++) {
    qv[e] = *(const v4f*)(q + ((size_t)m * a.nh + j) * HD + sl * KSL + 4 * e);
    kv[e] = *(const v4f*)(kb + ((size_t)(s * a.B + keyc) * a.kvh + g) * HD + sl * KSL + 4 * e);
  }
  float vv[VPG];
#pragma unroll
  for (int k = 0; k < VPG; k++) {
    const int i = min(gi + NG * k, a.B - 1);
    vv[k] = vb[((size_t)(s * a.B + i) * a.kvh + g) * HD + d];
  }
  const int cm = min(tid, clast);
  double mc = ml[row_of(cm) * 2], lc = ml[row_of(cm) * 2 + 1];
  if (tid >= nch) {
    mc = -INFINITY;
    lc = 0.0;
  }

  // the block's scores: f32 products are exact in f64
  double sc = 0.0;
#pragma unroll
  for (int e = 0; e < KSL / 4; e++)
#pragma unroll
    for (int f = 0; f < 4; f++) sc += (double)qv[e][f] * (double)kv[e][f];
  sc = row16_sum_f64(sc);
  if (sl == 0 && key < a.B) s_sc[key] = sc * (double)a.scale;
  if (tid < nch) s_e[16 + tid] = mc;
  __syncthreads();

  // the common maximum, the weights and the denominator (wave 0)
  if (tid < 64) {
    double mx = tid < a.B ? s_sc[tid] : -INFINITY;
    if (tid < nch) mx = fmax(mx, s_e[16 + tid]);
    mx = wave_max_f64(mx);
    double lsum = 0.0;
    if (tid < a.B) {
      const double e = exp(s_sc[tid] - mx);
      s_e[tid] = e;
      lsum = e;
    }
    if (tid < nch) {
      const double e = exp(mc - mx);
      s_e[16 + tid] = e;
      lsum += lc * e;
    }
    lsum = wave_sum_f64(lsum);
    if (tid == 0) s_l = lsum;
  }
  __syncthreads();

  double y = 0.0;
#pragma unroll
  for (int k = 0; k < CPG; k++) {
    const int c = gi + k * NG;
    if (c < nch) y += accp[k] * s_e[16 + c];
  }
#pragma unroll
  for (int k = 0; k < VPG; k++) {
    const int i = gi + NG * k;
    if (i < a.B) y += (double)vv[k] * s_e[i];
  }
  s_y[gi][d] = y;
  __syncthreads();
  if (gi != 0) return;  // threads d < HD: whole waves
  double yt = s_y[0][d];
#pragma unroll
  for (int v = 1; v < NG; v++) yt += s_y[v][d];
  const float val = (float)(yt / s_l);
  const size_t qd = (size_t)a.nh * HD;
  const size_t colx = (size_t)j * HD + d;
  if (QUANT)
    emit_a8(val, (size_t)m * qd + colx, xq, dxT, (colx >> 5) * Mpad + m, lane);
  else
    xf[(size_t)m * qd + colx] = val;
}

template <int HD, typename CT, bool WIN>
static hipError_t attn_partial_inst(const AttnShape& a, const SeqInfo& si, int maxn, const float* q, const CT* kc,
                                    const CT* vc, double* part, double* ml, hipStream_t st) {
  const size_t lds = attn_lds_bytes<HD>();
  hipError_t e = allow_lds((const void*)k_attn_partial<HD, CT, WIN>, lds);
  if (e != hipSuccess) return e;
  const int tasks = si.n * a.kvh * maxn, rep = a.nh / a.kvh;
  const int grid = (tasks + 7) / 8 * 8 * rep;
  hipLaunchKernelGGL((k_attn_partial<HD, CT, WIN>), dim3(grid), dim3(ATTN_THREADS), lds, st, a, si, maxn, q, kc, vc,
                     part, ml);
  return hipGetLastError();
}

template <int HD, typename CT>
static hipError_t attn_partial_hd(const AttnShape& a, const SeqInfo& si, const float* q, const CT* kc,
                                  const CT* vc, double* part, double* ml, hipStream_t st) {
  int maxn = 0;
  for (int i = 0; i < si.n; i++) {
    const int nch = si.nctx[i] > 0 ? (si.nctx[i] + a.ck - 1) / a.ck : 0;
    if (nch > maxn) maxn = nch;
  }
  if (maxn > a.maxch) return hipErrorInvalidValue;
  if (maxn == 0) return hipSuccess;  // no sequence has context rows: the merge does it all
  // the masked instance only where some row of some sequence has keys before its window
  bool win = false;
  for (int i = 0; i < si.n; i++)
    if (si.nctx[i] > 0 && si.mask0[i] + a.B - 1 > 0) win = true;
  return win ? attn_partial_inst<HD, CT, true>(a, si, maxn, q, kc, vc, part, ml, st)
             : attn_partial_inst<HD, CT, false>(a, si, maxn, q, kc, vc, part, ml, st);
}

template <int HD, int MAXC>
static void attn_merge_launch(const AttnShape& a, const SeqInfo& si, const float* q, const float* kb, const float* vb,
                              const double* part, const double* ml, int Mpad, bool quant, int8_t* xq, float* dxT,
                              float* xf, hipStream_t st) {
  if (quant)
    hipLaunchKernelGGL((k_attn_merge<HD, true, MAXC>), dim3(a.nh, a.B, si.n), dim3(MERGE_THREADS), 0, st, a, si, q,
                       kb, vb, part, ml, Mpad, xq, dxT, xf);
  else
    hipLaunchKernelGGL((k_attn_merge<HD, false, MAXC>), dim3(a.nh, a.B, si.n), dim3(MERGE_THREADS), 0, st, a, si, q,
                       kb, vb, part, ml, Mpad, xq, dxT, xf);
}

template <int HD>
static hipError_t attn_merge_hd(const AttnShape& a, const SeqInfo& si, const float* q, const float* kb,
                                const float* vb, const double* part, const double* ml, int Mpad, bool quant,
                                int8_t* xq, float* dxT, float* xf, hipStream_t st) {
  int maxn = 0;
  for (int i = 0; i < si.n; i++) {
    const int nch = si.nctx[i] > 0 ? (si.nctx[i] + a.ck - 1) / a.ck : 0;
    if (nch > maxn) maxn = nch;
  }
  if (maxn > ATTN_MAXCH) return hipErrorInvalidValue;
  if (maxn <= 8)
    attn_merge_launch<HD, 8>(a, si, q, kb, vb, part, ml, Mpad, quant, xq, dxT, xf, st);
  else if (maxn <= 32)
    attn_merge_launch<HD, 32>(a, si, q, kb, vb, part, ml, Mpad, quant, xq, dxT, xf, st);
  else
    attn_merge_launch<HD, ATTN_MAXCH>(a, si, q, kb, vb, part, ml, Mpad, quant, xq, dxT, xf, st);
  return hipGetLastError();
}

static bool attn_shape_ok(const AttnShape& a) {
  return !(a.nh % a.kvh || a.nh / a.kvh > 16 || a.B > 16 || a.ck % 32 || a.ck <= 0 || a.maxch > ATTN_MAXCH) &&
         (a.hd == 64 || a.hd == 128);
}

template <typename CT, bool WIN>
static hipError_t attn_gqa_dig_inst(const AttnShape& a, const SeqInfo& si, int maxn, const int8_t* qd, const int* qe,
                                    const CT* vc, const int8_t* kd, const int* ke, double* part, double* ml,
                                    hipStream_t st) {
  hipError_t e = allow_lds((const void*)k_attn_gqa_dig<CT, WIN>, GQ_LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_attn_gqa_dig<CT, WIN>), dim3(si.n * a.kvh * maxn), dim3(GQ_THREADS), GQ_LDS, st, a, si, maxn, qd,
                     qe, vc, kd, ke, part, ml);
  return hipGetLastError();
}

template <typename CT>
static hipError_t attn_gqa_dig(const AttnShape& a, const SeqInfo& si, const int8_t* qd, const int* qe, const CT* vc,
                               const int8_t* kd, const int* ke, double* part, double* ml, hipStream_t st) {
  int maxn = 0;
  bool win = false;
  for (int i = 0; i < si.n; i++) {
    const int nch = si.nctx[i] > 0 ? (si.nctx[i] + a.ck - 1) / a.ck : 0;
    if (nch > maxn) maxn = nch;
    if (si.nctx[i] > 0 && si.mask0[i] + a.B - 1 > 0) win = true;
  }
  if (maxn > a.maxch) return hipErrorInvalidValue;
  if (maxn == 0) return hipSuccess;  // no sequence has context rows: the merge does it all
  return win ? attn_gqa_dig_inst<CT, true>(a, si, maxn, qd, qe, vc, kd, ke, part, ml, st)
             : attn_gqa_dig_inst<CT, false>(a, si, maxn, qd, qe, vc, kd, ke, part, ml, st);
}

bool attn_digit_scores(int nh, int kvh, int hd) { return hd == 128 && nh == GQ_REP * kvh; }

hipError_t launch_attention_chunks(const AttnShape& a, const SeqInfo& si, const float* q, const void* kc,
                                   const void* vc, const DigitRows* dig, double* part, double* ml, hipStream_t st) {
  if (!attn_shape_ok(a)) return hipErrorInvalidValue;
  if (dig) {
    if (!attn_digit_scores(a.nh, a.kvh, a.hd) || !dig->qd || !dig->qe || !dig->kd || !dig->ke)
      return hipErrorInvalidValue;
    if (a.kv_f16)
      return attn_gqa_dig(a, si, dig->qd, dig->qe, (const _Float16*)vc, dig->kd, dig->ke, part, ml, st);
    return attn_gqa_dig(a, si, dig->qd, dig->qe, (const float*)vc, dig->kd, dig->ke, part, ml, st);
  }
  if (a.kv_f16) {
    const _Float16 *k = (const _Float16*)kc, *v = (const _Float16*)vc;
    return a.hd == 64 ? attn_partial_hd<64>(a, si, q, k, v, part, ml, st) : attn_partial_hd<128>(a, si, q, k, v, part, ml, st);
  }
  const float *k = (const float*)kc, *v = (const float*)vc;
  return a.hd == 64 ? attn_partial_hd<64>(a, si, q, k, v, part, ml, st) : attn_partial_hd<128>(a, si, q, k, v, part, ml, st);
}

hipError_t launch_attention_merge(const AttnShape& a, const SeqInfo& si, const float* q, const float* kb,
                                  const float* vb, const double* part, const double* ml, int Mpad, bool quant,
                                  int8_t* xq, float* dxT, float* xf, hipStream_t st) {
  if (!attn_shape_ok(a)) return hipErrorInvalidValue;
  if (a.hd == 64) return attn_merge_hd<64>(a, si, q, kb, vb, part, ml, Mpad, quant, xq, dxT, xf, st);
  return attn_merge_hd<128>(a, si, q, kb, vb, part, ml, Mpad, quant, xq, dxT, xf, st);
}

}  // namespace dfl
