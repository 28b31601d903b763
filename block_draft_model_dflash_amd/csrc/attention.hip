// Block-vs-context attention (cortiq-engine "dflash.rs", Drafter::block: each q head j reads
// kv head j / rep; its keys and values are the context rows before the anchor followed by the
// block's own rows, with no causal mask; s = (q . k) * hd^-0.5, softmax, y = sum p v).
//
// The pages' device kernel (gpu_wgpu/dflash_dev.rs, dflash_attn) writes every score to a global
// scratch and re-reads it; here the context is split into chunks, each wave keeps a running
// (max, sum, acc) per query in registers (online softmax), and a merge combines the chunks.
// A workgroup serves one (sequence, kv head, chunk) with eight waves: wave w takes q head w % 4
// of the group and the chunk's even (w < 4) or odd (w >= 4) 16-key tiles; the two halves of a
// head are combined in LDS before the chunk's result is written.  The chunks hold context rows
// only (so every key lane of the grid gets the same number of tiles); the block's own 16 keys,
// a few thousand flops per (head, row), are scored by the merge, which then combines them with
// the chunks.  The 16 block rows of a head are the 16 columns of v_mfma_f64_16x16x4f64 tiles:
//   S^T[key][q] = K . Q^T   (A = 16 keys staged in LDS, B = the wave's queries in registers)
//   Y^T[d][q]  += V^T . P^T (A = 16-dim slices of V from LDS, B = the wave's probabilities,
//                            already in the accumulator layout of S^T)
// so the probabilities never leave registers.  Context K/V is f32 [slot][kvh][max_ctx][hd].
// Lane layout of the f64 16x16x4 MFMA: lane l gives A[l%16][l/16] and B[l/16][l%16] and holds
// D[l/16 + 4r][l%16] in accumulator slot r (rows interleaved, unlike the f32 16x16 forms).
//
// Scores, softmax and values are evaluated in f64 (the f32 keys, values and queries are exact
// in f64) and the output is rounded once to f32: it feeds an int8 quantizer, where a value one
// ulp off flips codes that the following layers amplify, so it has to be the correctly rounded
// result that any exact evaluation gives.
#include "common.h"

namespace dfl {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef double v4d __attribute__((ext_vector_type(4)));

constexpr int ATTN_HEADS = 4;                   // q heads served at once (one wave each per half)
constexpr int ATTN_THREADS = 64 * 2 * ATTN_HEADS;  // two key halves

// Chunks a sequence with n context rows takes (the block's own rows are the merge's part).
__device__ __forceinline__ int attn_chunks(int nctx, int ck) { return nctx > 0 ? (nctx + ck - 1) / ck : 0; }

template <int HD>
__global__ __launch_bounds__(ATTN_THREADS) void k_attn_partial(AttnShape a, SeqInfo si, const float* __restrict__ q,
                                                               const float* __restrict__ kc,
                                                               const float* __restrict__ vc,
                                                               double* __restrict__ part, double* __restrict__ ml) {
  // LDS rows: keys HD + 4 floats apart (each 16-lane group of a 128-bit read covers all banks),
  // values HD + 1 apart (the 64 lanes' 32-bit reads of rows 4k + quarter, columns 4*col + e
  // fall in 64 different banks)
  constexpr int KS = HD + 4, VS = HD + 1;
  constexpr int TILE = 16 * KS;        // one 16-key tile of K (V uses 16 * VS <= TILE)
  constexpr int HALF = ATTN_THREADS / 2;
  constexpr int NL = 16 * (HD / 4) / HALF;  // float4 of K (and of V) each thread stages per tile
  constexpr int CD = 64;                    // dims combined per LDS round
  constexpr int COMB = ATTN_HEADS * (16 * CD + 32);  // doubles: acc slice + (m, l) per row
  constexpr int KV_BYTES = 2 * 2 * TILE * 4;
  constexpr int LDS_BYTES = KV_BYTES > COMB * 8 ? KV_BYTES : COMB * 8;
  __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];
  const int c = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int nctx = si.nctx[s];
  const int nch = attn_chunks(nctx, a.ck);
  if (c >= nch) return;  // the whole workgroup: this sequence has fewer chunks
  const int rep = a.nh / a.kvh;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int half = w / ATTN_HEADS, hw0 = w % ATTN_HEADS, htid = tid % HALF;
  const int quarter = lane >> 4, col = lane & 15;
  float* Ks = (float*)lds + half * 2 * TILE;
  float* Vs = Ks + TILE;
  const int k0 = c * a.ck, kend = min(nctx, k0 + a.ck);
  const int nt = (kend - k0 + 15) / 16;  // >= 1: every launched chunk holds context rows
  const int rounds = (nt + 1) / 2;
  const float* Kctx = kc + ((size_t)si.slot[s] * a.kvh + g) * a.max_ctx * HD;
  const float* Vctx = vc + ((size_t)si.slot[s] * a.kvh + g) * a.max_ctx * HD;

  // the group's q heads, ATTN_HEADS at a time; the chunk's keys are re-staged per round when a
  // group has more heads than that
  for (int h0 = 0; h0 < rep; h0 += ATTN_HEADS) {
    const int hw = h0 + hw0;  // this wave's head within the group
    const bool live = hw < rep;
    const int j = g * rep + (live ? hw : 0);
    v4f qr[HD / 16];
#pragma unroll
    for (int i4 = 0; i4 < HD / 16; i4++)
      qr[i4] = col < a.B ? *(const v4f*)(q + ((size_t)(s * a.B + col) * a.nh + j) * HD + 16 * i4 + 4 * quarter)
                         : (v4f){0.f, 0.f, 0.f, 0.f};
    double m_run = -INFINITY, l_run = 0.0;
    v4d acc[HD / 16];
#pragma unroll
    for (int dt = 0; dt < HD / 16; dt++) acc[dt] = (v4d){0.0, 0.0, 0.0, 0.0};

    // tile i of the chunk: context keys k0 + 16i..; the next tile of this half travels to
    // registers while the current one is computed
    v4f pk[NL], pv[NL];
    auto fetch = [&](int i) {
#pragma unroll
      for (int u = 0; u < NL; u++) {
        const int e = htid + u * HALF;
        const int r = e / (HD / 4), c4 = e % (HD / 4);
        const int key = k0 + 16 * i + r;
        pk[u] = pv[u] = (v4f){0.f, 0.f, 0.f, 0.f};
        if (i < nt && key < kend) {
          pk[u] = *(const v4f*)(Kctx + (size_t)key * HD + 4 * c4);
          pv[u] = *(const v4f*)(Vctx + (size_t)key * HD + 4 * c4);
        }
      }
    };
    fetch(half);
    for (int rd = 0; rd < rounds; rd++) {
      const int i = 2 * rd + half;  // this half's tile in this round
      __syncthreads();
#pragma unroll
      for (int u = 0; u < NL; u++) {
        const int e = htid + u * HALF;
        const int r = e / (HD / 4), c4 = e % (HD / 4);
        *(v4f*)(Ks + r * KS + 4 * c4) = pk[u];
#pragma unroll
        for (int f = 0; f < 4; f++) Vs[r * VS + 4 * c4 + f] = pv[u][f];
      }
      __syncthreads();
      if (i + 2 < nt) fetch(i + 2);
      if (!live || i >= nt) continue;
      const int nvalid = min(16, kend - (k0 + 16 * i));  // keys of this tile
      v4d st0 = (v4d){0.0, 0.0, 0.0, 0.0}, st1 = st0;
#pragma unroll
      for (int i4 = 0; i4 < HD / 16; i4++) {
        const v4f kv = *(const v4f*)(Ks + col * KS + 16 * i4 + 4 * quarter);
        st0 = __builtin_amdgcn_mfma_f64_16x16x4f64((double)kv[0], (double)qr[i4][0], st0, 0, 0, 0);
        st1 = __builtin_amdgcn_mfma_f64_16x16x4f64((double)kv[1], (double)qr[i4][1], st1, 0, 0, 0);
        st0 = __builtin_amdgcn_mfma_f64_16x16x4f64((double)kv[2], (double)qr[i4][2], st0, 0, 0, 0);
        st1 = __builtin_amdgcn_mfma_f64_16x16x4f64((double)kv[3], (double)qr[i4][3], st1, 0, 0, 0);
      }
      double p[4], mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int key = quarter + 4 * r;  // accumulator slot r holds key row quarter + 4r
        p[r] = key < nvalid ? (st0[r] + st1[r]) * (double)a.scale : -INFINITY;
        mx = fmax(mx, p[r]);
      }
      mx = fmax(mx, __shfl_xor(mx, 16));
      mx = fmax(mx, __shfl_xor(mx, 32));
      const double m_new = fmax(m_run, mx);
      const double corr = exp(m_run - m_new);
      double ps = 0.0;
#pragma unroll
      for (int r = 0; r < 4; r++) {
        p[r] = exp(p[r] - m_new);
        ps += p[r];
      }
      ps += __shfl_xor(ps, 16);
      ps += __shfl_xor(ps, 32);
      l_run = l_run * corr + ps;
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < HD / 16; dt++) {
        acc[dt] *= corr;
#pragma unroll
        for (int k = 0; k < 4; k++) {
          // step k pairs the probabilities of slot k (keys quarter + 4k) with those keys' values
          const float va = Vs[(4 * k + quarter) * VS + 64 * (dt >> 2) + 4 * col + (dt & 3)];
          acc[dt] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)va, p[k], acc[dt], 0, 0, 0);
        }
      }
    }

    // combine the halves: (m, l, acc) of the odd tiles join those of the even tiles through LDS,
    // CD dims per round.  Half 0 always has tile 0, so its maximum is finite.
    double* cb = (double*)lds + hw0 * (16 * CD + 32);
    const size_t prow = ((((size_t)s * a.kvh + g) * a.maxch + c) * rep + hw) * 16 + col;
    double e0 = 1.0, e1 = 0.0;
    for (int d0 = 0; d0 < HD; d0 += CD) {
      __syncthreads();
      if (half == 1 && live) {
#pragma unroll
        for (int d4 = 0; d4 < CD / 64; d4++)
#pragma unroll
          for (int r = 0; r < 4; r++)
#pragma unroll
            for (int e = 0; e < 4; e++)
              cb[col * CD + 64 * d4 + 16 * r + 4 * quarter + e] = acc[4 * ((d0 >> 6) + d4) + e][r];
        if (d0 == 0 && quarter == 0) {
          cb[16 * CD + 2 * col] = m_run;
          cb[16 * CD + 2 * col + 1] = l_run;
        }
      }
      __syncthreads();
      if (half == 1 || !live) continue;
      if (d0 == 0) {
        const double m1 = cb[16 * CD + 2 * col], l1 = cb[16 * CD + 2 * col + 1];
        const double m = fmax(m_run, m1);
        e0 = exp(m_run - m);
        e1 = m1 == -INFINITY ? 0.0 : exp(m1 - m);
        l_run = l_run * e0 + l1 * e1;
        m_run = m;
      }
      if (col >= a.B) continue;
      double* dst = part + prow * HD + d0;
#pragma unroll
      for (int d4 = 0; d4 < CD / 64; d4++)
#pragma unroll
        for (int r = 0; r < 4; r++) {
          // accumulator (dt = 4*d4 + e, slot r) is row quarter + 4r of tile dt: dim 64*d4 + 16*r + 4*quarter + e
          const int o = 64 * d4 + 16 * r + 4 * quarter;
#pragma unroll
          for (int e = 0; e < 4; e++)
            dst[o + e] = acc[4 * ((d0 >> 6) + d4) + e][r] * e0 + cb[col * CD + o + e] * e1;
        }
    }
    if (half == 0 && live && col < a.B && quarter == 0) {
      ml[prow * 2] = m_run;
      ml[prow * 2 + 1] = l_run;
    }
  }
}

__device__ __forceinline__ void emit_q8(float y, size_t qi, int8_t* __restrict__ xq, float* __restrict__ dx,
                                        size_t di, int lane) {
  float amax = fabsf(y);
#pragma unroll
  for (int o = 16; o; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 32));
  int8_t qv = 0;
  float d = 0.f;
  if (amax > 0.f) {
    d = amax / 127.0f;
    const float inv = 127.0f / amax;
    float r = __builtin_rintf(y * inv);
    r = fminf(fmaxf(r, -127.f), 127.f);
    qv = (int8_t)r;
  }
  xq[qi] = qv;
  if ((lane & 31) == 0) dx[di] = d;
}

// One workgroup per (q head, block row, sequence) finishes the row: it scores the block's own
// keys (f64 dot products of the f32 query and keys, then the same scale), takes the common
// maximum of those scores and of the chunks' maxima, and adds the block's values and the
// chunks' partial sums with weights exp(m - max) in a fixed order.  Every load (the chunk
// partials, the block's keys and values, the query) is issued before the first wait.
constexpr int MERGE_THREADS = 256;
template <int HD, bool QUANT>
__global__ __launch_bounds__(MERGE_THREADS) void k_attn_merge(AttnShape a, SeqInfo si, const float* __restrict__ q,
                                                              const float* __restrict__ kb,
                                                              const float* __restrict__ vb,
                                                              const double* __restrict__ part,
                                                              const double* __restrict__ ml, int Mpad,
                                                              int8_t* __restrict__ xq, float* __restrict__ dxT,
                                                              float* __restrict__ xf) {
  constexpr int NG = MERGE_THREADS / HD;       // chunk groups: thread (d, gi) adds chunks gi, gi+NG, ...
  constexpr int CPG = ATTN_MAXCH / NG;         // chunks per group at most
  constexpr int KSL = HD / 16;                 // dims per thread of a block score (16 threads a key)
  constexpr int VPG = 16 / NG;                 // block values per thread
  __shared__ double s_sc[16];                  // block scores
  __shared__ double s_e[16 + ATTN_MAXCH];      // weights: block keys, then chunks
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
  // so they are in flight together
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
  sc += __shfl_xor(sc, 1);
  sc += __shfl_xor(sc, 2);
  sc += __shfl_xor(sc, 4);
  sc += __shfl_xor(sc, 8);
  if (sl == 0 && key < a.B) s_sc[key] = sc * (double)a.scale;
  if (tid < nch) s_e[16 + tid] = mc;
  __syncthreads();

  // the common maximum, the weights and the denominator (wave 0)
  if (tid < 64) {
    double mx = tid < a.B ? s_sc[tid] : -INFINITY;
    if (tid < nch) mx = fmax(mx, s_e[16 + tid]);
#pragma unroll
    for (int o = 32; o; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o));
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
#pragma unroll
    for (int o = 32; o; o >>= 1) lsum += __shfl_xor(lsum, o);
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
    emit_q8(val, (size_t)m * qd + colx, xq, dxT, (colx >> 5) * Mpad + m, lane);
  else
    xf[(size_t)m * qd + colx] = val;
}

template <int HD>
static hipError_t attn_partial_hd(const AttnShape& a, const SeqInfo& si, const float* q, const float* kc,
                                  const float* vc, double* part, double* ml, hipStream_t st) {
  int maxn = 0;
  for (int i = 0; i < si.n; i++) {
    const int nch = si.nctx[i] > 0 ? (si.nctx[i] + a.ck - 1) / a.ck : 0;
    if (nch > maxn) maxn = nch;
  }
  if (maxn > a.maxch) return hipErrorInvalidValue;
  if (maxn == 0) return hipSuccess;  // no sequence has context rows: the merge does it all
  hipLaunchKernelGGL(k_attn_partial<HD>, dim3(maxn, a.kvh, si.n), dim3(ATTN_THREADS), 0, st, a, si, q, kc, vc, part,
                     ml);
  return hipGetLastError();
}

template <int HD>
static hipError_t attn_merge_hd(const AttnShape& a, const SeqInfo& si, const float* q, const float* kb,
                                const float* vb, const double* part, const double* ml, int Mpad, bool quant,
                                int8_t* xq, float* dxT, float* xf, hipStream_t st) {
  if (quant)
    hipLaunchKernelGGL((k_attn_merge<HD, true>), dim3(a.nh, a.B, si.n), dim3(MERGE_THREADS), 0, st, a, si, q, kb, vb,
                       part, ml, Mpad, xq, dxT, xf);
  else
    hipLaunchKernelGGL((k_attn_merge<HD, false>), dim3(a.nh, a.B, si.n), dim3(MERGE_THREADS), 0, st, a, si, q, kb,
                       vb, part, ml, Mpad, xq, dxT, xf);
  return hipGetLastError();
}

static bool attn_shape_ok(const AttnShape& a) {
  return !(a.nh % a.kvh || a.nh / a.kvh > 16 || a.B > 16 || a.ck % 32 || a.ck <= 0 || a.maxch > ATTN_MAXCH) &&
         (a.hd == 64 || a.hd == 128);
}

hipError_t launch_attention_chunks(const AttnShape& a, const SeqInfo& si, const float* q, const float* kc,
                                   const float* vc, double* part, double* ml, hipStream_t st) {
  if (!attn_shape_ok(a)) return hipErrorInvalidValue;
  if (a.hd == 64) return attn_partial_hd<64>(a, si, q, kc, vc, part, ml, st);
  return attn_partial_hd<128>(a, si, q, kc, vc, part, ml, st);
}

hipError_t launch_attention_merge(const AttnShape& a, const SeqInfo& si, const float* q, const float* kb,
                                  const float* vb, const double* part, const double* ml, int Mpad, bool quant,
                                  int8_t* xq, float* dxT, float* xf, hipStream_t st) {
  if (!attn_shape_ok(a)) return hipErrorInvalidValue;
  if (a.hd == 64) return attn_merge_hd<64>(a, si, q, kb, vb, part, ml, Mpad, quant, xq, dxT, xf, st);
  return attn_merge_hd<128>(a, si, q, kb, vb, part, ml, Mpad, quant, xq, dxT, xf, st);
}

}  // namespace dfl
