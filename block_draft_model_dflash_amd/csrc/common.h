// Internal declarations of the gfx950 DFlash library: packed weight layout, kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dfl {

enum Fmt { F32 = 0, Q4 = 1, Q8 = 2 };

// Packed ("tiled") quantized weights.  A superblock covers 16 output rows (an n-tile) and 128
// input columns (4 groups of 32).  Superblocks are stored [n-tile][k-block], so one wave
// streams one n-tile's row of superblocks front to back.
//
// Q4 superblock, 1152 bytes:
//   bytes [0, 1024): 64 lanes x 16 bytes.  Lane l's dword j (group g = 4*kb + j) holds the
//     codes of row 16*t + l%16, columns k0 = 32*g + 8*(l/16) .. k0+7: byte b keeps column
//     k0+b in its low nibble and column k0+4+b in its high nibble (two's complement nibbles).
//     (dword << 4) & 0xF0F0F0F0 then gives 16*q of columns k0..k0+3 as signed bytes and
//     dword & 0xF0F0F0F0 gives 16*q of k0+4..k0+7: the B operand of one 16x16x32 int8 MFMA.
//   bytes [1024, 1152): f16 scales [16 rows][4 groups].
// Q8 superblock, 2176 bytes:
//   bytes [0, 1024): lane l 16 bytes = groups j = 0, 1 (8 codes each, columns k0..k0+7);
//   bytes [1024, 2048): the same for groups 2, 3; bytes [2048, 2176): f16 scales [16][4].
// F32 matrices stay row-major [rows][cols] (rows permuted the same way as tiles below).
constexpr int SB_Q4 = 1152, SB_Q8 = 2176;
constexpr int SB_SCALES_Q4 = 1024, SB_SCALES_Q8 = 2048;

inline size_t packed_bytes(int fmt, long rows, long cols) {
  if (fmt == F32) return (size_t)rows * cols * 4;
  return (size_t)(rows / 16) * (cols / 128) * (fmt == Q4 ? SB_Q4 : SB_Q8);
}

constexpr int MAX_SEQS_ARG = 64;  // sequences of one block call (max_seqs*block <= 128)

// Per-call sequence table passed by value to the block kernels.
struct SeqInfo {
  int n;                        // sequences in this call
  int slot[MAX_SEQS_ARG];       // cache slot of each
  int ctx0[MAX_SEQS_ARG];       // cache row of its first context key (position - first)
  int nctx[MAX_SEQS_ARG];       // context keys it attends to (cache rows ctx0 .. ctx0+nctx-1)
  int mask0[MAX_SEQS_ARG];      // block row r does not see keys i < mask0 + r (a window)
  long long pos0[MAX_SEQS_ARG]; // position of block row 0 (the anchor)
};

// ---- launchers (return the launch's hipError_t) ----

// Repack a canonical matrix into tiles; destination n-tile of source tile t is
// tile_off + t * tile_stride (used to concatenate and interleave matrices).
hipError_t launch_pack(int fmt, const void* codes, const void* scales, int rows, int cols, void* out, long tile_off,
                       long tile_stride, hipStream_t st);

// Quantized weight-streaming GEMM: xq [Mpad][K] int8 (rows >= M zero), dxT [K/32][Mpad] f32
// activation scales, y = W . x for the Mpad rows, then one epilogue:
enum GemmEpi {
  EPI_F64 = 0,    // double y[m*N + n] for m < Mpad
  EPI_F32 = 1,    // float y[m*ld + n] for m < m_store
  EPI_RESID = 2,  // h[m*N + n] += f32(y) for m < M; ssq[m*(N/16) + n/16] = sum of h^2 over the
                  // 16 columns of n's tile (f64; 0 for rows >= M), m < Mpad
  EPI_SWIGLU = 3,  // N = 2I with gate|up interleaved by 16-column tiles: a = silu(gate) * up
                   // (f64 from the f32 products, one rounding) -> A8_32 into xq [Mpad][I] and
                   // dxT [I/32][Mpad], or f32 into xf [Mpad][I] when xq is null
  EPI_CONV = 4     // as EPI_RESID, with the row convolution's stage 1 on f32(y) before the add:
                   // h[m] += conv(f32(y))[m] (kernels cd [M][2*ckn*N/cgs], cbase [2][ckn][N]; rows
                   // of one sequence's block, cB of them, lie in one workgroup's row group)
};
struct GemmOut {
  int epi;
  int M, Mpad;
  void* y;
  int ld, m_store;
  float* h;
  double* ssq;
  int8_t* xq;
  float* dxT;
  float* xf;
  const float* cd;
  const float* cbase;
  int cB, cgs, ckn;
};
// layout < 0: chosen from the shape (0: four n-tiles x two k-waves per workgroup; 1: K split
// over the waves of one (two) n-tile(s); 2: four n-tiles, one wave each; 3: eight n-tiles, one
// wave each); SwiGLU takes whole groups of four n-tiles (layouts 0, 2, 3).
hipError_t launch_gemm_q(int fmt, const void* W, int N, int K, const int8_t* xq, const float* dxT, int layout,
                         const GemmOut& o, hipStream_t st);
int gemm_layout(int N, int Mpad, int epi);
hipError_t launch_group_sums(int fmt, const void* W, int N, int K, const int8_t* xq, int Mpad, int M,
                             int32_t* sums, hipStream_t st);
// f32 GEMM: x [Mpad][K] f32.  direct: float out[m*out_ld + n] for m < m_store; else double
// out[m*N + n] (one slice of partial sums, S = 1).
hipError_t launch_gemm_f32(const float* W, int N, int K, const float* x, int Mpad, int M, void* out, bool direct,
                           int out_ld, int m_store, hipStream_t st);

// Activation producers.  Every one writes rows [0, Mpad): rows >= M are zero.  quant: xq
// [Mpad][N] int8 + dxT [N/32][Mpad]; else xf [Mpad][N] f32.
//
// v = (resid ? resid[m] : 0) + o, o = f32(sum_{s<S} part[(s*part_mstride + m)*N + i]) (f64
// partials) or, with part NULL, o = x[m*N + i] (f32 rows); h_out (optional) receives v; with a
// norm weight w the row is RMSNormed first.  One workgroup per row.
hipError_t launch_norm_act(const double* part, const float* x, int S, int part_mstride, const float* resid,
                           float* h_out, const float* w, float eps, int M, int Mpad, int N, bool quant, int8_t* xq,
                           float* dxT, float* xf, hipStream_t st);
// RMSNorm + activation output of rows h [M][N] whose sums of squares arrive in nparts f64
// pieces ssq[m*nparts + i]; many workgroups per row.
hipError_t launch_rms_act(const float* h, const double* ssq, int nparts, const float* w, float eps, int M, int Mpad,
                          int N, bool quant, int8_t* xq, float* dxT, float* xf, hipStream_t st, float* xc = nullptr);
// Row convolutions over each sequence's B block rows (rows of one call: M = sequences * B).
// d [M][2*kn*N/gs] the rows' dynamic kernels, base [2][kn][N] the static ones.  conv_in: stage
// 0 of x [M][N] f32, then A8_32 into xq/dxT (quant) or f32 into xf, rows M..Mpad zero.
// conv_out: stage 1 of o [M][N] added to h, with the sums of squares of h in 16-column pieces.
hipError_t launch_conv_in(const float* x, const float* d, const float* base, int M, int Mpad, int B, int N, int gs,
                          int kn, bool quant, int8_t* xq, float* dxT, float* xf, hipStream_t st);
hipError_t launch_conv_out(const float* o, const float* d, const float* base, int M, int B, int N, int gs, int kn,
                           float* h, double* ssq, hipStream_t st);
// h = x (M rows of N) and the rows' sums of squares in N/256 pieces ssq[m*(N/256) + i].
hipError_t launch_copy_ssq(const float* x, float* h, int M, int N, double* ssq, hipStream_t st);
// a = silu(gate) * up from the interleaved gate|up partials [S][Mpad][2I].
hipError_t launch_swiglu_act(const double* part, int S, int M, int Mpad, int I, bool quant, int8_t* xq, float* dxT,
                             float* xf, hipStream_t st);
// q/k/v of the block rows from the fused projection partials [S][Mpad][qd + 2 kvd]:
// q-norm / k-norm, then (rope) RoPE at si.pos0[m / B] + m % B; with qd / qe (head_dim 128) also
// each query row's int8 digits [M][nh][7*128] and exponent [M][nh] (digits.h).
hipError_t launch_qkv_epilogue(const double* part, int S, int Mpad, int M, int B, const SeqInfo& si, int nh, int kvh,
                               int hd, const float* q_norm, const float* k_norm, const float* inv_freq, float eps,
                               bool rope, float* q, float* k, float* v, int8_t* qd, int* qe, hipStream_t st);
// Context rows into the cache from the all-layer K|V partials [S][Mpad][L * 2 kvd]; layer l's
// keys are rotated when bit l of rot_mask is set (layers >= 64 always are).  kd / ke (head_dim
// 128, else null): each key row's int8 digits [L][max_seqs][kvh][max_ctx][7][128] and exponent
// [L][max_seqs][kvh][max_ctx] (digits.h), of the value the cache holds.
hipError_t launch_kv_append(const double* part, int S, int Mpad, int n, int layers, int kvh, int hd,
                            const float* k_norms, const float* inv_freq, float eps, unsigned long long rot_mask,
                            long long pos0, int row0, int slot, int max_seqs, int max_ctx, bool f16, void* kc,
                            void* vc, int8_t* kd, int* ke, hipStream_t st);
// n rows of one (layer, sequence) of the cache, every kv head, into out [n][kvh][hd] f32.
hipError_t launch_read_cache(const void* cache, bool f16, size_t layer_elems, int layer, int seq, int row0, int n,
                             int kvh, int hd, int max_ctx, float* out, hipStream_t st);

// Attention of the block rows over context + block keys, split over context chunks.
struct AttnShape {
  int nh, kvh, hd, B, max_ctx, max_seqs, ck, maxch;
  float scale;
  int kv_f16;  // the cache holds f16 elements
};
// The chunk kernel writes per-chunk (max, sum, acc) of the context keys in f64 to part/ml; the
// merge scores the block's own keys, combines them with a sequence's chunks per (q head, row)
// and writes the f32 result (A8 into xq/dxT, or f32 xf).
constexpr int ATTN_MAXCH = 64;  // context chunks per (sequence, kv head) at most
// The digit rows of integer scores (digits.h): the block's queries qd [M][nh][7*128] with
// exponents qe [M][nh], the layer's keys kd [slot][kvh][max_ctx][7*128] with ke [slot][kvh][max_ctx].
struct DigitRows {
  const int8_t* qd;
  const int* qe;
  const int8_t* kd;
  const int* ke;
};
// whether a geometry scores with digits (the grouped-query kernel: head_dim 128, four q heads per
// kv head); then the q/k epilogue and the append write the digit rows and dig is given here, else
// dig is null and the scores are f64 from kc
bool attn_digit_scores(int nh, int kvh, int hd);
hipError_t launch_attention_chunks(const AttnShape& a, const SeqInfo& si, const float* q, const void* kc,
                                   const void* vc, const DigitRows* dig, double* part, double* ml, hipStream_t st);
hipError_t launch_attention_merge(const AttnShape& a, const SeqInfo& si, const float* q, const float* kb,
                                  const float* vb, const double* part, const double* ml, int Mpad, bool quant,
                                  int8_t* xq, float* dxT, float* xf, hipStream_t st);

// Dynamic LDS a workgroup may use on the current device (queried once per device), and a
// helper that raises a kernel's dynamic-LDS limit when a launch needs more than the default.
size_t max_dynamic_lds();
hipError_t allow_lds(const void* kernel, size_t bytes);

// Candidate selection: per-row top T (chunk lists in part_v/part_i, top_k_scratch bytes), and
// the greedy re-scoring of the draft rows' candidates (cv/ci [rows][T]).
hipError_t launch_top_k(const float* x, int rows, int width, int ld, int T, float* part_v, int* part_i, float* vals,
                        int* idx, hipStream_t st);
size_t top_k_scratch(int rows, int width, int T);
// The chunk lists of a row (ceil(width/4096) * T entries) must fit the merge's 4096 slots.
bool top_k_fits(int width, int T);
hipError_t launch_select(const float* cv, const int* ci, int rows, int T, const float* hp, int rank,
                         const uint16_t* pred, const uint16_t* succ, int anchor, int* chosen, int* plain,
                         float* scores, hipStream_t st);
size_t select_scratch(int rows, int T);

hipError_t launch_inv_freq(double theta, int hd, float* out, hipStream_t st);

// Records the error of a call without a ctx (dflash_last_error(NULL) returns it) and gives back
// `code`.
int unit_error(int code, const char* what, hipError_t e = hipSuccess);
hipError_t launch_quant_rows(const float* x, int rows, int cols, int8_t* q, float* d, hipStream_t st);
hipError_t launch_transpose_scales(const float* d, int rows, int groups, int Mpad, float* dT, hipStream_t st);

}  // namespace dfl
