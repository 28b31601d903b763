/* DFlash 2 block drafter -- CPU oracle (TEST INFRASTRUCTURE ONLY).
 *
 * A plain, slow, obviously correct host implementation of what the GPU path computes:
 * context append (FC, RMSNorm, per-layer K/V, k-norm, RoPE into a K/V store) and the block
 * forward (per layer RMSNorm, Wq/Wk/Wv, q/k-norm, RoPE, non-causal attention over the
 * context and the block's own rows, Wo + residual, RMSNorm, SwiGLU MLP + residual; final
 * RMSNorm and the head's logits), with the quantized formats of the drafter's matrices.
 *
 * Only the tests, the package's smoke check and the benchmark's CPU-baseline leg may load
 * this.  It shares no code with the GPU library and neither side includes the other.
 *
 * All pointers are host pointers.  Status codes: 0 ok, -1 invalid argument, -2 capacity.
 */
#ifndef DFLASH_ORACLE_H
#define DFLASH_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { OG_F32 = 0, OG_Q4_32 = 1, OG_Q8_32 = 2 };

typedef struct {
  double rope_theta, eps;
  int32_t layers, hidden, heads, kv_heads, head_dim, intermediate, vocab, block, n_taps;
  int32_t body_fmt, fc_fmt, head_fmt;
  int32_t max_seqs, max_ctx;
  /* row convolutions (dflash.rs Geometry conv_group / conv_kernel; 0: none): the kernel
   * projections are in conv_fmt */
  int32_t conv_group, conv_kernel, conv_fmt;
  /* the K/V cache keeps every element as f16 (1) instead of f32 (0) */
  int32_t kv_f16;
  /* context rows that may wait unsettled (dflash.rs PENDING_ROWS; 0: none wait) */
  int32_t pending_rows;
} og_geometry;

/* canonical matrix: F32 float [rows][cols]; Q4_32 uint8 [rows][cols/2] (low nibble = even
 * column) + f16 bits [rows][cols/32]; Q8_32 int8 [rows][cols] + f16 bits [rows][cols/32]. */
typedef struct {
  const void* codes;
  const uint16_t* scales;
} og_matrix;

typedef struct {
  const float *in_norm, *post_norm, *q_norm, *k_norm;
  og_matrix q, k, v, o, gate, up, down;
  /* with row convolutions: kernel projections [2*conv_kernel*hidden/conv_group][hidden] and
   * static kernels [2][conv_kernel][hidden] of the attention's and the MLP's convolution */
  og_matrix attn_kp, mlp_kp;
  const float *attn_base, *mlp_base;
} og_layer;

typedef struct {
  og_matrix fc, head;
  const float *hidden_norm, *norm;
  const og_layer* layer; /* [layers] */
} og_weights;

typedef struct og_model og_model;

void og_set_threads(int n);
int og_get_threads(void);

/* ---- unit steps (each is what the model functions below call) ---- */
double og_f16_to_f64(uint16_t h);
/* x rounded to the nearest IEEE binary16 value, ties to even (overflow to +-inf), as a double */
double og_round_f16(float x);
void og_inv_freq(double theta, int head_dim, float* out /* [head_dim/2] */);
void og_rmsnorm_row(const float* x, const float* w, int n, float eps, float* y);
void og_rope_head(float* x, int head_dim, int64_t pos, const float* inv_freq);
void og_quant_act_row(const float* x, int n, int8_t* q, float* d /* [n/32] */);
/* y[m][rows] = W . x[m]: quantized W times A8_32 activations (codes xq [m][cols], scales dx
 * [m][cols/32]); exact int32 group sums, f64 accumulation, one rounding to f32. */
void og_matmul_q(int fmt, og_matrix w, int rows, int cols, const int8_t* xq, const float* dx, int m, float* y);
/* per-group integer sums s[m][rows][cols/32] = sum over the group of q_w * q_x */
void og_group_sums(int fmt, og_matrix w, int rows, int cols, const int8_t* xq, int m, int32_t* s);
/* y[m][rows] = W . x[m] for an f32 matrix, f64 accumulation */
void og_matmul_f32(const float* w, int rows, int cols, const float* x, int m, float* y);
/* attention of nq query rows over nk keys: y = softmax(q k^T * scale) v, all f64 inside;
 * p (optional, [nq][nk]) receives the probabilities. */
void og_attend(const float* q, int nq, const float* k, const float* v, int nk, int head_dim, float scale,
               float* y, double* p);
void og_silu_mul(const float* g, const float* u, int n, float* a);
/* one stage of a grouped causal row convolution over the rows of one block (dflash.rs,
 * Drafter::conv): y[r][i] = sum over o < min(kn, r+1) of (base[stage][o][i] +
 * d[r][stage][o][i/gs]) * x[r-o][i]; d is [rows][2*kn*(hidden/gs)]; f64 inside, f32 out */
void og_row_conv(const float* x, int rows, int hidden, int gs, int kn, int stage, const float* base,
                 const float* d, float* y);

/* ---- the drafter ---- */
og_model* og_create(const og_geometry* g, const og_weights* w);
void og_destroy(og_model* m);
int og_ctx_append(og_model* m, int seq, int64_t pos, const float* taps /* [n][n_taps*hidden] */, int n);
/* the same rows queued (Drafter::queue_context: they wait, the oldest settled past pending_rows),
 * and every waiting row settled (Drafter::settle); og_pending: rows waiting.  A block settles the
 * waiting rows of its sequences first. */
int og_ctx_queue(og_model* m, int seq, int64_t pos, const float* taps, int n);
int og_ctx_settle(og_model* m, int seq);
int64_t og_pending(const og_model* m, int seq);
int og_ctx_truncate(og_model* m, int seq, int64_t pos);
int og_ctx_reset(og_model* m, int seq);
int og_ctx_span(const og_model* m, int seq, int64_t* first, int64_t* end);
/* K and V of context rows (index = position - first) for one layer: [n][kv_heads][head_dim] */
int og_read_kv(const og_model* m, int layer, int seq, int row0, int n, float* k, float* v);
/* Per-layer attention options (dflash.rs Geometry: window / windows, no_rope; window_of,
 * rotary): windows[l] = positions a block row of layer l sees back (0: all), rotary[l] = 0 for a
 * layer whose queries and keys carry no rotary position.  NULL keeps the default (0 / 1).
 * Accepted only while every sequence holds no context rows (-1 otherwise, or on a negative
 * window). */
int og_set_layer_options(og_model* m, const int32_t* windows, const int32_t* rotary);
/* rows of layer l's context that fell out of its window and were dropped (Drafter::settle_rows) */
int64_t og_dropped(const og_model* m, int seq, int layer);
/* logits[s][block][vocab] of the block rows h[s][block][hidden] anchored at anchors[s] */
int og_block_forward(og_model* m, int n_seqs, const int32_t* seqs, const int64_t* anchors, const float* h,
                     float* logits);
/* the same with the block cut to its first block_rows rows (h [s][block_rows][hidden]) and the
 * head over its first head_rows rows (a shortlist): logits[s][block_rows][head_rows] */
int og_block_forward_rows(og_model* m, int n_seqs, const int32_t* seqs, const int64_t* anchors, const float* h,
                          int block_rows, int head_rows, float* logits);
/* the same, stopping after the final norm: hidden[s][block][hidden] */
int og_block_hidden(og_model* m, int n_seqs, const int32_t* seqs, const int64_t* anchors, const float* h,
                    float* hidden);

/* ---- candidate selection (dflash.rs, top_k and Drafter::select_with) ---- */
/* The k largest of x[0..n) with their indices, largest first; of equal values the earlier index
 * comes first.  k <= n.  vals/idx [k]. */
void og_top_k(const float* x, int n, int k, float* vals, int32_t* idx);
/* Greedy left-to-right choice of the draft tokens of `rows` rows: row j's candidates are the top
 * `top` of its logits (logits + j*ld, width entries); each is scored in f32 as
 *   logit + sum_r (pred[prev][r] * hp[j][r]) * succ[tok][r]   (the sum from r = 0 upward)
 * where prev is the token chosen for the row before (anchor for row 0) and pred/succ are f16 bit
 * patterns [vocab][rank]; the first candidate with the largest score is chosen.  chosen/plain
 * [rows] receive the chosen tokens and each row's own top token. */
void og_select(const float* logits, int rows, int width, int ld, const float* hp, int rank,
               const uint16_t* pred, const uint16_t* succ, int top, int32_t anchor, int32_t* chosen,
               int32_t* plain);

#ifdef __cplusplus
}
#endif
#endif
