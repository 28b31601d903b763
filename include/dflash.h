/* dflash.h -- C ABI of the MI355X (gfx950) DFlash 2 block-drafter library.
 *
 * What it computes (cortiq-engine "dflash.rs", module header; Drafter::settle_rows and
 * Drafter::block): a drafter of a few Qwen3-shaped layers keeps, per position of its context,
 *     t   = RMSNorm(FC . taps, hidden_norm)            taps = the target's tapped layer outputs
 *     K_l = RoPE(RMSNorm(Wk_l . t, k_norm_l), pos)     V_l = Wv_l . t        for every layer l
 * and a block of rows [anchor, MASK, ..., MASK] at positions a, a+1, ... runs through the
 * layers (RMSNorm, Wq/Wk/Wv, q/k RMSNorm, RoPE, attention over the context before a and the
 * block's own rows -- not causal --, Wo + residual, RMSNorm, SwiGLU MLP + residual), then
 * logits = Head . RMSNorm(h, norm) for every block row (row j >= 1 drafts position a + j).
 *
 * Matrices come in three formats (the pages name a 4-bit and an 8-bit format without their
 * bytes, gpu_wgpu/dflash_dev.rs kind_of; these layouts are this library's contract):
 *   DFLASH_F32    float [rows][cols], activations stay f32;
 *   DFLASH_Q4_32  per row and group of 32 columns one IEEE f16 scale d and 32 signed 4-bit
 *                 codes q (weight = d*q): codes uint8 [rows][cols/2], column 2j in the low
 *                 nibble of byte j; scales f16 [rows][cols/32];
 *   DFLASH_Q8_32  the same with int8 codes [rows][cols].
 * Before a quantized matrix the activations are quantized per row and group of 32 (A8_32):
 *   amax = max|x|; d = amax/127 and inv = 127/amax (f32 divisions);
 *   q = clamp(rint(x*inv), -127, 127) (f32 product, ties to even); amax == 0 -> d = 0, q = 0.
 * The quantized product sums q_w*q_x exactly per group and scales each group's sum by
 * d_w*d_x (gpu_wgpu/dflash_dev.rs, Dev::q4: int8 activations per group of 32).
 *
 * Conventions for every call:
 *  - Device pointers are device-global memory of the GPU current when dflash_create ran
 *    (e.g. torch tensors' data_ptr()); host pointers are marked "host".
 *  - All GPU work of a ctx is enqueued on its stream (dflash_create / dflash_set_stream) and
 *    nothing synchronizes except dflash_create; a call returns once its work is enqueued.
 *  - Every call checks its arguments on the host before enqueueing anything and, on error,
 *    returns a negative status with the ctx state unchanged (dflash_last_error says why).  A
 *    launch the runtime refuses after that (DFLASH_EHIP) leaves the context's rows undefined:
 *    reset the sequences involved (or destroy the ctx) before using them again.
 *  - The library never allocates device memory: the caller hands dflash_create one workspace
 *    buffer (packed weights, K/V cache, activations) and owns it, the taps, block inputs and
 *    logits.  Borrowed buffers must stay valid until the work enqueued on them has run.
 *  - Not thread safe: one ctx is used by one host thread at a time.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum dflash_status {
  DFLASH_OK = 0,
  DFLASH_EINVAL = -1,    /* a bad argument (null pointer, out-of-range index, ...) */
  DFLASH_ECAPACITY = -2, /* the context would exceed max_ctx rows of a sequence */
  DFLASH_EHIP = -3,      /* the HIP runtime reported an error */
  DFLASH_ENOTSUP = -4    /* a geometry outside the kernels' limits */
};

enum dflash_format { DFLASH_F32 = 0, DFLASH_Q4_32 = 1, DFLASH_Q8_32 = 2 };

/* The drafter's geometry (cortiq-engine dflash.rs, struct Geometry, minus the row
 * convolutions, the selector, windows and target binding) plus the cache's capacity.
 * Limits: layers >= 1; 2 <= block <= 16; heads % kv_heads == 0 and heads/kv_heads <= 16;
 * head_dim 64 or 128; hidden, heads*head_dim, intermediate and n_taps*hidden multiples of 128
 * (of 4 for f32 matrices); vocab a multiple of 16; max_seqs*block <= 128; max_ctx >= 0 and
 * max_ctx * head_dim * (2 for an f16 cache, else 4) < 2^31 (DFLASH_ENOTSUP past that). */
typedef struct {
  double rope_theta; /* RoPE base (inv_freq[i] = theta^(-2i/head_dim)) */
  double eps;        /* RMSNorm epsilon, applied in f32 */
  int32_t layers, hidden, heads, kv_heads, head_dim, intermediate, vocab, block, n_taps;
  int32_t body_fmt; /* Wq, Wk, Wv, Wo, gate, up, down */
  int32_t fc_fmt;   /* FC [hidden][n_taps*hidden] */
  int32_t head_fmt; /* head [vocab][hidden] */
  int32_t max_seqs; /* independent sequences (separate contexts, shared weights) */
  int32_t max_ctx;  /* context rows a sequence can hold */
  /* Row convolutions around the attention and the MLP (dflash.rs, Geometry conv_group /
   * conv_kernel; Drafter::conv_in and Drafter::conv).  conv_kernel 0: none (the plain Qwen3
   * layer; the conv fields of the weights are then ignored).  Else conv_group divides hidden,
   * the kernel projections have 2*conv_kernel*hidden/conv_group rows (a multiple of 16) and
   * conv_fmt is DFLASH_F32 with an f32 body, DFLASH_Q4_32 / DFLASH_Q8_32 with a quantized one. */
  int32_t conv_group, conv_kernel, conv_fmt;
  /* 1: the K/V cache keeps each element as f16 (the f32 value rounded to nearest even; half
   * the bytes), 0: f32 */
  int32_t kv_f16;
  /* context rows a sequence may keep waiting, unsettled (dflash.rs PENDING_ROWS, 512 there;
   * dflash_ctx_queue); 0: every row settles at once.  Each sequence gets a device ring of
   * pending_rows * n_taps * hidden f32 in the workspace. */
  int32_t pending_rows;
} dflash_geometry;

/* A matrix in the canonical layout above (device pointers; scales NULL for DFLASH_F32). */
typedef struct {
  const void* codes;
  const void* scales;
} dflash_matrix;

typedef struct {
  const float *in_norm, *post_norm; /* [hidden] */
  const float *q_norm, *k_norm;     /* [head_dim] */
  dflash_matrix q;                  /* [heads*head_dim][hidden] */
  dflash_matrix k, v;               /* [kv_heads*head_dim][hidden] */
  dflash_matrix o;                  /* [hidden][heads*head_dim] */
  dflash_matrix gate, up;           /* [intermediate][hidden] */
  dflash_matrix down;               /* [hidden][intermediate] */
  /* with row convolutions: the kernel projections [2*conv_kernel*(hidden/conv_group)][hidden]
   * (conv_fmt) of the attention's and the MLP's convolution, and their static kernels
   * [2][conv_kernel][hidden] (stage 0 before the sub-layer, stage 1 after) */
  dflash_matrix attn_kp, mlp_kp;
  const float *attn_base, *mlp_base;
} dflash_layer_weights;

typedef struct {
  dflash_matrix fc, head;
  const float *hidden_norm, *norm;   /* [hidden] */
  const dflash_layer_weights* layer; /* host array [layers] */
} dflash_weights;

typedef struct dflash_ctx dflash_ctx;

/* Bytes of workspace dflash_create needs for g (packed weights, the K/V cache of max_seqs x
 * max_ctx rows in f32, activations).  *bytes receives the size. */
int dflash_workspace_bytes(const dflash_geometry* g, size_t* bytes);

/* Build a drafter: checks g, carves `workspace` (device, >= dflash_workspace_bytes, 256-byte
 * aligned), repacks every matrix of w into the kernels' tiled layout inside it, copies the norm
 * weights, computes the RoPE table, and waits for that work on `stream` (a hipStream_t, or NULL
 * for the default stream) so w may be freed on return.  Every sequence starts empty at
 * position 0.  *out receives the ctx (free it with dflash_destroy; the workspace stays the
 * caller's). */
int dflash_create(const dflash_geometry* g, const dflash_weights* w, void* workspace, size_t bytes, void* stream,
                  dflash_ctx** out);

/* Later calls enqueue on `stream` (hipStream_t; NULL = default stream).  A different stream first
 * waits (on the device, through an event) for the work already enqueued on the old one, since
 * both use the same workspace; the host does not wait. */
int dflash_set_stream(dflash_ctx* c, void* stream);

/* Add context rows (cortiq-engine dflash.rs, Drafter::push_context / queue_context /
 * settle_rows): `taps` is device [n][n_taps*hidden] f32, the rows of positions pos..pos+n-1.
 * If first <= pos <= first+len, positions >= pos are forgotten first; if pos < first or
 * pos > first+len the sequence starts over with first = pos.  Each row's K and V (every
 * layer, k-norm and RoPE at its absolute position) go to the device cache at index
 * position - first.  n == 0 only applies that bookkeeping.  DFLASH_ECAPACITY if the sequence
 * would pass max_ctx rows (nothing changes then). */
int dflash_ctx_append(dflash_ctx* c, int32_t seq, int64_t pos, const float* taps, int32_t n);

/* The deferred form of append (dflash.rs, Drafter::queue_context and Drafter::settle).
 * dflash_ctx_queue takes the same arguments and bookkeeping as dflash_ctx_append, with the
 * waiting rows counted in the span, but the rows wait (their taps are copied into the
 * sequence's ring on the ctx stream); once more than pending_rows wait, the oldest are settled,
 * a whole number of 64-row chunks (CONTEXT_CHUNK) at a time.  dflash_ctx_settle settles every
 * waiting row of a sequence; dflash_ctx_append is queue then settle (Drafter::push_context).
 * Every settle applies the window drop once at its end, so the rows a window drops follow the
 * settles.  A block first settles the waiting rows of the sequences it is given.  A truncation
 * forgets waiting rows at positions >= pos too.  dflash_ctx_pending: host *n receives the
 * number of waiting rows. */
int dflash_ctx_queue(dflash_ctx* c, int32_t seq, int64_t pos, const float* taps, int32_t n);
int dflash_ctx_settle(dflash_ctx* c, int32_t seq);
int dflash_ctx_pending(const dflash_ctx* c, int32_t seq, int64_t* n);

/* Per-layer attention options (dflash.rs, Geometry window / windows / no_rope with window_of
 * and rotary): windows host [layers], positions a block row of that layer sees back (0: all of
 * them; row r of a block anchored at a sees context positions >= a + r + 1 - w, and all block
 * rows); rotary host [layers], 0 for a layer whose queries and keys carry no rotary position.
 * NULL keeps the default (0, resp. 1 for every layer).  After every append a windowed layer
 * holding more than twice its window drops its oldest rows down to one window
 * (Drafter::settle_rows); dropped rows are never read again (a truncation clips the count to
 * what it keeps).  The cache keeps its max_ctx rows per sequence: dropping frees no memory.
 * Allowed only while no sequence holds context rows, and at most 64 layers may be unrotated;
 * otherwise DFLASH_EINVAL with nothing changed. */
int dflash_set_layer_options(dflash_ctx* c, const int32_t* windows, const int32_t* rotary);

/* How the block-vs-context attention scores its context keys (the attention step of dflash.rs,
 * Drafter::block).  Both modes round the f64-evaluated softmax-weighted sum once to f32; the
 * scores' dot products lie within f64 rounding of the exact ones (F64) or within
 * 2^-41 * 2^(Eq+Ek) of them, where 2^Eq and 2^Ek are the powers of two just above twice the
 * two rows' largest magnitudes (DIGITS).  The outputs agree except where an exact value lies
 * within that difference of an f32 rounding boundary.
 * DFLASH_SCORES_F64: f64 products of the f32 queries and keys.
 * DFLASH_SCORES_DIGITS: exact int8 digit splits of the queries and keys (seven base-128 digits a
 * value) multiplied on the int8 matrix unit, the digit sums combined in f64; available where
 * head_dim is 128 and every kv head has four q heads, the key digits then kept beside the cache.
 * DFLASH_SCORES_AUTO (the default): digits from 16384 context rows in a call (over all its
 * sequences), f64 below.  A mode the geometry cannot take: DFLASH_EINVAL, nothing changed. */
enum { DFLASH_SCORES_AUTO = 0, DFLASH_SCORES_F64 = 1, DFLASH_SCORES_DIGITS = 2 };
int dflash_set_score_mode(dflash_ctx* c, int32_t mode);

/* host *mode receives what the last block call scored its context keys with:
 * DFLASH_SCORES_F64 or DFLASH_SCORES_DIGITS (DFLASH_SCORES_AUTO before the first call).
 * A null ctx or mode: DFLASH_EINVAL. */
int dflash_last_scores(const dflash_ctx* c, int32_t* mode);

/* host *dropped receives how many of a sequence's oldest context rows layer `layer` dropped. */
int dflash_ctx_dropped(const dflash_ctx* c, int32_t seq, int32_t layer, int64_t* dropped);

/* Forget positions >= pos of a sequence (dflash.rs, Drafter::truncate); the first stays. */
int dflash_ctx_truncate(dflash_ctx* c, int32_t seq, int64_t pos);

/* Empty a sequence and set its first position to 0 (dflash.rs, Drafter::reset). */
int dflash_ctx_reset(dflash_ctx* c, int32_t seq);

/* host *first, *end receive the positions a sequence holds, [first, end) (dflash.rs,
 * Drafter::span and Drafter::next_position: end is the next position to append, waiting rows
 * included). */
int dflash_ctx_span(const dflash_ctx* c, int32_t seq, int64_t* first, int64_t* end);

/* One block for each of n_seqs distinct sequences (dflash.rs, Drafter::block, and the head of
 * the module header): seqs and anchors are host [n_seqs]; h is device [n_seqs][block][hidden]
 * f32, the rows' embeddings ([anchor, MASK...]) at positions anchors[i]+r; logits receives
 * device [n_seqs][block][vocab] f32 for every block row.  Layer l of sequence s attends to its
 * context positions [lo, hi) and to all block rows: base = first + the rows l dropped,
 * hi = max(min(anchor, first+len), base), lo = base, or under a window w
 * clamp(anchor + 1 - w, base, hi) with row r's positions before anchor + r + 1 - w masked.
 * The context is not modified. */
int dflash_block_forward(dflash_ctx* c, int32_t n_seqs, const int32_t* seqs, const int64_t* anchors,
                         const float* h, float* logits);

/* The same block cut to its first block_rows rows, with the head over its first head_rows rows
 * only.  The cut block (gpu_wgpu/dflash_dev.rs, Dev::block: the anchor and the rows after it,
 * eight there) is a whole block of block_rows rows, the attention among block rows included;
 * the shortlist (dflash.rs, Drafter::block_dev: the drafts' head over the table's first rows)
 * is a prefix of the vocabulary.  h is device [n_seqs][block_rows][hidden] f32, logits
 * receives device [n_seqs][block_rows][head_rows] f32.  block_rows in [1, block]; head_rows a
 * multiple of 16 in [16, vocab], or vocab itself; else DFLASH_EINVAL. */
int dflash_block_forward_rows(dflash_ctx* c, int32_t n_seqs, const int32_t* seqs, const int64_t* anchors,
                              const float* h, int32_t block_rows, int32_t head_rows, float* logits);

/* The same block, stopping after the final RMSNorm: hidden receives device
 * [n_seqs][block][hidden] f32 (the rows the head reads; a diagnostic of the block body). */
int dflash_block_hidden(dflash_ctx* c, int32_t n_seqs, const int32_t* seqs, const int64_t* anchors,
                        const float* h, float* hidden);

/* The last error message of c (or of the last failed dflash_create when c is NULL);
 * valid until the next call on c. */
const char* dflash_last_error(const dflash_ctx* c);

void dflash_destroy(dflash_ctx* c);

/* ---- unit entry points (tests and microbenchmarks); each enqueues on `stream` ---- */

/* A8_32 of rows x rows: x device [rows][cols] f32 -> q device [rows][cols] int8 and
 * d device [rows][cols/32] f32.  cols % 32 == 0. */
int dflash_quant_act(const float* x, int32_t rows, int32_t cols, int8_t* q, float* d, void* stream);

/* Bytes of the tiled (packed) form of a [rows][cols] matrix of format fmt. */
int dflash_packed_bytes(int32_t fmt, int32_t rows, int32_t cols, size_t* bytes);

/* Repack a canonical matrix (device) into the tiled form (device, dflash_packed_bytes). */
int dflash_pack(int32_t fmt, int32_t rows, int32_t cols, dflash_matrix w, void* packed, void* stream);

/* y device [m][rows] f32 = W . x through the production weight-streaming kernel, for a packed
 * quantized W and A8_32 activations xq device [m][cols] int8, dx device [m][cols/32] f32;
 * splits: how the kernel divides K among the waves of a workgroup: 0 = the library's choice,
 * 1 = one wave per n-tile, 2..7 = two k-waves per group of four n-tiles, >= 8 = K split over
 * the waves of one n-tile
 * (negative: DFLASH_EINVAL).  m <= 128.  Each output is the f32 rounding of the product's f64
 * accumulation, whatever the split.  `scratch` is device memory of at least
 * dflash_gemm_scratch_bytes() bytes (padded activations and their scales). */
int dflash_gemm_scratch_bytes(int32_t rows, int32_t cols, int32_t m, int32_t splits, size_t* bytes);
int dflash_gemm(int32_t fmt, const void* packed, int32_t rows, int32_t cols, const int8_t* xq, const float* dx,
                int32_t m, float* y, int32_t splits, void* scratch, void* stream);

/* Exact per-group integer sums of the same kernel: sums device [m][rows][cols/32] int32,
 * sum over the group of q_w*q_x (the quantized product's integer accumulators). */
int dflash_group_sums(int32_t fmt, const void* packed, int32_t rows, int32_t cols, const int8_t* xq, int32_t m,
                      int32_t* sums, void* scratch, void* stream);

/* Stage timing (the pages time a block's stages with GPU timestamps; here HIP events on the
 * ctx stream).  dflash_time_stage(c, stage) adds a stage to the timed set (stage < 0 empties
 * the set and forgets every recorded pair): each later launch of a timed stage is bracketed by
 * an event pair.  dflash_read_timing(c, stage, ...) waits for that stage's recorded pairs and
 * returns their summed milliseconds and count, then forgets them.  Stages: */
enum dflash_stage {
  DFLASH_STAGE_HEAD = 0,        /* the head's matrix product (logits) */
  DFLASH_STAGE_QKV = 1,         /* every layer's Wq|Wk|Wv product */
  DFLASH_STAGE_ATTENTION = 2,   /* every layer's attention (chunks + merge) */
  DFLASH_STAGE_O = 3,           /* every layer's Wo product (+ residual) */
  DFLASH_STAGE_GATE_UP = 4,     /* every layer's gate|up product (+ SwiGLU) */
  DFLASH_STAGE_DOWN = 5,        /* every layer's down product (+ residual) */
  DFLASH_STAGE_BLOCK = 6,       /* the whole block call */
  DFLASH_STAGE_APPEND = 7,      /* the whole append call */
  DFLASH_STAGE_ATTN_CHUNKS = 8, /* every layer's attention chunk kernel alone (no merge) */
  DFLASH_STAGE_LAST = 8
};
int dflash_time_stage(dflash_ctx* c, int32_t stage);
int dflash_read_timing(dflash_ctx* c, int32_t stage, double* total_ms, int64_t* count);

/* ---- Candidate selection (cortiq-engine dflash.rs: top_k, Drafter::select_with) ----
 *
 * dflash_top_k: the k largest entries of each of `rows` rows of x (device f32, row r at
 * x + r*ld, `width` entries, ld >= width) with their indices, largest first and, among equal
 * values, the earlier index first (the order the pages' top_k list keeps).  vals device
 * [rows][k] f32, idx device [rows][k] int32; vals[r][i] compares equal to the entry at
 * idx[r][i] (a -0 entry ties with +0 and comes back as +0).  1 <= k <= min(width, 64) and
 * ceil(width / 4096) * k <= 4096 (the chunks' lists of a row fit one merge; with k = 64 width is
 * at most 262144); values must be finite.
 * `scratch`: device memory of dflash_top_k_scratch_bytes() bytes.
 *
 * dflash_select: the draft tokens of `rows` rows from their logits (device, as for top_k; row j
 * is the block row j + 1 when the anchor's row is left out) under the candidate selector:
 * row j's candidates are its top `top` logits; candidate t scores, in f32 and in this order,
 *   logit_t + (sum over r = 0, 1, ..., rank-1 of (pred[prev][r] * hp[j][r]) * succ[t][r])
 * with every product and sum rounded on its own; the first candidate with the largest score is
 * chosen and becomes prev for row j + 1 (prev = anchor, a token id, for row 0).  hp device
 * [rows][rank] f32 (the selector's projection of the rows); pred/succ device [vocab][rank] f16
 * bit patterns (the predecessor and successor codebooks); width <= vocab (candidates index the
 * codebooks).  chosen/plain device [rows] int32: the chosen tokens and each row's own top token.
 * 1 <= top <= 64, 1 <= rank <= 4096, 0 <= anchor < vocab.  `scratch`: device memory of
 * dflash_select_scratch_bytes() bytes.  All four return DFLASH_EINVAL on bad arguments (nothing
 * enqueued) and DFLASH_EHIP on a launch error; work goes on `stream` and is not waited for. */
int dflash_top_k_scratch_bytes(int32_t rows, int32_t width, int32_t k, size_t* bytes);
int dflash_top_k(const float* x, int32_t rows, int32_t width, int32_t ld, int32_t k, float* vals, int32_t* idx,
                 void* scratch, void* stream);
/* dflash_top_k without caller scratch, for callers that cannot allocate device memory (code
 * under graph capture, serving loops that forbid allocation): the same arguments, kernels and
 * results as dflash_top_k, with the chunk lists kept in a fixed 1 MiB device array of the library
 * (each GPU holds its own copy until the process ends; nothing is allocated per call).  Sizes
 * with rows * ceil(width / 4096) * k > 131072 return DFLASH_EINVAL with nothing enqueued.  Every
 * call on one GPU uses that GPU's one array: calls that overlap on one GPU (other streams, other
 * host threads) race and must be ordered by the caller. */
int dflash_top_k_noalloc(const float* x, int32_t rows, int32_t width, int32_t ld, int32_t k, float* vals,
                         int32_t* idx, void* stream);
int dflash_select_scratch_bytes(int32_t rows, int32_t width, int32_t top, size_t* bytes);
int dflash_select(const float* logits, int32_t rows, int32_t width, int32_t ld, const float* hp, int32_t rank,
                  const uint16_t* pred, const uint16_t* succ, int32_t vocab, int32_t top, int32_t anchor,
                  int32_t* chosen, int32_t* plain, void* scratch, void* stream);

/* Copy K and V of context rows row0..row0+n-1 (index = position - first) of one layer and
 * sequence into device k, v [n][kv_heads][head_dim] f32 (a read-back of the cache; an f16
 * cache's elements converted exactly). */
int dflash_read_kv(const dflash_ctx* c, int32_t layer, int32_t seq, int32_t row0, int32_t n, float* k, float* v);

#ifdef __cplusplus
}
#endif
#endif
