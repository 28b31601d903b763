/* DFlash 2 block drafter -- CPU oracle (TEST INFRASTRUCTURE ONLY; see dflash_oracle.h).
 *
 * Sources: the docs.rs source pages of the Rust crate cortiq-engine --
 *   "dflash.rs" (0.8.71): the module header (the method in brief), fn rms, Drafter::new
 *   (inv_freq), Drafter::rotate, Drafter::mlp, Drafter::queue_context / truncate / reset,
 *   Drafter::settle_rows (context append), Drafter::block (the block forward);
 *   "gpu_wgpu/dflash_dev.rs" (0.8.75): the module header (the device block keeps the host
 *   block's f32 arithmetic), Dev::q4 (int8 activations per group of 32).
 * Readings where those pages are silent (formats, the activation quantizer, which rows get
 * logits, eps/theta) are this project's contract, restated at each function.
 *
 * Precision: f64 inside every step, f32 storage between steps (the pages keep f32 buffers),
 * except where the pages fix the arithmetic: RMSNorm's scale and products (fn rms), the RoPE
 * angle (Drafter::rotate), the attention scale (Drafter::block) and the activation quantizer's
 * f32 decisions.  Built without fast-math and with fp-contract off, so every expression is
 * rounded as written.
 */
#include "dflash_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int g_threads = 1;

void og_set_threads(int n) { g_threads = n < 1 ? 1 : n; }
int og_get_threads(void) { return g_threads; }

/* IEEE 754 binary16 -> value, from the format's definition (sign, 5-bit biased exponent,
 * 10-bit fraction; exponent 0 subnormal, 31 inf/nan). */
double og_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1, e = (h >> 10) & 31, f = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24);
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + f), e - 25);
  return sign ? -v : v;
}

/* dflash.rs, Drafter::new: inv_freq[i] = theta^(-2i/hd) evaluated in f64, stored f32. */
/* IEEE 754 binary16, round to nearest with ties to even: the value's binade [2^(e-1), 2^e)
 * holds 1024 steps of 2^(e-11), never finer than the subnormal step 2^-24; x / step is exact
 * in f64, so rounding it to an integer (nearbyint under the default mode: ties to even) and
 * scaling back gives the rounded value.  Past the largest finite half, 65504, values from 65520
 * (the tie with 65536, whose even neighbour is out of range) overflow to infinity. */
double og_round_f16(float xf) {
  const double x = xf, a = fabs(x);
  if (isnan(x)) return x;
  if (a >= 65520.0) return copysign(INFINITY, x);
  if (a == 0.0) return x;
  int e;
  (void)frexp(a, &e); /* a = m * 2^e, m in [0.5, 1) */
  const double step = ldexp(1.0, e - 11 > -24 ? e - 11 : -24);
  return copysign(nearbyint(a / step) * step, x);
}

void og_inv_freq(double theta, int head_dim, float* out) {
  for (int i = 0; i < head_dim / 2; i++) out[i] = (float)pow(theta, -(2.0 * i) / (double)head_dim);
}

/* dflash.rs, fn rms: mean of squares accumulated in f64; s = 1/sqrt(f32(ms) + eps) in f32;
 * each element (x * s) * w in f32. */
void og_rmsnorm_row(const float* x, const float* w, int n, float eps, float* y) {
  double ms = 0.0;
  for (int i = 0; i < n; i++) ms += (double)x[i] * (double)x[i];
  ms /= (double)n;
  float s = 1.0f / sqrtf((float)ms + eps);
  for (int i = 0; i < n; i++) {
    float t = x[i] * s;
    y[i] = t * w[i];
  }
}

/* dflash.rs, Drafter::rotate: half-split pairs (i, i + hd/2); the angle is the f32 product
 * f32(pos) * inv_freq[i]; lo' = a cos - b sin, hi' = b cos + a sin.  cos/sin and the rotation
 * are evaluated in f64 on that f32 angle. */
void og_rope_head(float* x, int head_dim, int64_t pos, const float* inv_freq) {
  int half = head_dim / 2;
  float p = (float)pos;
  for (int i = 0; i < half; i++) {
    float ang = p * inv_freq[i];
    double c = cos((double)ang), s = sin((double)ang);
    double a = x[i], b = x[i + half];
    x[i] = (float)(a * c - b * s);
    x[i + half] = (float)(b * c + a * s);
  }
}

/* Activations before a quantized matrix: int8 per row and group of 32 consecutive columns
 * (gpu_wgpu/dflash_dev.rs, Dev::q4: "int8 activations", 32 codes plus side data per group).
 * The pages give no rounding rule, so this is the contract: amax = max |x| of the group;
 * d = amax / 127 and inv = 127 / amax as f32 divisions; q = clamp(rint(x * inv), -127, 127)
 * with the f32 product rounded to nearest even; a zero group has d = 0 and q = 0. */
void og_quant_act_row(const float* x, int n, int8_t* q, float* d) {
  for (int g = 0; g < n / 32; g++) {
    const float* xs = x + 32 * g;
    float amax = 0.0f;
    for (int i = 0; i < 32; i++) {
      float a = fabsf(xs[i]);
      if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
      d[g] = 0.0f;
      for (int i = 0; i < 32; i++) q[32 * g + i] = 0;
      continue;
    }
    d[g] = amax / 127.0f;
    float inv = 127.0f / amax;
    for (int i = 0; i < 32; i++) {
      float t = xs[i] * inv;
      float r = nearbyintf(t); /* default rounding mode: to nearest, ties to even */
      if (r > 127.0f) r = 127.0f;
      if (r < -127.0f) r = -127.0f;
      q[32 * g + i] = (int8_t)r;
    }
  }
}

/* the integer code of column k of row r */
static int code_at(int fmt, og_matrix w, int cols, int r, int k) {
  if (fmt == OG_Q8_32) return ((const int8_t*)w.codes)[(size_t)r * cols + k];
  uint8_t b = ((const uint8_t*)w.codes)[(size_t)r * (cols / 2) + k / 2];
  int nib = (k & 1) ? (b >> 4) : (b & 15);
  return nib >= 8 ? nib - 16 : nib;
}

/* Quantized matrix times A8_32 activations: for each group, s = sum q_w * q_x exactly; then
 * y = sum over groups of f16(d_w) * d_x * s, accumulated in f64 and rounded once. */
void og_matmul_q(int fmt, og_matrix w, int rows, int cols, const int8_t* xq, const float* dx, int m, float* y) {
  int groups = cols / 32;
#pragma omp parallel for schedule(static) num_threads(g_threads)
  for (int r = 0; r < rows; r++) {
    int8_t* wr = (int8_t*)malloc((size_t)cols);
    double* dw = (double*)malloc(sizeof(double) * (size_t)groups);
    for (int k = 0; k < cols; k++) wr[k] = (int8_t)code_at(fmt, w, cols, r, k);
    for (int g = 0; g < groups; g++) dw[g] = og_f16_to_f64(w.scales[(size_t)r * groups + g]);
    for (int i = 0; i < m; i++) {
      const int8_t* xr = xq + (size_t)i * cols;
      double acc = 0.0;
      for (int g = 0; g < groups; g++) {
        int s = 0;
        for (int k = 32 * g; k < 32 * g + 32; k++) s += (int)wr[k] * (int)xr[k];
        acc += dw[g] * (double)dx[(size_t)i * groups + g] * (double)s;
      }
      y[(size_t)i * rows + r] = (float)acc;
    }
    free(dw);
    free(wr);
  }
}

void og_group_sums(int fmt, og_matrix w, int rows, int cols, const int8_t* xq, int m, int32_t* s) {
  int groups = cols / 32;
  for (int i = 0; i < m; i++)
    for (int r = 0; r < rows; r++)
      for (int g = 0; g < groups; g++) {
        int acc = 0;
        for (int k = 32 * g; k < 32 * g + 32; k++) acc += code_at(fmt, w, cols, r, k) * (int)xq[(size_t)i * cols + k];
        s[((size_t)i * rows + r) * groups + g] = acc;
      }
}

void og_matmul_f32(const float* w, int rows, int cols, const float* x, int m, float* y) {
#pragma omp parallel for schedule(static) num_threads(g_threads)
  for (int r = 0; r < rows; r++) {
    const float* wr = w + (size_t)r * cols;
    for (int i = 0; i < m; i++) {
      const float* xr = x + (size_t)i * cols;
      double acc = 0.0;
      for (int k = 0; k < cols; k++) acc += (double)wr[k] * (double)xr[k];
      y[(size_t)i * rows + r] = (float)acc;
    }
  }
}

/* dflash.rs, Drafter::block (the per-head scores, softmax and values): s = (q . k) * scale,
 * p = exp(s - max) / sum, y = sum p v; in f64. */
void og_attend(const float* q, int nq, const float* k, const float* v, int nk, int head_dim, float scale,
               float* y, double* p) {
  double* s = (double*)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
  for (int i = 0; i < nq; i++) {
    const float* qi = q + (size_t)i * head_dim;
    double top = -INFINITY;
    for (int j = 0; j < nk; j++) {
      double dot = 0.0;
      for (int d = 0; d < head_dim; d++) dot += (double)qi[d] * (double)k[(size_t)j * head_dim + d];
      s[j] = dot * (double)scale;
      if (s[j] > top) top = s[j];
    }
    double sum = 0.0;
    for (int j = 0; j < nk; j++) {
      s[j] = exp(s[j] - top);
      sum += s[j];
    }
    for (int j = 0; j < nk; j++) {
      s[j] /= sum;
      if (p) p[(size_t)i * nk + j] = s[j];
    }
    for (int d = 0; d < head_dim; d++) {
      double acc = 0.0;
      for (int j = 0; j < nk; j++) acc += s[j] * (double)v[(size_t)j * head_dim + d];
      y[(size_t)i * head_dim + d] = (float)acc;
    }
  }
  free(s);
}

/* dflash.rs, Drafter::mlp: a = g / (1 + e^-g) * u, in f64, stored f32. */
void og_silu_mul(const float* g, const float* u, int n, float* a) {
  for (int i = 0; i < n; i++) {
    double gv = g[i];
    a[i] = (float)(gv / (1.0 + exp(-gv)) * (double)u[i]);
  }
}

/* dflash.rs, Drafter::conv: row r of the output mixes rows r, r-1, ..., r-kn+1 of the block
 * (fewer near its start), column by column, with the static kernel of that offset plus the
 * row's dynamic kernel of the column's group; the sum is taken in f64 and rounded once. */
void og_row_conv(const float* x, int rows, int hidden, int gs, int kn, int stage, const float* base,
                 const float* d, float* y) {
  const int groups = hidden / gs, pr = 2 * kn * groups;
  for (int r = 0; r < rows; r++)
    for (int i = 0; i < hidden; i++) {
      double acc = 0.0;
      for (int o = 0; o < kn && o <= r; o++) {
        const int so = stage * kn + o;
        const double k = (double)base[(size_t)so * hidden + i] + (double)d[(size_t)r * pr + (size_t)so * groups + i / gs];
        acc += k * (double)x[(size_t)(r - o) * hidden + i];
      }
      y[(size_t)r * hidden + i] = (float)acc;
    }
}

/* ------------------------------------------------------------------------------------------ */

typedef struct {
  int64_t first, len;
  int64_t npend;    /* rows waiting to be settled, at positions first+len, ... */
  float* pend;      /* their taps [npend][n_taps*hidden] */
  int64_t* dropped; /* [layers]: context rows a layer no longer holds (the oldest) */
  float* k;         /* [layers][max_ctx][kv_heads][head_dim] */
  float* v;
} og_seq;

struct og_model {
  og_geometry g;
  og_weights w;
  og_layer* layers;
  float* inv_freq;
  int32_t* window; /* [layers] positions a block row sees back, 0 = all */
  int32_t* rotary; /* [layers] 0 = no rotary position */
  og_seq* seqs;
};

static size_t seq_floats(const og_geometry* g) {
  return (size_t)g->layers * (size_t)g->max_ctx * (size_t)g->kv_heads * (size_t)g->head_dim;
}

og_model* og_create(const og_geometry* g, const og_weights* w) {
  if (!g || !w || g->layers <= 0 || g->block < 1 || g->kv_heads <= 0 || g->heads % g->kv_heads ||
      g->head_dim % 2 || g->max_seqs <= 0 || g->max_ctx < 0 || g->conv_kernel < 0 ||
      (g->conv_kernel > 0 && (g->conv_group <= 0 || g->hidden % g->conv_group)))
    return NULL;
  og_model* m = (og_model*)calloc(1, sizeof(og_model));
  m->g = *g;
  m->w = *w;
  m->layers = (og_layer*)malloc(sizeof(og_layer) * (size_t)g->layers);
  memcpy(m->layers, w->layer, sizeof(og_layer) * (size_t)g->layers);
  m->w.layer = m->layers;
  m->inv_freq = (float*)malloc(sizeof(float) * (size_t)(g->head_dim / 2));
  og_inv_freq(g->rope_theta, g->head_dim, m->inv_freq);
  m->window = (int32_t*)calloc((size_t)g->layers, sizeof(int32_t));
  m->rotary = (int32_t*)malloc(sizeof(int32_t) * (size_t)g->layers);
  for (int l = 0; l < g->layers; l++) m->rotary[l] = 1;
  m->seqs = (og_seq*)calloc((size_t)g->max_seqs, sizeof(og_seq));
  for (int s = 0; s < g->max_seqs; s++) {
    m->seqs[s].dropped = (int64_t*)calloc((size_t)g->layers, sizeof(int64_t));
    m->seqs[s].k = (float*)calloc(seq_floats(g) ? seq_floats(g) : 1, sizeof(float));
    m->seqs[s].v = (float*)calloc(seq_floats(g) ? seq_floats(g) : 1, sizeof(float));
  }
  return m;
}

void og_destroy(og_model* m) {
  if (!m) return;
  for (int s = 0; s < m->g.max_seqs; s++) {
    free(m->seqs[s].dropped);
    free(m->seqs[s].pend);
    free(m->seqs[s].k);
    free(m->seqs[s].v);
  }
  free(m->seqs);
  free(m->rotary);
  free(m->window);
  free(m->inv_freq);
  free(m->layers);
  free(m);
}

/* dflash.rs, Geometry::window_of and Geometry::rotary: the per-layer options */
int og_set_layer_options(og_model* m, const int32_t* windows, const int32_t* rotary) {
  for (int s = 0; s < m->g.max_seqs; s++)
    if (m->seqs[s].len > 0) return -1;
  for (int l = 0; l < m->g.layers; l++)
    if (windows && windows[l] < 0) return -1;
  for (int l = 0; l < m->g.layers; l++) {
    m->window[l] = windows ? windows[l] : 0;
    m->rotary[l] = rotary ? (rotary[l] != 0) : 1;
  }
  return 0;
}

int64_t og_dropped(const og_model* m, int seq, int layer) {
  if (seq < 0 || seq >= m->g.max_seqs || layer < 0 || layer >= m->g.layers) return -1;
  return m->seqs[seq].dropped[layer];
}

/* dflash.rs, Drafter::truncate: keep positions before pos (the first stays); a layer's dropped
 * rows are clipped to what is kept */
static void keep_rows(og_model* m, og_seq* s, int64_t keep) {
  for (int l = 0; l < m->g.layers; l++)
    if (s->dropped[l] > keep) s->dropped[l] = keep;
  s->len = keep;
}

/* y[n][rows] = W . x[n] with x f32: A8_32 first when W is quantized */
static void mm(int fmt, og_matrix w, int rows, int cols, const float* x, int n, float* y) {
  if (fmt == OG_F32) {
    og_matmul_f32((const float*)w.codes, rows, cols, x, n, y);
    return;
  }
  int8_t* xq = (int8_t*)malloc((size_t)n * cols);
  float* dx = (float*)malloc(sizeof(float) * (size_t)n * (cols / 32));
  for (int i = 0; i < n; i++) og_quant_act_row(x + (size_t)i * cols, cols, xq + (size_t)i * cols, dx + (size_t)i * (cols / 32));
  og_matmul_q(fmt, w, rows, cols, xq, dx, n, y);
  free(dx);
  free(xq);
}

/* dflash.rs, Drafter::settle_rows: the rows of positions first+len, ... become context: t =
 * rms(FC . taps, hidden_norm); every layer's k, v of t; k = rotate(rms(k, k_norm), position);
 * then a layer holding more than twice its window keeps only the last window's worth. */
static void settle_rows(og_model* m, og_seq* s, const float* taps, int n) {
  const og_geometry* g = &m->g;
  const int64_t pos = s->first + s->len;
  const int H = g->hidden, T = g->n_taps * g->hidden, kvh = g->kv_heads, hd = g->head_dim, kvd = kvh * hd;
  float* t = (float*)malloc(sizeof(float) * (size_t)n * H);
  float* tn = (float*)malloc(sizeof(float) * (size_t)n * H);
  float* k = (float*)malloc(sizeof(float) * (size_t)n * kvd);
  float* v = (float*)malloc(sizeof(float) * (size_t)n * kvd);
  float* tmp = (float*)malloc(sizeof(float) * (size_t)hd);
  mm(g->fc_fmt, m->w.fc, H, T, taps, n, t);
  for (int i = 0; i < n; i++) og_rmsnorm_row(t + (size_t)i * H, m->w.hidden_norm, H, (float)g->eps, tn + (size_t)i * H);
  for (int l = 0; l < g->layers; l++) {
    const og_layer* L = &m->layers[l];
    mm(g->body_fmt, L->k, kvd, H, tn, n, k);
    mm(g->body_fmt, L->v, kvd, H, tn, n, v);
    for (int i = 0; i < n; i++) {
      int64_t p = pos + i;
      size_t row = (size_t)(p - s->first);
      for (int h = 0; h < kvh; h++) {
        float* kh = k + (size_t)i * kvd + (size_t)h * hd;
        og_rmsnorm_row(kh, L->k_norm, hd, (float)g->eps, tmp);
        if (m->rotary[l]) og_rope_head(tmp, hd, p, m->inv_freq);
        size_t off = (((size_t)l * g->max_ctx + row) * kvh + h) * hd;
        memcpy(s->k + off, tmp, sizeof(float) * hd);
        memcpy(s->v + off, v + (size_t)i * kvd + (size_t)h * hd, sizeof(float) * hd);
        if (g->kv_f16) /* an f16 cache keeps each f32 element rounded to binary16 */
          for (int d = 0; d < hd; d++) {
            s->k[off + d] = (float)og_round_f16(s->k[off + d]);
            s->v[off + d] = (float)og_round_f16(s->v[off + d]);
          }
      }
    }
  }
  s->len += n;
  for (int l = 0; l < g->layers; l++) {
    const int64_t w = m->window[l], held = s->len - s->dropped[l];
    if (w > 0 && held > 2 * w) s->dropped[l] += held - w;
  }
  free(tmp);
  free(v);
  free(k);
  free(tn);
  free(t);
}

/* dflash.rs, Drafter::truncate: forget positions >= pos, the waiting rows among them too (the
 * first stays); a layer's dropped rows are clipped to what is kept */
static void truncate_to(og_model* m, og_seq* s, int64_t pos) {
  const int64_t held = s->first + s->len;
  const int64_t wait = pos > held ? pos - held : 0;
  if (s->npend > wait) s->npend = wait;
  int64_t keep = pos - s->first;
  if (keep < 0) keep = 0;
  if (keep > s->len) keep = s->len;
  keep_rows(m, s, keep);
}

/* dflash.rs, Drafter::queue_context: a position inside the span (waiting rows included)
 * replaces it and what follows; a gap, or a position before the first, starts over there.  The
 * rows wait; past pending_rows waiting rows the oldest are settled, a whole number of 64-row
 * chunks (CONTEXT_CHUNK) at a time. */
int og_ctx_queue(og_model* m, int seq, int64_t pos, const float* taps, int n) {
  const og_geometry* g = &m->g;
  if (seq < 0 || seq >= g->max_seqs || pos < 0 || n < 0 || (n > 0 && !taps)) return -1;
  og_seq* s = &m->seqs[seq];
  const int64_t next = s->first + s->len + s->npend;
  const int restart = pos > next || pos < s->first;
  if (pos + n - (restart ? pos : s->first) > g->max_ctx) return -2;
  if (restart) {
    truncate_to(m, s, 0);
    s->first = pos;
  } else {
    truncate_to(m, s, pos);
  }
  const size_t T = (size_t)g->n_taps * g->hidden;
  if (n > 0) {
    s->pend = (float*)realloc(s->pend, sizeof(float) * T * (size_t)(s->npend + n));
    memcpy(s->pend + (size_t)s->npend * T, taps, sizeof(float) * T * (size_t)n);
    s->npend += n;
  }
  if (s->npend > g->pending_rows) {
    int64_t over = (s->npend - g->pending_rows + 63) / 64 * 64;
    if (over > s->npend) over = s->npend;
    settle_rows(m, s, s->pend, (int)over);
    memmove(s->pend, s->pend + (size_t)over * T, sizeof(float) * T * (size_t)(s->npend - over));
    s->npend -= over;
  }
  return 0;
}

/* dflash.rs, Drafter::settle: every waiting row becomes context */
int og_ctx_settle(og_model* m, int seq) {
  if (seq < 0 || seq >= m->g.max_seqs) return -1;
  og_seq* s = &m->seqs[seq];
  if (s->npend > 0) settle_rows(m, s, s->pend, (int)s->npend);
  s->npend = 0;
  return 0;
}

/* dflash.rs, Drafter::push_context: queue_context, then settle */
int og_ctx_append(og_model* m, int seq, int64_t pos, const float* taps, int n) {
  const int rc = og_ctx_queue(m, seq, pos, taps, n);
  return rc ? rc : og_ctx_settle(m, seq);
}

int64_t og_pending(const og_model* m, int seq) {
  if (seq < 0 || seq >= m->g.max_seqs) return -1;
  return m->seqs[seq].npend;
}

/* dflash.rs, Drafter::truncate: keep positions before pos (the first stays). */
int og_ctx_truncate(og_model* m, int seq, int64_t pos) {
  if (seq < 0 || seq >= m->g.max_seqs || pos < 0) return -1;
  truncate_to(m, &m->seqs[seq], pos);
  return 0;
}

/* dflash.rs, Drafter::reset */
int og_ctx_reset(og_model* m, int seq) {
  if (seq < 0 || seq >= m->g.max_seqs) return -1;
  truncate_to(m, &m->seqs[seq], 0);
  m->seqs[seq].first = 0;
  return 0;
}

int og_ctx_span(const og_model* m, int seq, int64_t* first, int64_t* end) {
  if (seq < 0 || seq >= m->g.max_seqs) return -1;
  *first = m->seqs[seq].first;
  *end = m->seqs[seq].first + m->seqs[seq].len + m->seqs[seq].npend; /* Drafter::next_position */
  return 0;
}

int og_read_kv(const og_model* m, int layer, int seq, int row0, int n, float* k, float* v) {
  const og_geometry* g = &m->g;
  if (layer < 0 || layer >= g->layers || seq < 0 || seq >= g->max_seqs || row0 < 0 || n < 0 || row0 + n > g->max_ctx)
    return -1;
  size_t per = (size_t)g->kv_heads * g->head_dim;
  size_t off = ((size_t)layer * g->max_ctx + (size_t)row0) * per;
  memcpy(k, m->seqs[seq].k + off, sizeof(float) * per * (size_t)n);
  memcpy(v, m->seqs[seq].v + off, sizeof(float) * per * (size_t)n);
  return 0;
}

/* dflash.rs, Drafter::block, for one sequence: rows [anchor, MASK...] at positions a, a+1, ...
 * pass every layer; returns the rows after the last norm.  Per layer its window and rotary
 * option, and, when the geometry declares them, the row convolutions around attention and
 * the MLP (Drafter::conv_in before the sub-layer, the second stage on its output). */
static void block_one(og_model* m, int seq, int64_t anchor, int B, const float* h_in, float* out) {
  const og_geometry* g = &m->g;
  const int H = g->hidden, nh = g->heads, kvh = g->kv_heads, hd = g->head_dim;
  const int qd = nh * hd, kvd = kvh * hd, I = g->intermediate, rep = nh / kvh;
  const float eps = (float)g->eps;
  const float scale = powf((float)hd, -0.5f); /* Drafter::block: (hd as f32).powf(-0.5) */
  og_seq* s = &m->seqs[seq];

  float* h = (float*)malloc(sizeof(float) * (size_t)B * H);
  memcpy(h, h_in, sizeof(float) * (size_t)B * H);
  float* x = (float*)malloc(sizeof(float) * (size_t)B * H);
  float* q = (float*)malloc(sizeof(float) * (size_t)B * qd);
  float* k = (float*)malloc(sizeof(float) * (size_t)B * kvd);
  float* v = (float*)malloc(sizeof(float) * (size_t)B * kvd);
  float* y = (float*)malloc(sizeof(float) * (size_t)B * qd);
  float* o = (float*)malloc(sizeof(float) * (size_t)B * H);
  float* gt = (float*)malloc(sizeof(float) * (size_t)B * I);
  float* up = (float*)malloc(sizeof(float) * (size_t)B * I);
  float* a = (float*)malloc(sizeof(float) * (size_t)B * I);
  float* tmp = (float*)malloc(sizeof(float) * (size_t)hd);
  /* row convolutions: the kernels of both stages per row ([B][pr]) and a staging row block */
  const int kn = g->conv_kernel, pr = kn ? 2 * kn * (H / g->conv_group) : 0;
  float* da = (float*)malloc(sizeof(float) * (size_t)B * (pr ? pr : 1));
  float* dm = (float*)malloc(sizeof(float) * (size_t)B * (pr ? pr : 1));
  float* xc = (float*)malloc(sizeof(float) * (size_t)B * H);

  for (int l = 0; l < g->layers; l++) {
    const og_layer* L = &m->layers[l];
    /* the key range of this layer (cortiq-engine dflash.rs, Drafter::block): every kept row is
     * readable from base = first + dropped; the range ends at hi = max(min(anchor, first + len),
     * base) and starts at lo = base, or under a window w at clamp(anchor + 1 - w, base, hi) */
    const int64_t w = m->window[l], base = s->first + s->dropped[l];
    int64_t hi = anchor < s->first + s->len ? anchor : s->first + s->len;
    if (hi < base) hi = base;
    int64_t lo = base;
    if (w > 0) {
      lo = anchor + 1 - w;
      if (lo < base) lo = base;
      if (lo > hi) lo = hi;
    }
    const int nctx = (int)(hi - lo);
    const int nk = nctx + B;
    for (int r = 0; r < B; r++) og_rmsnorm_row(h + (size_t)r * H, L->in_norm, H, eps, x + (size_t)r * H);
    /* Drafter::conv_in: the second stage's kernels from the normed rows, the first stage on them */
    if (kn) {
      mm(g->conv_fmt, L->attn_kp, pr, H, x, B, da);
      og_row_conv(x, B, H, g->conv_group, kn, 0, L->attn_base, da, xc);
      memcpy(x, xc, sizeof(float) * (size_t)B * H);
    }
    mm(g->body_fmt, L->q, qd, H, x, B, q);
    mm(g->body_fmt, L->k, kvd, H, x, B, k);
    mm(g->body_fmt, L->v, kvd, H, x, B, v);
    for (int r = 0; r < B; r++) {
      for (int j = 0; j < nh; j++) {
        float* qh = q + (size_t)r * qd + (size_t)j * hd;
        og_rmsnorm_row(qh, L->q_norm, hd, eps, tmp);
        if (m->rotary[l]) og_rope_head(tmp, hd, anchor + r, m->inv_freq);
        memcpy(qh, tmp, sizeof(float) * hd);
      }
      for (int j = 0; j < kvh; j++) {
        float* kh = k + (size_t)r * kvd + (size_t)j * hd;
        og_rmsnorm_row(kh, L->k_norm, hd, eps, tmp);
        if (m->rotary[l]) og_rope_head(tmp, hd, anchor + r, m->inv_freq);
        memcpy(kh, tmp, sizeof(float) * hd);
      }
    }
    /* per kv head gi: its keys and values are the context rows then the block's rows (not
     * causal); q head j reads kv head j / rep.  The keys and values are gathered per kv head
     * first; then every (q head, row) is one independent og_attend call (threads share them out,
     * each call's arithmetic is unchanged) */
    float** kks = (float**)malloc(sizeof(float*) * (size_t)kvh);
    float** vvs = (float**)malloc(sizeof(float*) * (size_t)kvh);
#pragma omp parallel for schedule(static) num_threads(g_threads)
    for (int gi = 0; gi < kvh; gi++) {
      float* kk = (float*)malloc(sizeof(float) * (size_t)nk * hd);
      float* vv = (float*)malloc(sizeof(float) * (size_t)nk * hd);
      for (int c = 0; c < nctx; c++) {
        size_t off = (((size_t)l * g->max_ctx + (size_t)(lo - s->first + c)) * kvh + gi) * hd;
        memcpy(kk + (size_t)c * hd, s->k + off, sizeof(float) * hd);
        memcpy(vv + (size_t)c * hd, s->v + off, sizeof(float) * hd);
      }
      for (int r = 0; r < B; r++) {
        memcpy(kk + (size_t)(nctx + r) * hd, k + (size_t)r * kvd + (size_t)gi * hd, sizeof(float) * hd);
        memcpy(vv + (size_t)(nctx + r) * hd, v + (size_t)r * kvd + (size_t)gi * hd, sizeof(float) * hd);
      }
      kks[gi] = kk;
      vvs[gi] = vv;
    }
#pragma omp parallel for schedule(dynamic) num_threads(g_threads)
    for (int jr = 0; jr < nh * B; jr++) {
      const int j = jr / B, r = jr % B, gi = j / rep;
      /* under a window, row r sees context positions from anchor + r + 1 - w on (the
       * earlier ones are masked out); the block's own rows are all seen */
      int64_t c0 = 0;
      if (w > 0) {
        int64_t from = anchor + r + 1 - w;
        if (from < 0) from = 0;
        c0 = from - lo;
        if (c0 < 0) c0 = 0;
        if (c0 > nctx) c0 = nctx;
      }
      og_attend(q + (size_t)r * qd + (size_t)j * hd, 1, kks[gi] + (size_t)c0 * hd, vvs[gi] + (size_t)c0 * hd, nk - (int)c0, hd, scale,
                y + (size_t)r * qd + (size_t)j * hd, NULL);
    }
    for (int gi = 0; gi < kvh; gi++) {
      free(kks[gi]);
      free(vvs[gi]);
    }
    free(vvs);
    free(kks);
    mm(g->body_fmt, L->o, H, qd, y, B, o);
    if (kn) { /* the second stage on the sub-layer's output, before the residual */
      og_row_conv(o, B, H, g->conv_group, kn, 1, L->attn_base, da, xc);
      memcpy(o, xc, sizeof(float) * (size_t)B * H);
    }
    for (size_t i = 0; i < (size_t)B * H; i++) h[i] = h[i] + o[i];
    for (int r = 0; r < B; r++) og_rmsnorm_row(h + (size_t)r * H, L->post_norm, H, eps, x + (size_t)r * H);
    if (kn) {
      mm(g->conv_fmt, L->mlp_kp, pr, H, x, B, dm);
      og_row_conv(x, B, H, g->conv_group, kn, 0, L->mlp_base, dm, xc);
      memcpy(x, xc, sizeof(float) * (size_t)B * H);
    }
    mm(g->body_fmt, L->gate, I, H, x, B, gt);
    mm(g->body_fmt, L->up, I, H, x, B, up);
    og_silu_mul(gt, up, B * I, a);
    mm(g->body_fmt, L->down, H, I, a, B, o);
    if (kn) {
      og_row_conv(o, B, H, g->conv_group, kn, 1, L->mlp_base, dm, xc);
      memcpy(o, xc, sizeof(float) * (size_t)B * H);
    }
    for (size_t i = 0; i < (size_t)B * H; i++) h[i] = h[i] + o[i];
  }
  for (int r = 0; r < B; r++) og_rmsnorm_row(h + (size_t)r * H, m->w.norm, H, eps, out + (size_t)r * H);
  free(xc);
  free(dm);
  free(da);
  free(tmp);
  free(a);
  free(up);
  free(gt);
  free(o);
  free(y);
  free(v);
  free(k);
  free(q);
  free(x);
  free(h);
}

static int check_block_args(const og_model* m, int n_seqs, const int32_t* seqs, const int64_t* anchors) {
  if (n_seqs < 0 || n_seqs > m->g.max_seqs || (n_seqs > 0 && (!seqs || !anchors))) return -1;
  for (int i = 0; i < n_seqs; i++) {
    if (seqs[i] < 0 || seqs[i] >= m->g.max_seqs || anchors[i] < 0) return -1;
    for (int j = 0; j < i; j++)
      if (seqs[j] == seqs[i]) return -1;
  }
  return 0;
}

int og_block_hidden(og_model* m, int n_seqs, const int32_t* seqs, const int64_t* anchors, const float* h,
                    float* hidden) {
  if (check_block_args(m, n_seqs, seqs, anchors)) return -1;
  for (int i = 0; i < n_seqs; i++) og_ctx_settle(m, seqs[i]); /* a block reads settled rows */
  size_t per = (size_t)m->g.block * m->g.hidden;
  for (int i = 0; i < n_seqs; i++) block_one(m, seqs[i], anchors[i], m->g.block, h + per * i, hidden + per * i);
  return 0;
}

/* dflash.rs, module header: logits = head . norm(h); every block row gets its logits.  The
 * device block (gpu_wgpu/dflash_dev.rs, Dev::block) may cut the block to its first block_rows
 * rows (the anchor and the next rows, up to eight there), which then are the whole block of the
 * forward, the attention among block rows included; Drafter::block_dev may take the head's
 * first rows only, a shortlist of the vocabulary: the same product over those rows.  h and
 * logits hold block_rows rows per sequence. */
int og_block_forward_rows(og_model* m, int n_seqs, const int32_t* seqs, const int64_t* anchors, const float* h,
                          int block_rows, int head_rows, float* logits) {
  if (check_block_args(m, n_seqs, seqs, anchors) || head_rows < 1 || head_rows > m->g.vocab || block_rows < 1 ||
      block_rows > m->g.block)
    return -1;
  for (int i = 0; i < n_seqs; i++) og_ctx_settle(m, seqs[i]); /* a block reads settled rows */
  const og_geometry* g = &m->g;
  size_t per = (size_t)block_rows * g->hidden;
  float* x = (float*)malloc(sizeof(float) * per * (size_t)(n_seqs > 0 ? n_seqs : 1));
  for (int i = 0; i < n_seqs; i++) block_one(m, seqs[i], anchors[i], block_rows, h + per * i, x + per * i);
  if (n_seqs > 0) mm(g->head_fmt, m->w.head, head_rows, g->hidden, x, n_seqs * block_rows, logits);
  free(x);
  return 0;
}

int og_block_forward(og_model* m, int n_seqs, const int32_t* seqs, const int64_t* anchors, const float* h,
                     float* logits) {
  return og_block_forward_rows(m, n_seqs, seqs, anchors, h, m->g.block, m->g.vocab, logits);
}

/* ---- candidate selection ---- */

/* dflash.rs, top_k: an ordered list of the best so far; a value enters after every kept value
 * that is >= it, so equal values keep their index order. */
void og_top_k(const float* x, int n, int k, float* vals, int32_t* idx) {
  int len = 0;
  for (int i = 0; i < n; i++) {
    float v = x[i];
    if (len == k && v <= vals[k - 1]) continue;
    int at = 0;
    while (at < len && vals[at] >= v) at++;
    int end = len < k ? len : k - 1; /* the last entry falls off a full list */
    for (int j = end; j > at; j--) {
      vals[j] = vals[j - 1];
      idx[j] = idx[j - 1];
    }
    vals[at] = v;
    idx[at] = i;
    if (len < k) len++;
  }
}

static float f16f(uint16_t h) { return (float)og_f16_to_f64(h); }

/* dflash.rs, Drafter::select_with (book rows through book_row: f16 to f32). */
void og_select(const float* logits, int rows, int width, int ld, const float* hp, int rank,
               const uint16_t* pred, const uint16_t* succ, int top, int32_t anchor, int32_t* chosen,
               int32_t* plain) {
  float* cv = (float*)malloc(sizeof(float) * (size_t)top);
  int32_t* ci = (int32_t*)malloc(sizeof(int32_t) * (size_t)top);
  float* pc = (float*)malloc(sizeof(float) * (size_t)rank);
  int32_t prev = anchor;
  for (int j = 0; j < rows; j++) {
    og_top_k(logits + (size_t)j * ld, width, top, cv, ci);
    plain[j] = ci[0];
    for (int r = 0; r < rank; r++) pc[r] = f16f(pred[(size_t)prev * rank + r]) * hp[(size_t)j * rank + r];
    float best = -INFINITY;
    int32_t tok = ci[0];
    for (int c = 0; c < top; c++) {
      float sum = 0.0f;
      for (int r = 0; r < rank; r++) sum = sum + pc[r] * f16f(succ[(size_t)ci[c] * rank + r]);
      float sc = cv[c] + sum;
      if (sc > best) {
        best = sc;
        tok = ci[c];
      }
    }
    prev = tok;
    chosen[j] = tok;
  }
  free(cv);
  free(ci);
  free(pc);
}
