// The C ABI (include/dflash.h): argument checks, workspace carving, weight repacking, context
// bookkeeping and the enqueue order of the append and block paths on the caller's stream.
//
// Bookkeeping follows cortiq-engine "dflash.rs" (Drafter::queue_context: a position inside the
// held span replaces it and what follows, a gap or a position before the first starts over;
// Drafter::truncate; Drafter::reset; Drafter::block: layer context = [first, clamp(min(anchor,
// first+len), >= first))).  The stage order of a block follows gpu_wgpu/dflash_dev.rs,
// Dev::block (norm, q k v, q/k norm + rotation, attention, o + residual, norm, gate/up + silu,
// down + residual; final norm; head), without the row convolutions and the selector.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <string>
#include <vector>

#include "../../include/dflash.h"
#include "common.h"
#include "digits.h"

using namespace dfl;

namespace {

constexpr int APPEND_CHUNK = 128;  // context rows per append pass (8 row tiles of 16)
constexpr int MROWS = 128;         // activation rows the workspace holds
constexpr int MAXCH = ATTN_MAXCH;  // attention chunks per (sequence, kv head)

thread_local std::string g_create_err;  // last error of a call without a ctx

int unit_fail(int code, const char* what, hipError_t e = hipSuccess) {
  g_create_err = std::string(what) + (e != hipSuccess ? std::string(": ") + hipGetErrorString(e) : std::string());
  return code;
}

}  // namespace

int dfl::unit_error(int code, const char* what, hipError_t e) { return unit_fail(code, what, e); }

namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
int round16(int x) { return (x + 15) & ~15; }

struct Layout {
  size_t fc, head, kvall;
  std::vector<size_t> qkv, o, gu, down;
  size_t hidden_norm, norm, in_norm, post_norm, q_norm, k_norm, inv_freq;
  size_t kc, vc;
  // integer scores (head_dim 128, four q heads per kv head): the keys' int8 digits and row
  // exponents beside the cache, the block queries' beside q (digits.h)
  size_t kd = 0, ke = 0, qd = 0, qe = 0;
  size_t h, xq, dxT, xq2, dxT2, xf, q, kb, vb, part, ssq, apart, aml;
  size_t act_begin, total;
  size_t part_floats;
  // row convolutions: packed kernel projections per layer, static kernels, and activations
  std::vector<size_t> kpa, kpm;
  size_t base_a = 0, base_m = 0, da = 0, dm = 0, xn = 0, ob = 0;
  size_t pend = 0;  // waiting context rows: [max_seqs][pending_rows][n_taps*hidden] f32
};

bool is_fmt(int f) { return f == DFLASH_F32 || f == DFLASH_Q4_32 || f == DFLASH_Q8_32; }

// Geometry checks (cortiq-engine dflash.rs, Geometry::of, plus this library's kernel limits).
int check_geometry(const dflash_geometry* g, std::string* err) {
  char buf[256];
  auto fail = [&](int code, const char* msg) {
    snprintf(buf, sizeof buf, "geometry: %s", msg);
    *err = buf;
    return code;
  };
  if (!g) return fail(DFLASH_EINVAL, "null");
  if (g->layers < 1 || g->hidden < 1 || g->heads < 1 || g->kv_heads < 1 || g->head_dim < 2 || g->intermediate < 1 ||
      g->vocab < 1 || g->n_taps < 1 || g->max_seqs < 1 || g->max_ctx < 0)
    return fail(DFLASH_EINVAL, "a size is not positive");
  if (g->block < 2) return fail(DFLASH_EINVAL, "block must hold the anchor and at least one draft row");
  if (g->heads % g->kv_heads) return fail(DFLASH_EINVAL, "heads must be a multiple of kv_heads");
  if (!(g->eps >= 0) || !(g->rope_theta > 0)) return fail(DFLASH_EINVAL, "eps / rope_theta out of range");
  if (!is_fmt(g->body_fmt) || !is_fmt(g->fc_fmt) || !is_fmt(g->head_fmt)) return fail(DFLASH_EINVAL, "unknown format");
  if (g->block > 16) return fail(DFLASH_ENOTSUP, "block > 16 rows");
  if (g->heads / g->kv_heads > 16) return fail(DFLASH_ENOTSUP, "more than 16 q heads per kv head");
  if (g->head_dim != 64 && g->head_dim != 128) return fail(DFLASH_ENOTSUP, "head_dim must be 64 or 128");
  if ((long)g->max_seqs * g->block > MROWS) return fail(DFLASH_ENOTSUP, "max_seqs * block > 128 rows");
  const long H = g->hidden, qd = (long)g->heads * g->head_dim, kvd = (long)g->kv_heads * g->head_dim;
  const long I = g->intermediate, T = (long)g->n_taps * g->hidden, V = g->vocab;
  auto mat_ok = [&](int fmt, long rows, long cols) {
    if (rows % 16) return false;
    return fmt == DFLASH_F32 ? cols % 4 == 0 : cols % 128 == 0;
  };
  if (!mat_ok(g->fc_fmt, H, T)) return fail(DFLASH_ENOTSUP, "fc shape outside the kernels' tiles");
  if (!mat_ok(g->head_fmt, V, H)) return fail(DFLASH_ENOTSUP, "head shape outside the kernels' tiles");
  if (!mat_ok(g->body_fmt, qd + 2 * kvd, H) || !mat_ok(g->body_fmt, H, qd) || !mat_ok(g->body_fmt, 2 * I, H) ||
      !mat_ok(g->body_fmt, H, I) || !mat_ok(g->body_fmt, 2 * kvd, H))
    return fail(DFLASH_ENOTSUP, "body shapes outside the kernels' tiles");
  if (H % 32 || I % 32 || qd % 32 || T % 32) return fail(DFLASH_ENOTSUP, "activation widths must be multiples of 32");
  if (H * 4 > 96 * 1024) return fail(DFLASH_ENOTSUP, "hidden too wide for one workgroup's row");
  if (g->kv_f16 != 0 && g->kv_f16 != 1) return fail(DFLASH_EINVAL, "kv_f16 must be 0 or 1");
  // attention addresses one (sequence, kv head)'s cache rows through a buffer resource with
  // 32-bit byte offsets
  if ((size_t)g->max_ctx * g->head_dim * (g->kv_f16 ? 2 : 4) >= ((size_t)1 << 31))
    return fail(DFLASH_ENOTSUP, "max_ctx * head_dim * element bytes must stay below 2^31");
  if (attn_digit_scores(g->heads, g->kv_heads, g->head_dim) && (size_t)g->max_ctx * DIG_ROW >= ((size_t)1 << 31))
    return fail(DFLASH_ENOTSUP, "max_ctx * 896 digit bytes must stay below 2^31");  // the keys' digit rows
  if (g->pending_rows < 0) return fail(DFLASH_EINVAL, "negative pending_rows");
  if (g->conv_kernel < 0) return fail(DFLASH_EINVAL, "negative conv_kernel");
  if (g->conv_kernel > 0) {
    if (g->conv_group < 1 || H % g->conv_group) return fail(DFLASH_EINVAL, "conv_group must divide hidden");
    if (!is_fmt(g->conv_fmt)) return fail(DFLASH_EINVAL, "unknown conv format");
    if ((g->conv_fmt == DFLASH_F32) != (g->body_fmt == DFLASH_F32))
      return fail(DFLASH_ENOTSUP, "conv_fmt must be f32 with an f32 body and quantized with a quantized one");
    if (!mat_ok(g->conv_fmt, 2L * g->conv_kernel * (H / g->conv_group), H))
      return fail(DFLASH_ENOTSUP, "kernel projection shape outside the kernels' tiles");
  }
  return DFLASH_OK;
}

// Rows of a kernel projection: both stages' kernels of every offset and column group.
long conv_rows(const dflash_geometry* g) {
  return g->conv_kernel > 0 ? 2L * g->conv_kernel * (g->hidden / g->conv_group) : 0;
}

void plan(const dflash_geometry* g, Layout* L) {
  const long H = g->hidden, qd = (long)g->heads * g->head_dim, kvd = (long)g->kv_heads * g->head_dim;
  const long I = g->intermediate, T = (long)g->n_taps * g->hidden, V = g->vocab, hd = g->head_dim;
  const long NL = g->layers, kvh = g->kv_heads, rep = g->heads / g->kv_heads;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  L->fc = take(packed_bytes(g->fc_fmt, H, T));
  L->head = take(packed_bytes(g->head_fmt, V, H));
  L->kvall = take(packed_bytes(g->body_fmt, NL * 2 * kvd, H));
  L->qkv.resize(NL);
  L->o.resize(NL);
  L->gu.resize(NL);
  L->down.resize(NL);
  for (long l = 0; l < NL; l++) {
    L->qkv[l] = take(packed_bytes(g->body_fmt, qd + 2 * kvd, H));
    L->o[l] = take(packed_bytes(g->body_fmt, H, qd));
    L->gu[l] = take(packed_bytes(g->body_fmt, 2 * I, H));
    L->down[l] = take(packed_bytes(g->body_fmt, H, I));
  }
  const long PR = conv_rows(g);
  if (PR) {
    L->kpa.resize(NL);
    L->kpm.resize(NL);
    for (long l = 0; l < NL; l++) {
      L->kpa[l] = take(packed_bytes(g->conv_fmt, PR, H));
      L->kpm[l] = take(packed_bytes(g->conv_fmt, PR, H));
    }
    L->base_a = take(NL * 2 * g->conv_kernel * H * 4);
    L->base_m = take(NL * 2 * g->conv_kernel * H * 4);
  }
  L->hidden_norm = take(H * 4);
  L->norm = take(H * 4);
  L->in_norm = take(NL * H * 4);
  L->post_norm = take(NL * H * 4);
  L->q_norm = take(NL * hd * 4);
  L->k_norm = take(NL * hd * 4);
  L->inv_freq = take(hd / 2 * 4);
  const size_t cache = (size_t)NL * g->max_seqs * kvh * (size_t)g->max_ctx * hd * (g->kv_f16 ? 2 : 4);
  L->kc = take(cache);
  L->vc = take(cache);
  const bool digits = attn_digit_scores((int)g->heads, (int)kvh, (int)hd);
  if (digits) {
    const size_t rows = (size_t)NL * g->max_seqs * kvh * (size_t)g->max_ctx;
    L->kd = take(rows * DIG_ROW);
    L->ke = take(rows * 4);
  }
  if (g->pending_rows > 0) L->pend = take((size_t)g->max_seqs * g->pending_rows * T * 4);
  L->act_begin = off;
  long Kmax = H;
  if (qd > Kmax) Kmax = qd;
  if (I > Kmax) Kmax = I;
  if (T > Kmax) Kmax = T;
  L->h = take((size_t)MROWS * H * 4);
  L->xq = take((size_t)MROWS * Kmax);
  L->dxT = take((size_t)(Kmax / 32) * MROWS * 4);
  L->xf = take((size_t)MROWS * Kmax * 4);
  L->q = take((size_t)MROWS * qd * 4);
  if (digits) {
    L->qd = take((size_t)MROWS * g->heads * DIG_ROW);
    L->qe = take((size_t)MROWS * g->heads * 4);
  }
  L->kb = take((size_t)MROWS * kvd * 4);
  L->vb = take((size_t)MROWS * kvd * 4);
  // the second activation buffer: SwiGLU's output, read by down while gate|up's input stays put
  L->xq2 = take((size_t)MROWS * I);
  L->dxT2 = take((size_t)(I / 32) * MROWS * 4);
  // f64 products of the projections that leave the GEMM unreduced (q|k|v, fc, the append's K|V)
  long pn = H;
  if (qd + 2 * kvd > pn) pn = qd + 2 * kvd;
  if (NL * 2 * kvd > pn) pn = NL * 2 * kvd;
  if (2 * I > pn) pn = 2 * I;  // the f32 drafter's gate|up
  if (qd > pn) pn = qd;
  L->part_floats = (size_t)MROWS * pn;
  L->part = take(L->part_floats * 8);
  L->ssq = take((size_t)MROWS * (H / 16 + 1) * 8);  // per-row sums of squares in pieces
  const size_t arows = (size_t)g->max_seqs * kvh * MAXCH * rep * 16;
  L->apart = take(arows * hd * 8);
  L->aml = take(arows * 2 * 8);
  if (PR) {  // the kernels of a call's rows (kept from stage 0 to stage 1), x, the sub-layer's output
    L->da = take((size_t)MROWS * PR * 4);
    L->dm = take((size_t)MROWS * PR * 4);
    L->xn = take((size_t)MROWS * H * 4);
    L->ob = take((size_t)MROWS * H * 4);
  }
  L->total = off;
}

}  // namespace

struct dflash_ctx {
  dflash_geometry g;
  hipStream_t st = nullptr;
  std::string err;
  Layout lay;
  uint8_t* ws = nullptr;
  std::vector<int64_t> first, len;
  std::vector<int64_t> npend, pstart;  // waiting rows of each sequence and the ring's oldest slot
  // per-layer options (0 = every position; 1 = rotary) and, per (sequence, layer), the oldest
  // context rows the layer dropped
  std::vector<int32_t> window, rotary;
  std::vector<int64_t> dropped;  // [max_seqs][layers]
  unsigned long long rot_mask = ~0ull;  // bit l: layer l rotates (layers >= 64 always do)
  int score_mode = DFLASH_SCORES_AUTO;
  int last_scores = DFLASH_SCORES_AUTO;  // what the last block call scored with
  int64_t& drop(int seq, int l) { return dropped[(size_t)seq * g.layers + l]; }
  // Drafter::truncate: a layer's dropped rows are clipped to what a sequence keeps
  void keep_rows(int seq, int64_t keep) {
    for (int l = 0; l < g.layers; l++)
      if (drop(seq, l) > keep) drop(seq, l) = keep;
    len[seq] = keep;
  }
  // stage timing: event pairs recorded around the launches of the timed stages
  unsigned timed_mask = 0;
  std::vector<hipEvent_t> ev_pool;  // created on first use, reused
  size_t ev_used = 0;
  std::vector<int> ev_stage;  // stage of each recorded pair

  hipError_t mark() {  // record the next event of a pair
    if (ev_used == ev_pool.size()) {
      hipEvent_t e;
      hipError_t r = hipEventCreate(&e);
      if (r != hipSuccess) return r;
      ev_pool.push_back(e);
    }
    return hipEventRecord(ev_pool[ev_used++], st);
  }
  hipEvent_t switch_ev = nullptr;  // orders a stream switch after the old stream's work
  ~dflash_ctx() {
    for (hipEvent_t e : ev_pool) (void)hipEventDestroy(e);
    if (switch_ev) (void)hipEventDestroy(switch_ev);
  }

  template <class T>
  T* at(size_t off) const {
    return (T*)(ws + off);
  }
  int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    err = buf;
    return code;
  }
  int hip(hipError_t e, const char* what) {
    if (e == hipSuccess) return DFLASH_OK;
    return fail(DFLASH_EHIP, "%s: %s", what, hipGetErrorString(e));
  }
};

#define TRY_HIP(c, expr, what)                     \
  do {                                             \
    int _rc = (c)->hip((expr), (what));            \
    if (_rc != DFLASH_OK) return _rc;              \
  } while (0)

// Brackets a stage with an event pair when that stage is being timed.
struct StageTimer {
  dflash_ctx* c;
  bool on;
  StageTimer(dflash_ctx* c_, int stage)
      : c(c_), on(((c_->timed_mask >> stage) & 1u) && c_->ev_used + 2 <= 65536) {
    if (on && c->mark() != hipSuccess) on = false;
    if (on) c->ev_stage.push_back(stage);
  }
  ~StageTimer() {
    if (on) (void)c->mark();
  }
};

namespace {

bool bodyq(const dflash_ctx* c) { return c->g.body_fmt != DFLASH_F32; }

GemmOut gemm_out(int epi, int M, int Mpad) {
  GemmOut o;
  memset(&o, 0, sizeof o);
  o.epi = epi;
  o.M = M;
  o.Mpad = Mpad;
  return o;
}

// One quantized matrix product over activations (ax, ad) with the given epilogue.
int run_gemm_q(dflash_ctx* c, int fmt, size_t woff, int N, int K, const int8_t* ax, const float* ad, const GemmOut& o,
               const char* what) {
  return c->hip(launch_gemm_q(fmt, c->ws + woff, N, K, ax, ad, -1, o, c->st), what);
}

// One f32 matrix product over the f32 activations xf: f64 products [Mpad][N] or f32 out.
int run_gemm_f32(dflash_ctx* c, size_t woff, int N, int K, int Mpad, int M, void* out, bool direct, int out_ld,
                 int m_store) {
  return c->hip(launch_gemm_f32((const float*)(c->ws + woff), N, K, c->at<float>(c->lay.xf), Mpad, M, out, direct,
                                out_ld, m_store, c->st),
                "f32 gemm");
}

int check_weights(const dflash_geometry* g, const dflash_weights* w, std::string* err) {
  auto bad = [&](const char* m) {
    *err = std::string("weights: ") + m;
    return DFLASH_EINVAL;
  };
  auto mat = [&](const dflash_matrix& m, int fmt) { return m.codes && (fmt == DFLASH_F32 || m.scales); };
  if (!w || !w->layer) return bad("null");
  if (!mat(w->fc, g->fc_fmt) || !mat(w->head, g->head_fmt) || !w->hidden_norm || !w->norm) return bad("fc/head/norms");
  for (int l = 0; l < g->layers; l++) {
    const dflash_layer_weights& L = w->layer[l];
    const int f = g->body_fmt;
    if (!L.in_norm || !L.post_norm || !L.q_norm || !L.k_norm || !mat(L.q, f) || !mat(L.k, f) || !mat(L.v, f) ||
        !mat(L.o, f) || !mat(L.gate, f) || !mat(L.up, f) || !mat(L.down, f))
      return bad("a layer matrix or norm is null");
    if (g->conv_kernel > 0 &&
        (!mat(L.attn_kp, g->conv_fmt) || !mat(L.mlp_kp, g->conv_fmt) || !L.attn_base || !L.mlp_base))
      return bad("a layer's convolution weights are null");
  }
  return DFLASH_OK;
}

// The context keys layer l of each sequence attends to (dflash.rs, Drafter::block): base =
// first + dropped, hi = max(min(anchor, first+len), base), lo = base or, under a window w,
// clamp(anchor + 1 - w, base, hi); row r masks the keys before position anchor + r + 1 - w.
// Cache rows are position - first; key index i of the call is cache row ctx0 + i.
void layer_ranges(const dflash_ctx* c, int l, const int32_t* seqs, const int64_t* anchors, SeqInfo& si) {
  const int64_t w = c->window[l];
  for (int i = 0; i < si.n; i++) {
    const int sq = seqs[i];
    const int64_t first = c->first[sq], end = first + c->len[sq];
    const int64_t base = first + c->dropped[(size_t)sq * c->g.layers + l];
    int64_t hi = anchors[i] < end ? anchors[i] : end;
    if (hi < base) hi = base;
    int64_t lo = base;
    if (w > 0) {
      lo = anchors[i] + 1 - w;
      if (lo < base) lo = base;
      if (lo > hi) lo = hi;
    }
    si.ctx0[i] = (int)(lo - first);
    si.nctx[i] = (int)(hi - lo);
    int64_t m0 = w > 0 ? anchors[i] + 1 - w - lo : -(1ll << 30);
    if (m0 < -(1ll << 30)) m0 = -(1ll << 30);
    if (m0 > (1ll << 30)) m0 = 1ll << 30;
    si.mask0[i] = (int)m0;
  }
}

int settle_seq(dflash_ctx* c, int seq);

int block_common(dflash_ctx* c, int32_t n_seqs, const int32_t* seqs, const int64_t* anchors, const float* h,
                 float* out, bool hidden_only, int head_rows, int block_rows) {
  const dflash_geometry& g = c->g;
  if (n_seqs < 1 || n_seqs > g.max_seqs) return c->fail(DFLASH_EINVAL, "n_seqs %d outside [1, %d]", n_seqs, g.max_seqs);
  if (!seqs || !anchors || !h || !out) return c->fail(DFLASH_EINVAL, "null pointer");
  SeqInfo si;
  memset(&si, 0, sizeof si);
  si.n = n_seqs;
  for (int i = 0; i < n_seqs; i++) {
    if (seqs[i] < 0 || seqs[i] >= g.max_seqs) return c->fail(DFLASH_EINVAL, "sequence %d out of range", seqs[i]);
    for (int j = 0; j < i; j++)
      if (seqs[j] == seqs[i]) return c->fail(DFLASH_EINVAL, "sequence %d given twice", seqs[i]);
    if (anchors[i] < 0) return c->fail(DFLASH_EINVAL, "negative anchor");
    si.slot[i] = seqs[i];
    si.pos0[i] = anchors[i];
  }
  for (int i = 0; i < n_seqs; i++) {  // a block reads settled rows (Drafter::settle first)
    const int rc = settle_seq(c, seqs[i]);
    if (rc) return rc;
  }
  // the block's rows: all of them, or the first block_rows (the anchor and the rows after it)
  const int B = block_rows, H = g.hidden, nh = g.heads, kvh = g.kv_heads, hd = g.head_dim, NL = g.layers;
  const int qd = nh * hd, kvd = kvh * hd, I = g.intermediate;
  const int M = n_seqs * B, Mpad = round16(M);
  const float eps = (float)g.eps;
  const Layout& L = c->lay;
  float* hbuf = c->at<float>(L.h);
  double* part = c->at<double>(L.part);
  int8_t* xq = c->at<int8_t>(L.xq);
  float* dxT = c->at<float>(L.dxT);
  float* xf = c->at<float>(L.xf);
  const bool bq = bodyq(c);

  AttnShape as;
  as.nh = nh;
  as.kvh = kvh;
  as.hd = hd;
  as.B = B;
  as.max_ctx = g.max_ctx;
  as.max_seqs = g.max_seqs;
  as.maxch = MAXCH;
  as.scale = powf((float)hd, -0.5f);  // dflash.rs, Drafter::block: (hd as f32).powf(-0.5)
  as.kv_f16 = g.kv_f16;
  // about one workgroup per CU: n_seqs * q heads * chunks ~ 256 (a workgroup serves one q head
  // of one chunk), chunks a multiple of 32 keys; per layer, as its windows give it keys.  The
  // integer-score kernel serves a kv head's four q heads with four waves: two workgroups a CU,
  // n_seqs * kv heads * chunks ~ 512
  long call_rows = 0;  // context rows of the call, over its sequences (windows aside)
  for (int i = 0; i < n_seqs; i++) {
    const int64_t f = c->first[seqs[i]], hi = std::min<int64_t>(anchors[i], f + c->len[seqs[i]]);
    call_rows += (long)std::max<int64_t>(0, hi - f);
  }
  const bool dig = L.kd != 0 && (c->score_mode == DFLASH_SCORES_DIGITS ||
                                 (c->score_mode == DFLASH_SCORES_AUTO && call_rows >= DIG_AUTO_ROWS));
  c->last_scores = dig ? DFLASH_SCORES_DIGITS : DFLASH_SCORES_F64;
  int nch_target = dig ? (512 + n_seqs * kvh - 1) / (n_seqs * kvh) : (256 + n_seqs * nh - 1) / (n_seqs * nh);
  if (nch_target > MAXCH) nch_target = MAXCH;
  auto chunk_keys = [&]() {
    int nmax = 0;
    for (int i = 0; i < n_seqs; i++)
      if (si.nctx[i] > nmax) nmax = si.nctx[i];
    const int ck = ((nmax + nch_target - 1) / nch_target + 31) / 32 * 32;
    return ck < 32 ? 32 : ck;
  };

  double* ssq = c->at<double>(L.ssq);
  int8_t* xq2 = c->at<int8_t>(L.xq2);
  float* dxT2 = c->at<float>(L.dxT2);
  const int fmt = g.body_fmt;
  const int copy_parts = (H + 255) / 256, tile_parts = H / 16;

  // row convolutions (dflash.rs, Drafter::conv_in / conv): with them the normed rows are also
  // kept in f32 (xn), a sub-layer's input is stage 0 of them with kernels projected from them
  // (da / dm, kept for stage 1), and its output o goes through stage 1 before the residual
  const int kn = g.conv_kernel, gs = g.conv_group, PR = (int)conv_rows(&g);
  float* xn = kn ? c->at<float>(L.xn) : nullptr;
  float* ob = kn ? c->at<float>(L.ob) : nullptr;
  const size_t nbase = (size_t)2 * kn * H;
  // d = KP . x (KP over A8(x), or f32 x), then x <- stage 0 of x, as the next matrix's input
  auto conv_in = [&](size_t kp, float* d, const float* base) -> int {
    int rc;
    if (bq) {
      GemmOut o = gemm_out(EPI_F32, M, Mpad);
      o.y = d;
      o.ld = PR;
      o.m_store = M;
      rc = run_gemm_q(c, g.conv_fmt, kp, PR, H, xq, dxT, o, "kernel projection");
    } else {
      rc = run_gemm_f32(c, kp, PR, H, Mpad, M, d, true, PR, M);
    }
    if (rc) return rc;
    return c->hip(launch_conv_in(xn, d, base, M, Mpad, B, H, gs, kn, bq, xq, dxT, xf, c->st), "conv in");
  };

  // h = the block rows; x = A8(RMSNorm(h, in_norm_0))
  TRY_HIP(c, launch_copy_ssq(h, hbuf, M, H, ssq, c->st), "copy block rows");
  TRY_HIP(c,
          launch_rms_act(hbuf, ssq, copy_parts, c->at<float>(L.in_norm), eps, M, Mpad, H, bq, xq, dxT, xf, c->st, xn),
          "in-norm");
  // bytes of one layer's cache
  const size_t layer_cache = (size_t)g.max_seqs * kvh * (size_t)g.max_ctx * hd * (g.kv_f16 ? 2 : 4);
  const size_t layer_rows = (size_t)g.max_seqs * kvh * (size_t)g.max_ctx;  // key rows of a layer's digits
  for (int l = 0; l < NL; l++) {
    int rc;
    float* da = kn ? c->at<float>(L.da) : nullptr;
    float* dm = kn ? c->at<float>(L.dm) : nullptr;
    const float* base_a = kn ? c->at<float>(L.base_a) + (size_t)l * nbase : nullptr;
    const float* base_m = kn ? c->at<float>(L.base_m) + (size_t)l * nbase : nullptr;
    if (kn && (rc = conv_in(L.kpa[l], da, base_a))) return rc;
    {
      StageTimer t(c, DFLASH_STAGE_QKV);
      if (bq) {
        GemmOut o = gemm_out(EPI_F64, M, Mpad);
        o.y = part;
        rc = run_gemm_q(c, fmt, L.qkv[l], qd + 2 * kvd, H, xq, dxT, o, "q|k|v");
      } else {
        rc = run_gemm_f32(c, L.qkv[l], qd + 2 * kvd, H, Mpad, M, part, false, 0, 0);
      }
      if (rc) return rc;
    }
    TRY_HIP(c,
            launch_qkv_epilogue(part, 1, Mpad, M, B, si, nh, kvh, hd, c->at<float>(L.q_norm) + (size_t)l * hd,
                                c->at<float>(L.k_norm) + (size_t)l * hd, c->at<float>(L.inv_freq), eps,
                                c->rotary[l] != 0, c->at<float>(L.q), c->at<float>(L.kb), c->at<float>(L.vb),
                                dig ? c->at<int8_t>(L.qd) : nullptr, dig ? c->at<int>(L.qe) : nullptr, c->st),
            "q/k norm + rope");
    layer_ranges(c, l, seqs, anchors, si);
    as.ck = chunk_keys();
    DigitRows digs{};
    if (dig)
      digs = DigitRows{c->at<int8_t>(L.qd), c->at<int>(L.qe), c->at<int8_t>(L.kd) + (size_t)l * layer_rows * DIG_ROW,
                       c->at<int>(L.ke) + (size_t)l * layer_rows};
    {
      StageTimer t(c, DFLASH_STAGE_ATTENTION);
      {
        StageTimer tc(c, DFLASH_STAGE_ATTN_CHUNKS);
        TRY_HIP(c,
                launch_attention_chunks(as, si, c->at<float>(L.q), c->ws + L.kc + (size_t)l * layer_cache,
                                        c->ws + L.vc + (size_t)l * layer_cache, dig ? &digs : nullptr,
                                        c->at<double>(L.apart), c->at<double>(L.aml), c->st),
                "attention chunks");
      }
      TRY_HIP(c,
              launch_attention_merge(as, si, c->at<float>(L.q), c->at<float>(L.kb), c->at<float>(L.vb),
                                     c->at<double>(L.apart), c->at<double>(L.aml), Mpad, bq, xq, dxT, xf, c->st),
              "attention merge");
    }
    const bool last = l + 1 == NL;
    const float* nw = last ? c->at<float>(L.norm) : c->at<float>(L.in_norm) + (size_t)(l + 1) * H;
    const bool nq = last ? (!hidden_only && g.head_fmt != DFLASH_F32) : bq;
    if (kn) {
      // o = Wo y; h += stage 1 of o; x = RMSNorm(h, post_norm); x <- stage 0 of x (MLP kernels);
      // a = silu(gate x) * up x; o = down a; h += stage 1 of o; the next norm
      // stage 1 in the product's epilogue where a block's rows stay inside a 16-row group
      const bool fused = bq && 16 % B == 0;
      auto conv_epi = [&](const float* d, const float* base) {
        GemmOut o = gemm_out(EPI_CONV, M, Mpad);
        o.h = hbuf;
        o.ssq = ssq;
        o.cd = d;
        o.cbase = base;
        o.cB = B;
        o.cgs = gs;
        o.ckn = kn;
        return o;
      };
      {
        StageTimer t(c, DFLASH_STAGE_O);
        if (fused) {
          rc = run_gemm_q(c, fmt, L.o[l], H, qd, xq, dxT, conv_epi(da, base_a), "o + conv + residual");
        } else if (bq) {
          GemmOut o = gemm_out(EPI_F32, M, Mpad);
          o.y = ob;
          o.ld = H;
          o.m_store = M;
          rc = run_gemm_q(c, fmt, L.o[l], H, qd, xq, dxT, o, "o");
        } else {
          rc = run_gemm_f32(c, L.o[l], H, qd, Mpad, M, ob, true, H, M);
        }
        if (rc) return rc;
      }
      if (!fused) TRY_HIP(c, launch_conv_out(ob, da, base_a, M, B, H, gs, kn, hbuf, ssq, c->st), "conv out");
      TRY_HIP(c,
              launch_rms_act(hbuf, ssq, tile_parts, c->at<float>(L.post_norm) + (size_t)l * H, eps, M, Mpad, H, bq, xq,
                             dxT, xf, c->st, xn),
              "post-norm");
      if ((rc = conv_in(L.kpm[l], dm, base_m))) return rc;
      {
        StageTimer t(c, DFLASH_STAGE_GATE_UP);
        if (bq) {
          GemmOut o = gemm_out(EPI_SWIGLU, M, Mpad);
          o.xq = xq2;
          o.dxT = dxT2;
          rc = run_gemm_q(c, fmt, L.gu[l], 2 * I, H, xq, dxT, o, "gate|up + swiglu");
        } else {
          rc = run_gemm_f32(c, L.gu[l], 2 * I, H, Mpad, M, part, false, 0, 0);
          if (!rc) rc = c->hip(launch_swiglu_act(part, 1, M, Mpad, I, false, xq, dxT, xf, c->st), "swiglu");
        }
        if (rc) return rc;
      }
      {
        StageTimer t(c, DFLASH_STAGE_DOWN);
        if (fused) {
          rc = run_gemm_q(c, fmt, L.down[l], H, I, xq2, dxT2, conv_epi(dm, base_m), "down + conv + residual");
        } else if (bq) {
          GemmOut o = gemm_out(EPI_F32, M, Mpad);
          o.y = ob;
          o.ld = H;
          o.m_store = M;
          rc = run_gemm_q(c, fmt, L.down[l], H, I, xq2, dxT2, o, "down");
        } else {
          rc = run_gemm_f32(c, L.down[l], H, I, Mpad, M, ob, true, H, M);
        }
        if (rc) return rc;
      }
      if (!fused) TRY_HIP(c, launch_conv_out(ob, dm, base_m, M, B, H, gs, kn, hbuf, ssq, c->st), "conv out");
      TRY_HIP(c, launch_rms_act(hbuf, ssq, tile_parts, nw, eps, M, Mpad, H, nq, xq, dxT, xf, c->st, xn), "next norm");
    } else if (bq) {
      // h += Wo y; x = A8(RMSNorm(h, post_norm)); a = A8(silu(gate x) * up x); h += down a
      {
        StageTimer t(c, DFLASH_STAGE_O);
        GemmOut o = gemm_out(EPI_RESID, M, Mpad);
        o.h = hbuf;
        o.ssq = ssq;
        if ((rc = run_gemm_q(c, fmt, L.o[l], H, qd, xq, dxT, o, "o + residual"))) return rc;
      }
      TRY_HIP(c,
              launch_rms_act(hbuf, ssq, tile_parts, c->at<float>(L.post_norm) + (size_t)l * H, eps, M, Mpad, H, true,
                             xq, dxT, xf, c->st),
              "post-norm");
      {
        StageTimer t(c, DFLASH_STAGE_GATE_UP);
        GemmOut o = gemm_out(EPI_SWIGLU, M, Mpad);
        o.xq = xq2;
        o.dxT = dxT2;
        if ((rc = run_gemm_q(c, fmt, L.gu[l], 2 * I, H, xq, dxT, o, "gate|up + swiglu"))) return rc;
      }
      {
        StageTimer t(c, DFLASH_STAGE_DOWN);
        GemmOut o = gemm_out(EPI_RESID, M, Mpad);
        o.h = hbuf;
        o.ssq = ssq;
        if ((rc = run_gemm_q(c, fmt, L.down[l], H, I, xq2, dxT2, o, "down + residual"))) return rc;
      }
      TRY_HIP(c, launch_rms_act(hbuf, ssq, tile_parts, nw, eps, M, Mpad, H, nq, xq, dxT, xf, c->st), "next norm");
    } else {
      {
        StageTimer t(c, DFLASH_STAGE_O);
        if ((rc = run_gemm_f32(c, L.o[l], H, qd, Mpad, M, part, false, 0, 0))) return rc;
      }
      TRY_HIP(c,
              launch_norm_act(part, nullptr, 1, Mpad, hbuf, hbuf, c->at<float>(L.post_norm) + (size_t)l * H, eps, M,
                              Mpad, H, false, xq, dxT, xf, c->st),
              "o residual + post-norm");
      {
        StageTimer t(c, DFLASH_STAGE_GATE_UP);
        if ((rc = run_gemm_f32(c, L.gu[l], 2 * I, H, Mpad, M, part, false, 0, 0))) return rc;
      }
      TRY_HIP(c, launch_swiglu_act(part, 1, M, Mpad, I, false, xq, dxT, xf, c->st), "swiglu");
      {
        StageTimer t(c, DFLASH_STAGE_DOWN);
        if ((rc = run_gemm_f32(c, L.down[l], H, I, Mpad, M, part, false, 0, 0))) return rc;
      }
      TRY_HIP(c, launch_norm_act(part, nullptr, 1, Mpad, hbuf, hbuf, nw, eps, M, Mpad, H, nq, xq, dxT, xf, c->st),
              "down residual + next norm");
    }
  }
  if (hidden_only) {
    TRY_HIP(c, hipMemcpyAsync(out, xf, (size_t)M * H * 4, hipMemcpyDeviceToDevice, c->st), "copy hidden");
    return DFLASH_OK;
  }
  // the head's first head_rows rows (all V of them unless a shortlist is asked for): rows of
  // the packed head are n-tiles stored front to back, so a shortlist is a prefix
  StageTimer t(c, DFLASH_STAGE_HEAD);
  const int HN = head_rows;
  if (g.head_fmt == DFLASH_F32) return run_gemm_f32(c, L.head, HN, H, Mpad, M, out, true, HN, M);
  GemmOut o = gemm_out(EPI_F32, M, Mpad);
  o.y = out;
  o.ld = HN;
  o.m_store = M;
  return run_gemm_q(c, g.head_fmt, L.head, HN, H, xq, dxT, o, "head");
}

}  // namespace

extern "C" {

int dflash_workspace_bytes(const dflash_geometry* g, size_t* bytes) {
  std::string err;
  int rc = check_geometry(g, &err);
  if (rc) {
    g_create_err = err;
    return rc;
  }
  if (!bytes) return DFLASH_EINVAL;
  Layout L;
  plan(g, &L);
  *bytes = L.total;
  return DFLASH_OK;
}

int dflash_create(const dflash_geometry* g, const dflash_weights* w, void* workspace, size_t bytes, void* stream,
                  dflash_ctx** out) {
  std::string err;
  int rc = check_geometry(g, &err);
  if (!rc) rc = check_weights(g, w, &err);
  if (!rc && (!workspace || !out)) {
    err = "null workspace or out";
    rc = DFLASH_EINVAL;
  }
  if (!rc && ((uintptr_t)workspace & 255)) {
    err = "workspace must be 256-byte aligned";
    rc = DFLASH_EINVAL;
  }
  Layout L;
  if (!rc) {
    plan(g, &L);
    if (bytes < L.total) {
      err = "workspace too small";
      rc = DFLASH_EINVAL;
    }
  }
  if (rc) {
    g_create_err = err;
    return rc;
  }
  dflash_ctx* c = new dflash_ctx();
  c->g = *g;
  c->lay = L;
  c->ws = (uint8_t*)workspace;
  c->st = (hipStream_t)stream;
  c->first.assign(g->max_seqs, 0);
  c->len.assign(g->max_seqs, 0);
  c->npend.assign(g->max_seqs, 0);
  c->pstart.assign(g->max_seqs, 0);
  c->window.assign(g->layers, 0);
  c->rotary.assign(g->layers, 1);
  c->dropped.assign((size_t)g->max_seqs * g->layers, 0);
  const long H = g->hidden, qd = (long)g->heads * g->head_dim, kvd = (long)g->kv_heads * g->head_dim;
  const long I = g->intermediate, T = (long)g->n_taps * g->hidden, V = g->vocab, hd = g->head_dim;
  auto fin = [&](int code) -> int {
    if (code) {
      g_create_err = c->err;
      delete c;
      return code;
    }
    *out = c;
    return DFLASH_OK;
  };
  auto pack = [&](int fmt, const dflash_matrix& m, long rows, long cols, size_t off, long tile_off, long stride) {
    return c->hip(launch_pack(fmt, m.codes, m.scales, (int)rows, (int)cols, c->ws + off, tile_off, stride, c->st),
                  "pack");
  };
  int e;
  // activations start at zero (rows past a call's last row are read as zeros)
  if ((e = c->hip(hipMemsetAsync(c->ws + L.act_begin, 0, L.total - L.act_begin, c->st), "clear activations")))
    return fin(e);
  if ((e = pack(g->fc_fmt, w->fc, H, T, L.fc, 0, 1))) return fin(e);
  if ((e = pack(g->head_fmt, w->head, V, H, L.head, 0, 1))) return fin(e);
  const int bf = g->body_fmt;
  for (int l = 0; l < g->layers; l++) {
    const dflash_layer_weights& W = w->layer[l];
    if ((e = pack(bf, W.q, qd, H, L.qkv[l], 0, 1))) return fin(e);
    if ((e = pack(bf, W.k, kvd, H, L.qkv[l], qd / 16, 1))) return fin(e);
    if ((e = pack(bf, W.v, kvd, H, L.qkv[l], (qd + kvd) / 16, 1))) return fin(e);
    if ((e = pack(bf, W.o, H, qd, L.o[l], 0, 1))) return fin(e);
    if ((e = pack(bf, W.gate, I, H, L.gu[l], 0, 2))) return fin(e);
    if ((e = pack(bf, W.up, I, H, L.gu[l], 1, 2))) return fin(e);
    if ((e = pack(bf, W.down, H, I, L.down[l], 0, 1))) return fin(e);
    if ((e = pack(bf, W.k, kvd, H, L.kvall, (2 * l) * kvd / 16, 1))) return fin(e);
    if ((e = pack(bf, W.v, kvd, H, L.kvall, (2 * l + 1) * kvd / 16, 1))) return fin(e);
    auto cp = [&](size_t off, const float* src, long n) {
      return c->hip(hipMemcpyAsync(c->ws + off, src, n * 4, hipMemcpyDeviceToDevice, c->st), "copy norm");
    };
    if ((e = cp(L.in_norm + (size_t)l * H * 4, W.in_norm, H))) return fin(e);
    if ((e = cp(L.post_norm + (size_t)l * H * 4, W.post_norm, H))) return fin(e);
    if ((e = cp(L.q_norm + (size_t)l * hd * 4, W.q_norm, hd))) return fin(e);
    if ((e = cp(L.k_norm + (size_t)l * hd * 4, W.k_norm, hd))) return fin(e);
    if (g->conv_kernel > 0) {
      const long PR = conv_rows(g), nb = 2L * g->conv_kernel * H;
      if ((e = pack(g->conv_fmt, W.attn_kp, PR, H, L.kpa[l], 0, 1))) return fin(e);
      if ((e = pack(g->conv_fmt, W.mlp_kp, PR, H, L.kpm[l], 0, 1))) return fin(e);
      if ((e = cp(L.base_a + (size_t)l * nb * 4, W.attn_base, nb))) return fin(e);
      if ((e = cp(L.base_m + (size_t)l * nb * 4, W.mlp_base, nb))) return fin(e);
    }
  }
  if ((e = c->hip(hipMemcpyAsync(c->ws + L.hidden_norm, w->hidden_norm, H * 4, hipMemcpyDeviceToDevice, c->st),
                  "copy norm")))
    return fin(e);
  if ((e = c->hip(hipMemcpyAsync(c->ws + L.norm, w->norm, H * 4, hipMemcpyDeviceToDevice, c->st), "copy norm")))
    return fin(e);
  if ((e = c->hip(launch_inv_freq(g->rope_theta, (int)hd, c->at<float>(L.inv_freq), c->st), "rope table")))
    return fin(e);
  if ((e = c->hip(hipStreamSynchronize(c->st), "create sync"))) return fin(e);
  return fin(DFLASH_OK);
}

// Work already enqueued on the old stream uses the same workspace (activations, partials, the
// waiting rows), so the new stream first waits for it: an event recorded on the old stream and
// a device-side wait on the new one (the host does not wait).
int dflash_set_stream(dflash_ctx* c, void* stream) {
  if (!c) return DFLASH_EINVAL;
  hipStream_t ns = (hipStream_t)stream;
  if (ns == c->st) return DFLASH_OK;
  if (!c->switch_ev) TRY_HIP(c, hipEventCreateWithFlags(&c->switch_ev, hipEventDisableTiming), "stream switch event");
  TRY_HIP(c, hipEventRecord(c->switch_ev, c->st), "stream switch record");
  TRY_HIP(c, hipStreamWaitEvent(ns, c->switch_ev, 0), "stream switch wait");
  c->st = ns;
  return DFLASH_OK;
}

}  // extern "C"

namespace {

// Drafter::settle_rows: n rows of taps (device) become the context rows at positions first+len,
// ...; then a layer holding more than twice its window keeps only the last window's worth (the
// rows stay in the cache; they are never read again).
int settle_rows(dflash_ctx* c, int seq, const float* taps, int n) {
  const dflash_geometry& g = c->g;
  const int H = g.hidden, T = g.n_taps * g.hidden, kvd = g.kv_heads * g.head_dim, NL = g.layers;
  const float eps = (float)g.eps;
  const Layout& L = c->lay;
  double* part = c->at<double>(L.part);
  int8_t* xq = c->at<int8_t>(L.xq);
  float* dxT = c->at<float>(L.dxT);
  float* xf = c->at<float>(L.xf);
  const int64_t pos = c->first[seq] + c->len[seq];
  const int row = (int)c->len[seq];
  for (int c0 = 0; c0 < n; c0 += APPEND_CHUNK) {
    const int nn = n - c0 < APPEND_CHUNK ? n - c0 : APPEND_CHUNK;
    const int Mpad = round16(nn);
    const float* rows = taps + (size_t)c0 * T;
    int rc;
    if (g.fc_fmt != DFLASH_F32) {
      TRY_HIP(c,
              launch_norm_act(nullptr, rows, 1, Mpad, nullptr, nullptr, nullptr, eps, nn, Mpad, T, true, xq, dxT, xf,
                              c->st),
              "taps quant");
      GemmOut o = gemm_out(EPI_F64, nn, Mpad);
      o.y = part;
      rc = run_gemm_q(c, g.fc_fmt, L.fc, H, T, xq, dxT, o, "fc");
    } else {
      rc = c->hip(launch_gemm_f32((const float*)(c->ws + L.fc), H, T, rows, Mpad, nn, part, false, 0, 0, c->st),
                  "f32 gemm");
    }
    if (rc) return rc;
    TRY_HIP(c,
            launch_norm_act(part, nullptr, 1, Mpad, nullptr, nullptr, c->at<float>(L.hidden_norm), eps, nn, Mpad, H,
                            bodyq(c), xq, dxT, xf, c->st),
            "hidden norm");
    if (bodyq(c)) {
      GemmOut o = gemm_out(EPI_F64, nn, Mpad);
      o.y = part;
      rc = run_gemm_q(c, g.body_fmt, L.kvall, NL * 2 * kvd, H, xq, dxT, o, "k|v of every layer");
    } else {
      rc = run_gemm_f32(c, L.kvall, NL * 2 * kvd, H, Mpad, nn, part, false, 0, 0);
    }
    if (rc) return rc;
    TRY_HIP(c,
            launch_kv_append(part, 1, Mpad, nn, NL, g.kv_heads, g.head_dim, c->at<float>(L.k_norm),
                             c->at<float>(L.inv_freq), eps, c->rot_mask, pos + c0, row + c0, seq, g.max_seqs,
                             g.max_ctx, g.kv_f16 != 0, c->ws + L.kc, c->ws + L.vc,
                             L.kd ? c->at<int8_t>(L.kd) : nullptr, L.ke ? c->at<int>(L.ke) : nullptr, c->st),
            "k/v into the cache");
  }
  c->len[seq] += n;
  return DFLASH_OK;
}

void drop_rows(dflash_ctx* c, int seq) {
  for (int l = 0; l < c->g.layers; l++) {
    const int64_t w = c->window[l], held = c->len[seq] - c->drop(seq, l);
    if (w > 0 && held > 2 * w) c->drop(seq, l) += held - w;
  }
}

// The waiting rows of a sequence sit in a ring of pending_rows taps rows in the workspace:
// the oldest at index pstart.  ring_row(seq, i) is the i-th waiting row's slot.
float* ring_row(dflash_ctx* c, int seq, int64_t i) {
  const int64_t cap = c->g.pending_rows;
  const size_t T = (size_t)c->g.n_taps * c->g.hidden;
  return c->at<float>(c->lay.pend) + ((size_t)seq * cap + (size_t)((c->pstart[seq] + i) % cap)) * T;
}
// the ring's first k waiting rows settled, in at most two contiguous pieces
int settle_ring(dflash_ctx* c, int seq, int64_t k) {
  const int64_t cap = c->g.pending_rows;
  while (k > 0) {
    const int64_t run = std::min(k, cap - c->pstart[seq]);
    const int rc = settle_rows(c, seq, ring_row(c, seq, 0), (int)run);
    if (rc) return rc;
    c->pstart[seq] = (c->pstart[seq] + run) % cap;
    c->npend[seq] -= run;
    k -= run;
  }
  return DFLASH_OK;
}

// Drafter::truncate: positions >= pos are forgotten, waiting rows among them too
void truncate_seq(dflash_ctx* c, int seq, int64_t pos) {
  const int64_t held = c->first[seq] + c->len[seq];
  const int64_t wait = pos > held ? pos - held : 0;
  if (c->npend[seq] > wait) c->npend[seq] = wait;
  int64_t keep = pos - c->first[seq];
  if (keep < 0) keep = 0;
  if (keep > c->len[seq]) keep = c->len[seq];
  c->keep_rows(seq, keep);
}

int settle_seq(dflash_ctx* c, int seq) {
  if (c->npend[seq] == 0) return DFLASH_OK;
  StageTimer timer(c, DFLASH_STAGE_APPEND);
  const int rc = settle_ring(c, seq, c->npend[seq]);
  if (rc) return rc;
  drop_rows(c, seq);
  c->pstart[seq] = 0;
  return DFLASH_OK;
}

}  // namespace

extern "C" {

// Drafter::queue_context: a position inside the span (waiting rows included) replaces it and
// what follows; a gap, or a position before the first, starts over there.  The rows wait; past
// pending_rows waiting rows the oldest settle, a whole number of 64-row chunks at a time (the
// rows that stay waiting never exceed pending_rows, so new rows settled at once never pass
// through the ring).
int dflash_ctx_queue(dflash_ctx* c, int32_t seq, int64_t pos, const float* taps, int32_t n) {
  if (!c) return DFLASH_EINVAL;
  const dflash_geometry& g = c->g;
  if (seq < 0 || seq >= g.max_seqs) return c->fail(DFLASH_EINVAL, "sequence %d out of range", seq);
  if (pos < 0 || n < 0 || (n > 0 && !taps)) return c->fail(DFLASH_EINVAL, "bad position, count or taps");
  const int64_t next = c->first[seq] + c->len[seq] + c->npend[seq];
  const bool restart = pos > next || pos < c->first[seq];
  const int64_t first = restart ? pos : c->first[seq];
  if (pos + n - first > g.max_ctx)
    return c->fail(DFLASH_ECAPACITY, "sequence %d: positions %lld..%lld exceed max_ctx %d from %lld", seq,
                   (long long)pos, (long long)(pos + n), g.max_ctx, (long long)first);
  if (restart) {
    truncate_seq(c, seq, 0);
    c->first[seq] = pos;
  } else {
    truncate_seq(c, seq, pos);
  }
  const int64_t cap = g.pending_rows, held = c->npend[seq] + n;
  int64_t over = 0;
  if (held > cap) {
    over = (held - cap + 63) / 64 * 64;
    if (over > held) over = held;
  }
  const int64_t from_ring = std::min(over, c->npend[seq]), from_taps = over - from_ring;
  if (over > 0) {
    StageTimer timer(c, DFLASH_STAGE_APPEND);
    int rc = settle_ring(c, seq, from_ring);
    if (!rc && from_taps > 0) rc = settle_rows(c, seq, taps, (int)from_taps);
    if (rc) return rc;
    drop_rows(c, seq);
  }
  if (c->npend[seq] == 0) c->pstart[seq] = 0;
  const size_t T = (size_t)g.n_taps * g.hidden;
  for (int64_t r = from_taps; r < n;) {  // the rest waits: copied into the ring, in order
    const int64_t slot = (c->pstart[seq] + c->npend[seq]) % cap;
    const int64_t run = std::min(n - r, cap - slot);
    TRY_HIP(c,
            hipMemcpyAsync(ring_row(c, seq, c->npend[seq]), taps + (size_t)r * T, (size_t)run * T * 4,
                           hipMemcpyDeviceToDevice, c->st),
            "queue rows");
    c->npend[seq] += run;
    r += run;
  }
  return DFLASH_OK;
}

int dflash_ctx_settle(dflash_ctx* c, int32_t seq) {
  if (!c) return DFLASH_EINVAL;
  if (seq < 0 || seq >= c->g.max_seqs) return c->fail(DFLASH_EINVAL, "sequence %d out of range", seq);
  return settle_seq(c, seq);
}

int dflash_ctx_pending(const dflash_ctx* c, int32_t seq, int64_t* n) {
  if (!c || !n || seq < 0 || seq >= c->g.max_seqs) return DFLASH_EINVAL;
  *n = c->npend[seq];
  return DFLASH_OK;
}

// Drafter::push_context: queue_context, then settle.
int dflash_ctx_append(dflash_ctx* c, int32_t seq, int64_t pos, const float* taps, int32_t n) {
  const int rc = dflash_ctx_queue(c, seq, pos, taps, n);
  return rc ? rc : settle_seq(c, seq);
}

int dflash_ctx_truncate(dflash_ctx* c, int32_t seq, int64_t pos) {
  if (!c) return DFLASH_EINVAL;
  if (seq < 0 || seq >= c->g.max_seqs || pos < 0) return c->fail(DFLASH_EINVAL, "bad sequence or position");
  truncate_seq(c, seq, pos);
  return DFLASH_OK;
}

int dflash_ctx_reset(dflash_ctx* c, int32_t seq) {
  if (!c) return DFLASH_EINVAL;
  if (seq < 0 || seq >= c->g.max_seqs) return c->fail(DFLASH_EINVAL, "bad sequence");
  truncate_seq(c, seq, 0);
  c->first[seq] = 0;
  return DFLASH_OK;
}

int dflash_set_layer_options(dflash_ctx* c, const int32_t* windows, const int32_t* rotary) {
  if (!c) return DFLASH_EINVAL;
  const int NL = c->g.layers;
  for (int s = 0; s < c->g.max_seqs; s++)
    if (c->len[s] > 0) return c->fail(DFLASH_EINVAL, "layer options change only while no context is held");
  unsigned long long mask = ~0ull;
  for (int l = 0; l < NL; l++) {
    if (windows && windows[l] < 0) return c->fail(DFLASH_EINVAL, "layer %d: negative window", l);
    if (rotary && !rotary[l]) {
      if (l >= 64) return c->fail(DFLASH_EINVAL, "layer %d: only the first 64 layers can be unrotated", l);
      mask &= ~(1ull << l);
    }
  }
  for (int l = 0; l < NL; l++) {
    c->window[l] = windows ? windows[l] : 0;
    c->rotary[l] = rotary ? (rotary[l] != 0) : 1;
  }
  c->rot_mask = mask;
  std::fill(c->dropped.begin(), c->dropped.end(), 0);
  return DFLASH_OK;
}

int dflash_set_score_mode(dflash_ctx* c, int32_t mode) {
  if (!c) return DFLASH_EINVAL;
  if (mode != DFLASH_SCORES_AUTO && mode != DFLASH_SCORES_F64 && mode != DFLASH_SCORES_DIGITS)
    return c->fail(DFLASH_EINVAL, "score mode %d", mode);
  if (mode == DFLASH_SCORES_DIGITS && !c->lay.kd)
    return c->fail(DFLASH_EINVAL, "digit scores need head_dim 128 and four q heads per kv head");
  c->score_mode = mode;
  return DFLASH_OK;
}

int dflash_last_scores(const dflash_ctx* c, int32_t* mode) {
  if (!c || !mode) return DFLASH_EINVAL;
  *mode = c->last_scores;
  return DFLASH_OK;
}

int dflash_ctx_dropped(const dflash_ctx* c, int32_t seq, int32_t layer, int64_t* dropped) {
  if (!c || !dropped || seq < 0 || seq >= c->g.max_seqs || layer < 0 || layer >= c->g.layers) return DFLASH_EINVAL;
  *dropped = c->dropped[(size_t)seq * c->g.layers + layer];
  return DFLASH_OK;
}

// dflash.rs, Drafter::span and Drafter::next_position: the first position held and the next one
// to append (waiting rows count as held).
int dflash_ctx_span(const dflash_ctx* c, int32_t seq, int64_t* first, int64_t* end) {
  if (!c || !first || !end || seq < 0 || seq >= c->g.max_seqs) return DFLASH_EINVAL;
  *first = c->first[seq];
  *end = c->first[seq] + c->len[seq] + c->npend[seq];  // Drafter::next_position
  return DFLASH_OK;
}

int dflash_block_forward(dflash_ctx* c, int32_t n_seqs, const int32_t* seqs, const int64_t* anchors, const float* h,
                         float* logits) {
  if (!c) return DFLASH_EINVAL;
  StageTimer t(c, DFLASH_STAGE_BLOCK);
  return block_common(c, n_seqs, seqs, anchors, h, logits, false, c->g.vocab, c->g.block);
}

int dflash_block_forward_rows(dflash_ctx* c, int32_t n_seqs, const int32_t* seqs, const int64_t* anchors,
                              const float* h, int32_t block_rows, int32_t head_rows, float* logits) {
  if (!c) return DFLASH_EINVAL;
  if (block_rows < 1 || block_rows > c->g.block)
    return c->fail(DFLASH_EINVAL, "block_rows %d outside [1, %d]", block_rows, c->g.block);
  if (head_rows != c->g.vocab && (head_rows < 16 || head_rows > c->g.vocab || head_rows % 16))
    return c->fail(DFLASH_EINVAL, "head_rows %d: a multiple of 16 in [16, %d], or %d", head_rows, c->g.vocab,
                   c->g.vocab);
  StageTimer t(c, DFLASH_STAGE_BLOCK);
  return block_common(c, n_seqs, seqs, anchors, h, logits, false, head_rows, block_rows);
}

int dflash_time_stage(dflash_ctx* c, int32_t stage) {
  if (!c || stage > DFLASH_STAGE_LAST) return DFLASH_EINVAL;
  if (stage < 0) {
    c->timed_mask = 0;
    c->ev_used = 0;
    c->ev_stage.clear();
  } else {
    c->timed_mask |= 1u << stage;
  }
  return DFLASH_OK;
}

int dflash_read_timing(dflash_ctx* c, int32_t stage, double* total_ms, int64_t* count) {
  if (!c || !total_ms || !count || stage < 0 || stage > DFLASH_STAGE_LAST) return DFLASH_EINVAL;
  double tot = 0.0;
  int64_t n = 0;
  const size_t pairs = c->ev_used / 2;
  for (size_t i = 0; i < pairs; i++) {
    if (c->ev_stage[i] != stage) continue;
    TRY_HIP(c, hipEventSynchronize(c->ev_pool[2 * i + 1]), "timing sync");
    float ms = 0.f;
    TRY_HIP(c, hipEventElapsedTime(&ms, c->ev_pool[2 * i], c->ev_pool[2 * i + 1]), "timing");
    tot += ms;
    n++;
  }
  // forget the pairs once every stage that recorded some has been read: keep the others
  bool others = false;
  for (size_t i = 0; i < pairs; i++) {
    if (c->ev_stage[i] == stage) c->ev_stage[i] = -1;
    else if (c->ev_stage[i] >= 0) others = true;
  }
  if (!others) {
    TRY_HIP(c, pairs ? hipEventSynchronize(c->ev_pool[2 * pairs - 1]) : hipSuccess, "timing sync");
    c->ev_used = 0;
    c->ev_stage.clear();
  }
  *total_ms = tot;
  *count = n;
  return DFLASH_OK;
}

int dflash_block_hidden(dflash_ctx* c, int32_t n_seqs, const int32_t* seqs, const int64_t* anchors, const float* h,
                        float* hidden) {
  if (!c) return DFLASH_EINVAL;
  return block_common(c, n_seqs, seqs, anchors, h, hidden, true, c->g.vocab, c->g.block);
}

const char* dflash_last_error(const dflash_ctx* c) { return c ? c->err.c_str() : g_create_err.c_str(); }

void dflash_destroy(dflash_ctx* c) { delete c; }

int dflash_read_kv(const dflash_ctx* c, int32_t layer, int32_t seq, int32_t row0, int32_t n, float* k, float* v) {
  if (!c || !k || !v) return DFLASH_EINVAL;
  const dflash_geometry& g = c->g;
  if (layer < 0 || layer >= g.layers || seq < 0 || seq >= g.max_seqs || row0 < 0 || n < 0 || row0 + n > g.max_ctx)
    return DFLASH_EINVAL;
  if (n == 0) return DFLASH_OK;
  const size_t hd = g.head_dim, kvh = g.kv_heads;
  const size_t layer_elems = (size_t)g.max_seqs * kvh * (size_t)g.max_ctx * hd;
  hipError_t e = launch_read_cache(c->ws + c->lay.kc, g.kv_f16 != 0, layer_elems, layer, seq, row0, n, (int)kvh,
                                   (int)hd, g.max_ctx, k, c->st);
  if (e == hipSuccess)
    e = launch_read_cache(c->ws + c->lay.vc, g.kv_f16 != 0, layer_elems, layer, seq, row0, n, (int)kvh, (int)hd,
                          g.max_ctx, v, c->st);
  return e == hipSuccess ? DFLASH_OK : DFLASH_EHIP;
}

int dflash_quant_act(const float* x, int32_t rows, int32_t cols, int8_t* q, float* d, void* stream) {
  if (!x || !q || !d || rows < 0 || cols <= 0 || cols % 32) return unit_fail(DFLASH_EINVAL, "quant_act: arguments");
  if (rows == 0) return DFLASH_OK;
  hipError_t e = launch_quant_rows(x, rows, cols, q, d, (hipStream_t)stream);
  return e == hipSuccess ? DFLASH_OK : unit_fail(DFLASH_EHIP, "quant_act", e);
}

int dflash_packed_bytes(int32_t fmt, int32_t rows, int32_t cols, size_t* bytes) {
  if (!bytes || !is_fmt(fmt) || rows <= 0 || cols <= 0 || rows % 16) return DFLASH_EINVAL;
  if (fmt != DFLASH_F32 && cols % 128) return DFLASH_EINVAL;
  *bytes = packed_bytes(fmt, rows, cols);
  return DFLASH_OK;
}

int dflash_pack(int32_t fmt, int32_t rows, int32_t cols, dflash_matrix w, void* packed, void* stream) {
  size_t b;
  if (dflash_packed_bytes(fmt, rows, cols, &b) || !packed || !w.codes || (fmt != DFLASH_F32 && !w.scales))
    return unit_fail(DFLASH_EINVAL, "pack: arguments");
  hipError_t e = launch_pack(fmt, w.codes, w.scales, rows, cols, packed, 0, 1, (hipStream_t)stream);
  return e == hipSuccess ? DFLASH_OK : unit_fail(DFLASH_EHIP, "pack", e);
}

// scratch: padded activations [Mpad][cols] int8 and their scales [cols/32][Mpad] f32.
int dflash_gemm_scratch_bytes(int32_t rows, int32_t cols, int32_t m, int32_t splits, size_t* bytes) {
  if (!bytes || rows <= 0 || cols <= 0 || cols % 128 || rows % 16 || m < 1 || m > MROWS || splits < 0) return DFLASH_EINVAL;
  const int Mpad = round16(m);
  *bytes = align256((size_t)Mpad * cols) + align256((size_t)(cols / 32) * Mpad * 4);
  return DFLASH_OK;
}

int dflash_gemm(int32_t fmt, const void* packed, int32_t rows, int32_t cols, const int8_t* xq, const float* dx,
                int32_t m, float* y, int32_t splits, void* scratch, void* stream) {
  size_t need;
  if ((fmt != DFLASH_Q4_32 && fmt != DFLASH_Q8_32) || !packed || !xq || !dx || !y || !scratch ||
      dflash_gemm_scratch_bytes(rows, cols, m, splits, &need))
    return unit_fail(DFLASH_EINVAL, "gemm: arguments");
  hipStream_t st = (hipStream_t)stream;
  const int Mpad = round16(m);
  // splits: 0 lets the library choose; 1 four n-tiles, one wave each; 2..7 four n-tiles x two
  // k-waves per workgroup; 8 and more K split over the waves of one n-tile
  const int layout = splits == 0 ? -1 : splits == 1 ? 2 : splits < 8 ? 0 : 1;
  int8_t* xp = (int8_t*)scratch;
  float* dT = (float*)((uint8_t*)scratch + align256((size_t)Mpad * cols));
  hipError_t e;
  if ((e = hipMemsetAsync(xp, 0, (size_t)Mpad * cols, st)) != hipSuccess) return unit_fail(DFLASH_EHIP, "gemm: clear", e);
  if ((e = hipMemcpyAsync(xp, xq, (size_t)m * cols, hipMemcpyDeviceToDevice, st)) != hipSuccess)
    return unit_fail(DFLASH_EHIP, "gemm: copy", e);
  if ((e = launch_transpose_scales(dx, m, cols / 32, Mpad, dT, st)) != hipSuccess)
    return unit_fail(DFLASH_EHIP, "gemm: scales", e);
  GemmOut o = gemm_out(EPI_F32, m, Mpad);
  o.y = y;
  o.ld = rows;
  o.m_store = m;
  if ((e = launch_gemm_q(fmt, packed, rows, cols, xp, dT, layout, o, st)) != hipSuccess)
    return unit_fail(DFLASH_EHIP, "gemm: kernel", e);
  return DFLASH_OK;
}

int dflash_group_sums(int32_t fmt, const void* packed, int32_t rows, int32_t cols, const int8_t* xq, int32_t m,
                      int32_t* sums, void* scratch, void* stream) {
  size_t need;
  if ((fmt != DFLASH_Q4_32 && fmt != DFLASH_Q8_32) || !packed || !xq || !sums || !scratch ||
      dflash_gemm_scratch_bytes(rows, cols, m, 1, &need))
    return unit_fail(DFLASH_EINVAL, "group_sums: arguments");
  hipStream_t st = (hipStream_t)stream;
  const int Mpad = round16(m);
  int8_t* xp = (int8_t*)scratch;
  hipError_t e;
  if ((e = hipMemsetAsync(xp, 0, (size_t)Mpad * cols, st)) != hipSuccess)
    return unit_fail(DFLASH_EHIP, "group_sums: clear", e);
  if ((e = hipMemcpyAsync(xp, xq, (size_t)m * cols, hipMemcpyDeviceToDevice, st)) != hipSuccess)
    return unit_fail(DFLASH_EHIP, "group_sums: copy", e);
  if ((e = launch_group_sums(fmt, packed, rows, cols, xp, Mpad, m, sums, st)) != hipSuccess)
    return unit_fail(DFLASH_EHIP, "group_sums: kernel", e);
  return DFLASH_OK;
}

}  // extern "C"

extern "C" {

int dflash_top_k_scratch_bytes(int32_t rows, int32_t width, int32_t k, size_t* bytes) {
  if (!bytes || rows < 1 || width < 1 || k < 1 || k > 64 || k > width) return DFLASH_EINVAL;
  if (!top_k_fits(width, k)) return DFLASH_EINVAL;  // the chunks' lists must fit one merge
  *bytes = top_k_scratch(rows, width, k);
  return DFLASH_OK;
}

int dflash_top_k(const float* x, int32_t rows, int32_t width, int32_t ld, int32_t k, float* vals, int32_t* idx,
                 void* scratch, void* stream) {
  size_t need;
  if (!x || !vals || !idx || !scratch || ld < width || dflash_top_k_scratch_bytes(rows, width, k, &need))
    return unit_fail(DFLASH_EINVAL, "top_k: arguments");
  float* pv = (float*)scratch;
  int* pi = (int*)((uint8_t*)scratch + need / 2);
  hipError_t e = launch_top_k(x, rows, width, ld, k, pv, pi, vals, idx, (hipStream_t)stream);
  return e == hipSuccess ? DFLASH_OK : unit_fail(DFLASH_EHIP, "top_k", e);
}

int dflash_select_scratch_bytes(int32_t rows, int32_t width, int32_t top, size_t* bytes) {
  size_t tk;
  if (!bytes || dflash_top_k_scratch_bytes(rows, width, top, &tk)) return DFLASH_EINVAL;
  *bytes = tk + 2 * align256((size_t)rows * top * 4) + align256(select_scratch(rows, top));
  return DFLASH_OK;
}

int dflash_select(const float* logits, int32_t rows, int32_t width, int32_t ld, const float* hp, int32_t rank,
                  const uint16_t* pred, const uint16_t* succ, int32_t vocab, int32_t top, int32_t anchor,
                  int32_t* chosen, int32_t* plain, void* scratch, void* stream) {
  size_t need, tk;
  if (!logits || !hp || !pred || !succ || !chosen || !plain || !scratch || ld < width || width > vocab ||
      rank < 1 || rank > 4096 || anchor < 0 || anchor >= vocab || dflash_select_scratch_bytes(rows, width, top, &need))
    return unit_fail(DFLASH_EINVAL, "select: arguments");
  dflash_top_k_scratch_bytes(rows, width, top, &tk);
  hipStream_t st = (hipStream_t)stream;
  float* pv = (float*)scratch;
  int* pi = (int*)((uint8_t*)scratch + tk / 2);
  float* cv = (float*)((uint8_t*)scratch + tk);
  int* ci = (int*)((uint8_t*)scratch + tk + align256((size_t)rows * top * 4));
  float* scores = (float*)((uint8_t*)scratch + tk + 2 * align256((size_t)rows * top * 4));
  hipError_t e = launch_top_k(logits, rows, width, ld, top, pv, pi, cv, ci, st);
  if (e == hipSuccess) e = launch_select(cv, ci, rows, top, hp, rank, pred, succ, anchor, chosen, plain, scores, st);
  return e == hipSuccess ? DFLASH_OK : unit_fail(DFLASH_EHIP, "select", e);
}

}  // extern "C"
