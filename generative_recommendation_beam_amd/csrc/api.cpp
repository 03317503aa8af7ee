// C ABI of the decode step: host-side validation, workspace layout, launches.
//
// Every check here runs before anything is enqueued, so a nonzero status
// means no device work was issued (except GR_ERR_HIP, which reports a failed
// launch).  No allocation, no synchronisation, no global state.

#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "gr_beam.h"
#include "gr_launch.h"

namespace {

constexpr size_t kAlign = 256;

inline size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }
inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
inline int elem_bytes(int dtype) { return dtype == GR_BF16 ? 2 : 4; }

gr_status check_shape(const gr_shape *s) {
  if (!s) return GR_ERR_NULL;
  if (s->R <= 0 || s->H <= 0 || s->prompt_len <= 0 || s->window < 0) return GR_ERR_SHAPE;
  if (s->dtype != GR_BF16 && s->dtype != GR_F32) return GR_ERR_UNSUPPORTED;
  if (s->head_dim != 32 && s->head_dim != 64) return GR_ERR_UNSUPPORTED;
  if (!(s->scale >= 0.f) || !isfinite(s->scale)) return GR_ERR_SHAPE;
  // every tensor index must fit comfortably in 63 bits and grids in 31 bits
  const long long D = (long long)s->H * s->head_dim;
  if (D > 4096 || (long long)s->R * s->prompt_len * D > (1ll << 40)) return GR_ERR_SHAPE;
  // one request's prompt is addressed with 32-bit element offsets
  if ((long long)s->prompt_len * D >= (1ll << 31)) return GR_ERR_SHAPE;
  return GR_OK;
}

gr_status check_trie(const gr_shape *s, const gr_trie *t, bool need) {
  if (!need) return GR_OK;
  if (!t || !t->k || !t->v || !t->parent) return GR_ERR_NULL;
  if (t->capacity <= 0) return GR_ERR_SHAPE;
  if (t->max_depth < 1 || t->max_depth > GR_MAX_DEPTH) return GR_ERR_UNSUPPORTED;
  if (!aligned16(t->k) || !aligned16(t->v)) return GR_ERR_UNSUPPORTED;
  const long long D = (long long)s->H * s->head_dim;
  if ((long long)s->R * t->capacity * D > (1ll << 40)) return GR_ERR_SHAPE;
  return GR_OK;
}

int prompt_window(const gr_shape *s) {
  return (s->window <= 0 || s->window >= s->prompt_len) ? s->prompt_len : s->window;
}
float eff_scale(const gr_shape *s) {
  return s->scale > 0.f ? s->scale : 1.0f / sqrtf((float)s->head_dim);
}

// Partial-list geometry of a selection over n_in x vocab candidates.  The
// MFMA codebook path selects per group of 128 beams (32768 candidates), or of
// 64 beams when several 128-beam groups per request still leave CUs idle.
// score_select uses the same groups unless they leave most CUs idle (few
// requests, many candidates each): then groups of 8192, as long as their
// partial lists still fit the final merge.
struct SelGeo {
  int n_groups, kk, gpos;
  size_t bytes;  // partial lists (0 with a single group)
};
SelGeo make_geo(int R, int n_in, int vocab, int k, int gpos) {
  SelGeo g;
  g.gpos = gpos;
  g.n_groups = gr::select_groups(n_in, vocab, gpos);
  g.kk = k < gpos ? k : gpos;
  g.bytes = g.n_groups > 1 ? align_up((size_t)R * g.n_groups * g.kk * sizeof(uint64_t)) : 0;
  return g;
}
SelGeo sel_geo(int R, int n_in, int vocab, int k, bool mfma_logits = false) {
  const SelGeo big = make_geo(R, n_in, vocab, k, gr::kGroupPositions);
  if ((long long)R * big.n_groups >= gr::kSelectCUs) return big;
  if (mfma_logits) {
    // groups of 64 beams when 128-beam groups already need the merge and
    // leave CUs idle (many beams, few requests)
    const SelGeo half = make_geo(R, n_in, vocab, k, gr::kGroupPositions / 2);
    if (big.n_groups > 1 && (long long)half.n_groups * half.kk <= gr::kMergeCapacity) return half;
    return big;
  }
  const SelGeo small = make_geo(R, n_in, vocab, k, gr::kSmallGroupPositions);
  if (small.n_groups > big.n_groups && (long long)small.n_groups * small.kk <= gr::kMergeCapacity) return small;
  return big;
}

gr_status check_select(int R, int n_in, int vocab, int k, int flags) {
  if (R <= 0 || n_in <= 0 || k <= 0) return GR_ERR_SHAPE;
  if (vocab != 1 && vocab != 256) return GR_ERR_UNSUPPORTED;
  if (flags & ~GR_TOPK_LOG_SOFTMAX) return GR_ERR_UNSUPPORTED;
  if (vocab == 1 && flags) return GR_ERR_UNSUPPORTED;   // a 1-way softmax is constant
  if ((long long)n_in * vocab > (1ll << 30)) return GR_ERR_SHAPE;
  if (k > GR_MAX_K || (long long)k > (long long)n_in * vocab) return GR_ERR_K_TOO_LARGE;
  const SelGeo g = sel_geo(R, n_in, vocab, k);
  if (g.n_groups > 1 && (long long)g.n_groups * g.kk > gr::kMergeCapacity) return GR_ERR_UNSUPPORTED;
  return GR_OK;
}

// bf16 attention: resolved chain ids ([R][GR_MAX_DEPTH][beams padded to whole
// workgroups] int32), written by the chain-resolve kernel each call
size_t attn_ids_bytes(const gr_shape *s, int n_beams) {
  return s->dtype == GR_BF16 ? align_up(gr::attn_ids_bytes(s->R, n_beams)) : 0;
}
// bf16 attention with few (request, head, beam group) units: the partial
// states of the split prompt window
size_t attn_split_ws_bytes(const gr_shape *s, int n_beams) {
  if (s->dtype != GR_BF16) return 0;
  const int Lw = (s->window <= 0 || s->window >= s->prompt_len) ? s->prompt_len : s->window;
  return align_up(gr::attn_split_bytes(s->R, s->H, s->head_dim, n_beams, Lw));
}

// The bf16 codebook step feeds the attention output to the projection MFMA
// in bf16.  Its rounding perturbs a logit by about 2^-9 rms(W) |o| (RMS over
// the codes).  o is an average of the window's value rows, so |o| grows like
// sqrt(D / Lw) (D = H * head_dim): over a long window the perturbation stays
// far below the near-tie scale of the selection, but with a handful of keys
// |o| can be as large as one value row, and a wide model with a short window
// (D = 4096, 80 keys) swaps picks 1.2e-3 apart.  The bf16 projection is kept
// for windows of at least 64 keys and at least D / 8 keys (the ratio of a
// 512-wide model at 64 keys); other shapes take the fp32 path (fp32 o, fp32
// projection, scoring from fp32 logits).
constexpr int kMfmaLogitsMinWindow = 64;
constexpr int kMfmaLogitsWidthPerKey = 8;
bool use_mfma_logits(const gr_shape *s, int vocab) {
  const int Lw = prompt_window(s);
  return s->dtype == GR_BF16 && vocab == 256 && Lw >= kMfmaLogitsMinWindow &&
         (long long)Lw * kMfmaLogitsWidthPerKey >= (long long)s->H * s->head_dim;
}

struct DecodeLayout {
  size_t o_off, o_bytes, z_off, z_bytes, part_off, part_bytes, ids_off, ids_bytes, split_off, split_bytes, w_off,
      w_bytes, total;
};
DecodeLayout decode_layout(const gr_shape *s, int n_beams, int vocab, int k) {
  DecodeLayout L;
  const size_t rows = (size_t)s->R * n_beams;
  const size_t D = (size_t)s->H * s->head_dim;
  const bool mfma_logits = use_mfma_logits(s, vocab);
  // bf16 codebook path feeds the MFMA projection with a bf16 copy of o; the
  // other paths keep o in fp32 and write logits / scalar scores to z.
  L.o_bytes = align_up(rows * D * (mfma_logits ? 2 : 4));
  L.z_bytes = mfma_logits ? 0 : align_up(rows * (size_t)vocab * sizeof(float));
  const SelGeo g = sel_geo(s->R, n_beams, vocab, k, mfma_logits);
  L.part_bytes = g.bytes;
  L.o_off = 0;
  L.z_off = L.o_off + L.o_bytes;
  L.part_off = L.z_off + L.z_bytes;
  L.ids_bytes = attn_ids_bytes(s, n_beams);
  L.ids_off = L.part_off + L.part_bytes;
  L.split_bytes = attn_split_ws_bytes(s, n_beams);
  L.split_off = L.ids_off + L.ids_bytes;
  // the code-major copy of a dimension-major W (GR_W_DIM_MAJOR)
  L.w_bytes = align_up((size_t)vocab * D * elem_bytes(s->dtype));
  L.w_off = L.split_off + L.split_bytes;
  L.total = L.w_off + L.w_bytes + kAlign;  // slack for aligning ws
  return L;
}

inline char *align_ptr(void *p) {
  return (char *)(((uintptr_t)p + kAlign - 1) & ~(uintptr_t)(kAlign - 1));
}

gr::SelectOut make_out(float *score, int32_t *token, int32_t *parent, void *part, int R, int n_in, int vocab,
                       int k, bool mfma_logits = false) {
  const SelGeo g = sel_geo(R, n_in, vocab, k, mfma_logits);
  gr::SelectOut o;
  o.score = score;
  o.token = token;
  o.parent = parent;
  o.partial = (uint64_t *)part;
  o.n_groups = g.n_groups;
  o.kk = g.kk;
  o.gpos = g.gpos;
  return o;
}

gr_status attn_common(const gr_shape *shape, const void *prompt_k, const void *prompt_v, const void *q,
                      int32_t n_beams, const gr_trie *trie, const int32_t *beam_node, int32_t *dev_err) {
  gr_status st = check_shape(shape);
  if (st) return st;
  if (!prompt_k || !prompt_v || !q || !dev_err) return GR_ERR_NULL;
  if (n_beams <= 0) return GR_ERR_SHAPE;
  if ((long long)shape->R * n_beams * shape->H > (1ll << 30)) return GR_ERR_SHAPE;
  if (!aligned16(prompt_k) || !aligned16(prompt_v) || !aligned16(q)) return GR_ERR_UNSUPPORTED;
  return check_trie(shape, trie, beam_node != nullptr);
}

gr::AttnArgs attn_args(const gr_shape *shape, const void *prompt_k, const void *prompt_v, const void *q,
                       int32_t n_beams, const gr_trie *trie, const int32_t *beam_node, int32_t *dev_err) {
  gr::AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.dtype = shape->dtype;
  a.pk = prompt_k;
  a.pv = prompt_v;
  a.q = q;
  if (beam_node) {
    a.ak = trie->k;
    a.av = trie->v;
    a.parent = trie->parent;
    a.cap = trie->capacity;
    a.max_depth = trie->max_depth;
  }
  a.beam_node = beam_node;
  a.dev_err = dev_err;
  a.R = shape->R;
  a.H = shape->H;
  a.hd = shape->head_dim;
  a.Lp = shape->prompt_len;
  a.Lw = prompt_window(shape);
  a.nb = n_beams;
  a.scale = eff_scale(shape);
  return a;
}

inline gr_status hip_status(hipError_t e) {
  if (e == hipSuccess) return GR_OK;
  fprintf(stderr, "gr_beam: HIP launch failed: %s (%s)\n", hipGetErrorName(e), hipGetErrorString(e));
  return GR_ERR_HIP;
}

// hipGetLastError is sticky per thread: drop an error some earlier, unrelated
// runtime call left behind so that a launch is judged on its own status.
inline void clear_stale_error() { (void)hipGetLastError(); }

// The scoring half of a decode step (codebook logits of the current level,
// log-softmax, prior add, exact top-k) on the attention output the attention
// half left behind: bf16 head-major in the workspace for the MFMA codebook
// path, else fp32 at o_f32 (logits then go through the workspace).
gr_status enqueue_scoring(const gr_shape *shape, int n_beams, const void *W, int vocab, const float *prior,
                          int beam_width, int lsm, float *cand_out, const gr::SelectOut &so,
                          const DecodeLayout &L, char *base, const float *o_f32, hipStream_t stream) {
  const int R = shape->R;
  const int D = shape->H * shape->head_dim;
  void *o_buf = base + L.o_off;
  float *z_buf = (float *)(base + L.z_off);
  if (use_mfma_logits(shape, vocab)) {
    gr::LogitsArgs l;
    l.o = (const uint16_t *)o_buf;
    l.W = (const uint16_t *)W;
    l.prior = prior;
    l.cand_out = cand_out;
    l.R = R;
    l.n_in = n_beams;
    l.D = D;
    l.hd = shape->head_dim;
    l.k = beam_width;
    l.log_softmax = lsm;
    return hip_status(gr::launch_logits_select_bf16(l, so, stream));
  }
  gr::ProjArgs pj;
  pj.dtype = shape->dtype;
  pj.o = o_f32;
  pj.W = W;
  pj.prior = prior;
  pj.z = z_buf;
  pj.R = R;
  pj.n = n_beams;
  pj.D = D;
  pj.vocab = vocab;
  pj.add_prior = vocab == 1 ? 1 : 0;
  hipError_t e = gr::launch_project(pj, stream);
  if (e != hipSuccess) return hip_status(e);
  gr::ScoreSelectArgs sa;
  sa.logits = z_buf;
  sa.prior = vocab == 1 ? nullptr : prior;   // the scalar path added it already
  sa.cand_out = cand_out;
  sa.R = R;
  sa.n_in = n_beams;
  sa.vocab = vocab;
  sa.k = beam_width;
  sa.log_softmax = lsm;
  return hip_status(gr::launch_score_select(sa, so, stream));
}

gr_status linear_common(const gr_shape *shape, const float *state, const float *norm, const void *q,
                        int32_t n_beams, const gr_trie *trie, const int32_t *beam_node, int32_t *dev_err) {
  gr_status st = check_shape(shape);
  if (st) return st;
  if (!state || !norm || !q || !dev_err) return GR_ERR_NULL;
  if (n_beams <= 0) return GR_ERR_SHAPE;
  if ((long long)shape->R * n_beams * shape->H > (1ll << 30)) return GR_ERR_SHAPE;
  if (!aligned16(state) || !aligned16(q)) return GR_ERR_UNSUPPORTED;
  return check_trie(shape, trie, beam_node != nullptr);
}

gr::LinearAttnArgs linear_args(const gr_shape *shape, const float *state, const float *norm, const void *q,
                               int32_t n_beams, const gr_trie *trie, const int32_t *beam_node, int32_t *dev_err) {
  gr::LinearAttnArgs a;
  memset(&a, 0, sizeof(a));
  a.dtype = shape->dtype;
  a.S = state;
  a.z = norm;
  a.q = q;
  if (beam_node) {
    a.ak = trie->k;
    a.av = trie->v;
    a.parent = trie->parent;
    a.cap = trie->capacity;
    a.max_depth = trie->max_depth;
  }
  a.beam_node = beam_node;
  a.dev_err = dev_err;
  a.R = shape->R;
  a.H = shape->H;
  a.hd = shape->head_dim;
  a.nb = n_beams;
  return a;
}

// Beams in and out of every step of a generation: n_0 = 1,
// k_l = min(beam_width, n_l * vocab), n_{l+1} = k_l.
struct GenLevels {
  int n[gr::kMaxLevels], k[gr::kMaxLevels];
  long long records;  // k_0 + ... + k_{levels-2}
  int k_max;
};
GenLevels gen_levels(int levels, int vocab, int beam_width) {
  GenLevels g;
  long long n = 1;
  g.records = 0;
  g.k_max = 0;
  for (int l = 0; l < levels; ++l) {
    const long long k = n * vocab < beam_width ? n * vocab : beam_width;
    g.n[l] = (int)n;
    g.k[l] = (int)k;
    if (l + 1 < levels) g.records += k;
    if (k > g.k_max) g.k_max = (int)k;
    n = k;
  }
  return g;
}

// Workspace of a generation: the decode workspace (the largest step), the
// queries of the next step [R][k_max][D], two node-id buffers [R][k_max]
// (the nodes of a step's input beams, and of its output beams once appended)
// and the code-table row of every node [R][records].
struct GenLayout {
  size_t dec_bytes, q_off, node_off[2], row_off, total;
};
GenLayout gen_layout(const gr_shape *s, int levels, int vocab, int beam_width) {
  const GenLevels g = gen_levels(levels, vocab, beam_width);
  GenLayout L;
  L.dec_bytes = 0;
  for (int l = 0; l < levels; ++l) {
    const size_t b = decode_layout(s, g.n[l], vocab, g.k[l]).total;
    if (b > L.dec_bytes) L.dec_bytes = b;
  }
  L.dec_bytes = align_up(L.dec_bytes);
  const size_t rows = (size_t)s->R * g.k_max;
  L.q_off = L.dec_bytes;
  L.node_off[0] = L.q_off + align_up(rows * s->H * s->head_dim * elem_bytes(s->dtype));
  L.node_off[1] = L.node_off[0] + align_up(rows * sizeof(int32_t));
  L.row_off = L.node_off[1] + align_up(rows * sizeof(int32_t));
  L.total = L.row_off + align_up((size_t)s->R * (g.records > 0 ? g.records : 1) * sizeof(int32_t)) + kAlign;
  return L;
}

}  // namespace

extern "C" {

const char *gr_status_string(gr_status s) {
  switch (s) {
    case GR_OK: return "ok";
    case GR_ERR_NULL: return "a required pointer is NULL";
    case GR_ERR_SHAPE: return "a size is out of range or inconsistent";
    case GR_ERR_UNSUPPORTED: return "unsupported dtype, head_dim, vocab, flags, alignment or limit";
    case GR_ERR_CAPACITY: return "append past the arena capacity";
    case GR_ERR_K_TOO_LARGE: return "k exceeds the candidate count or GR_MAX_K";
    case GR_ERR_WORKSPACE: return "workspace too small";
    case GR_ERR_HIP: return "a HIP launch failed";
    case GR_ERR_SCRATCH_LIMIT: return "the step needs more scratch than the static no-alloc buffer holds";
    default: return "unknown status";
  }
}

// ---- multi-layer broadcast scoring

namespace {

gr_status check_xf(const gr_xf_shape *s, int32_t k) {
  if (!s) return GR_ERR_NULL;
  if (s->R <= 0 || s->n_cand <= 0 || s->user_len <= 0 || s->n_layers <= 0 || k <= 0) return GR_ERR_SHAPE;
  if (s->d_model != 128 || s->user_len % 32 != 0 || s->user_len > GR_XF_MAX_USER ||
      s->n_layers > GR_XF_MAX_LAYERS)
    return GR_ERR_UNSUPPORTED;
  if ((long long)s->R * s->n_cand * s->d_model > (1ll << 40) || s->n_cand > (1 << 30)) return GR_ERR_SHAPE;
  return check_select(s->R, s->n_cand, 1, k, 0);
}

struct XfLayout {
  size_t ukv_off, ukv_bytes, st_off, st_bytes, sc_off, sc_bytes, tok_off, tok_bytes, part_off, part_bytes, total;
};
XfLayout xf_layout(const gr_xf_shape *s, int32_t k) {
  XfLayout L;
  L.ukv_bytes = align_up(gr::xf_ukv_bytes(s->R, s->n_layers, s->user_len));
  L.st_bytes = align_up(gr::xf_user_state_bytes(s->R, s->user_len));
  L.sc_bytes = align_up((size_t)s->R * s->n_cand * sizeof(float));
  L.tok_bytes = align_up((size_t)s->R * k * sizeof(int32_t));
  L.part_bytes = sel_geo(s->R, s->n_cand, 1, k).bytes;
  L.ukv_off = 0;
  L.st_off = L.ukv_off + L.ukv_bytes;
  L.sc_off = L.st_off + L.st_bytes;
  L.tok_off = L.sc_off + L.sc_bytes;
  L.part_off = L.tok_off + L.tok_bytes;
  L.total = L.part_off + L.part_bytes + kAlign;
  return L;
}

}  // namespace

size_t gr_broadcast_workspace_size(const gr_xf_shape *shape, int32_t k) {
  if (!shape || shape->R <= 0 || shape->n_cand <= 0 || shape->user_len <= 0 || shape->n_layers <= 0 || k <= 0)
    return 0;
  return xf_layout(shape, k).total;
}

gr_status gr_broadcast_score(const gr_xf_shape *shape, const void *user_tok, const void *cand_tok,
                             const void *w_mat, const float *w_vec, int32_t k, float *out_score,
                             int32_t *out_index, float *cand_scores, void *ws, size_t ws_bytes,
                             hipStream_t stream) {
  gr_status st = check_xf(shape, k);
  if (st) return st;
  if (!user_tok || !cand_tok || !w_mat || !w_vec || !out_score || !out_index) return GR_ERR_NULL;
  if (!aligned16(user_tok) || !aligned16(cand_tok) || !aligned16(w_mat) || !aligned16(w_vec) ||
      (cand_scores && !aligned16(cand_scores)))
    return GR_ERR_UNSUPPORTED;
  const XfLayout L = xf_layout(shape, k);
  if (!ws || ws_bytes < L.total) return GR_ERR_WORKSPACE;
  char *base = align_ptr(ws);
  gr::XfArgs a;
  a.user = user_tok;
  a.cand = cand_tok;
  a.w_mat = w_mat;
  a.w_vec = w_vec;
  a.ukv = base + L.ukv_off;
  a.user_state = base + L.st_off;
  a.score = cand_scores ? cand_scores : (float *)(base + L.sc_off);
  a.R = shape->R;
  a.N = shape->n_cand;
  a.Lu = shape->user_len;
  a.L = shape->n_layers;
  clear_stale_error();
  hipError_t e = gr::launch_xf_scores(a, stream);
  if (e != hipSuccess) return hip_status(e);
  gr::ScoreSelectArgs sa;
  sa.logits = a.score;
  sa.prior = nullptr;
  sa.cand_out = nullptr;
  sa.R = shape->R;
  sa.n_in = shape->n_cand;
  sa.vocab = 1;
  sa.k = k;
  sa.log_softmax = 0;
  const gr::SelectOut o = make_out(out_score, (int32_t *)(base + L.tok_off), out_index,
                                   L.part_bytes ? base + L.part_off : nullptr, shape->R, shape->n_cand, 1, k);
  return hip_status(gr::launch_score_select(sa, o, stream));
}

size_t gr_attn_workspace_size(const gr_shape *shape, int32_t n_beams) {
  if (check_shape(shape) || n_beams <= 0) return 0;
  const size_t b = attn_ids_bytes(shape, n_beams) + attn_split_ws_bytes(shape, n_beams);
  return b ? b + kAlign : 0;
}

size_t gr_topk_workspace_size(int32_t R, int32_t n_in, int32_t vocab, int32_t k) {
  if (R <= 0 || n_in <= 0 || k <= 0 || (vocab != 1 && vocab != 256)) return 0;
  const SelGeo g = sel_geo(R, n_in, vocab, k);
  return g.bytes ? g.bytes + kAlign : 0;
}

size_t gr_decode_workspace_size(const gr_shape *shape, int32_t n_beams, int32_t vocab, int32_t k) {
  if (check_shape(shape) || n_beams <= 0 || k <= 0 || (vocab != 1 && vocab != 256)) return 0;
  return decode_layout(shape, n_beams, vocab, k).total;
}

gr_status gr_trie_append(const gr_shape *shape, const gr_trie *trie, int32_t base, int32_t n_new,
                         const void *k_new, const void *v_new, const int32_t *parent_beam,
                         const int32_t *prev_nodes, int32_t n_prev, int32_t *node_out, int32_t *dev_err,
                         hipStream_t stream) {
  gr_status st = check_shape(shape);
  if (st) return st;
  if (!trie || !k_new || !v_new || !dev_err) return GR_ERR_NULL;
  if (!trie->k || !trie->v || !trie->parent) return GR_ERR_NULL;
  if (n_new <= 0 || base < 0 || trie->capacity <= 0) return GR_ERR_SHAPE;
  if ((parent_beam == nullptr) != (prev_nodes == nullptr)) return GR_ERR_NULL;
  if (prev_nodes && n_prev <= 0) return GR_ERR_SHAPE;
  if ((long long)base + n_new > trie->capacity) return GR_ERR_CAPACITY;
  if (!aligned16(trie->k) || !aligned16(trie->v) || !aligned16(k_new) || !aligned16(v_new))
    return GR_ERR_UNSUPPORTED;
  if ((long long)shape->R * trie->capacity * shape->H * shape->head_dim > (1ll << 40)) return GR_ERR_SHAPE;
  gr::AppendArgs a;
  a.elem_bytes = elem_bytes(shape->dtype);
  a.ak = trie->k;
  a.av = trie->v;
  a.parent = trie->parent;
  a.k_new = k_new;
  a.v_new = v_new;
  a.parent_beam = parent_beam;
  a.prev_nodes = prev_nodes;
  a.node_out = node_out;
  a.dev_err = dev_err;
  a.R = shape->R;
  a.H = shape->H;
  a.hd = shape->head_dim;
  a.cap = trie->capacity;
  a.base = base;
  a.n_new = n_new;
  a.n_prev = prev_nodes ? n_prev : 0;
  clear_stale_error();
  return hip_status(gr::launch_trie_append(a, stream));
}

gr_status gr_prefix_attn(const gr_shape *shape, const void *prompt_k, const void *prompt_v, const void *q,
                         int32_t n_beams, const gr_trie *trie, const int32_t *beam_node, float *out, void *ws,
                         size_t ws_bytes, int32_t *dev_err, hipStream_t stream) {
  gr_status st = attn_common(shape, prompt_k, prompt_v, q, n_beams, trie, beam_node, dev_err);
  if (st) return st;
  if (!out) return GR_ERR_NULL;
  if (!aligned16(out)) return GR_ERR_UNSUPPORTED;
  gr::AttnArgs a = attn_args(shape, prompt_k, prompt_v, q, n_beams, trie, beam_node, dev_err);
  a.out_f32 = out;
  const size_t ids_bytes = attn_ids_bytes(shape, n_beams), split_bytes = attn_split_ws_bytes(shape, n_beams);
  if ((beam_node && ids_bytes) || split_bytes) {
    if (!ws || ws_bytes < gr_attn_workspace_size(shape, n_beams)) return GR_ERR_WORKSPACE;
    a.chain_ids = (int32_t *)align_ptr(ws);
    a.split_ws = split_bytes ? (float *)(align_ptr(ws) + ids_bytes) : nullptr;
  }
  clear_stale_error();
  return hip_status(gr::launch_attn(a, stream));
}

gr_status gr_beam_topk(int32_t R, int32_t n_in, int32_t vocab, int32_t k, int32_t flags, const float *logits,
                       const float *prior, float *out_score, int32_t *out_token, int32_t *out_parent,
                       float *cand_out, void *ws, size_t ws_bytes, hipStream_t stream) {
  gr_status st = check_select(R, n_in, vocab, k, flags);
  if (st) return st;
  if (!logits || !out_score || !out_token || !out_parent) return GR_ERR_NULL;
  if (!aligned16(logits) || (cand_out && !aligned16(cand_out))) return GR_ERR_UNSUPPORTED;
  const size_t need = gr_topk_workspace_size(R, n_in, vocab, k);
  if (need && (!ws || ws_bytes < need)) return GR_ERR_WORKSPACE;
  gr::ScoreSelectArgs a;
  a.logits = logits;
  a.prior = prior;
  a.cand_out = cand_out;
  a.R = R;
  a.n_in = n_in;
  a.vocab = vocab;
  a.k = k;
  a.log_softmax = (flags & GR_TOPK_LOG_SOFTMAX) ? 1 : 0;
  const gr::SelectOut o = make_out(out_score, out_token, out_parent, need ? align_ptr(ws) : nullptr, R, n_in,
                                   vocab, k);
  clear_stale_error();
  return hip_status(gr::launch_score_select(a, o, stream));
}

}  // extern "C"

namespace {

// Chain records and queries left in the code tables of a generation (bf16,
// small arenas): node n of request r is row row[r][n] of tab
// ([tab_rows][3][H][head_dim]), n < rows.
struct RecTable {
  const void *tab;
  int32_t *row;
  int rows, tab_rows;
};

gr_status decode_step_impl(const gr_shape *shape, const void *prompt_k, const void *prompt_v, const void *q,
                           int32_t n_beams, const gr_trie *trie, const int32_t *beam_node, const void *W,
                           int32_t vocab, const float *prior, int32_t beam_width, int32_t flags, float *out_score,
                           int32_t *out_token, int32_t *out_parent, float *attn_out, float *cand_out, void *ws,
                           size_t ws_bytes, int32_t *dev_err, hipStream_t stream, const RecTable *rt) {
  gr_status st = attn_common(shape, prompt_k, prompt_v, q, n_beams, trie, beam_node, dev_err);
  if (st) return st;
  const int32_t stage = flags & (GR_STEP_ATTENTION | GR_STEP_SELECTION);
  const bool run_attn = stage != GR_STEP_SELECTION;
  const bool run_select = stage != GR_STEP_ATTENTION;
  const bool w_dim_major = (flags & GR_W_DIM_MAJOR) != 0;
  flags &= ~(GR_STEP_ATTENTION | GR_STEP_SELECTION | GR_W_DIM_MAJOR);
  st = check_select(shape->R, n_beams, vocab, beam_width, flags);
  if (st) return st;
  if (!W || !out_score || !out_token || !out_parent) return GR_ERR_NULL;
  if (!aligned16(W) || (attn_out && !aligned16(attn_out)) || (cand_out && !aligned16(cand_out)))
    return GR_ERR_UNSUPPORTED;
  const DecodeLayout L = decode_layout(shape, n_beams, vocab, beam_width);
  if (!ws || ws_bytes < L.total) return GR_ERR_WORKSPACE;
  char *base = align_ptr(ws);
  void *o_buf = base + L.o_off;
  void *part = L.part_bytes ? base + L.part_off : nullptr;
  const int lsm = (flags & GR_TOPK_LOG_SOFTMAX) ? 1 : 0;
  const gr::SelectOut so = make_out(out_score, out_token, out_parent, part, shape->R, n_beams, vocab, beam_width,
                                    use_mfma_logits(shape, vocab));

  gr::AttnArgs a = attn_args(shape, prompt_k, prompt_v, q, n_beams, trie, beam_node, dev_err);
  if (rt && beam_node) {
    a.rec_tab = rt->tab;
    a.rec_row = rt->row;
    a.rec_rows = rt->rows;
    a.rec_tab_rows = rt->tab_rows;
  }
  a.chain_ids = L.ids_bytes ? (int32_t *)(base + L.ids_off) : nullptr;
  a.split_ws = L.split_bytes ? (float *)(base + L.split_off) : nullptr;
  const bool mfma_logits = use_mfma_logits(shape, vocab);
  const float *o_f32 = nullptr;
  if (mfma_logits) {
    a.out_lowp = o_buf;
    a.out_f32 = attn_out;
  } else {
    a.out_f32 = attn_out ? attn_out : (float *)o_buf;
    o_f32 = a.out_f32;
  }
  clear_stale_error();
  hipError_t e = hipSuccess;
  if (run_attn) {
    e = gr::launch_attn(a, stream);
    if (e != hipSuccess) return hip_status(e);
  }
  if (!run_select) return GR_OK;
  if (w_dim_major) {
    // [D][vocab] -> [vocab][D] in the workspace
    void *wt = base + L.w_off;
    e = gr::launch_transpose(W, wt, shape->H * shape->head_dim, vocab, elem_bytes(shape->dtype), stream);
    if (e != hipSuccess) return hip_status(e);
    W = wt;
  }
  return enqueue_scoring(shape, n_beams, W, vocab, prior, beam_width, lsm, cand_out, so, L, base,
                         o_f32, stream);
}

}  // namespace

extern "C" {

gr_status gr_decode_step(const gr_shape *shape, const void *prompt_k, const void *prompt_v, const void *q,
                         int32_t n_beams, const gr_trie *trie, const int32_t *beam_node, const void *W,
                         int32_t vocab, const float *prior, int32_t beam_width, int32_t flags, float *out_score,
                         int32_t *out_token, int32_t *out_parent, float *attn_out, float *cand_out, void *ws,
                         size_t ws_bytes, int32_t *dev_err, hipStream_t stream) {
  return decode_step_impl(shape, prompt_k, prompt_v, q, n_beams, trie, beam_node, W, vocab, prior, beam_width,
                          flags, out_score, out_token, out_parent, attn_out, cand_out, ws, ws_bytes, dev_err, stream,
                          nullptr);
}

gr_status gr_linear_state(const gr_shape *shape, const void *prompt_k, const void *prompt_v, float *state,
                          float *norm, hipStream_t stream) {
  gr_status st = check_shape(shape);
  if (st) return st;
  if (!prompt_k || !prompt_v || !state || !norm) return GR_ERR_NULL;
  if (!aligned16(prompt_k) || !aligned16(prompt_v) || !aligned16(state)) return GR_ERR_UNSUPPORTED;
  gr::LinearStateArgs a;
  a.dtype = shape->dtype;
  a.pk = prompt_k;
  a.pv = prompt_v;
  a.S = state;
  a.z = norm;
  a.R = shape->R;
  a.H = shape->H;
  a.hd = shape->head_dim;
  a.Lp = shape->prompt_len;
  a.Lw = prompt_window(shape);
  clear_stale_error();
  return hip_status(gr::launch_linear_state(a, stream));
}

gr_status gr_linear_attn(const gr_shape *shape, const float *state, const float *norm, const void *q,
                         int32_t n_beams, const gr_trie *trie, const int32_t *beam_node, float *out,
                         int32_t *dev_err, hipStream_t stream) {
  gr_status st = linear_common(shape, state, norm, q, n_beams, trie, beam_node, dev_err);
  if (st) return st;
  if (!out) return GR_ERR_NULL;
  if (!aligned16(out)) return GR_ERR_UNSUPPORTED;
  gr::LinearAttnArgs a = linear_args(shape, state, norm, q, n_beams, trie, beam_node, dev_err);
  a.out_f32 = out;
  clear_stale_error();
  return hip_status(gr::launch_linear_attn(a, stream));
}

gr_status gr_linear_decode_step(const gr_shape *shape, const float *state, const float *norm, const void *q,
                                int32_t n_beams, const gr_trie *trie, const int32_t *beam_node, const void *W,
                                int32_t vocab, const float *prior, int32_t beam_width, int32_t flags,
                                float *out_score, int32_t *out_token, int32_t *out_parent, float *attn_out,
                                float *cand_out, void *ws, size_t ws_bytes, int32_t *dev_err,
                                hipStream_t stream) {
  gr_status st = linear_common(shape, state, norm, q, n_beams, trie, beam_node, dev_err);
  if (st) return st;
  const int32_t stage = flags & (GR_STEP_ATTENTION | GR_STEP_SELECTION);
  const bool run_attn = stage != GR_STEP_SELECTION;
  const bool run_select = stage != GR_STEP_ATTENTION;
  flags &= ~(GR_STEP_ATTENTION | GR_STEP_SELECTION);
  st = check_select(shape->R, n_beams, vocab, beam_width, flags);
  if (st) return st;
  if (!W || !out_score || !out_token || !out_parent) return GR_ERR_NULL;
  if (!aligned16(W) || (attn_out && !aligned16(attn_out)) || (cand_out && !aligned16(cand_out)))
    return GR_ERR_UNSUPPORTED;
  const DecodeLayout L = decode_layout(shape, n_beams, vocab, beam_width);
  if (!ws || ws_bytes < L.total) return GR_ERR_WORKSPACE;
  char *base = align_ptr(ws);
  void *o_buf = base + L.o_off;
  void *part = L.part_bytes ? base + L.part_off : nullptr;
  const int lsm = (flags & GR_TOPK_LOG_SOFTMAX) ? 1 : 0;
  const bool mfma_logits = use_mfma_logits(shape, vocab);
  const gr::SelectOut so = make_out(out_score, out_token, out_parent, part, shape->R, n_beams, vocab, beam_width,
                                    mfma_logits);
  gr::LinearAttnArgs a = linear_args(shape, state, norm, q, n_beams, trie, beam_node, dev_err);
  const float *o_f32 = nullptr;
  if (mfma_logits) {
    a.out_lowp = o_buf;
    a.out_f32 = attn_out;
  } else {
    a.out_f32 = attn_out ? attn_out : (float *)o_buf;
    o_f32 = a.out_f32;
  }
  clear_stale_error();
  if (run_attn) {
    const hipError_t e = gr::launch_linear_attn(a, stream);
    if (e != hipSuccess) return hip_status(e);
  }
  if (!run_select) return GR_OK;
  return enqueue_scoring(shape, n_beams, W, vocab, prior, beam_width, lsm, cand_out, so, L, base, o_f32,
                         stream);
}

gr_status gr_code_table(const gr_shape *shape, int32_t levels, int32_t vocab, int32_t d_emb, const void *emb,
                        const void *w_qkv, void *table, hipStream_t stream) {
  gr_status st = check_shape(shape);
  if (st) return st;
  if (!emb || !w_qkv || !table) return GR_ERR_NULL;
  if (levels <= 0) return GR_ERR_SHAPE;
  if (levels > gr::kMaxLevels || vocab != 256) return GR_ERR_UNSUPPORTED;
  if (d_emb <= 0 || d_emb % 16 != 0 || d_emb > 16384) return GR_ERR_UNSUPPORTED;
  if (!aligned16(emb) || !aligned16(w_qkv) || !aligned16(table)) return GR_ERR_UNSUPPORTED;
  gr::CodeTableArgs a;
  a.dtype = shape->dtype;
  a.emb = emb;
  a.w_qkv = w_qkv;
  a.table = table;
  a.levels = levels;
  a.V = vocab;
  a.D = shape->H * shape->head_dim;
  a.De = d_emb;
  clear_stale_error();
  return hip_status(gr::launch_code_table(a, stream));
}

}  // extern "C"

namespace {

// rt: the records stay in the code tables, whose row row0 + code each new
// node gets in rt->row; the arena's keys and values are not written.
gr_status append_codes_impl(const gr_shape *shape, const gr_trie *trie, int32_t base, int32_t n_new,
                            const void *table, int32_t vocab, const int32_t *token, const int32_t *parent_beam,
                            const int32_t *prev_nodes, int32_t n_prev, void *q_out, int32_t *node_out,
                            int32_t *dev_err, hipStream_t stream, const RecTable *rt, int32_t row0) {
  gr_status st = check_shape(shape);
  if (st) return st;
  if (!trie || !table || !token || !dev_err) return GR_ERR_NULL;
  if (!trie->k || !trie->v || !trie->parent) return GR_ERR_NULL;
  if (vocab != 256) return GR_ERR_UNSUPPORTED;
  if (n_new <= 0 || base < 0 || trie->capacity <= 0) return GR_ERR_SHAPE;
  if ((parent_beam == nullptr) != (prev_nodes == nullptr)) return GR_ERR_NULL;
  if (prev_nodes && n_prev <= 0) return GR_ERR_SHAPE;
  if ((long long)base + n_new > trie->capacity) return GR_ERR_CAPACITY;
  if (!aligned16(trie->k) || !aligned16(trie->v) || !aligned16(table) || (q_out && !aligned16(q_out)))
    return GR_ERR_UNSUPPORTED;
  if ((long long)shape->R * trie->capacity * shape->H * shape->head_dim > (1ll << 40)) return GR_ERR_SHAPE;
  gr::AppendCodesArgs a;
  a.elem_bytes = elem_bytes(shape->dtype);
  a.ak = trie->k;
  a.av = trie->v;
  a.q_out = q_out;
  a.parent = trie->parent;
  a.table = table;
  a.token = token;
  a.parent_beam = parent_beam;
  a.prev_nodes = prev_nodes;
  a.node_out = node_out;
  a.dev_err = dev_err;
  a.R = shape->R;
  a.H = shape->H;
  a.hd = shape->head_dim;
  a.cap = trie->capacity;
  a.base = base;
  a.n_new = n_new;
  a.n_prev = prev_nodes ? n_prev : 0;
  a.V = vocab;
  if (rt) {
    if ((long long)base + n_new > rt->rows) return GR_ERR_CAPACITY;
    a.rec_row = rt->row;
    a.row_n = rt->rows;
    a.row0 = row0;
  }
  clear_stale_error();
  return hip_status(gr::launch_append_codes(a, stream));
}

}  // namespace

extern "C" {

gr_status gr_append_codes(const gr_shape *shape, const gr_trie *trie, int32_t base, int32_t n_new,
                          const void *table, int32_t vocab, const int32_t *token, const int32_t *parent_beam,
                          const int32_t *prev_nodes, int32_t n_prev, void *q_out, int32_t *node_out,
                          int32_t *dev_err, hipStream_t stream) {
  return append_codes_impl(shape, trie, base, n_new, table, vocab, token, parent_beam, prev_nodes, n_prev, q_out,
                           node_out, dev_err, stream, nullptr, 0);
}

size_t gr_workspace_size(const gr_shape *shape, int32_t n_beams, int32_t vocab, int32_t k) {
  const size_t d = gr_decode_workspace_size(shape, n_beams, vocab, k);
  const size_t a = gr_attn_workspace_size(shape, n_beams);
  const size_t t = shape ? gr_topk_workspace_size(shape->R, n_beams, vocab, k) : 0;
  return d > a ? (d > t ? d : t) : (a > t ? a : t);
}

size_t gr_generate_workspace_size(const gr_shape *shape, int32_t levels, int32_t vocab, int32_t beam_width) {
  if (check_shape(shape) || levels < 1 || levels > gr::kMaxLevels || vocab != 256 || beam_width <= 0 ||
      beam_width > GR_MAX_K)
    return 0;
  return gen_layout(shape, levels, vocab, beam_width).total;
}

gr_status gr_generate(const gr_shape *shape, const void *prompt_k, const void *prompt_v, const void *q0,
                      int32_t levels, const void *W, const void *tables, int32_t vocab, int32_t beam_width,
                      const gr_trie *trie, float *out_score, int32_t *out_token, int32_t *out_parent,
                      int32_t *out_ids, void *ws, size_t ws_bytes, int32_t *dev_err, hipStream_t stream) {
  gr_status st = check_shape(shape);
  if (st) return st;
  if (!prompt_k || !prompt_v || !q0 || !W || !out_score || !out_token || !out_parent || !out_ids || !dev_err)
    return GR_ERR_NULL;
  if (levels < 1 || levels > gr::kMaxLevels || vocab != 256) return GR_ERR_UNSUPPORTED;
  if (beam_width <= 0) return GR_ERR_SHAPE;
  if (beam_width > GR_MAX_K) return GR_ERR_K_TOO_LARGE;
  if (!aligned16(W) || !aligned16(q0) || (tables && !aligned16(tables))) return GR_ERR_UNSUPPORTED;
  const GenLevels g = gen_levels(levels, vocab, beam_width);
  if (levels > 1) {
    if (!tables || !trie) return GR_ERR_NULL;
    st = check_trie(shape, trie, true);
    if (st) return st;
    if (g.records > trie->capacity) return GR_ERR_CAPACITY;
    if (trie->max_depth < levels - 1) return GR_ERR_UNSUPPORTED;
  }
  // every step's own checks, before anything is enqueued
  for (int l = 0; l < levels; ++l) {
    st = attn_common(shape, prompt_k, prompt_v, q0, g.n[l], nullptr, nullptr, dev_err);
    if (st) return st;
    st = check_select(shape->R, g.n[l], vocab, g.k[l], GR_TOPK_LOG_SOFTMAX);
    if (st) return st;
  }
  const GenLayout L = gen_layout(shape, levels, vocab, beam_width);
  if (!ws || ws_bytes < L.total) return GR_ERR_WORKSPACE;
  char *base = align_ptr(ws);
  void *dec_ws = base;
  void *qbuf = base + L.q_off;
  int32_t *nodes[2] = {(int32_t *)(base + L.node_off[0]), (int32_t *)(base + L.node_off[1])};
  const int R = shape->R;
  const size_t D = (size_t)shape->H * shape->head_dim;
  const size_t eb = elem_bytes(shape->dtype);
  const size_t w_level = (size_t)vocab * D * eb;
  const size_t t_level = (size_t)vocab * 3 * D * eb;
  // bf16 chains small enough to resolve inside the attention kernel read
  // their records and queries straight from the tables (a few hundred KB per
  // level, held in L2), so neither the arena's keys and values nor the next
  // queries are written.
  RecTable rt;
  rt.tab = tables;
  rt.row = (int32_t *)(base + L.row_off);
  rt.rows = (int)g.records;
  rt.tab_rows = (levels - 1) * vocab;
  const RecTable *rtp =
      levels > 1 && shape->dtype == GR_BF16 && trie->capacity <= gr::kLdsChainNodes ? &rt : nullptr;

  gr::TraceArgs tr;
  tr.R = R;
  tr.levels = levels;
  long long off = 0, rec_base = 0;
  for (int l = 0; l < levels; ++l) {
    tr.off[l] = off;
    tr.k[l] = g.k[l];
    float *score = out_score + off;
    int32_t *token = out_token + off;
    int32_t *parent = out_parent + off;
    const int32_t *beam_node = l > 0 ? nodes[(l - 1) & 1] : nullptr;
    st = decode_step_impl(shape, prompt_k, prompt_v, l > 0 ? qbuf : q0, g.n[l], l > 0 ? trie : nullptr,
                          beam_node, (const char *)W + l * w_level, vocab,
                          l > 0 ? out_score + tr.off[l - 1] : nullptr, g.k[l], GR_TOPK_LOG_SOFTMAX, score, token,
                          parent, nullptr, nullptr, dec_ws, L.dec_bytes, dev_err, stream, rtp);
    if (st) return st;
    if (l + 1 < levels) {
      // the chosen codes become the next step's beams: records at nodes
      // [rec_base, rec_base + k_l), their queries into qbuf
      st = append_codes_impl(shape, trie, (int32_t)rec_base, g.k[l], (const char *)tables + l * t_level, vocab,
                             token, l > 0 ? parent : nullptr, l > 0 ? beam_node : nullptr, g.n[l],
                             rtp ? nullptr : qbuf, nodes[l & 1], dev_err, stream, rtp, l * vocab);
      if (st) return st;
      rec_base += g.k[l];
    }
    off += (long long)R * g.k[l];
  }
  tr.token = out_token;
  tr.parent = out_parent;
  tr.ids = out_ids;
  tr.dev_err = dev_err;
  clear_stale_error();
  return hip_status(gr::launch_trace_ids(tr, stream));
}

}  // extern "C"
