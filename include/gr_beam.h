/*
 * gr_beam.h -- C ABI of the shared-prefix large-beam decode step (gfx950).
 *
 * One decode step of semantic-ID generative recall in which every beam of a
 * request shares one prompt:
 *   1. each beam's query attends once to the shared prompt K/V (stored a
 *      single time) plus its own short chain of ancestor records;
 *   2. the attention output is projected onto the 256 codes of the current
 *      semantic-ID level;
 *   3. log-softmax over those 256 codes;
 *   4. the running beam score is added;
 *   5. the best B of the B_in x 256 candidates are selected.
 * Around the step: whole semantic-ID generation with every level enqueued on
 * the device (gr_code_table, gr_append_codes, gr_generate), and the same step
 * with linear attention over one shared prompt state (gr_linear_state,
 * gr_linear_attn, gr_linear_decode_step).
 *
 * Sources (page title, section):
 *   - Engineering Exploration of Generative Recall (ASGR), 4.1 Superman
 *     Optimizer (attention as QK^T, scale, mask, softmax, weighted sum),
 *     4.2 Custom Beam Search (only the 256 codes of the current position are
 *     scored and ranked), 4.4 Tree-Based Attention (beams in a trie, shared
 *     prefixes stored once, a token sees only ancestors on its own branch),
 *     4.5 Sliding-Window Attention (window over the most recent prompt
 *     tokens).
 *   - TransRetrieval, Hardware-aware inference optimization (one user KV
 *     cache broadcast to all candidates without copies; packed single-query
 *     candidates isolated by masking) and Model-based Retrieval / GPU
 *     retrieval (scalar candidate scores, candidate selection on the GPU).
 *   - OneLA, Abstract (one shared prompt-derived state, compact append-only
 *     records of each beam's divergent transitions, a light ancestry index,
 *     beams advance without moving or copying records).
 *
 * Conventions for every entry point:
 *   - All tensor arguments are DEVICE pointers, row-major, owned by the
 *     caller.  The library never allocates, frees or synchronises; it keeps no
 *     global state and is re-entrant across streams.  Work is enqueued on
 *     `stream` and the call returns at once.
 *   - The return value reports host-checkable errors, plus GR_ERR_HIP for a
 *     launch the HIP runtime refused.  With any other status nothing was
 *     enqueued and no output was touched; after GR_ERR_HIP, launches that
 *     the same call made earlier may have been enqueued.
 *   - Data-dependent errors are found on the device and OR-ed into *dev_err
 *     (a device int32 the caller zeroes before the call and reads after
 *     synchronising).  Outputs are undefined when it is nonzero.
 *   - Element type `dtype`: GR_BF16 (bfloat16 storage, fp32 accumulation) or
 *     GR_F32 (fp32 storage and arithmetic).  Attention outputs and scores are
 *     always fp32.
 *   - head_dim must be 32 or 64; vocab must be 256 (codebook step) or 1
 *     (scalar scoring).
 */
#ifndef GR_BEAM_H
#define GR_BEAM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t gr_status;
enum {
  GR_OK = 0,
  GR_ERR_NULL = 1,         /* a required pointer is NULL */
  GR_ERR_SHAPE = 2,        /* a size is <= 0 or inconsistent */
  GR_ERR_UNSUPPORTED = 3,  /* dtype, head_dim, vocab, flags or depth limit */
  GR_ERR_CAPACITY = 4,     /* base + n_new > capacity */
  GR_ERR_K_TOO_LARGE = 5,  /* k > n_in * vocab, or k above GR_MAX_K */
  GR_ERR_WORKSPACE = 6,    /* ws too small (see the *_workspace_size calls) */
  GR_ERR_HIP = 7,          /* a HIP launch failed */
  GR_ERR_SCRATCH_LIMIT = 8 /* gr_decode_step_noalloc: the step needs more
                              scratch than GR_NOALLOC_SCRATCH_BYTES */
};
enum { GR_F32 = 0, GR_BF16 = 1 };

/* Bits OR-ed into *dev_err by the device. */
enum {
  GR_DEVERR_PARENT_RANGE = 1, /* a node or parent id outside [-1, capacity) */
  GR_DEVERR_PARENT_ORDER = 2, /* a parent id not older than its child */
  GR_DEVERR_DEPTH = 4,        /* a chain longer than max_depth */
  GR_DEVERR_BEAM_RANGE = 8,   /* parent_beam outside [0, n_prev) */
  GR_DEVERR_TOKEN_RANGE = 16  /* a chosen code outside [0, vocab), or a traced
                                 parent outside the previous step's beams */
};

/* gr_beam_topk / gr_decode_step flags */
enum {
  GR_TOPK_LOG_SOFTMAX = 1,
  /* gr_decode_step only: enqueue just one stage of the step.  With neither
   * bit (or both) the whole step runs.  ATTENTION writes the attention output
   * into the workspace; SELECTION reads it from there, so a SELECTION call
   * must follow an ATTENTION call with the same arguments and workspace on the
   * same stream.  Splitting lets a caller place other work or timing events
   * between the stages; the kernels and their arguments are the same as in
   * the single call. */
  GR_STEP_ATTENTION = 2,
  GR_STEP_SELECTION = 4,
  /* gr_decode_step only: W is given dimension-major, [H*head_dim][vocab]
   * (the orientation of the pages' D x 256 projection), instead of the
   * default code-major [vocab][H*head_dim].  The step then transposes it
   * into its workspace first (one small extra launch). */
  GR_W_DIM_MAJOR = 8
};

#define GR_MAX_DEPTH 8    /* longest ancestor chain a beam may have */
#define GR_MAX_K 2048     /* largest k (beam width / selected count) */

/* Shape of one batched step.  R requests, each with prompt_len prompt rows of
 * H heads x head_dim.  window = number of most recent prompt rows attended
 * (0 = all; values >= prompt_len mean all).  scale = score scale (0 means
 * 1/sqrt(head_dim)). */
typedef struct {
  int32_t R, H, head_dim, prompt_len, window, dtype;
  float scale;
} gr_shape;

/* The append-only record arena (the trie).  For request r and node n:
 *   k[r][n][H][head_dim], v[r][n][H][head_dim]  (dtype)
 *   parent[r][n] in [-1, n)  (-1 = child of the prompt)
 * capacity = nodes per request; max_depth <= GR_MAX_DEPTH bounds the chain
 * length a step walks (a longer chain sets GR_DEVERR_DEPTH). */
typedef struct {
  void *k, *v;
  int32_t *parent;
  int32_t capacity, max_depth;
} gr_trie;

/* gr_trie_append -- append one record per new beam (OneLA, Abstract:
 * append-only records; existing records are neither moved nor copied).
 *   For every request r and j < n_new, node n = base + j receives
 *     trie.k[r][n] = k_new[r][j],  trie.v[r][n] = v_new[r][j]
 *     trie.parent[r][n] = prev_nodes[r][parent_beam[r][j]]   (or -1 when
 *                         parent_beam and prev_nodes are both NULL: a first
 *                         level hanging off the prompt)
 *     node_out[r][j] = n   (optional, may be NULL)
 *   k_new, v_new: [R][n_new][H][head_dim] dtype.  parent_beam: [R][n_new]
 *   int32 index of the previous beam each new beam extends.  prev_nodes:
 *   [R][n_prev] int32 arena node of each previous beam.
 *   Host errors: NULL pointers (shape, trie, k_new, v_new, dev_err, trie
 *   arrays), n_new <= 0, base < 0, base + n_new > capacity (CAPACITY),
 *   exactly one of parent_beam / prev_nodes NULL, n_prev <= 0 with
 *   prev_nodes.  Device errors: parent_beam outside [0, n_prev)
 *   (BEAM_RANGE), a previous node outside [-1, n) (PARENT_ORDER or
 *   PARENT_RANGE); the offending parent is stored as -1. */
gr_status gr_trie_append(const gr_shape *shape, const gr_trie *trie,
                         int32_t base, int32_t n_new, const void *k_new,
                         const void *v_new, const int32_t *parent_beam,
                         const int32_t *prev_nodes, int32_t n_prev,
                         int32_t *node_out, int32_t *dev_err,
                         hipStream_t stream);

/* gr_prefix_attn -- attention of every beam over the shared prompt plus its
 * own ancestor chain (ASGR 4.1, 4.4, 4.5; TransRetrieval, Hardware-aware
 * inference optimization; OneLA, Abstract).
 *   keys(r,b) = prompt rows [prompt_len - Lw, prompt_len) then the chain of
 *               beam_node[r][b] from its root-most record down to itself;
 *   s_j = scale * q[r][b][h] . k_j[h];  p = softmax(s) over keys(r,b);
 *   out[r][b][h*head_dim + i] = sum_j p_j v_j[h][i].
 *   prompt_k, prompt_v: [R][prompt_len][H][head_dim] dtype (read once per
 *   request and head, never copied per beam).  q: [R][n_beams][H][head_dim].
 *   beam_node: [R][n_beams] int32 arena node of each beam, or NULL for
 *   prompt-only beams (trie may then be NULL).  out: [R][n_beams][H*head_dim]
 *   fp32.  ws / ws_bytes: scratch, gr_attn_workspace_size() bytes (currently
 *   0; NULL is accepted then).
 *   Host errors: NULL pointers, sizes <= 0, unsupported dtype/head_dim,
 *   max_depth outside [1, GR_MAX_DEPTH].  Device errors: PARENT_RANGE,
 *   PARENT_ORDER, DEPTH while walking a chain. */
gr_status gr_prefix_attn(const gr_shape *shape, const void *prompt_k,
                         const void *prompt_v, const void *q, int32_t n_beams,
                         const gr_trie *trie, const int32_t *beam_node,
                         float *out, void *ws, size_t ws_bytes,
                         int32_t *dev_err, hipStream_t stream);

/* gr_beam_topk -- candidate scores and exact top-k (ASGR 4.2).
 *   c[r][b][t] = prior[r][b] + (flags & GR_TOPK_LOG_SOFTMAX
 *                               ? logits[r][b][t] - logsumexp_t logits[r][b]
 *                               : logits[r][b][t])
 *   Per request, the k candidates with the largest c, ordered by c
 *   descending and then by the flat index f = b*vocab + t ascending:
 *     out_score[r][j] = c,  out_token[r][j] = f mod vocab,
 *     out_parent[r][j] = f div vocab (index into the input beams).
 *   logits: [R][n_in][vocab] fp32.  prior: [R][n_in] fp32 or NULL (= 0).
 *   cand_out: optional [R][n_in][vocab] fp32 copy of c.  ws: at least
 *   gr_topk_workspace_size(R, n_in, vocab, k) bytes.
 *   Host errors: NULL pointers, sizes <= 0, vocab not 1 or 256, unknown
 *   flags, k > n_in*vocab or k > GR_MAX_K, workspace too small. */
gr_status gr_beam_topk(int32_t R, int32_t n_in, int32_t vocab, int32_t k,
                       int32_t flags, const float *logits, const float *prior,
                       float *out_score, int32_t *out_token,
                       int32_t *out_parent, float *cand_out, void *ws,
                       size_t ws_bytes, hipStream_t stream);

/* gr_decode_step -- the whole step: gr_prefix_attn, then the codebook
 * projection of the current level z[r][b][t] = sum_i o[r][b][i] W[t][i]
 * (only the vocab = 256 valid codes, ASGR 4.2), then gr_beam_topk's scoring
 * and selection with k = beam_width.  flags: GR_TOPK_LOG_SOFTMAX, plus the
 * optional stage bits GR_STEP_ATTENTION / GR_STEP_SELECTION.
 *   W: [vocab][H*head_dim] dtype (row t = code t's projection vector).
 *   Layout note: this default is the TRANSPOSE of the D x 256 projection
 *   matrix as the pages write it (Engineering Exploration of Generative
 *   Recall, 4.2), i.e. of a [H*head_dim][vocab] array: code t's D weights
 *   are contiguous, which makes each code one contiguous MFMA operand row.
 *   A caller holding the [H*head_dim][vocab] array passes it as is with
 *   flags | GR_W_DIM_MAJOR; passing it without that flag computes the
 *   logits of the transposed matrix (wrong codes, no error).
 *   vocab = 1 is scalar scoring (TransRetrieval): score = o . W[0] (+ prior),
 *   flags must be 0 (GR_W_DIM_MAJOR aside).
 *   Precision: for bf16 with vocab = 256 and a prompt window Lw of at least
 *   64 keys and at least H*head_dim / 8 keys, o enters the projection (a
 *   bf16 MFMA) rounded to bf16, which moves a logit by about
 *   2^-9 rms(W) |o|: negligible when o averages many keys.  Shorter windows,
 *   where a few keys can dominate o (|o| grows like sqrt(H*head_dim / Lw)),
 *   use fp32 o and an fp32 projection instead (slower, same results up to
 *   fp32 rounding).
 *   attn_out: optional [R][n_beams][H*head_dim] fp32 copy of the attention
 *   output; cand_out: optional [R][n_beams][vocab] fp32 copy of c.
 *   ws: at least gr_decode_workspace_size(shape, n_beams, vocab, beam_width)
 *   bytes.  Errors: those of gr_prefix_attn and gr_beam_topk. */
gr_status gr_decode_step(const gr_shape *shape, const void *prompt_k,
                         const void *prompt_v, const void *q, int32_t n_beams,
                         const gr_trie *trie, const int32_t *beam_node,
                         const void *W, int32_t vocab, const float *prior,
                         int32_t beam_width, int32_t flags, float *out_score,
                         int32_t *out_token, int32_t *out_parent,
                         float *attn_out, float *cand_out, void *ws,
                         size_t ws_bytes, int32_t *dev_err,
                         hipStream_t stream);

/* gr_linear_state -- the shared prompt-derived state of linear-attention
 * decoding (OneLA, Abstract: one state derived from the shared prompt serves
 * every beam).  For every request r and head h, over the prompt window rows
 * j in [prompt_len - Lw, prompt_len):
 *   state[r][h][a][c] = sum_j phi(k_j[h][a]) * v_j[h][c]
 *   norm[r][h][a]     = sum_j phi(k_j[h][a])
 * with the feature map phi(x) = elu(x) + 1 (x + 1 for x > 0, e^x otherwise).
 *   prompt_k, prompt_v: [R][prompt_len][H][head_dim] dtype.  state:
 *   [R][H][head_dim][head_dim] fp32, norm: [R][H][head_dim] fp32.  bf16:
 *   the contraction runs on bf16 MFMA with fp32 accumulation, phi(k) split
 *   into two bf16 terms (about 16 mantissa bits); norm sums phi(k) in fp32;
 *   fp32: all fp32.
 *   Host errors: NULL pointers, sizes <= 0, unsupported dtype/head_dim,
 *   unaligned pointers. */
gr_status gr_linear_state(const gr_shape *shape, const void *prompt_k,
                          const void *prompt_v, float *state, float *norm,
                          hipStream_t stream);

/* gr_linear_attn -- linear attention of every beam over the shared prompt
 * state plus its own chain of records (OneLA, Abstract: each beam is the
 * shared state plus compact append-only records of its own transitions; only
 * the state information a step needs is computed, no per-beam state):
 *   num = phi(q)^T state[r][h] + sum_{n in chain} (phi(q).phi(k_n)) v_n
 *   den = phi(q) . norm[r][h]  + sum_{n in chain}  phi(q).phi(k_n)
 *   out[r][b][h*head_dim + i] = num[i] / den          (fp32 arithmetic)
 *   state, norm: gr_linear_state's outputs.  q, trie, beam_node, out and
 *   the device errors: as gr_prefix_attn (shape->scale is not used).
 *   Host errors: NULL pointers, sizes <= 0, unsupported dtype/head_dim,
 *   unaligned pointers, max_depth outside [1, GR_MAX_DEPTH]. */
gr_status gr_linear_attn(const gr_shape *shape, const float *state,
                         const float *norm, const void *q, int32_t n_beams,
                         const gr_trie *trie, const int32_t *beam_node,
                         float *out, int32_t *dev_err, hipStream_t stream);

/* gr_linear_decode_step -- gr_decode_step with gr_linear_attn in place of
 * the softmax attention: the same codebook projection, log-softmax, prior
 * add and exact top-k on the linear-attention output, the same arguments
 * (state and norm replace the prompt K/V), flags, outputs and errors.
 *   ws: at least gr_decode_workspace_size(shape, n_beams, vocab, beam_width)
 *   bytes. */
gr_status gr_linear_decode_step(const gr_shape *shape, const float *state,
                                const float *norm, const void *q,
                                int32_t n_beams, const gr_trie *trie,
                                const int32_t *beam_node, const void *W,
                                int32_t vocab, const float *prior,
                                int32_t beam_width, int32_t flags,
                                float *out_score, int32_t *out_token,
                                int32_t *out_parent, float *attn_out,
                                float *cand_out, void *ws, size_t ws_bytes,
                                int32_t *dev_err, hipStream_t stream);

/* gr_code_table -- query, key and value of every code of each level
 * (Engineering Exploration of Generative Recall, 4.1: attention starts from
 * the per-token query, key and value; 4.2: each level has its own 256
 * codes).  A code chosen at one step enters the next as a token whose
 * embedding is projected by the model's query, key and value projections; as
 * that depends only on (level, code), the vocab rows of each level are
 * projected once:
 *   table[l][t][c] = sum_i emb[l][t][i] * w_qkv[c][i],  c < 3*D, D = H*head_dim,
 * so that table[l][t] = [q | k | v] of code t of level l, each [H][head_dim].
 *   emb: [levels][vocab][d_emb] dtype.  w_qkv: [3*D][d_emb] dtype (the D
 *   query projection rows, then the key rows, then the value rows).  table:
 *   [levels][vocab][3][H][head_dim] dtype (fp32 accumulation, one rounding to
 *   the storage dtype, round to nearest even for bf16).  Only shape->H,
 *   head_dim and dtype are used.
 *   Host errors: NULL pointers, levels <= 0 (SHAPE) or above GR_MAX_DEPTH + 1,
 *   vocab != 256, d_emb not a positive multiple of 16 or above 16384,
 *   unsupported dtype/head_dim, unaligned pointers. */
gr_status gr_code_table(const gr_shape *shape, int32_t levels, int32_t vocab,
                        int32_t d_emb, const void *emb, const void *w_qkv,
                        void *table, hipStream_t stream);

/* gr_append_codes -- gr_trie_append for beams that just chose a code (OneLA,
 * Abstract: one append-only record per surviving beam).  For every request r
 * and j < n_new, with t = token[r][j] and node n = base + j:
 *     trie.k[r][n] = table[t][1],  trie.v[r][n] = table[t][2],
 *     q_out[r][j] = table[t][0]    (q_out optional, may be NULL),
 *     trie.parent[r][n], node_out[r][j]: as gr_trie_append.
 *   table: [vocab][3][H][head_dim] dtype (gr_code_table).  token: [R][n_new]
 *   int32 (a step's out_token).  parent_beam / prev_nodes / n_prev: as
 *   gr_trie_append (a step's out_parent and the nodes of its input beams).
 *   q_out: [R][n_new][H][head_dim] dtype, the next step's queries.
 *   Host errors: those of gr_trie_append, plus NULL table/token and
 *   vocab != 256.  Device errors: those of gr_trie_append, and TOKEN_RANGE for
 *   a code outside [0, vocab) (code 0 is used in its place). */
gr_status gr_append_codes(const gr_shape *shape, const gr_trie *trie,
                          int32_t base, int32_t n_new, const void *table,
                          int32_t vocab, const int32_t *token,
                          const int32_t *parent_beam,
                          const int32_t *prev_nodes, int32_t n_prev,
                          void *q_out, int32_t *node_out, int32_t *dev_err,
                          hipStream_t stream);

/* gr_generate -- a whole semantic ID: `levels` decode steps, each followed
 * (but the last) by gr_append_codes of its chosen codes, then the trace-back
 * of the final beams' code sequences; all enqueued on `stream` with no host
 * synchronisation, so the whole call can be captured in one HIP graph
 * (TransRetrieval, GPU retrieval: the iterations of the search stay on the
 * device; Engineering Exploration of Generative Recall, 4.2: level l is
 * scored over its own 256 codes with W_l).
 *   Step 0 has one root hypothesis per request (query q0, prior 0, no
 *   records); step l keeps k_l = min(beam_width, n_l * vocab) beams, with
 *   n_0 = 1 and n_{l+1} = k_l.  Step l+1's beams are step l's output slots:
 *   their queries and records come from tables[l] at their chosen codes, and
 *   their priors are step l's scores.
 *   q0: [R][1][H][head_dim] dtype.  W: [levels][vocab][H*head_dim] dtype.
 *   tables: [levels-1][vocab][3][H][head_dim] dtype (gr_code_table per
 *   level; NULL when levels == 1).  trie: arena for the appended records,
 *   capacity >= k_0 + ... + k_{levels-2} and max_depth >= levels - 1 (NULL
 *   when levels == 1); nodes [0, k_0) hold level-1 records, the next k_1
 *   level-2 records, and so on.  Their parent links are always written; in
 *   bf16 with capacity <= 4096 the attention reads each record's key and
 *   value straight from its row of `tables`, and the arena's k and v are
 *   left unwritten (otherwise they receive the records' rows).
 *   out_score / out_token / out_parent: per-step results packed step after
 *   step; step l's block is [R][k_l] and starts at element
 *   R * (k_0 + ... + k_{l-1}) (for beam_width <= 256 simply
 *   [levels][R][beam_width]).  out_parent indexes the step's input beams.
 *   out_ids: [R][k_{levels-1}][levels] int32, the code of every level of
 *   each final beam.  ws: gr_generate_workspace_size() bytes.
 *   Host errors: those of gr_decode_step and gr_append_codes, vocab != 256,
 *   levels outside [1, GR_MAX_DEPTH + 1], capacity or max_depth too small
 *   (CAPACITY / UNSUPPORTED).  Device errors: those of both, OR-ed into
 *   *dev_err; the outputs are undefined when it is nonzero.  GR_ERR_HIP can
 *   leave earlier levels enqueued. */
gr_status gr_generate(const gr_shape *shape, const void *prompt_k,
                      const void *prompt_v, const void *q0, int32_t levels,
                      const void *W, const void *tables, int32_t vocab,
                      int32_t beam_width, const gr_trie *trie,
                      float *out_score, int32_t *out_token,
                      int32_t *out_parent, int32_t *out_ids, void *ws,
                      size_t ws_bytes, int32_t *dev_err, hipStream_t stream);

/* gr_broadcast_score -- multi-layer broadcast scoring of single-token
 * candidates (TransRetrieval: Architecture Overview, stage 4: an N-layer
 * Pre-LN Transformer with a ReLU FFN whose user-side keys and values are
 * computed once per request and reused by every candidate; the
 * per-candidate cost paragraph: each candidate has its own Q/K/V/output
 * projections and FFN and attends to the whole user sequence;
 * Hardware-aware inference optimization: the user cache is broadcast to all
 * candidates without copies, single-token candidates are packed into batched
 * products; GPU retrieval: the selection stays on the device).
 *   Per request r: the user tokens user_tok[r] (L_u of them) pass through
 *   the layers attending to one another; at each layer l their keys and
 *   values K_l, V_l are kept.  Each candidate token cand_tok[r][i] passes
 *   through the same layers attending to K_l, V_l and to its own key and
 *   value only.  A layer is x += MHA(LN1(x)) W_o^T + b_o;
 *   x += ReLU(LN2(x) W_1^T + b_1) W_2^T + b_2, with [q|k|v] = LN1(x)
 *   w_qkv^T + b_qkv, heads of 32, scores scaled by 1/sqrt(32), LayerNorm
 *   over the D features (biased variance, eps 1e-5, gain and bias).  The
 *   score is s_i = LN_f(x_i) . w_score + b_score after the last layer, and
 *   the call returns the k best of each request by (score desc, index asc).
 *   The FFN width 2D follows the page's per-layer cost of 16 D^2 FLOPs per
 *   candidate for the four D x D projections (8 D^2) and the FFN.
 *   shape: R requests, n_cand candidates and user_len user tokens each
 *   (user_len a multiple of 32, <= GR_XF_MAX_USER), d_model = 128,
 *   n_layers <= GR_XF_MAX_LAYERS.
 *   user_tok: [R][user_len][d_model] bf16.  cand_tok: [R][n_cand][d_model]
 *   bf16.  w_mat: bf16, per layer (8 d_model^2 values, layer after layer):
 *   w_qkv [3D][D] (rows: query, key, value output features; weights are
 *   [out][in]), w_o [D][D], w_1 [2D][D], w_2 [D][2D].  w_vec: fp32, per
 *   layer (11 D values): b_qkv [3D], b_o [D], b_1 [2D], b_2 [D], ln1_gain,
 *   ln1_bias, ln2_gain, ln2_bias [D]; then lnf_gain, lnf_bias, w_score [D]
 *   and b_score [1].
 *   out_score [R][k] fp32, out_index [R][k] int32 (candidate index).
 *   cand_scores: optional [R][n_cand] fp32, every candidate's score.
 *   Products run in bf16 with fp32 accumulation (activations rounded to
 *   bf16 where they enter a product), LayerNorm, softmax and the residual
 *   stream in fp32; the selection is exact on those fp32 scores.
 *   ws: gr_broadcast_workspace_size() bytes (caller-owned; holds the user
 *   keys/values of every layer, broadcast in place to all candidates).
 *   Host errors: NULL pointers (NULL), sizes <= 0 (SHAPE), d_model != 128,
 *   user_len not a multiple of 32 or too long, too many layers, unaligned
 *   pointers (UNSUPPORTED), k > n_cand or above GR_MAX_K (K_TOO_LARGE), a
 *   small workspace (WORKSPACE).  No device errors. */
#define GR_XF_MAX_USER 1024
#define GR_XF_MAX_LAYERS 8
typedef struct {
  int32_t R, n_cand, user_len, d_model, n_layers;
} gr_xf_shape;
gr_status gr_broadcast_score(const gr_xf_shape *shape, const void *user_tok,
                             const void *cand_tok, const void *w_mat,
                             const float *w_vec, int32_t k, float *out_score,
                             int32_t *out_index, float *cand_scores, void *ws,
                             size_t ws_bytes, hipStream_t stream);
size_t gr_broadcast_workspace_size(const gr_xf_shape *shape, int32_t k);

/* gr_decode_step_noalloc -- gr_decode_step for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, hosts
 * that forbid hipMalloc.  Same arguments, semantics, outputs and errors as
 * gr_decode_step, without ws / ws_bytes: the step's scratch is a static
 * device array of GR_NOALLOC_SCRATCH_BYTES (48 MiB) that every GPU the
 * library runs on holds from the library's first use on it until the
 * process ends.  Its device address is looked up once per device
 * (hipGetSymbolAddress, on the current device); the call allocates and
 * frees nothing.
 *   Limit: a step whose gr_decode_workspace_size() exceeds
 *   GR_NOALLOC_SCRATCH_BYTES returns GR_ERR_SCRATCH_LIMIT before any device
 *   call (the 256-request, beam-100, 600-token step needs 26 MiB).
 *   Sharing: every call on one GPU uses that GPU's one array, which keeps
 *   the last call's contents; no part of it needs to start at zero.  Calls
 *   that overlap on one GPU (other streams, other threads) race on it and
 *   must be serialised by the caller. */
#define GR_NOALLOC_SCRATCH_BYTES (48u << 20)
gr_status gr_decode_step_noalloc(const gr_shape *shape, const void *prompt_k,
                                 const void *prompt_v, const void *q,
                                 int32_t n_beams, const gr_trie *trie,
                                 const int32_t *beam_node, const void *W,
                                 int32_t vocab, const float *prior,
                                 int32_t beam_width, int32_t flags,
                                 float *out_score, int32_t *out_token,
                                 int32_t *out_parent, float *attn_out,
                                 float *cand_out, int32_t *dev_err,
                                 hipStream_t stream);

/* Scratch sizes in bytes (0 when none is needed; sizes <= 0 give 0).
 * gr_workspace_size(shape, n_beams, vocab, k) is the scratch that is enough
 * for every call of the step on these sizes: gr_prefix_attn(shape, n_beams),
 * gr_beam_topk(shape->R, n_beams, vocab, k) and gr_decode_step(shape,
 * n_beams, vocab, k) (equal to gr_decode_workspace_size, which covers the
 * other two).  The per-call sizes below may be smaller. */
size_t gr_workspace_size(const gr_shape *shape, int32_t n_beams,
                         int32_t vocab, int32_t k);
size_t gr_attn_workspace_size(const gr_shape *shape, int32_t n_beams);
size_t gr_topk_workspace_size(int32_t R, int32_t n_in, int32_t vocab,
                              int32_t k);
size_t gr_decode_workspace_size(const gr_shape *shape, int32_t n_beams,
                                int32_t vocab, int32_t k);
size_t gr_generate_workspace_size(const gr_shape *shape, int32_t levels,
                                  int32_t vocab, int32_t beam_width);

/* Human-readable name of a status code (static string, never NULL). */
const char *gr_status_string(gr_status status);

#ifdef __cplusplus
}
#endif
#endif /* GR_BEAM_H */
