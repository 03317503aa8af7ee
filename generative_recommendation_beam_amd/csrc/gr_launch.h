// Host-side launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gr_beam.h"

namespace gr {

// Attention of every beam over the shared prompt window plus its own chain.
struct AttnArgs {
  int dtype;                       // GR_BF16 or GR_F32
  const void *pk, *pv, *q;         // [R][Lp][H][hd], [R][Lp][H][hd], [R][nb][H][hd]
  const void *ak, *av;             // arena [R][cap][H][hd] (may be null if no chains)
  const int32_t *parent;           // [R][cap]
  const int32_t *beam_node;        // [R][nb] or null (prompt only)
  int32_t *chain_ids;              // bf16 path: workspace for the resolved chains, attn_ids_bytes(R, nb)
  float *split_ws;                 // bf16 path with a split prompt: partial states, attn_split_bytes(...)
  float *out_f32;                  // optional [R][nb][H*hd]
  void *out_lowp;                  // optional head-major [R][H][nb][hd] in dtype (bf16 feed of the logits)
  int32_t *dev_err;
  int R, H, hd, Lp, Lw, nb, cap, max_depth;
  float scale;
  // Records and queries read from code tables instead of the arena and q
  // (whole-ID generation, bf16, arenas of at most kLdsChainNodes nodes): node
  // n's key and value, and the query of a beam at node n, are row
  // rec_row[r][n] of rec_tab ([rec_tab_rows][3][H][hd]: q, k, v), for the
  // nodes n < rec_rows <= cap that chains reach.  Null: the arena and q.
  const void *rec_tab = nullptr;
  const int32_t *rec_row = nullptr;   // [R][rec_rows]
  int rec_rows = 0, rec_tab_rows = 0;
};
hipError_t launch_attn(const AttnArgs &a, hipStream_t s);

// Arenas up to this many nodes per request have their parent array staged in
// LDS and the chains resolved inside the bf16 attention kernel; larger ones go
// through the chain-resolve pre-pass (and cannot read records from tables).
constexpr int kLdsChainNodes = 4096;

// bf16 attention geometry: a workgroup holds NW waves of 32 beams; the chain
// ids of a request are stored level-major, [max_depth][beams padded to whole
// workgroups].
inline int attn_waves(int nb) {
  const int nblk = (nb + 31) / 32;
  return nblk <= 1 ? 1 : (nblk == 2 ? 2 : 4);
}
inline int attn_beam_pad(int nb) {
  const int per = attn_waves(nb) * 32;
  return (nb + per - 1) / per * per;
}
inline size_t attn_ids_bytes(int R, int nb) {
  return (size_t)R * GR_MAX_DEPTH * attn_beam_pad(nb) * sizeof(int32_t);
}

// Split of the prompt window (bf16 path).  With too few (request, head, beam
// group) units to fill the GPU, each unit's window is cut into n_split runs
// of tiles_per_split 64-key tiles, one workgroup each; every workgroup leaves
// its partial online-softmax state (unnormalised o, running max, sum) in the
// workspace and a merge pass combines them with their log-sum-exp weights.
// The chain records go with the last run.
constexpr int kAttnSplitBelow = 384;   // units below which the window is split
constexpr int kAttnSplitTarget = 384;  // workgroups aimed at (measured: 6 to 12 runs of an 8192-key
                                       // window, 4 requests x 8 heads, all within 3 %; 16 or more
                                       // runs are slower, the partial states growing with them)
constexpr int kAttnSplitMinTiles = 4;  // tiles (256 keys) per run at least
struct AttnSplit {
  int n_split, tiles_per_split;
};
inline AttnSplit attn_split(int R, int H, int nb, int Lw) {
  const long long units = (long long)R * H * (attn_beam_pad(nb) / (attn_waves(nb) * 32));
  const int n_tiles = (Lw + 63) / 64;
  AttnSplit sp = {1, n_tiles};
  if (units >= kAttnSplitBelow) return sp;
  const long long want = (kAttnSplitTarget + units - 1) / units;
  const int most = n_tiles / kAttnSplitMinTiles;
  const int ns = (int)(want < most ? want : most);
  if (ns < 2) return sp;
  sp.tiles_per_split = (n_tiles + ns - 1) / ns;
  sp.n_split = (n_tiles + sp.tiles_per_split - 1) / sp.tiles_per_split;
  return sp;
}
// partial states: o [R][H][n_split][nb_pad][hd] fp32, then (max, sum) [R][H][n_split][nb_pad][2]
inline size_t attn_split_bytes(int R, int H, int hd, int nb, int Lw) {
  const AttnSplit sp = attn_split(R, H, nb, Lw);
  if (sp.n_split == 1) return 0;
  return (size_t)R * H * sp.n_split * attn_beam_pad(nb) * (hd + 2) * sizeof(float);
}

struct AppendArgs {
  int elem_bytes;
  void *ak, *av;
  int32_t *parent;
  const void *k_new, *v_new;
  const int32_t *parent_beam, *prev_nodes;
  int32_t *node_out, *dev_err;
  int R, H, hd, cap, base, n_new, n_prev;
};
hipError_t launch_trie_append(const AppendArgs &a, hipStream_t s);

// Linear-attention decoding (linear.hip).
struct LinearStateArgs {
  int dtype;
  const void *pk, *pv;
  float *S, *z;                // [R][H][hd][hd], [R][H][hd]
  int R, H, hd, Lp, Lw;
};
hipError_t launch_linear_state(const LinearStateArgs &a, hipStream_t s);

struct LinearAttnArgs {
  int dtype;
  const float *S, *z;
  const void *q, *ak, *av;
  const int32_t *parent, *beam_node;
  int32_t *dev_err;
  float *out_f32;              // [R][nb][H*hd] or NULL
  void *out_lowp;              // bf16 head-major [R][H][nb][hd] or NULL
  int R, H, hd, nb, cap, max_depth;
};
hipError_t launch_linear_attn(const LinearAttnArgs &a, hipStream_t s);

// Whole-ID generation (generate.hip).  Levels of one generation call.
constexpr int kMaxLevels = GR_MAX_DEPTH + 1;

struct CodeTableArgs {
  int dtype;
  const void *emb, *w_qkv;     // [levels][V][De], [3D][De]
  void *table;                 // [levels][V][3D]
  int levels, V, D, De;
};
hipError_t launch_code_table(const CodeTableArgs &a, hipStream_t s);

struct AppendCodesArgs {
  int elem_bytes;
  void *ak, *av, *q_out;
  int32_t *parent;
  const void *table;
  const int32_t *token, *parent_beam, *prev_nodes;
  int32_t *node_out, *dev_err;
  int R, H, hd, cap, base, n_new, n_prev, V;
  // Records left in the code tables: node n's table row (row0 + its code) is
  // written to rec_row[r][n] ([R][row_n], n < row_n) and ak / av are not
  // touched (q_out may then be null too).  Null: the rows are copied into the
  // arena.
  int32_t *rec_row = nullptr;
  int row_n = 0, row0 = 0;
};
hipError_t launch_append_codes(const AppendCodesArgs &a, hipStream_t s);

struct TraceArgs {
  const int32_t *token, *parent;   // per-level blocks [R][k[l]] at offset off[l]
  int32_t *ids, *dev_err;          // ids [R][k[levels-1]][levels]
  long long off[kMaxLevels];
  int k[kMaxLevels];
  int R, levels;
};
hipError_t launch_trace_ids(const TraceArgs &a, hipStream_t s);

// Multi-layer broadcast scoring (xf.hip): D = 128, 4 heads of 32, FFN 2D.
struct XfArgs {
  const void *user, *cand;     // [R][Lu][D], [R][N][D] bf16
  const void *w_mat;           // [L][8 D^2] bf16: w_qkv [3D][D], w_o [D][D], w_1 [2D][D], w_2 [D][2D]
  const float *w_vec;          // [L][11 D] fp32 (b_qkv, b_o, b_1, b_2, ln1 g/b, ln2 g/b), then lnf g/b, w_score, b_score
  void *ukv;                   // workspace: the user keys/values of every layer, xf_ukv_bytes
  void *user_state;            // workspace: the user tokens' x and queries between layers, xf_user_state_bytes
  float *score;                // [R][N]
  int R, N, Lu, L;
};
size_t xf_ukv_bytes(int R, int L, int Lu);
size_t xf_user_state_bytes(int R, int Lu);
hipError_t launch_xf_scores(const XfArgs &a, hipStream_t s);

// Selection outputs / partial lists shared by the scoring kernels.
struct SelectOut {
  float *score;
  int32_t *token, *parent;
  uint64_t *partial;               // [R][n_groups][kk] when n_groups > 1
  int n_groups, kk;
  int gpos;                        // candidates per group: kGroupPositions, or kGroupPositions / 2 (MFMA scoring) or kSmallGroupPositions (score_select) when groups that size leave CUs idle
};

// Codebook projection on MFMA (bf16 o, bf16 W [256][D]), log-softmax, prior,
// selection of each group of <= 128 beams.
struct LogitsArgs {
  const uint16_t *o;               // head-major [R][H][n_in][hd] bf16, D = H * hd
  const uint16_t *W;               // [256][D] bf16
  const float *prior;              // [R][n_in] or null
  float *cand_out;                 // optional [R][n_in][256]
  int R, n_in, D, hd, k, log_softmax;
};
hipError_t launch_logits_select_bf16(const LogitsArgs &a, const SelectOut &o, hipStream_t s);

// Scores from fp32 logits in global memory ([R][n_in][vocab]), then selection.
struct ScoreSelectArgs {
  const float *logits;
  const float *prior;              // [R][n_in] or null
  float *cand_out;                 // optional
  int R, n_in, vocab, k, log_softmax;
};
hipError_t launch_score_select(const ScoreSelectArgs &a, const SelectOut &o, hipStream_t s);

// out[c][r] = in[r][c] for an in of rows x cols elements of elem_bytes (2 or 4).
hipError_t launch_transpose(const void *in, void *out, int rows, int cols, int elem_bytes, hipStream_t s);

// Final merge of per-group partial lists.
hipError_t launch_select_merge(const SelectOut &o, int R, int k, int vocab, hipStream_t s);

// fp32 projections: z = o . W^T ([R][n][vocab]); scalar path uses vocab = 1.
struct ProjArgs {
  int dtype;                       // dtype of o and W
  const void *o, *W;               // o [R][n][D], W [vocab][D]
  const float *prior;              // added when add_prior (scalar path)
  float *z;                        // [R][n][vocab]
  int R, n, D, vocab, add_prior;
};
hipError_t launch_project(const ProjArgs &a, hipStream_t s);

// Group geometry shared by host sizing and the kernels.
constexpr int kGroupBeams = 128;          // beams per selection group at vocab 256
constexpr int kGroupPositions = 32768;    // candidates per selection group
constexpr int kSmallGroupPositions = 8192;   // score_select groups when few requests leave CUs idle
constexpr int kSelectCUs = 256;           // workgroups below which score_select splits finer
constexpr int kMergeCapacity = 16384;     // partial entries the final merge holds
inline int select_groups(int n_in, int vocab, int gpos = kGroupPositions) {
  const long long n = (long long)n_in * vocab;
  return (int)((n + gpos - 1) / gpos);
}

}  // namespace gr
