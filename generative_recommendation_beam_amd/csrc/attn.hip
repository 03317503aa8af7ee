// Attention of every beam over the shared prompt plus its own ancestor chain.
//
// Per request r, beam b, head h (Engineering Exploration of Generative Recall,
// 4.1 Superman Optimizer: QK^T, scale, softmax, weighted sum; 4.4 Tree-Based
// Attention: a beam sees only its own branch; 4.5 Sliding-Window Attention;
// TransRetrieval, Hardware-aware inference optimization: one user cache for
// all candidates; OneLA, Abstract: shared prompt + append-only records + an
// ancestry index):
//   keys = prompt rows [Lp-Lw, Lp) then the records on chain(beam_node[b]),
//   o[b][h*hd+i] = sum_j softmax_j(scale * q.k_j) v_j[i].
//
// bf16 path (gfx950 MFMA).
//
// attn_bf16: one workgroup per (request, head, group of NW x 32 beams).
// Everything the workgroup reads goes HBM -> LDS with global_load_lds through
// one NS-stage ring of 64-row tiles, NS-1 tiles in flight, in this order: the
// request's parent ids and the workgroup's beam nodes, the queries, the prompt
// window (read from HBM once per (request, head), never copied per beam), then
// the chain records gathered row by row (128-beam workgroups: per chain
// level a tile of the key rows of all beams, then one of their value rows).
// Vector loads complete in issue order, so keeping every load on this one
// in-order stream makes each wait exact and keeps the ring full while the
// chains are processed.  At the first tile each beam's chain is resolved in
// LDS (parent links from the beam's own record to the root, with range, order
// and depth checks) into level-major node ids: the ancestry index of the step.
// The attention output leaves through LDS so that stores write whole lines.
//
// chain_resolve: the same chain walk, one thread per beam in global memory,
// for arenas too large to stage in LDS; its ids reach the attention kernel
// through the workspace.
//
// With too few (request, head, beam group) units to fill the GPU (few
// requests with long prompts), the window is cut into runs of tiles, one
// workgroup per run; each leaves its partial online-softmax state in the
// workspace (the chain records go with the last run) and attn_merge combines
// the runs with their log-sum-exp weights.
//
// Scores are formed transposed, S^T = K Q^T (keys x beams), with
// v_mfma_f32_32x32x16_bf16: the accumulator holds one beam per lane column,
// so the softmax reductions are in-lane plus one lane^32 swap, and the
// probabilities are already the B operand of O^T += V^T P^T.  The V^T operand
// comes from the row-major V tile through ds_read_b64_tr_b16.  Each lane
// fetches its 16 bytes from an XOR-permuted source address, so LDS rows come
// out bank-swizzled for both the K reads and the transposed V reads.  Chain
// records (one distinct key per beam) are folded into the same online-softmax
// state on the VALU.
//
// fp32 path: plain VALU kernel, one thread per beam, same semantics.

#include "gr_device.h"
#include "gr_launch.h"

namespace gr {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
// Ring depth of the bf16 kernel: 3 stages of 64 keys (2 tiles in flight)
// keep a 4-wave workgroup at 52 KB of LDS and <= 168 VGPRs, so three
// workgroups share a CU.
#ifndef GR_ATTN_STAGES
#define GR_ATTN_STAGES 3
#endif
constexpr int kAttnStages = GR_ATTN_STAGES;

typedef __attribute__((ext_vector_type(4))) short i16x4;

template <int I>
struct Stage {
  static constexpr int value = I;
};
#define GR_LDS4(p) ((__attribute__((address_space(3))) i16x4 *)(p))
// Every lambda of the attention kernel is inlined: a call would put the
// by-reference captures (offset tables, the queries) in scratch memory.
#define GR_INLINE __attribute__((always_inline))

// ------------------------------------------------------------ chain resolve
struct ChainP {
  const int32_t *parent, *beam_node;
  int32_t *ids;        // [R][D][nb_pad]
  int32_t *dev_err;
  int R, nb, nb_pad, cap, D;
};

__global__ __launch_bounds__(256) void chain_resolve_kernel(ChainP p) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)p.R * p.nb_pad) return;
  const int r = (int)(i / p.nb_pad), b = (int)(i % p.nb_pad);
  const int32_t *par = p.parent + (size_t)r * p.cap;
  int32_t *out = p.ids + (size_t)r * p.D * p.nb_pad + b;
  int n = b < p.nb ? p.beam_node[(size_t)r * p.nb + b] : -1;
  int err = 0;
  for (int d = 0; d < p.D; ++d) {
    int id = -1;
    if (n != -1) {
      if (n < 0 || n >= p.cap) {
        err |= GR_DEVERR_PARENT_RANGE;
        n = -1;
      } else {
        id = n;
        const int pn = par[n];
        if (pn < -1 || pn >= p.cap) { err |= GR_DEVERR_PARENT_RANGE; n = -1; }
        else if (pn >= n) { err |= GR_DEVERR_PARENT_ORDER; n = -1; }
        else n = pn;
      }
    }
    out[(size_t)d * p.nb_pad] = id;
  }
  if (n != -1) err |= GR_DEVERR_DEPTH;   // longer than max_depth
  if (err) atomicOr(p.dev_err, err);
}

// ------------------------------------------------------------ bf16 attention
struct AttnP {
  const uint16_t *pk, *pv, *q, *ak, *av;
  const int32_t *ids;                  // chains resolved by chain_resolve ([R][D][nb_pad]), or null
  const int32_t *parent, *beam_node;   // chains resolved in the kernel (small arenas), or null
  int32_t *dev_err;
  float *out_f32;
  uint16_t *out_bf16;
  int R, H, Lp, Lw, nb, cap, D, nb_pad, n_grp;
  int n_split, tps;          // prompt runs per unit and 64-key tiles per run
  float *part;               // n_split > 1: partial states (see attn_split_bytes)
  int ids_words, par_words;  // dynamic LDS: ids [ids_words], parents [par_words], beam nodes, table rows
  float sl2;                 // scale * log2(e)
  const uint16_t *rtab;      // records from code tables: [rows][3][H][HD] (q, k, v), or null
  const int32_t *rrow;       // [R][rrow_n]: the table row of each node
  int rrow_n, rtab_rows;
};

template <int HD, int NW, int NS>
struct Geo {
  static constexpr int KT = 64;                 // rows per tile
  static constexpr int RB = HD * 2;             // bytes per tile row
  static constexpr int TB = KT * RB;            // bytes per tile (K or V)
  static constexpr int NBLK = TB / 1024;        // 1 KB DMA blocks per tile
  static constexpr int IPW = NBLK / NW;         // DMA blocks per wave (K or V)
  static constexpr int KSTEP = HD / 16;         // MFMA k-steps over the head dim
  static constexpr int DT = HD / 32;            // 32-row d tiles of O^T
  static constexpr int NB = NW * 32;            // beams per workgroup
  static constexpr int NRB = (NB + KT - 1) / KT;  // record tiles per chain level
};

// Bank swizzles (physical chunk = logical chunk ^ swizzle(row)).  K: 16
// consecutive lanes read 16 consecutive rows at one logical chunk; the
// swizzle spreads them over distinct 16-byte slots of a 256-byte bank row
// (and any 8 of them over a 128-byte one).  V: a 16-lane transposed read
// touches 4 consecutive rows (from a multiple of 4) x 2 adjacent chunks.
template <int HD>
__device__ __forceinline__ int swz_k(int row) {
  return HD == 64 ? ((row & 7) ^ ((row >> 3) & 1)) : (((row >> 1) & 3) ^ ((row >> 3) & 1));
}
template <int HD>
__device__ __forceinline__ int swz_v(int row) {
  return HD == 64 ? 2 * (row & 3) : 2 * ((row >> 1) & 1);
}

// TAB: the chain records and the queries are rows of code tables (p.rtab,
// one row index per node in p.rrow, staged in LDS with the parents; a beam's
// query is the row of its node); else the arena and p.q.
template <int HD, int NW, int NS, int OCC, bool TAB>
__global__ __launch_bounds__(NW * 64, OCC) void attn_bf16_kernel(AttnP p) {
  using G = Geo<HD, NW, NS>;
  static_assert(NS >= 2 && NS <= 4, "ring depth: the last stage carries the queries until it is first refilled");
  static_assert(G::NBLK % NW == 0, "every wave moves the same number of 1 KB blocks");
  static_assert(G::NB <= 2 * G::KT, "queries of a workgroup fit the two buffers of one stage");
  // One LDS object per ring stage (its K half, then its V half): the
  // compiler then sees that a DMA into one stage does not touch the stage
  // being read, and adds no waits for it.  (It tells apart only a few LDS
  // DMA targets, so there are just five: four stages and the chain ids.)
  __shared__ __attribute__((aligned(1024))) uint16_t KV0[G::TB], KV1[G::TB], KV2[NS > 2 ? G::TB : 8],
      KV3[NS > 3 ? G::TB : 8];
  // dynamic LDS: chain ids [D][NB] (level-major; int32 as delivered by the
  // pre-pass, or int16 when the chains are resolved here, the arena then
  // holding at most kLdsChainNodes nodes), then in the second case the
  // request's parent array and the workgroup's beam nodes
  extern __shared__ __attribute__((aligned(1024))) int32_t dyn_s[];
  int32_t *const ids_s = dyn_s;
  int16_t *const ids16 = reinterpret_cast<int16_t *>(dyn_s);
  int32_t *const par_s = dyn_s + p.ids_words;
  int32_t *const bn_s = par_s + p.par_words;
  int32_t *const row_s = bn_s + (G::NB + 63) / 64 * 64;   // TAB: the request's table row per node
  auto chain_id = [&](int d, int b) GR_INLINE -> int {
    return p.parent != nullptr ? (int)ids16[d * G::NB + b] : ids_s[d * G::NB + b];
  };
  auto kst = [&](auto S) GR_INLINE -> uint16_t * {
    constexpr int st = decltype(S)::value;
    if constexpr (st == 0) return KV0;
    else if constexpr (st == 1) return KV1;
    else if constexpr (st == 2) return KV2;
    else return KV3;
  };
  auto vst = [&](auto S) GR_INLINE -> uint16_t * { return kst(S) + G::TB / 2; };
  uint16_t *const K3 = kst(Stage<NS - 1>{}), *const V3 = vst(Stage<NS - 1>{});

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, c = lane & 31;
  // Consecutive workgroup ids go to the 8 XCDs in turn; give each XCD a
  // contiguous range of (request, head) units so that the heads of one
  // request stream their interleaved prompt rows from one L2 at about the
  // same time.
  int bid = blockIdx.x;
  if ((gridDim.x & 7) == 0) bid = (bid & 7) * (int)(gridDim.x >> 3) + (bid >> 3);
  const int split = bid % p.n_split;           // run of the prompt window (0 unless it is split)
  bid /= p.n_split;
  const int grp = bid % p.n_grp;
  bid /= p.n_grp;
  const int h = bid % p.H, r = bid / p.H;
  const int wb = wave * 32 + c;                 // workgroup-local beam of this lane
  const int beam = grp * G::NB + wb;
  const bool valid = beam < p.nb;
  const size_t row = (size_t)p.H * HD;          // elements between tokens
  const uint32_t row32 = (uint32_t)row;
  const uint16_t *pk = p.pk + (size_t)r * p.Lp * row + (size_t)h * HD;
  const uint16_t *pv = p.pv + (size_t)r * p.Lp * row + (size_t)h * HD;
  // this workgroup's run of the window: tiles [split * tps, ...); the chain
  // records go with the last run
  const int k_begin = p.Lp - p.Lw + split * p.tps * G::KT;
  const int n_tiles = (min(p.tps * G::KT, p.Lw - split * p.tps * G::KT) + G::KT - 1) / G::KT;
  const bool chains = (p.ids != nullptr || p.parent != nullptr) && split == p.n_split - 1;
  const int n_pre = max(n_tiles, NS - 1);       // prompt tiles, padded to fill the prologue
  int n_total = n_pre;                          // + chain-record tiles, known after tile 0
  int rec_fill = 0;     // a written record, gathered for the rows of beams without one at a level

  // Per-lane tile row and (swizzled) element offsets of this lane's DMA
  // pieces: wave w moves 1 KB blocks w*IPW..; lane l lands at byte 16*l of its
  // block and fetches the logical chunk the swizzle assigns to that position.
  int dma_row[G::IPW];
  uint32_t dma_k[G::IPW], dma_v[G::IPW];
#pragma unroll
  for (int i = 0; i < G::IPW; ++i) {
    const int byte = (wave * G::IPW + i) * 1024 + 16 * lane;
    const int tr = byte / G::RB, pch = (byte % G::RB) / 16;
    dma_row[i] = tr;
    dma_k[i] = (uint32_t)((pch ^ swz_k<HD>(tr)) * 8);
    dma_v[i] = (uint32_t)((pch ^ swz_v<HD>(tr)) * 8);
  }
  // prompt tile: rows past the window end read the last prompt row (masked
  // or never used)
  auto issue_prompt = [&](int tile, auto S) GR_INLINE {
    const int key0 = k_begin + tile * G::KT;
#pragma unroll
    for (int i = 0; i < G::IPW; ++i) {
      const int blk = wave * G::IPW + i;
      const uint32_t src = (uint32_t)min(key0 + dma_row[i], p.Lp - 1) * row32;
      dma16_stream(pk + (src + dma_k[i]), kst(S) + blk * 512);
      dma16_stream(pv + (src + dma_v[i]), vst(S) + blk * 512);
    }
  };
  // chain-record tiles.  128-beam workgroups: two tiles per chain level,
  // the key rows (bb = 0), then the value rows (bb = 1) of all 128 beams,
  // beams 0..63 in the stage's first half and 64..127 in its second, so that
  // every wave folds every tile.  Smaller workgroups: one tile per level, row
  // t holding beam t's key in the first half and its value in the second (a
  // beam without a record at the level reads record 0 of the request,
  // unused: these fold each beam's own row only).
  // the key (kv = 1) or value (kv = 2) row of record `id` for this head, at
  // element offset sw: in the arena, or the node's row of the code tables
  auto rec_src = [&](int id, int kv, uint32_t sw) GR_INLINE -> const uint16_t * {
    if constexpr (TAB) {
      const uint32_t tr = min((uint32_t)row_s[id], (uint32_t)p.rtab_rows - 1);
      return p.rtab + ((size_t)tr * 3 + kv) * row + (size_t)h * HD + sw;
    }
    else return (kv == 1 ? p.ak : p.av) + ((size_t)r * p.cap + id) * row + (size_t)h * HD + sw;
  };
  auto issue_records = [&](int d, int bb, uint16_t *ks, uint16_t *vs) GR_INLINE {
    if constexpr (G::NRB == 2) {
      // A beam without a record at level d gathers `rec_fill`, a record of
      // the workgroup: the value product multiplies every row of the tile, by 0
      // for such a beam, so every row must be written data.  It is the
      // deepest record of the first beam that has a chain (any written record
      // would do), found when the first level is issued: mid-stream, off the
      // unit's first wait.
      if (d == 0 && bb == 0) {
        const uint64_t m0 = __builtin_amdgcn_ballot_w64(chain_id(0, lane) >= 0);
        const uint64_t m1 = __builtin_amdgcn_ballot_w64(chain_id(0, G::KT + lane) >= 0);
        const int fb = m0 ? (int)__builtin_ctzll(m0) : (m1 ? G::KT + (int)__builtin_ctzll(m1) : 0);
        rec_fill = __builtin_amdgcn_readfirstlane(max(chain_id(0, fb), 0));
      }
#pragma unroll
      for (int i = 0; i < G::IPW; ++i) {
        const int blk = wave * G::IPW + i;
        const uint32_t sw = bb ? dma_v[i] : dma_k[i];
        const int id0 = chain_id(d, dma_row[i]), id1 = chain_id(d, G::KT + dma_row[i]);
        dma16(rec_src(id0 >= 0 ? id0 : rec_fill, 1 + bb, sw), ks + blk * 512);
        dma16(rec_src(id1 >= 0 ? id1 : rec_fill, 1 + bb, sw), vs + blk * 512);
      }
    } else {
#pragma unroll
      for (int i = 0; i < G::IPW; ++i) {
        const int blk = wave * G::IPW + i;
        const int b = bb * G::KT + dma_row[i];
        const int id = b < G::NB ? chain_id(d, b) : -1;
        dma16(rec_src(id >= 0 ? id : 0, 1, dma_k[i]), ks + blk * 512);
        dma16(rec_src(id >= 0 ? id : 0, 2, dma_v[i]), vs + blk * 512);
      }
    }
  };
  auto issue = [&](int tile, auto S) GR_INLINE {
    if (tile < n_pre) {
      issue_prompt(tile, S);
    } else {
      const int k = tile - n_pre;
      issue_records(k / G::NRB, k % G::NRB, kst(S), vst(S));
    }
  };
  // wait until this wave's DMAs of all but the `ahead` most recent tiles landed
  auto wait_tiles = [&](int ahead) GR_INLINE {
    constexpr int per = 2 * G::IPW;
    if (ahead >= 2) GR_WAIT_VMCNT(2 * per);
    else if (ahead == 1) GR_WAIT_VMCNT(per);
    else GR_WAIT_VMCNT(0);
  };

  // TAB: this lane's query pieces are the query part of the table row of
  // each beam's node
  size_t q_tab[TAB ? G::IPW : 1][2];
  if constexpr (TAB) {
#pragma unroll
    for (int i = 0; i < G::IPW; ++i) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int b = min(grp * G::NB + dma_row[i] + u * G::KT, p.nb - 1);
        const int node = min(max(p.beam_node[(size_t)r * p.nb + b], 0), p.rrow_n - 1);
        const uint32_t tr = min((uint32_t)p.rrow[(size_t)r * p.rrow_n + node], (uint32_t)p.rtab_rows - 1);
        q_tab[i][u] = (size_t)tr * 3 * row + (size_t)h * HD;
      }
    }
  }

  // ---- prologue, in stream order: chain ids or the parent array and beam
  // nodes (wave 0), the queries of the workgroup into the last stage (its K
  // half: beams 0..63, V half: beams 64..127, K-swizzled rows), then prompt
  // tiles 0..NS-2.
  if (chains && p.parent != nullptr && wave == 0) {
    const int32_t *par = p.parent + (size_t)r * p.cap;
    for (int i = 0; i * 64 < p.cap; ++i) dma4(par + min(i * 64 + lane, p.cap - 1), par_s + i * 64);
    const int32_t *bnp = p.beam_node + (size_t)r * p.nb;
    for (int i = 0; i * 64 < G::NB; ++i) dma4(bnp + min(grp * G::NB + i * 64 + lane, p.nb - 1), bn_s + i * 64);
    if constexpr (TAB) {
      const int32_t *rr = p.rrow + (size_t)r * p.rrow_n;
      for (int i = 0; i * 64 < p.rrow_n; ++i) dma4(rr + min(i * 64 + lane, p.rrow_n - 1), row_s + i * 64);
    }
  }
  if (chains && p.ids != nullptr && wave == 0) {
    const int words = p.D * G::NB;
    const int32_t *src0 = p.ids + (size_t)r * p.D * p.nb_pad + (size_t)grp * G::NB;
    for (int i = 0; i * 256 < words; ++i) {
      const int e = min(i * 256 + 4 * lane, words - 4);   // 4 ids per lane
      const int d = e / G::NB, b = e % G::NB;
      dma16(src0 + (size_t)d * p.nb_pad + b, ids_s + i * 256);
    }
  }
#pragma unroll
  for (int i = 0; i < G::IPW; ++i) {
    const int blk = wave * G::IPW + i;
    if constexpr (TAB) {
      dma16(p.rtab + q_tab[i][0] + dma_k[i], K3 + blk * 512);
      if constexpr (G::NB > G::KT) dma16(p.rtab + q_tab[i][1] + dma_k[i], V3 + blk * 512);
    } else {
      const int b0 = grp * G::NB + dma_row[i];
      const size_t s0 = ((size_t)r * p.nb + min(b0, p.nb - 1)) * row + (size_t)h * HD;
      dma16(p.q + s0 + dma_k[i], K3 + blk * 512);
      if constexpr (G::NB > G::KT) {
        const size_t s1 = ((size_t)r * p.nb + min(b0 + G::KT, p.nb - 1)) * row + (size_t)h * HD;
        dma16(p.q + s1 + dma_k[i], V3 + blk * 512);
      }
    }
  }
  issue_prompt(0, Stage<0>{});
  if constexpr (NS > 2) issue_prompt(1, Stage<1>{});
  if constexpr (NS > 3) issue_prompt(2, Stage<2>{});

  // per-lane LDS byte offsets of the operand reads (stage base added later)
  int koff[2][G::KSTEP];
#pragma unroll
  for (int sub = 0; sub < 2; ++sub)
#pragma unroll
    for (int j = 0; j < G::KSTEP; ++j) {
      const int tr = 32 * sub + c;
      koff[sub][j] = tr * G::RB + ((((HD / 16) * g + j) ^ swz_k<HD>(tr)) << 4);
    }
  int voff[G::DT][4][2];
  {
    const int q16 = lane >> 4, j16 = lane & 15;
#pragma unroll
    for (int dt = 0; dt < G::DT; ++dt)
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int tr = 16 * t + 8 * hh + 4 * g + (j16 >> 2);
          const int d = 32 * dt + 16 * (q16 & 1) + 4 * (j16 & 3);
          voff[dt][t][hh] = tr * G::RB + (((d >> 3) ^ swz_v<HD>(tr)) << 4) + ((d & 7) << 1);
        }
  }
  // this lane's row in a query / chain-record tile: row wb % 64 of tile wb / 64
  const int my_bb = (wave * 32) / G::KT;        // wave-uniform
  const int rrow = wb % G::KT;
  int roff_k[G::KSTEP], roff_v[G::DT][4];
#pragma unroll
  for (int j = 0; j < G::KSTEP; ++j) roff_k[j] = rrow * G::RB + ((((HD / 16) * g + j) ^ swz_k<HD>(rrow)) << 4);
#pragma unroll
  for (int dt = 0; dt < G::DT; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      roff_v[dt][q4] = rrow * G::RB + (((4 * dt + q4) ^ swz_v<HD>(rrow)) << 4) + 8 * g;

  float m_run = -__builtin_inff(), l_run = 0.f;
  f32x16 O[G::DT];
#pragma unroll
  for (int t = 0; t < G::DT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) O[t][i] = 0.f;
  bf16x8 qf[G::KSTEP];  // B operand of S^T: lane (g, c) holds head dims (HD/2)*g + 8j .. +8 of its beam
  int cnt = 0;          // chain records of this lane's beam
  float rec_alpha = 1.f, rec_p = 0.f;   // a record's rescale and weight, from its key tile to its value tile
  // The B operand of a record value product: in k-step st, lane (c, g) holds
  // rows 16 st + 8 (e >> 2) + 4 g + (e & 3) of column c at element e (the
  // order the prompt's P and V operands use), so beam c's weight sits in the
  // lanes with g = bit 2 of c, k-step c >> 4, element e below.
  const int rec_e = 4 * ((c >> 3) & 1) + (c & 3);
  const int rec_bi = g == ((c >> 2) & 1) ? 4 * (c >> 4) + (rec_e >> 1) : 8;   // 32-bit word of bd[], or none
  const int rec_sh = 16 * (rec_e & 1);

  // Per tile: wait until its stage has landed, then refill the stage of
  // tile - 1.  The prompt loop's stage-0 head also does the tile-0 work.
  auto head = [&](int tile, auto S, auto in_prompt) GR_INLINE {
    constexpr int st = decltype(S)::value;
    // at tile 0 the prologue has put exactly NS-2 tiles behind it
    wait_tiles(tile == 0 ? NS - 2 : min(NS - 2, n_total - 1 - tile));
    ring_barrier();
    if constexpr (st == 0 && decltype(in_prompt)::value) {
      if (tile == 0) {
        // queries and chain ids / parents have landed (they precede tile 0)
        if (chains && p.parent != nullptr && tid < G::NB) {
          // resolve the chain of workgroup beam tid in LDS, checking range,
          // order and depth (heads of one request see the same chains; the
          // head-0 workgroup reports)
          int n = grp * G::NB + tid < p.nb ? bn_s[tid] : -1;
          int err = 0;
          for (int d = 0; d < p.D; ++d) {
            int id = -1;
            if (n != -1) {
              if (n < 0 || n >= (TAB ? p.rrow_n : p.cap)) {   // TAB: only nodes with a table row
                err |= GR_DEVERR_PARENT_RANGE;
                n = -1;
              } else {
                id = n;
                const int pn = par_s[n];
                if (pn < -1 || pn >= p.cap) { err |= GR_DEVERR_PARENT_RANGE; n = -1; }
                else if (pn >= n) { err |= GR_DEVERR_PARENT_ORDER; n = -1; }
                else n = pn;
              }
            }
            ids16[d * G::NB + tid] = (int16_t)id;
          }
          if (n != -1) err |= GR_DEVERR_DEPTH;
          if (err && h == 0) atomicOr(p.dev_err, err);
        }
        if (wave * 32 < G::KT) {
#pragma unroll
          for (int j = 0; j < G::KSTEP; ++j) qf[j] = *(const bf16x8 *)((const char *)K3 + roff_k[j]);
        } else {
#pragma unroll
          for (int j = 0; j < G::KSTEP; ++j) qf[j] = *(const bf16x8 *)((const char *)V3 + roff_k[j]);
        }
        // every wave holds its queries before the last stage is refilled,
        // and the chain ids are visible to all
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
        ring_barrier();
        if (chains) {
          int depth = 0;
          for (int d = 0; d < p.D; ++d) {
            const int own = chain_id(d, wb);
            cnt += own >= 0 ? 1 : 0;
            bool any = lane < G::NB && chain_id(d, lane) >= 0;
            if constexpr (G::NB > 64) any = any || chain_id(d, 64 + lane) >= 0;
            if (__ballot(any)) depth = d + 1;
          }
          n_total = n_pre + depth * G::NRB;
        }
      }
    }
    // every wave is past tile-1: its stage can be refilled
    if (tile + NS - 1 < n_total) issue(tile + NS - 1, Stage<(st + NS - 1) % NS>{});
  };
  auto prompt_tile = [&](int tile, auto S) GR_INLINE {
    const char *kb = (const char *)kst(S);
    const char *vb = (const char *)vst(S);
    // ---- shared prompt window
    f32x16 S0, S1;
#pragma unroll
    for (int i = 0; i < 16; ++i) { S0[i] = 0.f; S1[i] = 0.f; }
#pragma unroll
    for (int j = 0; j < G::KSTEP; ++j) {
      const bf16x8 a0 = *(const bf16x8 *)(kb + koff[0][j]);
      const bf16x8 a1 = *(const bf16x8 *)(kb + koff[1][j]);
      S0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[j], S0, 0, 0, 0);
      S1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[j], S1, 0, 0, 0);
    }
    const int key0 = k_begin + tile * G::KT;
    if (key0 + G::KT > p.Lp) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kk = 8 * (i >> 2) + 4 * g + (i & 3);
        if (key0 + kk >= p.Lp) S0[i] = -__builtin_inff();
        if (key0 + 32 + kk >= p.Lp) S1[i] = -__builtin_inff();
      }
    }
    // IEEE maximum (v_maximum3_f32): no operand canonicalisation needed
    // two chains of v_maximum3, each folding two scores per instruction
    float mx0 = __builtin_elementwise_maximum(S0[0], S1[0]);
    float mx1 = __builtin_elementwise_maximum(S0[1], S1[1]);
#pragma unroll
    for (int i = 2; i < 16; i += 2) {
      mx0 = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mx0, S0[i]), S1[i]);
      mx1 = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mx1, S0[i + 1]), S1[i + 1]);
    }
    float mx = xor32_max(__builtin_elementwise_maximum(mx0, mx1)) * p.sl2;
    // Exact running max: the key that sets it gets weight exactly 1, which
    // bf16 holds exactly (it dominates a peaked softmax).  The rescale is
    // skipped only when no lane's max grew (then alpha would be 1).
    if (__ballot(mx > m_run)) {
      const float m_new = __builtin_elementwise_maximum(m_run, mx);
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < G::DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) O[dt][i] *= alpha;
    }
    uint32_t pw[16];
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      pw[i >> 1] = pack_bf16x2(fast_exp2(fmaf(S0[i], p.sl2, -m_run)), fast_exp2(fmaf(S0[i + 1], p.sl2, -m_run)));
      pw[8 + (i >> 1)] =
          pack_bf16x2(fast_exp2(fmaf(S1[i], p.sl2, -m_run)), fast_exp2(fmaf(S1[i + 1], p.sl2, -m_run)));
    }
    // row sums of the rounded weights the PV product uses
#pragma unroll
    for (int i = 0; i < 16; ++i) l_run = add_bf16x2(pw[i], l_run);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint4 pk4 = make_uint4(pw[4 * t], pw[4 * t + 1], pw[4 * t + 2], pw[4 * t + 3]);
      const bf16x8 pf = __builtin_bit_cast(bf16x8, pk4);
#pragma unroll
      for (int dt = 0; dt < G::DT; ++dt) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(GR_LDS4(vb + voff[dt][t][0]));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(GR_LDS4(vb + voff[dt][t][1]));
        const i16x4 a8[2] = {lo, hi};
        const bf16x8 a = __builtin_bit_cast(bf16x8, a8);
        O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf, O[dt], 0, 0, 0);
      }
    }
  };
  // Chain levels of 128-beam workgroups: the key tile folds each beam's
  // record score into its running max and sum, the value tile its value row
  // into O.  rb is the half of the stage holding this wave's beams.
  auto rec_key = [&](int d, const char *rb) GR_INLINE {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < G::KSTEP; ++j)
      s += dot8_bf16(__builtin_bit_cast(uint4, qf[j]), *(const uint4 *)(rb + roff_k[j]));
    s = xor32_sum(s);
    rec_alpha = 1.f;                     // a level the beam's chain does not reach adds nothing
    rec_p = 0.f;
    if (d < cnt) {
      const float t = s * p.sl2;
      const float m_new = __builtin_elementwise_maximum(m_run, t);
      rec_alpha = fast_exp2(m_run - m_new);
      // rounded to bf16, as it enters the value product as an MFMA operand
      rec_p = bf16_to_f32(f32_to_bf16(fast_exp2(t - m_new)));
      l_run = l_run * rec_alpha + (g == 0 ? rec_p : 0.f);
      m_run = m_new;
    }
  };
  // O^T = alpha O^T + V^T diag(p) on the MFMA.  A is the value rows of this
  // wave's 32 beams, read transposed like the prompt's value tile; B holds
  // each beam's weight at its own row and column and zeros elsewhere.  alpha
  // is 1 in every lane unless a record raised some beam's running max.
  auto rec_value = [&](const char *rb) GR_INLINE {
    if (__ballot(rec_alpha != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < G::DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) O[dt][i] *= rec_alpha;
    }
    const uint32_t pw = (uint32_t)f32_to_bf16(rec_p) << rec_sh;
    bf16x8 bd[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const uint4 w = make_uint4(rec_bi == 4 * st ? pw : 0u, rec_bi == 4 * st + 1 ? pw : 0u,
                                 rec_bi == 4 * st + 2 ? pw : 0u, rec_bi == 4 * st + 3 ? pw : 0u);
      bd[st] = __builtin_bit_cast(bf16x8, w);
    }
    const char *const ab = rb + 32 * (wave & 1) * G::RB;   // this wave's 32 rows
#pragma unroll
    for (int dt = 0; dt < G::DT; ++dt)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(GR_LDS4(ab + st * 16 * G::RB + voff[dt][0][0]));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(GR_LDS4(ab + st * 16 * G::RB + voff[dt][0][1]));
        const i16x4 a8[2] = {lo, hi};
        O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a8), bd[st], O[dt], 0, 0, 0);
      }
  };
  // Smaller workgroups: one tile per chain level, beam t's key in row t of
  // the stage's first half and its value in the second.
  auto record_tile = [&](int tile, auto S) GR_INLINE {
    const char *kb = (const char *)kst(S);
    const char *vb = (const char *)vst(S);
    const int k = tile - n_pre;
    const int d = k / G::NRB, bb = k % G::NRB;
    if (bb != my_bb) return;
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < G::KSTEP; ++j)
      s += dot8_bf16(__builtin_bit_cast(uint4, qf[j]), *(const uint4 *)(kb + roff_k[j]));
    s = xor32_sum(s);
    if (d < cnt) {
      const float t = s * p.sl2;
      const float m_new = fmaxf(m_run, t);
      const float alpha = fast_exp2(m_run - m_new);
      const float pr = fast_exp2(t - m_new);
      l_run = l_run * alpha + (g == 0 ? pr : 0.f);
#pragma unroll
      for (int dt = 0; dt < G::DT; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const uint2 vv = *(const uint2 *)(vb + roff_v[dt][q4]);
          O[dt][4 * q4 + 0] = fmaf(pr, bf16_lo(vv.x), O[dt][4 * q4 + 0] * alpha);
          O[dt][4 * q4 + 1] = fmaf(pr, bf16_hi(vv.x), O[dt][4 * q4 + 1] * alpha);
          O[dt][4 * q4 + 2] = fmaf(pr, bf16_lo(vv.y), O[dt][4 * q4 + 2] * alpha);
          O[dt][4 * q4 + 3] = fmaf(pr, bf16_hi(vv.y), O[dt][4 * q4 + 3] * alpha);
        }
      m_run = m_new;
    }
  };
  // The prompt tiles [0, n_pre) and the chain-record tiles [n_pre, n_total)
  // run in loops of their own: with both kinds in one loop body the register
  // allocator moves the O accumulators between register ranges at every tile.
  auto pstep = [&](int t0, auto S) GR_INLINE {
    const int tile = t0 + decltype(S)::value;
    if (tile < n_pre) {
      head(tile, S, std::true_type{});
      if (tile < n_tiles) prompt_tile(tile, S);
    }
  };
  auto rstep = [&](int t0, auto S) GR_INLINE {
    const int tile = t0 + decltype(S)::value;
    if (tile >= n_pre && tile < n_total) {
      head(tile, S, std::false_type{});
      record_tile(tile, S);
    }
  };
  for (int t0 = 0; t0 < n_pre; t0 += NS) {
    pstep(t0, Stage<0>{});
    pstep(t0, Stage<1>{});
    if constexpr (NS > 2) pstep(t0, Stage<2>{});
    if constexpr (NS > 3) pstep(t0, Stage<3>{});
  }
  if constexpr (G::NRB == 2) {
    // One chain level per iteration, its key tile then its value tile: the
    // levels do not follow the ring's period, so the stage is picked at run
    // time (the DMAs are asm the compiler does not track, and every wait is
    // explicit, so a run-time stage costs only its address).
    auto stage_at = [&](int st) GR_INLINE -> uint16_t * {
      if constexpr (NS > 3) if (st == 3) return KV3;
      if constexpr (NS > 2) if (st == 2) return KV2;
      return st == 1 ? KV1 : KV0;
    };
    auto rec_head = [&](int tile) GR_INLINE {
      wait_tiles(min(NS - 2, n_total - 1 - tile));
      ring_barrier();
      const int nt = tile + NS - 1;      // every wave is past tile - 1: refill its stage
      if (nt < n_total) {
        uint16_t *const ks = stage_at(nt % NS);
        const int k = nt - n_pre;
        issue_records(k / G::NRB, k % G::NRB, ks, ks + G::TB / 2);
      }
    };
    for (int tile = n_pre; tile < n_total; tile += 2) {
      const int d = (tile - n_pre) >> 1;
      rec_head(tile);
      {
        const char *const sb = (const char *)stage_at(tile % NS);
        rec_key(d, my_bb ? sb + G::TB : sb);
      }
      rec_head(tile + 1);
      {
        const char *const sb = (const char *)stage_at((tile + 1) % NS);
        rec_value(my_bb ? sb + G::TB : sb);
      }
    }
  } else {
    for (int t0 = n_pre - n_pre % NS; t0 < n_total; t0 += NS) {
      rstep(t0, Stage<0>{});
      rstep(t0, Stage<1>{});
      if constexpr (NS > 2) rstep(t0, Stage<2>{});
      if constexpr (NS > 3) rstep(t0, Stage<3>{});
    }
  }

  // ---- epilogue.  o leaves through LDS: each lane holds 4-element pieces of
  // one beam's row, and storing them directly would write 16 bytes into each
  // of 32 rows per instruction (partial lines, several times their bytes in
  // HBM time).  The rows are staged in the (now free) first ring stage with
  // XOR-swizzled 16-byte chunks, then written with consecutive lanes covering
  // whole rows.
  const float l_tot = xor32_sum(l_run);
  const size_t out_row0 = ((size_t)r * p.nb + (size_t)grp * G::NB) * row + (size_t)h * HD;
  const int n_rows = min(G::NB, p.nb - grp * G::NB);   // rows of this workgroup that exist
  // bf16 feed of the projection: head-major [R][H][nb][HD], so that this
  // workgroup's rows form one contiguous block
  const size_t lowp_row0 = (((size_t)r * p.H + h) * p.nb + (size_t)grp * G::NB) * HD;
  __syncthreads();                                      // every wave is past its last tile
  // fp32 rows o * sc to dst0 + row_index * stride, staged in the first ring
  // stage (64 rows at a time) and written with consecutive lanes per row
  auto store_f32 = [&](float *dst0, size_t stride, float sc) GR_INLINE {
    constexpr int CPR = HD / 4;                         // 16-byte chunks per fp32 row
    float *st = (float *)KV0;                           // 64 rows x HD fp32 (<= 16 KB)
#pragma unroll
    for (int half = 0; half < (G::NB + 63) / 64; ++half) {
      if ((wb >> 6) == half) {                          // wave-uniform
        const int lr = wb & 63;
#pragma unroll
        for (int dt = 0; dt < G::DT; ++dt)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int pch = (8 * dt + 2 * q4 + g) ^ (lr & (CPR - 1));
            *(float4 *)(st + lr * HD + pch * 4) = make_float4(O[dt][4 * q4] * sc, O[dt][4 * q4 + 1] * sc,
                                                              O[dt][4 * q4 + 2] * sc, O[dt][4 * q4 + 3] * sc);
          }
      }
      __syncthreads();
      const int rows_h = min(64, n_rows - 64 * half);
      for (int id = tid; id < rows_h * CPR; id += NW * 64) {
        const int lr = id / CPR, ch = id % CPR;
        const float4 v = *(const float4 *)(st + lr * HD + ((ch ^ (lr & (CPR - 1))) << 2));
        *(float4 *)(dst0 + (size_t)(64 * half + lr) * stride + ch * 4) = v;
      }
      __syncthreads();
    }
  };
  if (p.n_split > 1) {
    // partial state of this run: unnormalised o rows, then (max, sum) per
    // beam (the max in the exp2 domain of the scores times scale*log2(e))
    const size_t slot = (((size_t)r * p.H + h) * p.n_split + split) * p.nb_pad + (size_t)grp * G::NB;
    store_f32(p.part + slot * HD, HD, 1.f);
    float2 *ml = reinterpret_cast<float2 *>(p.part + (size_t)p.R * p.H * p.n_split * p.nb_pad * HD);
    if (g == 0 && valid) ml[slot + wb] = make_float2(m_run, l_tot);
    return;
  }
  const float inv = valid ? 1.f / l_tot : 0.f;
  if (p.out_bf16 != nullptr) {
    constexpr int CPR = HD / 8;                         // 16-byte chunks per bf16 row
    uint16_t *st = KV0;                                 // NB rows x HD bf16 (<= 16 KB)
#pragma unroll
    for (int dt = 0; dt < G::DT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int pch = (4 * dt + q4) ^ (wb & (CPR - 1));
        *(uint2 *)(st + wb * HD + pch * 8 + 4 * g) =
            make_uint2(pack_bf16x2(O[dt][4 * q4] * inv, O[dt][4 * q4 + 1] * inv),
                       pack_bf16x2(O[dt][4 * q4 + 2] * inv, O[dt][4 * q4 + 3] * inv));
      }
    __syncthreads();
    for (int id = tid; id < n_rows * CPR; id += NW * 64) {
      const int rr = id / CPR, ch = id % CPR;
      const uint4 v = *(const uint4 *)(st + rr * HD + ((ch ^ (rr & (CPR - 1))) << 3));
      *(uint4 *)(p.out_bf16 + lowp_row0 + (size_t)rr * HD + ch * 8) = v;
    }
    __syncthreads();
  }
  if (p.out_f32 != nullptr) store_f32(p.out_f32 + out_row0, row, inv);
}

// The runs of a split window, merged per (request, head, beam) with their
// log-sum-exp weights: m = max_s m_s, w_s = 2^(m_s - m) / sum_s' 2^(m_s' - m) l_s',
// o = sum_s w_s o_s.  One workgroup per (request, head, MB beams); thread t
// serves beam t / CH and, in turn, the runs t % CH, t % CH + CH, ... (the
// weights, reduced across the CH threads of a beam and kept in LDS) and the
// 16-byte chunk t % CH of the beam's row (summed over the runs, four runs'
// loads at a time).
struct MergeP {
  const float *part;
  float *out_f32;
  uint16_t *out_bf16;
  int R, H, nb, nb_pad, n_split;
};

template <int HD>
__global__ __launch_bounds__(256) void attn_merge_kernel(MergeP p) {
  constexpr int CH = HD / 4, MB = 256 / CH;           // chunks per row, beams per workgroup
  __shared__ float wts[MB][kAttnSplitTarget];         // attn_split keeps the runs at or below this
  const int n_bt = (p.nb + MB - 1) / MB;
  int bid = blockIdx.x;
  const int bt = bid % n_bt;
  bid /= n_bt;
  const int h = bid % p.H, r = bid / p.H;
  const int tid = threadIdx.x, b = tid / CH, li = tid % CH;
  const int beam = bt * MB + b;
  const bool valid = beam < p.nb;
  const int bq = valid ? beam : p.nb - 1;
  const size_t unit = ((size_t)r * p.H + h) * p.n_split;
  const float2 *ml = reinterpret_cast<const float2 *>(p.part + (size_t)p.R * p.H * p.n_split * p.nb_pad * HD);
  float m = -__builtin_inff();
  for (int sp = li; sp < p.n_split; sp += CH) m = fmaxf(m, ml[(unit + sp) * p.nb_pad + bq].x);
#pragma unroll
  for (int o = CH / 2; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  float l = 0.f;
  for (int sp = li; sp < p.n_split; sp += CH) {
    const float2 e = ml[(unit + sp) * p.nb_pad + bq];
    l = fmaf(fast_exp2(e.x - m), e.y, l);
  }
#pragma unroll
  for (int o = CH / 2; o > 0; o >>= 1) l += __shfl_xor(l, o);
  const float inv = 1.f / l;
  for (int sp = li; sp < p.n_split; sp += CH) wts[b][sp] = fast_exp2(ml[(unit + sp) * p.nb_pad + bq].x - m) * inv;
  __syncthreads();
  const size_t run = (size_t)p.nb_pad * HD;
  const float *src = p.part + (unit * p.nb_pad + bq) * HD + li * 4;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  auto add = [&](float w, float4 v) {
    o.x = fmaf(w, v.x, o.x);
    o.y = fmaf(w, v.y, o.y);
    o.z = fmaf(w, v.z, o.z);
    o.w = fmaf(w, v.w, o.w);
  };
  int sp = 0;
  for (; sp + 4 <= p.n_split; sp += 4) {
    const float4 v0 = *(const float4 *)(src + sp * run), v1 = *(const float4 *)(src + (sp + 1) * run);
    const float4 v2 = *(const float4 *)(src + (sp + 2) * run), v3 = *(const float4 *)(src + (sp + 3) * run);
    add(wts[b][sp], v0);
    add(wts[b][sp + 1], v1);
    add(wts[b][sp + 2], v2);
    add(wts[b][sp + 3], v3);
  }
  for (; sp < p.n_split; ++sp) add(wts[b][sp], *(const float4 *)(src + sp * run));
  if (!valid) return;
  if (p.out_f32)
    *(float4 *)(p.out_f32 + ((size_t)r * p.nb + beam) * p.H * HD + (size_t)h * HD + li * 4) = o;
  if (p.out_bf16)
    *(uint2 *)(p.out_bf16 + (((size_t)r * p.H + h) * p.nb + beam) * HD + li * 4) =
        make_uint2(pack_bf16x2(o.x, o.y), pack_bf16x2(o.z, o.w));
}

// ------------------------------------------------------------------ fp32
struct AttnPF {
  const float *pk, *pv, *q, *ak, *av;
  const int32_t *parent, *beam_node;
  float *out;
  int32_t *dev_err;
  int R, H, Lp, Lw, nb, cap, max_depth, n_chunk;
  float scale;
};

template <int HD>
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnPF p) {
  constexpr int KT = 32;
  __shared__ float Ks[KT][HD], Vs[KT][HD];
  int bid = blockIdx.x;
  const int chunk = bid % p.n_chunk;
  bid /= p.n_chunk;
  const int h = bid % p.H, r = bid / p.H;
  const int beam = chunk * 64 + threadIdx.x;
  const bool valid = beam < p.nb;
  const size_t row = (size_t)p.H * HD;
  float q[HD], o[HD];
  const float *qp = p.q + ((size_t)r * p.nb + (valid ? beam : 0)) * row + (size_t)h * HD;
#pragma unroll
  for (int i = 0; i < HD; ++i) { q[i] = valid ? qp[i] : 0.f; o[i] = 0.f; }
  float m = -__builtin_inff(), l = 0.f;

  if (p.beam_node != nullptr && valid) {
    int n = p.beam_node[(size_t)r * p.nb + beam];
    int err = 0;
    const int32_t *par = p.parent + (size_t)r * p.cap;
    for (int depth = 0; n != -1; ++depth) {
      if (n < 0 || n >= p.cap) { err |= GR_DEVERR_PARENT_RANGE; break; }
      if (depth >= p.max_depth) { err |= GR_DEVERR_DEPTH; break; }
      const int pn = par[n];
      const float *kn = p.ak + ((size_t)r * p.cap + n) * row + (size_t)h * HD;
      const float *vn = p.av + ((size_t)r * p.cap + n) * row + (size_t)h * HD;
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < HD; ++i) s = fmaf(q[i], kn[i], s);
      s *= p.scale;
      const float m_new = fmaxf(m, s);
      const float alpha = expf(m - m_new), pr = expf(s - m_new);
      l = l * alpha + pr;
#pragma unroll
      for (int i = 0; i < HD; ++i) o[i] = fmaf(pr, vn[i], o[i] * alpha);
      m = m_new;
      if (pn < -1 || pn >= p.cap) { err |= GR_DEVERR_PARENT_RANGE; break; }
      if (pn >= n) { err |= GR_DEVERR_PARENT_ORDER; break; }
      n = pn;
    }
    if (err) atomicOr(p.dev_err, err);
  }

  const float *pk = p.pk + (size_t)r * p.Lp * row + (size_t)h * HD;
  const float *pv = p.pv + (size_t)r * p.Lp * row + (size_t)h * HD;
  for (int k0 = p.Lp - p.Lw; k0 < p.Lp; k0 += KT) {
    const int nk = min(KT, p.Lp - k0);
    __syncthreads();
    for (int e = threadIdx.x; e < KT * HD; e += 64) {
      const int kk = e / HD, i = e % HD;
      Ks[kk][i] = kk < nk ? pk[(size_t)(k0 + kk) * row + i] : 0.f;
      Vs[kk][i] = kk < nk ? pv[(size_t)(k0 + kk) * row + i] : 0.f;
    }
    __syncthreads();
    float s[KT];
    float mx = -__builtin_inff();
#pragma unroll
    for (int kk = 0; kk < KT; ++kk) {
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < HD; ++i) a = fmaf(q[i], Ks[kk][i], a);
      s[kk] = kk < nk ? a * p.scale : -__builtin_inff();
      mx = fmaxf(mx, s[kk]);
    }
    const float m_new = fmaxf(m, mx);
    const float alpha = expf(m - m_new);
    l *= alpha;
#pragma unroll
    for (int i = 0; i < HD; ++i) o[i] *= alpha;
#pragma unroll
    for (int kk = 0; kk < KT; ++kk) {
      const float pr = expf(s[kk] - m_new);
      l += pr;
#pragma unroll
      for (int i = 0; i < HD; ++i) o[i] = fmaf(pr, Vs[kk][i], o[i]);
    }
    m = m_new;
  }
  if (!valid) return;
  const float inv = 1.f / l;
  float *op = p.out + ((size_t)r * p.nb + beam) * row + (size_t)h * HD;
#pragma unroll
  for (int i = 0; i < HD; ++i) op[i] = o[i] * inv;
}


template <int HD, int NW>
hipError_t launch_bf16(const AttnArgs &a, hipStream_t s) {
  constexpr int NS = kAttnStages, OCC = NW == 4 ? 6 - NS : (NW == 2 ? 2 : 1);
  constexpr int NB = NW * 32;
  AttnP p;
  p.pk = (const uint16_t *)a.pk; p.pv = (const uint16_t *)a.pv; p.q = (const uint16_t *)a.q;
  p.ak = (const uint16_t *)a.ak; p.av = (const uint16_t *)a.av;
  p.rtab = (const uint16_t *)a.rec_tab; p.rrow = a.rec_row; p.rrow_n = a.rec_rows; p.rtab_rows = a.rec_tab_rows;
  p.ids = nullptr; p.parent = nullptr; p.beam_node = nullptr; p.dev_err = a.dev_err;
  p.out_f32 = a.out_f32; p.out_bf16 = (uint16_t *)a.out_lowp;
  p.R = a.R; p.H = a.H; p.Lp = a.Lp; p.Lw = a.Lw; p.nb = a.nb; p.cap = a.cap;
  p.D = a.max_depth;
  p.nb_pad = attn_beam_pad(a.nb);
  p.n_grp = p.nb_pad / NB;
  p.sl2 = a.scale * kLog2e;
  p.ids_words = 0;
  p.par_words = 0;
  // The in-kernel resolve stages the parent array; when that would cost a
  // resident workgroup per CU (and the pre-pass ids would not), the chains
  // go through the pre-pass instead.
  using G = Geo<HD, NW, NS>;
  const size_t static_lds = (size_t)(NS < 4 ? NS : 4) * G::TB * sizeof(uint16_t) + 1024;   // upper bound
  const size_t lds_per_cu = 160 * 1024;
  const size_t inkernel_dyn = ((size_t)(a.max_depth * NB + 1) / 2 + (a.cap + 63) / 64 * 64 + (NB + 63) / 64 * 64) * 4;
  const size_t prepass_dyn = (size_t)(a.max_depth * NB + 255) / 256 * 256 * 4;
  const bool inkernel_fits = (static_lds + inkernel_dyn) * OCC <= lds_per_cu;
  const bool prepass_fits = (static_lds + prepass_dyn) * OCC <= lds_per_cu;
  const bool tab = a.rec_tab != nullptr;
  if (tab && (a.beam_node == nullptr || a.rec_row == nullptr || a.cap > kLdsChainNodes || a.rec_rows < 1 ||
              a.rec_rows > a.cap || a.rec_tab_rows < 1))
    return hipErrorInvalidValue;
  if (a.beam_node != nullptr) {
    if (tab || (a.cap <= kLdsChainNodes && (inkernel_fits || !prepass_fits || a.chain_ids == nullptr))) {
      p.parent = a.parent;
      p.beam_node = a.beam_node;
      p.ids_words = (a.max_depth * NB + 1) / 2;           // int16 ids, two per word
      p.par_words = (a.cap + 63) / 64 * 64;
    } else {
      ChainP c;
      c.parent = a.parent; c.beam_node = a.beam_node; c.ids = a.chain_ids; c.dev_err = a.dev_err;
      c.R = a.R; c.nb = a.nb; c.nb_pad = p.nb_pad; c.cap = a.cap; c.D = a.max_depth;
      const long long n = (long long)a.R * p.nb_pad;
      hipLaunchKernelGGL(chain_resolve_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, c);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      p.ids = a.chain_ids;
      p.ids_words = (a.max_depth * NB + 255) / 256 * 256;   // the ids arrive in 1 KB DMA blocks
    }
  }
  const AttnSplit sp = attn_split(a.R, a.H, a.nb, a.Lw);
  p.n_split = sp.n_split;
  p.tps = sp.tiles_per_split;
  p.part = a.split_ws;
  if (sp.n_split > 1 && a.split_ws == nullptr) return hipErrorInvalidValue;   // the caller checks this
  const size_t dyn = (size_t)(p.ids_words + p.par_words + (p.parent ? (NB + 63) / 64 * 64 : 0) +
                              (tab ? p.par_words : 0)) * sizeof(int32_t);
  const long long grid = (long long)a.R * a.H * p.n_grp * p.n_split;
  if (tab)
    hipLaunchKernelGGL((attn_bf16_kernel<HD, NW, NS, OCC, true>), dim3((unsigned)grid), dim3(NW * 64), dyn, s, p);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<HD, NW, NS, OCC, false>), dim3((unsigned)grid), dim3(NW * 64), dyn, s, p);
  if (sp.n_split == 1) return hipGetLastError();
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  MergeP m;
  m.part = a.split_ws; m.out_f32 = a.out_f32; m.out_bf16 = (uint16_t *)a.out_lowp;
  m.R = a.R; m.H = a.H; m.nb = a.nb; m.nb_pad = p.nb_pad; m.n_split = sp.n_split;
  const long long n_wg = (long long)a.R * a.H * ((a.nb + 256 / (HD / 4) - 1) / (256 / (HD / 4)));
  hipLaunchKernelGGL(attn_merge_kernel<HD>, dim3((unsigned)n_wg), dim3(256), 0, s, m);
  return hipGetLastError();
}

template <int HD>
hipError_t launch_bf16_nw(const AttnArgs &a, hipStream_t s) {
  switch (attn_waves(a.nb)) {
    case 1: return launch_bf16<HD, 1>(a, s);
    case 2: return launch_bf16<HD, 2>(a, s);
    default: return launch_bf16<HD, 4>(a, s);
  }
}

template <int HD>
hipError_t launch_f32(const AttnArgs &a, hipStream_t s) {
  AttnPF p;
  p.pk = (const float *)a.pk; p.pv = (const float *)a.pv; p.q = (const float *)a.q;
  p.ak = (const float *)a.ak; p.av = (const float *)a.av;
  p.parent = a.parent; p.beam_node = a.beam_node; p.out = a.out_f32 ? a.out_f32 : (float *)a.out_lowp;
  p.dev_err = a.dev_err;
  p.R = a.R; p.H = a.H; p.Lp = a.Lp; p.Lw = a.Lw; p.nb = a.nb; p.cap = a.cap;
  p.max_depth = a.max_depth; p.n_chunk = (a.nb + 63) / 64; p.scale = a.scale;
  const long long grid = (long long)a.R * a.H * p.n_chunk;
  hipLaunchKernelGGL((attn_f32_kernel<HD>), dim3((unsigned)grid), dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn(const AttnArgs &a, hipStream_t s) {
  if (a.dtype == GR_BF16) return a.hd == 32 ? launch_bf16_nw<32>(a, s) : launch_bf16_nw<64>(a, s);
  return a.hd == 32 ? launch_f32<32>(a, s) : launch_f32<64>(a, s);
}

}  // namespace gr
