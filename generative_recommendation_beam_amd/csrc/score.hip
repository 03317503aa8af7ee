// Codebook scoring, log-softmax, prior add and exact top-k of the decode step.
//
// Engineering Exploration of Generative Recall, 4.2 Custom Beam Search: only
// the 256 codes of the current semantic-ID level are scored and ranked; the
// candidate score is the running beam score plus the code's log-probability
// and the best B of B_in x 256 survive.  TransRetrieval, GPU retrieval:
// candidate selection runs on the device, next to scoring.
//
// logits_select_bf16: one workgroup (8 waves) per (request, group of <= 128
// beams).  z^T = W o^T on v_mfma_f32_32x32x16_bf16 (codes x beams; wave w
// owns codes 32w.. for all beams).  o and W stream HBM/L2 -> LDS in 64-column
// blocks (global_load_lds, two blocks in flight): o into a ring shared by the
// workgroup, W into a ring of each wave's own rows.  Each lane then holds 16
// codes of each of four beams: the log-softmax is in-lane plus one lane^32
// swap and one LDS exchange between the 8 waves.  The selection bounds the
// k-th best score from the lanes' per-beam minima, stages only the
// candidates at or above the bound, finds the bin of the k-th among them in
// one 256-bin histogram and orders the few candidates up to that bin by
// counting ranks (the general radix selection of gr_select.h when the bound
// prunes too little); scores never leave the chip unless the caller asks for
// them.
//
// score_select: the same scoring and selection starting from fp32 logits in
// global memory (the standalone top-k entry point, the fp32 path and scalar
// scoring).  select_merge: final selection over per-group partial lists.
// project: VALU projection z = o . W^T for the fp32 path and the scalar
// score o . w.

#include <type_traits>

#include "gr_device.h"
#include "gr_launch.h"
#include "gr_select.h"

namespace gr {
namespace {

constexpr int kNT = 512;
constexpr int kCB = 64;                    // o columns per LDS block (four MFMA k-steps)
constexpr int kFastK = 512;                // largest k of the bounded selection
constexpr int kWaveStage = 512;            // staged candidates per wave, at most
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// o column block in LDS: 128 beam rows x 64 columns bf16 (128-byte rows).
// Logical 16-byte chunk q of row b sits at physical chunk q ^ swz(b): any 16
// consecutive rows read at one logical chunk then touch 16 distinct 16-byte
// slots of two 128-byte rows pairs, and any 8 of them distinct slots.
__device__ __forceinline__ int swz_o(int row) { return (row & 7) ^ ((row >> 3) & 1); }

constexpr int kOS = 3;                     // ring slots: the block in use and two in flight
struct LogitsSmem {
  union {
    struct {
      uint16_t ob[kOS][kGroupBeams * kCB];          // o blocks (3 x 16 KB)
      uint16_t wr[kNT / 64][kOS][32 * kCB];         // per wave: its 32 W rows of a block (8 x 3 x 4 KB)
    } ring;
    SelectSmem<kNT> sel;                   // selection afterwards (staging in sel.tmp)
  } u;
  float red_max[kNT / 64][kGroupBeams];    // per-wave partial max / sum of each beam's logits
  float red_sum[kNT / 64][kGroupBeams];
  uint4 wbest[kNT / 64];                   // per wave: (unused, unused, its best score, its lane-maximum bound) as rank keys
  uint32_t wpick[kNT / 64][4];             // per wave: its four best lane bounds (rank keys)
  uint32_t wcnt[kNT / 64];                 // per wave: staged candidates
  uint32_t n_final;                        // candidates gathered for the final ordering
};
static_assert(kWaveStage * (kNT / 64) <= kListCap, "staging area");

struct LP {
  const uint16_t *o, *W;
  const float *prior;
  float *cand;
  float *score;
  int32_t *token, *parent;
  uint64_t *partial;
  int R, n_in, D, hd_log2, k, lsm, n_groups, kk;
};

// NB: number of 64-column blocks of D when fixed at compile time (the
// block loop is then unrolled, and the compiler's waits count the loads in
// flight across blocks), 0 for any D.  BT: 32-beam tiles per group, 4
// (groups of 128 beams) or 2 (groups of 64: half the products, exps and
// selection work of a workgroup, for small beams or to spread many beams of
// few requests over more CUs).
template <int NB, int BT>
__global__ __launch_bounds__(kNT) void logits_select_bf16_kernel(LP p) {
  __shared__ LogitsSmem sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, c = lane & 31;
  // Consecutive workgroup ids go to the 8 XCDs in turn; XCD x takes the
  // x-th eighth of the requests, the same eighth whose attention output its
  // L2 received from the attention kernel (which maps its units alike).
  int bid = blockIdx.x;
  if ((gridDim.x & 7) == 0) bid = (bid & 7) * (int)(gridDim.x >> 3) + (bid >> 3);
  const int r = bid / p.n_groups, grp = bid % p.n_groups;
  const int b_begin = grp * 32 * BT;                   // groups of 32 BT beams
  const int nbg = min(32 * BT, p.n_in - b_begin);
  const int hd = 1 << p.hd_log2, H = p.D >> p.hd_log2;
  const uint16_t *o_req = p.o + (size_t)r * H * p.n_in * hd;
  const int n_blk = NB > 0 ? NB : (p.D + kCB - 1) / kCB;

  // priors of this lane's beams 32 t + c (read now, used after the projection)
  float pr[BT];
#pragma unroll
  for (int t = 0; t < BT; ++t) {
    const int bl = 32 * t + c;
    pr[t] = (bl < nbg && p.prior) ? p.prior[(size_t)r * p.n_in + b_begin + bl] : 0.f;
  }

  // ---- z^T = W o^T on v_mfma_f32_32x32x16_bf16: wave w forms codes
  // 32w .. 32w+31 (A: its own W rows) for all 128 beam rows (B: o, four
  // 32-beam tiles), 64 columns of D per block.  Both operands stream
  // HBM/L2 -> LDS by global_load_lds (whole 128-byte rows, two blocks ahead
  // of the MFMAs, three ring slots): o blocks into a ring shared by the
  // workgroup, W rows into a ring of the wave's own.  o is head-major
  // ([R][H][n_in][hd]); a 16-byte chunk never straddles heads.  Rows past
  // the group's beams repeat its last beam (never selected); columns past D
  // (a last half block) repeat the last chunk (never read).
  // Per wave and block: 2 o pieces + 4 W pieces of 1 KB (6 loads in flight
  // per block).
  constexpr int kDmaPerBlock = 6;
  auto issue = [&](int cb) {
    const int slot = cb % kOS;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int j = 2 * wave + i, row = 8 * j + (lane >> 3);
      const int col = min(cb * kCB + 8 * ((lane & 7) ^ swz_o(row)), p.D - 8);
      const int h = col >> p.hd_log2, ci = col & (hd - 1);
      const int b = min(b_begin + row, p.n_in - 1);
      dma16(o_req + ((size_t)h * p.n_in + b) * hd + ci, &sm.u.ring.ob[slot][j * 512]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int lr = 8 * i + (lane >> 3);
      const int col = min(cb * kCB + 8 * ((lane & 7) ^ swz_o(lr)), p.D - 8);
      dma16(p.W + (size_t)(32 * wave + lr) * p.D + col, &sm.u.ring.wr[wave][slot][i * 512]);
    }
  };
  f32x16 acc[BT];
#pragma unroll
  for (int t = 0; t < BT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[t][i] = 0.f;
  const int swb = swz_o(c);                 // rows c and 32 t + c share the swizzle of c
  // A block's operands (20 LDS reads) are all issued before its 16 MFMAs,
  // so that the LDS latency is paid once per block, not once per MFMA.
  auto mma = [&](int cb) {
    const int slot = cb % kOS;
    const bool full = NB > 0 || (p.D - cb * kCB) >= kCB;   // else a half block (2 k-steps)
    const uint16_t *ob = &sm.u.ring.ob[slot][c * kCB];
    const uint16_t *wb = &sm.u.ring.wr[wave][slot][c * kCB];
    bf16x8 a[4], bo[4][BT];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int off = ((2 * ks + g) ^ swb) << 3;
      a[ks] = *(const bf16x8 *)(wb + off);
#pragma unroll
      for (int t = 0; t < BT; ++t) bo[ks][t] = *(const bf16x8 *)(ob + 32 * t * kCB + off);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks < 2 || full) {
#pragma unroll
        for (int t = 0; t < BT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], bo[ks][t], acc[t], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4 + 4 * BT, 0);   // the LDS reads first,
    __builtin_amdgcn_sched_group_barrier(0x008, 4 * BT, 0);       // then the MFMAs
  };
  issue(0);
  if (n_blk > 1) issue(1);
  // Step cb: block cb has landed once at most the next block's loads are in
  // flight, and this wave's reads of block cb - 1 have completed; after the
  // barrier every wave is done with block cb - 1, whose slots receive block
  // cb + 2.
#pragma unroll
  for (int cb = 0; cb < n_blk; ++cb) {
    if (cb + 1 < n_blk) GR_WAIT_VMCNT_LGKM0(kDmaPerBlock);
    else GR_WAIT_VMCNT_LGKM0(0);
    ring_barrier();
    if (cb + 2 < n_blk) issue(cb + 2);
    mma(cb);
  }
  // Lane (c, g) now holds, for beam row 32 t + c, the logits of codes
  // 32 w + 8 (j >> 2) + 4 g + (j & 3) in acc[t][j].

  // ---- log-softmax over the 256 codes of each beam: partial max / sum over
  // the lane's 16 codes, the lane 32 apart (same beam), then the 8 waves.
  // The lane's smallest (NaN-propagating) and largest logit of each beam
  // also bound its 16 candidate scores, rounding being monotonic.
  float lo[BT], hi[BT];
#pragma unroll
  for (int t = 0; t < BT; ++t) {
    float mn = acc[t][0], mx = acc[t][0];
#pragma unroll
    for (int j = 1; j < 16; ++j) {
      mn = __builtin_elementwise_minimum(mn, acc[t][j]);
      mx = fmaxf(mx, acc[t][j]);
    }
    lo[t] = mn;
    hi[t] = mx;
  }
  float lse[BT];
#pragma unroll
  for (int t = 0; t < BT; ++t) lse[t] = 0.f;
  if (p.lsm) {
    float M[BT];
#pragma unroll
    for (int t = 0; t < BT; ++t) {
      const float mx = xor32_max(hi[t]);
      if (g == 0) sm.red_max[wave][32 * t + c] = mx;
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < BT; ++t) {
      float mx = sm.red_max[0][32 * t + c];
#pragma unroll
      for (int w = 1; w < kNT / 64; ++w) mx = fmaxf(mx, sm.red_max[w][32 * t + c]);
      M[t] = mx;
      const float Ml = mx * kLog2e;
      float se = 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) se += fast_exp2(fmaf(acc[t][j], kLog2e, -Ml));
      se = xor32_sum(se);
      if (g == 0) sm.red_sum[wave][32 * t + c] = se;
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < BT; ++t) {
      float se = sm.red_sum[0][32 * t + c];
#pragma unroll
      for (int w = 1; w < kNT / 64; ++w) se += sm.red_sum[w][32 * t + c];
      lse[t] = M[t] + __builtin_amdgcn_logf(se) * kLn2;
    }
  }

  // ---- candidate scores (z - lse) + prior, in place
  const int n = nbg * 256;
  const int k_sel = min(p.k, n);
  bool valid[BT];
#pragma unroll
  for (int t = 0; t < BT; ++t) {
    valid[t] = 32 * t + c < nbg;
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[t][j] = (acc[t][j] - lse[t]) + pr[t];
    if (valid[t] && p.cand) {
      float *crow = p.cand + ((size_t)r * p.n_in + b_begin + 32 * t + c) * 256 + 32 * wave + 4 * g;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *(float4 *)(crow + 8 * q) = make_float4(acc[t][4 * q], acc[t][4 * q + 1], acc[t][4 * q + 2], acc[t][4 * q + 3]);
    }
  }
  auto flat_of = [&](int t, int j) -> uint32_t {
    return (uint32_t)(b_begin + 32 * t + c) * 256u + 32u * wave + 8u * (uint32_t)(j >> 2) + 4u * g + (uint32_t)(j & 3);
  };

  // ---- bounded selection (k <= 512).  A unit is the 16 scores one lane
  // holds for one beam; its minimum u means 16 candidates score >= u.  The
  // lane bound is its best unit minimum (a unit with a NaN score bounds
  // nothing).  T is the ml-th best (ml = ceil(k/16)) of the waves' two best
  // lane bounds (four when ml > 16): ml units hold 16 ml >= k candidates scoring >= T, so every
  // selected candidate scores >= T, and only those are staged (by ballot,
  // into one region per wave).  One 256-bin histogram of the staged rank
  // keys over [best, T] finds the bin holding the k-th; the candidates up to
  // that bin are gathered and ordered (counting ranks up to 256 entries,
  // else a bucket pass or a sort).  A second bound, from the waves' best lane maxima,
  // tightens T when it can.  Too many staged candidates or a degenerate
  // bound go through the selection over all registers.  Every decision is
  // block-uniform.
  bool done = false;
  if (k_sel <= kFastK) {
    const int ml = (k_sel + 15) >> 4;                   // <= 32
    float lb = -__builtin_inff(), best = -__builtin_inff(), umax[BT];
    bool any = false;
#pragma unroll
    for (int t = 0; t < BT; ++t) {
      const float u = (lo[t] - lse[t]) + pr[t];
      umax[t] = (hi[t] - lse[t]) + pr[t];
      if (valid[t]) {
        lb = fmaxf(lb, u != u ? -__builtin_inff() : u);
        best = fmaxf(best, umax[t]);
        any = true;
      }
    }
    // picks: each wave's two best lane bounds, or its four best when the
    // bound needs more than 16 units (k > 256)
    const int np = ml > 16 ? 4 : 2;
    uint32_t w4[4] = {kInvalidKey, kInvalidKey, kInvalidKey, kInvalidKey};
    if (np == 4) wave_smallest4_u32(any ? rank_key(lb) : kInvalidKey, w4);
    else wave_small2_pair_u32(any ? rank_key(lb) : kInvalidKey, w4[0], w4[1]);
    const uint32_t wh = wave_min_u32(any ? rank_key(best) : kInvalidKey);
    // A second bound from the lanes' best candidates: the mw-th best lane
    // maximum of a wave (mw = ceil(k/8)) has mw candidates of that wave at or
    // above it, so the worst of the eight waves' values has 8 mw >= k
    // candidates at or above it.  It is the tighter one when the beams'
    // running scores lie close together (many beams share the best
    // candidates, and a unit's minimum says little).
    const uint32_t wv = wave_kth_smallest_u32(any ? rank_key(best) : kInvalidKey, (k_sel + 7) >> 3);
    if (lane < 4) sm.wpick[wave][lane] = lane == 0 ? w4[0] : lane == 1 ? w4[1] : lane == 2 ? w4[2] : w4[3];
    if (lane == 0) sm.wbest[wave] = make_uint4(0u, 0u, wh, wv);
    __syncthreads();                                    // also: the o buffers are no longer read
    uint32_t kmin = kInvalidKey, T = kInvalidKey;
    {
      // lane i < 8 np holds pick i (wave i / np's (i % np)-th best lane
      // bound); its rank among the 8 np picks (ties by position)
      uint32_t v = kInvalidKey;
      int rank = 0;
#pragma unroll
      for (int w = 0; w < kNT / 64; ++w) kmin = min(kmin, sm.wbest[w].z);
      const int npk = 8 * np;
      if (lane < npk) v = np == 4 ? sm.wpick[lane >> 2][lane & 3] : sm.wpick[lane >> 1][lane & 1];
      if (np == 4) {
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const uint32_t pi = sm.wpick[i >> 2][i & 3];
          rank += (pi < v || (pi == v && i < lane)) ? 1 : 0;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t pi = sm.wpick[i >> 1][i & 1];
          rank += (pi < v || (pi == v && i < lane)) ? 1 : 0;
        }
      }
      const uint64_t m = __builtin_amdgcn_ballot_w64(lane < npk && rank == ml - 1);
      T = (uint32_t)__builtin_amdgcn_readlane((int)v, (int)__builtin_ctzll(m));
      uint32_t T2 = 0u;
#pragma unroll
      for (int w = 0; w < kNT / 64; ++w) T2 = max(T2, sm.wbest[w].w);
      T = min(T, T2);
    }
    const float Ts = key_score(T);
    if (T != kInvalidKey && Ts > -__builtin_inff()) {
      uint64_t *reg = sm.u.sel.tmp + wave * kWaveStage;
      uint32_t *hist = sm.u.sel.bstart;
      uint32_t wc = 0;                                  // wave-uniform
#pragma unroll
      for (int t = 0; t < BT; ++t) {
        const bool ut = valid[t] && umax[t] >= Ts;
        if (!__builtin_amdgcn_ballot_w64(ut)) continue;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const bool q = ut && acc[t][j] >= Ts;
          const uint64_t m = __builtin_amdgcn_ballot_w64(q);
          if (m) {
            // staged as (score, register slot and lane); keyed below, one entry a thread
            const uint32_t pos = wc + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
            if (q && pos < kWaveStage)
              reg[pos] = ((uint64_t)(uint32_t)((16 * t + j) * 64 + lane) << 32) | __float_as_uint(acc[t][j]);
            wc += (uint32_t)__builtin_popcountll(m);
          }
        }
      }
      if (tid < 256) hist[tid] = 0u;
      if (lane == 0) sm.wcnt[wave] = wc;
      if (tid == 0) sm.n_final = 0u;
      __syncthreads();
      int wmax = 0;
#pragma unroll
      for (int w = 0; w < kNT / 64; ++w) wmax = max(wmax, (int)sm.wcnt[w]);
      if (wmax <= kWaveStage) {
        // staged keys lie in [kmin, T]: digit = (key - kmin) >> shift < 256
        const uint32_t range = T - kmin;
        const int shift = range >> 8 ? 24 - __builtin_clz(range) : 0;
        for (int i = lane; i < (int)wc; i += 64) {
          const uint64_t e = reg[i];
          const uint32_t sl = (uint32_t)(e >> 32), ln = sl & 63u, tj = sl >> 6;
          const uint32_t key = rank_key(__uint_as_float((uint32_t)e));
          const uint32_t flat = (uint32_t)(b_begin + 32 * (tj >> 4) + (ln & 31u)) * 256u + 32u * wave +
                                8u * ((tj & 15u) >> 2) + 4u * (ln >> 5) + (tj & 3u);
          reg[i] = ((uint64_t)key << 32) | flat;
          atomicAdd(&hist[(key - kmin) >> shift], 1u);
        }
        __syncthreads();
        // the bin holding the k-th: every wave scans the 256 bins (4 a lane)
        const uint4 h4 = reinterpret_cast<const uint4 *>(hist)[lane];
        const uint32_t hs = h4.x + h4.y + h4.z + h4.w;
        const uint32_t inc = wave_incl_scan_u32(hs), exc = inc - hs;
        const bool mine = exc < (uint32_t)k_sel && inc >= (uint32_t)k_sel;
        uint32_t bin = 0, below = exc, hb = h4.x;
        if (mine) {
          if (below + h4.x < (uint32_t)k_sel) {
            below += h4.x; bin = 1; hb = h4.y;
            if (below + h4.y < (uint32_t)k_sel) {
              below += h4.y; bin = 2; hb = h4.z;
              if (below + h4.z < (uint32_t)k_sel) { below += h4.z; bin = 3; hb = h4.w; }
            }
          }
        }
        const int src = (int)__builtin_ctzll(__builtin_amdgcn_ballot_w64(mine));
        const uint32_t bstar = 4u * (uint32_t)src + (uint32_t)__builtin_amdgcn_readlane((int)bin, src);
        const int L = __builtin_amdgcn_readlane((int)(below + hb), src);
        {
          done = true;
          uint64_t *list = sm.u.sel.u.list;
          for (int i0 = 0; i0 < (int)wc; i0 += 64) {
            const int i = i0 + lane;
            const uint64_t x = i < (int)wc ? reg[i] : ~0ull;
            const bool q = i < (int)wc && (((uint32_t)(x >> 32) - kmin) >> shift) <= bstar;
            const uint64_t m = __builtin_amdgcn_ballot_w64(q);
            if (m) {
              uint32_t base = 0;
              if (lane == 0) base = atomicAdd(&sm.n_final, (uint32_t)__builtin_popcountll(m));
              base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
              if (q) list[base + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u))] = x;
            }
          }
          __syncthreads();
          // all gathered keys lie in [kmin, the top of bin bstar]
          const uint64_t top = min((uint64_t)T, (uint64_t)kmin + ((uint64_t)(bstar + 1u) << shift) - 1ull);
          order_list<kNT>(sm.u.sel, L, k_sel, (uint64_t)kmin << 32, (top << 32) | 0xFFFFFFFFull);
        }
      }
    }
  }
  if (!done) {
    uint32_t key[16 * BT];
#pragma unroll
    for (int t = 0; t < BT; ++t)
#pragma unroll
      for (int j = 0; j < 16; ++j) key[16 * t + j] = valid[t] ? rank_key(acc[t][j]) : kInvalidKey;
    __syncthreads();                                    // the o buffers / staging area are no longer read
    select_regs<kNT, 16 * BT>(key, [&](int i) -> uint32_t { return flat_of(i >> 4, i & 15); }, n, k_sel, sm.u.sel);
  }
  emit_selection<kNT>(sm.u.sel, k_sel, r, grp, 256, p.score, p.token, p.parent, p.partial, p.n_groups, p.kk);
}

struct SP {
  const float *z, *prior;
  float *cand;
  float *score;
  int32_t *token, *parent;
  uint64_t *partial;
  int R, n_in, vocab, k, lsm, n_groups, kk;
};

struct ScoreSmem {
  SelectSmem<kNT> sel;
  float lse[kGroupBeams];
  float prior[kGroupBeams];                // vocab 256: the group's rows
};

// J register slots per thread: groups of kNT * J candidates (32768 or 8192).
template <int J>
__global__ __launch_bounds__(kNT) void score_select_kernel(SP p) {
  constexpr int GPOS = kNT * J;
  static_assert(GPOS / 256 <= kGroupBeams, "log-softmax rows per group");
  __shared__ ScoreSmem sm;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = blockIdx.x / p.n_groups, grp = blockIdx.x % p.n_groups;
  const int p0 = grp * GPOS;                              // first position of the group
  const long long total = (long long)p.n_in * p.vocab;
  const int n = (int)min((long long)GPOS, total - p0);
  const float *zr = p.z + (size_t)r * total;
  if (p.vocab == 256 && p.lsm) {
    const int nrows = n / 256;
    for (int row = wave; row < nrows; row += kNT / 64) {
      const float4 z = *(const float4 *)(zr + (size_t)p0 + row * 256 + lane * 4);
      const float mx = wave_max(fmaxf(fmaxf(z.x, z.y), fmaxf(z.z, z.w)));
      const float ml = mx * kLog2e;
      const float se = wave_sum(fast_exp2(fmaf(z.x, kLog2e, -ml)) + fast_exp2(fmaf(z.y, kLog2e, -ml)) +
                                fast_exp2(fmaf(z.z, kLog2e, -ml)) + fast_exp2(fmaf(z.w, kLog2e, -ml)));
      if (lane == 0) sm.lse[row] = mx + __builtin_amdgcn_logf(se) * kLn2;
    }
    __syncthreads();
  }
  // All loads before any candidate store (the compiler cannot know that the
  // output aliases no input): one memory latency for the J slots.  With 256
  // codes the priors of the group's rows come from LDS.
  if (p.vocab == 256 && p.prior) {
    for (int row = tid; row < (n + 255) / 256; row += kNT) sm.prior[row] = p.prior[(size_t)r * p.n_in + p0 / 256 + row];
    __syncthreads();
  }
  float zv[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int i = j * kNT + tid;
    zv[j] = i < n ? zr[p0 + i] : 0.f;
  }
  uint32_t key[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int i = j * kNT + tid;
    key[j] = kInvalidKey;
    if (i < n) {
      float v = zv[j];
      if (p.vocab == 256) {
        if (p.lsm) v -= sm.lse[i >> 8];
        if (p.prior) v += sm.prior[i >> 8];
      } else if (p.prior) {
        v += p.prior[(size_t)r * p.n_in + p0 + i];
      }
      key[j] = rank_key(v);
      if (p.cand) p.cand[(size_t)r * total + p0 + i] = v;
    }
  }
  auto idx_of = [&](int j) -> uint32_t { return (uint32_t)(p0 + j * kNT + tid); };
  const int k_sel = min(p.k, n);
  // a bucket of at most pow2(k) + 1 - k members keeps the list within pow2(k)
  select_regs<kNT, J>(key, idx_of, n, k_sel, sm.sel, max(pow2_ceil(k_sel) + 1 - k_sel, 16));
  emit_selection<kNT>(sm.sel, k_sel, r, grp, p.vocab, p.score, p.token, p.parent, p.partial, p.n_groups, p.kk);
}

// Final selection from n_groups sorted partial lists of kk composites each
// (ascending, padded with ~0): the k smallest of their union.  Composites are
// unique, so the output slot of an entry is its index in its own list plus,
// for every other list, the number of entries below it (one binary search in
// LDS each); entries whose slot falls below k are written directly.  Block
// (r, y) stages all lists of request r and ranks entries y*kMergeNT onwards,
// one per thread.
constexpr int kMergeNT = 1024;

__global__ __launch_bounds__(kMergeNT) void select_merge_kernel(const uint64_t *partial, int n_groups, int kk, int k,
                                                                int vocab, float *score, int32_t *token,
                                                                int32_t *parent) {
  extern __shared__ uint64_t lists[];              // n_groups * kk entries
  const int r = blockIdx.x, tid = threadIdx.x;
  const int n = n_groups * kk;
  const uint64_t *src = partial + (size_t)r * n;
  // all loads first (n <= kMergeCapacity = kMergeLoads * kMergeNT), then the
  // LDS stores: one memory latency rather than one per pass
  constexpr int kMergeLoads = kMergeCapacity / kMergeNT;
  uint64_t ld[kMergeLoads];
#pragma unroll
  for (int j = 0; j < kMergeLoads; ++j) {
    const int i = j * kMergeNT + tid;
    ld[j] = i < n ? src[i] : 0ull;
  }
#pragma unroll
  for (int j = 0; j < kMergeLoads; ++j) {
    const int i = j * kMergeNT + tid;
    if (i < n) lists[i] = ld[j];
  }
  __syncthreads();
  const int e = blockIdx.y * kMergeNT + tid;
  if (e >= n) return;
  const uint64_t x = lists[e];
  if (x == ~0ull) return;                          // group padding
  const int g = e / kk;
  int slot = e - g * kk;
  // entries of list g2 below x: a branch-free lower bound whose step count
  // does not depend on the data, four lists at a time so that their LDS
  // reads are in flight together (list g itself counts 0)
  for (int g0 = 0; g0 < n_groups && slot < k; g0 += 4) {
    int base[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) base[u] = 0;
    for (int len = kk; len > 1; len -= len >> 1) {
      const int half = len >> 1;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int g2 = min(g0 + u, n_groups - 1);
        base[u] = lists[g2 * kk + base[u] + half] < x ? base[u] + half : base[u];
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int g2 = g0 + u;
      if (g2 < n_groups && g2 != g) slot += base[u] + (lists[g2 * kk + base[u]] < x ? 1 : 0);
    }
  }
  if (slot < k) {
    const uint32_t f = (uint32_t)x;
    score[(size_t)r * k + slot] = key_score((uint32_t)(x >> 32));
    token[(size_t)r * k + slot] = (int32_t)(f % (uint32_t)vocab);
    parent[(size_t)r * k + slot] = (int32_t)(f / (uint32_t)vocab);
  }
}

// z[row][t] = sum_i o[row][i] W[t][i] (+ prior[row] for the scalar path).
__device__ __forceinline__ float ldv(const float *p, size_t i) { return p[i]; }
__device__ __forceinline__ float ldv(const uint16_t *p, size_t i) { return bf16_to_f32(p[i]); }

template <typename TO, typename TW>
__global__ __launch_bounds__(256) void project_kernel(const TO *o, const TW *W, const float *prior, float *z,
                                                      int rows, int D, int vocab, int add_prior) {
  if (vocab == 1) {
    // 16 lanes per row (one DPP row), 4 consecutive elements per lane and
    // step: a 16-lane group reads 256 contiguous bytes of fp32 o per step
    const int row = blockIdx.x * 16 + (threadIdx.x >> 4), l16 = threadIdx.x & 15;
    if (row >= rows) return;                      // whole 16-lane groups leave together
    float s = 0.f;
    for (int i = 4 * l16; i < D; i += 64) {
#pragma unroll
      for (int e = 0; e < 4; ++e) s = fmaf(ldv(o, (size_t)row * D + i + e), ldv(W, (size_t)(i + e)), s);
    }
    s += __uint_as_float(xor_lane<1>(__float_as_uint(s)));
    s += __uint_as_float(xor_lane<2>(__float_as_uint(s)));
    s += __uint_as_float(xor_lane<4>(__float_as_uint(s)));
    s += __uint_as_float(xor_lane<8>(__float_as_uint(s)));
    if (l16 == 0) z[row] = s + (add_prior && prior ? prior[row] : 0.f);
    return;
  }
  __shared__ float orow[4096];
  const int row = blockIdx.x;
  for (int i = threadIdx.x; i < D; i += 256) orow[i] = ldv(o, (size_t)row * D + i);
  __syncthreads();
  for (int t = threadIdx.x; t < vocab; t += 256) {
    float s = 0.f;
    for (int i = 0; i < D; ++i) s = fmaf(orow[i], ldv(W, (size_t)t * D + i), s);
    z[(size_t)row * vocab + t] = s;
  }
}

}  // namespace

hipError_t launch_logits_select_bf16(const LogitsArgs &a, const SelectOut &o, hipStream_t s) {
  LP p;
  p.o = a.o; p.W = a.W; p.prior = a.prior; p.cand = a.cand_out;
  p.score = o.score; p.token = o.token; p.parent = o.parent; p.partial = o.partial;
  p.R = a.R; p.n_in = a.n_in; p.D = a.D; p.hd_log2 = __builtin_ctz((unsigned)a.hd); p.k = a.k;
  p.lsm = a.log_softmax; p.n_groups = o.n_groups; p.kk = o.kk;
  const dim3 grid((unsigned)(a.R * o.n_groups));
  const bool half = o.gpos == kGroupPositions / 2 || a.n_in <= kGroupBeams / 2;   // groups of at most 64 beams
  if (a.D == 8 * kCB) {
    if (half) hipLaunchKernelGGL((logits_select_bf16_kernel<8, 2>), grid, dim3(kNT), 0, s, p);
    else hipLaunchKernelGGL((logits_select_bf16_kernel<8, 4>), grid, dim3(kNT), 0, s, p);
  } else if (a.D == 16 * kCB) {
    if (half) hipLaunchKernelGGL((logits_select_bf16_kernel<16, 2>), grid, dim3(kNT), 0, s, p);
    else hipLaunchKernelGGL((logits_select_bf16_kernel<16, 4>), grid, dim3(kNT), 0, s, p);
  } else {
    if (half) hipLaunchKernelGGL((logits_select_bf16_kernel<0, 2>), grid, dim3(kNT), 0, s, p);
    else hipLaunchKernelGGL((logits_select_bf16_kernel<0, 4>), grid, dim3(kNT), 0, s, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || o.n_groups == 1) return e;
  return launch_select_merge(o, a.R, a.k, 256, s);
}

hipError_t launch_score_select(const ScoreSelectArgs &a, const SelectOut &o, hipStream_t s) {
  SP p;
  p.z = a.logits; p.prior = a.prior; p.cand = a.cand_out;
  p.score = o.score; p.token = o.token; p.parent = o.parent; p.partial = o.partial;
  p.R = a.R; p.n_in = a.n_in; p.vocab = a.vocab; p.k = a.k; p.lsm = a.log_softmax;
  p.n_groups = o.n_groups; p.kk = o.kk;
  if (o.gpos == kSmallGroupPositions)
    hipLaunchKernelGGL(score_select_kernel<kSmallGroupPositions / kNT>, dim3((unsigned)(a.R * o.n_groups)), dim3(kNT),
                       0, s, p);
  else
    hipLaunchKernelGGL(score_select_kernel<kGroupPositions / kNT>, dim3((unsigned)(a.R * o.n_groups)), dim3(kNT), 0,
                       s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || o.n_groups == 1) return e;
  return launch_select_merge(o, a.R, a.k, a.vocab, s);
}

hipError_t launch_select_merge(const SelectOut &o, int R, int k, int vocab, hipStream_t s) {
  const int n = o.n_groups * o.kk;                 // <= kMergeCapacity (checked by the caller)
  const dim3 grid((unsigned)R, (unsigned)((n + kMergeNT - 1) / kMergeNT));
  hipLaunchKernelGGL(select_merge_kernel, grid, dim3(kMergeNT), (size_t)n * sizeof(uint64_t), s, o.partial,
                     o.n_groups, o.kk, k, vocab, o.score, o.token, o.parent);
  return hipGetLastError();
}

hipError_t launch_project(const ProjArgs &a, hipStream_t s) {
  const int rows = a.R * a.n;
  const dim3 grid(a.vocab == 1 ? (unsigned)((rows + 15) / 16) : (unsigned)rows);
  if (a.dtype == GR_F32) {
    hipLaunchKernelGGL((project_kernel<float, float>), grid, dim3(256), 0, s, (const float *)a.o,
                       (const float *)a.W, a.prior, a.z, rows, a.D, a.vocab, a.add_prior);
  } else {
    hipLaunchKernelGGL((project_kernel<float, uint16_t>), grid, dim3(256), 0, s, (const float *)a.o,
                       (const uint16_t *)a.W, a.prior, a.z, rows, a.D, a.vocab, a.add_prior);
  }
  return hipGetLastError();
}

}  // namespace gr
