// Codebook scoring, log-softmax, prior add and exact top-k of the decode step.
//
// Engineering Exploration of Generative Recall, 4.2 Custom Beam Search: only
// the 256 codes of the current semantic-ID level are scored and ranked; the
// candidate score is the running beam score plus the code's log-probability
// and the best B of B_in x 256 survive.  TransRetrieval, GPU retrieval:
// candidate selection runs on the device, next to scoring.
//
// logits_select_bf16: one workgroup (8 waves) per (request, group of <= 128
// beams).  z^T = W o^T on v_mfma_f32_32x32x16_bf16 (codes x beams; wave w owns
// beams 32*(w/2).. and codes 128*(w%2)..).  W and o stream HBM/L2 -> LDS
// through a ring of 32-column chunks (global_load_lds, several chunks in
// flight, each read once per workgroup).  Each lane then holds 64 codes of one
// beam in registers: the log-softmax is in-lane plus one lane^32 swap and one
// LDS exchange between the two code halves.  The selection first bounds the
// k-th best score from lane minima and stages only the lanes that can reach
// the bound, then runs the exact selection (gr_select.h) on the staged
// candidates (on all registers when the bound prunes too little); scores never
// leave the chip unless the caller asks for them.
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
constexpr int kOC = 32;                    // D columns per ring chunk (two MFMA k-steps)
constexpr int kRS = 6;                     // ring stages (5 chunks in flight)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// One ring stage: a 32-column chunk of W (256 code rows) and of o (128 beam
// rows), 64-byte rows whose 16-byte chunks are XOR-swizzled so that 16
// consecutive rows read at one logical chunk hit 16 distinct 16-byte slots of
// a 256-byte bank row (and any 8 of them distinct slots of a 128-byte one).
struct LogitsStage {
  uint16_t w[256 * kOC];                   // 16 KB
  uint16_t o[kGroupBeams * kOC];           // 8 KB
};
struct LogitsSmem {
  union {
    LogitsStage ring[kRS];                 // projection
    SelectSmem<kNT> sel;                   // selection afterwards
  } u;
  float red_max[4][2][32];
  float red_sum[4][2][32];
  uint32_t bound[kNT / 64];                // per-wave bound keys of the fast selection
  uint32_t fast_cnt[kNT / 64];             // per-wave counts of staged lanes
};
// Fast selection: at most 8 staged candidates per thread, staged (scores
// and the row bases of their lanes) in the then idle ring.
constexpr int kFastList = 8 * kNT;
static_assert(sizeof(LogitsStage) * kRS >= (sizeof(float) + sizeof(uint32_t)) * kFastList, "staging area");

struct LP {
  const uint16_t *o, *W;
  const float *prior;
  float *cand;
  float *score;
  int32_t *token, *parent;
  uint64_t *partial;
  int R, n_in, D, hd_log2, k, lsm, n_groups, kk;
};

__device__ __forceinline__ int swz64(int row) { return ((row >> 1) & 3) ^ ((row >> 3) & 1); }

__global__ __launch_bounds__(kNT) void logits_select_bf16_kernel(LP p) {
  __shared__ LogitsSmem sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, c = lane & 31;
  const int r = blockIdx.x / p.n_groups, grp = blockIdx.x % p.n_groups;
  const int b_begin = grp * kGroupBeams;
  const int nbg = min(kGroupBeams, p.n_in - b_begin);
  const int bb = wave >> 1, ch = wave & 1;
  const int bl = bb * 32 + c;
  const bool valid = bl < nbg;
  const int beam = b_begin + bl;
  const int n_chunks = p.D / kOC;

  // ---- z^T = W o^T, W and o streamed HBM/L2 -> LDS through the ring.  A
  // 1 KB DMA block is 16 rows x 64 B; lane l fetches row l/4 of its block at
  // the logical chunk that the swizzle puts at physical chunk l%4.  Wave w
  // moves W blocks 2w, 2w+1 and o block w of every chunk (3 DMAs per chunk).
  // Chunks past the end re-read the last one (never used), so every step
  // has the same number of chunks in flight.
  // o is head-major ([R][H][n_in][hd]); a 32-column chunk lies inside one head.
  const int drow = lane >> 2, dpc = lane & 3;
  const int hd = 1 << p.hd_log2, H = p.D >> p.hd_log2;
  const uint16_t *o_req = p.o + (size_t)r * H * p.n_in * hd;
  auto issue = [&](int chunk, int st) {
    const int col0 = min(chunk, n_chunks - 1) * kOC;
    const int hc = col0 >> p.hd_log2, c_in = col0 & (hd - 1);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int blk = wave * 2 + i, row = blk * 16 + drow;
      const int lc = dpc ^ swz64(row);
      dma16(p.W + (size_t)row * p.D + col0 + lc * 8, &sm.u.ring[st].w[blk * 512]);
    }
    {
      const int row = wave * 16 + drow, lc = dpc ^ swz64(row);
      const int b = min(b_begin + row, p.n_in - 1);
      dma16(o_req + ((size_t)hc * p.n_in + b) * hd + c_in + lc * 8, &sm.u.ring[st].o[wave * 512]);
    }
  };
  // per-lane LDS element offsets of the operand reads (logical chunk 2kk+g)
  const int sw = swz64(c);                  // rows bl and ch*128+32m+c share bits 1..3 with c
  int aoff[4][2], boff[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    boff[kk] = bl * kOC + (((2 * kk + g) ^ sw) << 3);
#pragma unroll
    for (int m = 0; m < 4; ++m) aoff[m][kk] = (ch * 128 + 32 * m + c) * kOC + (((2 * kk + g) ^ sw) << 3);
  }

  f32x16 acc[4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[m][i] = 0.f;

  // Operands of chunk c+1 are read from LDS into registers while the MFMAs
  // of chunk c run, so LDS reads, DMA fills and MFMAs overlap.
  bf16x8 opa[2][2][4], opb[2][2];
  auto read_ops = [&](int chunk, int buf) {
    const LogitsStage &S = sm.u.ring[chunk % kRS];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      opb[buf][kk] = *(const bf16x8 *)&S.o[boff[kk]];
#pragma unroll
      for (int m = 0; m < 4; ++m) opa[buf][kk][m] = *(const bf16x8 *)&S.w[aoff[m][kk]];
    }
  };
  auto mfma_ops = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int m = 0; m < 4; ++m)
        acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opa[buf][kk][m], opb[buf][kk], acc[m], 0, 0, 0);
  };
#pragma unroll
  for (int c0 = 0; c0 < kRS - 1; ++c0) issue(c0, c0);
  GR_WAIT_VMCNT(3 * (kRS - 2));             // this wave's pieces of chunk 0 landed
  ring_barrier();                           // everyone's
  read_ops(0, 0);
  // Iteration c: chunk c+1 must have landed (chunks c+2 .. c+kRS-2 may still
  // be in flight); after the barrier every wave has consumed chunk c-1, whose
  // stage receives chunk c+kRS-1.  The loop runs in pairs so that the two
  // register buffers are fixed; an odd last chunk leaves after the first half.
  for (int chunk = 0; chunk < n_chunks; chunk += 2) {
    GR_WAIT_VMCNT(3 * (kRS - 3));
    ring_barrier();
    issue(chunk + kRS - 1, (chunk + kRS - 1) % kRS);
    read_ops(chunk + 1, 1);                 // past the end: a landed re-read, unused
    mfma_ops(0);
    if (chunk + 1 == n_chunks) break;
    GR_WAIT_VMCNT(3 * (kRS - 3));
    ring_barrier();
    issue(chunk + kRS, (chunk + kRS) % kRS);
    read_ops(chunk + 2, 0);
    mfma_ops(1);
  }
  GR_WAIT_VMCNT(0);                         // the trailing re-reads landed
  ring_barrier();                           // before the LDS is reused

  // log-softmax over the 256 codes of each beam (two waves hold its halves)
  float lse = 0.f;
  float amax = acc[0][0];                   // this lane's largest logit
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, acc[m][i]);
  if (p.lsm) {
    const float mx = fmaxf(amax, __shfl_xor(amax, 32));
    if (lane < 32) sm.red_max[bb][ch][c] = mx;
    __syncthreads();
    const float M = fmaxf(sm.red_max[bb][0][c], sm.red_max[bb][1][c]);
    const float Ml = M * kLog2e;
    float se = 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int i = 0; i < 16; ++i) se += fast_exp2(fmaf(acc[m][i], kLog2e, -Ml));
    se += __shfl_xor(se, 32);
    if (lane < 32) sm.red_sum[bb][ch][c] = se;
    __syncthreads();
    lse = M + __builtin_amdgcn_logf(sm.red_sum[bb][0][c] + sm.red_sum[bb][1][c]) * kLn2;
  }

  // ---- selection.  Candidate score of register slot j = 16 m + 4 q4 + e:
  // (acc[m][4 q4 + e] - lse) + prior.  Each lane holds 64 candidates of one
  // beam, or none.
  const float pr = (valid && p.prior) ? p.prior[(size_t)r * p.n_in + beam] : 0.f;
  float *crow = (valid && p.cand) ? p.cand + ((size_t)r * p.n_in + beam) * 256 : nullptr;
  const uint32_t row_base = (uint32_t)beam * 256u + ch * 128 + 4 * g;
  auto idx_of = [&](int j) -> uint32_t {
    return row_base + 32u * (uint32_t)(j >> 4) + 8u * (uint32_t)((j >> 2) & 3) + (uint32_t)(j & 3);
  };
  const int n = nbg * 256;
  const int k_sel = min(p.k, n);

  // Fast path.  If ml = ceil(k/64) lanes of one wave have no score below s,
  // at least k candidates score >= s, so the k best all do.  s is the ml-th
  // largest lane minimum of a wave (the largest such bound over the waves;
  // lane extremes come from those of acc, the score being monotonic in it).
  // Only lanes whose maximum reaches s can hold a selected candidate: they
  // stage their 64 scores in LDS, and the exact selection runs over the
  // staged candidates, 8 per thread.  If too many lanes qualify, or the bound
  // is degenerate, it runs over all 64 register slots.  Every decision is
  // block-uniform.
  bool cand_done = false, fast = false;
  {
    float amin = acc[0][0];
    bool nan_in = false;                                // fminf / fmaxf skip NaN
    if (p.lsm) {
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < 16; ++i) amin = fminf(amin, acc[m][i]);
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          amin = fminf(amin, acc[m][i]);
          nan_in = nan_in || acc[m][i] != acc[m][i];
        }
    }
    // A lane with a NaN score (which ranks like -inf) bounds nothing.  With
    // the log-softmax a NaN logit makes every score of its beam NaN, and so
    // the lane minimum too.
    const float lmin = nan_in ? -__builtin_inff() : (amin - lse) + pr, lmax = (amax - lse) + pr;
    const uint32_t wkey = valid ? rank_key(lmin) : kInvalidKey;
    const int ml = (k_sel + 63) >> 6;
    uint32_t tw;                                        // ml-th smallest lane-minimum key of the wave
    if (ml <= 2) {
      tw = wave_small2_u32(wkey, ml);
    } else {
      uint64_t wv[1] = {((uint64_t)wkey << 32) | (uint32_t)lane};
      wave_bitonic_sort_u64<1>(wv);                     // ascending keys: best lane minima first
      tw = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(wv[0] >> 32), ml - 1);
    }
    if (lane == 0) sm.bound[wave] = tw;
    __syncthreads();
    uint32_t T = sm.bound[0];
#pragma unroll
    for (int w = 1; w < kNT / 64; ++w) T = min(T, sm.bound[w]);
    const float Ts = key_score(T);
    if (T != kInvalidKey && Ts > -__builtin_inff()) {
      const bool has = valid && lmax >= Ts;
      const uint64_t hm = __builtin_amdgcn_ballot_w64(has);
      if (lane == 0) sm.fast_cnt[wave] = (uint32_t)__builtin_popcountll(hm);
      __syncthreads();
      int n_st = 0, base_w = 0;
#pragma unroll
      for (int w = 0; w < kNT / 64; ++w) {
        base_w += w < wave ? (int)sm.fast_cnt[w] : 0;
        n_st += (int)sm.fast_cnt[w];
      }
      const int S = n_st * 64;                           // staged candidates
      if (S <= kFastList) {
        fast = true;
        cand_done = true;
        float *st_v = reinterpret_cast<float *>(&sm.u.ring[0]);     // [n_st][64] scores
        uint32_t *st_row = reinterpret_cast<uint32_t *>(st_v + kFastList);   // [n_st] row bases
        const int s_idx = base_w + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(hm >> 32),
                                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)hm, 0u));
        if (has || crow) {
#pragma unroll
          for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              float v[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = (acc[m][4 * q4 + e] - lse) + pr;
              const float4 v4 = make_float4(v[0], v[1], v[2], v[3]);
              if (crow) *(float4 *)(crow + ch * 128 + 32 * m + 8 * q4 + 4 * g) = v4;
              if (has) *(float4 *)(st_v + s_idx * 64 + 16 * m + 4 * q4) = v4;
            }
          if (has) st_row[s_idx] = row_base;
        }
        __syncthreads();
        // a bucket of at most pow2(k) + 1 - k members keeps the list within pow2(k)
        const int cap = max(pow2_ceil(k_sel) + 1 - k_sel, 16);
        // staged candidate t -> (key, flat index), NJ per thread (t = i kNT + tid)
        auto select_staged = [&](auto nj) {
          constexpr int NJ = decltype(nj)::value;
          uint32_t keyj[NJ], idxj[NJ];
#pragma unroll
          for (int i = 0; i < NJ; ++i) {
            const int t = i * kNT + tid, sl = t >> 6, j = t & 63;
            keyj[i] = kInvalidKey;
            idxj[i] = 0u;
            if (t < S) {
              keyj[i] = rank_key(st_v[t]);
              idxj[i] = st_row[sl] + 32u * (uint32_t)(j >> 4) + 8u * (uint32_t)((j >> 2) & 3) + (uint32_t)(j & 3);
            }
          }
          __syncthreads();                                 // the staging area overlaps the selection state
          select_regs<kNT, NJ>(keyj, [&](int i) -> uint32_t { return idxj[i]; }, S, k_sel, sm.u.sel, cap);
        };
        if (S <= kNT) select_staged(std::integral_constant<int, 1>{});
        else select_staged(std::integral_constant<int, kFastList / kNT>{});
      }
    }
  }
  if (!fast) {
    uint32_t key[64];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = (acc[m][4 * q4 + e] - lse) + pr;
          key[16 * m + 4 * q4 + e] = valid ? rank_key(v[e]) : kInvalidKey;
        }
        if (crow && !cand_done)
          *(float4 *)(crow + ch * 128 + 32 * m + 8 * q4 + 4 * g) = make_float4(v[0], v[1], v[2], v[3]);
      }
    __syncthreads();                                       // survivor regions may still be read
    select_regs<kNT, 64>(key, idx_of, n, k_sel, sm.u.sel);
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
  hipLaunchKernelGGL(logits_select_bf16_kernel, dim3((unsigned)(a.R * o.n_groups)), dim3(kNT), 0, s, p);
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
