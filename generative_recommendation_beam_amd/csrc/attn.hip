// Attention of every beam over the shared prompt plus its own ancestor chain.
//
// Per request r, beam b, head h (Engineering Exploration of Generative Recall,
// 4.1 attention steps, 4.4 tree-aware mask, 4.5 window; TransRetrieval,
// Hardware-aware inference optimization: one user cache for all candidates;
// OneLA, Abstract: shared prompt + append-only records + ancestry index):
//   keys = prompt rows [Lp-Lw, Lp) then the records on chain(beam_node[b]),
//   o[b][h*hd+i] = sum_j softmax_j(scale * q.k_j) v_j[i].
//
// bf16 path (gfx950 MFMA).  One workgroup per (request, head, group of NW x 32
// beams).  The prompt window of (r, h) streams from HBM straight into an
// NS-stage LDS ring (global_load_lds_dwordx4, no register staging) in tiles
// of 64 keys, NS-1 tiles in flight; every wave reuses each tile for its own
// 32 beams, so the prompt is read from HBM once per (request, head) and never
// copied per beam.  Scores are formed transposed, S^T = K Q^T (keys x beams),
// with v_mfma_f32_32x32x16_bf16: the accumulator holds one beam per lane
// column, so the softmax reductions are in-lane plus one lane^32 swap, and the
// probabilities are already the B operand of O^T += V^T P^T.  The V^T operand
// comes from the row-major V tile through ds_read_b64_tr_b16 (each 16-lane
// group reads a 4 key x 16 dim block transposed).  Each lane fetches its 16
// bytes from an XOR-permuted source address, so the dense LDS rows come out
// bank-swizzled for both the K reads and the transposed V reads.  The chain
// records are walked per lane through the parent array (pointer chasing, no
// mask tensor) and folded into the same online-softmax state.
//
// fp32 path: plain VALU kernel, one thread per beam, same semantics.

#include "gr_device.h"
#include "gr_launch.h"

namespace gr {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

typedef __attribute__((ext_vector_type(4))) short i16x4;

template <int I>
struct Stage {
  static constexpr int value = I;
};
#define GR_LDS(p) ((__attribute__((address_space(3))) void *)(p))
#define GR_LDS4(p) ((__attribute__((address_space(3))) i16x4 *)(p))

// s_waitcnt with only the vector-memory counter constrained to <= n.
#define GR_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))

struct AttnP {
  const uint16_t *pk, *pv, *q, *ak, *av;
  const int32_t *parent, *beam_node;
  float *out_f32;
  uint16_t *out_bf16;
  int32_t *dev_err;
  int R, H, Lp, Lw, nb, cap, max_depth, n_grp;
  float sl2;  // scale * log2(e)
};

template <int HD, int NW, int NS>
struct Geo {
  static constexpr int KT = 64;                 // keys per tile
  static constexpr int RB = HD * 2;             // bytes per tile row
  static constexpr int CPR = RB / 16;           // 16-byte chunks per row
  static constexpr int RPW = 128 / RB;          // rows per 128-byte bank window
  static constexpr int TB = KT * RB;            // bytes per tile (K or V)
  static constexpr int NBLK = TB / 1024;        // 1 KB DMA blocks per tile
  static constexpr int IPW = (NBLK + NW - 1) / NW;  // DMA blocks per wave (K or V)
  static constexpr int KSTEP = HD / 16;         // MFMA k-steps over the head dim
  static constexpr int DT = HD / 32;            // 32-row d tiles of O^T
};

// Bank swizzles (physical chunk = logical chunk ^ swizzle(row)).  K: the 8
// lanes of one b128 read cycle read 8 consecutive rows at one logical chunk.
// V: a 16-lane transposed read touches 4 consecutive rows (from a multiple of
// 4) x 2 adjacent chunks.
template <int HD>
__device__ __forceinline__ int swz_k(int row) {
  return HD == 64 ? (row & 7) : ((row >> 1) & 3);
}
template <int HD>
__device__ __forceinline__ int swz_v(int row) {
  return HD == 64 ? 2 * (row & 3) : 2 * ((row >> 1) & 1);
}

template <int HD, int NW, int NS>
__global__ __launch_bounds__(NW * 64) void attn_bf16_kernel(AttnP p) {
  using G = Geo<HD, NW, NS>;
  static_assert(NS >= 2 && NS <= 4, "ring depth");
  static_assert(G::NBLK % NW == 0, "every wave moves the same number of 1 KB blocks");
  // One LDS object per ring stage: the compiler then sees that a DMA into one
  // stage does not touch the stage being read, and adds no waits for it.
  __shared__ __attribute__((aligned(1024))) uint16_t K0[G::TB / 2], K1[G::TB / 2], K2[NS > 2 ? G::TB / 2 : 8],
      K3[NS > 3 ? G::TB / 2 : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t V0[G::TB / 2], V1[G::TB / 2], V2[NS > 2 ? G::TB / 2 : 8],
      V3[NS > 3 ? G::TB / 2 : 8];
  auto kst = [&](auto S) -> uint16_t * {
    constexpr int st = decltype(S)::value;
    if constexpr (st == 0) return K0;
    else if constexpr (st == 1) return K1;
    else if constexpr (st == 2) return K2;
    else return K3;
  };
  auto vst = [&](auto S) -> uint16_t * {
    constexpr int st = decltype(S)::value;
    if constexpr (st == 0) return V0;
    else if constexpr (st == 1) return V1;
    else if constexpr (st == 2) return V2;
    else return V3;
  };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, c = lane & 31;
  int bid = blockIdx.x;
  const int grp = bid % p.n_grp;
  bid /= p.n_grp;
  const int h = bid % p.H, r = bid / p.H;
  const int beam = (grp * NW + wave) * 32 + c;
  const bool valid = beam < p.nb;
  const size_t row = (size_t)p.H * HD;          // elements between tokens
  const uint16_t *pk = p.pk + (size_t)r * p.Lp * row + (size_t)h * HD;
  const uint16_t *pv = p.pv + (size_t)r * p.Lp * row + (size_t)h * HD;
  const int k_begin = p.Lp - p.Lw;
  const int n_tiles = (p.Lw + G::KT - 1) / G::KT;

  // DMA of one tile into ring stage `st`: wave w moves 1 KB blocks w*IPW..;
  // lane l lands at byte 16*l of its block; it fetches the logical chunk that
  // the swizzle assigns to that physical position.  Rows past the prompt end
  // read the last prompt row (their scores are masked to -inf).
  // per-lane tile row and (swizzled) element offsets of its DMA pieces
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
  const uint32_t row32 = (uint32_t)row;
  auto issue = [&](int tile, auto S) {
    const int key0 = k_begin + tile * G::KT;
#pragma unroll
    for (int i = 0; i < G::IPW; ++i) {
      const int blk = wave * G::IPW + i;
      const uint32_t src = (uint32_t)min(key0 + dma_row[i], p.Lp - 1) * row32;
      __builtin_amdgcn_global_load_lds((const void *)(pk + (src + dma_k[i])), GR_LDS(kst(S) + blk * 512), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void *)(pv + (src + dma_v[i])), GR_LDS(vst(S) + blk * 512), 16, 0, 0);
    }
  };
  // wait until this wave's DMAs of all but the `ahead` most recent tiles landed
  auto wait_tiles = [&](int ahead) {
    constexpr int per = 2 * G::IPW;
    if (ahead >= 3) GR_WAIT_VMCNT(3 * per);
    else if (ahead == 2) GR_WAIT_VMCNT(2 * per);
    else if (ahead == 1) GR_WAIT_VMCNT(per);
    else GR_WAIT_VMCNT(0);
  };

  // Query fragments (B operand of S^T): lane (g, c) holds beam c, head dims
  // (HD/2)*g + 8j .. +8 for k-step j.
  bf16x8 qf[G::KSTEP];
  const uint16_t *qp = p.q + ((size_t)r * p.nb + (valid ? beam : 0)) * row + (size_t)h * HD + (HD / 2) * g;
#pragma unroll
  for (int j = 0; j < G::KSTEP; ++j) {
    const uint4 raw = valid ? *(const uint4 *)(qp + 8 * j) : make_uint4(0, 0, 0, 0);
    qf[j] = __builtin_bit_cast(bf16x8, raw);
  }

  float m_run = -__builtin_inff(), l_run = 0.f;
  f32x16 O[G::DT];
#pragma unroll
  for (int t = 0; t < G::DT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) O[t][i] = 0.f;

  // ---- ancestor chain ids.  The parent links are chased before any prompt
  // DMA is issued: vector loads complete in issue order, so a link fetched
  // behind the prompt tiles would wait for all of them.
  int ids[GR_MAX_DEPTH];
  int cnt = 0;
#pragma unroll
  for (int d = 0; d < GR_MAX_DEPTH; ++d) ids[d] = -1;
  if (p.beam_node != nullptr) {
    int n = valid ? p.beam_node[(size_t)r * p.nb + beam] : -1;
    int err = 0;
    const int32_t *par = p.parent + (size_t)r * p.cap;
#pragma unroll
    for (int d = 0; d < GR_MAX_DEPTH; ++d) {
      if (n != -1) {
        if (n < 0 || n >= p.cap) {
          err |= GR_DEVERR_PARENT_RANGE; n = -1;
        } else if (d >= p.max_depth) {
          err |= GR_DEVERR_DEPTH; n = -1;
        } else {
          const int pn = par[n];
          ids[d] = n;
          cnt = d + 1;
          if (pn < -1 || pn >= p.cap) { err |= GR_DEVERR_PARENT_RANGE; n = -1; }
          else if (pn >= n) { err |= GR_DEVERR_PARENT_ORDER; n = -1; }
          else n = pn;
        }
      }
    }
    if (n != -1) err |= GR_DEVERR_DEPTH;
    if (err) atomicOr(p.dev_err, err);
  }

  // ---- chain records, CH at a time.  The first batch is requested together
  // with the prompt prologue.  Lanes past their chain read their own query
  // row instead (a cache hit, no extra HBM traffic).
  constexpr int CH = 4;
  const size_t qrow = ((size_t)r * p.nb + (valid ? beam : 0)) * row + (size_t)h * HD;
#pragma unroll
  for (int d0 = 0; d0 < GR_MAX_DEPTH; d0 += CH) {
    if (d0 == 0 || __ballot(cnt > d0)) {
      uint4 kr[CH][G::KSTEP];
      uint2 vr[CH][G::DT][4];
#pragma unroll
      for (int c4 = 0; c4 < CH; ++c4) {
        const int n = ids[d0 + c4];
        const uint16_t *kb = n >= 0 ? p.ak + ((size_t)r * p.cap + n) * row + (size_t)h * HD : p.q + qrow;
        const uint16_t *vb = n >= 0 ? p.av + ((size_t)r * p.cap + n) * row + (size_t)h * HD : p.q + qrow;
#pragma unroll
        for (int j = 0; j < G::KSTEP; ++j) kr[c4][j] = *(const uint4 *)(kb + (HD / 2) * g + 8 * j);
#pragma unroll
        for (int dt = 0; dt < G::DT; ++dt)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) vr[c4][dt][q4] = *(const uint2 *)(vb + 32 * dt + 8 * q4 + 4 * g);
      }
      if (d0 == 0) {
        // prologue: tiles 0 .. NS-2 in flight, issued without a branch (a
        // tile past the window reads the last prompt row and is never used;
        // the first tile's wait covers it).
        issue(0, Stage<0>{});
        if constexpr (NS > 2) issue(1, Stage<1>{});
        if constexpr (NS > 3) issue(2, Stage<2>{});
        // keep the whole prologue ahead of the first wait for the records
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int c4 = 0; c4 < CH; ++c4) {
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < G::KSTEP; ++j) s += dot8_bf16(__builtin_bit_cast(uint4, qf[j]), kr[c4][j]);
        s = xor32_sum(s);
        if (d0 + c4 < cnt) {
          const float t = s * p.sl2;
          const float m_new = fmaxf(m_run, t);
          const float alpha = fast_exp2(m_run - m_new);
          const float pr = fast_exp2(t - m_new);
          l_run = l_run * alpha + (g == 0 ? pr : 0.f);
#pragma unroll
          for (int dt = 0; dt < G::DT; ++dt)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const uint2 vv = vr[c4][dt][q4];
              O[dt][4 * q4 + 0] = fmaf(pr, bf16_lo(vv.x), O[dt][4 * q4 + 0] * alpha);
              O[dt][4 * q4 + 1] = fmaf(pr, bf16_hi(vv.x), O[dt][4 * q4 + 1] * alpha);
              O[dt][4 * q4 + 2] = fmaf(pr, bf16_lo(vv.y), O[dt][4 * q4 + 2] * alpha);
              O[dt][4 * q4 + 3] = fmaf(pr, bf16_hi(vv.y), O[dt][4 * q4 + 3] * alpha);
            }
          m_run = m_new;
        }
      }
    }
  }

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

  // ---- shared prompt window through the LDS ring
  auto step = [&](int t0, auto S) {
    constexpr int st = decltype(S)::value;
    const int tile = t0 + st;
    if (tile < n_tiles) {
        wait_tiles(min(NS - 2, n_tiles - 1 - tile));
        __builtin_amdgcn_s_barrier();
        // every wave is past tile-1: its stage can be refilled
        if (tile + NS - 1 < n_tiles) issue(tile + NS - 1, Stage<(st + NS - 1) % NS>{});
        const char *kb = (const char *)kst(S);
        const char *vb = (const char *)vst(S);

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
        float mx = __builtin_elementwise_maximum(S0[0], S1[0]);
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(S0[i], S1[i]));
        mx = xor32_max(mx) * p.sl2;
        // Exact running max: the key that sets it gets weight exactly 1, which
        // bf16 holds exactly (it dominates a peaked softmax).  The rescale is
        // skipped only when no lane's max grew (then alpha would be 1).
        if (__ballot(mx > m_run)) {
          const float m_new = fmaxf(m_run, mx);
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
    }
  };
  for (int t0 = 0; t0 < n_tiles; t0 += NS) {
    step(t0, Stage<0>{});
    step(t0, Stage<1>{});
    if constexpr (NS > 2) step(t0, Stage<2>{});
    if constexpr (NS > 3) step(t0, Stage<3>{});
  }

  const float l_tot = xor32_sum(l_run);
  if (!valid) return;
  const float inv = 1.f / l_tot;
  const size_t obase = ((size_t)r * p.nb + beam) * row + (size_t)h * HD;
#pragma unroll
  for (int dt = 0; dt < G::DT; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = 32 * dt + 8 * q4 + 4 * g;
      const float o0 = O[dt][4 * q4] * inv, o1 = O[dt][4 * q4 + 1] * inv;
      const float o2 = O[dt][4 * q4 + 2] * inv, o3 = O[dt][4 * q4 + 3] * inv;
      if (p.out_f32) *(float4 *)(p.out_f32 + obase + d0) = make_float4(o0, o1, o2, o3);
      if (p.out_bf16) *(uint2 *)(p.out_bf16 + obase + d0) = make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
    }
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

template <int HD, int NW, int NS>
hipError_t launch_bf16(const AttnArgs &a, hipStream_t s) {
  AttnP p;
  p.pk = (const uint16_t *)a.pk; p.pv = (const uint16_t *)a.pv; p.q = (const uint16_t *)a.q;
  p.ak = (const uint16_t *)a.ak; p.av = (const uint16_t *)a.av;
  p.parent = a.parent; p.beam_node = a.beam_node;
  p.out_f32 = a.out_f32; p.out_bf16 = (uint16_t *)a.out_lowp; p.dev_err = a.dev_err;
  p.R = a.R; p.H = a.H; p.Lp = a.Lp; p.Lw = a.Lw; p.nb = a.nb; p.cap = a.cap;
  p.max_depth = a.max_depth;
  const int nblk = (a.nb + 31) / 32;
  p.n_grp = (nblk + NW - 1) / NW;
  p.sl2 = a.scale * kLog2e;
  const long long grid = (long long)a.R * a.H * p.n_grp;
  hipLaunchKernelGGL((attn_bf16_kernel<HD, NW, NS>), dim3((unsigned)grid), dim3(NW * 64), 0, s, p);
  return hipGetLastError();
}

template <int HD>
hipError_t launch_bf16_nw(const AttnArgs &a, hipStream_t s) {
  const int nblk = (a.nb + 31) / 32;
  constexpr int NS = 4;
  if (nblk <= 1) return launch_bf16<HD, 1, NS>(a, s);
  if (nblk == 2) return launch_bf16<HD, 2, NS>(a, s);
  return launch_bf16<HD, 4, NS>(a, s);
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
