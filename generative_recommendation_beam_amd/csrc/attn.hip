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
// beams).  The prompt window of (r, h) streams through LDS in tiles of 64
// keys; every wave of the workgroup reuses each tile for its own 32 beams, so
// the prompt is read from HBM once per (request, head) and never copied per
// beam.  Scores are formed transposed, S^T = K Q^T (keys x beams), with
// v_mfma_f32_32x32x16_bf16: the accumulator then holds one beam per lane
// column, so the softmax row reductions are in-lane plus one lane^32 swap, and
// the probabilities are already in the B-operand layout of O^T += V^T P^T.
// V is written to LDS transposed (d-major) with a key permutation that matches
// the S^T accumulator order.  The chain records are walked per lane through the
// parent array (pointer chasing, no mask tensor) and folded into the same
// online-softmax state before the prompt tiles.
//
// fp32 path: plain VALU kernel, one thread per beam, same semantics.

#include "gr_device.h"
#include "gr_launch.h"

namespace gr {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

struct AttnP {
  const uint16_t *pk, *pv, *q, *ak, *av;
  const int32_t *parent, *beam_node;
  float *out_f32;
  uint16_t *out_bf16;
  int32_t *dev_err;
  int R, H, Lp, Lw, nb, cap, max_depth, n_grp;
  float sl2;  // scale * log2(e)
};

// Position of tile key kk in the transposed V tile: inside each group of 16
// keys the order is (lane group, half, 4 keys) so that a lane's 8 B-operand
// elements of one MFMA k-step are 8 contiguous bf16.
__device__ __forceinline__ int vt_pos(int kk) {
  const int t = kk >> 4, w = kk & 15;
  return (t << 4) + (((w >> 2) & 1) << 3) + ((w >> 3) << 2) + (w & 3);
}

template <int HD, int NW>
struct Geo {
  static constexpr int KT = 64;                 // keys per tile
  static constexpr int NT = NW * 64;            // threads
  static constexpr int KS = HD + 8;             // K tile row stride (bf16), 16 B pad
  static constexpr int VS = KT + 8;             // V^T tile row stride (bf16), 144 B
  static constexpr int CPR = HD / 8;            // 16-byte chunks per row
  static constexpr int NCH = KT * CPR;          // chunks per tile (K or V)
  static constexpr int CPT = (NCH + NT - 1) / NT;
  static constexpr int KSTEP = HD / 16;         // MFMA k-steps over the head dim
  static constexpr int DT = HD / 32;            // 32-row d tiles of O^T
};

template <int HD, int NW>
__global__ __launch_bounds__(NW * 64) void attn_bf16_kernel(AttnP p) {
  using G = Geo<HD, NW>;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][G::KT * G::KS];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][HD * G::VS];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
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

  uint4 kreg[G::CPT], vreg[G::CPT];
  auto load_tile = [&](int tile) {
#pragma unroll
    for (int i = 0; i < G::CPT; ++i) {
      const int ch = tid + i * G::NT;
      if (G::NCH % G::NT == 0 || ch < G::NCH) {
        const int kk = ch / G::CPR, dc = ch % G::CPR;
        const int key = k_begin + tile * G::KT + kk;
        if (key < p.Lp) {
          kreg[i] = *(const uint4 *)(pk + (size_t)key * row + dc * 8);
          vreg[i] = *(const uint4 *)(pv + (size_t)key * row + dc * 8);
        } else {
          kreg[i] = make_uint4(0, 0, 0, 0);
          vreg[i] = make_uint4(0, 0, 0, 0);
        }
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < G::CPT; ++i) {
      const int ch = tid + i * G::NT;
      if (G::NCH % G::NT == 0 || ch < G::NCH) {
        const int kk = ch / G::CPR, dc = ch % G::CPR;
        *(uint4 *)&Ks[buf][kk * G::KS + dc * 8] = kreg[i];
        const int pos = vt_pos(kk);
        // 16-byte chunk index of this key inside a V^T row, XOR-swizzled by
        // the row's d/8 so that rows 8 apart land in different banks.
        const int phys = (((pos >> 3) ^ (dc & 7)) << 3) + (pos & 7);
        const uint32_t w[4] = {vreg[i].x, vreg[i].y, vreg[i].z, vreg[i].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint16_t val = (e & 1) ? (uint16_t)(w[e >> 1] >> 16) : (uint16_t)(w[e >> 1] & 0xFFFFu);
          Vt[buf][(dc * 8 + e) * G::VS + phys] = val;
        }
      }
    }
  };

  load_tile(0);

  // Query fragments (B operand of S^T): lane (g, c) holds beam c, head dims
  // (HD/2)*g + 8j .. +8 for k-step j.
  bf16x8 qf[G::KSTEP];
  uint4 qraw[G::KSTEP];
  const uint16_t *qp = p.q + ((size_t)r * p.nb + (valid ? beam : 0)) * row + (size_t)h * HD + (HD / 2) * g;
#pragma unroll
  for (int j = 0; j < G::KSTEP; ++j) {
    qraw[j] = valid ? *(const uint4 *)(qp + 8 * j) : make_uint4(0, 0, 0, 0);
    qf[j] = __builtin_bit_cast(bf16x8, qraw[j]);
  }

  float m_run = -__builtin_inff(), l_run = 0.f;
  f32x16 O[G::DT];
#pragma unroll
  for (int t = 0; t < G::DT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) O[t][i] = 0.f;

  // ---- ancestor chain: walk parent ids from the beam's own record upward.
  if (p.beam_node != nullptr) {
    int n = valid ? p.beam_node[(size_t)r * p.nb + beam] : -1;
    int err = 0;
    const int32_t *par = p.parent + (size_t)r * p.cap;
    for (int depth = 0; n != -1; ++depth) {
      if (n < 0 || n >= p.cap) { err |= GR_DEVERR_PARENT_RANGE; break; }
      if (depth >= p.max_depth) { err |= GR_DEVERR_DEPTH; break; }
      const int pn = par[n];
      const size_t rec = ((size_t)r * p.cap + n) * row + (size_t)h * HD;
      const uint16_t *kn = p.ak + rec + (HD / 2) * g;
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < G::KSTEP; ++j) s += dot8_bf16(qraw[j], *(const uint4 *)(kn + 8 * j));
      s += __shfl_xor(s, 32);
      const float t = s * p.sl2;
      const float m_new = fmaxf(m_run, t);
      const float alpha = fast_exp2(m_run - m_new);
      const float pr = fast_exp2(t - m_new);
      l_run = l_run * alpha + (g == 0 ? pr : 0.f);
      const uint16_t *vn = p.av + rec;
#pragma unroll
      for (int dt = 0; dt < G::DT; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const uint2 vv = *(const uint2 *)(vn + 32 * dt + 8 * q4 + 4 * g);
          O[dt][4 * q4 + 0] = fmaf(pr, bf16_lo(vv.x), O[dt][4 * q4 + 0] * alpha);
          O[dt][4 * q4 + 1] = fmaf(pr, bf16_hi(vv.x), O[dt][4 * q4 + 1] * alpha);
          O[dt][4 * q4 + 2] = fmaf(pr, bf16_lo(vv.y), O[dt][4 * q4 + 2] * alpha);
          O[dt][4 * q4 + 3] = fmaf(pr, bf16_hi(vv.y), O[dt][4 * q4 + 3] * alpha);
        }
      m_run = m_new;
      if (pn < -1 || pn >= p.cap) { err |= GR_DEVERR_PARENT_RANGE; break; }
      if (pn >= n) { err |= GR_DEVERR_PARENT_ORDER; break; }
      n = pn;
    }
    if (err) atomicOr(p.dev_err, err);
  }

  // ---- shared prompt window, tile by tile.
  store_tile(0);
  __syncthreads();
  for (int tile = 0; tile < n_tiles; ++tile) {
    const int buf = tile & 1;
    if (tile + 1 < n_tiles) load_tile(tile + 1);

    f32x16 S0, S1;
#pragma unroll
    for (int i = 0; i < 16; ++i) { S0[i] = 0.f; S1[i] = 0.f; }
#pragma unroll
    for (int j = 0; j < G::KSTEP; ++j) {
      const bf16x8 a0 = *(const bf16x8 *)&Ks[buf][c * G::KS + (HD / 2) * g + 8 * j];
      const bf16x8 a1 = *(const bf16x8 *)&Ks[buf][(32 + c) * G::KS + (HD / 2) * g + 8 * j];
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
    float mx = fmaxf(S0[0], S1[0]);
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, fmaxf(S0[i], S1[i]));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * p.sl2);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    float ls = 0.f;
    uint32_t pw[16];
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const float e0 = fast_exp2(fmaf(S0[i], p.sl2, -m_new));
      const float e1 = fast_exp2(fmaf(S0[i + 1], p.sl2, -m_new));
      const float f0 = fast_exp2(fmaf(S1[i], p.sl2, -m_new));
      const float f1 = fast_exp2(fmaf(S1[i + 1], p.sl2, -m_new));
      ls += (e0 + e1) + (f0 + f1);
      pw[i >> 1] = pack_bf16x2(e0, e1);
      pw[8 + (i >> 1)] = pack_bf16x2(f0, f1);
    }
    l_run = l_run * alpha + ls;
#pragma unroll
    for (int dt = 0; dt < G::DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) O[dt][i] *= alpha;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint4 pk4 = make_uint4(pw[4 * t], pw[4 * t + 1], pw[4 * t + 2], pw[4 * t + 3]);
      const bf16x8 pf = __builtin_bit_cast(bf16x8, pk4);
#pragma unroll
      for (int dt = 0; dt < G::DT; ++dt) {
        const int d = 32 * dt + c;
        const int phys = ((2 * t + g) ^ ((d >> 3) & 7)) << 3;
        const bf16x8 a = *(const bf16x8 *)&Vt[buf][d * G::VS + phys];
        O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf, O[dt], 0, 0, 0);
      }
    }
    if (tile + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
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

template <int HD, int NW>
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
  hipLaunchKernelGGL((attn_bf16_kernel<HD, NW>), dim3((unsigned)grid), dim3(NW * 64), 0, s, p);
  return hipGetLastError();
}

template <int HD>
hipError_t launch_bf16_nw(const AttnArgs &a, hipStream_t s) {
  const int nblk = (a.nb + 31) / 32;
  if (nblk <= 1) return launch_bf16<HD, 1>(a, s);
  if (nblk == 2) return launch_bf16<HD, 2>(a, s);
  return launch_bf16<HD, 4>(a, s);
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
