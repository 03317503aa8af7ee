// Linear-attention decoding over one shared prompt state (OneLA, Abstract).
//
// With recurrent linear attention a beam's state is the sum of phi(k) v^T over
// its history.  Every beam of a request shares the prompt, so its state is
// one shared prompt-derived state plus the terms of its own append-only
// records, found through the ancestry index; a step computes only what it
// needs from them and never builds a per-beam state:
//   S_p = sum_{prompt window} phi(k) v^T,   z_p = sum_{prompt window} phi(k)
//   o_b = (phi(q)^T S_p + sum_{n in chain(b)} (phi(q).phi(k_n)) v_n)
//       / (phi(q).z_p  + sum_{n in chain(b)}  phi(q).phi(k_n))
// with phi(x) = elu(x) + 1 (positive, so the normaliser never vanishes).
//
// linear_state_bf16_kernel computes S_p, z_p once per (request, head):
// Phi(K)^T V over the window is a dense contraction and runs on MFMA.
// linear_attn_bf16_kernel reads S_p once per (request, head, 128 beams) into
// LDS; phi(Q) S_p for the 128 beams is again a dense contraction (MFMA), and
// each lane then folds its beam's chain records in fp32.  fp32 workloads use
// VALU kernels throughout.  The scoring and selection after it are those of
// the softmax step.

#include "gr_device.h"
#include "gr_launch.h"

namespace gr {
namespace {

__device__ __forceinline__ float phi(float x) { return x > 0.f ? x + 1.f : __expf(x); }

struct StateP {
  const void *pk, *pv;
  float *S, *z;
  int R, H, Lp, Lw;
};

// One workgroup of 4 waves per (request, head), 64-key tiles through a
// double-buffered LDS stage.  Wave w owns the 32 x 32 output tile
// (d_k half w >> 1, d_v half w & 1) of S (for head dim 32 only wave 0 has a
// tile).  A operand: phi(K)^T (row = d_k, k = key), split into two bf16
// terms hi + lo (hi = phi rounded to bf16, lo = the rest rounded again) that
// go through two MFMAs, so phi keeps about 16 mantissa bits instead of 8;
// B operand: V (k = key, column = d_v), exact in bf16.  Lane (g, c) of an
// MFMA k-step holds keys 8g .. 8g+7 of column c for both, read as single
// bf16 elements.  z sums phi in fp32.
// Tile rows past the prompt end re-read its last row and are excluded from
// phi by the row count (their V rows then meet a zero A operand).
template <int HD>
__global__ __launch_bounds__(256) void linear_state_bf16_kernel(StateP p) {
  constexpr int KT = 64, CH = HD / 8;                 // 16-byte chunks per row
  constexpr int PER = KT * CH / 256;                  // chunks per thread per tile (K or V)
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][KT * HD], Vs[2][KT * HD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, c = lane & 31;
  const int h = blockIdx.x % p.H, r = blockIdx.x / p.H;
  const size_t row = (size_t)p.H * HD;
  const uint16_t *pk = (const uint16_t *)p.pk + (size_t)r * p.Lp * row + (size_t)h * HD;
  const uint16_t *pv = (const uint16_t *)p.pv + (size_t)r * p.Lp * row + (size_t)h * HD;
  const int k_begin = p.Lp - p.Lw;
  const int n_tiles = (p.Lw + KT - 1) / KT;
  constexpr int NT = (HD / 32) * (HD / 32);           // output tiles
  const bool owner = wave < NT;
  const int dk0 = (wave >> 1) * 32, dv0 = (wave & 1) * 32;

  // tile t's chunks of this thread: e = tid + 256 i -> row e / CH, chunk e % CH
  // (PER is 1 or 2; named registers rather than an array keep them out of
  // scratch memory)
  static_assert(PER == 1 || PER == 2, "chunks per thread");
  uint4 kr0, vr0, kr1, vr1;
  auto chunk_off = [&](int t, int i) -> size_t {
    const int e = tid + 256 * i, key = k_begin + t * KT + e / CH;
    return (size_t)min(key, p.Lp - 1) * row + (e % CH) * 8;
  };
#define GR_STATE_LOAD(t)                                                           \
  {                                                                                \
    const size_t o0 = chunk_off((t), 0);                                           \
    kr0 = *(const uint4 *)(pk + o0);                                               \
    vr0 = *(const uint4 *)(pv + o0);                                               \
    if constexpr (PER == 2) {                                                      \
      const size_t o1 = chunk_off((t), 1);                                         \
      kr1 = *(const uint4 *)(pk + o1);                                             \
      vr1 = *(const uint4 *)(pv + o1);                                             \
    }                                                                              \
  }
#define GR_STATE_STORE(b)                                                          \
  {                                                                                \
    *(uint4 *)&Ks[b][tid * 8] = kr0;                                               \
    *(uint4 *)&Vs[b][tid * 8] = vr0;                                               \
    if constexpr (PER == 2) {                                                      \
      *(uint4 *)&Ks[b][(tid + 256) * 8] = kr1;                                     \
      *(uint4 *)&Vs[b][(tid + 256) * 8] = vr1;                                     \
    }                                                                              \
  }

  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  float zpart = 0.f;
  GR_STATE_LOAD(0)
  GR_STATE_STORE(0)
  __syncthreads();
  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_tiles) GR_STATE_LOAD(t + 1)
    if (owner) {
      const int valid = min(KT, p.Lp - (k_begin + t * KT));   // keys of this tile inside the prompt
#pragma unroll
      for (int ks = 0; ks < KT / 16; ++ks) {
        bf16x8 a_hi, a_lo, b;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int kk = ks * 16 + 8 * g + u;
          const float kv = bf16_to_f32(Ks[buf][kk * HD + dk0 + c]);
          const float f = kk < valid ? phi(kv) : 0.f;
          const __bf16 hi = (__bf16)f;
          a_hi[u] = hi;
          a_lo[u] = (__bf16)(f - (float)hi);
          zpart += f;
          b[u] = __builtin_bit_cast(__bf16, Vs[buf][kk * HD + dv0 + c]);
        }
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_hi, b, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_lo, b, acc, 0, 0, 0);
      }
    }
    __syncthreads();                       // everyone is done with the other buffer
    if (t + 1 < n_tiles) {
      GR_STATE_STORE(buf ^ 1)
      __syncthreads();
    }
  }
#undef GR_STATE_LOAD
#undef GR_STATE_STORE
  if (!owner) return;
  float *S = p.S + ((size_t)r * p.H + h) * HD * HD;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int m = 8 * (i >> 2) + 4 * g + (i & 3);
    S[(size_t)(dk0 + m) * HD + dv0 + c] = acc[i];
  }
  // z: the two lane halves hold disjoint key sets of the same column
  const float zsum = zpart + __shfl_xor(zpart, 32);
  if ((wave & 1) == 0 && g == 0) p.z[((size_t)r * p.H + h) * HD + dk0 + c] = zsum;
}

// fp32 storage: one workgroup per (request, head); thread t owns entries
// t, t + 256, ... of the HD x HD state; 32-key tiles with phi(k) staged in LDS.
template <int HD>
__global__ __launch_bounds__(256) void linear_state_f32_kernel(StateP p) {
  constexpr int KT = 32, PER = HD * HD / 256;
  __shared__ float Fk[KT][HD], Vs[KT][HD];
  const int tid = threadIdx.x;
  const int h = blockIdx.x % p.H, r = blockIdx.x / p.H;
  const size_t row = (size_t)p.H * HD;
  const float *pk = (const float *)p.pk + (size_t)r * p.Lp * row + (size_t)h * HD;
  const float *pv = (const float *)p.pv + (size_t)r * p.Lp * row + (size_t)h * HD;
  float s[PER], zs = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) s[i] = 0.f;
  for (int k0 = p.Lp - p.Lw; k0 < p.Lp; k0 += KT) {
    const int nk = min(KT, p.Lp - k0);
    __syncthreads();
    for (int e = tid; e < KT * HD; e += 256) {
      const int kk = e / HD, i = e % HD;
      Fk[kk][i] = kk < nk ? phi(pk[(size_t)(k0 + kk) * row + i]) : 0.f;
      Vs[kk][i] = kk < nk ? pv[(size_t)(k0 + kk) * row + i] : 0.f;
    }
    __syncthreads();
    // entry tid + 256 i is (a, cc) = (tid / HD + i * 256 / HD, tid % HD)
#pragma unroll 2
    for (int kk = 0; kk < KT; ++kk) {
      const float v = Vs[kk][tid % HD];
#pragma unroll
      for (int i = 0; i < PER; ++i) s[i] = fmaf(Fk[kk][tid / HD + i * (256 / HD)], v, s[i]);
    }
    if (tid < HD)
      for (int kk = 0; kk < KT; ++kk) zs += Fk[kk][tid];
  }
  float *S = p.S + ((size_t)r * p.H + h) * HD * HD;
#pragma unroll
  for (int i = 0; i < PER; ++i) S[tid + 256 * i] = s[i];
  if (tid < HD) p.z[((size_t)r * p.H + h) * HD + tid] = zs;
}

struct LinP {
  const float *S, *z;
  const void *q, *ak, *av;
  const int32_t *parent, *beam_node;
  int32_t *dev_err;
  float *out_f32;
  uint16_t *out_bf16;          // head-major [R][H][nb][HD]
  int R, H, nb, cap, max_depth, n_chunk;
  int par_words;               // ring kernel: parent words staged in LDS
};

template <typename T>
__device__ __forceinline__ void load8(const T *src, float *dst);
template <>
__device__ __forceinline__ void load8<float>(const float *src, float *dst) {
  const float4 a = *(const float4 *)src, b = *(const float4 *)(src + 4);
  dst[0] = a.x; dst[1] = a.y; dst[2] = a.z; dst[3] = a.w;
  dst[4] = b.x; dst[5] = b.y; dst[6] = b.z; dst[7] = b.w;
}
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t *src, float *dst) {
  const uint4 a = *(const uint4 *)src;
  dst[0] = bf16_lo(a.x); dst[1] = bf16_hi(a.x); dst[2] = bf16_lo(a.y); dst[3] = bf16_hi(a.y);
  dst[4] = bf16_lo(a.z); dst[5] = bf16_hi(a.z); dst[6] = bf16_lo(a.w); dst[7] = bf16_hi(a.w);
}

// fp32 storage: one workgroup of 128 threads per (request, head, 128 beams);
// S_p and z_p of the (request, head) in LDS, read as broadcasts, one thread
// per beam, all fp32.  (Every lane reads all of S_p, so this form is LDS-bound
// at scale; the bf16 path below uses MFMA.)
template <typename T, int HD>
__global__ __launch_bounds__(128) void linear_attn_kernel(LinP p) {
  __shared__ __attribute__((aligned(16))) float Ss[HD * HD];
  __shared__ float zs[HD];
  int bid = blockIdx.x;
  const int chunk = bid % p.n_chunk;
  bid /= p.n_chunk;
  const int h = bid % p.H, r = bid / p.H;
  const float *Sg = p.S + ((size_t)r * p.H + h) * HD * HD;
  for (int e = threadIdx.x * 4; e < HD * HD; e += 128 * 4) *(float4 *)&Ss[e] = *(const float4 *)&Sg[e];
  if (threadIdx.x < HD) zs[threadIdx.x] = p.z[((size_t)r * p.H + h) * HD + threadIdx.x];
  __syncthreads();
  const int beam = chunk * 128 + threadIdx.x;
  if (beam >= p.nb) return;
  const size_t row = (size_t)p.H * HD;
  const T *qp = (const T *)p.q + ((size_t)r * p.nb + beam) * row + (size_t)h * HD;
  float fq[HD], num[HD], den = 0.f;
#pragma unroll
  for (int i = 0; i < HD; i += 8) load8<T>(qp + i, fq + i);
#pragma unroll
  for (int i = 0; i < HD; ++i) {
    fq[i] = phi(fq[i]);
    num[i] = 0.f;
  }
  // phi(q)^T S_p and phi(q) . z_p (fully unrolled: fq and num stay in
  // registers)
#pragma unroll
  for (int a = 0; a < HD; ++a) {
    const float f = fq[a];
    den = fmaf(f, zs[a], den);
#pragma unroll
    for (int i = 0; i < HD; i += 4) {
      const float4 s4 = *(const float4 *)&Ss[a * HD + i];
      num[i] = fmaf(f, s4.x, num[i]);
      num[i + 1] = fmaf(f, s4.y, num[i + 1]);
      num[i + 2] = fmaf(f, s4.z, num[i + 2]);
      num[i + 3] = fmaf(f, s4.w, num[i + 3]);
    }
  }
  // the beam's own records, from its node up to the root
  if (p.beam_node != nullptr) {
    int n = p.beam_node[(size_t)r * p.nb + beam];
    int err = 0;
    const int32_t *par = p.parent + (size_t)r * p.cap;
    for (int depth = 0; n != -1; ++depth) {
      if (n < 0 || n >= p.cap) { err |= GR_DEVERR_PARENT_RANGE; break; }
      if (depth >= p.max_depth) { err |= GR_DEVERR_DEPTH; break; }
      const int pn = par[n];
      const T *kn = (const T *)p.ak + ((size_t)r * p.cap + n) * row + (size_t)h * HD;
      const T *vn = (const T *)p.av + ((size_t)r * p.cap + n) * row + (size_t)h * HD;
      float w = 0.f;
#pragma unroll
      for (int i = 0; i < HD; i += 8) {
        float kk[8];
        load8<T>(kn + i, kk);
#pragma unroll
        for (int u = 0; u < 8; ++u) w = fmaf(fq[i + u], phi(kk[u]), w);
      }
      den += w;
#pragma unroll
      for (int i = 0; i < HD; i += 8) {
        float vv[8];
        load8<T>(vn + i, vv);
#pragma unroll
        for (int u = 0; u < 8; ++u) num[i + u] = fmaf(w, vv[u], num[i + u]);
      }
      if (pn < -1 || pn >= p.cap) { err |= GR_DEVERR_PARENT_RANGE; break; }
      if (pn >= n) { err |= GR_DEVERR_PARENT_ORDER; break; }
      n = pn;
    }
    if (err) atomicOr(p.dev_err, err);
  }
  const float inv = 1.f / den;
  if (p.out_f32) {
    float *op = p.out_f32 + ((size_t)r * p.nb + beam) * row + (size_t)h * HD;
#pragma unroll
    for (int i = 0; i < HD; i += 4) *(float4 *)(op + i) = make_float4(num[i] * inv, num[i + 1] * inv,
                                                                       num[i + 2] * inv, num[i + 3] * inv);
  }
  if (p.out_bf16) {
    uint16_t *op = p.out_bf16 + (((size_t)r * p.H + h) * p.nb + beam) * HD;
#pragma unroll
    for (int i = 0; i < HD; i += 8)
      *(uint4 *)(op + i) = make_uint4(pack_bf16x2(num[i] * inv, num[i + 1] * inv),
                                      pack_bf16x2(num[i + 2] * inv, num[i + 3] * inv),
                                      pack_bf16x2(num[i + 4] * inv, num[i + 5] * inv),
                                      pack_bf16x2(num[i + 6] * inv, num[i + 7] * inv));
  }
}

// bf16: one workgroup of 4 waves per (request, head, 128 beams), wave w
// owning beams 32w .. 32w+31.  The shared-state term is a dense contraction,
// O^T = S_p^T Phi(Q)^T ([HD x HD] by [HD x 32] per wave), on
// v_mfma_f32_32x32x16_bf16 with both operands split into bf16 hi + lo terms
// (three MFMAs: hi.hi + hi.lo + lo.hi), which keeps about 16 mantissa bits:
//   A = S_p^T (row = d_v, k = d_k) from S_p in LDS,
//   B = Phi(Q)^T (k = d_k, column = beam): lane (g, c) holds phi of dims
//       16 ks + 8g .. +8 of beam c, from one 16-byte load of its query.
// Accumulator i of tile dt is o[beam c][32 dt + 8(i/4) + 4g + i%4].  Each
// lane then folds its beam's records straight from global memory: the dot
// phi(q).phi(k_n) over the lane's HD/2 query dims, completed across the lane
// pair (c, c+32), updates the lane's HD/2 output rows and the normaliser.
// (Staging the record rows through LDS tiles level by level, 8 threads per
// row, was measured slower: it costs occupancy and a barrier per level.)
template <int HD>
__global__ __launch_bounds__(256) void linear_attn_bf16_kernel(LinP p) {
  constexpr int DT = HD / 32, KS = HD / 16;
  __shared__ __attribute__((aligned(16))) float Ss[HD * HD];
  __shared__ float zs[HD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, c = lane & 31;
  int bid = blockIdx.x;
  const int chunk = bid % p.n_chunk;
  bid /= p.n_chunk;
  const int h = bid % p.H, r = bid / p.H;
  const float *Sg = p.S + ((size_t)r * p.H + h) * HD * HD;
  for (int e = tid * 4; e < HD * HD; e += 256 * 4) *(float4 *)&Ss[e] = *(const float4 *)&Sg[e];
  if (tid < HD) zs[tid] = p.z[((size_t)r * p.H + h) * HD + tid];
  const int beam = chunk * 128 + wave * 32 + c;
  const bool valid = beam < p.nb;
  const size_t row = (size_t)p.H * HD;
  const uint16_t *qp = (const uint16_t *)p.q + ((size_t)r * p.nb + (valid ? beam : p.nb - 1)) * row +
                       (size_t)h * HD;
  // phi(q) of this lane's dims 16 ks + 8g + u, fp32 and as bf16 hi / lo
  float fq[KS][8];
  bf16x8 bhi[KS], blo[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    float v[8];
    load8<uint16_t>(qp + 16 * ks + 8 * g, v);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      fq[ks][u] = phi(v[u]);
      const __bf16 hi = (__bf16)fq[ks][u];
      bhi[ks][u] = hi;
      blo[ks][u] = (__bf16)(fq[ks][u] - (float)hi);
    }
  }
  __syncthreads();
  float den = 0.f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int u = 0; u < 8; ++u) den = fmaf(fq[ks][u], zs[16 * ks + 8 * g + u], den);
  den = xor32_sum(den);
  f32x16 O[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int i = 0; i < 16; ++i) O[dt][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 ahi, alo;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float sv = Ss[(16 * ks + 8 * g + u) * HD + 32 * dt + c];
        const __bf16 hi = (__bf16)sv;
        ahi[u] = hi;
        alo[u] = (__bf16)(sv - (float)hi);
      }
      O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, bhi[ks], O[dt], 0, 0, 0);
      O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, blo[ks], O[dt], 0, 0, 0);
      O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, bhi[ks], O[dt], 0, 0, 0);
    }
  }
  // the beam's own records, from its node up to the root
  if (p.beam_node != nullptr && valid) {
    int n = p.beam_node[(size_t)r * p.nb + beam];
    int err = 0;
    const int32_t *par = p.parent + (size_t)r * p.cap;
    for (int depth = 0; n != -1; ++depth) {
      if (n < 0 || n >= p.cap) { err |= GR_DEVERR_PARENT_RANGE; break; }
      if (depth >= p.max_depth) { err |= GR_DEVERR_DEPTH; break; }
      const int pn = par[n];
      const uint16_t *kn = (const uint16_t *)p.ak + ((size_t)r * p.cap + n) * row + (size_t)h * HD;
      const uint16_t *vn = (const uint16_t *)p.av + ((size_t)r * p.cap + n) * row + (size_t)h * HD;
      float w = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        float kk[8];
        load8<uint16_t>(kn + 16 * ks + 8 * g, kk);
#pragma unroll
        for (int u = 0; u < 8; ++u) w = fmaf(fq[ks][u], phi(kk[u]), w);
      }
      w = xor32_sum(w);
      den += w;
      // v: the lane needs half g (4 elements) of every 16-byte chunk j =
      // 4 dt + q4 of the row.  Lane g loads the chunks j = 2 jp + g whole,
      // keeps its half and trades the other half for the partner's
      // (one permlane32 swap per dword), so each lane issues HD/16 16-byte
      // loads instead of HD/8 8-byte ones.
#pragma unroll
      for (int jp = 0; jp < HD / 16; ++jp) {
        const uint4 cv = *(const uint4 *)(vn + 8 * (2 * jp + g));
        const uint32_t give0 = g ? cv.x : cv.z, give1 = g ? cv.y : cv.w;
        const uint32_t keep0 = g ? cv.z : cv.x, keep1 = g ? cv.w : cv.y;
        const auto t0 = __builtin_amdgcn_permlane32_swap(give0, give0, false, false);
        const auto t1 = __builtin_amdgcn_permlane32_swap(give1, give1, false, false);
        const uint32_t got0 = g ? t0[0] : t0[1], got1 = g ? t1[0] : t1[1];   // the partner's give
        // chunk 2 jp: half g is keep (g = 0) or got (g = 1); chunk 2 jp + 1: got (g = 0) or keep (g = 1)
        const uint2 ca = g ? make_uint2(got0, got1) : make_uint2(keep0, keep1);
        const uint2 cb = g ? make_uint2(keep0, keep1) : make_uint2(got0, got1);
        const int ja = 2 * jp, jb = 2 * jp + 1;
        O[ja >> 2][4 * (ja & 3) + 0] = fmaf(w, bf16_lo(ca.x), O[ja >> 2][4 * (ja & 3) + 0]);
        O[ja >> 2][4 * (ja & 3) + 1] = fmaf(w, bf16_hi(ca.x), O[ja >> 2][4 * (ja & 3) + 1]);
        O[ja >> 2][4 * (ja & 3) + 2] = fmaf(w, bf16_lo(ca.y), O[ja >> 2][4 * (ja & 3) + 2]);
        O[ja >> 2][4 * (ja & 3) + 3] = fmaf(w, bf16_hi(ca.y), O[ja >> 2][4 * (ja & 3) + 3]);
        O[jb >> 2][4 * (jb & 3) + 0] = fmaf(w, bf16_lo(cb.x), O[jb >> 2][4 * (jb & 3) + 0]);
        O[jb >> 2][4 * (jb & 3) + 1] = fmaf(w, bf16_hi(cb.x), O[jb >> 2][4 * (jb & 3) + 1]);
        O[jb >> 2][4 * (jb & 3) + 2] = fmaf(w, bf16_lo(cb.y), O[jb >> 2][4 * (jb & 3) + 2]);
        O[jb >> 2][4 * (jb & 3) + 3] = fmaf(w, bf16_hi(cb.y), O[jb >> 2][4 * (jb & 3) + 3]);
      }
      if (pn < -1 || pn >= p.cap) { err |= GR_DEVERR_PARENT_RANGE; break; }
      if (pn >= n) { err |= GR_DEVERR_PARENT_ORDER; break; }
      n = pn;
    }
    if (err) atomicOr(p.dev_err, err);
  }
  if (!valid) return;
  const float inv = 1.f / den;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = 32 * dt + 8 * q4 + 4 * g;
      const float o0 = O[dt][4 * q4] * inv, o1 = O[dt][4 * q4 + 1] * inv;
      const float o2 = O[dt][4 * q4 + 2] * inv, o3 = O[dt][4 * q4 + 3] * inv;
      if (p.out_f32)
        *(float4 *)(p.out_f32 + ((size_t)r * p.nb + beam) * row + (size_t)h * HD + d0) = make_float4(o0, o1, o2, o3);
      if (p.out_bf16)
        *(uint2 *)(p.out_bf16 + (((size_t)r * p.H + h) * p.nb + beam) * HD + d0) =
            make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
    }
}

// Arenas of up to this many nodes per request take the ring kernel below.
constexpr int kLinRingNodes = 4096;

// bf16, ring form: the same computation as linear_attn_bf16_kernel, with the
// record rows gathered by LDS DMA (global_load_lds) through a 3-stage ring of
// tiles, as the softmax kernel streams its records; the per-lane loads of the
// plain form gather 128-byte rows with 16-byte pieces from 32 rows per
// instruction and cost about 15 us per chain level at the headline shape.
// Stream order, each wait an exact vmcnt: the parent array and the
// workgroup's beam nodes (wave 0), S_p into stage 0 (and the queries, loaded
// to registers); then, once the chains are resolved in LDS, record tile k
// into stage (k + 1) % 3, two tiles ahead.  Tile k holds the key rows (k
// even) or the value rows (k odd) of the level k / 2 records of all 128
// beams, so that every wave folds every tile: a key tile gives each beam its
// record's weight, the value tile after it adds the weighted values (tiles of
// 64 beams holding both halves left half the waves idle at each tile and
// took 6 % longer).
// Stage 0 is free for records once the shared-state MFMAs have read S_p.
// Record rows are XOR-swizzled so that 16 lanes reading 16 consecutive rows
// at one logical 16-byte chunk hit 16 distinct bank slots.
typedef __attribute__((ext_vector_type(4))) short i16x4;
#define LIN_LDS4(p) ((__attribute__((address_space(3))) i16x4 *)(p))

template <int HD>
__device__ __forceinline__ int lswz(int row) {
  constexpr int RB = HD * 2, CPR = RB / 16;
  return (row / (256 / RB)) & (CPR - 1);
}

template <int HD>
__global__ __launch_bounds__(256) void linear_ring_bf16_kernel(LinP p) {
  constexpr int DT = HD / 32, KS = HD / 16;
  constexpr int NB = 128, KT = 64, NS = 3;
  constexpr int RB = HD * 2, CPR = RB / 16;          // bytes and 16-byte chunks per record row
  constexpr int TB = KT * RB;                        // bytes of the K (or V) half of a tile
  constexpr int NBLK = 2 * TB / 1024, BPW = NBLK / 4;   // 1 KB DMA blocks per tile, per wave
  constexpr int SBLK = HD * HD * 4 / 1024;           // 1 KB blocks of S_p
  static_assert(HD * HD * 4 <= 2 * TB, "S_p fits one ring stage");
  static_assert(NBLK % 4 == 0 && SBLK % 4 == 0, "every wave moves the same number of blocks");
  __shared__ __attribute__((aligned(1024))) unsigned char ring[NS][2 * TB];
  __shared__ float zs[HD];
  __shared__ int16_t ids16[GR_MAX_DEPTH][NB];
  extern __shared__ __attribute__((aligned(16))) int32_t dyn_l[];   // parents [par_words], beam nodes [NB]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, c = lane & 31;
  int bid = blockIdx.x;
  const int chunk = bid % p.n_chunk;
  bid /= p.n_chunk;
  const int h = bid % p.H, r = bid / p.H;
  const int wb = wave * 32 + c;
  const int beam = chunk * NB + wb;
  const bool valid = beam < p.nb;
  const size_t row = (size_t)p.H * HD;
  const bool chains = p.beam_node != nullptr;
  int32_t *const par_s = dyn_l;
  int32_t *const bn_s = dyn_l + p.par_words;

  // ---- prologue: parents and beam nodes, S_p, z_p, queries
  if (chains && wave == 0) {
    const int32_t *par = p.parent + (size_t)r * p.cap;
    for (int i = 0; i * 64 < p.cap; ++i) dma4(par + min(i * 64 + lane, p.cap - 1), par_s + i * 64);
    const int32_t *bnp = p.beam_node + (size_t)r * p.nb;
    for (int i = 0; i * 64 < NB; ++i) dma4(bnp + min(chunk * NB + i * 64 + lane, p.nb - 1), bn_s + i * 64);
  }
  const float *Sg = p.S + ((size_t)r * p.H + h) * HD * HD;
#pragma unroll
  for (int i = 0; i < SBLK / 4; ++i) {
    const int blk = wave * (SBLK / 4) + i;
    dma16((const char *)Sg + blk * 1024 + 16 * lane, ring[0] + blk * 1024);
  }
  if (tid < HD) zs[tid] = p.z[((size_t)r * p.H + h) * HD + tid];
  const uint16_t *qp = (const uint16_t *)p.q + ((size_t)r * p.nb + (valid ? beam : p.nb - 1)) * row +
                       (size_t)h * HD;
  // phi(q) of this lane's dims 16 ks + 8g + u as bf16 hi + lo (about 16
  // mantissa bits); the dots with z_p and the records use hi + lo as well
  bf16x8 bhi[KS], blo[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    float v[8];
    load8<uint16_t>(qp + 16 * ks + 8 * g, v);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float f = phi(v[u]);
      const __bf16 hi = (__bf16)f;
      bhi[ks][u] = hi;
      blo[ks][u] = (__bf16)(f - (float)hi);
    }
  }
  auto fq = [&](int ks, int u) -> float { return (float)bhi[ks][u] + (float)blo[ks][u]; };
  GR_WAIT_VMCNT(0);
  __syncthreads();

  // ---- chains: one thread per beam walks its parent links in LDS
  int depth = 0;
  if (chains) {
    if (tid < NB) {
      int n = chunk * NB + tid < p.nb ? bn_s[tid] : -1;
      int err = 0;
      for (int d = 0; d < p.max_depth; ++d) {
        int id = -1;
        if (n != -1) {
          if (n < 0 || n >= p.cap) {
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
        ids16[d][tid] = (int16_t)id;
      }
      for (int d = p.max_depth; d < GR_MAX_DEPTH; ++d) ids16[d][tid] = -1;
      if (n != -1) err |= GR_DEVERR_DEPTH;
      if (err) atomicOr(p.dev_err, err);
    }
    __syncthreads();
    for (int d = 0; d < p.max_depth; ++d)
      if (__syncthreads_or(tid < NB && ids16[d][tid] >= 0)) depth = d + 1;
  }
  const int n_tiles = depth * (NB / KT);
  // the deepest record of the first beam that has a chain (any written record
  // would do; with none, no level is issued)
  int rec_fill = 0;
  if (n_tiles > 0) {
    const uint64_t m0 = __builtin_amdgcn_ballot_w64(ids16[0][lane] >= 0);
    const uint64_t m1 = __builtin_amdgcn_ballot_w64(ids16[0][64 + lane] >= 0);
    const int fb = m0 ? (int)__builtin_ctzll(m0) : (m1 ? 64 + (int)__builtin_ctzll(m1) : 0);
    rec_fill = __builtin_amdgcn_readfirstlane(max((int)ids16[0][fb], 0));
  }

  // record tile k: the key (k even) or value (k odd) rows of the level k / 2
  // records, row t for workgroup beam t, so that every wave folds every tile
  static_assert(NB * RB == 2 * TB, "one half-record of every beam fills a stage");
  auto issue = [&](int k, unsigned char *st) {
    const int d = k >> 1, half = k & 1;
    // a beam without a record at level d gathers `rec_fill`, a record of
    // the workgroup: the value product multiplies every row, by 0 for such a
    // beam, so every row must be written data
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int blk = wave * BPW + i;
      const int byte = blk * 1024 + 16 * lane;
      const int t = byte / RB, pch = (byte % RB) / 16;
      const int id = ids16[d][t];
      const uint16_t *src = (const uint16_t *)(half ? p.av : p.ak) +
                            ((size_t)r * p.cap + (id >= 0 ? id : rec_fill)) * row + (size_t)h * HD +
                            (pch ^ lswz<HD>(t)) * 8;
      dma16(src, st + blk * 1024);
    }
  };
  if (n_tiles > 0) issue(0, ring[1]);
  if (n_tiles > 1) issue(1, ring[2]);

  // ---- phi(q)^T S_p and phi(q) . z_p (S_p from stage 0)
  const float *Ss = reinterpret_cast<const float *>(ring[0]);
  float den = 0.f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int u = 0; u < 8; ++u) den = fmaf(fq(ks, u), zs[16 * ks + 8 * g + u], den);
  den = xor32_sum(den);
  f32x16 O[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int i = 0; i < 16; ++i) O[dt][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 ahi, alo;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float sv = Ss[(16 * ks + 8 * g + u) * HD + 32 * dt + c];
        const __bf16 hi = (__bf16)sv;
        ahi[u] = hi;
        alo[u] = (__bf16)(sv - (float)hi);
      }
      O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, bhi[ks], O[dt], 0, 0, 0);
      O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, blo[ks], O[dt], 0, 0, 0);
      O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, bhi[ks], O[dt], 0, 0, 0);
    }
  }

  // ---- records, tile by tile
  float w_lev = 0.f;                           // weight of the level whose values come next (0: no record)
  // The value tile adds O^T += V^T diag(w) on the MFMA.  A: the value rows of
  // this wave's 32 beams, read transposed; per 16-row k-step, lane (c, g)
  // holds element e of rows 8 (e >> 2) + 4 g + (e & 3).  The row swizzle
  // depends only on a row's low four bits, so the offsets within a k-step
  // are the lane's own.  B: each beam's weight at its own row and column
  // (beam c's in the lanes with g = bit 2 of c, k-step c >> 4, element
  // rec_e), as bf16 hi + lo in two products.
  int rvo[DT][2];
  {
    const int q16 = lane >> 4, j16 = lane & 15;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int tr = 8 * hh + 4 * g + (j16 >> 2);
        const int dd = 32 * dt + 16 * (q16 & 1) + 4 * (j16 & 3);
        rvo[dt][hh] = tr * RB + (((dd >> 3) ^ lswz<HD>(tr)) << 4) + ((dd & 7) << 1);
      }
  }
  const int rec_e = 4 * ((c >> 3) & 1) + (c & 3);
  const int rec_bi = g == ((c >> 2) & 1) ? 4 * (c >> 4) + (rec_e >> 1) : 8;   // 32-bit word of the B operand, or none
  const int rec_sh = 16 * (rec_e & 1);
  // tile k has landed once at most the tiles issued after it (k + 1, the
  // ring being NS - 1 = 2 tiles deep) are in flight: BPW DMAs per tile and wave
  static_assert(NS == 3, "one tile ahead at each wait");
  auto tile_head = [&](int k) {
    if (k + 1 < n_tiles) GR_WAIT_VMCNT(BPW);
    else GR_WAIT_VMCNT(0);
    ring_barrier();                            // tile k landed for all; stage of tile k-1 (or S_p) free
    if (k + NS - 1 < n_tiles) issue(k + NS - 1, ring[(k + NS) % NS]);
  };
  // one chain level per iteration, its key tile then its value tile (with
  // both kinds in one loop body the register allocator moves O around the
  // value product at every tile)
  for (int k = 0; k < n_tiles; k += 2) {
    const int d = k >> 1;
    tile_head(k);
    {                                          // key rows: each beam's record weight
      const unsigned char *rr = ring[(k + 1) % NS] + wb * RB;
      float w = 0.f;
      if (d < p.max_depth && ids16[d][wb] >= 0) {   // the same for both lanes of a beam
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const uint4 k4 = *(const uint4 *)(rr + (((2 * ks + g) ^ lswz<HD>(wb)) << 4));
          const float kk[8] = {bf16_lo(k4.x), bf16_hi(k4.x), bf16_lo(k4.y), bf16_hi(k4.y),
                               bf16_lo(k4.z), bf16_hi(k4.z), bf16_lo(k4.w), bf16_hi(k4.w)};
#pragma unroll
          for (int u = 0; u < 8; ++u) w = fmaf(fq(ks, u), phi(kk[u]), w);
        }
        w = xor32_sum(w);
        den += w;
      }
      w_lev = w;
    }
    tile_head(k + 1);
    {                                          // value rows, weighted, for the whole wave
      const unsigned char *stage = ring[(k + 2) % NS];
      const __bf16 whi = (__bf16)w_lev;
      const __bf16 wlo = (__bf16)(w_lev - (float)whi);
      const uint32_t ph = (uint32_t)__builtin_bit_cast(uint16_t, whi) << rec_sh;
      const uint32_t pl = (uint32_t)__builtin_bit_cast(uint16_t, wlo) << rec_sh;
      bf16x8 bh[2], bl[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        bh[st] = __builtin_bit_cast(bf16x8, make_uint4(rec_bi == 4 * st ? ph : 0u, rec_bi == 4 * st + 1 ? ph : 0u,
                                                       rec_bi == 4 * st + 2 ? ph : 0u, rec_bi == 4 * st + 3 ? ph : 0u));
        bl[st] = __builtin_bit_cast(bf16x8, make_uint4(rec_bi == 4 * st ? pl : 0u, rec_bi == 4 * st + 1 ? pl : 0u,
                                                       rec_bi == 4 * st + 2 ? pl : 0u, rec_bi == 4 * st + 3 ? pl : 0u));
      }
      const unsigned char *ab = stage + 32 * wave * RB;   // this wave's 32 rows
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LIN_LDS4(ab + st * 16 * RB + rvo[dt][0]));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LIN_LDS4(ab + st * 16 * RB + rvo[dt][1]));
          const i16x4 a8[2] = {lo, hi};
          const bf16x8 a = __builtin_bit_cast(bf16x8, a8);
          O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bh[st], O[dt], 0, 0, 0);
          O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bl[st], O[dt], 0, 0, 0);
        }
    }
  }
  if (!valid) return;
  const float inv = 1.f / den;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = 32 * dt + 8 * q4 + 4 * g;
      const float o0 = O[dt][4 * q4] * inv, o1 = O[dt][4 * q4 + 1] * inv;
      const float o2 = O[dt][4 * q4 + 2] * inv, o3 = O[dt][4 * q4 + 3] * inv;
      if (p.out_f32)
        *(float4 *)(p.out_f32 + ((size_t)r * p.nb + beam) * row + (size_t)h * HD + d0) = make_float4(o0, o1, o2, o3);
      if (p.out_bf16)
        *(uint2 *)(p.out_bf16 + (((size_t)r * p.H + h) * p.nb + beam) * HD + d0) =
            make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
    }
}

}  // namespace

hipError_t launch_linear_state(const LinearStateArgs &a, hipStream_t s) {
  StateP p;
  p.pk = a.pk; p.pv = a.pv; p.S = a.S; p.z = a.z;
  p.R = a.R; p.H = a.H; p.Lp = a.Lp; p.Lw = a.Lw;
  const dim3 grid((unsigned)(a.R * a.H)), block(256);
  if (a.dtype == GR_BF16) {
    if (a.hd == 64) hipLaunchKernelGGL(linear_state_bf16_kernel<64>, grid, block, 0, s, p);
    else hipLaunchKernelGGL(linear_state_bf16_kernel<32>, grid, block, 0, s, p);
  } else {
    if (a.hd == 64) hipLaunchKernelGGL(linear_state_f32_kernel<64>, grid, block, 0, s, p);
    else hipLaunchKernelGGL(linear_state_f32_kernel<32>, grid, block, 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_linear_attn(const LinearAttnArgs &a, hipStream_t s) {
  LinP p;
  p.S = a.S; p.z = a.z; p.q = a.q; p.ak = a.ak; p.av = a.av;
  p.parent = a.parent; p.beam_node = a.beam_node; p.dev_err = a.dev_err;
  p.out_f32 = a.out_f32; p.out_bf16 = (uint16_t *)a.out_lowp;
  p.R = a.R; p.H = a.H; p.nb = a.nb; p.cap = a.cap; p.max_depth = a.max_depth;
  p.n_chunk = (a.nb + 127) / 128;
  const dim3 grid((unsigned)((long long)a.R * a.H * p.n_chunk));
  p.par_words = 0;
  if (a.dtype == GR_BF16 && (a.beam_node == nullptr || a.cap <= kLinRingNodes)) {
    p.par_words = a.beam_node ? (a.cap + 63) / 64 * 64 : 0;
    const size_t dyn = (size_t)(p.par_words + 128) * sizeof(int32_t);
    if (a.hd == 64) hipLaunchKernelGGL(linear_ring_bf16_kernel<64>, grid, dim3(256), dyn, s, p);
    else hipLaunchKernelGGL(linear_ring_bf16_kernel<32>, grid, dim3(256), dyn, s, p);
  } else if (a.dtype == GR_BF16) {
    if (a.hd == 64) hipLaunchKernelGGL(linear_attn_bf16_kernel<64>, grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL(linear_attn_bf16_kernel<32>, grid, dim3(256), 0, s, p);
  } else {
    const dim3 block(128);
    if (a.hd == 64) hipLaunchKernelGGL((linear_attn_kernel<float, 64>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((linear_attn_kernel<float, 32>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace gr
