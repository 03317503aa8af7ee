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
// owns beams 32*(w/2).. and codes 128*(w%2)..), so each lane holds one beam's
// codes and the log-softmax is in-lane plus one lane^32 swap and one LDS
// exchange between the two code halves.  The scores never leave the chip:
// they become ordering keys in LDS and are selected there (gr_select.h).
//
// score_select: same scoring and selection starting from fp32 logits in
// global memory (the standalone top-k entry point, the fp32 path and scalar
// scoring).  select_merge: final selection over per-group partial lists.
// project: VALU projection z = o . W^T for the fp32 path and the scalar
// score o . w.

#include "gr_device.h"
#include "gr_launch.h"
#include "gr_select.h"

namespace gr {
namespace {

constexpr int kNT = 512;

struct LogitsSmem {
  uint32_t keys[kGroupPositions];
  SelectSmem<kNT> sel;
  float red_max[4][2][32];
  float red_sum[4][2][32];
};

struct LP {
  const uint16_t *o, *W;
  const float *prior;
  float *cand;
  float *score;
  int32_t *token, *parent;
  uint64_t *partial;
  int R, n_in, D, k, lsm, n_groups, kk;
};

__global__ __launch_bounds__(kNT) void logits_select_bf16_kernel(LP p) {
  __shared__ LogitsSmem sm;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 5, c = lane & 31;
  const int r = blockIdx.x / p.n_groups, grp = blockIdx.x % p.n_groups;
  const int b_begin = grp * kGroupBeams;
  const int nbg = min(kGroupBeams, p.n_in - b_begin);
  const int bb = wave >> 1, ch = wave & 1;
  const int bl = bb * 32 + c;
  const bool valid = bl < nbg;
  const int beam = b_begin + bl;

  f32x16 acc[4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[m][i] = 0.f;
  if (bb * 32 < nbg) {
    const uint16_t *orow = p.o + ((size_t)r * p.n_in + (valid ? beam : 0)) * p.D + 8 * g;
    const uint16_t *wrow = p.W + (size_t)(ch * 128 + c) * p.D + 8 * g;
    const size_t wstep = (size_t)32 * p.D;
#pragma unroll 2
    for (int kk = 0; kk < p.D; kk += 16) {
      const uint4 braw = valid ? *(const uint4 *)(orow + kk) : make_uint4(0, 0, 0, 0);
      const bf16x8 b = __builtin_bit_cast(bf16x8, braw);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const bf16x8 a = *(const bf16x8 *)(wrow + m * wstep + kk);
        acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[m], 0, 0, 0);
      }
    }
  }

  float lse = 0.f;
  if (p.lsm) {
    float mx = acc[0][0];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, acc[m][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (lane < 32) sm.red_max[bb][ch][c] = mx;
    __syncthreads();
    const float M = fmaxf(sm.red_max[bb][0][c], sm.red_max[bb][1][c]);
    float se = 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int i = 0; i < 16; ++i) se += expf(acc[m][i] - M);
    se += __shfl_xor(se, 32);
    if (lane < 32) sm.red_sum[bb][ch][c] = se;
    __syncthreads();
    lse = M + logf(sm.red_sum[bb][0][c] + sm.red_sum[bb][1][c]);
  }
  if (valid) {
    const float pr = p.prior ? p.prior[(size_t)r * p.n_in + beam] : 0.f;
    float *crow = p.cand ? p.cand + ((size_t)r * p.n_in + beam) * 256 : nullptr;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int code = ch * 128 + 32 * m + 8 * q4 + 4 * g;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = (acc[m][4 * q4 + e] - lse) + pr;
          sm.keys[bl * 256 + code + e] = rank_key(v[e]);
        }
        if (crow) *(float4 *)(crow + code) = make_float4(v[0], v[1], v[2], v[3]);
      }
  }
  __syncthreads();
  const int n = nbg * 256;
  block_select<kNT>(sm.keys, nullptr, (uint32_t)b_begin * 256u, n, min(p.k, n), sm.sel);
  emit_selection<kNT>(sm.sel, min(p.k, n), r, grp, 256, p.score, p.token, p.parent, p.partial, p.n_groups, p.kk);
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
  uint32_t keys[kGroupPositions];
  SelectSmem<kNT> sel;
};

__global__ __launch_bounds__(kNT) void score_select_kernel(SP p) {
  __shared__ ScoreSmem sm;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = blockIdx.x / p.n_groups, grp = blockIdx.x % p.n_groups;
  int n;
  uint32_t base;
  if (p.vocab == 256) {
    const int b_begin = grp * kGroupBeams;
    const int nbg = min(kGroupBeams, p.n_in - b_begin);
    for (int row = wave; row < nbg; row += kNT / 64) {
      const int beam = b_begin + row;
      const size_t off = ((size_t)r * p.n_in + beam) * 256 + lane * 4;
      const float4 z = *(const float4 *)(p.z + off);
      float lse = 0.f;
      if (p.lsm) {
        const float mx = wave_max(fmaxf(fmaxf(z.x, z.y), fmaxf(z.z, z.w)));
        const float se = wave_sum(expf(z.x - mx) + expf(z.y - mx) + expf(z.z - mx) + expf(z.w - mx));
        lse = mx + logf(se);
      }
      const float pr = p.prior ? p.prior[(size_t)r * p.n_in + beam] : 0.f;
      const float v0 = (z.x - lse) + pr, v1 = (z.y - lse) + pr;
      const float v2 = (z.z - lse) + pr, v3 = (z.w - lse) + pr;
      uint32_t *kr = sm.keys + row * 256 + lane * 4;
      kr[0] = rank_key(v0); kr[1] = rank_key(v1); kr[2] = rank_key(v2); kr[3] = rank_key(v3);
      if (p.cand) *(float4 *)(p.cand + off) = make_float4(v0, v1, v2, v3);
    }
    n = nbg * 256;
    base = (uint32_t)b_begin * 256u;
  } else {
    const int p0 = grp * kGroupPositions;
    n = min(kGroupPositions, p.n_in - p0);
    for (int i = tid; i < n; i += kNT) {
      const size_t off = (size_t)r * p.n_in + p0 + i;
      const float v = p.z[off] + (p.prior ? p.prior[off] : 0.f);
      sm.keys[i] = rank_key(v);
      if (p.cand) p.cand[off] = v;
    }
    base = (uint32_t)p0;
  }
  __syncthreads();
  block_select<kNT>(sm.keys, nullptr, base, n, min(p.k, n), sm.sel);
  emit_selection<kNT>(sm.sel, min(p.k, n), r, grp, p.vocab, p.score, p.token, p.parent, p.partial, p.n_groups, p.kk);
}

struct MergeSmem {
  uint32_t rk[kMergeCapacity];
  uint32_t ix[kMergeCapacity];
  SelectSmem<kNT> sel;
};

__global__ __launch_bounds__(kNT) void select_merge_kernel(const uint64_t *partial, int n_groups, int kk, int k,
                                                           int vocab, float *score, int32_t *token,
                                                           int32_t *parent) {
  __shared__ MergeSmem sm;
  const int r = blockIdx.x;
  const int n = n_groups * kk;
  const uint64_t *src = partial + (size_t)r * n;
  for (int i = threadIdx.x; i < n; i += kNT) {
    const uint64_t x = src[i];
    sm.rk[i] = (uint32_t)(x >> 32);
    sm.ix[i] = (uint32_t)x;
  }
  __syncthreads();
  block_select<kNT>(sm.rk, sm.ix, 0u, n, k, sm.sel);
  emit_selection<kNT>(sm.sel, k, r, 0, vocab, score, token, parent, nullptr, 1, k);
}

// z[row][t] = sum_i o[row][i] W[t][i] (+ prior[row] for the scalar path).
__device__ __forceinline__ float ldv(const float *p, size_t i) { return p[i]; }
__device__ __forceinline__ float ldv(const uint16_t *p, size_t i) { return bf16_to_f32(p[i]); }

template <typename TO, typename TW>
__global__ __launch_bounds__(256) void project_kernel(const TO *o, const TW *W, const float *prior, float *z,
                                                      int rows, int D, int vocab, int add_prior) {
  if (vocab == 1) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (row >= rows) return;
    float s = 0.f;
    for (int i = lane; i < D; i += 64) s = fmaf(ldv(o, (size_t)row * D + i), ldv(W, (size_t)i), s);
    s = wave_sum(s);
    if (lane == 0) z[row] = s + (add_prior && prior ? prior[row] : 0.f);
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
  p.R = a.R; p.n_in = a.n_in; p.D = a.D; p.k = a.k; p.lsm = a.log_softmax;
  p.n_groups = o.n_groups; p.kk = o.kk;
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
  hipLaunchKernelGGL(score_select_kernel, dim3((unsigned)(a.R * o.n_groups)), dim3(kNT), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || o.n_groups == 1) return e;
  return launch_select_merge(o, a.R, a.k, a.vocab, s);
}

hipError_t launch_select_merge(const SelectOut &o, int R, int k, int vocab, hipStream_t s) {
  hipLaunchKernelGGL(select_merge_kernel, dim3((unsigned)R), dim3(kNT), 0, s, o.partial, o.n_groups, o.kk, k, vocab,
                     o.score, o.token, o.parent);
  return hipGetLastError();
}

hipError_t launch_project(const ProjArgs &a, hipStream_t s) {
  const int rows = a.R * a.n;
  const dim3 grid(a.vocab == 1 ? (unsigned)((rows + 3) / 4) : (unsigned)rows);
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
