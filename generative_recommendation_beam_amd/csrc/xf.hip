// Multi-layer broadcast scoring: one user sequence and many single-token
// candidates through a Pre-LN Transformer stack, one scalar score per
// candidate.
//
// TransRetrieval, Architecture Overview (stage 4: N-layer Pre-LN Transformer
// with a ReLU FFN; the user-side keys and values of a request are cached once
// and reused by all of its candidates), the per-candidate cost paragraph
// (each candidate has its own Q/K/V/output projections and FFN and attends to
// the whole user sequence), Hardware-aware inference optimization (the one
// user cache is broadcast to every candidate without copies; single-token
// candidates are packed into batched products and kept apart) and GPU
// retrieval (the selection stays on the device).
//
// Model: width D = 128 (4 heads of 32), FFN width 2D, LayerNorm eps 1e-5,
// biases on every projection; a candidate attends to the layer's user keys
// and to its own key; after the last layer a final LayerNorm and a linear
// head give the score.
//
// Layout of a wave's tokens (the user pass; the candidate kernel uses the
// 16-wide form of the same scheme, described at its section).  A wave owns
// 32 tokens and keeps everything about them in registers: the residual stream
// x in fp32, and each product's output, in the accumulator layout of
// v_mfma_f32_32x32x16_bf16 transposed (features x tokens: lane (c, g) holds
// token c).  The A operand of every product is a weight (or user key /
// value) row read from LDS, and its rows are taken in the order
// pi(m) = m with bits 2 and 3 swapped: output row m of the tile then holds
// feature 16 (i >> 3) + 8 g + (i & 7) at accumulator index i, i.e. eight
// consecutive features per half of the tile, which are exactly the eight
// k-values the lane supplies as the B operand of the next product.  No
// activation ever goes through LDS; LayerNorm statistics are in-lane sums
// plus one lane^32 swap.
//
// Weights, the per-layer vectors (biases, LayerNorm gains) and the user keys
// and values stream HBM/L2 -> LDS through a ring of two 32 KB slots
// (global_load_lds, one piece ahead of the products); all the workgroup's
// waves read each piece.  Weight rows are stored with a 16-byte chunk
// swizzle (chunk ^ row & 15) so that the 32 rows a read touches hit distinct
// banks.  The user keys and values of a layer are written by the user pass
// in exactly the ring's layout (per head, per 256 keys: K [key][32] with
// chunk ^ (key >> 2) & 3, then V^T [32][key] with chunk ^ dim & 15), so the
// candidates copy them as they are.
//
// xf_user_kernel: one launch per layer, one workgroup per 32 user tokens of
// a request; launch l finishes layer l-1 (attention over the user keys of
// l-1, output projection, FFN) and forms layer l's queries, keys and values,
// its four waves splitting every product by head or by output features.
// xf_cand16_kernel: all layers for 10 x 16 candidates per workgroup, then the
// final LayerNorm and the score (16-wide products; see its section).

#include "gr_device.h"
#include "gr_launch.h"

namespace gr {
namespace {

constexpr int kXD = 128;                // model width
constexpr int kXHeads = 4;
constexpr int kXHd = 32;                // head dim
constexpr int kXFF = 2 * kXD;           // FFN width
constexpr int kXSlot = 32768;           // ring slot bytes
constexpr int kXVecBytes = 6144;        // per-layer vectors (11 D floats) or the final ones (3 D + 1)
constexpr int kXLayerVec = 11 * kXD;    // floats per layer in the vector buffer
constexpr int kXMat = 8 * kXD * kXD;    // bf16 values per layer in the matrix buffer
// offsets inside a layer's vectors
constexpr int kVbQKV = 0, kVbO = 3 * kXD, kVb1 = 4 * kXD, kVb2 = 6 * kXD, kVln1g = 7 * kXD, kVln1b = 8 * kXD,
              kVln2g = 9 * kXD, kVln2b = 10 * kXD;
// offsets inside a layer's matrices
constexpr int kMqkv = 0, kMo = 3 * kXD * kXD, kM1 = 4 * kXD * kXD, kM2 = 6 * kXD * kXD;
constexpr float kXLog2e = 1.4426950408889634f;

__device__ __forceinline__ int xpi(int m) { return (m & 0x13) | ((m & 8) >> 1) | ((m & 4) << 1); }

// A copy of a lane value that the compiler must treat as changed here:
// offsets derived from it are recomputed at each use instead of being
// hoisted out of the piece loop and held in registers for the whole kernel.
__device__ __forceinline__ int fresh(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

struct XfSmem {
  unsigned char ring[2][kXSlot];
  float vec[kXVecBytes / 4];
};

// ---- ring pieces -----------------------------------------------------------
// Each DMA instruction moves 1 KB (64 lanes x 16 bytes) or, for vectors,
// 256 bytes (dma4).  Pieces are split over the workgroup's NW waves.

// nrows weight rows of 256 bytes (128 bf16) into a slot: row i comes from
// src_row(i); LDS chunk ^ (i & 15).
template <int NW, typename RowFn>
__device__ __forceinline__ void dma_rows(unsigned char *slot, int nrows, RowFn src_row, int wave, int lane) {
  const int nblk = nrows / 4;
  lane = fresh(lane);
  for (int b = wave; b < nblk; b += NW) {
    const int row = 4 * b + (lane >> 4), pc = lane & 15;
    const uint16_t *src = src_row(row) + 8 * (pc ^ (row & 15));
    dma16(src, slot + b * 1024);
  }
}
// the 32 columns 32 h .. of the 128 rows of W_o ([D][D]) into 64-byte rows
// (chunk ^ (row >> 2) & 3)
template <int NW>
__device__ __forceinline__ void dma_wo_cols(unsigned char *dst, const uint16_t *wo, int h, int wave, int lane) {
  lane = fresh(lane);
  for (int b = wave; b < 8; b += NW) {
    const int row = 16 * b + (lane >> 2), pc = lane & 3;
    dma16(wo + (size_t)row * kXD + 32 * h + 8 * (pc ^ ((row >> 2) & 3)), dst + b * 1024);
  }
}
// a contiguous run of bytes (a multiple of 1 KB)
template <int NW>
__device__ __forceinline__ void dma_copy(unsigned char *dst, const unsigned char *src, int bytes, int wave, int lane) {
  lane = fresh(lane);
  for (int b = wave; b < bytes / 1024; b += NW) dma16(src + b * 1024 + lane * 16, dst + b * 1024);
}
// n floats (dma4, 64 per instruction; the tail re-reads the last float)
template <int NW>
__device__ __forceinline__ void dma_floats(float *dst, const float *src, int n, int wave, int lane) {
  lane = fresh(lane);
  for (int b = wave; b < (n + 63) / 64; b += NW) dma4(src + min(64 * b + lane, n - 1), dst + 64 * b);
}

// ---- wave math ---------------------------------------------------------------
typedef f32x16 Acc;

__device__ __forceinline__ bf16x8 pack8(const Acc &a, int s) {
  bf16x8 r;
#pragma unroll
  for (int t = 0; t < 8; ++t) r[t] = (__bf16)a[8 * s + t];
  return r;
}

// LayerNorm of the wave's 32 tokens (x: 4 tiles of 32 features), gains and
// biases from LDS; writes the bf16 B operands h[ft][s].
__device__ __forceinline__ void layer_norm_b(const Acc (&x)[4], const float *gain, const float *bias, int g,
                                             bf16x8 (&h)[4][2]) {
  g = fresh(g);
  float s = 0.f;
#pragma unroll
  for (int ft = 0; ft < 4; ++ft)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += x[ft][i];
  const float mean = xor32_sum(s) * (1.f / kXD);
  float v = 0.f;
#pragma unroll
  for (int ft = 0; ft < 4; ++ft)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float d = x[ft][i] - mean;
      v = fmaf(d, d, v);
    }
  const float rstd = 1.f / sqrtf(xor32_sum(v) * (1.f / kXD) + 1e-5f);
#pragma unroll
  for (int ft = 0; ft < 4; ++ft)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int f0 = 32 * ft + 16 * s2 + 8 * g;
      const float4 g0 = *(const float4 *)(gain + f0), g1 = *(const float4 *)(gain + f0 + 4);
      const float4 b0 = *(const float4 *)(bias + f0), b1 = *(const float4 *)(bias + f0 + 4);
      const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
      const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
      bf16x8 r;
#pragma unroll
      for (int t = 0; t < 8; ++t) r[t] = (__bf16)fmaf((x[ft][8 * s2 + t] - mean) * rstd, gg[t], bb[t]);
      h[ft][s2] = r;
    }
}

__device__ __forceinline__ void zero(Acc &a) {
#pragma unroll
  for (int i = 0; i < 16; ++i) a[i] = 0.f;
}
// add the bias of features f0 + 16 s + 8 g + t
__device__ __forceinline__ void add_bias(Acc &a, const float *b, int g) {
  g = fresh(g);
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const float4 b0 = *(const float4 *)(b + 16 * s + 8 * g), b1 = *(const float4 *)(b + 16 * s + 8 * g + 4);
    a[8 * s + 0] += b0.x; a[8 * s + 1] += b0.y; a[8 * s + 2] += b0.z; a[8 * s + 3] += b0.w;
    a[8 * s + 4] += b1.x; a[8 * s + 5] += b1.y; a[8 * s + 6] += b1.z; a[8 * s + 7] += b1.w;
  }
}

// Online-softmax state of one head for the wave's 32 tokens.
struct HeadState {
  Acc o;          // output dims (accumulator layout), unnormalised
  float m, l;     // running max (log2 units) and this lane's partial sum
};

// One piece of user keys/values (up to 256 keys; n_kt tiles of 32) folded
// into the state: S^T = K q^T, p = exp2(S * sl2 - m), O^T += V^T P^T.  Two
// key tiles per round (one max, one rescale, two independent MFMA chains),
// so that a round's dependent MFMA -> softmax -> MFMA chain covers twice
// the keys.
__device__ __forceinline__ void scores_tile(Acc &s, const unsigned char *kp, int kt, int c, int g,
                                            const bf16x8 (&qb)[2]) {
  zero(s);
  const int key = 32 * kt + xpi(c);
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    const bf16x8 a = *(const bf16x8 *)(kp + key * 64 + 16 * ((2 * s2 + g) ^ ((key >> 2) & 3)));
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[s2], s, 0, 0, 0);
  }
}
__device__ __forceinline__ void values_tile(Acc &o, const unsigned char *vp, int kt, int c, int g, const Acc &p) {
  const int dim = xpi(c);
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    const int ch = 4 * kt + 2 * s2 + g;   // 16-byte chunk of the keys of this k-step
    const bf16x8 a = *(const bf16x8 *)(vp + dim * 512 + 16 * (ch ^ (dim & 15)));
    o = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pack8(p, s2), o, 0, 0, 0);
  }
}
__device__ __forceinline__ void attend_piece(HeadState &st, const unsigned char *piece, int n_kt, int c, int g,
                                             const bf16x8 (&qb)[2], float sl2) {
  const unsigned char *kp = piece, *vp = piece + 16384;
  c = fresh(c);
  g = fresh(g);
  Acc o2;                                  // the second tile's chain, summed at the end
  zero(o2);
  for (int kt = 0; kt < n_kt; kt += 2) {
    const bool two = kt + 1 < n_kt;
    Acc s0, s1;
    scores_tile(s0, kp, kt, c, g, qb);
    if (two) scores_tile(s1, kp, kt + 1, c, g, qb);
    float mx = s0[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s0[i]);
    if (two) {
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s1[i]);
    }
    const float m_new = fmaxf(st.m, xor32_max(mx) * sl2);
    const float corr = fast_exp2(st.m - m_new);
    st.l *= corr;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      st.o[i] *= corr;
      o2[i] *= corr;
    }
    st.m = m_new;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s0[i] = fast_exp2(fmaf(s0[i], sl2, -m_new));
      st.l += s0[i];
    }
    values_tile(st.o, vp, kt, c, g, s0);
    if (two) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s1[i] = fast_exp2(fmaf(s1[i], sl2, -m_new));
        st.l += s1[i];
      }
      values_tile(o2, vp, kt + 1, c, g, s1);
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) st.o[i] += o2[i];
}

// ---- candidate kernel --------------------------------------------------------
struct XfCandP {
  const uint16_t *cand;     // [R][N][D] bf16
  const uint16_t *w_mat;    // [L][8 D^2] bf16
  const float *w_vec;       // [L][11 D] + [3 D + 1]
  const unsigned char *ukv; // user K/V pieces [R][L][H][n_kc][32 KB]
  float *score;             // [R][N]
  int R, N, L, n_kc, Lu;
  float sl2;                // log2(e) / sqrt(32)
};

// ---- candidate kernel, 16-candidate waves ------------------------------------
// The same computation on v_mfma_f32_16x16x32_bf16, with half the tokens per
// wave: 40 000 candidates are then 2500 half-size waves, and ten-wave
// workgroups (160 candidates, one per CU) leave at most three of them on a
// SIMD, against two full waves on the busiest SIMDs of the 32-wide form.
// Lane (c, q) = (lane & 15, lane >> 4) holds token c and, of every
// 32-feature block b, the features 32 b + 8 q + 4 e + i in t[e][i]: the
// output tile e of a product takes its A rows in the order
// rho(m, e) = 8 (m >> 2) + 4 e + (m & 3), so the lane's eight features of a
// block are the eight k-values it supplies as the B operand of the next
// product.  A token's statistics are in-lane sums plus the exchanges with
// the lanes 16 and 32 apart.  Weights and user keys / values use the LDS
// layouts of the 32-wide kernel.
__device__ __forceinline__ int xrho(int m, int e) { return 8 * (m >> 2) + 4 * e + (m & 3); }

// Combine x of lane l with x of lane l^16 (one v_permlane16_swap: the two
// results hold the values of the even and of the odd 16-lane row of each
// pair of rows).
__device__ __forceinline__ float xor16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float tok_sum(float x) { return xor32_sum(xor16_sum(x)); }
__device__ __forceinline__ float tok_max(float x) { return xor32_max(xor16_max(x)); }

struct Blk {
  f32x4 t[2];
};
__device__ __forceinline__ void bzero(Blk &b) {
#pragma unroll
  for (int i = 0; i < 4; ++i) b.t[0][i] = b.t[1][i] = 0.f;
}
__device__ __forceinline__ bf16x8 bpack(const Blk &b) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = (__bf16)b.t[0][i];
    r[4 + i] = (__bf16)b.t[1][i];
  }
  return r;
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

__device__ __forceinline__ void layer_norm16(const Blk (&x)[4], const float *gain, const float *bias, int q,
                                             bf16x8 (&h)[4]) {
  q = fresh(q);
  float s = 0.f;
#pragma unroll
  for (int ft = 0; ft < 4; ++ft)
#pragma unroll
    for (int i = 0; i < 4; ++i) s += x[ft].t[0][i] + x[ft].t[1][i];
  const float mean = tok_sum(s) * (1.f / kXD);
  float v = 0.f;
#pragma unroll
  for (int ft = 0; ft < 4; ++ft)
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float d = x[ft].t[e][i] - mean;
        v = fmaf(d, d, v);
      }
  const float rstd = 1.f / sqrtf(tok_sum(v) * (1.f / kXD) + 1e-5f);
#pragma unroll
  for (int ft = 0; ft < 4; ++ft) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int f0 = 32 * ft + 8 * q + 4 * e;
      const float4 gg = *(const float4 *)(gain + f0), bb = *(const float4 *)(bias + f0);
      r[4 * e + 0] = (__bf16)fmaf((x[ft].t[e][0] - mean) * rstd, gg.x, bb.x);
      r[4 * e + 1] = (__bf16)fmaf((x[ft].t[e][1] - mean) * rstd, gg.y, bb.y);
      r[4 * e + 2] = (__bf16)fmaf((x[ft].t[e][2] - mean) * rstd, gg.z, bb.z);
      r[4 * e + 3] = (__bf16)fmaf((x[ft].t[e][3] - mean) * rstd, gg.w, bb.w);
    }
    h[ft] = r;
  }
}

// x[ot] += W_o[32 ot + rho(c, e)][head h's 32 columns] . o_h: one k-step per
// output tile (the W_o column block layout of the 32-wide kernel)
__device__ __forceinline__ void oproj16(Blk (&x)[4], const unsigned char *wo, int c, int q, bf16x8 ob) {
  const int cf = fresh(c), qf = fresh(q);
#pragma unroll
  for (int ot = 0; ot < 4; ++ot)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int row = 32 * ot + xrho(cf, e);
      const bf16x8 a = *(const bf16x8 *)(wo + row * 64 + 16 * (qf ^ ((row >> 2) & 3)));
      x[ot].t[e] = mfma16(a, ob, x[ot].t[e]);
    }
}

// acc[t] += W[rows row0 + 32 t + rho(c, e)] . h for t < NT (K = 128, four
// k-steps outermost so that the 2 NT chains interleave on the MFMA pipe)
template <int NT>
__device__ __forceinline__ void gemm16(Blk (&acc)[NT], const unsigned char *w, int row0, int c, int q,
                                       const bf16x8 (&h)[4]) {
  const int cf = fresh(c), qf = fresh(q);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int row = row0 + 32 * t + xrho(cf, e);
        const bf16x8 a = *(const bf16x8 *)(w + row * 256 + 16 * ((4 * ks + qf) ^ (row & 15)));
        acc[t].t[e] = mfma16(a, h[ks], acc[t].t[e]);
      }
}

// add the bias of features f0 + 8 q + 4 e + i (b points at f0)
__device__ __forceinline__ void add_bias16(Blk &a, const float *b, int q) {
  q = fresh(q);
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const float4 v = *(const float4 *)(b + 8 * q + 4 * e);
    a.t[e][0] += v.x; a.t[e][1] += v.y; a.t[e][2] += v.z; a.t[e][3] += v.w;
  }
}

struct HeadState16 {
  Blk o;          // output dims of the head, unnormalised
  float m, l;     // running max (log2 units, the same in the token's four lanes) and this lane's partial sum
};

// S^T for the 16 keys 32 kt + rho(c', e) of a key tile: one MFMA over the
// head's 32 dims (K layout [key][32], chunk ^ (key >> 2) & 3)
__device__ __forceinline__ f32x4 scores16(const unsigned char *kp, int kt, int e, int c, int q, bf16x8 qb) {
  const int key = 32 * kt + xrho(c, e);
  const bf16x8 a = *(const bf16x8 *)(kp + key * 64 + 16 * (q ^ ((key >> 2) & 3)));
  f32x4 z;
#pragma unroll
  for (int i = 0; i < 4; ++i) z[i] = 0.f;
  return mfma16(a, qb, z);
}
// O^T += V^T P^T over the 32 keys of tile kt; p holds the weights of keys
// 32 kt + 8 q .. + 7 (V^T layout [32][key], chunk ^ dim & 15)
__device__ __forceinline__ void values16(Blk &o, const unsigned char *vp, int kt, int c, int q, bf16x8 p) {
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int dim = xrho(c, e), ch = 4 * kt + q;
    const bf16x8 a = *(const bf16x8 *)(vp + dim * 512 + 16 * (ch ^ (dim & 15)));
    o.t[e] = mfma16(a, p, o.t[e]);
  }
}
// one piece of user keys / values (n_kt tiles of 32 keys), two tiles a round
__device__ __forceinline__ void attend_piece16(HeadState16 &st, const unsigned char *piece, int n_kt, int c, int q,
                                               bf16x8 qb, float sl2) {
  const unsigned char *kp = piece, *vp = piece + 16384;
  c = fresh(c);
  q = fresh(q);
  Blk o2;                                  // the second tile's chain, summed at the end
  bzero(o2);
  for (int kt = 0; kt < n_kt; kt += 2) {
    const bool two = kt + 1 < n_kt;
    f32x4 s0[2], s1[2];
    s0[0] = scores16(kp, kt, 0, c, q, qb);
    s0[1] = scores16(kp, kt, 1, c, q, qb);
    if (two) {
      s1[0] = scores16(kp, kt + 1, 0, c, q, qb);
      s1[1] = scores16(kp, kt + 1, 1, c, q, qb);
    }
    float mx = s0[0][0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, s0[i >> 2][i & 3]);
    if (two) {
#pragma unroll
      for (int i = 0; i < 8; ++i) mx = fmaxf(mx, s1[i >> 2][i & 3]);
    }
    const float m_new = fmaxf(st.m, tok_max(mx) * sl2);
    const float corr = fast_exp2(st.m - m_new);
    st.l *= corr;
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        st.o.t[e][i] *= corr;
        o2.t[e][i] *= corr;
      }
    st.m = m_new;
    bf16x8 p0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float v = fast_exp2(fmaf(s0[i >> 2][i & 3], sl2, -m_new));
      st.l += v;
      p0[i] = (__bf16)v;
    }
    values16(st.o, vp, kt, c, q, p0);
    if (two) {
      bf16x8 p1;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float v = fast_exp2(fmaf(s1[i >> 2][i & 3], sl2, -m_new));
        st.l += v;
        p1[i] = (__bf16)v;
      }
      values16(o2, vp, kt + 1, c, q, p1);
    }
  }
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int i = 0; i < 4; ++i) st.o.t[e][i] += o2.t[e][i];
}

constexpr int kXCand16Waves = 10;

__global__ __launch_bounds__(kXCand16Waves * 64, 1) void xf_cand16_kernel(XfCandP p) {
  constexpr int NW = kXCand16Waves;
  __shared__ __attribute__((aligned(1024))) XfSmem sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, c = lane & 15;
  const int tiles = (p.N + 16 * NW - 1) / (16 * NW);
  const int r = blockIdx.x / tiles, tb = blockIdx.x % tiles;
  const int n = (tb * NW + wave) * 16 + c;
  const int nl = min(n, p.N - 1);
  // the residual stream of this lane's token, features 32 ft + 8 q + 4 e + i
  Blk x[4];
  {
    const uint16_t *src = p.cand + ((size_t)r * p.N + nl) * kXD + 8 * q;
#pragma unroll
    for (int ft = 0; ft < 4; ++ft) {
      const bf16x8 v = *(const bf16x8 *)(src + 32 * ft);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[ft].t[0][i] = (float)v[i];
        x[ft].t[1][i] = (float)v[4 + i];
      }
    }
  }

  // Pieces of a layer: per head h, its q, k, v weight rows (24 KB) with
  // the W_o columns of head h - 1 (8 KB; the layer's vectors come with
  // head 0), then its user keys/values (n_kc pieces); the W_o columns of the
  // last head; two FFN halves (W1 rows, W2 columns).  After the last layer
  // the final vectors.  The output projection is applied head by head, at
  // the piece after the head's attention.
  const int per_head = 1 + p.n_kc;
  const int per_layer = kXHeads * per_head + 5;
  const int n_pieces = p.L * per_layer + 1;
  const unsigned char *ukv_r = p.ukv + (size_t)r * p.L * kXHeads * p.n_kc * kXSlot;
  auto issue = [&](int pc) {
    if (pc >= n_pieces) return;
    unsigned char *slot = sm.ring[pc & 1];
    if (pc == n_pieces - 1) {
      dma_floats<NW>(sm.vec, p.w_vec + (size_t)p.L * kXLayerVec, 3 * kXD + 1, wave, lane);
      return;
    }
    const int l = pc / per_layer, q = pc % per_layer;
    const uint16_t *wm = p.w_mat + (size_t)l * kXMat;
    if (q < kXHeads * per_head) {
      const int h = q / per_head, j = q % per_head;
      if (j == 0) {
        if (h == 0) dma_floats<NW>(sm.vec, p.w_vec + (size_t)l * kXLayerVec, kXLayerVec, wave, lane);
        else dma_wo_cols<NW>(slot + 24576, wm + kMo, h - 1, wave, lane);
        dma_rows<NW>(slot, 96, [&](int i) { return wm + kMqkv + (size_t)((i >> 5) * kXD + 32 * h + (i & 31)) * kXD; },
                     wave, lane);
      } else {
        dma_copy<NW>(slot, ukv_r + ((size_t)(l * kXHeads + h) * p.n_kc + (j - 1)) * kXSlot, kXSlot, wave, lane);
      }
      return;
    }
    const int e = q - kXHeads * per_head;
    if (e == 0) {
      dma_wo_cols<NW>(slot, wm + kMo, kXHeads - 1, wave, lane);
    } else if ((e & 1) == 1) {
      const int fh = e >> 1;
      dma_rows<NW>(slot, 128, [&](int i) { return wm + kM1 + (size_t)(128 * fh + i) * kXD; }, wave, lane);
    } else {
      const int fh = (e >> 1) - 1;
      dma_rows<NW>(slot, 128, [&](int i) { return wm + kM2 + (size_t)i * kXFF + 128 * fh; }, wave, lane);
    }
  };
  // wait for piece pc (the only one in flight), make it visible, prefetch
  // the next one into the other slot
  auto step = [&](int pc) -> const unsigned char * {
    GR_WAIT_VMCNT_LGKM0(0);
    ring_barrier();
    issue(pc + 1);
    return sm.ring[pc & 1];
  };

  issue(0);
  int pc = 0;
  bf16x8 hB[4];
  for (int l = 0; l < p.L; ++l) {
    bf16x8 ob;                                         // the previous head's output
    for (int h = 0; h < kXHeads; ++h) {
      const unsigned char *w = step(pc++);
      if (h == 0) {
        layer_norm16(x, sm.vec + kVln1g, sm.vec + kVln1b, q, hB);
      } else {
        oproj16(x, w + 24576, c, q, ob);
        if (h == 1) {
#pragma unroll
          for (int ot = 0; ot < 4; ++ot) add_bias16(x[ot], sm.vec + kVbO + 32 * ot, q);
        }
      }
      Blk qkv[3];
      bzero(qkv[0]); bzero(qkv[1]); bzero(qkv[2]);
      gemm16<3>(qkv, w, 0, c, q, hB);
      add_bias16(qkv[0], sm.vec + kVbQKV + 32 * h, q);
      add_bias16(qkv[1], sm.vec + kVbQKV + kXD + 32 * h, q);
      add_bias16(qkv[2], sm.vec + kVbQKV + 2 * kXD + 32 * h, q);
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int i = 0; i < 4; ++i) ss = fmaf(qkv[0].t[e][i], qkv[1].t[e][i], ss);
      const float s_self = tok_sum(ss) * p.sl2;       // own key, log2 units
      const bf16x8 qb = bpack(qkv[0]);
      const Blk va = qkv[2];
      HeadState16 st;
      bzero(st.o);
      st.m = s_self;                                   // the own key starts the running max
      st.l = 0.f;
      for (int j = 0; j < p.n_kc; ++j) {
        const unsigned char *kv = step(pc++);
        attend_piece16(st, kv, min(8, (p.Lu - 256 * j) >> 5), c, q, qb, p.sl2);
      }
      // own key: p_self = exp2(s_self - m), counted once in the sum
      const float p_self = fast_exp2(s_self - st.m);
      const float inv = 1.f / (tok_sum(st.l) + p_self);
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int i = 0; i < 4; ++i) st.o.t[e][i] = (st.o.t[e][i] + p_self * va.t[e][i]) * inv;
      ob = bpack(st.o);
    }
    {
      const unsigned char *w = step(pc++);
      oproj16(x, w, c, q, ob);
      layer_norm16(x, sm.vec + kVln2g, sm.vec + kVln2b, q, hB);
    }
    for (int fh = 0; fh < 2; ++fh) {
      bf16x8 uB[4];
      {
        const unsigned char *w = step(pc++);
        Blk a[4];
#pragma unroll
        for (int ot = 0; ot < 4; ++ot) bzero(a[ot]);
        gemm16<4>(a, w, 0, c, q, hB);
#pragma unroll
        for (int ot = 0; ot < 4; ++ot) {
          add_bias16(a[ot], sm.vec + kVb1 + 128 * fh + 32 * ot, q);
#pragma unroll
          for (int e = 0; e < 2; ++e)
#pragma unroll
            for (int i = 0; i < 4; ++i) a[ot].t[e][i] = fmaxf(a[ot].t[e][i], 0.f);
          uB[ot] = bpack(a[ot]);
        }
      }
      const unsigned char *w = step(pc++);
      gemm16<4>(x, w, 0, c, q, uB);
      if (fh == 0) {
#pragma unroll
        for (int ot = 0; ot < 4; ++ot) add_bias16(x[ot], sm.vec + kVb2 + 32 * ot, q);
      }
    }
  }
  // final LayerNorm and the score head
  step(pc++);
  {
    const float *gain = sm.vec, *bias = sm.vec + kXD, *w = sm.vec + 2 * kXD;
    float s = 0.f;
#pragma unroll
    for (int ft = 0; ft < 4; ++ft)
#pragma unroll
      for (int i = 0; i < 4; ++i) s += x[ft].t[0][i] + x[ft].t[1][i];
    const float mean = tok_sum(s) * (1.f / kXD);
    float v = 0.f;
#pragma unroll
    for (int ft = 0; ft < 4; ++ft)
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float d = x[ft].t[e][i] - mean;
          v = fmaf(d, d, v);
        }
    const float rstd = 1.f / sqrtf(tok_sum(v) * (1.f / kXD) + 1e-5f);
    const int qf = fresh(q);
    float dot = 0.f;
#pragma unroll
    for (int ft = 0; ft < 4; ++ft)
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int f = 32 * ft + 8 * qf + 4 * e + i;
          dot = fmaf(fmaf((x[ft].t[e][i] - mean) * rstd, gain[f], bias[f]), w[f], dot);
        }
    dot = tok_sum(dot) + sm.vec[3 * kXD];
    if (q == 0 && n < p.N) p.score[(size_t)r * p.N + n] = dot;
  }
}

// ---- user kernel ---------------------------------------------------------------
// Per (request, layer) launch, one workgroup per 32 user tokens.  The four
// waves split every product of the layer instead of each wave running the
// whole layer for tokens of its own: wave h attends for head h (its user
// keys and values staged in its own 32 KB of LDS), wave w forms output
// features 32w .. 32w+31 of the output projection and of the second FFN
// product, hidden units 64w .. 64w+63 of the first, and head w's queries,
// keys and values.  Between the products the waves exchange their slices
// of the activations through LDS (the heads' outputs, the residual stream,
// the hidden units), in the same accumulator layout the products use.  The
// weight rows a wave multiplies are its own, so they come from L2 straight
// into registers.  Every wave holds the whole residual stream of the 32
// tokens (for the LayerNorms); between launches it waits in the workspace
// with the queries.
struct XfUserP {
  const uint16_t *user;     // [R][Lu][D] bf16
  const uint16_t *w_mat;
  const float *w_vec;
  unsigned char *ukv;       // user K/V pieces [R][L][H][n_kc][32 KB]
  float *xs;                // [R][Lu/32][64 lanes][64] fp32
  uint16_t *qs;             // [R][Lu/32][64 lanes][4 heads][16] bf16
  int R, L, n_kc, Lu, layer;
  float sl2;
};

constexpr int kXUserNW = kXHeads;          // one wave per head / per output slice
static_assert(kXD == 32 * kXUserNW, "one 32-feature tile per wave");

struct XfUserSmem {
  unsigned char kv[kXUserNW][kXSlot];     // wave w: head w's user K/V piece, then its exchange slices
  float vec_prev[kXVecBytes / 4];         // vectors of layer l - 1
  float vec[kXVecBytes / 4];              // vectors of layer l
};
// exchange slices inside a wave's kv region (after its attention): two
// buffers, used in turn, so that a slice is never rewritten while another
// wave may still read the previous one
constexpr int kXchg = 8192;

// A operand rows of a product read from global memory: row `row` of a
// row-major bf16 matrix with `ld` elements per row, k-step (ft, s) of the
// lane's half g: elements 32 ft + 16 s + 8 g .. +7 (the B operand layout).
__device__ __forceinline__ bf16x8 wrow8(const uint16_t *w, int row, int ld, int ft, int s, int g) {
  return *(const bf16x8 *)(w + (size_t)row * ld + 32 * ft + 16 * s + 8 * g);
}

__global__ __launch_bounds__(kXUserNW * 64) void xf_user_kernel(XfUserP p) {
  __shared__ __attribute__((aligned(1024))) XfUserSmem sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, c = lane & 31;
  const int n_ut = p.Lu / 32;
  const int r = blockIdx.x / n_ut, ut = blockIdx.x % n_ut;
  const int l = p.layer;
  float *xs = p.xs + (((size_t)r * n_ut + ut) * 64 + lane) * 64;
  uint16_t *qs = p.qs + (((size_t)r * n_ut + ut) * 64 + lane) * 64;
  unsigned char *ukv_r = p.ukv + (size_t)r * p.L * kXHeads * p.n_kc * kXSlot;
  unsigned char *mine = sm.kv[wave];
  const int pr = xpi(c);                   // this lane's row within a 32-row weight tile

  // ---- in stream order: the vectors of both layers (shared), this wave's
  // head's first user K/V piece of layer l - 1 (its own region)
  if (l > 0) {
    dma_floats<kXUserNW>(sm.vec_prev, p.w_vec + (size_t)(l - 1) * kXLayerVec, kXLayerVec, wave, lane);
    dma_copy<1>(mine, ukv_r + ((size_t)((l - 1) * kXHeads + wave) * p.n_kc) * kXSlot, kXSlot, 0, lane);
  }
  dma_floats<kXUserNW>(sm.vec, p.w_vec + (size_t)l * kXLayerVec, kXLayerVec, wave, lane);

  // the residual stream of token c (features 32 ft + 16 (i >> 3) + 8 g + (i & 7))
  Acc x[4];
  if (l == 0) {
    const uint16_t *src = p.user + ((size_t)r * p.Lu + 32 * ut + c) * kXD + 8 * g;
#pragma unroll
    for (int ft = 0; ft < 4; ++ft)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bf16x8 v = *(const bf16x8 *)(src + 32 * ft + 16 * s);
#pragma unroll
        for (int t = 0; t < 8; ++t) x[ft][8 * s + t] = (float)v[t];
      }
  } else {
#pragma unroll
    for (int ft = 0; ft < 4; ++ft)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const float4 v = *(const float4 *)(xs + 16 * ft + 4 * i4);
        x[ft][4 * i4] = v.x; x[ft][4 * i4 + 1] = v.y; x[ft][4 * i4 + 2] = v.z; x[ft][4 * i4 + 3] = v.w;
      }
  }
  GR_WAIT_VMCNT(0);
  ring_barrier();

  int xb = 0;                              // exchange buffer in use
  // write this wave's slice (n16 16-byte pieces a lane) and read every wave's
  auto publish = [&](const uint4 *v, int n16) {
    uint4 *dst = (uint4 *)(mine + xb * kXchg) + lane * n16;
    for (int i = 0; i < n16; ++i) dst[i] = v[i];
  };
  auto slice_of = [&](int w) -> const uint4 * { return (const uint4 *)(sm.kv[w] + xb * kXchg); };
  // x[ft] += the update slice wave ft published (every wave sums alike)
  auto add_slices = [&](Acc(&xx)[4]) {
#pragma unroll
    for (int ft = 0; ft < 4; ++ft) {
      const uint4 *d4 = slice_of(ft) + lane * 4;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 v = d4[q];
        xx[ft][4 * q] += __uint_as_float(v.x); xx[ft][4 * q + 1] += __uint_as_float(v.y);
        xx[ft][4 * q + 2] += __uint_as_float(v.z); xx[ft][4 * q + 3] += __uint_as_float(v.w);
      }
    }
  };

  bf16x8 hB[4][2];
  if (l > 0) {
    const uint16_t *wm = p.w_mat + (size_t)(l - 1) * kXMat;
    // ---- attention of head `wave` of layer l - 1 over every user key
    bf16x8 qb[2];
    qb[0] = *(const bf16x8 *)(qs + 16 * wave);
    qb[1] = *(const bf16x8 *)(qs + 16 * wave + 8);
    HeadState st;
    zero(st.o);
    st.m = -__builtin_inff();
    st.l = 0.f;
    for (int j = 0; j < p.n_kc; ++j) {
      if (j > 0) {
        // this wave's reads of the previous piece are done; the region is its own
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
        dma_copy<1>(mine, ukv_r + ((size_t)((l - 1) * kXHeads + wave) * p.n_kc + j) * kXSlot, kXSlot, 0, lane);
        GR_WAIT_VMCNT(0);
        asm volatile("" ::: "memory");
      }
      attend_piece(st, mine, min(8, (p.Lu - 256 * j) >> 5), c, g, qb, p.sl2);
    }
    const float inv = 1.f / xor32_sum(st.l);
#pragma unroll
    for (int i = 0; i < 16; ++i) st.o[i] *= inv;
    {
      const bf16x8 ob[2] = {pack8(st.o, 0), pack8(st.o, 1)};
      __builtin_amdgcn_s_waitcnt(0xC07F);     // done reading the K/V piece
      publish((const uint4 *)ob, 2);
    }
    // output projection rows of this wave's features, prefetched
    bf16x8 wo[4][2];
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int s = 0; s < 2; ++s) wo[h][s] = wrow8(wm + kMo, 32 * wave + pr, kXD, h, s, g);
    __syncthreads();
    // ---- update slice of the wave's features: W_o[features] . o (all heads) + b_o
    {
      Acc d;
      zero(d);
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const uint4 *o4 = slice_of(h) + lane * 2;
#pragma unroll
        for (int s = 0; s < 2; ++s) d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wo[h][s], __builtin_bit_cast(bf16x8, o4[s]), d, 0, 0, 0);
      }
      add_bias(d, sm.vec_prev + kVbO + 32 * wave, g);
      xb ^= 1;
      publish((const uint4 *)&d, 4);
    }
    // first FFN product rows of this wave's hidden units, prefetched
    bf16x8 w1[2][4][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int ft = 0; ft < 4; ++ft)
#pragma unroll
        for (int s = 0; s < 2; ++s) w1[t][ft][s] = wrow8(wm + kM1, 64 * wave + 32 * t + pr, kXD, ft, s, g);
    // ---- every wave adds every wave's slice of the update
    __syncthreads();
    add_slices(x);
    // ---- FFN: hidden units 64 wave .. of ReLU(W1 LN2(x) + b1)
    layer_norm_b(x, sm.vec_prev + kVln2g, sm.vec_prev + kVln2b, g, hB);
    {
      bf16x8 ub[2][2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        Acc a;
        zero(a);
#pragma unroll
        for (int ft = 0; ft < 4; ++ft)
#pragma unroll
          for (int s = 0; s < 2; ++s) a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w1[t][ft][s], hB[ft][s], a, 0, 0, 0);
        add_bias(a, sm.vec_prev + kVb1 + 64 * wave + 32 * t, g);
#pragma unroll
        for (int i = 0; i < 16; ++i) a[i] = fmaxf(a[i], 0.f);
        ub[t][0] = pack8(a, 0);
        ub[t][1] = pack8(a, 1);
      }
      xb ^= 1;
      publish((const uint4 *)ub, 4);
    }
    // second FFN product rows of this wave's features, prefetched
    bf16x8 w2[8][2];
#pragma unroll
    for (int tt = 0; tt < 8; ++tt)
#pragma unroll
      for (int s = 0; s < 2; ++s) w2[tt][s] = wrow8(wm + kM2, 32 * wave + pr, kXFF, tt, s, g);
    __syncthreads();
    // ---- update slice of the wave's features: W2[features] . hidden (all 256) + b2
    {
      Acc d;
      zero(d);
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const uint4 *u4 = slice_of(tt >> 1) + lane * 4 + 2 * (tt & 1);
#pragma unroll
        for (int s = 0; s < 2; ++s) d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w2[tt][s], __builtin_bit_cast(bf16x8, u4[s]), d, 0, 0, 0);
      }
      add_bias(d, sm.vec_prev + kVb2 + 32 * wave, g);
      xb ^= 1;
      publish((const uint4 *)&d, 4);
    }
    __syncthreads();
    add_slices(x);
  }
  // ---- layer l: head `wave`'s queries, keys and values of the 32 tokens
  {
    const uint16_t *wq = p.w_mat + (size_t)l * kXMat + kMqkv;
    bf16x8 wa[3][4][2];
#pragma unroll
    for (int m = 0; m < 3; ++m)
#pragma unroll
      for (int ft = 0; ft < 4; ++ft)
#pragma unroll
        for (int s = 0; s < 2; ++s) wa[m][ft][s] = wrow8(wq, m * kXD + 32 * wave + pr, kXD, ft, s, g);
    layer_norm_b(x, sm.vec + kVln1g, sm.vec + kVln1b, g, hB);
    Acc a[3];
#pragma unroll
    for (int m = 0; m < 3; ++m) zero(a[m]);
#pragma unroll
    for (int ft = 0; ft < 4; ++ft)
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int m = 0; m < 3; ++m) a[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa[m][ft][s], hB[ft][s], a[m], 0, 0, 0);
#pragma unroll
    for (int m = 0; m < 3; ++m) add_bias(a[m], sm.vec + kVbQKV + m * kXD + 32 * wave, g);
    const int key = 32 * ut + c, kc = key >> 8, kl = key & 255;
    unsigned char *piece = ukv_r + ((size_t)(l * kXHeads + wave) * p.n_kc + kc) * kXSlot;
    // q: the B operand of the next launch's scores
    *(bf16x8 *)(qs + 16 * wave) = pack8(a[0], 0);
    *(bf16x8 *)(qs + 16 * wave + 8) = pack8(a[0], 1);
    // k: K [key][32], this lane's dims 16 s + 8 g .. +7 are one 16-byte chunk
#pragma unroll
    for (int s = 0; s < 2; ++s)
      *(bf16x8 *)(piece + kl * 64 + 16 * ((2 * s + g) ^ ((kl >> 2) & 3))) = pack8(a[1], s);
    // v: V^T [dim][key], one bf16 per (dim, key)
    uint16_t *vt = (uint16_t *)(piece + 16384);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int dim = 16 * (i >> 3) + 8 * g + (i & 7);
      const __bf16 b = (__bf16)a[2][i];
      vt[dim * 256 + 8 * ((kl >> 3) ^ (dim & 15)) + (kl & 7)] = *(const uint16_t *)&b;
    }
  }
  // the residual stream for the next launch (every wave holds all of it)
  if (wave == 0 && l + 1 < p.L) {
#pragma unroll
    for (int ft = 0; ft < 4; ++ft)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        *(float4 *)(xs + 16 * ft + 4 * i4) =
            make_float4(x[ft][4 * i4], x[ft][4 * i4 + 1], x[ft][4 * i4 + 2], x[ft][4 * i4 + 3]);
  }
}

}  // namespace

size_t xf_user_state_bytes(int R, int Lu) { return (size_t)R * (Lu / 32) * 64 * (64 * 4 + 64 * 2); }
size_t xf_ukv_bytes(int R, int L, int Lu) { return (size_t)R * L * kXHeads * ((Lu + 255) / 256) * kXSlot; }

hipError_t launch_xf_scores(const XfArgs &a, hipStream_t s) {
  const int n_kc = (a.Lu + 255) / 256;
  const int n_ut = a.Lu / 32;
  XfUserP u;
  u.user = (const uint16_t *)a.user; u.w_mat = (const uint16_t *)a.w_mat; u.w_vec = a.w_vec;
  u.ukv = (unsigned char *)a.ukv;
  u.xs = (float *)a.user_state;
  u.qs = (uint16_t *)((char *)a.user_state + (size_t)a.R * n_ut * 64 * 64 * 4);
  u.R = a.R; u.L = a.L; u.n_kc = n_kc; u.Lu = a.Lu;
  u.sl2 = kXLog2e / sqrtf((float)kXHd);
  for (int l = 0; l < a.L; ++l) {
    u.layer = l;
    hipLaunchKernelGGL(xf_user_kernel, dim3((unsigned)(a.R * n_ut)), dim3(kXUserNW * 64), 0, s, u);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  XfCandP c;
  c.cand = (const uint16_t *)a.cand; c.w_mat = (const uint16_t *)a.w_mat; c.w_vec = a.w_vec;
  c.ukv = (const unsigned char *)a.ukv;
  c.score = a.score;
  c.R = a.R; c.N = a.N; c.L = a.L; c.n_kc = n_kc; c.Lu = a.Lu;
  c.sl2 = u.sl2;
  const int tiles = (a.N + 16 * kXCand16Waves - 1) / (16 * kXCand16Waves);
  hipLaunchKernelGGL(xf_cand16_kernel, dim3((unsigned)(a.R * tiles)), dim3(kXCand16Waves * 64), 0, s, c);
  return hipGetLastError();
}

}  // namespace gr
