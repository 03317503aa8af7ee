// Device-side helpers shared by the gfx950 kernels of the decode step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gr_beam.h"

namespace gr {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round-to-nearest-even fp32 -> bf16 (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}
// Two fp32 -> one packed bf16 pair (one v_cvt_pk_bf16_f32, round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
// lo + hi of a packed bf16 pair added to acc in fp32 (v_dot2c_f32_bf16 with (1, 1)).
__device__ __forceinline__ float add_bf16x2(uint32_t packed, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed), one, acc, false);
}

// Dot product of 8 bf16 pairs held as two uint4 (fp32 accumulate, four
// v_dot2_f32_bf16).
__device__ __forceinline__ float dot8_bf16(uint4 a, uint4 b) {
  float s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.x), __builtin_bit_cast(bf16x2, b.x), 0.f, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.y), __builtin_bit_cast(bf16x2, b.y), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.z), __builtin_bit_cast(bf16x2, b.z), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.w), __builtin_bit_cast(bf16x2, b.w), s, false);
  return s;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- HBM -> LDS streaming (global_load_lds)
#define GR_LDS(p) ((__attribute__((address_space(3))) void *)(p))
#ifndef GR_STREAM_POLICY
#define GR_STREAM_POLICY "nt"
#endif

// s_waitcnt with only the vector-memory counter constrained to <= n.
#define GR_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))
// The same, and every LDS access of this wave completed (lgkmcnt 0).
#define GR_WAIT_VMCNT_LGKM0(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4))

// One global_load_lds_dwordx4: lane l's 16 bytes at src land at LDS byte
// lds + 16*l (lds wave-uniform).  Written as inline asm so that the compiler
// does not track these LDS writes: its own wait insertion would otherwise
// turn into vmcnt(0) before every LDS read once several ring stages have DMAs
// in flight.  Every read of DMA'd data is instead preceded by an explicit
// vmcnt wait and a barrier (ring_barrier below).  No VGPR is written, so
// nothing is left for the compiler to misjudge.  M0 (reserved by the
// compiler) is saved and restored around the load, and needs one wait state
// before the load reads it.  The LDS address goes through readfirstlane: it
// is wave-uniform, but the compiler cannot always prove it and would then
// hold it in a vector register, which the scalar move cannot take.
__device__ __forceinline__ void dma16(const void *src, const void *lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)GR_LDS(lds));
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(m0), "v"(src)
      : "memory");
}
// Streaming variant (read once): non-temporal cache policy.
__device__ __forceinline__ void dma16_stream(const void *src, const void *lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)GR_LDS(lds));
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off " GR_STREAM_POLICY "\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(m0), "v"(src)
      : "memory");
}
// The same for one dword per lane (global_load_lds_dword): lane l's 4 bytes
// land at LDS byte lds + 4*l.
__device__ __forceinline__ void dma4(const void *src, const void *lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)GR_LDS(lds));
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(m0), "v"(src)
      : "memory");
}
// Workgroup barrier that also keeps the compiler from moving LDS reads above
// it (DMA'd data is only valid past the wait + barrier).
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}


// Ordering key of a score: a smaller key means a larger score.  -0 is folded
// into +0 and NaN ranks like -inf, so the order is total on real scores.
__device__ __forceinline__ uint32_t rank_key(float s) {
  if (s != s) s = -__builtin_inff();
  s = s + 0.0f;
  const uint32_t u = __float_as_uint(s);
  const uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ~asc;
}
__device__ __forceinline__ float key_score(uint32_t rk) {
  const uint32_t asc = ~rk;
  const uint32_t u = (asc & 0x80000000u) ? (asc & 0x7FFFFFFFu) : ~asc;
  return __uint_as_float(u);
}

// Combine x of lane l with x of lane l^32 (one v_permlane32_swap: the two
// results hold the lower and the upper half-wave's values in every lane).
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---- VALU-only cross-lane exchanges (DPP and permlane swaps; no LDS pipe)
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
}
// value held by lane l ^ S, S in {1, 2, 4, 8}: quad permutes and row mirrors
// (xor 4 = half-mirror then quad reverse, xor 8 = mirror then half-mirror)
template <int S>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
  static_assert(S == 1 || S == 2 || S == 4 || S == 8, "DPP xor distance");
  if constexpr (S == 1) return dpp_u32<0xB1>(v);                     // quad_perm [1,0,3,2]
  else if constexpr (S == 2) return dpp_u32<0x4E>(v);                // quad_perm [2,3,0,1]
  else if constexpr (S == 4) return dpp_u32<0x1B>(dpp_u32<0x141>(v));  // row_half_mirror, quad_perm [3,2,1,0]
  else return dpp_u32<0x141>(dpp_u32<0x140>(v));                     // row_mirror, row_half_mirror
}
// {value of lane l, value of lane l ^ S} for S in {16, 32}, in a lane-
// dependent order (one v_permlane16_swap / v_permlane32_swap): enough for
// min, max and sums, which do not care which is which.
template <int S>
__device__ __forceinline__ void xor_pair(uint32_t v, uint32_t &a, uint32_t &b) {
  static_assert(S == 16 || S == 32, "permlane swap distance");
  if constexpr (S == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    a = r[0]; b = r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    a = r[0]; b = r[1];
  }
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, xor_lane<1>(v));
  v = min(v, xor_lane<2>(v));
  v = min(v, xor_lane<4>(v));
  v = min(v, xor_lane<8>(v));
  uint32_t a, b;
  xor_pair<16>(v, a, b);
  v = min(a, b);
  xor_pair<32>(v, a, b);
  return min(a, b);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, xor_lane<1>(v));
  v = max(v, xor_lane<2>(v));
  v = max(v, xor_lane<4>(v));
  v = max(v, xor_lane<8>(v));
  uint32_t a, b;
  xor_pair<16>(v, a, b);
  v = max(a, b);
  xor_pair<32>(v, a, b);
  return max(a, b);
}
// Inclusive prefix sum over the wave (row shifts within 16-lane rows, then
// the row totals broadcast into the rows above).
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
  v += dpp_u32<0x111>(v);          // row_shr:1
  v += dpp_u32<0x112>(v);          // row_shr:2
  v += dpp_u32<0x114>(v);          // row_shr:4
  v += dpp_u32<0x118>(v);          // row_shr:8
  v += dpp_u32<0x142, 0xA>(v);     // row_bcast:15 into rows 1 and 3
  v += dpp_u32<0x143, 0xC>(v);     // row_bcast:31 into rows 2 and 3
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

}  // namespace gr
