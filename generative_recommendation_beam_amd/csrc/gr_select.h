// Block-wide exact top-k selection over candidates held in LDS.
//
// Candidate selection on the GPU (TransRetrieval, GPU retrieval) for the
// 256-way beam search (Engineering Exploration of Generative Recall, 4.2).
// Every candidate has a unique 64-bit composite key
//     comp = rank_key(score) << 32 | flat index,
// so "best k by score, ties by lower index" is "k smallest composites".
// The k-th smallest is found by MSB-first radix select (8-bit digits,
// starting at the highest bit where the composites differ), with per-wave
// histograms in LDS.  As soon as the bucket holding the k-th candidate has at
// most kBinCap members the loop stops; everything below that bucket is taken,
// the bucket is sorted (bitonic) and its first `need` members complete the
// set, which is then sorted (bitonic) into the output order.  Integer counts
// only, so the result is deterministic.
#pragma once

#include "gr_device.h"

namespace gr {

constexpr int kBinCap = 512;      // bucket size that is sorted directly
constexpr int kMaxK = GR_MAX_K;   // 2048

// LDS scratch of the selection (one union: histograms during the radix
// passes, bucket + output lists afterwards).
template <int NT>
struct SelectSmem {
  static constexpr int NW = NT / 64;
  union {
    uint32_t hist[NW][256];
    struct {
      uint64_t bin[kBinCap];
      uint64_t out[kMaxK];
    } l;
  } u;
  uint32_t wave_tot[NW];
  uint64_t cmin, cmax, prefix;
  int fixed_lo, need, bin_cnt, n_out, n_bin;
  uint64_t red[NW];
  uint64_t red2[NW];
};

__device__ __forceinline__ uint64_t comp_of(const uint32_t *rk, const uint32_t *ix, uint32_t base, int i) {
  return ((uint64_t)rk[i] << 32) | (uint64_t)(ix ? ix[i] : (base + (uint32_t)i));
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m), hi = __shfl_xor((uint32_t)(v >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}

// Ascending bitonic sort of arr[0..P) (P a power of two, padded with ~0).
template <int NT>
__device__ void bitonic_sort_u64(uint64_t *arr, int P) {
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < (P >> 1); i += NT) {
        const int pos = 2 * i - (i & (stride - 1));
        const int partner = pos + stride;
        const bool up = (pos & size) == 0;
        const uint64_t a = arr[pos], b = arr[partner];
        if ((a > b) == up) { arr[pos] = b; arr[partner] = a; }
      }
      __syncthreads();
    }
  }
}

__device__ __forceinline__ int pow2_ceil(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// Selects the k smallest composites among n candidates (rk[i], ix[i] or
// base + i) and leaves them sorted ascending in sm.u.l.out[0..k).  Requires
// 1 <= k <= min(n, kMaxK).  All threads of the block must call it.
template <int NT>
__device__ void block_select(const uint32_t *rk, const uint32_t *ix, uint32_t base, int n, int k,
                             SelectSmem<NT> &sm) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

  // min / max composite
  uint64_t mn = ~0ull, mx = 0ull;
  for (int i = tid; i < n; i += NT) {
    const uint64_t x = comp_of(rk, ix, base, i);
    mn = x < mn ? x : mn;
    mx = x > mx ? x : mx;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t a = shfl_xor_u64(mn, o), b = shfl_xor_u64(mx, o);
    mn = a < mn ? a : mn;
    mx = b > mx ? b : mx;
  }
  if (lane == 0) { sm.red[wave] = mn; sm.red2[wave] = mx; }
  __syncthreads();
  if (tid == 0) {
    uint64_t a = sm.red[0], b = sm.red2[0];
    for (int w = 1; w < NW; ++w) {
      a = sm.red[w] < a ? sm.red[w] : a;
      b = sm.red2[w] > b ? sm.red2[w] : b;
    }
    const uint64_t diff = a ^ b;
    const int lo = diff ? 64 - __builtin_clzll(diff) : 0;
    sm.cmin = a;
    sm.cmax = b;
    sm.fixed_lo = lo;
    sm.prefix = lo >= 64 ? 0ull : (a & ~((1ull << lo) - 1ull));
    sm.need = k;
    sm.bin_cnt = n;
  }
  __syncthreads();

  // radix passes until the bucket of the k-th candidate is small
  static_assert(NT >= 256 && NT % 64 == 0, "the bin scan needs >= 256 threads");
  // each pass fixes up to 8 more bits of a 64-bit key: at most 8 passes
  for (int pass = 0; pass < 8 && sm.fixed_lo > 0 && sm.bin_cnt > kBinCap && k < n; ++pass) {
    const int fixed_lo = sm.fixed_lo;
    const uint32_t need = (uint32_t)sm.need;
    const int shift = fixed_lo > 8 ? fixed_lo - 8 : 0;
    const int nbins = 1 << (fixed_lo - shift);
    const uint64_t pre = fixed_lo >= 64 ? 0ull : (sm.prefix >> fixed_lo);
    for (int i = tid; i < NW * 256; i += NT) (&sm.u.hist[0][0])[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += NT) {
      const uint64_t x = comp_of(rk, ix, base, i);
      const uint64_t hi = fixed_lo >= 64 ? 0ull : (x >> fixed_lo);
      if (hi == pre) atomicAdd(&sm.u.hist[wave][(int)((x >> shift) & (uint64_t)(nbins - 1))], 1u);
    }
    __syncthreads();
    // bins 0..255: total over waves, inclusive scan across the block
    uint32_t cnt = 0;
    if (tid < 256) {
#pragma unroll
      for (int w = 0; w < NW; ++w) cnt += sm.u.hist[w][tid];
    }
    uint32_t inc = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t v = __shfl_up(inc, o);
      if (lane >= o) inc += v;
    }
    if (lane == 63 && wave < 4) sm.wave_tot[wave] = inc;
    __syncthreads();
    if (tid < 256) {
      uint32_t before_wave = 0;
      for (int w = 0; w < wave; ++w) before_wave += sm.wave_tot[w];
      inc += before_wave;
      const uint32_t excl = inc - cnt;
      if (cnt > 0 && excl < need && need <= inc) {
        sm.need = (int)(need - excl);
        sm.prefix |= ((uint64_t)tid) << shift;
        sm.fixed_lo = shift;
        sm.bin_cnt = (int)cnt;
      }
    }
    __syncthreads();
  }

  // compaction: everything below the bucket is taken, the bucket is sorted
  const int fixed_lo = sm.fixed_lo;
  const uint64_t lo_bound = sm.prefix;
  const uint64_t hi_bound = fixed_lo >= 64 ? ~0ull : lo_bound + ((1ull << fixed_lo) - 1ull);
  const bool take_all = k >= n;
  if (tid == 0) { sm.n_out = 0; sm.n_bin = 0; }
  __syncthreads();
  for (int i0 = 0; i0 < n; i0 += NT) {
    const int i = i0 + tid;
    const uint64_t x = i < n ? comp_of(rk, ix, base, i) : ~0ull;
    const bool to_out = i < n && (take_all || x < lo_bound);
    const bool to_bin = i < n && !to_out && x <= hi_bound;
    const uint64_t below = __lanemask_lt();
    const uint64_t mo = __ballot(to_out), mb = __ballot(to_bin);
    int bo = 0, bb = 0;
    if (lane == 0) {
      if (mo) bo = atomicAdd(&sm.n_out, (int)__popcll(mo));
      if (mb) bb = atomicAdd(&sm.n_bin, (int)__popcll(mb));
    }
    bo = __shfl(bo, 0);
    bb = __shfl(bb, 0);
    const int so = bo + (int)__popcll(mo & below), sb = bb + (int)__popcll(mb & below);
    if (to_out && so < kMaxK) sm.u.l.out[so] = x;
    if (to_bin && sb < kBinCap) sm.u.l.bin[sb] = x;
  }
  __syncthreads();
  if (!take_all) {
    const int nb = min(sm.n_bin, kBinCap);
    const int P = pow2_ceil(nb);
    for (int i = nb + tid; i < P; i += NT) sm.u.l.bin[i] = ~0ull;
    __syncthreads();
    bitonic_sort_u64<NT>(sm.u.l.bin, P);
    const int off = sm.n_out;
    const int need = sm.need;
    for (int i = tid; i < need && i < nb && off + i < kMaxK; i += NT) sm.u.l.out[off + i] = sm.u.l.bin[i];
    __syncthreads();
  }
  const int P = pow2_ceil(k);
  for (int i = k + tid; i < P; i += NT) sm.u.l.out[i] = ~0ull;
  __syncthreads();
  bitonic_sort_u64<NT>(sm.u.l.out, P);
}

// Writes the sorted selection of k_sel candidates: the final outputs (one
// group per request) or this group's partial list of kk entries (entries past
// k_sel are ~0, which sorts after every real candidate).
template <int NT>
__device__ void emit_selection(const SelectSmem<NT> &sm, int k_sel, int r, int grp, int vocab,
                               float *score, int32_t *token, int32_t *parent, uint64_t *partial,
                               int n_groups, int kk) {
  if (n_groups == 1) {
    for (int j = threadIdx.x; j < k_sel; j += NT) {
      const uint64_t x = sm.u.l.out[j];
      const uint32_t f = (uint32_t)x;
      score[(size_t)r * k_sel + j] = key_score((uint32_t)(x >> 32));
      token[(size_t)r * k_sel + j] = (int32_t)(f % (uint32_t)vocab);
      parent[(size_t)r * k_sel + j] = (int32_t)(f / (uint32_t)vocab);
    }
  } else {
    for (int j = threadIdx.x; j < kk; j += NT)
      partial[((size_t)r * n_groups + grp) * kk + j] = j < k_sel ? sm.u.l.out[j] : ~0ull;
  }
}

}  // namespace gr
