// Block-wide exact top-k selection over candidates held in registers.
//
// Candidate selection on the GPU (TransRetrieval, GPU retrieval) for the
// 256-way beam search (Engineering Exploration of Generative Recall, 4.2).
// Every candidate has a unique 64-bit composite key
//     comp = rank_key(score) << 32 | flat index,
// so "best k by score, ties by lower index" is "k smallest composites".
//
// Each thread holds J candidates in registers (rank key + a way to name its
// index).  The k-th smallest composite is located by MSB-first radix passes
// of 11-bit digits that start at the highest bit where the keys differ; each
// pass histograms the candidates still in play with non-returning LDS atomics
// and one block scan picks the bucket holding the k-th.  As soon as that
// bucket has at most kBucketCap members, every candidate at or below the
// bucket is copied to an LDS list (two ballot sweeps, one atomic per wave),
// and one bitonic sort orders the list; its first k entries are the answer.
// Integer counts only, so the result is deterministic.
#pragma once

#include "gr_device.h"

namespace gr {

constexpr uint32_t kInvalidKey = 0xFFFFFFFFu;   // empty register slot (never a real key)
constexpr int kHistBits = 11;
constexpr int kHistBins = 1 << kHistBits;
constexpr int kBucketCap = 512;
constexpr int kListCap = 4096;                  // >= GR_MAX_K + kBucketCap, power of two
constexpr int kMaxK = GR_MAX_K;

template <int NT>
struct SelectSmem {
  static constexpr int NW = NT / 64;
  union {
    uint32_t hist[kHistBins];
    uint64_t list[kListCap];
  } u;
  uint32_t wmin[NW], wmax[NW], wtot[NW];
  uint64_t prefix;
  int fixed_lo, need, bucket_cnt, n_list;
};

__device__ __forceinline__ int pow2_ceil(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// Ascending bitonic sort of arr[0..P) (P a power of two).
template <int NT>
__device__ __forceinline__ void bitonic_sort_u64(uint64_t *arr, int P) {
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

// The same sort for P <= NT entries, one per thread, in registers: strides
// below 64 exchange through lane shuffles, larger ones through LDS.  Entries
// L..P-1 are padding (~0).  The sorted list is written back to arr[0..P).
template <int NT>
__device__ __forceinline__ void bitonic_sort_u64_reg(uint64_t *arr, int L, int P) {
  const int tid = threadIdx.x;
  uint64_t x = tid < L ? arr[tid] : ~0ull;
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      uint64_t y;
      if (stride >= 64) {
        __syncthreads();
        if (tid < P) arr[tid] = x;
        __syncthreads();
        y = tid < P ? arr[tid ^ stride] : ~0ull;
      } else {
        const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)x, stride);
        const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(x >> 32), stride);
        y = ((uint64_t)hi << 32) | lo;
      }
      const bool up = (tid & size) == 0, lower = (tid & stride) == 0;
      x = (lower == up) ? (x < y ? x : y) : (x < y ? y : x);
    }
  }
  __syncthreads();
  if (tid < P) arr[tid] = x;
  __syncthreads();
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}

// Selects the k smallest composites among the valid register candidates of
// the block (key[j] != kInvalidKey; the index of slot j is idx_of(j)).  n_valid
// is their number, 1 <= k <= min(n_valid, kMaxK).  On return the first k
// entries of sm.u.list hold them in ascending order.  All threads call it.
// Always inlined: the candidates must stay in registers (a call would pass
// them through scratch memory).
template <int NT, int J, typename IdxFn>
__device__ __forceinline__ void select_regs(const uint32_t (&key)[J], IdxFn idx_of, int n_valid, int k, SelectSmem<NT> &sm) {
  static_assert(NT % 64 == 0 && kHistBins % NT == 0, "block size");
  constexpr int NW = NT / 64;
  constexpr int BPT = kHistBins / NT;   // histogram bins scanned per thread
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

  // ---- range of the keys: the bits above their highest difference are common
  uint32_t kmin = kInvalidKey, kmax = 0u;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    if (key[j] != kInvalidKey) {
      kmin = min(kmin, key[j]);
      kmax = max(kmax, key[j]);
    }
  }
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  if (lane == 0) { sm.wmin[wave] = kmin; sm.wmax[wave] = kmax; }
  __syncthreads();
  if (tid == 0) {
    uint32_t a = sm.wmin[0], b = sm.wmax[0];
    for (int w = 1; w < NW; ++w) { a = min(a, sm.wmin[w]); b = max(b, sm.wmax[w]); }
    const uint32_t diff = a ^ b;
    const int lo = diff ? 64 - __builtin_clz(diff) : 32;   // key bits differ, or only the index does
    sm.fixed_lo = lo;
    sm.prefix = lo >= 64 ? 0ull : (((uint64_t)a << 32) & ~((1ull << lo) - 1ull));
    sm.need = k;
    sm.bucket_cnt = n_valid;
    sm.n_list = 0;
  }
  __syncthreads();

  // ---- radix passes over the bucket of the k-th candidate
  for (int pass = 0; pass < 8; ++pass) {
    const int fixed_lo = sm.fixed_lo;
    const uint32_t need = (uint32_t)sm.need;
    if (fixed_lo == 0 || sm.bucket_cnt <= kBucketCap) break;
    const int shift = fixed_lo > kHistBits ? fixed_lo - kHistBits : 0;
    const uint32_t mask = (1u << (fixed_lo - shift)) - 1u;
    const uint64_t pre = fixed_lo >= 64 ? 0ull : (sm.prefix >> fixed_lo);
    for (int i = tid; i < kHistBins; i += NT) sm.u.hist[i] = 0;
    __syncthreads();
    if (shift >= 32) {
      // digit and prefix lie in the score key: 32-bit arithmetic only
      const int fl = fixed_lo - 32, sh = shift - 32;
      const uint32_t pre32 = (uint32_t)pre;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const uint32_t kj = key[j];
        const bool in = kj != kInvalidKey && (fl >= 32 || (kj >> fl) == pre32);
        if (in) atomicAdd(&sm.u.hist[(kj >> sh) & mask], 1u);
      }
    } else {
#pragma unroll
      for (int j = 0; j < J; ++j) {
        if (key[j] != kInvalidKey) {
          const uint64_t x = ((uint64_t)key[j] << 32) | idx_of(j);
          const uint64_t hi = fixed_lo >= 64 ? 0ull : (x >> fixed_lo);
          if (hi == pre) atomicAdd(&sm.u.hist[(uint32_t)(x >> shift) & mask], 1u);
        }
      }
    }
    __syncthreads();
    uint32_t c[BPT], s = 0;
#pragma unroll
    for (int q = 0; q < BPT; ++q) { c[q] = sm.u.hist[tid * BPT + q]; s += c[q]; }
    uint32_t inc = s;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t v = (uint32_t)__shfl_up((int)inc, o);
      if (lane >= o) inc += v;
    }
    if (lane == 63) sm.wtot[wave] = inc;
    __syncthreads();
    uint32_t excl = inc - s;
    for (int w = 0; w < wave; ++w) excl += sm.wtot[w];
    if (excl < need && need <= excl + s) {
#pragma unroll
      for (int q = 0; q < BPT; ++q) {
        if (c[q] > 0 && excl < need && need <= excl + c[q]) {
          sm.need = (int)(need - excl);
          sm.prefix |= ((uint64_t)(tid * BPT + q)) << shift;
          sm.fixed_lo = shift;
          sm.bucket_cnt = (int)c[q];
        }
        excl += c[q];
      }
    }
    __syncthreads();
  }

  // ---- everything at or below the bucket goes to the list
  const int fixed_lo = sm.fixed_lo;
  const uint64_t hi_bound = fixed_lo >= 64 ? ~0ull : (sm.prefix | ((1ull << fixed_lo) - 1ull));
  // With the bucket boundary inside the score key, the index half of
  // hi_bound is all ones and one 32-bit compare decides.
  const uint64_t below = __lanemask_lt();
  if (fixed_lo >= 32) {
    const uint32_t hi32 = (uint32_t)(hi_bound >> 32);
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < J; ++j) cnt += (int)__popcll(__ballot(key[j] <= hi32 && key[j] != kInvalidKey));
    int base = 0;
    if (lane == 0 && cnt) base = atomicAdd(&sm.n_list, cnt);
    base = __shfl(base, 0);
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const bool sel = key[j] <= hi32 && key[j] != kInvalidKey;
      const uint64_t m = __ballot(sel);
      const int at = base + (int)__popcll(m & below);
      if (sel && at < kListCap) sm.u.list[at] = ((uint64_t)key[j] << 32) | idx_of(j);
      base += (int)__popcll(m);
    }
  } else {
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const bool sel = key[j] != kInvalidKey && ((((uint64_t)key[j] << 32) | idx_of(j)) <= hi_bound);
      cnt += (int)__popcll(__ballot(sel));
    }
    int base = 0;
    if (lane == 0 && cnt) base = atomicAdd(&sm.n_list, cnt);
    base = __shfl(base, 0);
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const uint64_t x = ((uint64_t)key[j] << 32) | idx_of(j);
      const bool sel = key[j] != kInvalidKey && x <= hi_bound;
      const uint64_t m = __ballot(sel);
      const int at = base + (int)__popcll(m & below);
      if (sel && at < kListCap) sm.u.list[at] = x;
      base += (int)__popcll(m);
    }
  }
  __syncthreads();
  const int L = min(sm.n_list, kListCap);
  const int P = pow2_ceil(max(L, k));
  if (P <= NT) {
    bitonic_sort_u64_reg<NT>(sm.u.list, L, P);
  } else {
    for (int i = L + tid; i < P; i += NT) sm.u.list[i] = ~0ull;
    __syncthreads();
    bitonic_sort_u64<NT>(sm.u.list, P);
  }
}

// Writes the sorted selection of k_sel candidates: the final outputs (one
// group per request) or this group's partial list of kk entries (entries past
// k_sel are ~0, which sorts after every real candidate).
template <int NT>
__device__ __forceinline__ void emit_selection(const SelectSmem<NT> &sm, int k_sel, int r, int grp, int vocab, float *score,
                               int32_t *token, int32_t *parent, uint64_t *partial, int n_groups, int kk) {
  if (n_groups == 1) {
    for (int j = threadIdx.x; j < k_sel; j += NT) {
      const uint64_t x = sm.u.list[j];
      const uint32_t f = (uint32_t)x;
      score[(size_t)r * k_sel + j] = key_score((uint32_t)(x >> 32));
      token[(size_t)r * k_sel + j] = (int32_t)(f % (uint32_t)vocab);
      parent[(size_t)r * k_sel + j] = (int32_t)(f / (uint32_t)vocab);
    }
  } else {
    for (int j = threadIdx.x; j < kk; j += NT)
      partial[((size_t)r * n_groups + grp) * kk + j] = j < k_sel ? sm.u.list[j] : ~0ull;
  }
}

}  // namespace gr
