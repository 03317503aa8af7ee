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
// bucket is small enough, every candidate at or below the bucket is copied to
// an LDS list (per-lane counts, one prefix sum and one atomic per wave), and
// the list is ordered: by counting ranks up to 256 entries, by one bucket pass
// above (a bitonic or merge sort when ties crowd a bucket).  Its first k
// entries are the answer.
// Integer counts and comparisons only, so the result is deterministic.
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
  uint64_t tmp[kListCap];                       // merge-sort ping-pong buffer, bucket-sort scatter target
  uint32_t bstart[kHistBins + 1];               // bucket sort: bucket starts (exclusive scan)
  uint32_t bfill[kHistBins];                    // bucket sort: counts, then fill cursors
  uint32_t wmin[NW], wmax[NW], wtot[NW];
  uint64_t prefix;
  int fixed_lo, need, bucket_cnt, n_list, crowded;
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

// Value of lane l ^ S (S < 64) of a 64-bit composite: DPP for S <= 8, one
// permlane swap per half for 16 and 32 (the swap yields this lane's own half
// and the partner's; where the two are equal either one is the partner's).
template <int S>
__device__ __forceinline__ uint64_t lane_xor_u64(uint64_t x) {
  const uint32_t lo = (uint32_t)x, hi = (uint32_t)(x >> 32);
  if constexpr (S <= 8) {
    return ((uint64_t)xor_lane<S>(hi) << 32) | xor_lane<S>(lo);
  } else {
    uint32_t a0, b0, a1, b1;
    xor_pair<S>(lo, a0, b0);
    xor_pair<S>(hi, a1, b1);
    const uint32_t plo = a0 == lo ? b0 : a0, phi = a1 == hi ? b1 : a1;
    return ((uint64_t)phi << 32) | plo;
  }
}

// One compare-exchange step of the wave bitonic sort below (stride S < 64):
// positions 64 e + l and 64 e + (l ^ S) keep min / max by direction.
template <int E, int S>
__device__ __forceinline__ void wave_bitonic_step(uint64_t (&v)[E], int size, int lane, int base = 0) {
  const bool lower = (lane & S) == 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint64_t y = lane_xor_u64<S>(v[e]);
    const bool up = ((base + 64 * e + lane) & size) == 0;
    const uint64_t mn = v[e] < y ? v[e] : y, mx = v[e] < y ? y : v[e];
    v[e] = (lower == up) ? mn : mx;
  }
}

// Ascending bitonic sort of 64 E composites held by one wave, E per lane
// (v[e] of lane l is position 64 e + l).  Strides below 64 exchange across
// lanes without LDS, larger ones between a lane's own registers; no barrier.
template <int E>
__device__ __forceinline__ void wave_bitonic_sort_u64(uint64_t (&v)[E]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int size = 2; size <= 64 * E; size <<= 1) {
#pragma unroll
    for (int es = (size >> 7); es > 0; es >>= 1) {        // strides 64 es >= 64
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if (e & es) continue;
        const int f = e | es;
        const bool up = ((64 * e) & size) == 0;
        const uint64_t a = v[e], b = v[f];
        const uint64_t mn = a < b ? a : b, mx = a < b ? b : a;
        v[e] = up ? mn : mx;
        v[f] = up ? mx : mn;
      }
    }
    if (size >= 64) wave_bitonic_step<E, 32>(v, size, lane);
    if (size >= 32) wave_bitonic_step<E, 16>(v, size, lane);
    if (size >= 16) wave_bitonic_step<E, 8>(v, size, lane);
    if (size >= 8) wave_bitonic_step<E, 4>(v, size, lane);
    if (size >= 4) wave_bitonic_step<E, 2>(v, size, lane);
    wave_bitonic_step<E, 1>(v, size, lane);
  }
}

// Ascending bitonic sort of arr[0..P) (P <= NT a power of two; entries L..
// are padding), one entry per thread of the first ceil(P/64) waves: strides
// below 64 exchange across lanes without LDS (DPP / permlane), strides of 64
// and more through LDS with a barrier.  Every thread takes the barriers.
template <int NT>
__device__ __forceinline__ void block_bitonic_sort_u64(uint64_t *arr, int L, int P) {
  const int tid = threadIdx.x, lane = tid & 63, base = tid & ~63;
  const bool act = base < P;                             // whole waves
  uint64_t v[1] = {act && tid < L ? arr[tid] : ~0ull};
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride >= 64; stride >>= 1) {
      __syncthreads();
      if (act) arr[tid] = v[0];
      __syncthreads();
      if (act) {
        const uint64_t y = arr[tid ^ stride];
        const bool up = (tid & size) == 0, lower = (tid & stride) == 0;
        const uint64_t mn = v[0] < y ? v[0] : y, mx = v[0] < y ? y : v[0];
        v[0] = (lower == up) ? mn : mx;
      }
    }
    if (act) {
      if (size >= 64) wave_bitonic_step<1, 32>(v, size, lane, base);
      if (size >= 32) wave_bitonic_step<1, 16>(v, size, lane, base);
      if (size >= 16) wave_bitonic_step<1, 8>(v, size, lane, base);
      if (size >= 8) wave_bitonic_step<1, 4>(v, size, lane, base);
      if (size >= 4) wave_bitonic_step<1, 2>(v, size, lane, base);
      wave_bitonic_step<1, 1>(v, size, lane, base);
    }
  }
  __syncthreads();
  if (act) arr[tid] = v[0];
  __syncthreads();
}

// Ascending order of the unique composites arr[0..L) (L <= 256 <= NT/2) by
// ranking: the rank of x is the number of entries below it.  Entry e is
// counted by NT / Lp threads (Lp = 64, 128 or 256 >= L), each over one slice
// of the list (every lane of a wave reading the same addresses, 16 loads in
// flight, four independent partial counts); the slices' counts meet in LDS
// (arr[512..] as scratch) and x is stored at its rank.  The list is padded
// with ~0 to a multiple of 16 first, so the count needs no bound check.
// Every thread takes the barriers.
template <int NT>
__device__ __forceinline__ void rank_sort_u64(uint64_t *arr, int L) {
  static_assert(NT >= 512, "two or more slices per entry");
  const int tid = threadIdx.x;
  const int Lp = L <= 64 ? 64 : (L <= 128 ? 128 : 256);
  const int parts = NT / Lp;
  const int e = tid % Lp, part = tid / Lp;
  uint32_t *rank_s = reinterpret_cast<uint32_t *>(arr + 512);
  const uint64_t x = e < L ? arr[e] : ~0ull;
  if (tid < Lp) rank_s[tid] = 0u;
  if (tid >= L && tid < L + 16) arr[tid] = ~0ull;
  __syncthreads();
  const int chunk = ((L + parts - 1) / parts + 15) & ~15;
  const int i0 = part * chunk, i1 = min(L, i0 + chunk);
  if (e < L && i0 < i1) {
    int r4[4] = {0, 0, 0, 0};
    for (int i = i0; i < i1; i += 16) {
      uint64_t a[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) a[t] = arr[i + t];
#pragma unroll
      for (int t = 0; t < 16; ++t) r4[t & 3] += a[t] < x ? 1 : 0;
    }
    const int c = (r4[0] + r4[1]) + (r4[2] + r4[3]);
    if (c) atomicAdd(&rank_s[e], (uint32_t)c);
  }
  __syncthreads();
  if (part == 0 && e < L) arr[rank_s[e]] = x;
  __syncthreads();
}

// The smallest and second smallest (counting equal values) of one u32 per
// lane across the wave, in every lane: a butterfly that keeps each lane's two
// smallest.
__device__ __forceinline__ void wave_small2_pair_u32(uint32_t x, uint32_t &s1, uint32_t &s2) {
  uint32_t m1 = x, m2 = 0xFFFFFFFFu;
  auto merge = [&](uint32_t p1, uint32_t p2) {
    const uint32_t n2 = min(max(m1, p1), min(m2, p2));
    m1 = min(m1, p1);
    m2 = n2;
  };
  merge(xor_lane<1>(m1), xor_lane<1>(m2));
  merge(xor_lane<2>(m1), xor_lane<2>(m2));
  merge(xor_lane<4>(m1), xor_lane<4>(m2));
  merge(xor_lane<8>(m1), xor_lane<8>(m2));
  uint32_t a1, b1, a2, b2;
  xor_pair<16>(m1, a1, b1);
  xor_pair<16>(m2, a2, b2);
  merge(a1 == m1 ? b1 : a1, a2 == m2 ? b2 : a2);
  xor_pair<32>(m1, a1, b1);
  xor_pair<32>(m2, a2, b2);
  merge(a1 == m1 ? b1 : a1, a2 == m2 ? b2 : a2);
  s1 = m1;
  s2 = m2;
}
// The four smallest (counting equal values) of one u32 per lane across the
// wave, ascending, in every lane: four wave minima, each time taking one lane
// that holds the minimum out.
__device__ __forceinline__ void wave_smallest4_u32(uint32_t x, uint32_t (&out)[4]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t mn = wave_min_u32(x);
    out[i] = mn;
    const uint64_t at = __builtin_amdgcn_ballot_w64(x == mn);
    if (lane == (int)__builtin_ctzll(at)) x = kInvalidKey;
  }
}

// The m-th smallest (1 <= m <= 64, counting equal values) of one u32 per
// lane across the wave, in every lane: a binary search over the bits, each
// step one compare and one ballot (the answer is the largest value with
// fewer than m lanes below it).
__device__ __forceinline__ uint32_t wave_kth_smallest_u32(uint32_t x, int m) {
  uint32_t ans = 0u;
#pragma unroll
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = ans | (1u << bit);
    const int below = __builtin_popcountll(__builtin_amdgcn_ballot_w64(x < cand));
    if (below < m) ans = cand;
  }
  return ans;
}

// The m-th smallest (m = 1 or 2) of one u32 per lane across the wave.
__device__ __forceinline__ uint32_t wave_small2_u32(uint32_t x, int m) {
  uint32_t s1, s2;
  wave_small2_pair_u32(x, s1, s2);
  return m == 1 ? s1 : s2;
}

// Ascending sort of arr[0..NT E) (E = 2, 4 or 8; entries are unique): each
// thread sorts E consecutive entries in registers (a bitonic network), then
// log2(NT) merge-path rounds double the sorted runs, ping-ponging between arr
// and tmp with one barrier each.  In a round a thread finds where its E
// outputs start in the two runs (a binary search), loads the next E entries
// of each run at once, and merges them in registers: A ascending followed by
// B reversed is bitonic, its lower half-cleaner keeps the E smallest, and
// log2(E) further half-cleaners order them.
template <int NT, int E>
__device__ __forceinline__ void merge_sort_u64(uint64_t *arr, uint64_t *tmp) {
  constexpr int P = NT * E;
  const int tid = threadIdx.x;
  uint64_t v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) v[e] = arr[tid * E + e];
#pragma unroll
  for (int size = 2; size <= E; size <<= 1)
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1)
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int f = e ^ stride;
        if (f > e) {
          const bool up = (e & size) == 0;
          const uint64_t x = v[e], y = v[f];
          const uint64_t mn = x < y ? x : y, mx = x < y ? y : x;
          v[e] = up ? mn : mx;
          v[f] = up ? mx : mn;
        }
      }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < E; ++e) arr[tid * E + e] = v[e];
  __syncthreads();
  uint64_t *src = arr, *dst = tmp;
  for (int run = E; run < P; run <<= 1) {
    const int o0 = tid * E;
    const int base = o0 & ~(2 * run - 1), pos = o0 - base;
    const uint64_t *A = src + base, *B = A + run;
    int lo = max(0, pos - run), hi = min(pos, run);
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (A[mid] < B[pos - 1 - mid]) lo = mid + 1;
      else hi = mid;
    }
    const int i = lo, j = pos - lo;
    uint64_t c[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint64_t x = i + e < run ? A[i + e] : ~0ull;
      const uint64_t y = j + E - 1 - e < run ? B[j + E - 1 - e] : ~0ull;
      c[e] = x < y ? x : y;
    }
#pragma unroll
    for (int stride = E / 2; stride > 0; stride >>= 1)
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int f = e ^ stride;
        if (f > e) {
          const uint64_t x = c[e], y = c[f];
          c[e] = x < y ? x : y;
          c[f] = x < y ? y : x;
        }
      }
#pragma unroll
    for (int e = 0; e < E; ++e) dst[o0 + e] = c[e];
    __syncthreads();
    uint64_t *t = src; src = dst; dst = t;
  }
  if (src != arr) {
    for (int t = tid; t < P; t += NT) arr[t] = src[t];
    __syncthreads();
  }
}

// Ascending order of the unique composites list[0..L) (L <= kListCap), all
// in [lo, hi], by one bucket pass: the 11-bit digit (x - lo) >> shift (shift
// chosen so that hi maps below 2048) is histogrammed, scanned into bucket
// starts, entries are scattered to tmp through per-bucket cursors, and each
// entry's final slot is its bucket start plus the number of smaller entries
// in its bucket.  Returns false (list untouched) if some bucket holds more
// than kMaxBucket entries; the caller then sorts otherwise.  Every thread
// takes the barriers and gets the same result.
constexpr int kMaxBucket = 48;
template <int NT>
__device__ __forceinline__ bool bucket_sort_u64(SelectSmem<NT> &sm, int L, uint64_t lo, uint64_t hi) {
  constexpr int NW = NT / 64, BPT = kHistBins / NT;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const uint64_t span = hi - lo;
  const int bits = span ? 64 - __builtin_clzll(span) : 0;
  const int shift = bits > kHistBits ? bits - kHistBits : 0;
  for (int i = tid; i < kHistBins; i += NT) sm.bfill[i] = 0u;
  if (tid == 0) sm.crowded = 0;
  __syncthreads();
  for (int i = tid; i < L; i += NT) atomicAdd(&sm.bfill[(uint32_t)((sm.u.list[i] - lo) >> shift)], 1u);
  __syncthreads();
  uint32_t c[BPT], sum = 0, mx = 0;
#pragma unroll
  for (int q = 0; q < BPT; ++q) {
    c[q] = sm.bfill[tid * BPT + q];
    sum += c[q];
    mx = max(mx, c[q]);
  }
  const uint32_t inc = wave_incl_scan_u32(sum);
  if (lane == 63) sm.wtot[wave] = inc;
  if (mx > (uint32_t)kMaxBucket) sm.crowded = 1;
  __syncthreads();
  if (sm.crowded) return false;
  uint32_t excl = inc - sum;
  for (int w = 0; w < wave; ++w) excl += sm.wtot[w];
#pragma unroll
  for (int q = 0; q < BPT; ++q) {
    sm.bstart[tid * BPT + q] = excl;
    sm.bfill[tid * BPT + q] = excl;               // cursor
    excl += c[q];
  }
  if (tid == NT - 1) sm.bstart[kHistBins] = excl;
  __syncthreads();
  for (int i = tid; i < L; i += NT) {
    const uint64_t x = sm.u.list[i];
    sm.tmp[atomicAdd(&sm.bfill[(uint32_t)((x - lo) >> shift)], 1u)] = x;
  }
  __syncthreads();
  for (int i = tid; i < L; i += NT) {
    const uint64_t x = sm.tmp[i];
    const uint32_t d = (uint32_t)((x - lo) >> shift);
    const int b0 = (int)sm.bstart[d], b1 = (int)sm.bstart[d + 1];
    int rank = b0;
    for (int q = b0; q < b1; ++q) rank += sm.tmp[q] < x ? 1 : 0;
    sm.u.list[rank] = x;
  }
  __syncthreads();
  return true;
}

// Ascending order of the unique composites sm.u.list[0..L) (L <= kListCap),
// all in [lo, hi], of which the first k are wanted: counting ranks up to 256
// entries, else one bucket pass, else (ties crowd a bucket) a bitonic or
// merge sort of the list padded to a power of two.  Every thread takes the
// barriers.
template <int NT>
__device__ __forceinline__ void order_list(SelectSmem<NT> &sm, int L, int k, uint64_t lo, uint64_t hi) {
  const int tid = threadIdx.x;
  const int P = pow2_ceil(max(L, k));
  if (L <= 256) {
    rank_sort_u64<NT>(sm.u.list, L);
  } else if (bucket_sort_u64<NT>(sm, L, lo, hi)) {
  } else if (P <= NT) {
    block_bitonic_sort_u64<NT>(sm.u.list, L, P);
  } else {
    for (int i = L + tid; i < P; i += NT) sm.u.list[i] = ~0ull;
    __syncthreads();
    if (P == 2 * NT) merge_sort_u64<NT, 2>(sm.u.list, sm.tmp);
    else if (P == 4 * NT) merge_sort_u64<NT, 4>(sm.u.list, sm.tmp);
    else if (P == 8 * NT) merge_sort_u64<NT, 8>(sm.u.list, sm.tmp);
    else bitonic_sort_u64<NT>(sm.u.list, P);
  }
}

// Appends every register candidate j with sel(j) to list (composites, in no
// particular order): per-lane counts, one wave prefix sum and one LDS atomic
// per wave reserve the slots, so the per-candidate work is VALU only.
template <int J, typename IdxFn, typename Sel>
__device__ __forceinline__ void append_selected(const uint32_t (&key)[J], IdxFn idx_of, Sel sel, int &n_list,
                                                uint64_t *list) {
  const int lane = threadIdx.x & 63;
  int mine = 0;
#pragma unroll
  for (int j = 0; j < J; ++j) mine += sel(j) ? 1 : 0;
  const int incl = (int)wave_incl_scan_u32((uint32_t)mine);
  const int wave_tot = __builtin_amdgcn_readlane(incl, 63);
  int base = 0;
  if (lane == 63 && wave_tot) base = atomicAdd(&n_list, wave_tot);
  int at = __builtin_amdgcn_readlane(base, 63) + incl - mine;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    if (sel(j)) {
      if (at < kListCap) list[at] = ((uint64_t)key[j] << 32) | idx_of(j);
      ++at;
    }
  }
}

// Selects the k smallest composites among the valid register candidates of
// the block (key[j] != kInvalidKey; the index of slot j is idx_of(j)).  n_valid
// is their number, 1 <= k <= min(n_valid, kMaxK).  On return the first k
// entries of sm.u.list hold them in ascending order.  All threads call it.
// Radix passes continue while the bucket of the k-th candidate holds more
// than bucket_cap (<= kBucketCap) members; a small cap trades passes for a
// shorter list to sort.  Always inlined: the candidates must stay in
// registers (a call would pass them through scratch memory).
template <int NT, int J, typename IdxFn>
__device__ __forceinline__ void select_regs(const uint32_t (&key)[J], IdxFn idx_of, int n_valid, int k, SelectSmem<NT> &sm,
                                            int bucket_cap = kBucketCap) {
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
  if (tid == 0) sm.n_list = 0;
  __syncthreads();
  // every thread derives the same starting state from the wave extremes
  uint32_t a = sm.wmin[0], b = sm.wmax[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) { a = min(a, sm.wmin[w]); b = max(b, sm.wmax[w]); }
  const uint32_t diff = a ^ b;
  int fixed_lo = diff ? 64 - __builtin_clz(diff) : 32;   // key bits differ, or only the index does
  uint64_t prefix = fixed_lo >= 64 ? 0ull : (((uint64_t)a << 32) & ~((1ull << fixed_lo) - 1ull));
  uint32_t need = (uint32_t)k;
  int bucket_cnt = n_valid;

  // ---- radix passes over the bucket of the k-th candidate
  for (int pass = 0; pass < 8; ++pass) {
    if (fixed_lo == 0 || bucket_cnt <= bucket_cap) break;
    const int shift = fixed_lo > kHistBits ? fixed_lo - kHistBits : 0;
    const uint32_t mask = (1u << (fixed_lo - shift)) - 1u;
    const uint64_t pre = fixed_lo >= 64 ? 0ull : (prefix >> fixed_lo);
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
    const uint32_t inc = wave_incl_scan_u32(s);
    if (lane == 63) sm.wtot[wave] = inc;
    __syncthreads();
    uint32_t excl = inc - s;
    for (int w = 0; w < wave; ++w) excl += sm.wtot[w];
    if (excl < need && need <= excl + s) {
#pragma unroll
      for (int q = 0; q < BPT; ++q) {
        if (c[q] > 0 && excl < need && need <= excl + c[q]) {
          sm.need = (int)(need - excl);
          sm.prefix = prefix | (((uint64_t)(tid * BPT + q)) << shift);
          sm.fixed_lo = shift;
          sm.bucket_cnt = (int)c[q];
        }
        excl += c[q];
      }
    }
    __syncthreads();
    need = (uint32_t)sm.need;
    prefix = sm.prefix;
    fixed_lo = sm.fixed_lo;
    bucket_cnt = sm.bucket_cnt;
  }

  // ---- everything at or below the bucket goes to the list
  const uint64_t hi_bound = fixed_lo >= 64 ? ~0ull : (prefix | ((1ull << fixed_lo) - 1ull));
  // With the bucket boundary inside the score key, the index half of
  // hi_bound is all ones and one 32-bit compare decides.
  if (fixed_lo >= 32) {
    const uint32_t hi32 = (uint32_t)(hi_bound >> 32);
    append_selected<J>(key, idx_of, [&](int j) { return key[j] <= hi32 && key[j] != kInvalidKey; }, sm.n_list,
                       sm.u.list);
  } else {
    append_selected<J>(key, idx_of, [&](int j) {
      return key[j] != kInvalidKey && ((((uint64_t)key[j] << 32) | idx_of(j)) <= hi_bound);
    }, sm.n_list, sm.u.list);
  }
  __syncthreads();
  order_list<NT>(sm, min(sm.n_list, kListCap), k, (uint64_t)a << 32, hi_bound);
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
