// Whole semantic-ID generation: the pieces between two decode steps.
//
// Engineering Exploration of Generative Recall, 4.2: an ID is one code per
// level, each level scored over its own 256 codes; 4.1: attention starts from
// a query, key and value per token.  OneLA, Abstract: every surviving beam
// adds one compact record of its new transition to an append-only store.
// TransRetrieval, GPU retrieval: iterations of the search stay on the device,
// without host round trips.
//
// The code chosen by a beam enters the next step as a token: its level's
// embedding row, projected to a query (the beam's next query) and a key and
// value (the beam's new record).  These depend only on (level, code), so the
// V codes of a level are projected once (code_table_*: a V x 3D x De GEMM) and
// each step gathers rows by chosen code (append_codes_kernel), which gives the
// values a per-beam projection would give.  trace_ids_kernel follows the
// parents back from the last step to write each final beam's code sequence.

#include "gr_device.h"
#include "gr_launch.h"

namespace gr {
namespace {

// T[t][c] = sum_i E[t][i] Wq[c][i] in bf16 on v_mfma_f32_32x32x16_bf16.  One
// workgroup of 4 waves per 32 x 32 output tile of one level (A: 32 embedding
// rows, B: 32 projection rows, both contiguous along i).  The 16-wide k-steps
// are dealt round-robin to the 4 waves, each of which issues the loads of 8
// steps before their MFMAs (operands straight from global memory: the problem
// is a few hundred KB and stays in L2), and the partial tiles meet in LDS.
// Output element (row 8*(i/4) + 4*(lane/32) + i%4, column lane%32) sits in
// accumulator i.
__global__ __launch_bounds__(256) void code_table_bf16_kernel(const uint16_t *E, const uint16_t *Wq,
                                                              uint16_t *T, int V, int N, int De) {
  __shared__ float red[3][16][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tm = V / 32, tiles = tm * (N / 32);
  const int lv = blockIdx.x / tiles, tile = blockIdx.x % tiles;
  const int t0 = (tile % tm) * 32, c0 = (tile / tm) * 32;
  const int g = lane >> 5, c = lane & 31;
  const uint16_t *a = E + ((size_t)lv * V + t0 + c) * De + 8 * g;
  const uint16_t *b = Wq + (size_t)(c0 + c) * De + 8 * g;
  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  const int steps = De / 16;
  int st = wave;
  for (; st + 28 < steps; st += 32) {
    bf16x8 av[8], bv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      av[u] = *(const bf16x8 *)(a + (st + 4 * u) * 16);
      bv[u] = *(const bf16x8 *)(b + (st + 4 * u) * 16);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[u], bv[u], acc, 0, 0, 0);
  }
  for (; st < steps; st += 4) {
    const bf16x8 av = *(const bf16x8 *)(a + st * 16);
    const bf16x8 bv = *(const bf16x8 *)(b + st * 16);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
  }
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) red[wave - 1][i][lane] = acc[i];
  }
  __syncthreads();
  if (wave != 0) return;
  uint16_t *out = T + (size_t)lv * V * N;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float v = acc[i] + red[0][i][lane] + red[1][i][lane] + red[2][i][lane];
    const int t = t0 + 8 * (i >> 2) + 4 * g + (i & 3);
    out[(size_t)t * N + c0 + c] = f32_to_bf16(v);
  }
}

// fp32 storage: one thread per table entry, an fp32 fma chain over i.
__global__ __launch_bounds__(256) void code_table_f32_kernel(const float *E, const float *Wq, float *T,
                                                             int V, int N, int De, long long n) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n) return;
  const long long row = idx / N;                  // level * V + t
  const int c = (int)(idx % N);
  const float *a = E + (size_t)row * De, *b = Wq + (size_t)c * De;
  float s = 0.f;
  for (int i = 0; i < De; ++i) s = fmaf(a[i], b[i], s);
  T[idx] = s;
}

struct CodeAP {
  uint4 *ak, *av, *q_out;
  int32_t *parent;
  const uint4 *table;          // [V][3][cpr]: q, k, v rows of each code
  const int32_t *token, *parent_beam, *prev_nodes;
  int32_t *node_out, *dev_err;
  int32_t *rec_row;            // or [R][row_n]: the table row of each node, in place of ak / av
  long long total;             // R * n_new * cpt
  int cpr, cpt, cap, base, n_new, n_prev, V, row_n, row0;   // cpt: threads per node (cpr, or 1 with nothing to copy)
};

// One thread per 16-byte chunk of a record (per node when nothing is copied);
// the chunk-0 thread also links the parent (as in trie_append) and validates
// the code.
__global__ __launch_bounds__(256) void append_codes_kernel(CodeAP p) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= p.total) return;
  const long long rowi = idx / p.cpt;            // r * n_new + j
  const int ch = (int)(idx % p.cpt);
  const int r = (int)(rowi / p.n_new), j = (int)(rowi % p.n_new);
  int t = p.token[rowi];
  const bool bad_code = t < 0 || t >= p.V;
  if (bad_code) t = 0;
  const uint4 *src = p.table + (size_t)t * 3 * p.cpr;
  const long long dst = ((long long)r * p.cap + p.base + j) * p.cpr + ch;
  if (p.q_out) p.q_out[rowi * p.cpr + ch] = src[ch];
  if (p.rec_row == nullptr) {
    p.ak[dst] = src[p.cpr + ch];
    p.av[dst] = src[2 * p.cpr + ch];
  }
  if (ch != 0) return;
  const int n = p.base + j;
  if (p.rec_row != nullptr) p.rec_row[(long long)r * p.row_n + n] = p.row0 + t;
  int par = -1, err = bad_code ? GR_DEVERR_TOKEN_RANGE : 0;
  if (p.parent_beam != nullptr) {
    const int pb = p.parent_beam[rowi];
    if (pb < 0 || pb >= p.n_prev) {
      err |= GR_DEVERR_BEAM_RANGE;
    } else {
      const int q = p.prev_nodes[(long long)r * p.n_prev + pb];
      if (q < -1 || q >= p.cap) err |= GR_DEVERR_PARENT_RANGE;
      else if (q >= n) err |= GR_DEVERR_PARENT_ORDER;
      else par = q;
    }
  }
  p.parent[(long long)r * p.cap + n] = par;
  if (p.node_out) p.node_out[rowi] = n;
  if (err) atomicOr(p.dev_err, err);
}

// One thread per final beam: ids[r][j][l] for l = L-1 down to 0, following
// out_parent (an index into the previous step's kept beams).
__global__ __launch_bounds__(256) void trace_ids_kernel(TraceArgs a) {
  const int kL = a.k[a.levels - 1];
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)a.R * kL) return;
  const int r = (int)(idx / kL);
  int slot = (int)(idx % kL), err = 0;
  for (int lv = a.levels - 1; lv >= 0; --lv) {
    const long long e = a.off[lv] + (long long)r * a.k[lv] + slot;
    a.ids[idx * a.levels + lv] = a.token[e];
    const int par = a.parent[e];
    const int n_in = lv > 0 ? a.k[lv - 1] : 1;
    if (par < 0 || par >= n_in) { err = GR_DEVERR_TOKEN_RANGE; break; }
    slot = par;
  }
  if (err) atomicOr(a.dev_err, err);
}

}  // namespace

hipError_t launch_code_table(const CodeTableArgs &a, hipStream_t s) {
  const int N = 3 * a.D;
  if (a.dtype == GR_BF16) {
    const int tiles = (a.V / 32) * (N / 32);
    hipLaunchKernelGGL(code_table_bf16_kernel, dim3(tiles * a.levels), dim3(256), 0, s,
                       (const uint16_t *)a.emb, (const uint16_t *)a.w_qkv, (uint16_t *)a.table, a.V, N, a.De);
  } else {
    const long long n = (long long)a.levels * a.V * N;
    hipLaunchKernelGGL(code_table_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       (const float *)a.emb, (const float *)a.w_qkv, (float *)a.table, a.V, N, a.De, n);
  }
  return hipGetLastError();
}

hipError_t launch_append_codes(const AppendCodesArgs &a, hipStream_t s) {
  CodeAP p;
  p.ak = (uint4 *)a.ak; p.av = (uint4 *)a.av; p.q_out = (uint4 *)a.q_out;
  p.parent = a.parent;
  p.table = (const uint4 *)a.table;
  p.token = a.token; p.parent_beam = a.parent_beam; p.prev_nodes = a.prev_nodes;
  p.node_out = a.node_out; p.dev_err = a.dev_err;
  p.cpr = a.H * a.hd * a.elem_bytes / 16;
  p.cpt = a.rec_row != nullptr && a.q_out == nullptr ? 1 : p.cpr;
  p.total = (long long)a.R * a.n_new * p.cpt;
  p.cap = a.cap; p.base = a.base; p.n_new = a.n_new; p.n_prev = a.n_prev; p.V = a.V;
  p.rec_row = a.rec_row; p.row_n = a.row_n; p.row0 = a.row0;
  const long long blocks = (p.total + 255) / 256;
  hipLaunchKernelGGL(append_codes_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_trace_ids(const TraceArgs &a, hipStream_t s) {
  const long long n = (long long)a.R * a.k[a.levels - 1];
  hipLaunchKernelGGL(trace_ids_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace gr
