// Append-only record arena (the beam trie).
//
// OneLA, Abstract: each beam is the shared prompt plus compact append-only
// records of its own transitions, located through a light ancestry index;
// beams advance without moving or copying records already stored.
// Engineering Exploration of Generative Recall, 4.4: a shared prefix is
// stored once.  One new record per new beam lands at node base + j and its
// parent id is the node of the beam it extends; nothing else is written.
//
// One thread per 16-byte chunk of a (k, v) record pair; the first chunk's
// thread also resolves and validates the parent id.

#include "gr_device.h"
#include "gr_launch.h"

namespace gr {
namespace {

struct AP {
  uint4 *ak, *av;
  int32_t *parent;
  const uint4 *k_new, *v_new;
  const int32_t *parent_beam, *prev_nodes;
  int32_t *node_out, *dev_err;
  long long total;     // R * n_new * cpr
  int cpr;             // 16-byte chunks per record
  int cap, base, n_new, n_prev;
};

__global__ __launch_bounds__(256) void trie_append_kernel(AP p) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= p.total) return;
  const long long rowi = idx / p.cpr;            // r * n_new + j
  const int ch = (int)(idx % p.cpr);
  const int r = (int)(rowi / p.n_new), j = (int)(rowi % p.n_new);
  const long long dst = ((long long)r * p.cap + p.base + j) * p.cpr + ch;
  p.ak[dst] = p.k_new[idx];
  p.av[dst] = p.v_new[idx];
  if (ch != 0) return;
  const int n = p.base + j;
  int par = -1, err = 0;
  if (p.parent_beam != nullptr) {
    const int pb = p.parent_beam[rowi];
    if (pb < 0 || pb >= p.n_prev) {
      err = GR_DEVERR_BEAM_RANGE;
    } else {
      const int q = p.prev_nodes[(long long)r * p.n_prev + pb];
      if (q < -1 || q >= p.cap) err = GR_DEVERR_PARENT_RANGE;
      else if (q >= n) err = GR_DEVERR_PARENT_ORDER;
      else par = q;
    }
  }
  p.parent[(long long)r * p.cap + n] = par;
  if (p.node_out) p.node_out[rowi] = n;
  if (err) atomicOr(p.dev_err, err);
}

}  // namespace

hipError_t launch_trie_append(const AppendArgs &a, hipStream_t s) {
  AP p;
  p.ak = (uint4 *)a.ak; p.av = (uint4 *)a.av; p.parent = a.parent;
  p.k_new = (const uint4 *)a.k_new; p.v_new = (const uint4 *)a.v_new;
  p.parent_beam = a.parent_beam; p.prev_nodes = a.prev_nodes;
  p.node_out = a.node_out; p.dev_err = a.dev_err;
  p.cpr = a.H * a.hd * a.elem_bytes / 16;
  p.total = (long long)a.R * a.n_new * p.cpr;
  p.cap = a.cap; p.base = a.base; p.n_new = a.n_new; p.n_prev = a.n_prev;
  const long long blocks = (p.total + 255) / 256;
  hipLaunchKernelGGL(trie_append_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

// ---- transpose (a dimension-major codebook projection into code-major
// rows): 32 x 32 tiles through LDS, reads and writes along rows.
namespace {
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T *in, T *out, int rows, int cols) {
  __shared__ T tile[32][33];
  const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int i = ty; i < 32; i += 8) {
    const int r = r0 + i, c = c0 + tx;
    if (r < rows && c < cols) tile[i][tx] = in[(size_t)r * cols + c];
  }
  __syncthreads();
  for (int i = ty; i < 32; i += 8) {
    const int c = c0 + i, r = r0 + tx;
    if (r < rows && c < cols) out[(size_t)c * rows + r] = tile[tx][i];
  }
}
}  // namespace

hipError_t launch_transpose(const void *in, void *out, int rows, int cols, int elem_bytes, hipStream_t s) {
  const dim3 grid((unsigned)((cols + 31) / 32), (unsigned)((rows + 31) / 32));
  if (elem_bytes == 2)
    hipLaunchKernelGGL(transpose_kernel<uint16_t>, grid, dim3(256), 0, s, (const uint16_t *)in, (uint16_t *)out,
                       rows, cols);
  else
    hipLaunchKernelGGL(transpose_kernel<float>, grid, dim3(256), 0, s, (const float *)in, (float *)out, rows, cols);
  return hipGetLastError();
}

}  // namespace gr
