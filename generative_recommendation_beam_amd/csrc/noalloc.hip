// gr_decode_step_noalloc: gr_decode_step with its scratch in a static device
// array instead of a caller workspace, for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, hosts
// that forbid hipMalloc).
//
// `scratch` is a file-scope __device__ array: every GPU the library runs on
// holds its own copy, at its own address, from the moment the code object is
// loaded on that device until the process ends.  Host code never uses the
// array's name as a device address (in host code it names a host-side
// stand-in); the device address is looked up once per device with
// hipGetSymbolAddress and kept here.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "gr_beam.h"

namespace {

__device__ __attribute__((aligned(256))) unsigned char scratch[GR_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void *g_ptr[kMaxDevices];   // device address of `scratch` per device, once looked up

// The device address of this device's copy of `scratch`, or an error.
gr_status scratch_ptr(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GR_ERR_HIP;
  std::lock_guard<std::mutex> guard(g_lock);
  if (g_ptr[dev] == nullptr) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return GR_ERR_HIP;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return GR_OK;
}

}  // namespace

extern "C" gr_status gr_decode_step_noalloc(const gr_shape *shape, const void *prompt_k, const void *prompt_v,
                                            const void *q, int32_t n_beams, const gr_trie *trie,
                                            const int32_t *beam_node, const void *W, int32_t vocab,
                                            const float *prior, int32_t beam_width, int32_t flags,
                                            float *out_score, int32_t *out_token, int32_t *out_parent,
                                            float *attn_out, float *cand_out, int32_t *dev_err,
                                            hipStream_t stream) {
  // the size check runs first: an oversized step is refused before any
  // device call
  const size_t need = gr_decode_workspace_size(shape, n_beams, vocab, beam_width);
  if (need > (size_t)GR_NOALLOC_SCRATCH_BYTES) return GR_ERR_SCRATCH_LIMIT;
  void *ws = nullptr;
  const gr_status st = scratch_ptr(&ws);
  if (st != GR_OK) return st;
  return gr_decode_step(shape, prompt_k, prompt_v, q, n_beams, trie, beam_node, W, vocab, prior, beam_width,
                        flags, out_score, out_token, out_parent, attn_out, cand_out, ws,
                        (size_t)GR_NOALLOC_SCRATCH_BYTES, dev_err, stream);
}
