// The decode indexer chain for callers that cannot allocate device memory (code under HIP
// graph capture, serving loops, harnesses that forbid hipMalloc): csa2_index_chain with its
// workspace taken from a fixed array of this library instead of the caller.
//
// The array lives in device memory of every GPU the library runs on (each GPU has its own copy
// at its own address) and is held until the process ends.  Host code never uses the array's
// name as an address: the address of the current device's copy is looked up once per device
// with hipGetSymbolAddress and kept in g_scratch.  Calls on one GPU share that copy, which keeps
// the last call's contents; the chain needs no part of it zeroed (every kernel writes what it
// later reads), and calls that overlap on one GPU race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "api_internal.hpp"
#include "csa2.h"

namespace {

constexpr size_t kScratchBytes = (size_t)CSA2_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices];   // device address of `scratch` on each device (null: not looked up)

// The current device's copy of the array, or null (with *err set) if it cannot be had.
void* device_scratch(hipError_t* err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" {

size_t csa2_noalloc_scratch_bytes(void) { return kScratchBytes; }

csa2_status csa2_index_chain_noalloc(const uint8_t* idx_k, const uint8_t* idx_k_scales, int64_t k_rows_per_seq,
                                     const uint16_t* idx_q, const float* head_w, const int32_t* n_visible, int B,
                                     int T, int n_max, int block_size, int pool_blocks, int top_k,
                                     const uint16_t* ri_q, const float* ri_w, int L, int32_t* pool_pos,
                                     int32_t* pool_len, int32_t* topk_idx, float* topk_score, int32_t* ri_topk_idx,
                                     float* ri_topk_score, void* stream) {
  // The chain's own host-side checks first: without a workspace a call with valid arguments
  // stops at the workspace check, and one with invalid arguments reports them; neither enqueues
  // anything.
  csa2_status st = csa2_index_chain(idx_k, idx_k_scales, k_rows_per_seq, idx_q, head_w, n_visible, B, T, n_max,
                                    block_size, pool_blocks, top_k, ri_q, ri_w, L, pool_pos, pool_len, topk_idx,
                                    topk_score, ri_topk_idx, ri_topk_score, nullptr, 0, stream);
  if (st != CSA2_ERR_WORKSPACE) return st;
  const size_t need = csa2_index_chain_workspace(B, T, n_max, block_size, pool_blocks, top_k, L);
  if (need > kScratchBytes)
    return csa2::api_fail(CSA2_ERR_UNSUPPORTED,
                          "this shape needs %zu bytes of scratch; csa2_index_chain_noalloc holds %zu "
                          "(use csa2_index_chain with a workspace)",
                          need, kScratchBytes);
  hipError_t e = hipSuccess;
  void* ws = device_scratch(&e);
  if (!ws) return csa2::api_fail(CSA2_ERR_HIP, "no-allocation scratch lookup: %s", hipGetErrorString(e));
  return csa2_index_chain(idx_k, idx_k_scales, k_rows_per_seq, idx_q, head_w, n_visible, B, T, n_max, block_size,
                          pool_blocks, top_k, ri_q, ri_w, L, pool_pos, pool_len, topk_idx, topk_score, ri_topk_idx,
                          ri_topk_score, ws, kScratchBytes, stream);
}

}  // extern "C"
