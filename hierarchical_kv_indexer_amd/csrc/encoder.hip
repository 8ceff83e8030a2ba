// Causal visibility of one chunk of an encoder prefill (gfx950).
//
// The encoder's CSA2 layers run over a token sequence compressed m tokens per entry
// (blog.4sapi.com sec.3: m = 2 in the encoder's three groups of one Full and five Reuse
// layers).  Entry j summarises tokens [j*m, (j+1)*m) and becomes visible to the token at
// absolute position p once it is complete, (j+1)*m <= p+1 (a reading: the pages do not say
// how a partial entry is treated), so that token sees floor((p+1)/m) entries; its own most
// recent tokens are covered by the sliding window, which includes the token itself.
#include "common.hpp"
#include "kernels.hpp"

namespace csa2 {

// Token t of the chunk sits at position p0 + t.  The SWA rows of the chunk's layers hold tokens
// p0 - hist .. p0 + T - 1 (row r = token p0 - hist + r), so the window of token t ends at row
// hist + t + 1.  One thread per (sequence, token).
__global__ void k_causal_visibility(int BT, int T, int64_t p0, int m, int hist, int32_t* __restrict__ n_visible,
                                    int32_t* __restrict__ swa_end) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= BT) return;
  const int t = i % T;
  n_visible[i] = (int32_t)((p0 + t + 1) / m);
  swa_end[i] = hist + t + 1;
}

hipError_t launch_causal_visibility(int B, int T, int64_t p0, int m, int hist, int32_t* n_visible,
                                    int32_t* swa_end, hipStream_t s) {
  const int BT = B * T;
  if (BT <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_causal_visibility, dim3((BT + 255) / 256), dim3(256), 0, s, BT, T, p0, m, hist, n_visible,
                     swa_end);
  return hipGetLastError();
}

}  // namespace csa2
