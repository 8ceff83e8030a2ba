// Host-side check of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer (built by
// hierarchical_kv_indexer_amd/build.py --hostcheck, run by tests/test_hostcheck.py on a machine
// without a GPU).  It drives every entry point's host code: workspace-size queries over a sweep
// of shapes (the plan and carving arithmetic), the argument checks of every entry, and calls with
// valid arguments, which run the checks and the workspace carving and then fail at the first
// launch (no device: CSA2_ERR_HIP).  Pointers are fake, 16-byte aligned host addresses that
// nothing on the host dereferences.  With a GPU present the valid calls would launch kernels on
// those addresses, so the program refuses to run.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <cstring>

#include "csa2.h"

namespace {

int g_fail = 0, g_checks = 0;

void expect(csa2_status got, csa2_status want, const char* what, int line) {
  ++g_checks;
  if (got != want) {
    ++g_fail;
    std::printf("line %d: %s returned %d, expected %d (%s)\n", line, what, (int)got, (int)want, csa2_last_error());
  }
}
#define EXPECT(want, call) expect((call), (want), #call, __LINE__)

void* fake(uintptr_t k = 1) { return (void*)(uintptr_t)(k << 20); }
template <class T>
T* F(uintptr_t k = 1) { return (T*)fake(k); }

}  // namespace

int main() {
  int n_dev = 0;
  if (hipGetDeviceCount(&n_dev) == hipSuccess && n_dev > 0) {
    std::printf("abi_check: a GPU is present; this check runs only without one\n");
    return 2;
  }
  const auto u8 = F<uint8_t>(), u8b = F<uint8_t>(2);
  const auto u16 = F<uint16_t>();
  const auto f32 = F<float>();
  const auto i32 = F<int32_t>();
  auto* o32 = F<int32_t>(3);
  auto* of32 = F<float>(4);
  auto* o16 = F<uint16_t>(5);
  void* ws = fake(6);
  const size_t big = (size_t)1 << 40;

  // ---- workspace sizes over a sweep of shapes (plan and carving arithmetic)
  const int Bs[] = {0, 1, 2, 8, 16, 64, 65535};
  const int Ts[] = {0, 1, 7, 16, 17, 256, 4096};
  const int Ns[] = {-1, 0, 1, 7, 8, 4095, 4096, 9000, 131072, 1 << 20, 1 << 21, 1 << 22};
  const int Ps[] = {-1, 0, 1, 64, 2048, 4096};
  const int Ks[] = {0, 1, 64, 512, 2048, 4096};
  size_t acc = 0;
  for (int B : Bs)
    for (int T : Ts)
      for (int N : Ns)
        for (int P : Ps)
          for (int K : Ks) {
            if ((int64_t)B * T > 65535) continue;
            acc += csa2_index_full_workspace(B, T, N, 8, P, K) + csa2_index_stages_workspace(B, T, N, 8, P, K);
            for (int L = 0; L <= 4; L += 2) acc += csa2_index_chain_workspace(B, T, N, 8, P, K, L);
          }
  for (int L : {1, 4, 64})
    for (int B : {1, 8, 64})
      for (int H : {8, 16, 64, 128})
        for (int K : {1, 64, 512, 2048})
          for (int W : {0, 1, 128, 4096}) {
            acc += csa2_sparse_attn_workspace(L, B, 1, H, K, W);
            acc += csa2_reindex_workspace(L, B, 1, 16384, K);
          }
  acc += csa2_encoder_chunk_workspace(1, 64, 1 << 12, 6, 64, 512, 128);
  acc += csa2_encoder_chunk_workspace(2, 33, 1 << 19, 6, 64, 512, 128);
  acc += csa2_encoder_chunk_workspace(1, 256, 1 << 22, 6, 64, 512, 128);   // 0: beyond 2^21 entries
  std::printf("abi_check: workspace sweep sum %zu\n", acc);

  // ---- single steps
  EXPECT(CSA2_OK, csa2_quantize_query(nullptr, nullptr, 0, nullptr));
  EXPECT(CSA2_ERR_INVALID_ARG, csa2_quantize_query(u16, nullptr, 4, nullptr));
  EXPECT(CSA2_ERR_HIP, csa2_quantize_query(u16, F<uint8_t>(7), 4096, nullptr));
  EXPECT(CSA2_OK, csa2_quantize_kv_fp4(nullptr, 0, nullptr, nullptr, nullptr));
  EXPECT(CSA2_ERR_INVALID_ARG, csa2_quantize_kv_fp4(u16, -1, F<uint8_t>(7), F<uint8_t>(8), nullptr));
  EXPECT(CSA2_ERR_INVALID_ARG, csa2_quantize_kv_fp4(u16, 4, F<uint8_t>(7), (uint8_t*)fake(8) + 8, nullptr));
  EXPECT(CSA2_ERR_HIP, csa2_quantize_kv_fp4(u16, 1 << 20, F<uint8_t>(7), F<uint8_t>(8), nullptr));
  EXPECT(CSA2_ERR_INVALID_ARG, csa2_index_scores(u8, nullptr, 100, u16, f32, i32, 1, 1, 4096, of32, nullptr));
  EXPECT(CSA2_ERR_UNSUPPORTED, csa2_index_scores(u8, nullptr, 1 << 24, u16, f32, i32, 1, 1, (1 << 23) + 8, of32,
                                                 nullptr));
  EXPECT(CSA2_ERR_HIP, csa2_index_scores(u8, nullptr, 9000, u16, f32, i32, 2, 3, 9000, of32, nullptr));
  EXPECT(CSA2_ERR_HIP, csa2_index_scores(u8, u8b, 9000, u16, f32, i32, 1, 16, 9000, of32, nullptr));

  // ---- Full layer and its stages
  for (int P : {0, 64, 2048}) {
    const int N = P == 2048 ? (1 << 20) : 9000, K = 64;
    const size_t w = csa2_index_stages_workspace(2, 3, N, 8, P, K);
    EXPECT(CSA2_ERR_HIP, csa2_index_full(u8, nullptr, N, u16, f32, i32, 2, 3, N, 8, P, K, o32, o32, o32, of32, ws,
                                         w, nullptr));
    EXPECT(CSA2_ERR_WORKSPACE, csa2_index_full(u8, nullptr, N, u16, f32, i32, 2, 3, N, 8, P, K, o32, o32, o32,
                                               nullptr, ws, w - 1, nullptr));
    EXPECT(CSA2_ERR_HIP, csa2_index_scan(u8, u8b, N, u16, f32, i32, 2, 3, N, 8, P, K, ws, w, nullptr));
    EXPECT(CSA2_ERR_HIP, csa2_index_scan_blocks(u8, nullptr, N, u16, f32, i32, 2, 3, N, 8, P, K, 2, ws, w, nullptr));
    EXPECT(CSA2_ERR_HIP, csa2_index_select(i32, 2, 3, N, 8, P, K, o32, o32, o32, nullptr, ws, w, nullptr));
    EXPECT(CSA2_ERR_HIP, csa2_index_topk(2, 3, N, 8, P, K, i32, i32, o32, of32, ws, w, nullptr));
    if (P) EXPECT(CSA2_ERR_HIP, csa2_index_pool(i32, 2, 3, N, 8, P, K, o32, o32, ws, w, nullptr));
  }
  EXPECT(CSA2_ERR_HIP, csa2_index_full(u8, nullptr, 40000, u16, f32, i32, 1, 64, 40000, 8, 0, 512, nullptr,
                                       nullptr, o32, nullptr, ws, csa2_index_full_workspace(1, 64, 40000, 8, 0, 512),
                                       nullptr));
  EXPECT(CSA2_ERR_INVALID_ARG, csa2_index_full(nullptr, nullptr, 4096, u16, f32, i32, 1, 1, 4096, 8, 64, 64, o32,
                                               o32, o32, nullptr, ws, big, nullptr));
  EXPECT(CSA2_ERR_UNSUPPORTED, csa2_index_full(u8, nullptr, 4096, u16, f32, i32, 1, 1, 4096, 16, 64, 64, o32, o32,
                                               o32, nullptr, ws, big, nullptr));
  EXPECT(CSA2_ERR_INVALID_ARG, csa2_index_full(u8, nullptr, 4096, u16, f32, i32, 1, 1, 4096, 8, 64, 600, o32, o32,
                                               o32, nullptr, ws, big, nullptr));
  EXPECT(CSA2_ERR_UNSUPPORTED, csa2_index_full(u8, nullptr, 1 << 22, u16, f32, i32, 1, 1, (1 << 21) + 8, 8, 64, 64,
                                               o32, o32, o32, nullptr, ws, big, nullptr));
  EXPECT(CSA2_ERR_INVALID_ARG, csa2_index_full(u8, nullptr, 4000, u16, f32, i32, 1, 1, 5000, 8, 64, 64, o32, o32,
                                               o32, nullptr, ws, big, nullptr));
  EXPECT(CSA2_ERR_UNSUPPORTED, csa2_index_full(u8, nullptr, 4096, u16, f32, i32, 70000, 1, 4096, 8, 64, 64, o32,
                                               o32, o32, nullptr, ws, big, nullptr));

  // ---- Reindex, chain, no-allocation chain
  {
    const size_t w = csa2_reindex_workspace(4, 2, 1, 16384, 512);
    EXPECT(CSA2_ERR_HIP, csa2_reindex(u8, nullptr, 262144, u16, f32, i32, i32, 16384, 4, 2, 1, 512, o32, of32, ws, w,
                                      nullptr));
    EXPECT(CSA2_ERR_WORKSPACE, csa2_reindex(u8, nullptr, 262144, u16, f32, i32, i32, 16384, 4, 2, 1, 512, o32,
                                            of32, ws, w - 4, nullptr));
    EXPECT(CSA2_ERR_INVALID_ARG, csa2_reindex(u8, nullptr, 100, u16, f32, i32, i32, 512, 1, 1, 1, 1024, o32,
                                              nullptr, ws, big, nullptr));
    EXPECT(CSA2_ERR_UNSUPPORTED, csa2_reindex(u8, nullptr, 100, u16, f32, i32, i32, 20000, 1, 1, 1, 512, o32,
                                              nullptr, ws, big, nullptr));
  }
  for (int L : {0, 1, 4}) {
    for (int fp4 = 0; fp4 < 2; ++fp4) {
      const int N = 1 << 20;
      const size_t w = csa2_index_chain_workspace(1, 1, N, 8, 2048, 512, L);
      const uint8_t* ks = fp4 ? u8b : nullptr;
      EXPECT(CSA2_ERR_HIP, csa2_index_chain(u8, ks, N, u16, f32, i32, 1, 1, N, 8, 2048, 512, u16, f32, L, o32, o32,
                                            o32, of32, o32, of32, ws, w, nullptr));
      EXPECT(CSA2_ERR_HIP, csa2_index_select_reindex(u8, ks, N, i32, 1, 1, N, 8, 2048, 512, u16, f32, L, o32, o32,
                                                     o32, nullptr, o32, nullptr, ws, w, nullptr));
      EXPECT(CSA2_ERR_WORKSPACE, csa2_index_chain(u8, ks, N, u16, f32, i32, 1, 1, N, 8, 2048, 512, u16, f32, L, o32,
                                                  o32, o32, of32, o32, of32, ws, w - 256, nullptr));
      // no device: the scratch lookup fails after the argument checks
      EXPECT(CSA2_ERR_HIP, csa2_index_chain_noalloc(u8, ks, N, u16, f32, i32, 1, 1, N, 8, 2048, 512, u16, f32, L,
                                                    o32, o32, o32, of32, o32, of32, nullptr));
    }
  }
  EXPECT(CSA2_ERR_HIP, csa2_index_chain(u8, nullptr, 131072, u16, f32, i32, 8, 1, 131072, 8, 2048, 512, u16, f32, 4,
                                        o32, o32, o32, nullptr, o32, nullptr, ws,
                                        csa2_index_chain_workspace(8, 1, 131072, 8, 2048, 512, 4), nullptr));
  EXPECT(CSA2_ERR_UNSUPPORTED, csa2_index_chain_noalloc(u8, nullptr, 1 << 21, u16, f32, i32, 16, 1, 1 << 21, 8, 2048,
                                                        512, u16, f32, 4, o32, o32, o32, nullptr, o32, nullptr,
                                                        nullptr));
  EXPECT(CSA2_ERR_INVALID_ARG, csa2_index_chain_noalloc(u8, nullptr, 4096, u16, f32, i32, 1, 1, 4096, 8, 64, 64,
                                                        nullptr, f32, 2, o32, o32, o32, nullptr, o32, nullptr,
                                                        nullptr));
  EXPECT(CSA2_ERR_INVALID_ARG, csa2_index_chain(u8, nullptr, 4096, u16, f32, i32, 1, 1, 4096, 8, 0, 64, u16, f32, 2,
                                                o32, o32, o32, nullptr, o32, nullptr, ws, big, nullptr));

  // ---- attention
  {
    const int32_t sets1[2] = {0, 0};
    int32_t sets64[64];
    for (int l = 0; l < 64; ++l) sets64[l] = l % 3;
    for (int H : {16, 64})
      for (int L : {2, 20}) {
        const size_t w = csa2_sparse_attn_workspace(L, 1, 1, H, 512, 128);
        const int32_t* sets = L == 2 ? sets1 : sets64;
        EXPECT(CSA2_ERR_HIP, csa2_sparse_attn(u8, u8b, 1 << 20, u16, i32, sets, 3, u8, 128, i32, 128, L, 1, 1, H, 512,
                                              0.044f, o16, of32, w ? ws : nullptr, w, nullptr));
      }
    EXPECT(CSA2_ERR_HIP, csa2_sparse_attn(u8, u8b, 32768, u16, i32, sets1, 1, u8, 4096 + 127, i32, 128, 2, 1, 4096,
                                          64, 512, 0.044f, o16, nullptr, ws,
                                          csa2_sparse_attn_workspace(2, 1, 4096, 64, 512, 128), nullptr));
    EXPECT(CSA2_ERR_HIP, csa2_sparse_attn(u8, u8b, 1 << 20, u16, i32, sets64, 3, u8, 8192, i32, 4096, 64, 1, 1, 16,
                                          2048, 0.044f, o16, of32, ws,
                                          csa2_sparse_attn_workspace(64, 1, 1, 16, 2048, 4096), nullptr));
    EXPECT(CSA2_ERR_UNSUPPORTED, csa2_sparse_attn(u8, u8b, 100, u16, i32, sets1, 1, u8, 128, i32, 128, 2, 1, 1, 24,
                                                  512, 0.044f, o16, nullptr, ws, big, nullptr));
    const int32_t bad[2] = {0, 3};
    EXPECT(CSA2_ERR_INVALID_ARG, csa2_sparse_attn(u8, u8b, 100, u16, i32, bad, 2, u8, 128, i32, 128, 2, 1, 1, 16,
                                                  512, 0.044f, o16, nullptr, ws, big, nullptr));
    EXPECT(CSA2_ERR_WORKSPACE, csa2_sparse_attn(u8, u8b, 100, u16, i32, sets1, 1, u8, 128, i32, 128, 2, 1, 1, 16,
                                                512, 0.044f, o16, nullptr, nullptr, 0, nullptr));
  }

  // ---- encoder chunk
  {
    const size_t w = csa2_encoder_chunk_workspace(1, 128, 4096, 6, 64, 512, 128);
    EXPECT(CSA2_ERR_HIP, csa2_encoder_chunk(3, 6, u16, u16, F<uint8_t>(9), F<uint8_t>(10), F<uint8_t>(11), 4096, u16,
                                            f32, u16, u8, 127 + 128, 1, 128, 1024, 2, 64, 512, 128, 0.044f, o16, o32,
                                            ws, w, nullptr));
    EXPECT(CSA2_ERR_INVALID_ARG, csa2_encoder_chunk(3, 6, u16, u16, F<uint8_t>(9), F<uint8_t>(10), F<uint8_t>(11),
                                                    4096, nullptr, f32, u16, u8, 127 + 128, 1, 128, 1024, 2, 64, 512,
                                                    128, 0.044f, o16, o32, ws, w, nullptr));
    EXPECT(CSA2_ERR_INVALID_ARG, csa2_encoder_chunk(3, 6, u16, u16, F<uint8_t>(9), F<uint8_t>(10), F<uint8_t>(11),
                                                    4096, u16, f32, u16, u8, 128, 1, 128, 1024, 2, 64, 512, 128,
                                                    0.044f, o16, o32, ws, w, nullptr));
    EXPECT(CSA2_ERR_WORKSPACE, csa2_encoder_chunk(3, 6, u16, u16, F<uint8_t>(9), F<uint8_t>(10), F<uint8_t>(11), 4096,
                                                  u16, f32, u16, u8, 127 + 128, 1, 128, 1024, 2, 64, 512, 128, 0.044f,
                                                  o16, o32, ws, 64, nullptr));
  }

  std::printf("abi_check: %d checks, %d failed\n", g_checks, g_fail);
  return g_fail ? 1 : 0;
}
