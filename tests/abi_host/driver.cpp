// Calls every C-ABI entry point with arguments that must be rejected (with
// the documented status) or that are no-ops, under the host sanitizers.  No
// call reaches a kernel launch.  Exits 0 and prints "ALL OK" on success.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/fmlp.h"

namespace {
int failures = 0;
void expect(const char* what, fmlp_status got, fmlp_status want) {
  const char* detail = fmlp_last_error();
  if (got != want) {
    std::printf("FAIL %s: status %d (%s), expected %d\n", what, (int)got, detail, (int)want);
    ++failures;
  } else if (want != FMLP_OK && (detail == nullptr || std::strlen(detail) == 0)) {
    std::printf("FAIL %s: no error detail\n", what);
    ++failures;
  }
}
// 16-byte aligned stand-ins, never dereferenced
template <class T>
T* fake(uintptr_t a) { return reinterpret_cast<T*>(a); }
}  // namespace

int main() {
  const fmlp_bf16* X = fake<const fmlp_bf16>(0x10000);
  const fmlp_bf16* W = fake<const fmlp_bf16>(0x20000);
  const fmlp_bf16* B = fake<const fmlp_bf16>(0x30000);
  fmlp_bf16* Y = fake<fmlp_bf16>(0x40000);
  void* WS = fake<void>(0x50000);
  const fmlp_fp8* Q = fake<const fmlp_fp8>(0x60000);
  const float* S = fake<const float>(0x70000);
  const int32_t* ids = fake<const int32_t>(0x80000);
  const float* gw = fake<const float>(0x90000);

  // linear
  expect("linear null W", fmlp_linear(X, nullptr, nullptr, 0, 4, 32, 32, Y, nullptr), FMLP_E_NULL);
  expect("linear K%8", fmlp_linear(X, W, nullptr, 0, 4, 30, 32, Y, nullptr), FMLP_E_ALIGN);
  expect("linear misaligned x", fmlp_linear(fake<const fmlp_bf16>(0x10002), W, nullptr, 0, 4, 32, 32, Y, nullptr),
         FMLP_E_ALIGN);
  expect("linear negative M", fmlp_linear(X, W, nullptr, 0, -1, 32, 32, Y, nullptr), FMLP_E_SHAPE);
  expect("linear huge K", fmlp_linear(X, W, nullptr, 0, 4, int64_t(1) << 22, 32, Y, nullptr), FMLP_E_SHAPE);
  expect("linear bad act", fmlp_linear(X, W, nullptr, 99, 4, 32, 32, Y, nullptr), FMLP_E_ARG);
  expect("linear M=0", fmlp_linear(nullptr, W, B, 1, 0, 32, 32, nullptr, nullptr), FMLP_OK);
  // mlp2
  const size_t ws2 = fmlp_mlp2_workspace_size(16, 4096, 4096, 4096);
  expect("mlp2 small ws", fmlp_mlp2(X, W, B, W, B, 1, 16, 4096, 4096, 4096, Y, WS, ws2 - 1, nullptr),
         FMLP_E_WORKSPACE);
  expect("mlp2 null ws", fmlp_mlp2(X, W, B, W, B, 1, 16, 4096, 4096, 4096, Y, nullptr, 0, nullptr),
         FMLP_E_WORKSPACE);
  expect("mlp2 M=0", fmlp_mlp2(nullptr, W, B, W, B, 1, 0, 64, 64, 64, nullptr, WS, 1 << 20, nullptr), FMLP_OK);
  expect("set_path bad", fmlp_set_path(7), FMLP_E_ARG);
  expect("set_path decode", fmlp_set_path(1), FMLP_OK);
  expect("mlp2 forced decode, M=17", fmlp_mlp2(X, W, B, W, B, 1, 17, 64, 64, 64, Y, WS, 1 << 20, nullptr),
         FMLP_E_ARG);
  expect("set_path auto", fmlp_set_path(0), FMLP_OK);
  // geglu / glu
  const size_t wsg = fmlp_geglu_workspace_size(4096, 8192, 28672);
  expect("geglu small ws", fmlp_geglu(X, W, W, W, 4096, 8192, 28672, Y, WS, wsg / 2, nullptr), FMLP_E_WORKSPACE);
  expect("geglu H%8", fmlp_geglu(X, W, W, W, 4, 64, 100, Y, WS, 1 << 20, nullptr), FMLP_E_ALIGN);
  expect("glu bad gate", fmlp_glu(X, W, W, W, -1, 4, 64, 64, Y, WS, 1 << 20, nullptr), FMLP_E_ARG);
  expect("glu M=0", fmlp_glu(nullptr, W, W, W, 4, 0, 64, 64, nullptr, WS, 1 << 20, nullptr), FMLP_OK);
  // moe
  const size_t wsm = fmlp_moe_workspace_size(4096, 4096, 14336, 8, 2);
  expect("moe E=0", fmlp_moe_geglu(X, ids, gw, W, W, W, 4096, 4096, 14336, 0, 2, Y, WS, wsm, nullptr), FMLP_E_ARG);
  expect("moe k=9", fmlp_moe_geglu(X, ids, gw, W, W, W, 4096, 4096, 14336, 8, 9, Y, WS, wsm, nullptr), FMLP_E_ARG);
  expect("moe null ids", fmlp_moe_glu(X, nullptr, gw, W, W, W, 4, 4096, 4096, 14336, 8, 2, Y, WS, wsm, nullptr),
         FMLP_E_NULL);
  expect("moe small ws", fmlp_moe_geglu(X, ids, gw, W, W, W, 4096, 4096, 14336, 8, 2, Y, WS, wsm - 16, nullptr),
         FMLP_E_WORKSPACE);
  expect("moe T=0", fmlp_moe_geglu(nullptr, nullptr, nullptr, W, W, W, 0, 4096, 14336, 8, 2, nullptr, WS, wsm,
                                   nullptr),
         FMLP_OK);
  // router
  expect("route E=65", fmlp_moe_route(X, W, 16, 64, 65, 2, fake<int32_t>(0xA0000), fake<float>(0xB0000), nullptr,
                                      nullptr),
         FMLP_E_ARG);
  expect("route k>E", fmlp_moe_route(X, W, 16, 64, 2, 3, fake<int32_t>(0xA0000), fake<float>(0xB0000), nullptr,
                                     nullptr),
         FMLP_E_ARG);
  expect("route misaligned ids", fmlp_moe_route(X, W, 16, 64, 8, 2, fake<int32_t>(0xA0002), fake<float>(0xB0000),
                                                nullptr, nullptr),
         FMLP_E_ALIGN);
  // FP8 weights
  expect("linear_w8 M=17", fmlp_linear_w8(X, Q, S, nullptr, 0, 17, 64, 32, Y, nullptr), FMLP_E_ARG);
  expect("linear_w8 K%16", fmlp_linear_w8(X, Q, S, nullptr, 0, 4, 24, 32, Y, nullptr), FMLP_E_ALIGN);
  expect("linear_w8 scale align", fmlp_linear_w8(X, Q, fake<const float>(0x70002), nullptr, 0, 4, 64, 32, Y,
                                                 nullptr),
         FMLP_E_ALIGN);
  expect("mlp2_w8 small ws", fmlp_mlp2_w8(X, Q, S, nullptr, Q, S, nullptr, 1, 4, 64, 128, 64, Y, WS,
                                          fmlp_w8_workspace_size(4, 128) - 1, nullptr),
         FMLP_E_WORKSPACE);
  expect("glu_w8 null scale", fmlp_glu_w8(X, Q, S, Q, S, Q, nullptr, 2, 4, 64, 128, Y, WS, 1 << 20, nullptr),
         FMLP_E_NULL);
  // backward
  const size_t wsl = fmlp_linear_bwd_workspace_size(64, 256, 512);
  expect("linear_bwd null dW", fmlp_linear_bwd(X, W, B, 1, X, 64, 256, 512, Y, nullptr, nullptr, WS, wsl, nullptr),
         FMLP_E_NULL);
  expect("linear_bwd small ws", fmlp_linear_bwd(X, W, B, 1, X, 64, 256, 512, Y, Y, nullptr, WS, wsl - 1, nullptr),
         FMLP_E_WORKSPACE);
  expect("linear_bwd bad act", fmlp_linear_bwd(X, W, B, 7, X, 64, 256, 512, Y, Y, nullptr, WS, wsl, nullptr),
         FMLP_E_ARG);
  expect("linear_bwd K%8", fmlp_linear_bwd(X, W, B, 1, X, 64, 250, 512, Y, Y, nullptr, WS, wsl, nullptr),
         FMLP_E_ALIGN);
  expect("linear_bwd huge M", fmlp_linear_bwd(X, W, B, 1, X, int64_t(1) << 22, 256, 512, Y, Y, nullptr, WS,
                                              size_t(1) << 40, nullptr),
         FMLP_E_SHAPE);
  const size_t wsb = fmlp_glu_bwd_workspace_size(64, 256, 512);
  expect("glu_bwd small ws", fmlp_glu_bwd(X, W, W, W, 2, X, 64, 256, 512, Y, Y, Y, Y, WS, wsb - 1, nullptr),
         FMLP_E_WORKSPACE);
  expect("glu_bwd null dWd", fmlp_glu_bwd(X, W, W, W, 2, X, 64, 256, 512, Y, Y, Y, nullptr, WS, wsb, nullptr),
         FMLP_E_NULL);
  expect("glu_bwd bad gate", fmlp_glu_bwd(X, W, W, W, 9, X, 64, 256, 512, Y, Y, Y, Y, WS, wsb, nullptr),
         FMLP_E_ARG);
  expect("glu_bwd huge H", fmlp_glu_bwd(X, W, W, W, 2, X, 64, 256, int64_t(1) << 21, Y, Y, Y, Y, WS,
                                        size_t(1) << 50, nullptr),
         FMLP_E_SHAPE);
  // support calls
  for (int st = 0; st < 8; ++st)
    if (std::strncmp(fmlp_status_string((fmlp_status)st), "FMLP_", 5) != 0) {
      std::printf("FAIL status string %d\n", st);
      ++failures;
    }
  if (fmlp_status_string((fmlp_status)123) == nullptr) ++failures;
  if (fmlp_decode_timeout_offset() == fmlp_decode_generation_offset()) ++failures;
  if (fmlp_version() < 100) ++failures;
  if (failures) {
    std::printf("%d failure(s)\n", failures);
    return 1;
  }
  std::printf("ALL OK\n");
  return 0;
}
