// Host-only stand-ins for the kernel launchers, so the C-ABI layer (abi.cpp)
// can be built for the CPU alone under the host sanitizers.  The driver only
// makes calls that fail validation, are no-ops or stop at the device check,
// so none of these is ever reached; each fails loudly if it is.
#include <cstdio>
#include <cstdlib>

#include "../../gemm_epilogue_bf16_amd/csrc/decode_w8.h"
#include "../../gemm_epilogue_bf16_amd/csrc/kernels.h"

namespace fmlp {
namespace {
[[noreturn]] void reached(const char* what) {
  std::fprintf(stderr, "stub launcher %s reached: a host-only test enqueued work\n", what);
  std::abort();
}
}  // namespace

int gemm_tile_bm(int tile) { return tile == TILE_256x256 ? 256 : 128; }
int gemm_tile_bn(int tile) { return tile == TILE_256x256 ? 256 : tile == TILE_128x192 ? 192 : 128; }
hipError_t launch_gemm(int, bool, bool, int, GemmParams, hipStream_t) { reached("launch_gemm"); }
hipError_t launch_gemv(const GemvLayer&, int, hipStream_t) { reached("launch_gemv"); }
hipError_t launch_gemv2_persistent(const GemvLayer&, const GemvLayer&, int, uint32_t*, hipStream_t, bool) {
  reached("launch_gemv2_persistent");
}
hipError_t launch_small_mlp2(const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*,
                             int, int64_t, int, int, int, uint16_t*, hipStream_t) {
  reached("launch_small_mlp2");
}
hipError_t launch_moe_route(const int32_t*, const float*, int64_t, int, int, int, const MoeRouteOut&, int32_t*,
                            hipStream_t) {
  reached("launch_moe_route");
}
hipError_t launch_moe_combine(const float*, const int32_t*, int64_t, int, int64_t, int, int64_t, uint16_t*,
                              hipStream_t) {
  reached("launch_moe_combine");
}
hipError_t launch_moe_router(const uint16_t*, const uint16_t*, int64_t, int, int, int, int32_t*, float*, float*, int,
                             hipStream_t) {
  reached("launch_moe_router");
}
hipError_t launch_decode_w8(const W8Layer&, int, hipStream_t) { reached("launch_decode_w8"); }
bool decode_w8_two_applies(int, const W8Layer&, const W8Layer&, int) { reached("decode_w8_two_applies"); }
hipError_t launch_decode_w8_two(const W8Layer&, const W8Layer&, uint32_t*, int, hipStream_t, bool) {
  reached("launch_decode_w8_two");
}
hipError_t launch_transpose(const uint16_t*, int64_t, int64_t, int64_t, uint16_t*, int64_t, int64_t, hipStream_t) {
  reached("launch_transpose");
}
hipError_t launch_rowsum(const uint16_t*, int64_t, int64_t, int64_t, uint16_t*, hipStream_t) {
  reached("launch_rowsum");
}
hipError_t launch_fill_zero(uint16_t*, int64_t, hipStream_t) { reached("launch_fill_zero"); }
hipError_t launch_glu_fused(const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*, int, int64_t, int64_t,
                            int64_t, uint16_t*, void*, uint32_t, hipStream_t) {
  reached("launch_glu_fused");
}
uint32_t next_launch_salt() { return 1u; }
hipError_t launch_sum_parts(const float*, int, int64_t, int64_t, uint16_t*, hipStream_t) {
  reached("launch_sum_parts");
}
}  // namespace fmlp
