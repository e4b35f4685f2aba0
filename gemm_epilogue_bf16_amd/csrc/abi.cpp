// C ABI of the fused feed-forward library: argument validation (always before
// anything is enqueued), device check, path choice, workspace layout and
// launches on the caller's stream.  See include/fmlp.h for the contract.
#include "../../include/fmlp.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "decode_w8.h"
#include "kernels.h"

using namespace fmlp;

namespace {

thread_local std::string g_last_error;
thread_local int g_path = 0;   // 0 auto, 1 decode, 2 two-GEMM, 3 small fused, 4 fused gated block
thread_local bool g_coop = false;   // cooperative launch of the one-launch decode forms

constexpr int kPathAuto = 0, kPathDecode = 1, kPathGemm = 2, kPathSmall = 3, kPathFused = 4;
constexpr int64_t kDecodeMaxM = 16;
constexpr int64_t kSmallMaxDim = 128;
constexpr int64_t kMaxDim = int64_t(1) << 31;   // bound on a token count
constexpr int64_t kMaxInner = int64_t(1) << 22; // bound on an inner dimension: a 256-row
                                                // operand tile spans < 2^31 bytes
constexpr size_t kHeader = kWorkspaceHeaderBytes;  // barrier / error words

fmlp_status fail(fmlp_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

fmlp_status ok() {
  g_last_error.clear();
  return FMLP_OK;
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE_PTR(p)                                                      \
  do {                                                                      \
    if ((p) == nullptr) return fail(FMLP_E_NULL, "%s is NULL", #p);         \
    if (!aligned16(p)) return fail(FMLP_E_ALIGN, "%s is not 16-byte aligned", #p); \
  } while (0)

// Token-sized buffers (activations, outputs, routes) hold nothing when there
// are no tokens: NULL is then accepted, a misaligned pointer is still not.
#define TOKEN_PTR(p, rows)                                                  \
  do {                                                                      \
    if ((rows) > 0) REQUIRE_PTR(p);                                         \
    else if ((p) != nullptr && !aligned16(p))                               \
      return fail(FMLP_E_ALIGN, "%s is not 16-byte aligned", #p);           \
  } while (0)

#define OPTIONAL_PTR(p)                                                     \
  do {                                                                      \
    if ((p) != nullptr && !aligned16(p))                                    \
      return fail(FMLP_E_ALIGN, "%s is not 16-byte aligned", #p);           \
  } while (0)

fmlp_status check_rows(const char* name, int64_t v) {
  if (v < 0 || v >= kMaxDim) return fail(FMLP_E_SHAPE, "%s=%lld is out of range", name, (long long)v);
  return FMLP_OK;
}

fmlp_status check_inner(const char* name, int64_t v) {
  if (v <= 0 || v >= kMaxInner)
    return fail(FMLP_E_SHAPE, "%s=%lld must be in [8, 2^22)", name, (long long)v);
  if (v % 8 != 0) return fail(FMLP_E_ALIGN, "%s=%lld is not a multiple of 8", name, (long long)v);
  return FMLP_OK;
}

fmlp_status check_act(int act, const char* name = "act") {
  if (act != FMLP_ACT_NONE && act != FMLP_ACT_GELU_ERF && act != FMLP_ACT_GELU_TANH &&
      act != FMLP_ACT_RELU && act != FMLP_ACT_SILU)
    return fail(FMLP_E_ARG, "%s=%d is not an fmlp_act", name, act);
  return FMLP_OK;
}

#define TRY(expr)                              \
  do {                                         \
    fmlp_status s_ = (expr);                   \
    if (s_ != FMLP_OK) return s_;              \
  } while (0)

// ---- device check (cached per device) ---------------------------------------
struct DevInfo {
  bool probed = false;
  bool gfx950 = false;
  int cus = 0;
};
std::mutex g_dev_mu;
DevInfo g_dev[64];

fmlp_status check_device(int* cus_out = nullptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) return fail(FMLP_E_DEVICE, "no current HIP device (%s)", hipGetErrorString(e));
  if (dev >= 64) return fail(FMLP_E_DEVICE, "device index %d unsupported", dev);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DevInfo& d = g_dev[dev];
  if (!d.probed) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(FMLP_E_DEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    d.gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.cus = prop.multiProcessorCount;
    d.probed = true;
    if (!d.gfx950) {
      d.probed = true;
      return fail(FMLP_E_DEVICE, "device %d is %s; this library is built for gfx950 only", dev, prop.gcnArchName);
    }
  }
  if (!d.gfx950) return fail(FMLP_E_DEVICE, "current device is not gfx950");
  if (cus_out) *cus_out = d.cus;
  return FMLP_OK;
}

fmlp_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(FMLP_E_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// ---- tile choice --------------------------------------------------------------
int choose_tile(int64_t M, int64_t out_cols_per_256_tile_n, int cus) {
  // Big tiles when they alone fill the chip at least once.
  const int64_t tiles256 = ((M + 255) / 256) * out_cols_per_256_tile_n;
  return tiles256 >= cus ? TILE_256x256 : TILE_128x128;
}

GemmParams dense_params(const uint16_t* A, int64_t lda, const uint16_t* B0, const uint16_t* B1,
                        const uint16_t* bias, void* C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                        int act, int cus) {
  GemmParams p;
  std::memset(&p, 0, sizeof p);
  p.A = A;
  p.lda = lda;
  p.B0 = B0;
  p.B1 = B1;
  p.bias = bias;
  p.C = C;
  p.ldc = ldc;
  p.M = M;
  p.N = N;
  p.K = K;
  p.act = act;
  p.cus = cus;
  return p;
}

// Plain bf16-output GEMM.  Between "256 tiles fill the chip" and small
// shapes, a width that is a multiple of 192 whose 128x192 tiles fit in one
// round on the chip runs on those: every CU gets one tile, where 128x128
// tiles would leave a second, partial round (the 768-wide down projection:
// 256 tiles of 128x192 against 384 of 128x128 on 512 block slots).
int choose_tile_linear(int64_t M, int64_t N, int cus) {
  const int tile = choose_tile(M, (N + 255) / 256, cus);
  if (tile == TILE_256x256) return tile;
  const int64_t t192 = ((M + 127) / 128) * (N / 192);
  if (N % 192 == 0 && t192 <= cus && 4 * t192 >= 3 * (int64_t)cus) return TILE_128x192;
  return tile;
}

hipError_t gemm_linear(const uint16_t* x, const uint16_t* W, const uint16_t* b, int act, int64_t M,
                       int64_t K, int64_t N, uint16_t* y, int cus, hipStream_t s) {
  const int tile = choose_tile_linear(M, N, cus);
  return launch_gemm(GEMM_OUT_BF16, false, false, tile, dense_params(x, K, W, nullptr, b, y, N, M, N, K, act, cus), s);
}

hipError_t gemm_glu_gateup(const uint16_t* x, const uint16_t* Wg, const uint16_t* Wu, int gate_act,
                           int64_t M, int64_t D, int64_t H, uint16_t* m, int cus, hipStream_t s) {
  const int tile = choose_tile(M, (H + 127) / 128, cus);
  return launch_gemm(GEMM_OUT_GEGLU, false, false, tile,
                     dense_params(x, D, Wg, Wu, nullptr, m, H, M, H, D, gate_act, cus), s);
}

}  // namespace

namespace fmlp {
// The status and detail text of a failure found outside this file (the
// no-allocation entry point), for fmlp_last_error().
fmlp_status record_error(fmlp_status s, const char* msg) { return fail(s, "%s", msg); }
}  // namespace fmlp

extern "C" {

int fmlp_version(void) { return 106; }

const char* fmlp_status_string(fmlp_status s) {
  switch (s) {
    case FMLP_OK: return "FMLP_OK";
    case FMLP_E_NULL: return "FMLP_E_NULL: a required pointer is NULL";
    case FMLP_E_SHAPE: return "FMLP_E_SHAPE: a dimension is out of range";
    case FMLP_E_ALIGN: return "FMLP_E_ALIGN: inner dimension not a multiple of 8 or pointer not 16-byte aligned";
    case FMLP_E_ARG: return "FMLP_E_ARG: invalid argument";
    case FMLP_E_WORKSPACE: return "FMLP_E_WORKSPACE: workspace missing or too small";
    case FMLP_E_DEVICE: return "FMLP_E_DEVICE: no usable gfx950 device";
    case FMLP_E_HIP: return "FMLP_E_HIP: HIP launch failed";
  }
  return "unknown fmlp_status";
}

const char* fmlp_last_error(void) { return g_last_error.c_str(); }

fmlp_status fmlp_set_cooperative_decode(int on) {
  if (on != 0 && on != 1) return fail(FMLP_E_ARG, "on=%d is not 0 or 1", on);
  g_coop = on != 0;
  return ok();
}

fmlp_status fmlp_set_path(int path) {
  if (path < kPathAuto || path > kPathFused) return fail(FMLP_E_ARG, "path=%d is not 0..4", path);
  g_path = path;
  return ok();
}

// ---------------------------------------------------------------------------
fmlp_status fmlp_linear(const fmlp_bf16* x, const fmlp_bf16* W, const fmlp_bf16* b, int act,
                        int64_t M, int64_t K, int64_t N, fmlp_bf16* y, fmlp_stream stream) {
  TRY(check_rows("M", M));
  TRY(check_inner("K", K));
  TRY(check_inner("N", N));
  TRY(check_act(act));
  TOKEN_PTR(x, M);
  REQUIRE_PTR(W);
  OPTIONAL_PTR(b);
  TOKEN_PTR(y, M);
  if (M == 0) return ok();
  int cus = 0;
  TRY(check_device(&cus));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (M <= kDecodeMaxM) {
    GemvLayer L{x, W, nullptr, b, y, K, N, act, 0};
    return launched(launch_gemv(L, (int)M, s), "linear (decode) launch");
  }
  return launched(gemm_linear(x, W, b, act, M, K, N, y, cus, s), "linear launch");
}

// The hidden activation between the two layers: M x H bf16, or at one token
// H/2 words of {bf16 pair, epoch} (8 bytes each) for the decode kernel's
// word-flag publish.
size_t hidden_bytes(int64_t M, int64_t H) {
  const size_t plain = (size_t)M * (size_t)H * 2;
  const size_t words = M == 1 ? (size_t)H * 4 : 0;
  return round_up(plain > words ? plain : words, 256);
}

size_t fmlp_mlp2_workspace_size(int64_t M, int64_t K, int64_t H, int64_t N) {
  (void)K;
  (void)N;
  if (M < 0 || H <= 0) return 0;
  return kHeader + hidden_bytes(M, H);
}

fmlp_status fmlp_mlp2(const fmlp_bf16* x, const fmlp_bf16* W1, const fmlp_bf16* b1,
                      const fmlp_bf16* W2, const fmlp_bf16* b2, int act, int64_t M, int64_t K,
                      int64_t H, int64_t N, fmlp_bf16* y, void* workspace, size_t workspace_bytes,
                      fmlp_stream stream) {
  TRY(check_rows("M", M));
  TRY(check_inner("K", K));
  TRY(check_inner("H", H));
  TRY(check_inner("N", N));
  TRY(check_act(act));
  TOKEN_PTR(x, M);
  REQUIRE_PTR(W1);
  OPTIONAL_PTR(b1);
  REQUIRE_PTR(W2);
  OPTIONAL_PTR(b2);
  TOKEN_PTR(y, M);
  const bool small_ok = K <= kSmallMaxDim && H <= kSmallMaxDim && N <= kSmallMaxDim;
  int path = g_path;
  if (path == kPathAuto) path = (M <= kDecodeMaxM) ? kPathDecode : (small_ok ? kPathSmall : kPathGemm);
  if (path == kPathFused) return fail(FMLP_E_ARG, "the fused gated-block path is glu-only");
  if (path == kPathDecode && M > kDecodeMaxM)
    return fail(FMLP_E_ARG, "decode path needs M <= %lld (M=%lld)", (long long)kDecodeMaxM, (long long)M);
  if (path == kPathSmall && !small_ok)
    return fail(FMLP_E_ARG, "small fused path needs K, H, N <= %lld", (long long)kSmallMaxDim);
  const size_t need = (path == kPathSmall) ? 0 : fmlp_mlp2_workspace_size(M, K, H, N);
  if (need > 0) {
    if (workspace == nullptr) return fail(FMLP_E_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
    if (!aligned16(workspace)) return fail(FMLP_E_ALIGN, "workspace is not 16-byte aligned");
    if (workspace_bytes < need)
      return fail(FMLP_E_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  }
  if (M == 0) return ok();
  int cus = 0;
  TRY(check_device(&cus));
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint16_t* h = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + kHeader);
  if (path == kPathSmall)
    return launched(launch_small_mlp2(x, W1, b1, W2, b2, act, M, (int)K, (int)H, (int)N, y, s),
                    "mlp2 (small fused) launch");
  if (path == kPathDecode) {
    GemvLayer L1{x, W1, nullptr, b1, h, K, H, act, 0};
    GemvLayer L2{h, W2, nullptr, b2, y, H, N, FMLP_ACT_NONE, 0};
    return launched(launch_gemv2_persistent(L1, L2, (int)M, static_cast<uint32_t*>(workspace), s, g_coop),
                    "mlp2 (decode, persistent) launch");
  }
  hipError_t e = gemm_linear(x, W1, b1, act, M, K, H, h, cus, s);
  if (e != hipSuccess) return launched(e, "mlp2 layer-1 launch");
  return launched(gemm_linear(h, W2, b2, FMLP_ACT_NONE, M, H, N, y, cus, s), "mlp2 layer-2 launch");
}

size_t fmlp_geglu_workspace_size(int64_t M, int64_t D, int64_t H) {
  if (M < 0 || H <= 0) return 0;
  size_t body = hidden_bytes(M, H);                 // m of the two-launch and decode paths
  if (D > 0 && D <= kGluFusedMaxD) body = std::max(body, glu_fused_workspace_bytes(M, D, H));
  return kHeader + body;
}

size_t fmlp_glu_workspace_size(int64_t M, int64_t D, int64_t H) { return fmlp_geglu_workspace_size(M, D, H); }

fmlp_status fmlp_geglu(const fmlp_bf16* x, const fmlp_bf16* Wg, const fmlp_bf16* Wu,
                       const fmlp_bf16* Wd, int64_t M, int64_t D, int64_t H, fmlp_bf16* y,
                       void* workspace, size_t workspace_bytes, fmlp_stream stream) {
  return fmlp_glu(x, Wg, Wu, Wd, FMLP_ACT_GELU_TANH, M, D, H, y, workspace, workspace_bytes, stream);
}

fmlp_status fmlp_glu(const fmlp_bf16* x, const fmlp_bf16* Wg, const fmlp_bf16* Wu,
                     const fmlp_bf16* Wd, int gate_act, int64_t M, int64_t D, int64_t H, fmlp_bf16* y,
                     void* workspace, size_t workspace_bytes, fmlp_stream stream) {
  TRY(check_rows("M", M));
  TRY(check_inner("D", D));
  TRY(check_inner("H", H));
  TRY(check_act(gate_act, "gate_act"));
  TOKEN_PTR(x, M);
  REQUIRE_PTR(Wg);
  REQUIRE_PTR(Wu);
  REQUIRE_PTR(Wd);
  TOKEN_PTR(y, M);
  int path = g_path;
  if (path == kPathAuto) path = (M <= kDecodeMaxM) ? kPathDecode : kPathGemm;
  if (path == kPathSmall) return fail(FMLP_E_ARG, "the small fused path is mlp2-only");
  if (path == kPathFused && D > kGluFusedMaxD)
    return fail(FMLP_E_ARG, "the fused gated block needs D <= %lld (D=%lld)", (long long)kGluFusedMaxD, (long long)D);
  if (path == kPathFused && H > kGluFusedMaxH)
    return fail(FMLP_E_ARG, "the fused gated block needs H <= %lld (H=%lld)", (long long)kGluFusedMaxH, (long long)H);
  if (path == kPathDecode && M > kDecodeMaxM)
    return fail(FMLP_E_ARG, "decode path needs M <= %lld (M=%lld)", (long long)kDecodeMaxM, (long long)M);
  const size_t need = fmlp_geglu_workspace_size(M, D, H);
  if (workspace == nullptr) return fail(FMLP_E_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
  if (!aligned16(workspace)) return fail(FMLP_E_ALIGN, "workspace is not 16-byte aligned");
  if (workspace_bytes < need)
    return fail(FMLP_E_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  if (M == 0) return ok();
  int cus = 0;
  TRY(check_device(&cus));
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint16_t* m = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + kHeader);
  if (path == kPathDecode) {
    GemvLayer L1{x, Wg, Wu, nullptr, m, D, H, gate_act, 1};
    GemvLayer L2{m, Wd, nullptr, nullptr, y, H, D, FMLP_ACT_NONE, 0};
    return launched(launch_gemv2_persistent(L1, L2, (int)M, static_cast<uint32_t*>(workspace), s, g_coop),
                    "geglu (decode, persistent) launch");
  }
  if (path == kPathFused)
    return launched(launch_glu_fused(x, Wg, Wu, Wd, gate_act, M, D, H, y, m, next_launch_salt(), s),
                    "gated block (fused, one launch)");
  hipError_t e = gemm_glu_gateup(x, Wg, Wu, gate_act, M, D, H, m, cus, s);
  if (e != hipSuccess) return launched(e, "geglu gate+up launch");
  return launched(gemm_linear(m, Wd, nullptr, FMLP_ACT_NONE, M, H, D, y, cus, s), "geglu down launch");
}

// ---- mixture of experts --------------------------------------------------------
namespace {
struct MoeLayout {
  size_t tok_of, scale_of, pos_of, group_off, tile_off, counts, m, ytilde, total;
};
// Split-K of the MoE down projection (K = H): two halves when the 64-k stage
// count is even and long (the tail m-tile of every expert then costs half a
// pass over K, and the partial round shrinks); the combine adds the halves.
int moe_down_ksplit(int64_t H) {
  const int64_t nk = (H + 63) / 64;
  return (nk % 2 == 0 && nk >= 64) ? 2 : 1;
}

MoeLayout moe_layout(int64_t T, int64_t D, int64_t H, int32_t E, int32_t top_k) {
  MoeLayout L;
  const size_t P = (size_t)T * (size_t)top_k;
  size_t o = kHeader;
  L.tok_of = o;    o += round_up(P * 4, 256);
  L.scale_of = o;  o += round_up(P * 4, 256);
  L.pos_of = o;    o += round_up(P * 4, 256);
  L.group_off = o; o += round_up(((size_t)E + 1) * 4, 256);
  L.tile_off = o;  o += round_up(((size_t)E + 1) * 4, 256);
  L.counts = o;    o += round_up(moe_route_counts_bytes((int64_t)P, E), 256);
  L.m = o;         o += round_up(P * (size_t)H * 2, 256);
  L.ytilde = o;    o += round_up(P * (size_t)D * 4, 256) * (size_t)moe_down_ksplit(H);
  L.total = o;
  return L;
}
constexpr int kMoeTile = TILE_256x256;
}  // namespace

size_t fmlp_moe_workspace_size(int64_t T, int64_t D, int64_t H, int32_t E, int32_t top_k) {
  if (T < 0 || D <= 0 || H <= 0 || E <= 0 || top_k <= 0) return 0;
  return moe_layout(T, D, H, E, top_k).total;
}

size_t fmlp_moe_error_offset(void) { return 16; }

size_t fmlp_decode_timeout_offset(void) { return (size_t)kSyncTimeoutWord * 4; }
size_t fmlp_decode_generation_offset(void) { return (size_t)kSyncGenWord * 4; }

fmlp_status fmlp_moe_geglu(const fmlp_bf16* x, const int32_t* expert_ids, const float* gate_w,
                           const fmlp_bf16* Wg, const fmlp_bf16* Wu, const fmlp_bf16* Wd, int64_t T,
                           int64_t D, int64_t H, int32_t E, int32_t top_k, fmlp_bf16* y,
                           void* workspace, size_t workspace_bytes, fmlp_stream stream) {
  return fmlp_moe_glu(x, expert_ids, gate_w, Wg, Wu, Wd, FMLP_ACT_GELU_TANH, T, D, H, E, top_k, y, workspace,
                      workspace_bytes, stream);
}

fmlp_status fmlp_moe_glu(const fmlp_bf16* x, const int32_t* expert_ids, const float* gate_w,
                         const fmlp_bf16* Wg, const fmlp_bf16* Wu, const fmlp_bf16* Wd, int gate_act,
                         int64_t T, int64_t D, int64_t H, int32_t E, int32_t top_k, fmlp_bf16* y,
                         void* workspace, size_t workspace_bytes, fmlp_stream stream) {
  TRY(check_act(gate_act, "gate_act"));
  TRY(check_rows("T", T));
  TRY(check_inner("D", D));
  TRY(check_inner("H", H));
  if (E < 1 || E > kMoeRouteMaxExperts) return fail(FMLP_E_ARG, "E=%d must be in [1, %d]", E, kMoeRouteMaxExperts);
  if (top_k < 1 || top_k > 8) return fail(FMLP_E_ARG, "top_k=%d must be in [1, 8]", top_k);
  if ((int64_t)T * top_k >= (int64_t(1) << 31))
    return fail(FMLP_E_SHAPE, "T*top_k=%lld is too large", (long long)T * top_k);
  if (T * D >= (int64_t(1) << 30))
    return fail(FMLP_E_SHAPE, "T*D=%lld must be below 2^30", (long long)(T * D));
  TOKEN_PTR(x, T);
  if (T > 0 && expert_ids == nullptr) return fail(FMLP_E_NULL, "expert_ids is NULL");
  if (T > 0 && gate_w == nullptr) return fail(FMLP_E_NULL, "gate_w is NULL");
  REQUIRE_PTR(Wg);
  REQUIRE_PTR(Wu);
  REQUIRE_PTR(Wd);
  TOKEN_PTR(y, T);
  const MoeLayout L = moe_layout(T, D, H, E, top_k);
  if (workspace == nullptr) return fail(FMLP_E_WORKSPACE, "workspace is NULL (need %zu bytes)", L.total);
  if (!aligned16(workspace)) return fail(FMLP_E_ALIGN, "workspace is not 16-byte aligned");
  if (workspace_bytes < L.total)
    return fail(FMLP_E_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, L.total);
  if (T == 0) return ok();
  int cus = 0;
  TRY(check_device(&cus));
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  MoeRouteOut r;
  r.tok_of = reinterpret_cast<int32_t*>(ws + L.tok_of);
  r.scale_of = reinterpret_cast<float*>(ws + L.scale_of);
  r.pos_of = reinterpret_cast<int32_t*>(ws + L.pos_of);
  r.group_off = reinterpret_cast<int32_t*>(ws + L.group_off);
  r.tile_off = reinterpret_cast<int32_t*>(ws + L.tile_off);
  r.err = reinterpret_cast<int32_t*>(ws + fmlp_moe_error_offset());
  uint16_t* m = reinterpret_cast<uint16_t*>(ws + L.m);
  float* ytilde = reinterpret_cast<float*>(ws + L.ytilde);
  const int bm = gemm_tile_bm(kMoeTile);
  const int64_t P = T * top_k;

  hipError_t e = launch_moe_route(expert_ids, gate_w, T, top_k, E, bm, r,
                                  reinterpret_cast<int32_t*>(ws + L.counts), s);
  if (e != hipSuccess) return launched(e, "moe route launch");

  GemmParams g = dense_params(x, D, Wg, Wu, nullptr, m, H, P, H, D, gate_act, cus);
  g.a_rows = r.tok_of;
  g.a_src_rows = T;
  g.group_off = r.group_off;
  g.tile_off = r.tile_off;
  g.groups = E;
  g.strideB = H * D;
  g.tiles_m = (int)((P + bm - 1) / bm + E);
  e = launch_gemm(GEMM_OUT_GEGLU, true, true, kMoeTile, g, s);
  if (e != hipSuccess) return launched(e, "moe gate+up launch");

  GemmParams d = dense_params(m, H, Wd, nullptr, nullptr, ytilde, D, P, D, H, 0, cus);
  d.group_off = r.group_off;
  d.tile_off = r.tile_off;
  d.groups = E;
  d.strideB = D * H;
  d.row_scale = r.scale_of;
  d.tiles_m = (int)((P + bm - 1) / bm + E);
  const int ksplit = moe_down_ksplit(H);
  const int64_t kstride = (int64_t)(round_up(P * (size_t)D * 4, 256) / 4);   // floats between the parts
  d.ksplit = ksplit;
  d.c_kstride = kstride;
  e = launch_gemm(GEMM_OUT_F32_SCALED, false, true, kMoeTile, d, s);
  if (e != hipSuccess) return launched(e, "moe down launch");

  return launched(launch_moe_combine(ytilde, r.pos_of, T, top_k, D, ksplit, kstride, y, s), "moe combine launch");
}

fmlp_status fmlp_moe_route(const fmlp_bf16* x, const fmlp_bf16* Wr, int64_t T, int64_t D, int32_t E,
                           int32_t top_k, int32_t* expert_ids, float* gate_w, float* logits,
                           fmlp_stream stream) {
  TRY(check_rows("T", T));
  TRY(check_inner("D", D));
  if (E < 1 || E > kRouterMaxExperts) return fail(FMLP_E_ARG, "E=%d must be in [1, %d]", E, kRouterMaxExperts);
  if (top_k < 1 || top_k > 8 || top_k > E)
    return fail(FMLP_E_ARG, "top_k=%d must be in [1, min(8, E=%d)]", top_k, E);
  TOKEN_PTR(x, T);
  REQUIRE_PTR(Wr);
  if (T > 0 && expert_ids == nullptr) return fail(FMLP_E_NULL, "expert_ids is NULL");
  if (T > 0 && gate_w == nullptr) return fail(FMLP_E_NULL, "gate_w is NULL");
  if ((reinterpret_cast<uintptr_t>(expert_ids) | reinterpret_cast<uintptr_t>(gate_w) |
       reinterpret_cast<uintptr_t>(logits)) & 3u)
    return fail(FMLP_E_ALIGN, "expert_ids, gate_w and logits must be 4-byte aligned");
  if (T == 0) return ok();
  int cus = 0;
  TRY(check_device(&cus));
  return launched(launch_moe_router(x, Wr, T, (int)D, E, top_k, expert_ids, gate_w, logits, cus,
                                    static_cast<hipStream_t>(stream)),
                  "moe router launch");
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Backward pass
// ---------------------------------------------------------------------------
namespace {
// Token counts of a backward call bound the contraction over tokens, which the
// GEMM reads with 32-bit offsets like any inner dimension.
constexpr int64_t kBwdMaxTokens = kMaxInner;

size_t ws_bf16(int64_t rows, int64_t cols) { return round_up((size_t)rows * (size_t)cols * 2, 256); }
int64_t pad8(int64_t v) { return (v + 7) / 8 * 8; }

// Weight gradients contract over the tokens: C[R, Cc] = A[R, T] . B[Cc, T]^T
// with both operands transposed to token-contiguous rows (T = tokens padded
// to 8).  Few output tiles over a long token range leave most CUs idle (the
// 3072 x 768 gradient of the 768/3072 block: 36 tiles of 256 x 256 over 8192
// tokens), so when the 256 x 256 tiles do not fill a 256-CU device the token
// range is split in P parts, as many as fit one round (at most 8, at least
// 8 stages of 64 tokens each; parts may differ by one stage): each part writes
// an fp32 copy of C into the workspace and a fixed-order sum rounds once
// (deterministic).  P does not depend on the device, so the workspace size is
// known without one.
int wgrad_split(int64_t R, int64_t T, int64_t Cc) {
  const int64_t tiles = ((R + 255) / 256) * ((Cc + 255) / 256);
  if (tiles >= 256) return 1;
  const int64_t nk = (T + 63) / 64;
  const int64_t P = std::min<int64_t>({256 / tiles, 8, nk / 8});
  return P > 1 ? (int)P : 1;
}
size_t wgrad_parts_bytes(int64_t R, int64_t T, int64_t Cc) {
  const int P = wgrad_split(R, T, Cc);
  return P > 1 ? round_up((size_t)P * (size_t)R * (size_t)Cc * 4, 256) : 0;
}
hipError_t gemm_wgrad(const uint16_t* A, const uint16_t* B, int64_t R, int64_t T, int64_t Cc, uint16_t* C,
                      float* parts, int cus, hipStream_t s) {
  const int P = wgrad_split(R, T, Cc);
  if (P == 1) return gemm_linear(A, B, nullptr, FMLP_ACT_NONE, R, T, Cc, C, cus, s);
  GemmParams p = dense_params(A, T, B, nullptr, nullptr, parts, Cc, R, Cc, T, FMLP_ACT_NONE, cus);
  p.ksplit = P;
  p.c_kstride = R * Cc;
  const hipError_t e = launch_gemm(GEMM_OUT_F32_SCALED, false, false, TILE_256x256, p, s);
  if (e != hipSuccess) return e;
  return launch_sum_parts(parts, P, R * Cc, R * Cc, C, s);
}

// k-major operands (no transpose copies; the GEMM reads row-major [K, ld]
// operands with transposing LDS reads).  Only the 256x256 tile has this form,
// so a GEMM that would run on smaller tiles keeps the transposes.
bool kmajor_fits(int64_t rows, int64_t ld) { return rows * ld * 2 < (int64_t(1) << 31); }
// C[M, N] = A[M, K] . B[K, N] with B row-major [K, ldb]; with kb_split > 0
// (a multiple of 64) rows [0, kb_split) of B are B0's and the rest B1's.
bool gemm_bkmajor_ok(int64_t M, int64_t N, int64_t K, int64_t kb_split, int cus) {
  const int64_t rows = kb_split > 0 ? std::max(kb_split, K - kb_split) : K;
  return choose_tile_linear(M, N, cus) == TILE_256x256 && kmajor_fits(rows, N) && kb_split % 64 == 0;
}
hipError_t gemm_bkmajor(const uint16_t* A, const uint16_t* B0, const uint16_t* B1, int64_t kb_split, int64_t M,
                        int64_t N, int64_t K, uint16_t* C, int cus, hipStream_t s) {
  GemmParams p = dense_params(A, K, B0, B1, nullptr, C, N, M, N, K, FMLP_ACT_NONE, cus);
  p.kmajor = 2;
  p.ldb = N;
  p.kb_split = kb_split;
  return launch_gemm(GEMM_OUT_BF16, false, false, TILE_256x256, p, s);
}
// C[R, Cc] = A^T B over T token rows, A row-major [T, lda] (columns 0 .. R-1),
// B row-major [T, ldb] (columns 0 .. Cc-1): a weight gradient without copies
bool wgrad_kmajor_ok(int64_t R, int64_t T, int64_t Cc, int64_t lda, int64_t ldb, int cus) {
  const bool tile_ok = wgrad_split(R, T, Cc) > 1 || choose_tile_linear(R, Cc, cus) == TILE_256x256;
  return tile_ok && kmajor_fits(T, lda) && kmajor_fits(T, ldb);
}
hipError_t gemm_wgrad_kmajor(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int64_t R, int64_t T,
                             int64_t Cc, uint16_t* C, float* parts, int cus, hipStream_t s) {
  const int P = wgrad_split(R, T, Cc);
  GemmParams p = dense_params(A, lda, B, nullptr, nullptr, P > 1 ? static_cast<void*>(parts) : C, Cc, R, Cc, T,
                              FMLP_ACT_NONE, cus);
  p.kmajor = 3;
  p.ldb = ldb;
  if (P == 1) return launch_gemm(GEMM_OUT_BF16, false, false, TILE_256x256, p, s);
  p.ksplit = P;
  p.c_kstride = R * Cc;
  const hipError_t e = launch_gemm(GEMM_OUT_F32_SCALED, false, false, TILE_256x256, p, s);
  if (e != hipSuccess) return e;
  return launch_sum_parts(parts, P, R * Cc, R * Cc, C, s);
}

struct LinearBwdLayout {
  size_t dz, wt, dzt, xt, parts, total;
};
LinearBwdLayout linear_bwd_layout(int64_t M, int64_t K, int64_t N) {
  const int64_t Mp = pad8(M);
  LinearBwdLayout L;
  size_t o = kHeader;   // the decode header stays untouched: one workspace serves every call
  L.dz = o;  o += ws_bf16(M, N);
  L.wt = o;  o += ws_bf16(K, N);
  L.dzt = o; o += ws_bf16(N, Mp);
  L.xt = o;  o += ws_bf16(K, Mp);
  L.parts = o; o += wgrad_parts_bytes(N, Mp, K);
  L.total = o;
  return L;
}

struct GluBwdLayout {
  size_t wdt, dm, m, dgdu, wgut, dyt, mt, dgdut, xt, parts, total;
};
GluBwdLayout glu_bwd_layout(int64_t M, int64_t D, int64_t H) {
  const int64_t Mp = pad8(M);
  GluBwdLayout L;
  size_t o = kHeader;
  L.wdt = o;   o += ws_bf16(H, D);
  L.dm = o;    o += ws_bf16(M, H);
  L.m = o;     o += ws_bf16(M, H);
  L.dgdu = o;  o += ws_bf16(M, 2 * H);
  L.wgut = o;  o += ws_bf16(D, 2 * H);
  L.dyt = o;   o += ws_bf16(D, Mp);
  L.mt = o;    o += ws_bf16(H, Mp);
  L.dgdut = o; o += ws_bf16(2 * H, Mp);
  L.xt = o;    o += ws_bf16(D, Mp);
  L.parts = o; o += std::max(wgrad_parts_bytes(D, Mp, H), wgrad_parts_bytes(H, Mp, D));
  L.total = o;
  return L;
}

fmlp_status check_workspace(void* workspace, size_t workspace_bytes, size_t need) {
  if (need == 0) return FMLP_OK;
  if (workspace == nullptr) return fail(FMLP_E_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
  if (!aligned16(workspace)) return fail(FMLP_E_ALIGN, "workspace is not 16-byte aligned");
  if (workspace_bytes < need) return fail(FMLP_E_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  return FMLP_OK;
}

#define HIP_TRY(expr, what)                               \
  do {                                                    \
    hipError_t e_ = (expr);                               \
    if (e_ != hipSuccess) return launched(e_, what);      \
  } while (0)
}  // namespace

extern "C" {

size_t fmlp_linear_bwd_workspace_size(int64_t M, int64_t K, int64_t N) {
  if (M < 0 || K <= 0 || N <= 0) return 0;
  return linear_bwd_layout(M, K, N).total;
}

fmlp_status fmlp_linear_bwd(const fmlp_bf16* x, const fmlp_bf16* W, const fmlp_bf16* b, int act,
                            const fmlp_bf16* dy, int64_t M, int64_t K, int64_t N, fmlp_bf16* dx, fmlp_bf16* dW,
                            fmlp_bf16* db, void* workspace, size_t workspace_bytes, fmlp_stream stream) {
  TRY(check_rows("M", M));
  if (M >= kBwdMaxTokens) return fail(FMLP_E_SHAPE, "M=%lld must be below 2^22 for the backward pass", (long long)M);
  TRY(check_inner("K", K));
  TRY(check_inner("N", N));
  TRY(check_act(act));
  TOKEN_PTR(x, M);
  REQUIRE_PTR(W);
  OPTIONAL_PTR(b);
  TOKEN_PTR(dy, M);
  TOKEN_PTR(dx, M);
  REQUIRE_PTR(dW);
  OPTIONAL_PTR(db);
  const LinearBwdLayout L = linear_bwd_layout(M, K, N);
  TRY(check_workspace(workspace, workspace_bytes, L.total));
  int cus = 0;
  TRY(check_device(&cus));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (M == 0) {   // no tokens: the weight and bias gradients are sums over nothing
    HIP_TRY(launch_fill_zero(dW, N * K, s), "linear_bwd zero dW");
    if (db) HIP_TRY(launch_fill_zero(db, N, s), "linear_bwd zero db");
    return ok();
  }
  char* ws = static_cast<char*>(workspace);
  const int64_t Mp = pad8(M);
  uint16_t* wt = reinterpret_cast<uint16_t*>(ws + L.wt);
  uint16_t* dzt = reinterpret_cast<uint16_t*>(ws + L.dzt);
  uint16_t* xt = reinterpret_cast<uint16_t*>(ws + L.xt);
  const uint16_t* dz = dy;
  if (act != FMLP_ACT_NONE) {   // dz = dy * act'(x W^T + b): the forward GEMM with the derivative epilogue
    uint16_t* dzw = reinterpret_cast<uint16_t*>(ws + L.dz);
    GemmParams p = dense_params(x, K, W, nullptr, b, dzw, N, M, N, K, act, cus);
    p.E = dy;
    p.lde = N;
    HIP_TRY(launch_gemm(GEMM_OUT_DACT, false, false, choose_tile(M, (N + 255) / 256, cus), p, s),
            "linear_bwd dz launch");
    dz = dzw;
  }
  // dx = dz W: the contraction runs over W's rows (W read k-major, or
  // transposed first where the GEMM runs on smaller tiles)
  if (gemm_bkmajor_ok(M, K, N, 0, cus)) {
    HIP_TRY(gemm_bkmajor(dz, W, nullptr, 0, M, K, N, dx, cus, s), "linear_bwd dx launch");
  } else {
    HIP_TRY(launch_transpose(W, N, K, K, wt, N, N, s), "linear_bwd transpose W");
    HIP_TRY(gemm_linear(dz, wt, nullptr, FMLP_ACT_NONE, M, N, K, dx, cus, s), "linear_bwd dx launch");
  }
  // dW = dz^T x and db = sum over tokens: both contract over the token rows
  // (dz and x read k-major; dz transposed for the row sum of db)
  bool have_dzt = false;
  float* parts = reinterpret_cast<float*>(ws + L.parts);
  if (wgrad_kmajor_ok(N, M, K, N, K, cus)) {
    HIP_TRY(gemm_wgrad_kmajor(dz, N, x, K, N, M, K, dW, parts, cus, s), "linear_bwd dW launch");
  } else {
    HIP_TRY(launch_transpose(dz, M, N, N, dzt, Mp, Mp, s), "linear_bwd transpose dz");
    HIP_TRY(launch_transpose(x, M, K, K, xt, Mp, Mp, s), "linear_bwd transpose x");
    HIP_TRY(gemm_wgrad(dzt, xt, N, Mp, K, dW, parts, cus, s), "linear_bwd dW launch");
    have_dzt = true;
  }
  if (db) {
    if (!have_dzt) HIP_TRY(launch_transpose(dz, M, N, N, dzt, Mp, Mp, s), "linear_bwd transpose dz");
    HIP_TRY(launch_rowsum(dzt, N, Mp, Mp, db, s), "linear_bwd db launch");
  }
  return ok();
}

size_t fmlp_glu_bwd_workspace_size(int64_t M, int64_t D, int64_t H) {
  if (M < 0 || D <= 0 || H <= 0) return 0;
  return glu_bwd_layout(M, D, H).total;
}

fmlp_status fmlp_glu_bwd(const fmlp_bf16* x, const fmlp_bf16* Wg, const fmlp_bf16* Wu, const fmlp_bf16* Wd,
                         int gate_act, const fmlp_bf16* dy, int64_t M, int64_t D, int64_t H, fmlp_bf16* dx,
                         fmlp_bf16* dWg, fmlp_bf16* dWu, fmlp_bf16* dWd, void* workspace, size_t workspace_bytes,
                         fmlp_stream stream) {
  TRY(check_rows("M", M));
  if (M >= kBwdMaxTokens) return fail(FMLP_E_SHAPE, "M=%lld must be below 2^22 for the backward pass", (long long)M);
  TRY(check_inner("D", D));
  TRY(check_inner("H", H));
  if (2 * H >= kMaxInner) return fail(FMLP_E_SHAPE, "H=%lld: 2H must be below 2^22", (long long)H);
  TRY(check_act(gate_act, "gate_act"));
  TOKEN_PTR(x, M);
  REQUIRE_PTR(Wg);
  REQUIRE_PTR(Wu);
  REQUIRE_PTR(Wd);
  TOKEN_PTR(dy, M);
  TOKEN_PTR(dx, M);
  REQUIRE_PTR(dWg);
  REQUIRE_PTR(dWu);
  REQUIRE_PTR(dWd);
  const GluBwdLayout L = glu_bwd_layout(M, D, H);
  TRY(check_workspace(workspace, workspace_bytes, L.total));
  int cus = 0;
  TRY(check_device(&cus));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (M == 0) {
    HIP_TRY(launch_fill_zero(dWg, H * D, s), "glu_bwd zero dWg");
    HIP_TRY(launch_fill_zero(dWu, H * D, s), "glu_bwd zero dWu");
    HIP_TRY(launch_fill_zero(dWd, D * H, s), "glu_bwd zero dWd");
    return ok();
  }
  char* ws = static_cast<char*>(workspace);
  auto at = [&](size_t off) { return reinterpret_cast<uint16_t*>(ws + off); };
  const int64_t Mp = pad8(M);
  // dm = dy Wd: the contraction runs over Wd's rows (Wd read k-major, or
  // transposed first where the GEMM runs on smaller tiles)
  if (gemm_bkmajor_ok(M, H, D, 0, cus)) {
    HIP_TRY(gemm_bkmajor(dy, Wd, nullptr, 0, M, H, D, at(L.dm), cus, s), "glu_bwd dm launch");
  } else {
    HIP_TRY(launch_transpose(Wd, D, H, H, at(L.wdt), D, D, s), "glu_bwd transpose Wd");
    HIP_TRY(gemm_linear(dy, at(L.wdt), nullptr, FMLP_ACT_NONE, M, D, H, at(L.dm), cus, s), "glu_bwd dm launch");
  }
  // the gate+up GEMM again, with the derivative epilogue: m, and [dg | du]
  GemmParams p = dense_params(x, D, Wg, Wu, nullptr, at(L.m), H, M, H, D, gate_act, cus);
  p.E = at(L.dm);
  p.lde = H;
  p.C2 = at(L.dgdu);
  p.ldc2 = 2 * H;
  HIP_TRY(launch_gemm(GEMM_OUT_DGLU, false, false, choose_tile(M, (H + 127) / 128, cus), p, s),
          "glu_bwd gate+up launch");
  // dx = dg Wg + du Wu = [dg | du] [Wg ; Wu]: one GEMM over 2H (the weights
  // read k-major, B switching from Wg to Wu at row H, or transposed first)
  if (H % 64 == 0 && gemm_bkmajor_ok(M, D, 2 * H, H, cus)) {
    HIP_TRY(gemm_bkmajor(at(L.dgdu), Wg, Wu, H, M, D, 2 * H, dx, cus, s), "glu_bwd dx launch");
  } else {
    HIP_TRY(launch_transpose(Wg, H, D, D, at(L.wgut), 2 * H, H, s), "glu_bwd transpose Wg");
    HIP_TRY(launch_transpose(Wu, H, D, D, at(L.wgut) + H, 2 * H, H, s), "glu_bwd transpose Wu");
    HIP_TRY(gemm_linear(at(L.dgdu), at(L.wgut), nullptr, FMLP_ACT_NONE, M, 2 * H, D, dx, cus, s),
            "glu_bwd dx launch");
  }
  // weight gradients: contractions over the token rows (both operands read
  // k-major, or transposed first)
  float* parts = reinterpret_cast<float*>(ws + L.parts);
  if (wgrad_kmajor_ok(D, M, H, D, H, cus)) {
    HIP_TRY(gemm_wgrad_kmajor(dy, D, at(L.m), H, D, M, H, dWd, parts, cus, s), "glu_bwd dWd launch");
  } else {
    HIP_TRY(launch_transpose(dy, M, D, D, at(L.dyt), Mp, Mp, s), "glu_bwd transpose dy");
    HIP_TRY(launch_transpose(at(L.m), M, H, H, at(L.mt), Mp, Mp, s), "glu_bwd transpose m");
    HIP_TRY(gemm_wgrad(at(L.dyt), at(L.mt), D, Mp, H, dWd, parts, cus, s), "glu_bwd dWd launch");
  }
  if (wgrad_kmajor_ok(H, M, D, 2 * H, D, cus)) {
    HIP_TRY(gemm_wgrad_kmajor(at(L.dgdu), 2 * H, x, D, H, M, D, dWg, parts, cus, s), "glu_bwd dWg launch");
    HIP_TRY(gemm_wgrad_kmajor(at(L.dgdu) + H, 2 * H, x, D, H, M, D, dWu, parts, cus, s), "glu_bwd dWu launch");
  } else {
    HIP_TRY(launch_transpose(at(L.dgdu), M, 2 * H, 2 * H, at(L.dgdut), Mp, Mp, s), "glu_bwd transpose dg|du");
    HIP_TRY(launch_transpose(x, M, D, D, at(L.xt), Mp, Mp, s), "glu_bwd transpose x");
    HIP_TRY(gemm_wgrad(at(L.dgdut), at(L.xt), H, Mp, D, dWg, parts, cus, s), "glu_bwd dWg launch");
    HIP_TRY(gemm_wgrad(at(L.dgdut) + H * Mp, at(L.xt), H, Mp, D, dWu, parts, cus, s), "glu_bwd dWu launch");
  }
  return ok();
}

}  // extern "C"

// ---------------------------------------------------------------------------
// FP8-weight decode calls
// ---------------------------------------------------------------------------
extern "C" size_t fmlp_w8_workspace_size(int64_t M, int64_t H) {
  if (M <= 0 || H <= 0) return 0;
  // h after the decode header: M x H bf16, or at one token H / 2 words of
  // 8 bytes {bf16 pair, epoch} for the one-launch form
  const size_t h = std::max((size_t)M * (size_t)H * 2, M == 1 ? (size_t)H * 4 : (size_t)0);
  return kHeader + round_up(h, 256);
}

namespace {

#define SCALE_PTR(p)                                                        \
  do {                                                                      \
    if ((p) == nullptr) return fail(FMLP_E_NULL, "%s is NULL", #p);         \
    if ((reinterpret_cast<uintptr_t>(p) & 3u) != 0)                         \
      return fail(FMLP_E_ALIGN, "%s is not 4-byte aligned", #p);            \
  } while (0)

fmlp_status check_w8_rows(int64_t M) {
  TRY(check_rows("M", M));
  if (M > kDecodeMaxM)
    return fail(FMLP_E_ARG, "FP8-weight calls take M <= %lld tokens (M=%lld)", (long long)kDecodeMaxM,
                (long long)M);
  return FMLP_OK;
}

fmlp_status check_w8_inner(const char* name, int64_t v) {
  TRY(check_inner(name, v));
  if (v % 16 != 0) return fail(FMLP_E_ALIGN, "%s=%lld is not a multiple of 16", name, (long long)v);
  return FMLP_OK;
}

// The two-layer FP8 calls keep h (or m) after the same 8 KB header as the
// bf16 calls, which they never touch: one workspace can serve both kinds of
// call in any order without disturbing the decode barrier words.
fmlp_status check_w8_workspace(int64_t M, int64_t H, void* workspace, size_t workspace_bytes) {
  const size_t need = fmlp_w8_workspace_size(M, H);
  if (need == 0) return FMLP_OK;
  if (workspace == nullptr) return fail(FMLP_E_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
  if (!aligned16(workspace)) return fail(FMLP_E_ALIGN, "workspace is not 16-byte aligned");
  if (workspace_bytes < need)
    return fail(FMLP_E_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  return FMLP_OK;
}

}  // namespace

extern "C" {


fmlp_status fmlp_linear_w8(const fmlp_bf16* x, const fmlp_fp8* Wq, const float* w_scale,
                           const fmlp_bf16* b, int act, int64_t M, int64_t K, int64_t N,
                           fmlp_bf16* y, fmlp_stream stream) {
  TRY(check_w8_rows(M));
  TRY(check_w8_inner("K", K));
  TRY(check_inner("N", N));
  TRY(check_act(act));
  TOKEN_PTR(x, M);
  REQUIRE_PTR(Wq);
  SCALE_PTR(w_scale);
  OPTIONAL_PTR(b);
  TOKEN_PTR(y, M);
  if (M == 0) return ok();
  TRY(check_device());
  W8Layer L{x, Wq, w_scale, nullptr, nullptr, b, y, K, N, act};
  return launched(launch_decode_w8(L, (int)M, static_cast<hipStream_t>(stream)),
                  "linear (fp8 weights) launch");
}

fmlp_status fmlp_mlp2_w8(const fmlp_bf16* x, const fmlp_fp8* W1q, const float* s1,
                         const fmlp_bf16* b1, const fmlp_fp8* W2q, const float* s2,
                         const fmlp_bf16* b2, int act, int64_t M, int64_t K, int64_t H, int64_t N,
                         fmlp_bf16* y, void* workspace, size_t workspace_bytes, fmlp_stream stream) {
  TRY(check_w8_rows(M));
  TRY(check_w8_inner("K", K));
  TRY(check_w8_inner("H", H));
  TRY(check_inner("N", N));
  TRY(check_act(act));
  TOKEN_PTR(x, M);
  REQUIRE_PTR(W1q);
  SCALE_PTR(s1);
  OPTIONAL_PTR(b1);
  REQUIRE_PTR(W2q);
  SCALE_PTR(s2);
  OPTIONAL_PTR(b2);
  TOKEN_PTR(y, M);
  TRY(check_w8_workspace(M, H, workspace, workspace_bytes));
  if (M == 0) return ok();
  int cus = 0;
  TRY(check_device(&cus));
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint16_t* h = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + kHeader);
  W8Layer L1{x, W1q, s1, nullptr, nullptr, b1, h, K, H, act};
  W8Layer L2{h, W2q, s2, nullptr, nullptr, b2, y, H, N, FMLP_ACT_NONE};
  if (g_path != kPathGemm && decode_w8_two_applies((int)M, L1, L2, cus))
    return launched(launch_decode_w8_two(L1, L2, static_cast<uint32_t*>(workspace), cus, s, g_coop),
                    "mlp2 (fp8 weights, one launch)");
  hipError_t e = launch_decode_w8(L1, (int)M, s);
  if (e != hipSuccess) return launched(e, "mlp2 (fp8 weights) layer-1 launch");
  return launched(launch_decode_w8(L2, (int)M, s), "mlp2 (fp8 weights) layer-2 launch");
}

fmlp_status fmlp_glu_w8(const fmlp_bf16* x, const fmlp_fp8* Wgq, const float* sg,
                        const fmlp_fp8* Wuq, const float* su, const fmlp_fp8* Wdq, const float* sd,
                        int gate_act, int64_t M, int64_t D, int64_t H, fmlp_bf16* y,
                        void* workspace, size_t workspace_bytes, fmlp_stream stream) {
  TRY(check_w8_rows(M));
  TRY(check_w8_inner("D", D));
  TRY(check_w8_inner("H", H));
  TRY(check_act(gate_act, "gate_act"));
  TOKEN_PTR(x, M);
  REQUIRE_PTR(Wgq);
  SCALE_PTR(sg);
  REQUIRE_PTR(Wuq);
  SCALE_PTR(su);
  REQUIRE_PTR(Wdq);
  SCALE_PTR(sd);
  TOKEN_PTR(y, M);
  TRY(check_w8_workspace(M, H, workspace, workspace_bytes));
  if (M == 0) return ok();
  int cus = 0;
  TRY(check_device(&cus));
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint16_t* m = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + kHeader);
  W8Layer L1{x, Wgq, sg, Wuq, su, nullptr, m, D, H, gate_act};
  W8Layer L2{m, Wdq, sd, nullptr, nullptr, nullptr, y, H, D, FMLP_ACT_NONE};
  if (g_path != kPathGemm && decode_w8_two_applies((int)M, L1, L2, cus))
    return launched(launch_decode_w8_two(L1, L2, static_cast<uint32_t*>(workspace), cus, s, g_coop),
                    "glu (fp8 weights, one launch)");
  hipError_t e = launch_decode_w8(L1, (int)M, s);
  if (e != hipSuccess) return launched(e, "glu (fp8 weights) gate+up launch");
  return launched(launch_decode_w8(L2, (int)M, s), "glu (fp8 weights) down launch");
}

}  // extern "C"
