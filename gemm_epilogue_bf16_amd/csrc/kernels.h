// Internal launch interface between the C ABI (abi.cpp) and the gfx950
// kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fmlp {

// ---------------------------------------------------------------------------
// Tiled MFMA GEMM:  C[rows, N] = epilogue(A[rows, K] . B[N, K]^T)
// ---------------------------------------------------------------------------
enum GemmOut : int {
  GEMM_OUT_BF16 = 0,        // C bf16 = act(acc + bias)
  GEMM_OUT_GEGLU = 1,       // B0 = Wg, B1 = Wu; C bf16 [rows, N] = act(g) * u
  GEMM_OUT_F32_SCALED = 2,  // C fp32 = acc * row_scale[row]
  GEMM_OUT_DACT = 3,        // backward: C bf16 = E * act'(acc + bias)  (E = dy, z recomputed)
  GEMM_OUT_DGLU = 4,        // backward, B0 = Wg, B1 = Wu, E = dm [rows, N]: C = m = act(g) * u,
                            // C2 [rows, 2N]: columns [0, N) dg = dm * u * act'(g), [N, 2N) du = dm * act(g)
};

struct GemmParams {
  const uint16_t* A;       // activations, row stride lda (elements)
  int64_t lda;
  const uint16_t* B0;      // weights [N, K] (row stride K)
  const uint16_t* B1;      // second weight set for GEMM_OUT_GEGLU
  int64_t strideB;         // elements between consecutive groups' weights (grouped mode)
  const uint16_t* bias;    // [N] or nullptr (GEMM_OUT_BF16 only)
  void* C;                 // output, row stride ldc (elements)
  int64_t ldc;
  int64_t M, N, K;         // M: rows (dense mode)
  int act;                 // Act: of the output (GEMM_OUT_BF16) or of the gate (GEMM_OUT_GEGLU)
  // gather / grouped (mixture of experts)
  const int32_t* a_rows;     // gather: A row of each logical row, or nullptr
  int64_t a_src_rows;        // gather: rows of A (a_src_rows * lda * 2 < 2^31)
  const int32_t* group_off;  // grouped: [groups+1] logical row offsets
  const int32_t* tile_off;   // grouped: [groups+1] prefix of m-tiles per group
  int groups;
  const float* row_scale;    // GEMM_OUT_F32_SCALED: per logical row, or nullptr (1)
  int ksplit;                // GEMM_OUT_F32_SCALED: K split into this many equal parts (0 or 1: none);
                             // part j of a tile writes C + j * c_kstride
  int64_t c_kstride;
  const uint16_t* E;         // GEMM_OUT_DACT / GEMM_OUT_DGLU: the incoming gradient tile source
  int64_t lde;               //   (bf16, row stride lde)
  void* C2;                  // GEMM_OUT_DGLU: dg | du output, bf16, row stride ldc2
  int64_t ldc2;
  // k-major operands (the backward's contractions over rows, read without a
  // transpose copy; 256x256 tiles, plain bf16 or split fp32 output only):
  // bit 0: A is stored [K, lda] (the tile's rows are columns of A); bit 1: B is
  // stored [K, ldb] (the tile's columns are columns of B).  kb_split > 0 (a
  // multiple of 64, B k-major): k rows [0, kb_split) come from B0 and
  // [kb_split, K) from B1, both with row stride ldb.
  int kmajor;
  int64_t ldb;
  int64_t kb_split;
  int cus;                   // compute units: the persistent grid's size cap
  // launch geometry, filled by launch_gemm
  int tiles_m, tiles_n, group_m;
};

// ---------------------------------------------------------------------------
// Layout helpers of the backward pass (transpose.hip).
// ---------------------------------------------------------------------------
// out[c, r] = in[r, c] for bf16 in [R, C] (row stride ldi) into out with row
// stride ldo starting at column 0; columns R .. ldo_pad-1 of every output row
// are written as zeros (the contraction over R may then run to ldo_pad).
hipError_t launch_transpose(const uint16_t* in, int64_t R, int64_t C, int64_t ldi, uint16_t* out, int64_t ldo,
                            int64_t ldo_pad, hipStream_t s);
// out[r] = bf16(sum_c in[r, c]) for bf16 in [R, C] (row stride ld), summed in
// fp32 in a fixed order (deterministic).
hipError_t launch_rowsum(const uint16_t* in, int64_t R, int64_t C, int64_t ld, uint16_t* out, hipStream_t s);

// out[0, n) = 0 (bf16): the weight gradients of a call with no tokens.
hipError_t launch_fill_zero(uint16_t* out, int64_t n, hipStream_t s);

// out[i] = bf16(parts[0][i] + parts[1][i] + ... + parts[P-1][i]) for i < n
// (fp32 parts of a GEMM split over K, stride `stride` floats apart, added in
// part order: deterministic); n % 8 == 0.
hipError_t launch_sum_parts(const float* parts, int P, int64_t stride, int64_t n, uint16_t* out, hipStream_t s);

// Tile configurations compiled in.
enum GemmTile : int {
  TILE_128x128 = 0,   // 4 waves, 64x64 per wave
  TILE_256x256 = 1,   // 8 waves, 128x64 per wave
  TILE_128x192 = 2,   // 8 waves, 32x96 per wave; plain bf16 output only
  TILE_COUNT
};

int gemm_tile_bm(int tile);
int gemm_tile_bn(int tile);
// Launch one GEMM on a persistent grid of at most p.cus blocks.  For grouped
// mode p.tiles_m must be an upper bound on the number of m tiles over all
// groups (it sizes the grid; the kernel counts the tiles that exist).
hipError_t launch_gemm(int out_kind, bool gather, bool grouped, int tile, GemmParams p,
                       hipStream_t s);

// ---------------------------------------------------------------------------
// Skinny-M (decode) path: M <= 16 rows, weights streamed once with 16-byte
// loads, fp32 MFMA accumulation, fixed-order cross-wave reduction.
// ---------------------------------------------------------------------------
struct GemvLayer {
  const uint16_t* x;     // [M, K]
  const uint16_t* W0;    // [N, K]
  const uint16_t* W1;    // [N, K] (GeGLU up) or nullptr
  const uint16_t* bias;  // [N] or nullptr
  uint16_t* y;           // [M, N]
  int64_t K, N;
  int act;               // Act; for a gated layer, the gate's activation
  int geglu;             // 1: y = act(x W0^T) * (x W1^T)
};

// One layer, one launch.
hipError_t launch_gemv(const GemvLayer& L, int M, hipStream_t s);

// Workspace header shared by the two-layer decode kernel: 32-bit words.
// Word kSyncGenWord holds the barrier generation, kSyncTimeoutWord counts waits
// that gave up, and words kSyncFlagWord0 + b are block b's arrival flags.  The
// header must be zero before its first use; the kernel only ever moves the
// generation forward, so it stays valid across calls and grid sizes.
constexpr int kWorkspaceHeaderBytes = 8192;
constexpr int kSyncGenWord = 0;
constexpr int kSyncTimeoutWord = 2;
constexpr int kSyncFlagWord0 = 64;
constexpr int kDecodeMaxBlocks = kWorkspaceHeaderBytes / 4 - kSyncFlagWord0;
static_assert(kDecodeMaxBlocks % 4 == 0, "flags are read 4 at a time");

// Two dependent layers in ONE launch: every block is resident at once, layer-1
// outputs are published through device-coherent stores and a flag barrier,
// layer-2 weights stream across the barrier.  sync = the workspace header.
// The second layer has no activation (L2.act must be ACT_NONE).
hipError_t launch_gemv2_persistent(const GemvLayer& L1, const GemvLayer& L2, int M,
                                   uint32_t* sync, hipStream_t s, bool cooperative = false);

// A 32-bit tag per launch, different for every launch of this process (for
// 2^32 launches) and most likely for other processes: the epoch salt of the
// one-launch decode and of the fused gated block's arrival words.
uint32_t next_launch_salt();

// ---------------------------------------------------------------------------
// The gated block in one launch with m kept on chip (glu_fused.hip), for
// D <= kGluFusedMaxD: y = (act(x Wg^T) * (x Wu^T)) Wd^T.  ws holds
// glu_fused_workspace_bytes(M, D, H) bytes (no initialisation needed).
// ---------------------------------------------------------------------------
constexpr int64_t kGluFusedMaxD = 1024;
constexpr int64_t kGluFusedMaxH = 1 << 22;   // 32-bit byte offsets of a 256-row Wd stage
constexpr int kGluFusedRows = 64;      // token rows per block
constexpr int kGluFusedSub = 128;      // hidden units per sub-chunk
constexpr int kGluFusedMaxParts = 8;
// The hidden range splits into S parts of hc units (a multiple of 128), S
// chosen so that the m_tiles * S blocks fill a 256-CU device, with no empty
// part.  With S > 1 the workspace holds S fp32 partials of y.
struct GluFusedShape {
  int64_t m_tiles;
  int S, hc;
};
inline GluFusedShape glu_fused_shape(int64_t M, int64_t H) {
  GluFusedShape f;
  f.m_tiles = (M + kGluFusedRows - 1) / kGluFusedRows;
  const int64_t subs = (H + kGluFusedSub - 1) / kGluFusedSub;
  int64_t S = f.m_tiles > 0 ? (256 + f.m_tiles - 1) / f.m_tiles : 1;
  S = S < kGluFusedMaxParts ? S : kGluFusedMaxParts;
  S = S < subs ? S : subs;
  S = S > 1 ? S : 1;
  const int64_t per = (subs + S - 1) / S;   // sub-chunks per part
  f.hc = (int)(per * kGluFusedSub);
  f.S = (int)((subs + per - 1) / per);
  return f;
}
inline size_t glu_fused_arrive_bytes(int64_t m_tiles) { return ((size_t)m_tiles * 8 + 255) / 256 * 256; }
inline size_t glu_fused_workspace_bytes(int64_t M, int64_t D, int64_t H) {
  if (M <= 0 || D <= 0 || H <= 0) return 0;
  const GluFusedShape f = glu_fused_shape(M, H);
  const size_t parts = f.S > 1 ? (size_t)f.S * (size_t)f.m_tiles * kGluFusedRows * (size_t)D * 4 : 0;
  return glu_fused_arrive_bytes(f.m_tiles) + parts;
}
hipError_t launch_glu_fused(const uint16_t* x, const uint16_t* Wg, const uint16_t* Wu, const uint16_t* Wd, int act,
                            int64_t M, int64_t D, int64_t H, uint16_t* y, void* ws, uint32_t salt, hipStream_t s);

// ---------------------------------------------------------------------------
// Small fused MLP: K, H, N <= 128, any M; one launch.
// ---------------------------------------------------------------------------
hipError_t launch_small_mlp2(const uint16_t* x, const uint16_t* W1, const uint16_t* b1,
                             const uint16_t* W2, const uint16_t* b2, int act, int64_t M,
                             int K, int H, int N, uint16_t* y, hipStream_t s);

// ---------------------------------------------------------------------------
// Mixture of experts: routing buckets and weighted combine.
// ---------------------------------------------------------------------------
struct MoeRouteOut {
  int32_t* tok_of;      // [P] token of each sorted pair position
  float* scale_of;      // [P] gate weight of each sorted pair position
  int32_t* pos_of;      // [P] sorted position of pair p (-1: invalid id)
  int32_t* group_off;   // [E+1]
  int32_t* tile_off;    // [E+1] prefix of ceil(count/BM)
  int32_t* err;         // invalid-id count
};
// The route runs over blocks of kMoeRoutePairsPerBlock pairs; `counts` is a
// device scratch array of moe_route_counts_bytes(T * top_k, E) bytes (the
// blocks' per-expert counts, then their prefixes).
constexpr int kMoeRoutePairsPerBlock = 512;
constexpr int kMoeRouteMaxExperts = 1024;
inline size_t moe_route_counts_bytes(int64_t P, int E) {
  return (size_t)((P + kMoeRoutePairsPerBlock - 1) / kMoeRoutePairsPerBlock) * (size_t)(E + 1) * 4;
}
hipError_t launch_moe_route(const int32_t* ids, const float* gate_w, int64_t T, int top_k, int E,
                            int bm, const MoeRouteOut& o, int32_t* counts, hipStream_t s);
hipError_t launch_moe_combine(const float* ytilde, const int32_t* pos_of, int64_t T, int top_k,
                              int64_t D, int ksplit, int64_t kstride, uint16_t* y, hipStream_t s);
// Router: logits = x[T,D] . Wr[E,D]^T (fp32), top_k ids per token (ties to the
// lower id) and softmax gate weights over them; logits may be nullptr.  cus:
// the device's compute units (picks the load batching of the <= 16-expert form).
constexpr int kRouterMaxExperts = 64;
hipError_t launch_moe_router(const uint16_t* x, const uint16_t* Wr, int64_t T, int D, int E, int top_k,
                             int32_t* ids, float* gate_w, float* logits, int cus, hipStream_t s);

}  // namespace fmlp
