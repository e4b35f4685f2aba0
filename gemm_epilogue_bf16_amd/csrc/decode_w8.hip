// Decode path with FP8 weights (M <= 16 tokens) for gfx950.
//
// A decode feed-forward layer is bound by reading its weights once (ainews.cool
// "PyTorch fused MLP efficiency", section "architectural impact": decode is
// memory-bandwidth bound), so storing them as one byte each halves the bytes
// and the time floor of the bf16 path.  Weights are OCP FP8 E4M3 codes
// ("e4m3fn": bias 7, no infinities, 0x7F/0xFF are NaN, largest finite 448)
// with one fp32 scale per output row: W[n, k] = scale[n] * e4m3(q[n, k]).
// Activations stay bf16.
//
// Dequantisation is exact: every finite E4M3 value is a bf16 value (3 mantissa
// bits, exponents within bf16's range), so the hardware fp8 -> fp32 conversion
// followed by taking the upper 16 bits gives the bf16 operand with no
// rounding, and v_mfma_f32_16x16x32_bf16 accumulates x . q in fp32.  The scale
// multiplies the fp32 sum once, in the epilogue, with the bias and the
// activation; one rounding to bf16 at the store.
//
// Layout.  One block of 8 waves owns 16 output rows (16 gate and 16 up rows
// for a gated layer) over the whole k range, so no cross-block reduction is
// needed.  Weights go from memory straight into registers with 16-byte buffer
// loads: lane l reads row l % 16, and the four lanes of a row read 64
// consecutive bytes; two consecutive loads of a wave read the two halves of
// one 128-byte line of every row, and wave w takes lines w, w + 8, w + 16, ...,
// so the 8 waves together read 1 KB contiguous of every row per step and
// every byte once.  A lane's 16 codes are two MFMA k groups of 8: the
// contraction is order-free, so each 16-byte weight load is paired with the two
// 16-byte activation loads of the same 16 k (token l % 16, zero past M), which
// come from L2.  Batches of U loads per stream are double-buffered in
// registers, so the next batch is in flight while this one is converted and
// multiplied.  Rows past N, tokens past M and k past K are masked by buffer
// offsets (a load past the descriptor's end returns zero without a memory
// access), never by a branch around a load.
//
// The 8 partial 16 x 16 tiles are summed in a fixed order (bitwise
// deterministic) by wave 0, which applies the epilogue and stores.
#include <algorithm>

#include "common.h"
#include "decode_w8.h"
#include "exchange.h"
#include "kernels.h"

namespace fmlp {

namespace {

constexpr int kW8Waves = 8;
constexpr int kW8Threads = kW8Waves * 64;
constexpr uint32_t kW8OutOfRange = 0x80000000u;   // offset past any descriptor's end

__device__ __forceinline__ __amdgpu_buffer_rsrc_t w8_desc(const void* base, uint32_t bytes) {
  // raw buffer: stride 0, num_records = bytes, the gfx9 data-format word
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4_t w8_load(__amdgpu_buffer_rsrc_t d, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(d, (int)off, 0, 0));
}

// weights are read exactly once: the non-temporal policy keeps them from
// displacing the activations in L2
__device__ __forceinline__ u32x4_t w8_load_stream(__amdgpu_buffer_rsrc_t d, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(d, (int)off, 0, 2));
}

// 2 E4M3 codes (bytes 0, 1 of q, or 2, 3 with HI) -> 2 bf16 in one word, exact
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16(uint32_t q) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8((int)q, HI);
  return (__float_as_uint(a[0]) >> 16) | (__float_as_uint(a[1]) & 0xFFFF0000u);
}

// 16 codes (k 0..15 in byte order) -> the two 8-element bf16 MFMA operands
// (k 0..7 and k 8..15)
__device__ __forceinline__ void e4m3x16_to_bf16(const u32x4_t& q, u32x4_t& a0, u32x4_t& a1) {
  a0[0] = e4m3x2_to_bf16<false>(q[0]);
  a0[1] = e4m3x2_to_bf16<true>(q[0]);
  a0[2] = e4m3x2_to_bf16<false>(q[1]);
  a0[3] = e4m3x2_to_bf16<true>(q[1]);
  a1[0] = e4m3x2_to_bf16<false>(q[2]);
  a1[1] = e4m3x2_to_bf16<true>(q[2]);
  a1[2] = e4m3x2_to_bf16<false>(q[3]);
  a1[3] = e4m3x2_to_bf16<true>(q[3]);
}

template <bool DUAL, int U>
struct W8Batch {
  static_assert(U % 2 == 0, "loads pair up on 128-byte lines");
  u32x4_t w0[U];
  u32x4_t w1[DUAL ? U : 1];
  u32x4_t x[U][2];
};

// 64-byte k chunk of load j of batch b: loads j and j + 1 of a wave read the
// two halves of one 128-byte line of each row, so a line is requested by one
// wave only
__device__ __forceinline__ int w8_chunk(int b, int U, int j, int wave) {
  const int q = b * U + j;
  return 2 * ((q >> 1) * kW8Waves + wave) + (q & 1);
}

// XB > 0: the activations were staged in LDS and are not loaded here
template <bool DUAL, int U, int XB>
__device__ __forceinline__ void w8_issue(W8Batch<DUAL, U>& B, int b, int wave, int g, int K,
                                         __amdgpu_buffer_rsrc_t d0, __amdgpu_buffer_rsrc_t d1,
                                         __amdgpu_buffer_rsrc_t dx, uint32_t wrow, uint32_t xrow) {
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const int c = w8_chunk(b, U, j, wave);
    const bool in = c * 64 + g * 16 < K;            // K % 16 == 0: a lane's 16 k are all in or all out
    const uint32_t wo = in ? wrow + (uint32_t)c * 64u : kW8OutOfRange;
    B.w0[j] = w8_load_stream(d0, wo);
    if constexpr (DUAL) B.w1[j] = w8_load_stream(d1, wo);
    if constexpr (XB == 0) {
      const uint32_t xo = in ? xrow + (uint32_t)c * 128u : kW8OutOfRange;
      B.x[j][0] = w8_load(dx, xo);
      B.x[j][1] = w8_load(dx, in ? xo + 16u : kW8OutOfRange);
    }
  }
}

// An empty asm that takes a batch's registers as operands: the instruction
// scheduler must keep every use of the batch after the loads issued before
// this point, so the wait for the batch never drains the next batch's loads.
template <bool DUAL, int U, int XB>
__device__ __forceinline__ void w8_hold(W8Batch<DUAL, U>& B) {
#pragma unroll
  for (int j = 0; j < U; ++j) {
    asm volatile("" : "+v"(B.w0[j]));
    if constexpr (DUAL) asm volatile("" : "+v"(B.w1[j]));
    if constexpr (XB == 0) asm volatile("" : "+v"(B.x[j][0]), "+v"(B.x[j][1]));
  }
}

template <bool DUAL, int U, int XB>
__device__ __forceinline__ void w8_consume(const W8Batch<DUAL, U>& B, int b, int wave, int g, int K,
                                           bool xrow_ok, const uint8_t* xl, f32x4_t& acc0,
                                           f32x4_t& acc1) {
#pragma unroll
  for (int j = 0; j < U; ++j) {
    u32x4_t x0, x1;
    if constexpr (XB == 0) {
      x0 = B.x[j][0];
      x1 = B.x[j][1];
    } else {
      // zero for tokens past M and k past K (the padding is never read as data)
      const int c = w8_chunk(b, U, j, wave);
      const bool ok = xrow_ok && c * 64 + g * 16 < K;
      const int off = ok ? c * 128 : 0;
      x0 = *reinterpret_cast<const u32x4_t*>(xl + off);
      x1 = *reinterpret_cast<const u32x4_t*>(xl + off + 16);
      if (!ok) x0 = x1 = zero4();
    }
    u32x4_t a0, a1;
    e4m3x16_to_bf16(B.w0[j], a0, a1);
    acc0 = mfma_16x16x32(a0, x0, acc0);
    acc0 = mfma_16x16x32(a1, x1, acc0);
    if constexpr (DUAL) {
      e4m3x16_to_bf16(B.w1[j], a0, a1);
      acc1 = mfma_16x16x32(a0, x0, acc1);
      acc1 = mfma_16x16x32(a1, x1, acc1);
    }
  }
}

// XB: bytes of LDS for the activations, M rows of 2K + 16 bytes (the 16-byte
// pad puts the 16 token rows of a fragment read in different banks); 0: the
// activations are loaded from memory beside the weights.
template <bool DUAL, int U, int XB>
__global__ __launch_bounds__(kW8Threads) void decode_w8_kernel(W8Layer L, int M) {
  __shared__ f32x4_t red[DUAL ? 2 : 1][kW8Waves][64];
  __shared__ __attribute__((aligned(16))) uint8_t xs[XB > 0 ? XB : 16];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15;   // weight row in the tile; token for the activation operand
  const int g = lane >> 4;   // 16-byte k group within a 64-byte chunk
  const int K = (int)L.K;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int rows = (int)min<int64_t>(16, L.N - n0);

  const __amdgpu_buffer_rsrc_t d0 = w8_desc(L.W0 + n0 * L.K, (uint32_t)(rows * K));
  const __amdgpu_buffer_rsrc_t d1 = w8_desc(DUAL ? L.W1 + n0 * L.K : L.W0, (uint32_t)(rows * K));
  const __amdgpu_buffer_rsrc_t dx = w8_desc(L.x, (uint32_t)(M * K * 2));
  const uint32_t wrow = (uint32_t)(r * K + g * 16);
  const uint32_t xrow = (uint32_t)(r * K * 2 + g * 32);
  const int xstride = 2 * K + 16;
  // lanes of a token past M read token 0's row (inside xs) and drop the value
  const uint8_t* xl = xs + (r < M ? r : 0) * xstride + g * 32;

  const int chunks = (K + 63) / 64;
  const int nb = (chunks + kW8Waves * U - 1) / (kW8Waves * U);
  W8Batch<DUAL, U> A, B;
  // the first weight batch is in flight while the activations are staged
  w8_issue<DUAL, U, XB>(A, 0, wave, g, K, d0, d1, dx, wrow, xrow);
  if constexpr (XB > 0) {
    // Loads that write LDS, 1 KB of one activation row each (lanes past the
    // row's end masked off), all in flight before the one wait: a load into
    // registers and then LDS per 16-byte piece cost a round trip each (16 per
    // thread at 16 tokens).
    const int per_row = K / 8;                 // 16-byte pieces per row
    const int ipr = (per_row + 63) / 64;       // load instructions per row
    const i32x4_t xd = make_desc(reinterpret_cast<uint64_t>(L.x), (uint32_t)(M * K) * 2u);
    const uint32_t xs_lds = lds_addr(xs);
    for (int t = wave; t < M * ipr; t += kW8Waves) {   // wave-uniform
      const int m = t / ipr, q = t - m * ipr;
      const int c = q * 64 + lane;
      if (c < per_row)
        asm_load_lds(xd, uniform32(xs_lds + (uint32_t)(m * xstride + q * 1024)), (uint32_t)(m * K + c * 8) * 2u);
    }
    wait_vm<0>();
    __syncthreads();
  }
  f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f};
  f32x4_t acc1 = {0.f, 0.f, 0.f, 0.f};
  const bool xrow_ok = r < M;
  // Two register batches in ping-pong: each is consumed while the other is in
  // flight.  The loop runs while at least three batches remain; the last one
  // or two are peeled, so no batch past the end is issued.
  int b = 0;
  for (; b + 2 < nb; b += 2) {
    w8_issue<DUAL, U, XB>(B, b + 1, wave, g, K, d0, d1, dx, wrow, xrow);
    w8_hold<DUAL, U, XB>(A);
    w8_consume<DUAL, U, XB>(A, b, wave, g, K, xrow_ok, xl, acc0, acc1);
    w8_issue<DUAL, U, XB>(A, b + 2, wave, g, K, d0, d1, dx, wrow, xrow);
    w8_hold<DUAL, U, XB>(B);
    w8_consume<DUAL, U, XB>(B, b + 1, wave, g, K, xrow_ok, xl, acc0, acc1);
  }
  if (b + 1 < nb) {
    w8_issue<DUAL, U, XB>(B, b + 1, wave, g, K, d0, d1, dx, wrow, xrow);
    w8_hold<DUAL, U, XB>(A);
    w8_consume<DUAL, U, XB>(A, b, wave, g, K, xrow_ok, xl, acc0, acc1);
    w8_hold<DUAL, U, XB>(B);
    w8_consume<DUAL, U, XB>(B, b + 1, wave, g, K, xrow_ok, xl, acc0, acc1);
  } else {
    w8_hold<DUAL, U, XB>(A);
    w8_consume<DUAL, U, XB>(A, b, wave, g, K, xrow_ok, xl, acc0, acc1);
  }

  red[0][wave][lane] = acc0;
  if constexpr (DUAL) red[DUAL ? 1 : 0][wave][lane] = acc1;
  __syncthreads();
  if (wave != 0) return;
  f32x4_t s0 = red[0][0][lane];
  f32x4_t s1 = red[DUAL ? 1 : 0][0][lane];
#pragma unroll
  for (int w = 1; w < kW8Waves; ++w) {
    s0 += red[0][w][lane];
    if constexpr (DUAL) s1 += red[1][w][lane];
  }
  // lane holds rows 4g .. 4g+3 of the tile for token r
  const int m = r;
  if (m >= M) return;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int row = 4 * g + v;
    if (row >= rows) break;
    const int64_t n = n0 + row;
    float z;
    if constexpr (DUAL) {
      z = apply_act(s0[v] * L.s0[n], L.act) * (s1[v] * L.s1[n]);
    } else {
      z = s0[v] * L.s0[n];
      if (L.bias) z += bf16_to_f32(L.bias[n]);
      z = apply_act(z, L.act);
    }
    const __bf16 o = (__bf16)z;
    L.y[(int64_t)m * L.N + n] = __builtin_bit_cast(uint16_t, o);
  }
}

constexpr int kXSmall = 64 * 1024;    // one token up to K = 32760
constexpr int kXLarge = 136 * 1024;   // 16 tokens up to K = 4348

template <bool DUAL, int U>
hipError_t launch_w8(const W8Layer& L, int M, dim3 grid, hipStream_t s) {
  const int64_t xneed = (int64_t)M * (2 * L.K + 16);
  if (xneed <= kXSmall)
    hipLaunchKernelGGL((decode_w8_kernel<DUAL, U, kXSmall>), grid, dim3(kW8Threads), 0, s, L, M);
  else if (xneed <= kXLarge)
    hipLaunchKernelGGL((decode_w8_kernel<DUAL, U, kXLarge>), grid, dim3(kW8Threads), 0, s, L, M);
  else
    hipLaunchKernelGGL((decode_w8_kernel<DUAL, U, 0>), grid, dim3(kW8Threads), 0, s, L, M);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Both layers of a one-token FP8 forward in ONE launch (the bf16 engine's
// word-flag exchange, decode.hip): a persistent grid of at most one block per
// CU; each block streams its layer-1 tiles (16 output rows over the whole k
// range, as above, x staged once in LDS), publishes its h values as 8-byte
// words {bf16 pair, epoch} with device-coherent stores, gathers every block's
// words into LDS (polling until each carries this call's epoch, bounded and
// counted), then streams its layer-2 tiles against h in LDS.  Every block
// owns a layer-1 tile, so block 0 seeing every word means every block has
// read the generation: only then does block 0 advance it.
// ---------------------------------------------------------------------------

// The weight descriptors of a 16-row tile and the lane's row offset.
struct W8Tile {
  __amdgpu_buffer_rsrc_t d0, d1;
  uint32_t wrow;
};
template <bool DUAL>
__device__ __forceinline__ W8Tile w8_tile_at(const W8Layer& L, int64_t tile) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int K = (int)L.K;
  const int64_t n0 = tile * 16;
  const int rows = (int)min<int64_t>(16, L.N - n0);
  W8Tile t;
  t.d0 = w8_desc(L.W0 + n0 * L.K, (uint32_t)(rows * K));
  t.d1 = w8_desc(DUAL ? L.W1 + n0 * L.K : L.W0, (uint32_t)(rows * K));
  t.wrow = (uint32_t)(r * K + g * 16);
  return t;
}

// One 16-row tile over the whole k range with the activation row staged in
// LDS at xs (one token); wave 0 returns the summed accumulators.  A holds the
// first register batch (issued here).
template <bool DUAL, int U>
__device__ __forceinline__ void w8_tile_one_token(const W8Layer& L, int64_t tile, const uint8_t* xs,
                                                  f32x4_t (*red)[kW8Waves][64], f32x4_t& s0, f32x4_t& s1,
                                                  W8Batch<DUAL, U>& A) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int K = (int)L.K;
  const W8Tile tl = w8_tile_at<DUAL>(L, tile);
  const __amdgpu_buffer_rsrc_t d0 = tl.d0, d1 = tl.d1;
  const uint32_t wrow = tl.wrow;
  const uint8_t* xl = xs + g * 32;   // the one token's row; lanes of other tokens drop their value
  const bool xrow_ok = r == 0;
  const int chunks = (K + 63) / 64;
  const int nb = (chunks + kW8Waves * U - 1) / (kW8Waves * U);
  W8Batch<DUAL, U> B;
  f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f};
  f32x4_t acc1 = {0.f, 0.f, 0.f, 0.f};
  w8_issue<DUAL, U, 1>(A, 0, wave, g, K, d0, d1, d0, wrow, 0u);
  int b = 0;
  for (; b + 2 < nb; b += 2) {
    w8_issue<DUAL, U, 1>(B, b + 1, wave, g, K, d0, d1, d0, wrow, 0u);
    w8_hold<DUAL, U, 1>(A);
    w8_consume<DUAL, U, 1>(A, b, wave, g, K, xrow_ok, xl, acc0, acc1);
    w8_issue<DUAL, U, 1>(A, b + 2, wave, g, K, d0, d1, d0, wrow, 0u);
    w8_hold<DUAL, U, 1>(B);
    w8_consume<DUAL, U, 1>(B, b + 1, wave, g, K, xrow_ok, xl, acc0, acc1);
  }
  if (b + 1 < nb) {
    w8_issue<DUAL, U, 1>(B, b + 1, wave, g, K, d0, d1, d0, wrow, 0u);
    w8_hold<DUAL, U, 1>(A);
    w8_consume<DUAL, U, 1>(A, b, wave, g, K, xrow_ok, xl, acc0, acc1);
    w8_hold<DUAL, U, 1>(B);
    w8_consume<DUAL, U, 1>(B, b + 1, wave, g, K, xrow_ok, xl, acc0, acc1);
  } else {
    w8_hold<DUAL, U, 1>(A);
    w8_consume<DUAL, U, 1>(A, b, wave, g, K, xrow_ok, xl, acc0, acc1);
  }
  red[0][wave][lane] = acc0;
  if constexpr (DUAL) red[1][wave][lane] = acc1;
  __syncthreads();
  if (wave == 0) {
    s0 = red[0][0][lane];
    s1 = red[DUAL ? 1 : 0][0][lane];
#pragma unroll
    for (int w = 1; w < kW8Waves; ++w) {
      s0 += red[0][w][lane];
      if constexpr (DUAL) s1 += red[1][w][lane];
    }
  }
  __syncthreads();   // red is free for the next tile
}

constexpr int kW8TwoMaxH = 4096;   // h words gathered per block: 4 H bytes

template <bool DUAL1>
__global__ __launch_bounds__(kW8Threads) void decode_w8_two_kernel(W8Layer L1, W8Layer L2, uint32_t* sync,
                                                                   uint32_t salt) {
  __shared__ f32x4_t red[2][kW8Waves][64];
  __shared__ __attribute__((aligned(16))) uint8_t xs[kXSmall];   // x, then h: one bf16 row
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int G = (int)gridDim.x, blk = (int)blockIdx.x;
  const uint32_t gen_next = ld_coherent(sync + kSyncGenWord) + 1u;
  const uint32_t target = epoch_of(gen_next, salt);
  const int K1 = (int)L1.K, H = (int)L1.N;

  // the input row into LDS
  for (int i = tid; i < K1 / 8; i += kW8Threads)
    *reinterpret_cast<u32x4_t*>(xs + i * 16) = ld16(L1.x + (int64_t)i * 8);
  __syncthreads();

  // layer 1; wave 0's lanes of token 0 (r == 0) hold rows 4g .. 4g + 3 of a tile
  const __amdgpu_buffer_rsrc_t rh = make_rsrc(L1.y, (uint32_t)H * 4u);   // H / 2 words of 8 bytes
  const int64_t tiles1 = (L1.N + 15) / 16, tiles2 = (L2.N + 15) / 16;
  for (int64_t t = blk; t < tiles1; t += G) {
    f32x4_t s0, s1;
    W8Batch<DUAL1, DUAL1 ? 4 : 8> A1;
    w8_tile_one_token<DUAL1, DUAL1 ? 4 : 8>(L1, t, xs, red, s0, s1, A1);
    if (wave == 0 && r == 0) {
      const int64_t n = t * 16 + 4 * g;   // H % 16 == 0: all four rows exist
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (DUAL1) {
          v[i] = apply_act(s0[i] * L1.s0[n + i], L1.act) * (s1[i] * L1.s1[n + i]);
        } else {
          float z = s0[i] * L1.s0[n + i];
          if (L1.bias) z += bf16_to_f32(L1.bias[n + i]);
          v[i] = apply_act(z, L1.act);
        }
      }
      st_coherent_b128(rh, (uint32_t)n * 4u, u32x4_t{pack_bf16x2(v[0], v[1]), target, pack_bf16x2(v[2], v[3]), target});
    }
  }

  // (Issuing the first layer-2 weight batch here, to stream while h is
  // gathered, measured slower: 16.4 against 15.2 us for the 4096^3 forward,
  // since the gather's device-coherent polls then wait behind those loads.)
  // every block's h: 16-byte pieces of two words, each lane's pieces in flight
  // together, until both words carry this call's epoch
  {
    constexpr int kPer = kW8TwoMaxH / 4 / kW8Threads;   // pieces per thread
    const int pieces = H / 4;
    uint32_t pend = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (tid + kW8Threads * i < pieces) pend |= 1u << i;
    for (uint32_t spins = 0;; ++spins) {
      u32x4_t v[kPer];
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (pend & (1u << i))
          v[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                 rh, (uint32_t)(tid + kW8Threads * i) * 16u, 0, 16 /* sc1 */));
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        if ((pend & (1u << i)) && v[i][1] == target && v[i][3] == target) {
          *reinterpret_cast<u32x2_t*>(xs + (tid + kW8Threads * i) * 8) = u32x2_t{v[i][0], v[i][2]};
          pend &= ~(1u << i);
        }
      }
      if (__syncthreads_or(pend != 0) == 0) break;
      if (spins >= (1u << 20)) {
        if (tid == 0)
          __hip_atomic_fetch_add(sync + kSyncTimeoutWord, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (blk == 0 && tid == 0) st_coherent(sync + kSyncGenWord, gen_next);
  }

  // layer 2 against h in LDS
  for (int64_t t = blk; t < tiles2; t += G) {
    f32x4_t s0, s1;
    W8Batch<false, 8> A2;
    w8_tile_one_token<false, 8>(L2, t, xs, red, s0, s1, A2);
    if (wave == 0 && r == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t n = t * 16 + 4 * g + i;
        if (n >= L2.N) break;
        float z = s0[i] * L2.s0[n];
        if (L2.bias) z += bf16_to_f32(L2.bias[n]);
        const __bf16 o = (__bf16)z;
        L2.y[n] = __builtin_bit_cast(uint16_t, o);
      }
    }
  }
}

}  // namespace

bool decode_w8_two_applies(int M, const W8Layer& L1, const W8Layer& L2, int cus) {
  const int64_t tiles1 = (L1.N + 15) / 16;
  return M == 1 && L1.N <= kW8TwoMaxH && L1.N % 16 == 0 && L2.K == L1.N && 2 * L1.K <= kXSmall &&
         cus > 0 && cus <= kDecodeMaxBlocks && tiles1 >= 1;
}

hipError_t launch_decode_w8_two(const W8Layer& L1, const W8Layer& L2, uint32_t* sync, int cus, hipStream_t s,
                                bool cooperative) {
  if (!decode_w8_two_applies(1, L1, L2, cus)) return hipErrorInvalidValue;
  if (L1.K % 16 != 0 || L2.N <= 0) return hipErrorInvalidValue;
  const int64_t tiles1 = (L1.N + 15) / 16;
  // every block owns a layer-1 tile and all are resident at once: at most one per CU
  const unsigned grid = (unsigned)std::min<int64_t>(tiles1, cus);
  uint32_t salt = next_launch_salt();
  if (cooperative) {   // opt-in: the runtime refuses a grid that cannot be resident at once
    W8Layer a = L1, b = L2;
    void* args[] = {&a, &b, &sync, &salt};
    const void* f = L1.W1 ? reinterpret_cast<const void*>(&decode_w8_two_kernel<true>)
                          : reinterpret_cast<const void*>(&decode_w8_two_kernel<false>);
    return hipLaunchCooperativeKernel(f, dim3(grid), dim3(kW8Threads), args, 0, s);
  }
  if (L1.W1)
    hipLaunchKernelGGL((decode_w8_two_kernel<true>), dim3(grid), dim3(kW8Threads), 0, s, L1, L2, sync, salt);
  else
    hipLaunchKernelGGL((decode_w8_two_kernel<false>), dim3(grid), dim3(kW8Threads), 0, s, L1, L2, sync, salt);
  return hipGetLastError();
}

hipError_t launch_decode_w8(const W8Layer& L, int M, hipStream_t s) {
  if (M <= 0 || M > 16 || L.K <= 0 || L.K % 16 != 0 || L.N <= 0) return hipErrorInvalidValue;
  if (L.K * 16 * 2 >= (int64_t(1) << 31)) return hipErrorInvalidValue;   // descriptor sizes
  const int64_t tiles = (L.N + 15) / 16;
  if (tiles > (int64_t(1) << 31) - 1) return hipErrorInvalidValue;
  const dim3 grid((unsigned)tiles);
  return L.W1 ? launch_w8<true, 4>(L, M, grid, s) : launch_w8<false, 8>(L, M, grid, s);
}

}  // namespace fmlp
