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

// 2 E4M3 codes (bytes 0, 1 of q, or 2, 3 with HI) -> 2 bf16 in one word, exact:
// gfx950's scaled conversion with scale 1 (one instruction; an in-bounds check
// of all 65536 code pairs in both halves matched the fp32 conversion followed
// by taking the upper 16 bits, NaN codes included)
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16(uint32_t q) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q, 1.0f, HI));
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

// The activation operand of load j: from registers, or from the LDS row at xl
// (XB > 0), where tokens past M and k past K read the 32 zero bytes at xz
// instead (the padding is never read as data).
template <bool DUAL, int U, int XB>
__device__ __forceinline__ void w8_x(const W8Batch<DUAL, U>& B, int b, int j, int wave, int g, int K,
                                     bool xrow_ok, const uint8_t* xl, const uint8_t* xz, u32x4_t& x0,
                                     u32x4_t& x1) {
  if constexpr (XB == 0) {
    x0 = B.x[j][0];
    x1 = B.x[j][1];
  } else {
    const int c = w8_chunk(b, U, j, wave);
    const uint8_t* src = (xrow_ok && c * 64 + g * 16 < K) ? xl + c * 128 : xz;
    x0 = *reinterpret_cast<const u32x4_t*>(src);
    x1 = *reinterpret_cast<const u32x4_t*>(src + 16);
  }
}

// jmax < U: loads j >= jmax of the batch are not multiplied (wave-uniform)
template <bool DUAL, int U, int XB>
__device__ __forceinline__ void w8_consume(const W8Batch<DUAL, U>& B, int b, int wave, int g, int K,
                                           bool xrow_ok, const uint8_t* xl, const uint8_t* xz,
                                           f32x4_t& acc0, f32x4_t& acc1, int jmax = U) {
#pragma unroll
  for (int j = 0; j < U; ++j) {
    if (j >= jmax) break;
    u32x4_t x0, x1;
    w8_x<DUAL, U, XB>(B, b, j, wave, g, K, xrow_ok, xl, xz, x0, x1);
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

// Two batches of one wave (the k chunks of waves wa and wb of the one-role
// form) into their own accumulators, interleaved so that consecutive MFMAs
// never depend on each other; each accumulator sums in the one-role order.
template <bool DUAL>
__device__ __forceinline__ void w8_consume_two(const W8Batch<DUAL, 8>& A, const W8Batch<DUAL, 8>& B, int wa,
                                               int wb, int g, int K, bool xrow_ok, const uint8_t* xl,
                                               const uint8_t* xz, f32x4_t& a0, f32x4_t& a1, f32x4_t& b0,
                                               f32x4_t& b1, int jmax) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= jmax) break;
    u32x4_t xa0, xa1, xb0, xb1, wa0, wa1, wb0, wb1;
    w8_x<DUAL, 8, 1>(A, 0, j, wa, g, K, xrow_ok, xl, xz, xa0, xa1);
    w8_x<DUAL, 8, 1>(B, 0, j, wb, g, K, xrow_ok, xl, xz, xb0, xb1);
    e4m3x16_to_bf16(A.w0[j], wa0, wa1);
    e4m3x16_to_bf16(B.w0[j], wb0, wb1);
    a0 = mfma_16x16x32(wa0, xa0, a0);
    b0 = mfma_16x16x32(wb0, xb0, b0);
    a0 = mfma_16x16x32(wa1, xa1, a0);
    b0 = mfma_16x16x32(wb1, xb1, b0);
    if constexpr (DUAL) {
      e4m3x16_to_bf16(A.w1[j], wa0, wa1);
      e4m3x16_to_bf16(B.w1[j], wb0, wb1);
      a1 = mfma_16x16x32(wa0, xa0, a1);
      b1 = mfma_16x16x32(wb0, xb0, b1);
      a1 = mfma_16x16x32(wa1, xa1, a1);
      b1 = mfma_16x16x32(wb1, xb1, b1);
    }
  }
}

// The epilogue's per-row values of rows n .. n + 3 (the rows of lane group g
// in a tile): the scales and the bias, requested together at the start of the
// tile, so they cost no round trip of their own at the end.  A row past N
// reads row N - 1 (its value is never used); without a bias nothing is read
// (an empty buffer descriptor reads as zero).  The bias stays in its bf16
// bits until the epilogue: converting it where it is loaded would wait for the
// load there (the empty asm keeps the conversion from being hoisted).
template <bool DUAL>
struct W8Rows {
  float s0[4], s1[4];
  uint32_t b[4];
  __device__ __forceinline__ float bias(int i) const {
    uint32_t v = i == 0 ? b[0] : i == 1 ? b[1] : i == 2 ? b[2] : b[3];
    asm volatile("" : "+v"(v));
    return __uint_as_float(v << 16);
  }
  __device__ __forceinline__ float scale0(int i) const { return i == 0 ? s0[0] : i == 1 ? s0[1] : i == 2 ? s0[2] : s0[3]; }
  __device__ __forceinline__ float scale1(int i) const { return i == 0 ? s1[0] : i == 1 ? s1[1] : i == 2 ? s1[2] : s1[3]; }
};
template <bool DUAL>
__device__ __forceinline__ W8Rows<DUAL> w8_rows(const W8Layer& L, int64_t n) {
  W8Rows<DUAL> R;
  const __amdgpu_buffer_rsrc_t d0 = w8_desc(L.s0, (uint32_t)L.N * 4u);
  const __amdgpu_buffer_rsrc_t d1 = w8_desc(DUAL ? L.s1 : L.s0, (uint32_t)L.N * 4u);
  const __amdgpu_buffer_rsrc_t db = w8_desc(L.bias ? (const void*)L.bias : (const void*)L.s0,
                                            L.bias ? (uint32_t)L.N * 2u : 0u);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t row = (uint32_t)min<int64_t>(n + i, L.N - 1);
    R.s0[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(d0, (int)(row * 4u), 0, 0));
    if constexpr (DUAL)
      R.s1[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(d1, (int)(row * 4u), 0, 0));
    else
      R.s1[i] = 0.f;
    R.b[i] = __builtin_amdgcn_raw_buffer_load_b16(db, (int)(row * 2u), 0, 0);
  }
  return R;
}

// XB: bytes of LDS for the activations, M rows of 2K + 16 bytes (the 16-byte
// pad puts the 16 token rows of a fragment read in different banks) and 32
// zero bytes; 0: the activations are loaded from memory beside the weights.
template <bool DUAL, int U, int XB>
__global__ __launch_bounds__(kW8Threads) void decode_w8_kernel(W8Layer L, int M) {
  __shared__ f32x4_t red[DUAL ? 2 : 1][kW8Waves][64];
  __shared__ __attribute__((aligned(16))) uint8_t xs[XB > 0 ? XB : 16];
  // the activation operand of masked loads: the last 32 bytes of xs, past the
  // staged rows (a separate array would take the gated form's 80 KB past half
  // the CU's LDS, and two blocks would no longer fit)
  const uint8_t* xz = xs + (XB > 0 ? XB - 32 : 0);
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
  const W8Rows<DUAL> R = w8_rows<DUAL>(L, n0 + 4 * g);
  // The first weight batch is in flight while the activations are staged.  A
  // wave's loads return in issue order: with the larger staging (up to 16
  // token rows, several times the batch's bytes, from L2) the activations are
  // requested first, so that they do not land only after the batch.
  constexpr bool kXFirst = XB > 64 * 1024;
  if constexpr (!kXFirst) w8_issue<DUAL, U, XB>(A, 0, wave, g, K, d0, d1, dx, wrow, xrow);
  if constexpr (XB > 0) {
    // Loads that write LDS, 1 KB of one activation row each (lanes past the
    // row's end masked off), all in flight before the one wait: a load into
    // registers and then LDS per 16-byte piece cost a round trip each (16 per
    // thread at 16 tokens).
    const int per_row = K / 8;                 // 16-byte pieces per row
    const int ipr = (per_row + 63) / 64;       // load instructions per row
    const i32x4_t xd = make_desc(reinterpret_cast<uint64_t>(L.x), (uint32_t)(M * K) * 2u);
    const uint32_t xs_lds = lds_addr(xs);
    if (threadIdx.x < 2) *reinterpret_cast<u32x4_t*>(xs + XB - 32 + 16 * threadIdx.x) = zero4();
    for (int t = wave; t < M * ipr; t += kW8Waves) {   // wave-uniform
      const int m = t / ipr, q = t - m * ipr;
      const int c = q * 64 + lane;
      if (c < per_row)
        asm_load_lds(xd, uniform32(xs_lds + (uint32_t)(m * xstride + q * 1024)), (uint32_t)(m * K + c * 8) * 2u);
    }
    if constexpr (kXFirst) {
      w8_issue<DUAL, U, XB>(A, 0, wave, g, K, d0, d1, dx, wrow, xrow);
      wait_vm<(DUAL ? 2 : 1) * U>();   // everything but the batch: the rows' values and the activations
    } else {
      wait_vm<0>();
    }
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
    w8_consume<DUAL, U, XB>(A, b, wave, g, K, xrow_ok, xl, xz, acc0, acc1);
    w8_issue<DUAL, U, XB>(A, b + 2, wave, g, K, d0, d1, dx, wrow, xrow);
    w8_hold<DUAL, U, XB>(B);
    w8_consume<DUAL, U, XB>(B, b + 1, wave, g, K, xrow_ok, xl, xz, acc0, acc1);
  }
  if (b + 1 < nb) {
    w8_issue<DUAL, U, XB>(B, b + 1, wave, g, K, d0, d1, dx, wrow, xrow);
    w8_hold<DUAL, U, XB>(A);
    w8_consume<DUAL, U, XB>(A, b, wave, g, K, xrow_ok, xl, xz, acc0, acc1);
    w8_hold<DUAL, U, XB>(B);
    w8_consume<DUAL, U, XB>(B, b + 1, wave, g, K, xrow_ok, xl, xz, acc0, acc1);
  } else {
    w8_hold<DUAL, U, XB>(A);
    w8_consume<DUAL, U, XB>(A, b, wave, g, K, xrow_ok, xl, xz, acc0, acc1);
  }

  red[0][wave][lane] = acc0;
  if constexpr (DUAL) red[DUAL ? 1 : 0][wave][lane] = acc1;
  __syncthreads();
  // Waves 0-3 each finish one of the 4 rows a lane holds (rows 4g + v for
  // token r): the epilogue's activation is a chain of dependent instructions,
  // and one wave doing all 4 rows took about 1 us.  Each sum takes the 8
  // partial tiles in order, as one wave summing whole tiles would.
  if (wave >= 4) return;
  const int v = wave;
  const int m = r;
  const int row = 4 * g + v;
  if (m >= M || row >= rows) return;
  float s0 = reinterpret_cast<const float*>(&red[0][0][lane])[v];
  float s1 = reinterpret_cast<const float*>(&red[DUAL ? 1 : 0][0][lane])[v];
#pragma unroll
  for (int w = 1; w < kW8Waves; ++w) {
    s0 += reinterpret_cast<const float*>(&red[0][w][lane])[v];
    if constexpr (DUAL) s1 += reinterpret_cast<const float*>(&red[1][w][lane])[v];
  }
  const int64_t n = n0 + row;
  float z;
  if constexpr (DUAL) {
    z = apply_act(s0 * R.scale0(v), L.act) * (s1 * R.scale1(v));
  } else {
    z = s0 * R.scale0(v);
    if (L.bias) z += R.bias(v);
    z = apply_act(z, L.act);
  }
  const __bf16 o = (__bf16)z;
  L.y[(int64_t)m * L.N + n] = __builtin_bit_cast(uint16_t, o);
}

constexpr int kXSmall = 64 * 1024;    // one token up to K = 32736
constexpr int kXLarge = 136 * 1024;   // 16 tokens up to K = 4336

template <bool DUAL, int U>
hipError_t launch_w8(const W8Layer& L, int M, dim3 grid, hipStream_t s) {
  const int64_t xneed = (int64_t)M * (2 * L.K + 16) + 32;   // rows and the zero pad
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
                                                  const uint8_t* xz, f32x4_t (*red)[kW8Waves][64], f32x4_t& s0,
                                                  f32x4_t& s1, W8Batch<DUAL, U>& A) {
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
    w8_consume<DUAL, U, 1>(A, b, wave, g, K, xrow_ok, xl, xz, acc0, acc1);
    w8_issue<DUAL, U, 1>(A, b + 2, wave, g, K, d0, d1, d0, wrow, 0u);
    w8_hold<DUAL, U, 1>(B);
    w8_consume<DUAL, U, 1>(B, b + 1, wave, g, K, xrow_ok, xl, xz, acc0, acc1);
  }
  if (b + 1 < nb) {
    w8_issue<DUAL, U, 1>(B, b + 1, wave, g, K, d0, d1, d0, wrow, 0u);
    w8_hold<DUAL, U, 1>(A);
    w8_consume<DUAL, U, 1>(A, b, wave, g, K, xrow_ok, xl, xz, acc0, acc1);
    w8_hold<DUAL, U, 1>(B);
    w8_consume<DUAL, U, 1>(B, b + 1, wave, g, K, xrow_ok, xl, xz, acc0, acc1);
  } else {
    w8_hold<DUAL, U, 1>(A);
    w8_consume<DUAL, U, 1>(A, b, wave, g, K, xrow_ok, xl, xz, acc0, acc1);
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
  __shared__ u32x4_t xzero[2];   // the activation operand of masked loads
  const uint8_t* xz = reinterpret_cast<const uint8_t*>(xzero);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int G = (int)gridDim.x, blk = (int)blockIdx.x;
  const uint32_t gen_next = ld_coherent(sync + kSyncGenWord) + 1u;
  const uint32_t target = epoch_of(gen_next, salt);
  const int K1 = (int)L1.K, H = (int)L1.N;

  // the input row into LDS
  if (tid < 2) xzero[tid] = zero4();
  for (int i = tid; i < K1 / 8; i += kW8Threads)
    *reinterpret_cast<u32x4_t*>(xs + i * 16) = ld16(L1.x + (int64_t)i * 8);
  __syncthreads();

  // layer 1; wave 0's lanes of token 0 (r == 0) hold rows 4g .. 4g + 3 of a tile
  const __amdgpu_buffer_rsrc_t rh = make_rsrc(L1.y, (uint32_t)H * 4u);   // H / 2 words of 8 bytes
  const int64_t tiles1 = (L1.N + 15) / 16, tiles2 = (L2.N + 15) / 16;
  for (int64_t t = blk; t < tiles1; t += G) {
    f32x4_t s0, s1;
    W8Batch<DUAL1, DUAL1 ? 4 : 8> A1;
    const int64_t n = t * 16 + 4 * g;   // H % 16 == 0: all four rows exist
    const W8Rows<DUAL1> R = w8_rows<DUAL1>(L1, n);
    w8_tile_one_token<DUAL1, DUAL1 ? 4 : 8>(L1, t, xs, xz, red, s0, s1, A1);
    if (wave == 0 && r == 0) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (DUAL1) {
          v[i] = apply_act(s0[i] * R.s0[i], L1.act) * (s1[i] * R.s1[i]);
        } else {
          float z = s0[i] * R.s0[i];
          if (L1.bias) z += R.bias(i);
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
    const W8Rows<false> R = w8_rows<false>(L2, t * 16 + 4 * g);
    w8_tile_one_token<false, 8>(L2, t, xs, xz, red, s0, s1, A2);
    if (wave == 0 && r == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t n = t * 16 + 4 * g + i;
        if (n >= L2.N) break;
        float z = s0[i] * R.s0[i];
        if (L2.bias) z += R.bias(i);
        const __bf16 o = (__bf16)z;
        L2.y[n] = __builtin_bit_cast(uint16_t, o);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// The same two-layer forward with the block's waves in two roles, for rows of
// at most 4096 codes in both layers and one layer-1 tile per block.  A wave's
// loads return in the order it issued them, so in the one-role form a layer-2
// request made before the exchange delays the exchange's polls behind it.
// Here waves 4-7 stream the layer-1 tile, publish h and gather it, while
// waves 0-3 hold the block's first layer-2 tile (16 rows over every k) in
// registers, requested once layer 1's weights have landed and turned into
// bf16 operands during the exchange: no poll waits behind a layer-2 load, and
// once h is in LDS layer 2 is only multiplies.  (All 8 waves multiplying
// layer 1, 8 loads each, measured slower: 12.8 against 12.3 us for the 4096^3
// MLP.)  Wave p of a role does the work of waves p and p + 4 of the one-role
// form (their k chunks, in their order, into separate accumulators), and the
// 8 partial tiles are summed in the same order, so the result is bitwise that
// of the one-role form.
// ---------------------------------------------------------------------------
constexpr int kW8SplitMaxK = kW8Waves * 8 * 64;   // one 8-load batch of 8 waves
constexpr int kW8Role = kW8Waves / 2;

template <bool DUAL1>
__global__ __launch_bounds__(kW8Threads) void decode_w8_split_kernel(W8Layer L1, W8Layer L2, uint32_t* sync,
                                                                     uint32_t salt) {
  __shared__ f32x4_t red[2][kW8Waves][64];
  __shared__ __attribute__((aligned(16))) uint8_t xs[2 * kW8SplitMaxK];   // x, then h
  __shared__ u32x4_t xzero[2];   // the activation operand of masked loads
  const uint8_t* xz = reinterpret_cast<const uint8_t*>(xzero);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int G = (int)gridDim.x, blk = (int)blockIdx.x;
  const bool streamer = wave >= kW8Role;   // layer 1 and the exchange; waves below hold layer 2
  const int p = wave & (kW8Role - 1);
  const int K1 = (int)L1.K, H = (int)L1.N, K2 = (int)L2.K;
  const int64_t tiles2 = (L2.N + 15) / 16;
  const bool has2 = blk < tiles2;
  const uint8_t* xl = xs + g * 32;   // the one token's row; lanes of other tokens drop their value
  const bool xrow_ok = r == 0;

  W8Batch<false, 8> P0, P1;   // layer 2: the k chunks of waves p and p + 4
  W8Rows<false> R2;
  // layer 1: the one-role form multiplies 8 loads per wave, or 4 when one
  // gated batch of 4 covers k
  const int j1 = (DUAL1 && (K1 + 63) / 64 <= kW8Waves * 4) ? 4 : 8;
  W8Batch<DUAL1, 8> A0, A1;
  // The generation is read by the streaming waves only, between their weight
  // and activation loads, and its uses are pinned inside their branch: a use
  // on the path the holding waves share would make them wait for their own
  // layer-2 loads (wait counts are merged over both roles' paths).
  uint32_t gen_next = 0, target = 0;
  W8Rows<DUAL1> R1;
  if (streamer) {
    R1 = w8_rows<DUAL1>(L1, (int64_t)blk * 16 + 4 * g);
    const W8Tile t1 = w8_tile_at<DUAL1>(L1, blk);
    w8_issue<DUAL1, 8, 1>(A0, 0, p, g, K1, t1.d0, t1.d1, t1.d0, t1.wrow, 0u);
    w8_issue<DUAL1, 8, 1>(A1, 0, p + kW8Role, g, K1, t1.d0, t1.d1, t1.d0, t1.wrow, 0u);
    gen_next = ld_coherent(sync + kSyncGenWord) + 1u;
    // the input row, all pieces in flight together (pieces past K1 read as
    // zero and land in LDS that is never read as data)
    constexpr int kXPer = 2 * kW8SplitMaxK / 16 / (kW8Role * 64);
    const __amdgpu_buffer_rsrc_t rx = w8_desc(L1.x, (uint32_t)K1 * 2u);
    const int st = tid - kW8Role * 64;
    if (st < 2) xzero[st] = zero4();
    u32x4_t xv[kXPer];
#pragma unroll
    for (int k = 0; k < kXPer; ++k) xv[k] = w8_load(rx, (uint32_t)(st + kW8Role * 64 * k) * 16u);
#pragma unroll
    for (int k = 0; k < kXPer; ++k) *reinterpret_cast<u32x4_t*>(xs + (st + kW8Role * 64 * k) * 16) = xv[k];
    target = epoch_of(gen_next, salt);
    asm volatile("" : "+v"(gen_next), "+v"(target));
  }
  lds_barrier();   // x is in LDS, so layer 1's weights have landed
  // Only now the layer-2 request: made at kernel start it shares the memory
  // with layer 1's and delays layer 1 (and so the exchange) by as much as it
  // gains (15.3 against 13.5 us for the 4096^3 MLP); made here it streams
  // while layer 1 is multiplied and h is exchanged.
  if (!streamer && has2) {
    R2 = w8_rows<false>(L2, (int64_t)blk * 16 + 4 * g);
    const W8Tile t2 = w8_tile_at<false>(L2, blk);
    w8_issue<false, 8, 1>(P0, 0, p, g, K2, t2.d0, t2.d0, t2.d0, t2.wrow, 0u);
    w8_issue<false, 8, 1>(P1, 0, p + kW8Role, g, K2, t2.d0, t2.d0, t2.d0, t2.wrow, 0u);
  }
  if (streamer) {
    f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0, b0 = a0, b1 = a0;
    w8_hold<DUAL1, 8, 1>(A0);
    w8_hold<DUAL1, 8, 1>(A1);
    w8_consume_two<DUAL1>(A0, A1, p, p + kW8Role, g, K1, xrow_ok, xl, xz, a0, a1, b0, b1, j1);
    red[0][p][lane] = a0;
    red[0][p + kW8Role][lane] = b0;
    if constexpr (DUAL1) {
      red[1][p][lane] = a1;
      red[1][p + kW8Role][lane] = b1;
    }
  }
  lds_barrier();
  const __amdgpu_buffer_rsrc_t rh = make_rsrc(L1.y, (uint32_t)H * 4u);   // H / 2 words of 8 bytes
  // wave 4 publishes this block's 16 values of h (splitting the 4 rows of a
  // lane group over waves 4 and 5, one 8-byte word each, measured slower:
  // 12.7 against 12.3 us for the 4096^3 MLP)
  if (wave == kW8Role) {
    f32x4_t s0 = red[0][0][lane];
    f32x4_t s1 = red[DUAL1 ? 1 : 0][0][lane];
#pragma unroll
    for (int w = 1; w < kW8Waves; ++w) {
      s0 += red[0][w][lane];
      if constexpr (DUAL1) s1 += red[1][w][lane];
    }
    if (r == 0) {
      const int64_t n = (int64_t)blk * 16 + 4 * g;   // H % 16 == 0: all four rows exist
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (DUAL1) {
          v[i] = apply_act(s0[i] * R1.s0[i], L1.act) * (s1[i] * R1.s1[i]);
        } else {
          float z = s0[i] * R1.s0[i];
          if (L1.bias) z += R1.bias(i);
          v[i] = apply_act(z, L1.act);
        }
      }
      st_coherent_b128(rh, (uint32_t)n * 4u, u32x4_t{pack_bf16x2(v[0], v[1]), target, pack_bf16x2(v[2], v[3]), target});
    }
  }

  // every block's h into LDS: each streaming wave gathers its own pieces
  // (16-byte pieces of two words, a thread's in flight together) until both
  // words of every piece carry this call's epoch, with no barrier between its
  // polls.  Meanwhile the holding waves turn their layer-2 codes into bf16
  // operands, so that once h is in LDS only the multiplies remain.
  u32x4_t q0[8][2], q1[8][2];   // layer 2's operands: the chunks of waves p and p + 4
  if (streamer) {
    constexpr int kPer = kW8TwoMaxH / 4 / (kW8Role * 64);   // pieces per thread
    const int pieces = H / 4;
    const int st = tid - kW8Role * 64;
    uint32_t pend = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (st + kW8Role * 64 * i < pieces) pend |= 1u << i;
    for (uint32_t spins = 0;; ++spins) {
      u32x4_t v[kPer];
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (pend & (1u << i))
          v[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                 rh, (uint32_t)(st + kW8Role * 64 * i) * 16u, 0, 16 /* sc1 */));
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        if ((pend & (1u << i)) && v[i][1] == target && v[i][3] == target) {
          *reinterpret_cast<u32x2_t*>(xs + (st + kW8Role * 64 * i) * 8) = u32x2_t{v[i][0], v[i][2]};
          pend &= ~(1u << i);
        }
      }
      if (__builtin_amdgcn_ballot_w64(pend != 0) == 0) break;   // wave-uniform
      if (spins >= (1u << 20)) {
        if (lane == 0)
          __hip_atomic_fetch_add(sync + kSyncTimeoutWord, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  } else if (has2) {
    w8_hold<false, 8, 1>(P0);
    w8_hold<false, 8, 1>(P1);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      e4m3x16_to_bf16(P0.w0[j], q0[j][0], q0[j][1]);
      e4m3x16_to_bf16(P1.w0[j], q1[j][0], q1[j][1]);
    }
  }
  lds_barrier();   // h is in LDS: block 0 has seen every block's words
  if (blk == 0 && tid == kW8Role * 64) st_coherent(sync + kSyncGenWord, gen_next);

  // layer 2: the first tile from registers, any further ones streamed by all waves
  if (has2) {
    if (!streamer) {
      // each accumulator sums in the one-role order; consecutive MFMAs are independent
      f32x4_t c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        u32x4_t xa0, xa1, xb0, xb1;
        w8_x<false, 8, 1>(P0, 0, j, p, g, K2, xrow_ok, xl, xz, xa0, xa1);
        w8_x<false, 8, 1>(P1, 0, j, p + kW8Role, g, K2, xrow_ok, xl, xz, xb0, xb1);
        c0 = mfma_16x16x32(q0[j][0], xa0, c0);
        c1 = mfma_16x16x32(q1[j][0], xb0, c1);
        c0 = mfma_16x16x32(q0[j][1], xa1, c0);
        c1 = mfma_16x16x32(q1[j][1], xb1, c1);
      }
      red[0][p][lane] = c0;
      red[0][p + kW8Role][lane] = c1;
    }
    lds_barrier();
    f32x4_t s0 = red[0][0][lane];
    if (wave == 0) {
#pragma unroll
      for (int w = 1; w < kW8Waves; ++w) s0 += red[0][w][lane];
    }
    lds_barrier();   // red is free for the next tile
    if (wave == 0 && r == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t n = (int64_t)blk * 16 + 4 * g + i;
        if (n >= L2.N) break;
        float z = s0[i] * R2.s0[i];
        if (L2.bias) z += R2.bias(i);
        const __bf16 o = (__bf16)z;
        L2.y[n] = __builtin_bit_cast(uint16_t, o);
      }
    }
  }
  for (int64_t t = blk + G; t < tiles2; t += G) {
    f32x4_t s0, s1;
    W8Batch<false, 8> A2;
    const W8Rows<false> R = w8_rows<false>(L2, t * 16 + 4 * g);
    w8_tile_one_token<false, 8>(L2, t, xs, xz, red, s0, s1, A2);
    if (wave == 0 && r == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t n = t * 16 + 4 * g + i;
        if (n >= L2.N) break;
        float z = s0[i] * R.s0[i];
        if (L2.bias) z += R.bias(i);
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
  // the two-role form: one layer-1 tile per block, and both layers' rows read in one batch
  const bool split = tiles1 <= cus && L1.K <= kW8SplitMaxK;
  uint32_t salt = next_launch_salt();
  const void* f;
  if (split)
    f = L1.W1 ? reinterpret_cast<const void*>(&decode_w8_split_kernel<true>)
              : reinterpret_cast<const void*>(&decode_w8_split_kernel<false>);
  else
    f = L1.W1 ? reinterpret_cast<const void*>(&decode_w8_two_kernel<true>)
              : reinterpret_cast<const void*>(&decode_w8_two_kernel<false>);
  W8Layer a = L1, b = L2;
  void* args[] = {&a, &b, &sync, &salt};
  // cooperative (opt-in): the runtime refuses a grid that cannot be resident at once
  if (cooperative) return hipLaunchCooperativeKernel(f, dim3(grid), dim3(kW8Threads), args, 0, s);
  return hipLaunchKernel(f, dim3(grid), dim3(kW8Threads), args, 0, s);
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
