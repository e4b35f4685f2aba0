// Single-launch two-layer MLP for narrow layers (K, H, N <= 128), gfx950.
//
// The fused form of the two-layer MLP: load X once, compute W1*X+b1, apply the
// activation, compute W2*(.)+b2 and write only the final output, in ONE launch
// instead of three (ainews.cool "PyTorch fused MLP efficiency", section
// "technical deep dive").  The narrow shape is the page's profiled Linear
// 32 -> 64 at batch 1024 ("Profiling in PyTorch (Part 2)", section "From
// matmul-add to Linear"), stacked into 32 -> 64 -> 32.
//
// A block stages W1, W2 (bf16) and the biases (fp32) in LDS; each of its 4
// waves owns 16 token rows.  Layer 1 runs on v_mfma_f32_16x16x32_bf16 with the
// weight as the row operand and x (read straight from HBM) as the column
// operand; bias + activation run on the fp32 accumulator; h is rounded to bf16
// once and parked in the wave's LDS slice, re-read as the column operand of
// layer 2.  h never leaves the chip.
#include "common.h"
#include "kernels.h"

namespace fmlp {

namespace {

constexpr int kMaxDim = 128;
constexpr int kPad = 8;                         // bf16 padding per LDS row
constexpr int kStride = kMaxDim + kPad;         // LDS row stride (elements)
// 16 token rows per wave; 8 waves share one staging of the weights (1024 x
// 32 -> 64 -> 32: 5.7 us per forward against 6.0 with 4 waves, 6.5 with 2 or
// 16, 7.7 with 1)
constexpr int kWaves = 8;

// One kernel per activation: a runtime choice inlined at every output element
// made the kernel 25 KB of code against 10 KB with the tanh GELU alone, and a
// launch this short starts with its instructions out of cache (measured 6.8
// against 6.0 us per forward at 1024 x 32 -> 64 -> 32; requesting every load
// of the block before the first wait instead, at twice the code, was slower).
template <int ACT>
__global__ void __launch_bounds__(kWaves * 64)
small_mlp2_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ W1,
                  const uint16_t* __restrict__ b1, const uint16_t* __restrict__ W2,
                  const uint16_t* __restrict__ b2, int64_t M, int K, int H, int N,
                  uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint16_t sW1[kMaxDim * kStride];   // [H][K]
  __shared__ __attribute__((aligned(16))) uint16_t sW2[kMaxDim * kStride];   // [N][H]
  __shared__ __attribute__((aligned(16))) uint16_t sH[kWaves][16 * kStride]; // per wave [16][H]
  __shared__ float sb1[kMaxDim], sb2[kMaxDim];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;

  const int KP = (K + 31) & ~31;   // padded to whole k-steps
  const int HP = (H + 31) & ~31;
  const int NP = (N + 15) & ~15;

  // ---- stage weights (zero padding) and biases ----------------------------
  for (int q = tid; q < HP * (KP / 8); q += kWaves * 64) {
    const int r = q / (KP / 8), c = (q % (KP / 8)) * 8;
    const u32x4_t v = (r < H && c < K) ? ld16(W1 + (int64_t)r * K + c) : zero4();
    st16(&sW1[r * kStride + c], v);
  }
  for (int q = tid; q < NP * (HP / 8); q += kWaves * 64) {
    const int r = q / (HP / 8), c = (q % (HP / 8)) * 8;
    const u32x4_t v = (r < N && c < H) ? ld16(W2 + (int64_t)r * H + c) : zero4();
    st16(&sW2[r * kStride + c], v);
  }
  for (int i = tid; i < kMaxDim; i += kWaves * 64) {
    sb1[i] = (b1 && i < H) ? bf16_to_f32(b1[i]) : 0.f;
    sb2[i] = (b2 && i < N) ? bf16_to_f32(b2[i]) : 0.f;
  }
  __syncthreads();

  const int64_t m0 = (int64_t)blockIdx.x * (kWaves * 16) + wave * 16;
  const int64_t xm = m0 + li;
  const bool row_ok = xm < M;

  // ---- layer 1: h^T[H, 16] = W1 . x^T ---------------------------------------
  f32x4_t hacc[kMaxDim / 16];
#pragma unroll
  for (int f = 0; f < kMaxDim / 16; ++f) hacc[f] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < KP; k0 += 32) {
    const int k = k0 + 8 * lg;
    const u32x4_t xf = (row_ok && k < K) ? ld16(x + xm * K + k) : zero4();
#pragma unroll
    for (int f = 0; f < kMaxDim / 16; ++f) {
      if (f * 16 < HP) {
        const u32x4_t wf = ld16(&sW1[(f * 16 + li) * kStride + k]);
        hacc[f] = mfma_16x16x32(wf, xf, hacc[f]);
      }
    }
  }
  // bias + activation, round to bf16, park in LDS as h[m][hidden]
#pragma unroll
  for (int f = 0; f < kMaxDim / 16; ++f) {
    if (f * 16 < HP) {
      const int hb = f * 16 + 4 * lg;
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = (hb + r < H) ? act_of<ACT>(hacc[f][r] + sb1[hb + r]) : 0.f;
      uint2 pk;
      pk.x = pack_bf16x2(v[0], v[1]);
      pk.y = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<uint2*>(&sH[wave][li * kStride + hb]) = pk;
    }
  }
  __syncthreads();

  // ---- layer 2: y^T[N, 16] = W2 . h^T ---------------------------------------
  f32x4_t yacc[kMaxDim / 16];
#pragma unroll
  for (int f = 0; f < kMaxDim / 16; ++f) yacc[f] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < HP; k0 += 32) {
    const int k = k0 + 8 * lg;
    const u32x4_t hf = ld16(&sH[wave][li * kStride + k]);
#pragma unroll
    for (int f = 0; f < kMaxDim / 16; ++f) {
      if (f * 16 < NP) {
        const u32x4_t wf = ld16(&sW2[(f * 16 + li) * kStride + k]);
        yacc[f] = mfma_16x16x32(wf, hf, yacc[f]);
      }
    }
  }
  if (!row_ok) return;
#pragma unroll
  for (int f = 0; f < kMaxDim / 16; ++f) {
    const int nb = f * 16 + 4 * lg;
    if (f * 16 < NP && nb < N) {
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = yacc[f][r] + sb2[nb + r];
      uint2 pk;
      pk.x = pack_bf16x2(v[0], v[1]);
      pk.y = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<uint2*>(y + xm * N + nb) = pk;
    }
  }
}

}  // namespace

hipError_t launch_small_mlp2(const uint16_t* x, const uint16_t* W1, const uint16_t* b1,
                             const uint16_t* W2, const uint16_t* b2, int act, int64_t M, int K,
                             int H, int N, uint16_t* y, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (K > kMaxDim || H > kMaxDim || N > kMaxDim) return hipErrorInvalidValue;
  const int64_t blocks = (M + kWaves * 16 - 1) / (kWaves * 16);
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 g((unsigned)blocks), b(kWaves * 64);
  switch (act) {
    case ACT_GELU_ERF:
      hipLaunchKernelGGL(small_mlp2_kernel<ACT_GELU_ERF>, g, b, 0, s, x, W1, b1, W2, b2, M, K, H, N, y);
      break;
    case ACT_GELU_TANH:
      hipLaunchKernelGGL(small_mlp2_kernel<ACT_GELU_TANH>, g, b, 0, s, x, W1, b1, W2, b2, M, K, H, N, y);
      break;
    case ACT_RELU:
      hipLaunchKernelGGL(small_mlp2_kernel<ACT_RELU>, g, b, 0, s, x, W1, b1, W2, b2, M, K, H, N, y);
      break;
    case ACT_SILU:
      hipLaunchKernelGGL(small_mlp2_kernel<ACT_SILU>, g, b, 0, s, x, W1, b1, W2, b2, M, K, H, N, y);
      break;
    case ACT_NONE:
      hipLaunchKernelGGL(small_mlp2_kernel<ACT_NONE>, g, b, 0, s, x, W1, b1, W2, b2, M, K, H, N, y);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fmlp
