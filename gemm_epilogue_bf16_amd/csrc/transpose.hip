// Layout helpers of the backward pass, for gfx950.
//
// The backward GEMMs contract over the dimension that is the row index of a
// stored operand: dx = dz . W contracts over W's rows, dW = dz^T . x over the
// token rows of dz and x.  The MFMA GEMM reads both operands K-contiguous
// (the forward's layout, "Profiling in PyTorch (Part 2): From nn.Linear to a
// Fused MLP", section "Where did the transpose go? Kernel layouts and
// pre-ops": a GEMM variant reads each operand in the order it is stored), so
// these operands are first rewritten transposed.  A transpose moves each byte
// once in and once out of HBM; it is bound by HBM bandwidth and costs a few
// percent of the backward's MFMA time at the large shapes.
//
//   transpose_kernel  a 64 x 64 tile per block: 16-byte coalesced loads of the
//                     tile's rows into LDS, then 16-byte coalesced stores of
//                     its columns (8 consecutive rows of one column gathered
//                     from LDS per thread).  Rows past the input's end are
//                     written as zeros up to the requested padded width.
//   rowsum_kernel     one wave per row: 16-byte loads, fp32 partial sums per
//                     lane in a fixed order, then a fixed butterfly across the
//                     wave (deterministic), rounded to bf16 once.
//   sum_parts_kernel  the parts of a weight-gradient GEMM split over the
//                     tokens, added in part order in fp32 and rounded once.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace fmlp {

namespace {

constexpr int kT = 64;          // tile edge
constexpr int kPad = kT + 2;    // LDS row stride in bf16 (breaks the column reads' bank pattern)

__global__ void __launch_bounds__(256) transpose_kernel(const uint16_t* __restrict__ in, int64_t R, int64_t C,
                                                        int64_t ldi, uint16_t* __restrict__ out, int64_t ldo,
                                                        int64_t cols_out, int64_t tiles_r) {
  __shared__ uint16_t tile[kT * kPad];
  const int tid = threadIdx.x;
  const int64_t b = blockIdx.x;
  const int64_t r0 = (b % tiles_r) * kT;   // input rows = output columns
  const int64_t c0 = (b / tiles_r) * kT;   // input columns = output rows
  // load: 64 rows x 8 chunks of 8 bf16
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int q = tid + 256 * h;
    const int row = q >> 3, ch = q & 7;
    const int64_t r = r0 + row, c = c0 + 8 * ch;
    u32x4_t v = zero4();
    if (r < R && c < C) v = ld16(in + r * ldi + c);   // C % 8 == 0: a chunk is all in or all out
    uint16_t* t = &tile[row * kPad + 8 * ch];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      t[2 * e] = (uint16_t)(v[e] & 0xFFFFu);
      t[2 * e + 1] = (uint16_t)(v[e] >> 16);
    }
  }
  __syncthreads();
  // store: output row c0 + cc, columns r0 + 8 j .. + 7
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int q = tid + 256 * h;
    const int cc = q >> 3, j = q & 7;
    const int64_t orow = c0 + cc, ocol = r0 + 8 * j;
    if (orow >= C || ocol >= cols_out) continue;   // cols_out % 8 == 0
    u32x4_t v;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      v[e] = (uint32_t)tile[(8 * j + 2 * e) * kPad + cc] | ((uint32_t)tile[(8 * j + 2 * e + 1) * kPad + cc] << 16);
    st16(out + orow * ldo + ocol, v);
  }
}

__global__ void __launch_bounds__(256) rowsum_kernel(const uint16_t* __restrict__ in, int64_t R, int64_t C,
                                                     int64_t ld, uint16_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= R) return;   // wave-uniform
  const uint16_t* row = in + r * ld;
  float acc = 0.f;
  for (int64_t c = 8 * (int64_t)lane; c < C; c += 512) {   // C % 8 == 0
    float v[8];
    unpack_bf16x8(ld16(row + c), v);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += v[e];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (lane == 0) {
    const __bf16 b = (__bf16)acc;
    out[r] = __builtin_bit_cast(uint16_t, b);
  }
}

__global__ void __launch_bounds__(256) fill_zero_kernel(uint16_t* __restrict__ out, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) out[i] = 0;
}

__global__ void __launch_bounds__(256) sum_parts_kernel(const float* __restrict__ parts, int P, int64_t stride,
                                                        int64_t n, uint16_t* __restrict__ out) {
  for (int64_t i = 8 * ((int64_t)blockIdx.x * 256 + threadIdx.x); i < n; i += 8 * (int64_t)gridDim.x * 256) {
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int p = 0; p < P; ++p) {   // part order
      const float4 a = *reinterpret_cast<const float4*>(parts + p * stride + i);
      const float4 b = *reinterpret_cast<const float4*>(parts + p * stride + i + 4);
      v[0] += a.x; v[1] += a.y; v[2] += a.z; v[3] += a.w;
      v[4] += b.x; v[5] += b.y; v[6] += b.z; v[7] += b.w;
    }
    st16(out + i, pack_bf16x8(v));
  }
}

}  // namespace

hipError_t launch_sum_parts(const float* parts, int P, int64_t stride, int64_t n, uint16_t* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (P < 1 || n % 8 != 0 || stride < n || stride % 4 != 0) return hipErrorInvalidValue;
  const int64_t g = std::min<int64_t>((n / 8 + 255) / 256, 8192);
  hipLaunchKernelGGL(sum_parts_kernel, dim3((unsigned)g), dim3(256), 0, s, parts, P, stride, n, out);
  return hipGetLastError();
}

hipError_t launch_fill_zero(uint16_t* out, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t g = std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)g), dim3(256), 0, s, out, n);
  return hipGetLastError();
}

hipError_t launch_transpose(const uint16_t* in, int64_t R, int64_t C, int64_t ldi, uint16_t* out, int64_t ldo,
                            int64_t cols_out, hipStream_t s) {
  if (R <= 0 || C <= 0) return hipSuccess;
  if (C % 8 != 0 || cols_out % 8 != 0 || cols_out < R || ldo < cols_out || ldi < C) return hipErrorInvalidValue;
  const int64_t tiles_r = (cols_out + kT - 1) / kT, tiles_c = (C + kT - 1) / kT;
  if (tiles_r * tiles_c > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(transpose_kernel, dim3((unsigned)(tiles_r * tiles_c)), dim3(256), 0, s, in, R, C, ldi, out,
                     ldo, cols_out, tiles_r);
  return hipGetLastError();
}

hipError_t launch_rowsum(const uint16_t* in, int64_t R, int64_t C, int64_t ld, uint16_t* out, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  if (C % 8 != 0 || ld < C) return hipErrorInvalidValue;
  const int64_t g = (R + 3) / 4;
  if (g > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rowsum_kernel, dim3((unsigned)g), dim3(256), 0, s, in, R, C, ld, out);
  return hipGetLastError();
}

}  // namespace fmlp
