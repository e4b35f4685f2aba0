// Device helpers shared by the gfx950 kernels: bf16 <-> fp32, the activation
// epilogues, the bf16 MFMA wrapper and the XCD-aware tile order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fmlp {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

enum Act : int { ACT_NONE = 0, ACT_GELU_ERF = 1, ACT_GELU_TANH = 2, ACT_RELU = 3, ACT_SILU = 4 };
constexpr int kActCount = 5;

// ---------------------------------------------------------------------------
// bf16
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t two) { return __uint_as_float(two << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t two) { return __uint_as_float(two & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even (the hardware conversion on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo;
  __bf16 b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ __forceinline__ u32x4_t pack_bf16x8(const float v[8]) {
  u32x4_t r;
  r[0] = pack_bf16x2(v[0], v[1]);
  r[1] = pack_bf16x2(v[2], v[3]);
  r[2] = pack_bf16x2(v[4], v[5]);
  r[3] = pack_bf16x2(v[6], v[7]);
  return r;
}

__device__ __forceinline__ void unpack_bf16x8(const u32x4_t& p, float v[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_lo(p[i]);
    v[2 * i + 1] = bf16_hi(p[i]);
  }
}

// ---------------------------------------------------------------------------
// GELU epilogues, evaluated on the fp32 accumulator.
// Exact:  z * Phi(z) = z/2 * erfc(-z / sqrt 2)   (erfc keeps the negative tail
//         accurate where 1 + erf would cancel).
// Tanh:   z/2 * (1 + tanh(a)), a = sqrt(2/pi) (z + 0.044715 z^3), evaluated as
//         z * sigmoid(2a) = z / (1 + exp(-2a)), the same function without the
//         cancellation of 1 + tanh(a) for a << 0.  exp(-2a) = 2^(-2a log2 e)
//         and the reciprocal use the hardware's exp2 and reciprocal (each
//         within about 1 ulp of fp32): a few relative 1e-7 against the exact
//         value, far below the bf16 output's 2^-8, at a fraction of the cost
//         of a correctly rounded exp and divide (it is evaluated once per
//         output element in the GEMM epilogue).  Limits: z -> +inf gives z,
//         z -> -inf gives -0 (through 2^+inf = inf).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float gelu_erf(float z) {
  return 0.5f * z * erfcf(-0.70710678118654752440f * z);
}

__device__ __forceinline__ float gelu_tanh(float z) {
  const float a = 0.79788456080286535588f * fmaf(0.044715f * z, z * z, z);
  const float e = __builtin_amdgcn_exp2f(-2.88539008177792681472f * a);   // exp(-2a)
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}

// ReLU: max(z, 0) (the two-layer MLP of ainews.cool "PyTorch fused MLP
// efficiency", section "technical deep dive").
__device__ __forceinline__ float relu(float z) { return z > 0.f ? z : 0.f; }

// SiLU (swish): z * sigmoid(z) = z / (1 + exp(-z)), with the same hardware
// exp2 and reciprocal as the tanh GELU above (a few relative 1e-7).  Limits:
// z -> +inf gives z, z -> -inf gives -0.
__device__ __forceinline__ float silu(float z) {
  const float e = __builtin_amdgcn_exp2f(-1.44269504088896340736f * z);   // exp(-z)
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}

template <int ACT>
__device__ __forceinline__ float act_of(float z) {
  if constexpr (ACT == ACT_GELU_ERF) return gelu_erf(z);
  else if constexpr (ACT == ACT_GELU_TANH) return gelu_tanh(z);
  else if constexpr (ACT == ACT_RELU) return relu(z);
  else if constexpr (ACT == ACT_SILU) return silu(z);
  else return z;
}

// ---------------------------------------------------------------------------
// Backward epilogues: each activation and its derivative at z, from the same
// formulas (and the same hardware exp2 / reciprocal) as the forward ones.
//   gelu_erf   a = z Phi(z),        a' = Phi(z) + z phi(z)
//   gelu_tanh  a = z s, s = sigmoid(2u), u = sqrt(2/pi)(z + 0.044715 z^3),
//              a' = s + 2 z s (1 - s) sqrt(2/pi)(1 + 3*0.044715 z^2)
//              ((1 + tanh u)/2 = s and (1 - tanh^2 u)/2 = 2 s (1 - s))
//   relu       a = max(z, 0),       a' = 1 for z > 0, else 0
//   silu       a = z s, s = sigmoid(z), a' = s (1 + z (1 - s))
// In the far tails exp2 saturates to inf or 0 and s to 0 or 1, which gives
// the limits a' -> 0 and a' -> 1 with no NaN.
// ---------------------------------------------------------------------------
template <int ACT>
__device__ __forceinline__ void act_and_grad(float z, float& a, float& da) {
  if constexpr (ACT == ACT_GELU_ERF) {
    const float Phi = 0.5f * erfcf(-0.70710678118654752440f * z);
    const float phi = 0.39894228040143267794f * __builtin_amdgcn_exp2f(-0.72134752044448170368f * z * z);
    a = z * Phi;
    da = fmaf(z, phi, Phi);
  } else if constexpr (ACT == ACT_GELU_TANH) {
    const float k = 0.79788456080286535588f;
    const float u = k * fmaf(0.044715f * z, z * z, z);
    const float s = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-2.88539008177792681472f * u));
    a = z * s;
    da = fmaf(2.0f * z * s * (1.0f - s), k * fmaf(0.134145f * z, z, 1.0f), s);
  } else if constexpr (ACT == ACT_RELU) {
    a = z > 0.f ? z : 0.f;
    da = z > 0.f ? 1.f : 0.f;
  } else if constexpr (ACT == ACT_SILU) {
    const float s = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.44269504088896340736f * z));
    a = z * s;
    da = s * fmaf(z, 1.0f - s, 1.0f);
  } else {
    a = z;
    da = 1.f;
  }
}

__device__ __forceinline__ float apply_act(float z, int act) {
  if (act == ACT_GELU_ERF) return gelu_erf(z);
  if (act == ACT_GELU_TANH) return gelu_tanh(z);
  if (act == ACT_RELU) return relu(z);
  if (act == ACT_SILU) return silu(z);
  return z;
}

// ---------------------------------------------------------------------------
// MFMA: D[16x16] += A[16x32] * B[32x16], bf16 inputs, fp32 accumulate.
// Lane l supplies row (l % 16) of A and column (l % 16) of B, each as 8
// consecutive k values of k-group (l / 16); it receives D rows 4*(l/16)+r,
// r = 0..3, of column (l % 16).
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4_t mfma_16x16x32(const u32x4_t& a, const u32x4_t& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4_t zero4() {
  u32x4_t z;
  z[0] = z[1] = z[2] = z[3] = 0u;
  return z;
}

__device__ __forceinline__ u32x4_t ld16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }
__device__ __forceinline__ void st16(void* p, const u32x4_t& v) { *reinterpret_cast<u32x4_t*>(p) = v; }

// ---------------------------------------------------------------------------
// Workgroups are handed to the 8 XCDs round-robin (block b runs on XCD b % 8),
// and each XCD has its own L2.  xcd_remap() renumbers blocks so that each XCD
// receives one contiguous range of logical tile ids; neighbouring tiles (which
// share A rows or B columns) then share an L2.  Bijective for any count.
// ---------------------------------------------------------------------------
constexpr int kNumXcd = 8;

__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int q = nblocks / kNumXcd, r = nblocks % kNumXcd;
  const int xcd = bid % kNumXcd, idx = bid / kNumXcd;
  return (xcd < r) ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

// Grouped tile order: walk GROUP_M tile-rows down one tile-column, then move to
// the next column, so a group of consecutive tiles reuses the same B columns
// and GROUP_M A row-blocks.
__device__ __forceinline__ void grouped_tile(int t, int tiles_m, int tiles_n, int group_m,
                                             int& tm, int& tn) {
  const int per_group = group_m * tiles_n;
  const int g = t / per_group;
  const int first_m = g * group_m;
  const int gm = min(tiles_m - first_m, group_m);
  const int in = t - g * per_group;
  tm = first_m + in % gm;
  tn = in / gm;
}

}  // namespace fmlp
