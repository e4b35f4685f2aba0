// Decode path (M <= 16 tokens) for gfx950: weight-streaming GEMV on MFMA.
//
// At batch 1-16 a feed-forward layer is bound by reading its weights once
// from HBM (ainews.cool "PyTorch fused MLP efficiency", section
// "architectural impact": autoregressive decode is memory-bandwidth bound), and
// per-launch overhead matters (section "technical deep dive": the fused form is
// one launch that loads X once and writes only the final output).
//
// Work split.  A block owns 16 output rows (one MFMA row tile) and its NW
// waves split K: wave w walks k-steps of 32 in [w*per, (w+1)*per).  Each lane
// loads 16 contiguous bytes of a weight row per k-step straight into the MFMA
// row operand (v_mfma_f32_16x16x32_bf16: lane l supplies weight row l%16,
// k-group l/16); the <= 16 activation rows are the column operand (zero for
// columns >= M).  A batch of U k-steps is issued before the first MFMA so each
// wave keeps U*16 B per lane in flight.  Partial 16x16 fp32 tiles are summed
// across waves through LDS in a fixed order (bitwise deterministic), then the
// epilogue (bias, activation, or gelu_tanh(g)*u) runs in fp32 and rounds once
// to bf16.
//
// The two-layer forms (mlp2, GeGLU) run as one persistent cooperative launch:
// phase 1 writes the bf16 hidden vector to the workspace, a device-wide barrier
// orders it, and phase 2 streams the second weight.  In the one-tile-per-block
// layout the second layer's weights are requested before the barrier so that
// their HBM stream overlaps phase 1 and the barrier.
#include <algorithm>
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace fmlp {

namespace {

constexpr int kNW = 8;          // waves per block
constexpr int kThreads = kNW * 64;

struct TileCoords {
  int li, lg;                   // lane row-in-tile / k-group
  int64_t s_begin, s_end;       // this wave's k-steps (of 32)
};

__device__ __forceinline__ TileCoords coords(int64_t K) {
  TileCoords c;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  c.li = lane & 15;
  c.lg = lane >> 4;
  const int64_t steps = (K + 31) >> 5;
  const int64_t per = (steps + kNW - 1) / kNW;
  c.s_begin = min(steps, (int64_t)wave * per);
  c.s_end = min(steps, c.s_begin + per);
  return c;
}

// Registers holding one batch of U k-steps for one wave.
template <int U, bool DUAL>
struct Batch {
  u32x4_t w0[U];
  u32x4_t w1[DUAL ? U : 1];
  u32x4_t x[U];
};

template <int U, bool DUAL>
__device__ __forceinline__ void issue_weights(const GemvLayer& L, int64_t n0, const TileCoords& c,
                                              int64_t s0, Batch<U, DUAL>& b) {
  int64_t n = n0 + c.li;
  if (n >= L.N) n = L.N - 1;
  const uint16_t* w0 = L.W0 + n * L.K + 8 * c.lg;
  const uint16_t* w1 = DUAL ? L.W1 + n * L.K + 8 * c.lg : nullptr;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t s = s0 + u;
    const int64_t k = s * 32;
    const bool ok = (s < c.s_end) && (k + 8 * c.lg < L.K);
    b.w0[u] = ok ? ld16(w0 + k) : zero4();
    if constexpr (DUAL) b.w1[u] = ok ? ld16(w1 + k) : zero4();
  }
}

template <int U, bool DUAL>
__device__ __forceinline__ void issue_x(const GemvLayer& L, int M, const TileCoords& c, int64_t s0,
                                        Batch<U, DUAL>& b) {
  const bool row_ok = c.li < M;
  const uint16_t* xp = L.x + (int64_t)(row_ok ? c.li : 0) * L.K + 8 * c.lg;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t s = s0 + u;
    const int64_t k = s * 32;
    const bool ok = row_ok && (s < c.s_end) && (k + 8 * c.lg < L.K);
    b.x[u] = ok ? ld16(xp + k) : zero4();
  }
}

template <int U, bool DUAL>
__device__ __forceinline__ void consume(const Batch<U, DUAL>& b, f32x4_t& a0, f32x4_t& a1) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    a0 = mfma_16x16x32(b.w0[u], b.x[u], a0);
    if constexpr (DUAL) a1 = mfma_16x16x32(b.w1[u], b.x[u], a1);
  }
}

// Fixed-order cross-wave sum and epilogue; wave 0 stores.  red holds
// 2 * kNW * 64 * 4 floats.  Ends with a block barrier so red can be reused.
template <bool DUAL>
__device__ __forceinline__ void reduce_store(const GemvLayer& L, int M, int64_t n0, f32x4_t a0,
                                             f32x4_t a1, float* red) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  float4* r0 = reinterpret_cast<float4*>(red);
  float4* r1 = r0 + kNW * 64;
  r0[wave * 64 + lane] = make_float4(a0[0], a0[1], a0[2], a0[3]);
  if constexpr (DUAL) r1[wave * 64 + lane] = make_float4(a1[0], a1[1], a1[2], a1[3]);
  __syncthreads();
  if (wave == 0) {
    float g[4] = {0.f, 0.f, 0.f, 0.f}, u[4] = {0.f, 0.f, 0.f, 0.f};
    for (int w = 0; w < kNW; ++w) {
      const float4 t = r0[w * 64 + lane];
      g[0] += t.x; g[1] += t.y; g[2] += t.z; g[3] += t.w;
      if constexpr (DUAL) {
        const float4 v = r1[w * 64 + lane];
        u[0] += v.x; u[1] += v.y; u[2] += v.z; u[3] += v.w;
      }
    }
    const int m = lane & 15;
    const int64_t n = n0 + 4 * (lane >> 4);   // 4 consecutive outputs
    if (m < M && n < L.N) {
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (DUAL) {
          v[r] = gelu_tanh(g[r]) * u[r];
        } else {
          float z = g[r];
          if (L.bias) z += bf16_to_f32(L.bias[n + r]);
          v[r] = apply_act(z, L.act);
        }
      }
      uint2 out;
      out.x = pack_bf16x2(v[0], v[1]);
      out.y = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<uint2*>(L.y + (int64_t)m * L.N + n) = out;
    }
  }
  __syncthreads();
}

// One full tile (16 outputs) of one layer, looping over batches of U steps.
template <int U, bool DUAL>
__device__ void gemv_tile(const GemvLayer& L, int M, int64_t n0, float* red) {
  const TileCoords c = coords(L.K);
  f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
  for (int64_t s0 = c.s_begin; s0 < c.s_end; s0 += U) {
    Batch<U, DUAL> b;
    issue_weights<U, DUAL>(L, n0, c, s0, b);
    issue_x<U, DUAL>(L, M, c, s0, b);
    consume<U, DUAL>(b, a0, a1);
  }
  reduce_store<DUAL>(L, M, n0, a0, a1, red);
}

template <int U, bool DUAL>
__global__ void __launch_bounds__(kThreads) gemv_kernel(GemvLayer L, int M) {
  __shared__ float red[2 * kNW * 64 * 4];
  const int64_t tiles = (L.N + 15) / 16;
  for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) gemv_tile<U, DUAL>(L, M, t * 16, red);
}

// ---------------------------------------------------------------------------
// Device-wide barrier for a co-resident (cooperative) grid.
// bar[0] = arrival count, bar[1] = generation, bar[2] = timeout count.
// The last block to arrive resets the count and bumps the generation, so the
// words are left ready for the next barrier or call whatever the grid size.
// The wait is bounded: after ~0.5 s it records a timeout and proceeds, so the
// kernel always exits.
// ---------------------------------------------------------------------------
__device__ void grid_barrier(uint32_t* bar) {
  // every thread publishes its own global writes at device scope
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t gen = __hip_atomic_load(&bar[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t prev = __hip_atomic_fetch_add(&bar[0], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (prev == gridDim.x - 1) {
      __hip_atomic_store(&bar[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(&bar[1], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      uint32_t spins = 0;
      while (__hip_atomic_load(&bar[1], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) == gen) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins > (1u << 24)) {
          __hip_atomic_fetch_add(&bar[2], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
    }
  }
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// Generic persistent two-layer kernel: blocks stride over the tiles of each
// layer; the barrier separates the layers.
template <int U1, bool DUAL1, int U2>
__global__ void __launch_bounds__(kThreads) gemv2_persistent_kernel(GemvLayer L1, GemvLayer L2, int M,
                                                                    uint32_t* bar) {
  __shared__ float red[2 * kNW * 64 * 4];
  const int64_t tiles1 = (L1.N + 15) / 16;
  const int64_t tiles2 = (L2.N + 15) / 16;
  for (int64_t t = blockIdx.x; t < tiles1; t += gridDim.x) gemv_tile<U1, DUAL1>(L1, M, t * 16, red);
  grid_barrier(bar);
  for (int64_t t = blockIdx.x; t < tiles2; t += gridDim.x) gemv_tile<U2, false>(L2, M, t * 16, red);
}

// One-tile-per-block form (grid == tiles of both layers, each wave's K-slice
// fits one batch in both layers).  Straight-line: layer-1 weights and x, then
// layer-2 weights are all requested before the first MFMA, so the whole
// weight stream is in flight while phase 1 computes and the barrier waits.
template <int U1, bool DUAL1, int U2>
__global__ void __launch_bounds__(kThreads) gemv2_onetile_kernel(GemvLayer L1, GemvLayer L2, int M,
                                                                 uint32_t* bar) {
  __shared__ float red[2 * kNW * 64 * 4];
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const TileCoords c1 = coords(L1.K);
  const TileCoords c2 = coords(L2.K);
  Batch<U1, DUAL1> b1;
  Batch<U2, false> b2;
  issue_weights<U1, DUAL1>(L1, n0, c1, c1.s_begin, b1);
  issue_x<U1, DUAL1>(L1, M, c1, c1.s_begin, b1);
  issue_weights<U2, false>(L2, n0, c2, c2.s_begin, b2);   // prefetch, overlaps phase 1
  f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
  consume<U1, DUAL1>(b1, a0, a1);
  reduce_store<DUAL1>(L1, M, n0, a0, a1, red);
  grid_barrier(bar);
  issue_x<U2, false>(L2, M, c2, c2.s_begin, b2);
  a0 = f32x4_t{0.f, 0.f, 0.f, 0.f};
  consume<U2, false>(b2, a0, a1);
  reduce_store<false>(L2, M, n0, a0, a1, red);
}

struct Occ {
  bool probed = false;
  bool ok = false;
  int cus = 0;
  int per_cu_generic[2] = {0, 0};   // [DUAL1]
  int per_cu_onetile[2] = {0, 0};
};

constexpr int kU = 16;       // k-steps per batch, single weight set
constexpr int kUDual = 8;    // k-steps per batch, gate + up

std::mutex g_occ_mu;
Occ g_occ[64];

// Residency limits of the persistent kernels on the current device, queried
// once per device (the runtime's occupancy calculator, then cached).
Occ occ() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return Occ{};
  std::lock_guard<std::mutex> lk(g_occ_mu);
  Occ& o = g_occ[dev];
  if (!o.probed) {
    o.probed = true;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return o;
    o.cus = prop.multiProcessorCount;
    bool ok = true;
    ok &= hipOccupancyMaxActiveBlocksPerMultiprocessor(&o.per_cu_generic[0],
              reinterpret_cast<const void*>(&gemv2_persistent_kernel<kU, false, kU>), kThreads, 0) == hipSuccess;
    ok &= hipOccupancyMaxActiveBlocksPerMultiprocessor(&o.per_cu_generic[1],
              reinterpret_cast<const void*>(&gemv2_persistent_kernel<kUDual, true, kU>), kThreads, 0) == hipSuccess;
    ok &= hipOccupancyMaxActiveBlocksPerMultiprocessor(&o.per_cu_onetile[0],
              reinterpret_cast<const void*>(&gemv2_onetile_kernel<kU, false, kU>), kThreads, 0) == hipSuccess;
    ok &= hipOccupancyMaxActiveBlocksPerMultiprocessor(&o.per_cu_onetile[1],
              reinterpret_cast<const void*>(&gemv2_onetile_kernel<kUDual, true, kU>), kThreads, 0) == hipSuccess;
    o.ok = ok;
  }
  return o;
}

}  // namespace

hipError_t launch_gemv(const GemvLayer& L, int M, hipStream_t s) {
  const int64_t tiles = (L.N + 15) / 16;
  if (tiles <= 0 || M <= 0) return hipSuccess;
  const unsigned grid = (unsigned)std::min<int64_t>(tiles, 1 << 20);
  if (L.geglu)
    hipLaunchKernelGGL((gemv_kernel<kUDual, true>), dim3(grid), dim3(kThreads), 0, s, L, M);
  else
    hipLaunchKernelGGL((gemv_kernel<kU, false>), dim3(grid), dim3(kThreads), 0, s, L, M);
  return hipGetLastError();
}

int gemv2_persistent_max_blocks() {
  const Occ o = occ();
  if (!o.ok) return 0;
  return o.cus * min(o.per_cu_generic[0], o.per_cu_generic[1]);
}

hipError_t launch_gemv2_persistent(const GemvLayer& L1, const GemvLayer& L2, int M, uint32_t* bar,
                                   hipStream_t s) {
  const Occ o = occ();
  if (!o.ok || o.cus <= 0) return hipErrorInvalidDevice;
  const int dual = L1.geglu ? 1 : 0;
  const int64_t tiles1 = (L1.N + 15) / 16, tiles2 = (L2.N + 15) / 16;
  const int64_t steps1 = (L1.K + 31) / 32, steps2 = (L2.K + 31) / 32;
  const int64_t per1 = (steps1 + kNW - 1) / kNW, per2 = (steps2 + kNW - 1) / kNW;
  const int u1 = dual ? kUDual : kU;
  GemvLayer a = L1, b = L2;
  int Mi = M;
  void* args[] = {&a, &b, &Mi, &bar};
  const int64_t one_cap = (int64_t)o.cus * o.per_cu_onetile[dual];
  if (tiles1 == tiles2 && tiles1 <= one_cap && per1 <= u1 && per2 <= kU) {
    const void* fn = dual ? reinterpret_cast<const void*>(&gemv2_onetile_kernel<kUDual, true, kU>)
                          : reinterpret_cast<const void*>(&gemv2_onetile_kernel<kU, false, kU>);
    return hipLaunchCooperativeKernel(fn, dim3((unsigned)tiles1), dim3(kThreads), args, 0, s);
  }
  const int64_t cap = (int64_t)o.cus * o.per_cu_generic[dual];
  if (cap <= 0) return hipErrorInvalidConfiguration;
  const int64_t grid = std::min<int64_t>(cap, std::max(tiles1, tiles2));
  const void* fn = dual ? reinterpret_cast<const void*>(&gemv2_persistent_kernel<kUDual, true, kU>)
                        : reinterpret_cast<const void*>(&gemv2_persistent_kernel<kU, false, kU>);
  return hipLaunchCooperativeKernel(fn, dim3((unsigned)grid), dim3(kThreads), args, 0, s);
}

}  // namespace fmlp
