// Mixture-of-experts helpers for gfx950: route bucketing and weighted combine.
//
// An MoE layer routes each token to several experts, each an MLP, and fusing
// each expert's MLP cuts per-expert overhead (ainews.cool "PyTorch fused MLP
// efficiency", section "architectural impact").  Here the experts are GeGLU
// blocks; the routes (top_k expert ids and gate weights per token) are inputs.
//
//   route:   (token, slot) pairs are bucketed per expert, stable in pair order,
//            giving each expert one contiguous segment of rows; the grouped
//            GEMMs then run every expert over its segment with the token rows
//            gathered on the fly.  Integer work only: counts, an exclusive scan,
//            and a scatter, in a single block so the order is fixed.
//   combine: y[t] = sum_j ytilde[pos(t, j)] in slot order j = 0, 1, ... in fp32
//            (the gate weight was applied in the down-projection epilogue), then
//            one bf16 rounding.  No atomics: bitwise deterministic.
#include "common.h"
#include "kernels.h"

namespace fmlp {

namespace {

constexpr int kRouteThreads = 1024;

__device__ int block_inclusive_scan(int v, int* scan) {
  const int tid = threadIdx.x;
  scan[tid] = v;
  __syncthreads();
  for (int off = 1; off < kRouteThreads; off <<= 1) {
    const int add = (tid >= off) ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += add;
    __syncthreads();
  }
  return scan[tid];
}

__global__ void __launch_bounds__(kRouteThreads)
moe_route_kernel(const int32_t* __restrict__ ids, const float* __restrict__ gate_w, int64_t P,
                 int top_k, int E, int bm, MoeRouteOut o) {
  __shared__ int scan[kRouteThreads];
  const int tid = threadIdx.x;
  const int64_t chunk = (P + kRouteThreads - 1) / kRouteThreads;
  const int64_t p0 = min(P, (int64_t)tid * chunk);
  const int64_t p1 = min(P, p0 + chunk);

  int bad = 0;
  for (int64_t p = p0; p < p1; ++p) {
    const int e = ids[p];
    if (e < 0 || e >= E) {
      o.pos_of[p] = -1;
      ++bad;
    }
  }
  const int bad_total = block_inclusive_scan(bad, scan);
  if (tid == kRouteThreads - 1) o.err[0] = bad_total;
  __syncthreads();

  int running = 0, running_tiles = 0;
  for (int e = 0; e < E; ++e) {
    int cnt = 0;
    for (int64_t p = p0; p < p1; ++p) cnt += (ids[p] == e);
    const int incl = block_inclusive_scan(cnt, scan);
    const int total = scan[kRouteThreads - 1];
    int pos = running + incl - cnt;
    for (int64_t p = p0; p < p1; ++p) {
      if (ids[p] == e) {
        o.tok_of[pos] = (int32_t)(p / top_k);
        o.scale_of[pos] = gate_w[p];
        o.pos_of[p] = pos;
        ++pos;
      }
    }
    if (tid == 0) {
      o.group_off[e] = running;
      o.tile_off[e] = running_tiles;
    }
    running += total;
    running_tiles += (total + bm - 1) / bm;
    __syncthreads();
  }
  if (tid == 0) {
    o.group_off[E] = running;
    o.tile_off[E] = running_tiles;
  }
}

__global__ void __launch_bounds__(256)
moe_combine_kernel(const float* __restrict__ ytilde, const int32_t* __restrict__ pos_of, int64_t T,
                   int top_k, int64_t D, uint16_t* __restrict__ y) {
  const int64_t chunks = D / 8;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T * chunks) return;
  const int64_t t = i / chunks;
  const int64_t d = (i - t * chunks) * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < top_k; ++j) {
    const int pos = pos_of[t * top_k + j];
    if (pos < 0) continue;
    const float* src = ytilde + (int64_t)pos * D + d;
    const u32x4_t lo = ld16(src), hi = ld16(src + 4);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      acc[r] += __uint_as_float(lo[r]);
      acc[4 + r] += __uint_as_float(hi[r]);
    }
  }
  st16(y + t * D + d, pack_bf16x8(acc));
}

}  // namespace

hipError_t launch_moe_route(const int32_t* ids, const float* gate_w, int64_t T, int top_k, int E,
                            int bm, const MoeRouteOut& o, hipStream_t s) {
  hipLaunchKernelGGL(moe_route_kernel, dim3(1), dim3(kRouteThreads), 0, s, ids, gate_w,
                     T * (int64_t)top_k, top_k, E, bm, o);
  return hipGetLastError();
}

hipError_t launch_moe_combine(const float* ytilde, const int32_t* pos_of, int64_t T, int top_k,
                              int64_t D, uint16_t* y, hipStream_t s) {
  const int64_t work = T * (D / 8);
  if (work <= 0) return hipSuccess;
  const int64_t blocks = (work + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)blocks), dim3(256), 0, s, ytilde, pos_of, T,
                     top_k, D, y);
  return hipGetLastError();
}

}  // namespace fmlp
