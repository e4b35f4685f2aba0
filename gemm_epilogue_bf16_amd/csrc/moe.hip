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
//            and a scatter, in a single block so the order is fixed; each
//            thread keeps its contiguous run of pairs in registers and the
//            experts are counted four at a time per block scan.
//   combine: y[t] = sum_j ytilde[pos(t, j)] in slot order j = 0, 1, ... in fp32
//            (the gate weight was applied in the down-projection epilogue), then
//            one bf16 rounding.  No atomics: bitwise deterministic.
#include "common.h"
#include "kernels.h"

namespace fmlp {

namespace {

constexpr int kRouteThreads = 512;    // 8 waves
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kRouteCache = 16;       // pairs per thread held in registers
constexpr int kRouteBatch = 4;        // experts counted per block scan

typedef int i32x4v __attribute__((ext_vector_type(4)));

// Exclusive scan of a 4-vector over the block, in thread order: a wave-level
// shuffle scan, then each wave adds the totals of the waves before it.
// Returns the exclusive prefix; *total gets the block total.
__device__ i32x4v block_exclusive_scan4(i32x4v v, i32x4v* wave_tot, i32x4v* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  i32x4v incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    i32x4v up;
#pragma unroll
    for (int c = 0; c < 4; ++c) up[c] = __shfl_up(incl[c], off, 64);
    if (lane >= off) incl += up;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  i32x4v before = {0, 0, 0, 0}, all = {0, 0, 0, 0};
  for (int w = 0; w < kRouteWaves; ++w) {
    const i32x4v t = wave_tot[w];
    if (w < wave) before += t;
    all += t;
  }
  __syncthreads();   // wave_tot is reused by the next scan
  *total = all;
  return before + incl - v;
}

__global__ void __launch_bounds__(kRouteThreads)
moe_route_kernel(const int32_t* __restrict__ ids, const float* __restrict__ gate_w, int64_t P,
                 int top_k, int E, int bm, MoeRouteOut o) {
  __shared__ i32x4v wave_tot[kRouteWaves];
  const int tid = threadIdx.x;
  // thread tid owns the contiguous pairs [p0, p0 + n) (P < 2^31), the first
  // kRouteCache of them in registers
  const int chunk = (int)((P + kRouteThreads - 1) / kRouteThreads);
  const int p0 = (int)min(P, (int64_t)tid * chunk);
  const int n = (int)min((int64_t)chunk, P - p0);
  const int32_t* my_ids = ids + p0;
  const float* my_gw = gate_w + p0;
  int32_t* my_pos = o.pos_of + p0;
  int mine[kRouteCache];
  int bad = 0;
#pragma unroll
  for (int j = 0; j < kRouteCache; ++j) {
    mine[j] = j < n ? my_ids[j] : 0;
    if (j < n && (mine[j] < 0 || mine[j] >= E)) {
      my_pos[j] = -1;
      ++bad;
    }
    if (j >= n) mine[j] = -1;   // never matches an expert
  }
  for (int j = kRouteCache; j < n; ++j) {
    const int e = my_ids[j];
    if (e < 0 || e >= E) {
      my_pos[j] = -1;
      ++bad;
    }
  }

  i32x4v tot;
  (void)block_exclusive_scan4(i32x4v{bad, 0, 0, 0}, wave_tot, &tot);
  if (tid == 0) o.err[0] = tot[0];

  // places pair j (expert e0 + d, d in [0, kRouteBatch)) at the next slot of
  // its expert
  auto place = [&](int j, int d, i32x4v& pos) {
    int at = 0;
#pragma unroll
    for (int c = 0; c < kRouteBatch; ++c)
      if (d == c) at = pos[c]++;
    o.tok_of[at] = (p0 + j) / top_k;
    o.scale_of[at] = my_gw[j];
    my_pos[j] = at;
  };
  int running = 0, running_tiles = 0;
  for (int e0 = 0; e0 < E; e0 += kRouteBatch) {
    const int nb = min(kRouteBatch, E - e0);
    i32x4v cnt = {0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < kRouteCache; ++j) {
      const int d = mine[j] - e0;
#pragma unroll
      for (int c = 0; c < kRouteBatch; ++c) cnt[c] += (d == c && c < nb) ? 1 : 0;
    }
    for (int j = kRouteCache; j < n; ++j) {
      const int d = my_ids[j] - e0;
#pragma unroll
      for (int c = 0; c < kRouteBatch; ++c) cnt[c] += (d == c && c < nb) ? 1 : 0;
    }
    const i32x4v base = block_exclusive_scan4(cnt, wave_tot, &tot);
    i32x4v pos;
    int acc = running;
#pragma unroll
    for (int c = 0; c < kRouteBatch; ++c) {
      pos[c] = acc + base[c];
      acc += tot[c];
    }
#pragma unroll
    for (int j = 0; j < kRouteCache; ++j) {
      const int d = mine[j] - e0;
      if (d >= 0 && d < nb) place(j, d, pos);
    }
    for (int j = kRouteCache; j < n; ++j) {
      const int d = my_ids[j] - e0;
      if (d >= 0 && d < nb) place(j, d, pos);
    }
    for (int c = 0; c < nb; ++c) {
      if (tid == 0) {
        o.group_off[e0 + c] = running;
        o.tile_off[e0 + c] = running_tiles;
      }
      running += tot[c];
      running_tiles += (tot[c] + bm - 1) / bm;
    }
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
