// Mixture-of-experts helpers for gfx950: route bucketing and weighted combine.
//
// An MoE layer routes each token to several experts, each an MLP, and fusing
// each expert's MLP cuts per-expert overhead (ainews.cool "PyTorch fused MLP
// efficiency", section "architectural impact").  Here the experts are gated
// blocks (GeGLU, SwiGLU, ...); the routes (top_k expert ids and gate weights
// per token) are inputs, or come from the router at the end of this file.
//
//   route:   (token, slot) pairs are bucketed per expert, stable in pair order,
//            giving each expert one contiguous segment of rows; the grouped
//            GEMMs then run every expert over its segment with the token rows
//            gathered on the fly.  Integer work only, in three launches over
//            blocks of 512 pairs: per-block expert counts, their exclusive
//            scans (over the blocks per expert, then over the experts), and the
//            scatter, each pair ranked within its block by wave ballots.  The
//            place of every pair is fixed by pair order alone.
//   combine: y[t] = sum_j ytilde[pos(t, j)] in slot order j = 0, 1, ... in fp32
//            (the gate weight was applied in the down-projection epilogue; with
//            the down projection split over K, the parts of each row are added
//            in order), then one bf16 rounding.  No atomics: bitwise
//            deterministic.
//   router:  the routes computed on the device: logits = x . Wr^T (fp32), the
//            top_k experts by logit (a tie goes to the lower expert id), and
//            gate weights = softmax over the chosen logits.  Bound by reading x
//            once.  Up to 16 experts the logits are a 16 x 16 x 32 MFMA
//            contraction: a block takes 16 tokens, its 8 waves split D and
//            their partial tiles are summed in a fixed order.  Past 16 experts
//            a VALU form: the router weights in LDS when they fit
//            (E * D * 2 <= 64 KB), else read through the caches.
#include "common.h"
#include "kernels.h"
#include "lds_dma.h"

namespace fmlp {

namespace {

constexpr int kRouteThreads = kMoeRoutePairsPerBlock;   // one pair per thread
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kRouteScanThreads = 1024;

// count: the per-expert histogram of this block's pairs (invalid ids in column
// E), written as row blockIdx.x of cnt [G][E+1].
__global__ void __launch_bounds__(kRouteThreads)
moe_route_count_kernel(const int32_t* __restrict__ ids, int64_t P, int E, int32_t* __restrict__ cnt) {
  __shared__ int hist[kMoeRouteMaxExperts + 1];
  const int tid = threadIdx.x;
  for (int e = tid; e <= E; e += kRouteThreads) hist[e] = 0;
  __syncthreads();
  const int64_t p = (int64_t)blockIdx.x * kRouteThreads + tid;
  if (p < P) {
    const int e = ids[p];
    atomicAdd(&hist[(e < 0 || e >= E) ? E : e], 1);
  }
  __syncthreads();
  int32_t* row = cnt + (int64_t)blockIdx.x * (E + 1);
  for (int e = tid; e <= E; e += kRouteThreads) row[e] = hist[e];
}

// scan: each column of cnt becomes the exclusive prefix over the blocks (the
// first place, within its expert's segment, of each block's pairs); then the
// expert totals give group_off and tile_off (exclusive scans over the
// experts), and column E the invalid-id total.
__global__ void __launch_bounds__(kRouteScanThreads)
moe_route_scan_kernel(int32_t* __restrict__ cnt, int G, int E, int bm, MoeRouteOut o) {
  __shared__ int tot[kMoeRouteMaxExperts + 1];
  const int tid = threadIdx.x;
  constexpr int U = 16;   // blocks whose counts are requested together
  for (int e = tid; e <= E; e += kRouteScanThreads) {
    int run = 0;
    for (int b0 = 0; b0 < G; b0 += U) {
      int v[U];
#pragma unroll
      for (int j = 0; j < U; ++j) v[j] = b0 + j < G ? cnt[(int64_t)(b0 + j) * (E + 1) + e] : 0;
#pragma unroll
      for (int j = 0; j < U; ++j) {
        if (b0 + j < G) {
          cnt[(int64_t)(b0 + j) * (E + 1) + e] = run;
          run += v[j];
        }
      }
    }
    tot[e] = run;
  }
  __syncthreads();
  if (tid >= 64) return;
  // wave 0: the experts 64 at a time, a shuffle scan of counts and tiles each
  const int lane = tid;
  int base = 0, tbase = 0;
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int e = e0 + lane;
    const int c = e < E ? tot[e] : 0;
    const int t = (c + bm - 1) / bm;
    int ic = c, it = t;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int uc = __shfl_up(ic, off, 64), ut = __shfl_up(it, off, 64);
      if (lane >= off) {
        ic += uc;
        it += ut;
      }
    }
    if (e < E) {
      o.group_off[e] = base + ic - c;
      o.tile_off[e] = tbase + it - t;
    }
    base += __shfl(ic, 63, 64);
    tbase += __shfl(it, 63, 64);
  }
  if (lane == 0) {
    o.group_off[E] = base;
    o.tile_off[E] = tbase;
    o.err[0] = tot[E];
  }
}

// place: pair p of expert e goes to group_off[e] + (its block's first place
// in e) + (pairs of e in earlier waves of the block) + (pairs of e in earlier
// lanes of its wave), which keeps pair order within every expert.  A wave
// ranks its lanes one expert at a time: the lowest unranked lane names the
// expert, a ballot finds every lane with it.
__global__ void __launch_bounds__(kRouteThreads)
moe_route_place_kernel(const int32_t* __restrict__ ids, const float* __restrict__ gate_w, int64_t P, int top_k,
                       int E, const int32_t* __restrict__ cnt, MoeRouteOut o) {
  __shared__ int wcnt[kRouteWaves * kMoeRouteMaxExperts];   // [wave][expert]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t p = (int64_t)blockIdx.x * kRouteThreads + tid;
  const bool have = p < P;
  const int e = have ? ids[p] : -1;
  const float w = have ? gate_w[p] : 0.f;
  const bool valid = have && e >= 0 && e < E;
  for (int i = tid; i < kRouteWaves * E; i += kRouteThreads) wcnt[i] = 0;
  __syncthreads();
  const uint64_t below = lane == 0 ? 0ull : ~0ull >> (64 - lane);   // the lanes before this one
  int rank = 0;
  uint64_t pending = __builtin_amdgcn_ballot_w64(valid);
  while (pending != 0) {   // wave-uniform
    const int leader = __builtin_ctzll(pending);
    const int ec = __shfl(e, leader, 64);
    const bool mine = valid && e == ec;
    const uint64_t same = __builtin_amdgcn_ballot_w64(mine);
    if (mine) rank = __popcll(same & below);
    if (lane == leader) wcnt[wave * E + ec] = __popcll(same);
    pending &= ~same;
  }
  __syncthreads();
  if (valid) {
    int at = o.group_off[e] + cnt[(int64_t)blockIdx.x * (E + 1) + e] + rank;
    for (int v = 0; v < wave; ++v) at += wcnt[v * E + e];
    o.tok_of[at] = (int32_t)(p / top_k);
    o.scale_of[at] = w;
    o.pos_of[p] = at;
  } else if (have) {
    o.pos_of[p] = -1;
  }
}

__global__ void __launch_bounds__(256)
moe_combine_kernel(const float* __restrict__ ytilde, const int32_t* __restrict__ pos_of, int64_t T,
                   int top_k, int64_t D, int ksplit, int64_t kstride, uint16_t* __restrict__ y) {
  const int64_t chunks = D / 8;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T * chunks) return;
  const int64_t t = i / chunks;
  const int64_t d = (i - t * chunks) * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < top_k; ++j) {
    const int pos = pos_of[t * top_k + j];
    if (pos < 0) continue;
    for (int kp = 0; kp < ksplit; ++kp) {   // the split-K parts of the down projection, in order
      const float* src = ytilde + kp * kstride + (int64_t)pos * D + d;
      const u32x4_t lo = ld16(src), hi = ld16(src + 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        acc[r] += __uint_as_float(lo[r]);
        acc[4 + r] += __uint_as_float(hi[r]);
      }
    }
  }
  st16(y + t * D + d, pack_bf16x8(acc));
}

}  // namespace

// ---------------------------------------------------------------------------
// router
// ---------------------------------------------------------------------------
namespace {

constexpr int kRouterThreads = 256;   // 4 waves, each its own tokens

// acc + the dot product of two runs of 8 bf16 (exact fp32 products, fused
// multiply-adds in a fixed order)
__device__ __forceinline__ float dot8_bf16(const u32x4_t& a, const u32x4_t& b, float acc) {
  float av[8], bv[8];
  unpack_bf16x8(a, av);
  unpack_bf16x8(b, bv);
#pragma unroll
  for (int q = 0; q < 8; ++q) acc = fmaf(av[q], bv[q], acc);
  return acc;
}

// top_k of one token's logits by selection (the largest remaining logit, the
// lower id on a tie), then softmax over the chosen ones (sel[0] is their max).
template <int EC>
__device__ __forceinline__ void router_select(const float (&lg)[EC], int E, int top_k, int32_t* ids,
                                              float* gate_w) {
  uint64_t taken = 0;
  float sel[8];
  int id[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (k >= top_k) break;
    float best = 0.f;
    int bi = -1;
#pragma unroll
    for (int e = 0; e < EC; ++e) {
      if (e < E && !((taken >> e) & 1ull) && (bi < 0 || lg[e] > best)) {
        best = lg[e];
        bi = e;
      }
    }
    taken |= 1ull << bi;
    sel[k] = best;
    id[k] = bi;
  }
  float sum = 0.f, ex[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (k >= top_k) break;
    ex[k] = expf(sel[k] - sel[0]);
    sum += ex[k];
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (k >= top_k) break;
    ids[k] = id[k];
    gate_w[k] = ex[k] / sum;
  }
}

// EC: expert capacity (E <= EC); TW: tokens per wave.  Lane l owns the 16-byte
// chunks l, l + 64, ... of a row; its partial dot products are summed in that
// order and then over the wave by a butterfly, the same for every token.
template <int EC, int TW>
__global__ void __launch_bounds__(kRouterThreads)
moe_router_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ Wr, int64_t T, int D, int E,
                  int top_k, int32_t* __restrict__ ids, float* __restrict__ gate_w, float* __restrict__ logits) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t t0 = ((int64_t)blockIdx.x * (kRouterThreads / 64) + wave) * TW;
  if (t0 >= T) return;
  const int nch = D / 8;   // 16-byte chunks per row
  float acc[TW][EC];
#pragma unroll
  for (int j = 0; j < TW; ++j)
#pragma unroll
    for (int e = 0; e < EC; ++e) acc[j][e] = 0.f;
  for (int c = lane; c < nch; c += 64) {
    u32x4_t xv[TW];
#pragma unroll
    for (int j = 0; j < TW; ++j) {
      xv[j] = zero4();
      if (t0 + j < T) xv[j] = ld16(x + (t0 + j) * (int64_t)D + (int64_t)c * 8);
    }
#pragma unroll
    for (int e = 0; e < EC; ++e) {
      if (e < E) {
        const u32x4_t w = ld16(Wr + (int64_t)e * D + (int64_t)c * 8);
#pragma unroll
        for (int j = 0; j < TW; ++j) acc[j][e] = dot8_bf16(xv[j], w, acc[j][e]);
      }
    }
  }
  // butterfly over the wave: every lane ends with every total
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
    for (int j = 0; j < TW; ++j)
#pragma unroll
      for (int e = 0; e < EC; ++e) acc[j][e] += __shfl_xor(acc[j][e], off, 64);
#pragma unroll
  for (int j = 0; j < TW; ++j) {
    const int64_t t = t0 + j;
    if (t >= T) break;
    if (logits != nullptr) {
#pragma unroll
      for (int e = 0; e < EC; ++e)
        if (e < E && lane == (e & 63)) logits[t * E + e] = acc[j][e];
    }
    if (lane == 0) router_select<EC>(acc[j], E, top_k, ids + t * top_k, gate_w + t * top_k);
  }
}

// Up to 16 experts: logits on the matrix cores.  D[e][t] = sum_k Wr[e][k] x[t][k]
// with the router weights as the row operand (experts past E read as zero)
// and 16 tokens as the column operand.  Wave w takes the 32-k steps w, w + 8,
// ...; the 8 partial tiles go through LDS and wave 0 sums them in wave order.
// U k steps of a wave have their loads in flight together: 16 when the grid
// has at most one block per CU (about 200 VGPRs, so one 8-wave block fits a
// CU), 8 otherwise (about 100 VGPRs, two blocks per CU).  U changes only how
// many loads are issued before the MFMAs, not the order of the sums.
constexpr int kRouterMfmaWaves = 8;

template <int U>
__global__ void __launch_bounds__(kRouterMfmaWaves * 64)
moe_router_mfma_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ Wr, int64_t T, int D, int E,
                       int top_k, int32_t* __restrict__ ids, float* __restrict__ gate_w,
                       float* __restrict__ logits) {
  __shared__ float4 red[kRouterMfmaWaves][64];
  __shared__ float lg[16][17];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * 16;
  const int li = lane & 15, kq = lane >> 4;
  const bool row_ok = li < E;              // this lane's expert exists
  const bool col_ok = t0 + li < T;         // this lane's token exists
  const uint16_t* wrow = Wr + (int64_t)(row_ok ? li : 0) * D;
  const uint16_t* xrow = x + (col_ok ? t0 + li : 0) * (int64_t)D;
  const int steps = (D + 31) / 32;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = wave; s0 < steps; s0 += kRouterMfmaWaves * U) {
    u32x4_t a[U], b[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + kRouterMfmaWaves * u;
      const int k = s * 32 + kq * 8;
      const bool in = s < steps && k < D;
      a[u] = (in && row_ok) ? ld16(wrow + k) : zero4();
      b[u] = (in && col_ok) ? ld16(xrow + k) : zero4();
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc = mfma_16x16x32(a[u], b[u], acc);
  }
  red[wave][lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  __syncthreads();
  if (wave != 0) return;
  float sum[4] = {0.f, 0.f, 0.f, 0.f};
  for (int w = 0; w < kRouterMfmaWaves; ++w) {
    const float4 v = red[w][lane];
    sum[0] += v.x; sum[1] += v.y; sum[2] += v.z; sum[3] += v.w;
  }
  // lane holds D[4 * kq + r][li]: expert 4 * kq + r, token li
#pragma unroll
  for (int r = 0; r < 4; ++r) lg[li][4 * kq + r] = sum[r];
  __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0): this wave's LDS writes are done
  __builtin_amdgcn_wave_barrier();
  if (lane < 16 && t0 + lane < T) {
    const int64_t t = t0 + lane;
    float v[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = lg[lane][e];
    if (logits != nullptr)
      for (int e = 0; e < E; ++e) logits[t * E + e] = v[e];
    router_select<16>(v, E, top_k, ids + t * top_k, gate_w + t * top_k);
  }
}

// The same with Wr staged in LDS (E * D * 2 <= kRouterLdsBytes).
constexpr int kRouterLdsThreads = 512;          // 8 waves
constexpr int kRouterLdsBytes = 64 * 1024;

template <int EC, int TW>
__global__ void __launch_bounds__(kRouterLdsThreads)
moe_router_lds_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ Wr, int64_t T, int D, int E,
                      int top_k, int32_t* __restrict__ ids, float* __restrict__ gate_w,
                      float* __restrict__ logits) {
  __shared__ u32x4_t wlds[kRouterLdsBytes / 16];
  const int nch = D / 8;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  {
    // Wr into LDS by loads that write LDS, 1 KB each (lanes past the end
    // masked off), all in flight before one wait
    const int nchunks = E * nch;
    const i32x4_t wd = make_desc(reinterpret_cast<uint64_t>(Wr), (uint32_t)nchunks * 16u);
    const uint32_t wl = lds_addr(&wlds[0]);
    for (int j = wave; j < (nchunks + 63) / 64; j += kRouterLdsThreads / 64) {   // wave-uniform
      const int c = 64 * j + lane;
      if (c < nchunks) asm_load_lds(wd, uniform32(wl + 1024u * (uint32_t)j), (uint32_t)c * 16u);
    }
    wait_vm<0>();
    __syncthreads();
  }
  const int64_t t0 = ((int64_t)blockIdx.x * (kRouterLdsThreads / 64) + wave) * TW;
  if (t0 >= T) return;
  float acc[TW][EC];
#pragma unroll
  for (int j = 0; j < TW; ++j)
#pragma unroll
    for (int e = 0; e < EC; ++e) acc[j][e] = 0.f;
  constexpr int U = 4;   // chunk steps whose x loads are in flight together
  for (int c0 = lane; c0 < nch; c0 += 64 * U) {
    u32x4_t xr[U][TW];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < TW; ++j) {
        const int c = c0 + 64 * u;
        xr[u][j] = (c < nch && t0 + j < T) ? ld16(x + (t0 + j) * (int64_t)D + (int64_t)c * 8) : zero4();
      }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + 64 * u;
      if (c >= nch) break;
#pragma unroll
      for (int e = 0; e < EC; ++e) {
        if (e < E) {
          const u32x4_t w = wlds[e * nch + c];
#pragma unroll
          for (int j = 0; j < TW; ++j) acc[j][e] = dot8_bf16(xr[u][j], w, acc[j][e]);
        }
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
    for (int j = 0; j < TW; ++j)
#pragma unroll
      for (int e = 0; e < EC; ++e) acc[j][e] += __shfl_xor(acc[j][e], off, 64);
#pragma unroll
  for (int j = 0; j < TW; ++j) {
    const int64_t t = t0 + j;
    if (t >= T) break;
    if (logits != nullptr) {
#pragma unroll
      for (int e = 0; e < EC; ++e)
        if (e < E && lane == (e & 63)) logits[t * E + e] = acc[j][e];
    }
    if (lane == 0) router_select<EC>(acc[j], E, top_k, ids + t * top_k, gate_w + t * top_k);
  }
}

template <int EC, int TW>
hipError_t launch_router_lds_cfg(const uint16_t* x, const uint16_t* Wr, int64_t T, int D, int E, int top_k,
                                 int32_t* ids, float* gate_w, float* logits, hipStream_t s) {
  const int64_t per_block = (kRouterLdsThreads / 64) * TW;
  const int64_t blocks = (T + per_block - 1) / per_block;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((moe_router_lds_kernel<EC, TW>), dim3((unsigned)blocks), dim3(kRouterLdsThreads), 0, s, x,
                     Wr, T, D, E, top_k, ids, gate_w, logits);
  return hipGetLastError();
}

template <int EC, int TW>
hipError_t launch_router_cfg(const uint16_t* x, const uint16_t* Wr, int64_t T, int D, int E, int top_k,
                             int32_t* ids, float* gate_w, float* logits, hipStream_t s) {
  const int64_t per_block = (kRouterThreads / 64) * TW;
  const int64_t blocks = (T + per_block - 1) / per_block;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((moe_router_kernel<EC, TW>), dim3((unsigned)blocks), dim3(kRouterThreads), 0, s, x, Wr, T, D,
                     E, top_k, ids, gate_w, logits);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_moe_router(const uint16_t* x, const uint16_t* Wr, int64_t T, int D, int E, int top_k,
                             int32_t* ids, float* gate_w, float* logits, int cus, hipStream_t s) {
  if (E < 1 || E > kRouterMaxExperts || top_k < 1 || top_k > 8 || top_k > E || D % 8 != 0)
    return hipErrorInvalidValue;
  if (E <= 16) {
    const int64_t blocks = (T + 15) / 16;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    if (blocks <= cus)
      hipLaunchKernelGGL(moe_router_mfma_kernel<16>, dim3((unsigned)blocks), dim3(kRouterMfmaWaves * 64), 0, s, x,
                         Wr, T, D, E, top_k, ids, gate_w, logits);
    else
      hipLaunchKernelGGL(moe_router_mfma_kernel<8>, dim3((unsigned)blocks), dim3(kRouterMfmaWaves * 64), 0, s, x,
                         Wr, T, D, E, top_k, ids, gate_w, logits);
    return hipGetLastError();
  }
  if ((int64_t)E * D * 2 <= kRouterLdsBytes) {
    if (E <= 32) return launch_router_lds_cfg<32, 1>(x, Wr, T, D, E, top_k, ids, gate_w, logits, s);
    return launch_router_lds_cfg<64, 1>(x, Wr, T, D, E, top_k, ids, gate_w, logits, s);
  }
  if (E <= 32) return launch_router_cfg<32, 2>(x, Wr, T, D, E, top_k, ids, gate_w, logits, s);
  return launch_router_cfg<64, 1>(x, Wr, T, D, E, top_k, ids, gate_w, logits, s);
}

hipError_t launch_moe_route(const int32_t* ids, const float* gate_w, int64_t T, int top_k, int E,
                            int bm, const MoeRouteOut& o, int32_t* counts, hipStream_t s) {
  if (E < 1 || E > kMoeRouteMaxExperts || top_k < 1 || T < 0 || bm < 1) return hipErrorInvalidValue;
  const int64_t P = T * (int64_t)top_k;
  const int64_t G = (P + kRouteThreads - 1) / kRouteThreads;
  if (P >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  if (G > 0) {
    hipLaunchKernelGGL(moe_route_count_kernel, dim3((unsigned)G), dim3(kRouteThreads), 0, s, ids, P, E, counts);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(moe_route_scan_kernel, dim3(1), dim3(kRouteScanThreads), 0, s, counts, (int)G, E, bm, o);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || G == 0) return e;
  hipLaunchKernelGGL(moe_route_place_kernel, dim3((unsigned)G), dim3(kRouteThreads), 0, s, ids, gate_w, P, top_k, E,
                     counts, o);
  return hipGetLastError();
}

hipError_t launch_moe_combine(const float* ytilde, const int32_t* pos_of, int64_t T, int top_k,
                              int64_t D, int ksplit, int64_t kstride, uint16_t* y, hipStream_t s) {
  const int64_t work = T * (D / 8);
  if (work <= 0) return hipSuccess;
  const int64_t blocks = (work + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)blocks), dim3(256), 0, s, ytilde, pos_of, T,
                     top_k, D, ksplit, kstride, y);
  return hipGetLastError();
}

}  // namespace fmlp
