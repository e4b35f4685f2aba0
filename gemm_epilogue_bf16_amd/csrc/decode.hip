// Decode path (M <= 16 tokens) for gfx950: a weight-streaming engine on MFMA.
//
// At batch 1-16 a feed-forward layer is bound by reading its weights once from
// HBM (ainews.cool "PyTorch fused MLP efficiency", section "architectural
// impact": autoregressive decode is memory-bandwidth bound), and launches
// matter (section "technical deep dive": the fused MLP is one launch that
// loads X once and writes only the final output).  The two-layer forms run as
// ONE launch.
//
// Work unit.  A block owns 16 output rows of a layer (one MFMA row tile) and
// walks K in stages of kSK = 1024: one stage is the 16 x 1024 bf16 slab of the
// weight (32 KB, one contiguous 2 KB piece per row).  Each thread loads 4
// 16-byte chunks per stage so that every wave instruction reads 1 KB of one
// weight row (fully coalesced), into a register ring: three stages (two when
// the gate and up weights stream together) are in flight per block while the
// oldest is written to a double-buffered LDS slab and consumed.  The LDS slab is swizzled (chunk c of row r sits at
// c ^ (r & 15) within its 16-chunk group) so the MFMA fragment reads of 16 rows
// are bank-conflict free.  Wave w takes k-steps of 32 from its 16-chunk group
// of every stage; v_mfma_f32_16x16x32_bf16 gets the weight rows as the row
// operand and the <= 16 activation rows as the column operand (zero for
// columns >= M).  Per-wave fp32 partial tiles are summed in a fixed order
// through LDS (bitwise deterministic), then the epilogue (bias + activation, or
// gelu_tanh(g) * u) runs in fp32 and rounds once to bf16.
//
// One stream, two layers.  The stages of layer 2 follow those of layer 1 in
// the same ring, so layer-2 weights are already in flight while layer 1
// finishes and while the block waits at the device-wide barrier that makes the
// hidden vector h visible.  h is written and read with device-coherent (agent
// scope) 32-bit atomic accesses, and the barrier is a set of per-block arrival
// flags polled by block 0, so no L2 write-back / invalidate is needed.  Every
// wait is bounded: a wait that gives up is counted in the workspace and the
// kernel still exits.
//
// All loads are buffer loads whose out-of-range offsets return 0 without a
// memory access: ragged tiles, the k tail, stages past the end of the stream
// and h fragments requested before the barrier are masked by the offset, with
// no branch around a load, so the compiler can count loads in flight and only
// waits for the ring slot it is about to consume.
#include <algorithm>
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace fmlp {

namespace {

constexpr int kNW = 8;                      // waves per block
constexpr int kThreads = kNW * 64;
constexpr int kSK = 1024;                   // k per stage
constexpr int kCH = kSK / 8;                // 16-byte chunks per row per stage (128)
constexpr int kLoads = 16 * kCH / kThreads; // chunks per thread per stage (4)
constexpr int kKS = kSK / 32 / kNW;         // MFMA k-steps per wave per stage (4)
constexpr uint32_t kSpinLimit = 1u << 20;   // bounded waits

__device__ __forceinline__ uint32_t ld_coherent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coherent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }
// wait until every vector memory access this wave issued has completed
__device__ __forceinline__ void wait_vm_all() {
  compiler_fence();
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0); expcnt, lgkmcnt not waited
  compiler_fence();
}

// Buffer resources: loads through them return 0 for offsets past the end
// without touching memory, which masks ragged tiles, the k tail and stages
// past the end of the stream without a branch around the load.
constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// plain 16-byte load
__device__ __forceinline__ u32x4_t bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint2 bload8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
// device-coherent (agent scope, sc1) 16-byte load: sees h stored by other XCDs
__device__ __forceinline__ u32x4_t bload_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 16));
}

struct Stream {
  int nt[2];        // tiles this block owns in each layer
  int S[2];         // stages per tile in each layer
  int first2;       // index of the first layer-2 stage (= nt[0] * S[0])
  int total;        // stages of this block
};

template <bool TWO>
__device__ __forceinline__ Stream make_stream(const GemvLayer& L1, const GemvLayer& L2) {
  Stream st;
  const int64_t G = gridDim.x, b = blockIdx.x;
  const int64_t tiles1 = (L1.N + 15) / 16;
  st.nt[0] = b < tiles1 ? (int)((tiles1 - 1 - b) / G + 1) : 0;
  st.S[0] = (int)((L1.K + kSK - 1) / kSK);
  if (TWO) {
    const int64_t tiles2 = (L2.N + 15) / 16;
    st.nt[1] = b < tiles2 ? (int)((tiles2 - 1 - b) / G + 1) : 0;
    st.S[1] = (int)((L2.K + kSK - 1) / kSK);
  } else {
    st.nt[1] = 0;
    st.S[1] = 1;
  }
  st.first2 = st.nt[0] * st.S[0];
  st.total = st.first2 + st.nt[1] * st.S[1];
  return st;
}

struct StageId {
  int phase;        // 0: layer 1, 1: layer 2
  int64_t n0;       // first output row of the tile
  int64_t k0;       // first k of the stage
  bool last;        // last stage of its tile
};

__device__ __forceinline__ StageId stage_id(const Stream& st, int g) {
  StageId id;
  const int p = g < st.first2 ? 0 : 1;
  const int r = p ? g - st.first2 : g;
  const int i = r / st.S[p], s = r - i * st.S[p];
  id.phase = p;
  id.n0 = ((int64_t)blockIdx.x + (int64_t)i * gridDim.x) * 16;
  id.k0 = (int64_t)s * kSK;
  id.last = (s == st.S[p] - 1);
  return id;
}

template <bool DUAL1, bool TWO>
__global__ void __launch_bounds__(kThreads)
decode_kernel(GemvLayer L1, GemvLayer L2, int M, uint32_t* sync) {
  constexpr int kSets = DUAL1 ? 2 : 1;   // layer 1 of GeGLU streams Wg and Wu together
  // stages in flight: 3 x 32 KB per block, or 2 x 64 KB when two weights stream
  constexpr int kRing = DUAL1 ? 2 : 3;
  __shared__ u32x4_t slab[2][kSets][16 * kCH];
  __shared__ float4 red[kSets][kNW * 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const Stream st = make_stream<TWO>(L1, L2);

  uint32_t target = 0;
  if (TWO) target = ld_coherent(sync + kSyncGenWord) + 1u;

  u32x4_t wreg[kRing][kSets][kLoads];
  u32x4_t xreg[kRing][kKS];
  uint2 breg[kRing];                      // bias of the tile ending at that stage
  f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};

  // weight chunks of stage g: thread tid loads chunks tid + i*kThreads; a wave
  // instruction covers 64 consecutive chunks (1 KB) of one weight row.  A stage
  // past the end of the stream, or one held back (live == false), loads nothing.
  auto issue_w = [&](int g, bool live, u32x4_t (&dst)[kSets][kLoads], uint2& bias) {
    const bool in = live && g < st.total;
    const StageId id = stage_id(st, in ? g : 0);
    const GemvLayer& L = id.phase ? L2 : L1;
    {   // the tile's bias, fetched with its last stage so the epilogue never waits
      const bool want = in && id.last && L.bias != nullptr;
      const int64_t n = id.n0 + 4 * lg;
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(want ? L.bias : L.W0, want ? (uint32_t)(L.N * 2) : 0u);
      bias = bload8(rb, n < L.N ? (uint32_t)(n * 2) : kOutOfRange);
    }
    const int64_t left = L.N - id.n0;
    const int64_t rows = in ? (left < 16 ? left : 16) : 0;
    const uint32_t nrec = (uint32_t)(rows * L.K * 2);
#pragma unroll
    for (int set = 0; set < kSets; ++set) {
      const uint16_t* W = (set && id.phase == 0) ? L.W1 : L.W0;
      const __amdgpu_buffer_rsrc_t r = make_rsrc(W + id.n0 * L.K, (set && id.phase == 1) ? 0u : nrec);
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        const int q = tid + i * kThreads;
        const int row = q / kCH, c = q % kCH;
        const int64_t k = id.k0 + c * 8;
        const uint32_t off = k < L.K ? (uint32_t)((row * L.K + k) * 2) : kOutOfRange;
        dst[set][i] = bload(r, off);
      }
    }
  };
  // activation fragments of stage g: rows >= M fall past the end of x and read
  // 0.  Loaded device-coherent in both layers (layer 2 reads h).
  auto issue_x = [&](int g, bool live, u32x4_t (&dst)[kKS]) {
    const bool in = live && g < st.total;
    const StageId id = stage_id(st, in ? g : 0);
    const GemvLayer& L = id.phase ? L2 : L1;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(L.x, in ? (uint32_t)((int64_t)M * L.K * 2) : 0u);
#pragma unroll
    for (int j = 0; j < kKS; ++j) {
      const int64_t k = id.k0 + (int64_t)(wave * 16 + j * 4 + lg) * 8;
      const uint32_t off = k < L.K ? (uint32_t)(((int64_t)li * L.K + k) * 2) : kOutOfRange;
      dst[j] = bload_coherent(r, off);
    }
  };
  auto write_slab = [&](int buf, int phase, const u32x4_t (&src)[kSets][kLoads]) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int q = tid + i * kThreads;
      const int row = q / kCH, c = q % kCH;
      const int slot = row * kCH + ((c & ~15) | ((c & 15) ^ row));
#pragma unroll
      for (int set = 0; set < kSets; ++set) {
        if (set == 1 && phase == 1) break;
        slab[buf][set][slot] = src[set][i];
      }
    }
  };
  auto compute = [&](int buf, int phase, const u32x4_t (&x)[kKS]) {
#pragma unroll
    for (int j = 0; j < kKS; ++j) {
      const int c = wave * 16 + j * 4 + lg;
      const int slot = li * kCH + ((c & ~15) | ((c & 15) ^ li));
      acc0 = mfma_16x16x32(slab[buf][0][slot], x[j], acc0);
      if (DUAL1 && phase == 0) acc1 = mfma_16x16x32(slab[buf][kSets - 1][slot], x[j], acc1);
    }
  };
  // end of a tile: fixed-order sum of the wave partials, epilogue, store
  auto finish_tile = [&](const StageId& id, const uint2 bias) {
    const bool dual = DUAL1 && id.phase == 0;
    red[0][wave * 64 + lane] = make_float4(acc0[0], acc0[1], acc0[2], acc0[3]);
    if (dual) red[kSets - 1][wave * 64 + lane] = make_float4(acc1[0], acc1[1], acc1[2], acc1[3]);
    acc0 = f32x4_t{0.f, 0.f, 0.f, 0.f};
    acc1 = f32x4_t{0.f, 0.f, 0.f, 0.f};
    __syncthreads();
    if (wave == 0) {
      const GemvLayer& L = id.phase ? L2 : L1;
      float g[4] = {0.f, 0.f, 0.f, 0.f}, u[4] = {0.f, 0.f, 0.f, 0.f};
      for (int w = 0; w < kNW; ++w) {
        const float4 t = red[0][w * 64 + lane];
        g[0] += t.x; g[1] += t.y; g[2] += t.z; g[3] += t.w;
        if (dual) {
          const float4 v = red[kSets - 1][w * 64 + lane];
          u[0] += v.x; u[1] += v.y; u[2] += v.z; u[3] += v.w;
        }
      }
      const int m = li;
      const int64_t n = id.n0 + 4 * lg;   // this lane's 4 consecutive outputs
      if (m < M && n < L.N) {
        float v[4];
        const float b[4] = {bf16_lo(bias.x), bf16_hi(bias.x), bf16_lo(bias.y), bf16_hi(bias.y)};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (dual) {
            v[r] = gelu_tanh(g[r]) * u[r];
          } else {
            v[r] = apply_act(g[r] + b[r], L.act);   // b = 0 without a bias
          }
        }
        const uint32_t lo = pack_bf16x2(v[0], v[1]), hi = pack_bf16x2(v[2], v[3]);
        uint32_t* dst = reinterpret_cast<uint32_t*>(L.y + (int64_t)m * L.N + n);
        if (TWO && id.phase == 0) {   // h: read by every block after the barrier
          st_coherent(dst, lo);
          st_coherent(dst + 1, hi);
        } else {
          *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
        }
      }
    }
  };
  // this block's h is complete once wave 0's stores are: publish the flag
  auto arrive = [&]() {
    if (wave == 0) {
      wait_vm_all();
      if (lane == 0) st_coherent(sync + kSyncFlagWord0 + blockIdx.x, target);
    }
  };
  auto bounded_wait = [&](const uint32_t* p) {
    uint32_t spins = 0;
    while (ld_coherent(p) != target) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > kSpinLimit) {
        __hip_atomic_fetch_add(sync + kSyncTimeoutWord, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  };
  // block 0 waits for every flag, then opens the generation every block waits on
  auto wait_all = [&]() {
    if (blockIdx.x == 0) {
      for (int b = tid; b < (int)gridDim.x; b += kThreads) bounded_wait(sync + kSyncFlagWord0 + b);
      __syncthreads();
      if (tid == 0) st_coherent(sync + kSyncGenWord, target);
    } else {
      if (tid == 0) bounded_wait(sync + kSyncGenWord);
      __syncthreads();
    }
  };
  // Layer-2 stages issued before the barrier get their h fragments after it.
  auto x_live = [&](int gx, int g) { return !(TWO && gx >= st.first2 && g < st.first2); };

  // a block with no layer-1 tile has nothing to publish
  if (TWO && st.first2 == 0) arrive();

  // ---- prologue: fill the ring ------------------------------------------------
#pragma unroll
  for (int d = 0; d < kRing; ++d) {
    issue_w(d, true, wreg[d], breg[d]);
    issue_x(d, x_live(d, 0), xreg[d]);
  }

  // ---- main loop, unrolled by the ring size so ring slots are static --------
  for (int g0 = 0; g0 < st.total; g0 += kRing) {
#pragma unroll
    for (int d = 0; d < kRing; ++d) {
      const int g = g0 + d;
      const bool valid = g < st.total;
      const StageId id = stage_id(st, valid ? g : 0);
      const uint2 bias_g = breg[d];   // slot d is refilled below, before the epilogue
      if (TWO && valid && g == st.first2) {   // entering layer 2: h must be complete
        wait_all();
#pragma unroll
        for (int e = 0; e < kRing; ++e) issue_x(g + e, true, xreg[(d + e) % kRing]);
      }
      if (valid) write_slab(g & 1, id.phase, wreg[d]);
      __syncthreads();
      issue_w(g + kRing, true, wreg[d], breg[d]);
      if (valid) compute(g & 1, id.phase, xreg[d]);
      issue_x(g + kRing, x_live(g + kRing, g), xreg[d]);
      if (valid && id.last) {
        finish_tile(id, bias_g);
        if (TWO && g == st.first2 - 1) arrive();
      }
    }
  }
}

struct Occ {
  bool probed = false;
  bool ok = false;
  int cus = 0;
  int one = 0;      // blocks per CU, one-layer kernel
  int two = 0;      // blocks per CU, two-layer kernel
  int two_dual = 0; // blocks per CU, GeGLU two-layer kernel
};

std::mutex g_occ_mu;
Occ g_occ[64];

// Residency of the decode kernels on the current device, queried once per
// device with the runtime's occupancy calculator and cached.
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
    ok &= hipOccupancyMaxActiveBlocksPerMultiprocessor(
              &o.one, reinterpret_cast<const void*>(&decode_kernel<false, false>), kThreads, 0) == hipSuccess;
    ok &= hipOccupancyMaxActiveBlocksPerMultiprocessor(
              &o.two, reinterpret_cast<const void*>(&decode_kernel<false, true>), kThreads, 0) == hipSuccess;
    ok &= hipOccupancyMaxActiveBlocksPerMultiprocessor(
              &o.two_dual, reinterpret_cast<const void*>(&decode_kernel<true, true>), kThreads, 0) == hipSuccess;
    o.ok = ok && o.cus > 0 && o.one > 0 && o.two > 0 && o.two_dual > 0;
  }
  return o;
}

}  // namespace

hipError_t launch_gemv(const GemvLayer& L, int M, hipStream_t s) {
  if (L.geglu) return hipErrorInvalidValue;   // gate+up runs only in the two-layer kernel
  const int64_t tiles = (L.N + 15) / 16;
  if (tiles <= 0 || M <= 0) return hipSuccess;
  const Occ o = occ();
  if (!o.ok) return hipErrorInvalidDevice;
  // one layer has no barrier: cap the grid at one resident round of blocks
  const unsigned grid = (unsigned)std::min<int64_t>(tiles, (int64_t)o.cus * o.one);
  hipLaunchKernelGGL((decode_kernel<false, false>), dim3(grid), dim3(kThreads), 0, s, L, L, M,
                     static_cast<uint32_t*>(nullptr));
  return hipGetLastError();
}

hipError_t launch_gemv2_persistent(const GemvLayer& L1, const GemvLayer& L2, int M, uint32_t* sync,
                                   hipStream_t s) {
  const Occ o = occ();
  if (!o.ok) return hipErrorInvalidDevice;
  const bool dual = L1.geglu != 0;
  const int64_t tiles1 = (L1.N + 15) / 16, tiles2 = (L2.N + 15) / 16;
  // every block must be resident at once: the barrier waits for all of them
  const int64_t cap = std::min<int64_t>((int64_t)o.cus * (dual ? o.two_dual : o.two), kDecodeMaxBlocks);
  const unsigned grid = (unsigned)std::min<int64_t>(cap, std::max(tiles1, tiles2));
  if (grid == 0) return hipSuccess;
  if (dual)
    hipLaunchKernelGGL((decode_kernel<true, true>), dim3(grid), dim3(kThreads), 0, s, L1, L2, M, sync);
  else
    hipLaunchKernelGGL((decode_kernel<false, true>), dim3(grid), dim3(kThreads), 0, s, L1, L2, M, sync);
  return hipGetLastError();
}

}  // namespace fmlp
