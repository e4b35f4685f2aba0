// Decode path (M <= 16 tokens) for gfx950: a weight-streaming engine on MFMA.
//
// At batch 1-16 a feed-forward layer is bound by reading its weights once from
// HBM (ainews.cool "PyTorch fused MLP efficiency", section "architectural
// impact": autoregressive decode is memory-bandwidth bound), and launches
// matter (section "technical deep dive": the fused MLP is one launch that
// loads X once and writes only the final output).  The two-layer forms run as
// ONE launch.
//
// Roles.  A block has 7 worker waves and 1 control wave.  The workers stream
// weights and run the MFMAs; the control wave never loads a weight, so its
// waits cover only its own few accesses: it sums the workers' partial tiles,
// runs the epilogue, stores the result, and (two-layer form) publishes and
// awaits the hidden vector h.
//
// Work unit.  A block owns 16 output rows of a layer (one MFMA row tile) and
// walks K in stages of kSK = 896: one stage is the 16 x 896 bf16 slab of the
// weight (28 KB, one contiguous 1792-byte piece per row).  Each worker thread
// loads 4 16-byte chunks per stage, so a wave instruction reads 1 KB of one
// weight row (fully coalesced), into a register ring: three stages (two when
// the gate and up weights stream together) are in flight per block while the
// oldest is written to a double-buffered LDS slab and consumed.  The slab is
// swizzled (chunk c of row r sits at c ^ (r & 15) within its 16-chunk group)
// so the MFMA fragment reads of 16 rows are bank-conflict free.  Worker w takes
// 4 k-steps of 32 from its 16-chunk group of every stage;
// v_mfma_f32_16x16x32_bf16 gets the weight rows as the row operand and the
// <= 16 activation rows as the column operand (zero for columns >= M).  The
// control wave sums the 7 fp32 partial tiles in a fixed order (bitwise
// deterministic) and applies the epilogue (bias + activation, or
// gelu_tanh(g) * u) in fp32 with one rounding to bf16.
//
// One stream, two layers.  The stages of layer 2 follow those of layer 1 in
// the same ring, so layer-2 weights are in flight while layer 1 finishes and
// while the block waits for h.  The control wave stores h with device-coherent
// (agent scope) stores, waits for its own stores, and raises the block's
// arrival flag; every control wave then polls all flags (one hop, no L2
// write-back or invalidate) and releases its workers, which read h with plain
// loads: no h line is touched before every block has published, so no stale
// copy can sit in an L2.  Every wait is bounded: a wait that gives up is
// counted in the workspace and the kernel still exits.
//
// All worker loads are buffer loads whose out-of-range offsets return 0 without
// a memory access: ragged tiles, the k tail, stages past the end of the stream
// and h fragments requested before the barrier are masked by the offset, with
// no branch around a load, so the compiler counts the loads in flight and waits
// only for the ring slot it is about to consume.
#include <algorithm>
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace fmlp {

namespace {

constexpr int kWorkers = 7;                    // streaming + MFMA waves
constexpr int kThreads = (kWorkers + 1) * 64;  // + the control wave
constexpr int kWT = kWorkers * 64;             // worker threads
constexpr int kSK = kWorkers * 128;            // k per stage: 128 per worker wave
constexpr int kCH = kSK / 8;                   // 16-byte chunks per row per stage (112)
constexpr int kLoads = 16 * kCH / kWT;         // chunks per worker thread per stage (4)
constexpr int kKS = 4;                         // MFMA k-steps per worker wave per stage
constexpr uint32_t kSpinLimit = 1u << 20;      // bounded waits
static_assert(16 * kCH == kLoads * kWT, "stage tiling");

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
// without touching memory.
constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;
// Every descriptor here is wave-uniform by construction (it depends only on
// the stage, the layer and the block); readfirstlane puts it in SGPRs so the
// load needs no per-lane loop.  readfirstlane returns a signed int: each half
// is widened through uint32_t, never sign-extended into the other half.
__device__ __forceinline__ uint32_t uniform32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint64_t ua = ((uint64_t)uniform32((uint32_t)(a >> 32)) << 32) | (uint64_t)uniform32((uint32_t)a);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(ua), (short)0,
                                           (int)uniform32(bytes), 0x00020000);
}
__device__ __forceinline__ u32x4_t bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
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
  const int G = gridDim.x, b = blockIdx.x;
  const int tiles1 = (int)((L1.N + 15) / 16);
  st.nt[0] = b < tiles1 ? (tiles1 - 1 - b) / G + 1 : 0;
  st.S[0] = (int)((L1.K + kSK - 1) / kSK);
  if (TWO) {
    const int tiles2 = (int)((L2.N + 15) / 16);
    st.nt[1] = b < tiles2 ? (tiles2 - 1 - b) / G + 1 : 0;
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
  // stages in flight: 3 x 28 KB per block, or 2 x 56 KB when two weights stream
  constexpr int kRing = DUAL1 ? 2 : 3;
  __shared__ u32x4_t slab[2][kSets][16 * kCH];
  __shared__ float4 red[kSets][kWorkers * 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in an SGPR
  const int li = lane & 15, lg = lane >> 4;
  const bool worker = wave < kWorkers;
  const Stream st = make_stream<TWO>(L1, L2);

  uint32_t target = 0;
  if (TWO) target = ld_coherent(sync + kSyncGenWord) + 1u;

  u32x4_t wreg[kRing][kSets][kLoads];
  u32x4_t xreg[kRing][kKS];
  f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};

  // ---- worker side ---------------------------------------------------------
  // The control wave executes the same ring loads with every offset out of
  // range (no memory access), so all waves issue the same sequence of loads
  // and the compiler's count of loads in flight stays exact on every path.
  // weight chunks of stage g: worker thread tid loads chunks tid + i*kWT; a
  // wave instruction covers 64 consecutive chunks (1 KB) of one weight row.
  auto issue_w = [&](int g, u32x4_t (&dst)[kSets][kLoads]) {
    const bool in = worker && g < st.total;
    const StageId id = stage_id(st, in ? g : 0);
    const GemvLayer& L = id.phase ? L2 : L1;
    const int64_t left = L.N - id.n0;
    const int64_t rows = in ? (left < 16 ? left : 16) : 0;
    const uint32_t nrec = (uint32_t)(rows * L.K * 2);
#pragma unroll
    for (int set = 0; set < kSets; ++set) {
      const uint16_t* W = (set && id.phase == 0) ? L.W1 : L.W0;
      const __amdgpu_buffer_rsrc_t r = make_rsrc(W + id.n0 * L.K, (set && id.phase == 1) ? 0u : nrec);
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        const int q = tid + i * kWT;
        const int row = q / kCH, c = q % kCH;
        const int64_t k = id.k0 + c * 8;
        const uint32_t off = k < L.K ? (uint32_t)((row * L.K + k) * 2) : kOutOfRange;
        dst[set][i] = bload(r, off);
      }
    }
  };
  // activation fragments of stage g (x, or h after the barrier); rows >= M
  // fall past the end of the activation buffer and read 0.  live == false
  // (h before the barrier) loads nothing.
  auto issue_x = [&](int g, bool live, u32x4_t (&dst)[kKS]) {
    const bool in = worker && live && g < st.total;
    const StageId id = stage_id(st, in ? g : 0);
    const GemvLayer& L = id.phase ? L2 : L1;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(L.x, in ? (uint32_t)((int64_t)M * L.K * 2) : 0u);
#pragma unroll
    for (int j = 0; j < kKS; ++j) {
      const int64_t k = id.k0 + (int64_t)(wave * 16 + j * 4 + lg) * 8;
      const uint32_t off = k < L.K ? (uint32_t)(((int64_t)li * L.K + k) * 2) : kOutOfRange;
      dst[j] = bload(r, off);
    }
  };
  auto write_slab = [&](int buf, int phase, const u32x4_t (&src)[kSets][kLoads]) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int q = tid + i * kWT;
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
  auto post_partials = [&](int phase) {
    red[0][wave * 64 + lane] = make_float4(acc0[0], acc0[1], acc0[2], acc0[3]);
    if (DUAL1 && phase == 0)
      red[kSets - 1][wave * 64 + lane] = make_float4(acc1[0], acc1[1], acc1[2], acc1[3]);
    acc0 = f32x4_t{0.f, 0.f, 0.f, 0.f};
    acc1 = f32x4_t{0.f, 0.f, 0.f, 0.f};
  };

  // ---- control side --------------------------------------------------------
  // bias of the control wave's next tile, requested one tile ahead
  int ctile = 0;
  uint2 cbias = make_uint2(0u, 0u);
  auto ctrl_fetch_bias = [&](int t) {
    const int ntiles = st.nt[0] + st.nt[1];
    const int p = t < st.nt[0] ? 0 : 1;
    const GemvLayer& L = p ? L2 : L1;
    const int i = p ? t - st.nt[0] : t;
    const int64_t n = ((int64_t)blockIdx.x + (int64_t)i * gridDim.x) * 16 + 4 * lg;
    const bool want = t < ntiles && L.bias != nullptr;          // wave-uniform
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(want ? L.bias : L.W0, want ? (uint32_t)(L.N * 2) : 0u);
    const uint32_t off = n < L.N ? (uint32_t)(n * 2) : kOutOfRange;   // per lane
    cbias = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rb, off, 0, 0));
  };
  auto ctrl_epilogue = [&](const StageId& id) {
    const bool dual = DUAL1 && id.phase == 0;
    const GemvLayer& L = id.phase ? L2 : L1;
    float g[4] = {0.f, 0.f, 0.f, 0.f}, u[4] = {0.f, 0.f, 0.f, 0.f};
    for (int w = 0; w < kWorkers; ++w) {
      const float4 t = red[0][w * 64 + lane];
      g[0] += t.x; g[1] += t.y; g[2] += t.z; g[3] += t.w;
      if (dual) {
        const float4 v = red[kSets - 1][w * 64 + lane];
        u[0] += v.x; u[1] += v.y; u[2] += v.z; u[3] += v.w;
      }
    }
    const uint2 bias = cbias;
    ctrl_fetch_bias(++ctile);
    const int m = li;
    const int64_t n = id.n0 + 4 * lg;   // this lane's 4 consecutive outputs
    if (m < M && n < L.N) {
      float v[4];
      const float b[4] = {bf16_lo(bias.x), bf16_hi(bias.x), bf16_lo(bias.y), bf16_hi(bias.y)};
#pragma unroll
      for (int r = 0; r < 4; ++r)
        v[r] = dual ? gelu_tanh(g[r]) * u[r] : apply_act(g[r] + b[r], L.act);   // b = 0 without a bias
      const uint32_t lo = pack_bf16x2(v[0], v[1]), hi = pack_bf16x2(v[2], v[3]);
      uint32_t* dst = reinterpret_cast<uint32_t*>(L.y + (int64_t)m * L.N + n);
      if (TWO && id.phase == 0) {   // h: read by every block after the barrier
        st_coherent(dst, lo);
        st_coherent(dst + 1, hi);
      } else {
        *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
      }
    }
  };
  // this block's h is complete once the control wave's stores are: raise the flag
  auto ctrl_arrive = [&]() {
    wait_vm_all();
    if (lane == 0) st_coherent(sync + kSyncFlagWord0 + blockIdx.x, target);
  };
  // every control wave polls every block's flag (one hop)
  auto ctrl_wait_all = [&]() {
    for (int b = lane; b < (int)gridDim.x; b += 64) {
      uint32_t spins = 0;
      while (ld_coherent(sync + kSyncFlagWord0 + b) != target) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins > kSpinLimit) {
          __hip_atomic_fetch_add(sync + kSyncTimeoutWord, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
    }
    if (blockIdx.x == 0 && lane == 0) st_coherent(sync + kSyncGenWord, target);
  };

  // An h fragment may be requested only once the barrier has passed, i.e. from
  // iteration first2 on (its wait runs at the start of that iteration); the
  // ones requested earlier are re-requested right after the barrier.
  auto x_live = [&](int gx, int g) { return !(TWO && gx >= st.first2 && g < st.first2); };

  if (!worker) {
    ctrl_fetch_bias(0);
    if (TWO && st.first2 == 0) ctrl_arrive();   // no layer-1 tile: nothing to publish
  }
  // the prologue runs before iteration 0, i.e. before any barrier (g = -1):
  // touching h here would also pull not-yet-published lines into the L2
#pragma unroll
  for (int d = 0; d < kRing; ++d) {
    issue_w(d, wreg[d]);
    issue_x(d, x_live(d, -1), xreg[d]);
  }

  // ---- main loop, unrolled by the ring size so ring slots are static --------
  for (int g0 = 0; g0 < st.total; g0 += kRing) {
#pragma unroll
    for (int d = 0; d < kRing; ++d) {
      const int g = g0 + d;
      const bool valid = g < st.total;
      const StageId id = stage_id(st, valid ? g : 0);
      if (TWO && valid && g == st.first2) {   // entering layer 2: h must be complete
        if (!worker) ctrl_wait_all();
        __syncthreads();
#pragma unroll
        for (int e = 0; e < kRing; ++e) issue_x(g + e, true, xreg[(d + e) % kRing]);
      }
      if (worker && valid) write_slab(g & 1, id.phase, wreg[d]);
      __syncthreads();
      issue_w(g + kRing, wreg[d]);
      if (worker && valid) compute(g & 1, id.phase, xreg[d]);
      issue_x(g + kRing, x_live(g + kRing, g), xreg[d]);
      if (worker && valid && id.last) post_partials(id.phase);
      if (valid && id.last) {
        __syncthreads();
        if (!worker) {
          ctrl_epilogue(id);
          if (TWO && g == st.first2 - 1) ctrl_arrive();
        }
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
