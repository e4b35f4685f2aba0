// The whole gated feed-forward block in ONE launch with the intermediate kept
// on the compute unit, for gfx950:
//
//   y[M, D] = (act(x Wg^T) * (x Wu^T)) Wd^T,   Wg, Wu [H, D], Wd [D, H]
//
// "Profiling in PyTorch (Part 2): From nn.Linear to a Fused MLP", section "The
// fused Triton kernel": the [tokens, hidden] intermediate m costs a write and a
// read of global memory between the gate/up GEMMs and the down projection;
// ainews.cool "PyTorch fused MLP efficiency", section "technical deep dive": the
// fused MLP is one kernel that reads x once and writes only the output.  Here m
// exists only as a 64 x 128 bf16 tile in LDS.
//
// Work split.  A block owns 64 token rows and one of S contiguous ranges of the
// hidden units ("parts").  It walks its range in sub-chunks of 128 units:
//   gate+up  g, u [64 x 128] = x[64 x D] . Wg, Wu[128 rows]^T   (stages of 64 k)
//   m        act(g) * u, rounded to bf16 (the down MFMA's operand), into LDS
//   down     y[64 x D] += m[64 x 128] . Wd[:, 128 columns]^T    (stages of
//            256 Wd rows x 64 k)
// and y stays in fp32 registers over the whole range.  With S = 1 the block
// writes bf16 y.  With S > 1 every block writes its fp32 partial y; the block
// that arrives last for its token rows adds the S partials in part order (so
// the result does not depend on arrival order: bitwise deterministic) and
// writes bf16 y.
//
// Why only model widths up to 1024.  The accumulator of y is 64 x D fp32 per
// block; at D = 1024 that is 128 of a wave's registers with 8 waves.  Splitting
// the hidden range costs 8 * M * D * S bytes of partials (written and read),
// against 4 * M * H bytes for m's round trip in the two-launch form, so keeping
// m on chip saves traffic only while the part of the hidden range a block
// covers exceeds 2 D: at the 8192/28672 shape (D = 8192) no split pays, and a y
// accumulator of 8192 columns does not fit a compute unit.  Wider blocks use the
// two GEMM launches.
//
// Streaming.  Every stage (activation rows + 256 weight rows of 64 k, 40 KB)
// goes from memory straight into a 3-slot LDS ring with buffer loads that write
// LDS (16 bytes per lane; 1 KB per instruction, lane-ordered), two stages
// ahead of the MFMAs; each wave issues the same 5 loads per stage (down stages
// load no activation: that load is requested out of range and writes zeros),
// waits for its own loads of the stage it is about to read, and one workgroup
// barrier per stage publishes it and frees the slot the next loads go to.
// Rows past the end of x, Wg, Wu or Wd and chunks past K arrive as zeros with
// no branch (out-of-range buffer offsets).  Chunk c of a 128-byte stage row r
// sits at slot c ^ ((r >> 1) & 7) and chunk c of a 256-byte m row r at
// c ^ (r & 15), so every 16-row fragment read is bank-conflict free under the
// four 16-lane cycles of a ds_read_b128 on gfx950 (lane l's cycle is set by
// l >> 5 and the parity of (l >> 2) & 7).
#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "lds_dma.h"

namespace fmlp {

namespace {

constexpr int kBM = kGluFusedRows;        // token rows per block
constexpr int kHS = kGluFusedSub;         // hidden units per sub-chunk
constexpr int kBK = 64;                   // k per stage
constexpr int kWaves = 8;                 // 2 (tokens) x 4 (weight rows)
constexpr int kThreads = kWaves * 64;
constexpr int kR = 3;                     // ring slots: two stages in flight
constexpr int kXRows = kBM;               // activation rows of a stage
constexpr int kWRows = 2 * kHS;           // weight rows of a stage
constexpr int kSlotChunks = (kXRows + kWRows) * 8;   // 16-byte chunks of a slot (40 KB)
constexpr int kLoads = 5;                 // load instructions per wave and stage
constexpr int kMChunks = kBM * (kHS / 8);           // the m tile (16 KB)

__device__ __forceinline__ int sw8(int r) { return (r >> 1) & 7; }

struct FusedGluParams {
  const uint16_t* x;
  const uint16_t* Wg;
  const uint16_t* Wu;
  const uint16_t* Wd;
  uint16_t* y;
  float* part;          // [S][m_tiles][64][D] fp32 partials (S > 1)
  uint64_t* arrive;     // [m_tiles]: {salt (high word), arrivals (low word)}
  int64_t M;
  int D, H;
  int S, hc;            // parts of the hidden range; hidden units per part (multiple of 128)
  int m_tiles;
  uint32_t salt;        // this launch's tag of the arrival words
};

template <int ND, int ACT>
__global__ void __launch_bounds__(kThreads) glu_fused_kernel(FusedGluParams p) {
  __shared__ u32x4_t ring[kR * kSlotChunks];
  __shared__ u32x4_t mbuf[kMChunks];
  __shared__ uint32_t last_arrival;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int wm = w >> 2, wn = w & 3;

  // block -> (token tile, part): consecutive logical blocks share an XCD, so
  // the S parts of a token tile (and their partials) share an L2
  const int L = xcd_remap((int)blockIdx.x, (int)gridDim.x);
  const int mt = L / p.S, part = L - mt * p.S;
  const int64_t t0 = (int64_t)mt * kBM;
  const int rows = (int)min((int64_t)kBM, p.M - t0);
  const int D = p.D, H = p.H;
  const int h_begin = part * p.hc;
  const int h_end = min(H, h_begin + p.hc);
  const int nsub = h_end > h_begin ? (h_end - h_begin + kHS - 1) / kHS : 0;
  const int NA = (D + kBK - 1) / kBK;        // gate+up stages per sub-chunk
  constexpr int NB = 2 * ND;                 // down stages per sub-chunk
  const int PER = NA + NB;
  const int total = nsub * PER;

  // ---- per-lane load offsets ------------------------------------------------
  // Load instruction i of a stage fills stage rows 8 i .. 8 i + 7 (activation
  // rows first, then weight rows); lane l fills position l % 8 of row l / 8 and
  // fetches the global chunk whose swizzled home that is.  Wave w issues the
  // activation instruction w and weight instructions 4 w .. 4 w + 3 (waves 0-3:
  // gate rows, 4-7: up rows; in a down stage all 256 rows are Wd rows).
  const int pos = lane & 7;
  const int rx = 8 * w + (lane >> 3);
  const int cx = pos ^ sw8(rx);
  const uint32_t voff_x = (uint32_t)(rx * D + 8 * cx) * 2u;
  int cw[4];
  uint32_t voff_a[4], voff_b[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int rw = 8 * (4 * w + j) + (lane >> 3);   // weight row of the stage (0 .. 255)
    cw[j] = pos ^ sw8(rw);
    voff_a[j] = (uint32_t)((rw & (kHS - 1)) * D + 8 * cw[j]) * 2u;
    voff_b[j] = (uint32_t)(rw * H + 8 * cw[j]) * 2u;
  }
  const uint32_t ring_lds = lds_addr(&ring[0]);
  const i32x4_t none = make_desc(reinterpret_cast<uint64_t>(p.x), 0u);
  const uint16_t* const wgu = w < 4 ? p.Wg : p.Wu;   // wave-uniform

  auto issue = [&](int q) {   // stream stage q into slot q % kR
    const uint32_t sbase = ring_lds + (uint32_t)(q % kR) * (uint32_t)(kSlotChunks * 16);
    i32x4_t dx = none, dw = none;
    uint32_t xo = kOutOfRange, soff = 0;
    uint32_t wo[4] = {kOutOfRange, kOutOfRange, kOutOfRange, kOutOfRange};
    if (q < total) {
      const int sub = q / PER, r = q - sub * PER;
      const int h0 = h_begin + sub * kHS;
      if (r < NA) {            // gate+up: x rows and 128 gate or up rows, k range r
        const int k0 = r * kBK;
        soff = (uint32_t)k0 * 2u;
        dx = make_desc(reinterpret_cast<uint64_t>(p.x + t0 * D), (uint32_t)(rows * D) * 2u);
        xo = k0 + 8 * cx < D ? voff_x : kOutOfRange;
        dw = make_desc(reinterpret_cast<uint64_t>(wgu + (int64_t)h0 * D), (uint32_t)(min(kHS, H - h0) * D) * 2u);
#pragma unroll
        for (int j = 0; j < 4; ++j) wo[j] = k0 + 8 * cw[j] < D ? voff_a[j] : kOutOfRange;
      } else {                 // down: Wd rows 256 nb .. + 255, hidden k range h0 + 64 kh
        const int b = r - NA, nb = b >> 1, kh = b & 1;
        const int kk = h0 + kh * kBK;
        soff = (uint32_t)kk * 2u;
        dw = make_desc(reinterpret_cast<uint64_t>(p.Wd + (int64_t)(256 * nb) * H),
                       (uint32_t)(min(256, D - 256 * nb) * H) * 2u);
#pragma unroll
        for (int j = 0; j < 4; ++j) wo[j] = kk + 8 * cw[j] < H ? voff_b[j] : kOutOfRange;
      }
    }
    asm_load_lds(dx, sbase + (uint32_t)w * 1024u, xo, soff);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      asm_load_lds(dw, sbase + (uint32_t)(kXRows * 128) + (uint32_t)(4 * w + j) * 1024u, wo[j], soff);
  };

  // ---- fragment positions ---------------------------------------------------
  // MFMA 16x16x32: the weight rows are the row operand, the tokens the column
  // operand; lane (li, lg) reads row li of a fragment at k chunk 4 ks + lg and
  // receives rows 4 lg .. 4 lg + 3 (weight rows) of column li (token).
  int xa[2][2], ga[2][4], da[2][4], ma[2][2][2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int r = 32 * wm + 16 * f + li;
      xa[ks][f] = r * 8 + ((4 * ks + lg) ^ sw8(r));
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) ma[kh][ks][f] = r * 16 + ((8 * kh + 4 * ks + lg) ^ (r & 15));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rg = (j < 2 ? 32 * wn + 16 * j : kHS + 32 * wn + 16 * (j - 2)) + li;   // gate j = 0, 1; up 2, 3
      ga[ks][j] = (kXRows + rg) * 8 + ((4 * ks + lg) ^ sw8(rg));
      const int rd = 64 * wn + 16 * j + li;
      da[ks][j] = (kXRows + rd) * 8 + ((4 * ks + lg) ^ sw8(rd));
    }
  }

  f32x4_t accy[ND][2][4];
#pragma unroll
  for (int nb = 0; nb < ND; ++nb)
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int j = 0; j < 4; ++j) accy[nb][f][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int q = 0; q < kR - 1; ++q) issue(q);
  int g = 0;   // stream index of the stage being consumed
  auto top = [&]() -> const u32x4_t* {
    wait_vm<kLoads * (kR - 2)>();   // this wave's loads of stage g
    lds_barrier();                  // ... and every wave's; slot (g - 1) % kR is free
    issue(g + kR - 1);
    return ring + (g % kR) * kSlotChunks;
  };

  for (int sub = 0; sub < nsub; ++sub) {
    f32x4_t acc[2][4];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[f][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int a = 0; a < NA; ++a, ++g) {
      const u32x4_t* sl = top();
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32x4_t xf[2], wf[4];
#pragma unroll
        for (int f = 0; f < 2; ++f) xf[f] = sl[xa[ks][f]];
#pragma unroll
        for (int j = 0; j < 4; ++j) wf[j] = sl[ga[ks][j]];
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[f][j] = mfma_16x16x32(wf[j], xf[f], acc[f][j]);
      }
    }
    // m = act(g) * u for this wave's 32 tokens x 32 hidden units, into LDS:
    // lane (li, lg) holds hidden units 16 gi + 4 lg .. + 3 of token li
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int t = 32 * wm + 16 * f + li;
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        const int hcol = 32 * wn + 16 * gi + 4 * lg;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = act_of<ACT>(acc[f][gi][r]) * acc[f][gi + 2][r];
        uint2 pk;
        pk.x = pack_bf16x2(v[0], v[1]);
        pk.y = pack_bf16x2(v[2], v[3]);
        char* dst = reinterpret_cast<char*>(&mbuf[t * 16 + ((hcol >> 3) ^ (t & 15))]) + 8 * (lg & 1);
        *reinterpret_cast<uint2*>(dst) = pk;
      }
    }
    // down: the next stage's barrier also publishes m
#pragma unroll
    for (int nb = 0; nb < ND; ++nb) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh, ++g) {
        const u32x4_t* sl = top();
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          u32x4_t mf[2], wf[4];
#pragma unroll
          for (int f = 0; f < 2; ++f) mf[f] = mbuf[ma[kh][ks][f]];
#pragma unroll
          for (int j = 0; j < 4; ++j) wf[j] = sl[da[ks][j]];
#pragma unroll
          for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int j = 0; j < 4; ++j) accy[nb][f][j] = mfma_16x16x32(wf[j], mf[f], accy[nb][f][j]);
        }
      }
    }
  }
  wait_vm<0>();   // the stages issued past the end (loads of nothing) have landed

  // ---- output ---------------------------------------------------------------
  // lane (li, lg) holds y[token 32 wm + 16 f + li][256 nb + 64 wn + 16 j + 4 lg + r]
  auto store_y = [&](int nb, int f, int j, const float v[4]) {
    const int t = 32 * wm + 16 * f + li;
    const int d = 256 * nb + 64 * wn + 16 * j + 4 * lg;   // D % 8 == 0: d < D covers d + 3
    if (t < rows && d < D) {
      uint2 pk;
      pk.x = pack_bf16x2(v[0], v[1]);
      pk.y = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<uint2*>(p.y + (t0 + t) * D + d) = pk;
    }
  };
  if (p.S == 1) {
#pragma unroll
    for (int nb = 0; nb < ND; ++nb)
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float v[4] = {accy[nb][f][j][0], accy[nb][f][j][1], accy[nb][f][j][2], accy[nb][f][j][3]};
          store_y(nb, f, j, v);
        }
    return;
  }
  auto part_at = [&](int s) { return p.part + ((int64_t)s * p.m_tiles + mt) * (int64_t)(kBM * D); };
  float* mine = part_at(part);
#pragma unroll
  for (int nb = 0; nb < ND; ++nb)
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = 32 * wm + 16 * f + li;
        const int d = 256 * nb + 64 * wn + 16 * j + 4 * lg;
        if (t < rows && d < D) *reinterpret_cast<f32x4_t*>(mine + t * D + d) = accy[nb][f][j];
      }
  // Arrival: every wave's partial stores have completed, then one release at
  // device scope (the partials become visible to every XCD) and an arrival
  // count tagged with this launch's salt (a word carrying another salt is
  // left over from an earlier call and counts as zero arrivals).
  wait_vm<0>();
  __syncthreads();
  if (tid == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    uint64_t old = __hip_atomic_load(&p.arrive[mt], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint64_t want;
    do {
      const uint64_t before = (uint32_t)(old >> 32) == p.salt ? (old & 0xFFFFFFFFull) : 0ull;
      want = ((uint64_t)p.salt << 32) | (before + 1ull);
    } while (!__hip_atomic_compare_exchange_weak(&p.arrive[mt], &old, want, __ATOMIC_ACQ_REL, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT));
    last_arrival = (want & 0xFFFFFFFFull) == (uint64_t)p.S ? 1u : 0u;
  }
  __syncthreads();
  if (last_arrival == 0u) return;   // block-uniform
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
#pragma unroll
  for (int nb = 0; nb < ND; ++nb)
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = 32 * wm + 16 * f + li;
        const int d = 256 * nb + 64 * wn + 16 * j + 4 * lg;
        if (!(t < rows && d < D)) continue;
        float v[4] = {0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < p.S; ++s) {   // part order, whichever block arrived last
          const f32x4_t q = s == part ? accy[nb][f][j] : *reinterpret_cast<const f32x4_t*>(part_at(s) + t * D + d);
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] += q[r];
        }
        store_y(nb, f, j, v);
      }
}

template <int ND>
hipError_t launch_nd(const FusedGluParams& p, int act, unsigned grid, hipStream_t s) {
  switch (act) {
    case ACT_GELU_TANH: hipLaunchKernelGGL((glu_fused_kernel<ND, ACT_GELU_TANH>), dim3(grid), dim3(kThreads), 0, s, p); break;
    case ACT_GELU_ERF: hipLaunchKernelGGL((glu_fused_kernel<ND, ACT_GELU_ERF>), dim3(grid), dim3(kThreads), 0, s, p); break;
    case ACT_RELU: hipLaunchKernelGGL((glu_fused_kernel<ND, ACT_RELU>), dim3(grid), dim3(kThreads), 0, s, p); break;
    case ACT_SILU: hipLaunchKernelGGL((glu_fused_kernel<ND, ACT_SILU>), dim3(grid), dim3(kThreads), 0, s, p); break;
    case ACT_NONE: hipLaunchKernelGGL((glu_fused_kernel<ND, ACT_NONE>), dim3(grid), dim3(kThreads), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_glu_fused(const uint16_t* x, const uint16_t* Wg, const uint16_t* Wu, const uint16_t* Wd, int act,
                            int64_t M, int64_t D, int64_t H, uint16_t* y, void* ws, uint32_t salt, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (D <= 0 || D > kGluFusedMaxD || D % 8 != 0 || H <= 0 || H % 8 != 0 || H > kGluFusedMaxH)
    return hipErrorInvalidValue;
  const GluFusedShape f = glu_fused_shape(M, H);
  const int64_t grid = (int64_t)f.m_tiles * f.S;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  FusedGluParams p;
  p.x = x;
  p.Wg = Wg;
  p.Wu = Wu;
  p.Wd = Wd;
  p.y = y;
  p.arrive = static_cast<uint64_t*>(ws);
  p.part = reinterpret_cast<float*>(static_cast<char*>(ws) + glu_fused_arrive_bytes(f.m_tiles));
  p.M = M;
  p.D = (int)D;
  p.H = (int)H;
  p.S = f.S;
  p.hc = f.hc;
  p.m_tiles = (int)f.m_tiles;
  p.salt = salt;
  switch ((D + 255) / 256) {
    case 1: return launch_nd<1>(p, act, (unsigned)grid, s);
    case 2: return launch_nd<2>(p, act, (unsigned)grid, s);
    case 3: return launch_nd<3>(p, act, (unsigned)grid, s);
    case 4: return launch_nd<4>(p, act, (unsigned)grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fmlp
