// Decode path (M <= 16 tokens) for gfx950: a weight-streaming engine on MFMA.
//
// At batch 1-16 a feed-forward layer is bound by reading its weights once from
// HBM (ainews.cool "PyTorch fused MLP efficiency", section "architectural
// impact": autoregressive decode is memory-bandwidth bound), and launches
// matter (section "technical deep dive": the fused MLP is one launch that
// loads X once and writes only the final output).  The two-layer forms run as
// ONE launch.
//
// Streaming.  Weights and activation slices go from memory straight into an
// LDS ring with buffer loads that write LDS (no register staging): one block
// per CU keeps up to R - 1 = 3 stages in flight, which holds HBM at its
// streaming rate without a long per-CU request queue.  A stage is 16 weight
// rows x SK k plus the same k range of the <= 16 activation rows: SK = 1024
// (2 KB runs per row) up to 4 tokens, 512 at 16 tokens and on the one-token
// word-flag path (stage_k below).  Gate+up layers stream gate and up rows as
// alternating stages, or at 16 tokens as paired stages of 16 + 16 rows x 256
// k that share one activation slice (RingShape::PAIR).  Each 1 KB load
// instruction writes 1 KB of LDS contiguously, lane by lane; a lane picks the
// global 16-byte chunk whose swizzled home is its own LDS slot (chunk c of
// row r lives at c ^ (r & 15) within its group of 16), so loads stay fully
// coalesced and the MFMA fragment reads of 16 rows are bank-conflict free
// (for the four 16-lane cycles of a ds_read_b128 on gfx950, as measured: see
// the GEMM's LDS layout note).  The streaming loop is rolled (a ring slot is
// a runtime offset), so its few dozen instructions stay in the instruction
// cache.
//
// Roles.  A block has 8 worker waves and 1 control wave.  Every worker issues
// the same number of loads per stage, so a wave waits only for the stage it
// is about to consume, and one workgroup barrier per stage publishes it to all
// waves.  Worker w owns 1/8 of every stage's k range and runs
// v_mfma_f32_16x16x32_bf16 with the weight rows as the row operand and the
// activation rows as the column operand (zero for columns >= M).  The control
// wave never loads a weight: it sums the 8 partial tiles in a fixed order
// (bitwise deterministic), applies the epilogue (bias + activation, or
// act(g) * u for a gated layer) in fp32 with one rounding to bf16, stores the
// result and, in the two-layer form, publishes h and awaits every block's h
// (at one token as epoch-tagged words, below).
//
// One stream, two layers.  Layer-2 stages follow layer-1 stages in the same
// ring, so layer-2 weights are in flight while the block waits for h.  The
// control wave stores h with device-coherent stores, waits for its own
// stores, raises the block's flag, then reads every block's flag (one hop, no
// L2 write-back or invalidate).  Workers read h only after that: the h slices
// of the layer-2 stages issued before the barrier are requested empty and
// re-requested after it, so no h line is touched before every block has
// published and no stale copy can sit in an L2.  Every wait is bounded; a wait
// that gives up is counted in the workspace and the kernel still exits.
//
// Out-of-range rows, the k tail and stages past the end of the stream are
// masked by buffer offsets (loads past the end return 0 without a memory
// access), never by a branch around a load; fragments past K are also zeroed
// at the read, so stale LDS never meets the MFMA.
#include <unistd.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <mutex>

#include "common.h"
#include "kernels.h"
#include "exchange.h"
#include "lds_dma.h"

namespace fmlp {

namespace {

constexpr int kWorkers = 8;                    // streaming + MFMA waves
constexpr int kThreads = (kWorkers + 1) * 64;  // + the control wave
constexpr uint32_t kSpinLimit = 1u << 20;      // bounded waits
constexpr int kLdsBudget = 160 * 1024;
// Ring depth cap: R - 1 = 3 stages in flight per CU (51 KB at one token)
// already keep HBM at its streaming rate; a deeper ring only lengthens the
// per-CU request queue, which the latency-critical h exchange then waits
// behind (measured: 4 slots 17.8 us against 8 slots 19.4 us per 4096^3
// two-layer forward at one token, equal elsewhere).
constexpr int kRingMax = 4;
// One token and a hidden size up to kLLMaxH: h is published as 8-byte words
// (two bf16 and the call's epoch), gathered by every block straight into LDS.
constexpr int kLLMaxH = 4096;

// k per stage for a class of M.  A stage is 16 weight rows x SK k; longer
// runs per row stream faster from HBM (a probe of this pattern: 2 KB per row
// about 15-20 % above 1 KB), so up to 4 tokens a stage takes 1024 k.  At 16
// tokens the activation slice of such a stage would crowd the ring out of LDS,
// and with the word-flag publish (LL) bigger stages put more bytes in the
// CU's queue ahead of the h exchange (measured slower at one token, 4096^3).
template <int MC, bool LL>
constexpr int stage_k() { return (MC <= 4 && !LL) ? 1024 : 512; }

// Activation rows held per stage (a class of M) and the ring depth it leaves.
// Gate+up stages: up to 4 tokens the gate and up rows alternate as stages of
// 16 rows x SK (longer runs per row).  At 16 tokens that would load each
// activation slice twice, so a stage is paired: 16 gate + 16 up rows x 256 k
// sharing one activation slice (PAIR).
template <int MC, bool DUAL1, bool LL>
struct RingShape {
  static constexpr bool PAIR = DUAL1 && MC > 4;
  static constexpr int SK = stage_k<MC, LL>();
  static constexpr int SK1 = PAIR ? 256 : SK;                      // k per layer-1 stage
  static constexpr int CPR = SK / 8;                              // 16-byte chunks per stage row
  static constexpr int kWChunks = 16 * CPR;                       // weight chunks per stage
  static constexpr int NL = kWChunks / 64 / kWorkers;             // weight loads per wave and stage
  static constexpr int NT = CPR / 32;                             // MFMA k-steps per wave and stage
  static constexpr int kXChunks = MC * CPR;                       // MC activation rows
  static constexpr int kSlotBytes = (kWChunks + kXChunks) * 16;
  static constexpr int kRedBytes = (DUAL1 ? 2 : 1) * kWorkers * 64 * 16;
  static constexpr int kFixed = kRedBytes + 2 * 64 * 4 + 1024     // partials, bias, sink
                                + (LL ? kLLMaxH * 2 : 0);          // h gathered for layer 2
  static constexpr int kFit = (kLdsBudget - kFixed) / kSlotBytes;
  static constexpr int R = kFit < kRingMax ? kFit : kRingMax;
  static constexpr int XI = (MC * CPR / 64 + kWorkers - 1) / kWorkers;  // activation loads per wave and stage
  static constexpr int kLoads = NL + XI;                          // loads per wave and stage
  static_assert(R >= 3 && R * kSlotBytes + kFixed <= kLdsBudget, "ring does not fit");
  static_assert(kLoads * (R - 2) < 64, "vmcnt range");
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// c ? a : b on values: a conditional between two lvalues would select their
// addresses and load, which keeps the operands in private memory.
template <class T>
__device__ __forceinline__ T pick(bool c, T a, T b) { return c ? a : b; }

// A kernel-argument field as an opaque scalar register value: a later choice
// between two layers' fields then stays a register select.
template <class T>
__device__ __forceinline__ T in_sgpr(T v) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32/64-bit scalars");
  asm volatile("" : "+s"(v));
  return v;
}

// position of 16-byte chunk c of stage row r inside the row (an involution)
__device__ __forceinline__ int swz(int c, int r) { return (c & ~15) | ((c ^ r) & 15); }

struct Stream {
  int nt[2];        // tiles this block owns in each layer
  int S[2];         // stages per tile in each layer
  int first2;       // end of the layer-1 stages (= nt[0] * S[0])
  int total;        // stages of this block
};

// A gate+up layer streams its gate and up rows as alternating stages of the
// same k range (gate at even stage indices, up at odd), so every stage is 16
// rows of one matrix.
template <bool DUAL1, bool TWO, int SK, bool PAIR>
__device__ __forceinline__ Stream make_stream(const GemvLayer& L1, const GemvLayer& L2) {
  Stream st;
  const int G = gridDim.x, b = blockIdx.x;
  const int tiles1 = (int)((L1.N + 15) / 16);
  constexpr int SK1 = PAIR ? 256 : SK;
  st.nt[0] = b < tiles1 ? (tiles1 - 1 - b) / G + 1 : 0;
  st.S[0] = (int)((L1.K + SK1 - 1) / SK1) * ((DUAL1 && !PAIR) ? 2 : 1);
  st.first2 = st.nt[0] * st.S[0];
  if (TWO) {
    const int tiles2 = (int)((L2.N + 15) / 16);
    st.nt[1] = b < tiles2 ? (tiles2 - 1 - b) / G + 1 : 0;
    st.S[1] = (int)((L2.K + SK - 1) / SK);
  } else {
    st.nt[1] = 0;
    st.S[1] = 1;
  }
  st.total = st.first2 + st.nt[1] * st.S[1];
  return st;
}

// The block's stage stream as a run of segments: each layer-1 tile (S[0]
// stages), each layer-2 tile (S[1] stages), then an endless run of empty
// stages.  A walker moves one stage at a time; only entering a new segment
// costs more than a decrement.
enum SegKind : int { SEG_L1 = 0, SEG_L2 = 1, SEG_END = 2 };

struct Seg {
  int kind;
  int tile;   // tile index within its layer
  int left;   // stages left in the segment, the current one included
};

template <bool TWO>
__device__ __forceinline__ void seg_next(const Stream& st, Seg& q) {
  if (q.kind == SEG_L1 && q.tile + 1 < st.nt[0]) {
    ++q.tile;
    q.left = st.S[0];
  } else if (q.kind == SEG_L1 && TWO && st.nt[1] > 0) {
    q.kind = SEG_L2;
    q.tile = 0;
    q.left = st.S[1];
  } else if (q.kind == SEG_L2 && q.tile + 1 < st.nt[1]) {
    ++q.tile;
    q.left = st.S[1];
  } else {
    q.kind = SEG_END;
    q.left = 1 << 30;
  }
}

template <bool TWO>
__device__ __forceinline__ Seg seg_first(const Stream& st) {
  Seg q{SEG_L1, 0, st.S[0]};
  if (st.nt[0] == 0) {   // no layer-1 tile
    q.tile = st.nt[0];
    seg_next<TWO>(st, q);
  }
  return q;
}

// ACT: the activation of the first (or only) layer, fixed at compile time (a
// runtime choice inlines every activation into the epilogue); a second layer
// has none.
template <bool DUAL1, bool TWO, int MC, bool LL, int ACT>
__global__ void __launch_bounds__(kThreads)
decode_kernel(GemvLayer L1, GemvLayer L2, int M, uint32_t* sync, uint32_t salt) {
  static_assert(!LL || (TWO && MC == 1), "word-flag publish: two layers, one token");
  using RS = RingShape<MC, DUAL1, LL>;
  constexpr int R = RS::R, XI = RS::XI;
  constexpr int SK = RS::SK, CPR = RS::CPR, NL = RS::NL, NT = RS::NT;
  constexpr bool PAIR = RS::PAIR;
  constexpr int SK1 = RS::SK1;
  constexpr int kWChunks = RS::kWChunks;
  constexpr int kSets = DUAL1 ? 2 : 1;
  constexpr uint32_t kSlot = (uint32_t)RS::kSlotBytes;
  __shared__ u32x4_t ring[R][kWChunks + RS::kXChunks];
  __shared__ float4 red[kSets][kWorkers * 64];
  __shared__ uint32_t bias_lds[2][64];         // bias of the control wave's current and next tile
  __shared__ u32x4_t sink[64];                 // destination of activation loads with no row
  __shared__ u32x4_t h_lds[LL ? kLLMaxH / 8 : 1];   // layer-2 input, gathered (LL)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in an SGPR
  const int li = lane & 15, lg = lane >> 4;
  const Stream st = make_stream<DUAL1, TWO, SK, PAIR>(L1, L2);
  const int G = (int)gridDim.x, blk = (int)blockIdx.x;

  // This call's epoch (what its h words and flags carry): the generation it
  // advances the workspace to, mixed with the launch's salt, so that neither a
  // header zeroed again nor a replay of the same launch repeats an epoch that
  // words or flags of an earlier call still hold.
  uint32_t gen_next = 0, target = 0;
  if (TWO) {
    gen_next = ld_coherent(sync + kSyncGenWord) + 1u;
    target = epoch_of(gen_next, salt);
  }

  if (wave < kWorkers) {
    // ======================= worker waves =====================================
    const int w = wave;
    const int K0 = in_sgpr((int)L1.K), K1 = in_sgpr((int)L2.K);
    const int N0 = in_sgpr((int)L1.N), N1 = in_sgpr((int)L2.N);
    const uint64_t Wa0 = in_sgpr(reinterpret_cast<uint64_t>(L1.W0));
    const uint64_t Wb0 = in_sgpr(reinterpret_cast<uint64_t>(DUAL1 ? L1.W1 : L1.W0));
    const uint64_t Wa1 = in_sgpr(reinterpret_cast<uint64_t>(L2.W0));
    const uint64_t X0 = in_sgpr(reinterpret_cast<uint64_t>(L1.x));
    const uint64_t X1 = in_sgpr(reinterpret_cast<uint64_t>(L2.x));

    // Per-lane byte offsets, fixed for a whole layer.  A stage row holds
    // CPR chunks of 16 bytes (a paired layer-1 stage: 32 rows of 32 chunks,
    // gate rows 0-15 and up rows 16-31).  Load instruction g of a stage
    // (1 KB) fills LDS chunks 64 g .. 64 g + 63; lane l's chunk P = 64 g + l
    // is position P % CPR of stage row P / CPR, and the lane fetches the
    // global chunk c whose swizzled home is that position (chunk c of row r
    // lives at swz(c, r): an involution).  Weight load i of wave w is
    // instruction NL * w + i; activation load j of wave w is instruction
    // w + 8 * j of the activation area (MC rows).  The *t variants are for a
    // tile's last k range, whose chunks past K go out of range.
    uint32_t woff[2][NL], wofft[2][NL], xoff[2][XI], xofft[2][XI];
    bool xhas[2][XI];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const bool pr = PAIR && p == 0;
      const int cpr = pr ? 32 : CPR;
      const int sk = pr ? SK1 : SK;
      const int K = pick(p != 0, K1, K0);
      const int klast = ((K + sk - 1) / sk - 1) * sk;   // k0 of a tile's last k range
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int P = 64 * (NL * w + i) + lane;
        const int r = P / cpr;
        const int c = swz(P % cpr, r);
        woff[p][i] = (uint32_t)((r & 15) * K + c * 8) * 2u;   // paired: gate/up rows by wave
        wofft[p][i] = klast + c * 8 < K ? woff[p][i] : kOutOfRange;
      }
#pragma unroll
      for (int j = 0; j < XI; ++j) {
        const int P = 64 * (w + 8 * j) + lane;
        const int r = P / cpr;
        const int c = swz(P % cpr, r);
        xhas[p][j] = w + 8 * j < MC * cpr / 64;
        xoff[p][j] = (uint32_t)(r * K + c * 8) * 2u;
        xofft[p][j] = klast + c * 8 < K ? xoff[p][j] : kOutOfRange;
      }
    }
    // LDS: this wave's weight pieces of a slot, its activation pieces (or
    // the sink), and this lane's fragment positions
    const uint32_t ring0 = lds_addr(&ring[0][0]);
    const uint32_t lds_w = ring0 + (uint32_t)(NL * w) * 1024u;
    const uint32_t sink_lds = lds_addr(&sink[0]);
    uint32_t lds_x[2][XI];   // [layer][load]: offset inside a slot, or the sink (bit 31)
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int j = 0; j < XI; ++j)
        lds_x[p][j] = xhas[p][j] ? (uint32_t)(kWChunks * 16 + (w + 8 * j) * 1024) : 0x80000000u;
    // wave w owns chunks [w * CPR / 8, (w + 1) * CPR / 8) of every stage row:
    // NT k-steps of 4 chunks (32 k), lane group lg taking chunk 4 t + lg
    uint32_t apos[NT], bpos[NT];
    int kc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      kc[t] = w * (CPR / 8) + 4 * t + lg;
      apos[t] = (uint32_t)(li * CPR + swz(kc[t], li)) * 16u;
      bpos[t] = (uint32_t)(kWChunks * 16) + (uint32_t)((li < MC ? li : 0) * CPR + swz(kc[t], li)) * 16u;
    }
    // paired layer-1 stage: one k-step, chunk 4 w + lg of gate row li and up row 16 + li
    const int kcp = 4 * w + lg;
    const uint32_t gpos = (uint32_t)(li * 32 + swz(kcp, li)) * 16u;
    const uint32_t upos = gpos + 16u * 32u * 16u;
    const uint32_t bppos = (uint32_t)(kWChunks * 16) + (uint32_t)((li < MC ? li : 0) * 32 + swz(kcp, li)) * 16u;
    const bool bcol = li < M;    // this lane's activation row exists
    bool aok[2][NT];             // weight fragment inside K in a tile's last k range
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const bool pr = PAIR && p == 0;
      const int sk = pr ? SK1 : SK;
      const int K = pick(p != 0, K1, K0);
      const int klast = ((K + sk - 1) / sk - 1) * sk;
#pragma unroll
      for (int t = 0; t < NT; ++t) aok[p][t] = klast + (pr ? kcp : kc[t]) * 8 < K;
    }

    f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};

    // ---- issue side: the next stage to load ---------------------------------
    Seg is = seg_first<TWO>(st);
    bool h_ok = false;         // h may be read (the barrier has passed)
    uint64_t wtile[2] = {0, 0};   // this tile's first row: gate (or only) and up weights
    uint32_t wrows = 0;        // this tile's weight bytes per matrix (rows * K * 2)
    uint32_t xall = 0;         // activation bytes (M * K * 2), 0 when nothing is to be read
    uint64_t xb = 0;
    bool i_l2 = false, i_tailk = false, i_dual = false;
    int i_nk = 1;              // k ranges per tile
    int i_sk = SK;             // k per stage in this segment
    auto issue_enter = [&]() {   // issue state for the segment `is` begins
      i_l2 = TWO && is.kind == SEG_L2;
      const bool real = is.kind != SEG_END;
      i_dual = DUAL1 && !PAIR && is.kind == SEG_L1;
      const int K = pick(i_l2, K1, K0);
      const int N = pick(i_l2, N1, N0);
      const int sk = (PAIR && !i_l2) ? SK1 : SK;
      i_tailk = K % sk != 0;
      i_nk = (K + sk - 1) / sk;
      i_sk = sk;
      const int n0 = (blk + is.tile * G) * 16;
      const int left = N - n0;
      const int rows = real ? (left < 16 ? left : 16) : 0;
      const uint64_t off = rows ? (uint64_t)((int64_t)n0 * K) * 2u : 0u;
      wtile[0] = pick(i_l2, Wa1, Wa0) + off;
      wtile[1] = Wb0 + off;
      wrows = (uint32_t)(rows * K) * 2u;
      xb = pick(i_l2, X1, X0);
      xall = real && !(LL && i_l2) ? (uint32_t)(M * K) * 2u : 0u;   // LL: layer 2 reads h_lds
    };
    // all loads of one stage into ring slot `slot`: NL weight pieces, then XI
    // activation pieces (h only once the barrier has passed)
    int inext = 0;             // stream index of the next stage to load
    auto issue = [&](uint32_t slot) {
      if (inext >= st.total) return;   // past the end: nothing to load
      ++inext;
      if (is.left == 0) {
        seg_next<TWO>(st, is);
        issue_enter();
      }
      const int q = is.kind == SEG_END ? 0 : pick(i_l2, st.S[1], st.S[0]) - is.left;   // stage within the tile
      // gate (0) or up (1): alternating stages, or (paired) waves 4-7 load up rows
      const int sel = i_dual ? (q & 1) : ((PAIR && !i_l2 && w >= 4) ? 1 : 0);
      const int kidx = i_dual ? (q >> 1) : q;                   // k range
      const bool tail = i_tailk && kidx == i_nk - 1;
      const uint32_t koff = (uint32_t)(kidx * i_sk) * 2u;
      const i32x4_t wd = make_desc(pick(sel != 0, wtile[1], wtile[0]) + koff, wrows > koff ? wrows - koff : 0u);
      const uint32_t slot_lds = ring0 + slot * kSlot;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const uint32_t off = pick(tail, pick(i_l2, wofft[1][i], wofft[0][i]), pick(i_l2, woff[1][i], woff[0][i]));
        asm_load_lds_stream(wd, lds_w + slot * kSlot + (uint32_t)i * 1024u, off);
      }
      const uint32_t xrec = (i_l2 && !h_ok) ? 0u : (xall > koff ? xall - koff : 0u);
      const i32x4_t xd = make_desc(xb + koff, xrec);
#pragma unroll
      for (int j = 0; j < XI; ++j) {
        const uint32_t off = pick(tail, pick(i_l2, xofft[1][j], xofft[0][j]), pick(i_l2, xoff[1][j], xoff[0][j]));
        const uint32_t where = pick(i_l2, lds_x[1][j], lds_x[0][j]);
        asm_load_lds(xd, (where & 0x80000000u) ? sink_lds : slot_lds + where, off);
      }
      --is.left;
    };

    // ---- consume side: the stage in ring slot `slot` ------------------------
    // Once every stage has been requested (stream index >= quiet_from), the
    // first step waits for all loads and meets the other waves once; the
    // rest read resident stages with no wait and no barrier, except that a
    // tile ending there meets the control wave before writing its partials.
    Seg cs = seg_first<TWO>(st);
    const int quiet_from = st.total - (R - 1) > 0 ? st.total - (R - 1) : 0;
    int gidx = 0;              // stream index of the stage being consumed
    auto step = [&](uint32_t slot) {
      if (cs.left == 0) seg_next<TWO>(st, cs);
      const bool quiet = gidx > quiet_from;   // no barrier at the head of this step
      if (gidx < quiet_from) {
        wait_vm<RS::kLoads * (R - 2)>();   // this wave's loads of the stage
        lds_barrier();                     // the stage is in LDS for every wave; the slot before it is free
        issue(slot == 0 ? R - 1 : slot - 1);
      } else if (gidx == quiet_from) {
        wait_vm<0>();                      // every load of the stream has landed ...
        lds_barrier();                     // ... for every wave
      }
      ++gidx;
      const bool real = cs.kind != SEG_END;
      const bool last = real && cs.left == 1;
      if (real && PAIR && cs.kind == SEG_L1) {
        // paired stage: gate and up fragments share the activation fragment
        const bool tail = last && (K0 % SK1 != 0);
        const char* sp = reinterpret_cast<const char*>(&ring[0][0]) + slot * kSlot;
        u32x4_t g = *reinterpret_cast<const u32x4_t*>(sp + gpos);
        u32x4_t u = *reinterpret_cast<const u32x4_t*>(sp + upos);
        u32x4_t x = zero4();
        if (bcol) x = *reinterpret_cast<const u32x4_t*>(sp + bppos);
        if (tail && !aok[0][0]) g = u = zero4();
        acc0 = mfma_16x16x32(g, x, acc0);
        acc1 = mfma_16x16x32(u, x, acc1);
      } else if (real) {
        const bool c_l2 = TWO && cs.kind == SEG_L2;
        const bool dual = DUAL1 && !c_l2;
        const int K = pick(c_l2, K1, K0);
        const int q = pick(c_l2, st.S[1], st.S[0]) - cs.left;
        const bool up = dual && (q & 1);
        const int kidx = dual ? (q >> 1) : q;
        const bool tail = (K % SK != 0) && kidx == (K + SK - 1) / SK - 1;
        const char* sp = reinterpret_cast<const char*>(&ring[0][0]) + slot * kSlot;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          u32x4_t a = *reinterpret_cast<const u32x4_t*>(sp + apos[t]);
          u32x4_t x = zero4();               // lanes of absent rows read nothing
          if (LL && c_l2) {
            const int k = kidx * SK + kc[t] * 8;
            if (bcol && k < K1) x = h_lds[k >> 3];
          } else if (bcol) {
            x = *reinterpret_cast<const u32x4_t*>(sp + bpos[t]);
          }
          if (tail && !pick(c_l2, aok[1][t], aok[0][t])) a = zero4();
          if (up)
            acc1 = mfma_16x16x32(a, x, acc1);
          else
            acc0 = mfma_16x16x32(a, x, acc0);
        }
      }
      if (last) {                        // partial tile of this wave -> control wave
        // with no barrier since the previous tile's end, the control wave may
        // still be reading that tile's partials: meet it first
        if (quiet) lds_barrier();
        red[0][w * 64 + lane] = make_float4(acc0[0], acc0[1], acc0[2], acc0[3]);
        if (DUAL1 && cs.kind == SEG_L1)
          red[kSets - 1][w * 64 + lane] = make_float4(acc1[0], acc1[1], acc1[2], acc1[3]);
        acc0 = f32x4_t{0.f, 0.f, 0.f, 0.f};
        acc1 = f32x4_t{0.f, 0.f, 0.f, 0.f};
        lds_barrier();
      }
      --cs.left;
    };

    // prologue: stages 0 .. R-2.  It runs before any barrier: touching h here
    // would also pull unpublished lines into an L2.
    issue_enter();
    for (uint32_t d = 0; d < (uint32_t)R - 1; ++d) issue(d);
    uint32_t slot = 0;
    for (int g = 0; g < st.first2; ++g) {
      step(slot);
      slot = slot + 1 == (uint32_t)R ? 0 : slot + 1;
    }
    if (LL && st.total > st.first2) {
      lds_barrier();   // the control wave has gathered h into h_lds
      for (int g = st.first2; g < st.total; ++g) {
        step(slot);
        slot = slot + 1 == (uint32_t)R ? 0 : slot + 1;
      }
    } else if (TWO && st.total > st.first2) {
      lds_barrier();   // the control wave has seen every block's h
      h_ok = true;
      // h slices of the layer-2 stages already in flight, re-requested now
      // that h is complete (in order after the empty ones: they land later)
      const uint32_t hrec = (uint32_t)(M * K1) * 2u;
      const bool htailk = K1 % SK != 0;
      Seg hq = cs;
      uint32_t hs = slot;
      for (int e = 0; e < R - 1; ++e) {
        if (hq.left == 0) seg_next<TWO>(st, hq);
        if (hq.kind != SEG_L2) break;      // the rest was never requested
        const bool in = true;
        const uint32_t k0b = (uint32_t)((st.S[1] - hq.left) * SK) * 2u;   // k0 of the stage, in bytes
        const i32x4_t hd = make_desc(X1 + (in ? k0b : 0u), in ? hrec - k0b : 0u);
        const bool tail = in && htailk && hq.left == 1;
#pragma unroll
        for (int j = 0; j < XI; ++j) {
          const uint32_t where = lds_x[1][j];
          asm_load_lds(hd, (where & 0x80000000u) ? sink_lds : ring0 + hs * kSlot + where,
                       pick(tail, xofft[1][j], xoff[1][j]));
        }
        --hq.left;
        hs = hs + 1 == (uint32_t)R ? 0 : hs + 1;
      }
      wait_vm<0>();    // the steps below then wait as in steady state (their
      lds_barrier();   // counts only over-estimate what is younger); h is in LDS for every wave
      for (int g = st.first2; g < st.total; ++g) {
        step(slot);
        slot = slot + 1 == (uint32_t)R ? 0 : slot + 1;
      }
    }
    wait_vm<0>();      // nothing is left in flight into LDS at exit
    return;
  }

  // ========================= control wave =====================================
  const uint16_t* const bias1 = in_sgpr(L1.bias);
  const uint16_t* const bias2 = in_sgpr(L2.bias);
  uint16_t* const y1 = in_sgpr(L1.y);
  uint16_t* const y2 = in_sgpr(L2.y);
  const int N1 = in_sgpr((int)L1.N), N2 = in_sgpr((int)L2.N);
  // The bias of the next tile is requested one tile ahead, straight into LDS.
  auto ctrl_fetch_bias = [&](int bslot, const Seg& q) {
    const bool l2 = TWO && q.kind == SEG_L2;
    const bool real = q.kind != SEG_END;
    const uint16_t* bias = pick(l2, bias2, bias1);
    const int N = pick(l2, N2, N1);
    const int n = (blk + q.tile * G) * 16 + 2 * lane;   // 2 outputs per lane
    const bool want = real && bias != nullptr;          // wave-uniform
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(pick<const uint16_t*>(want, bias, y1), want ? (uint32_t)N * 2u : 0u);
    const uint32_t off = (lane < 8 && n < N) ? (uint32_t)n * 2u : kOutOfRange;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)&bias_lds[bslot][0], 4, off, 0, 0, 0);
  };
  auto ctrl_epilogue = [&](const Seg& q, int bslot) {
    const bool l2 = TWO && q.kind == SEG_L2;
    const bool dual = DUAL1 && q.kind == SEG_L1;
    const int N = pick(l2, N2, N1);
    uint16_t* const y = pick(l2, y2, y1);
    float g[4] = {0.f, 0.f, 0.f, 0.f}, u[4] = {0.f, 0.f, 0.f, 0.f};
    for (int v = 0; v < kWorkers; ++v) {
      const float4 t = red[0][v * 64 + lane];
      g[0] += t.x; g[1] += t.y; g[2] += t.z; g[3] += t.w;
      if (dual) {
        const float4 r = red[kSets - 1][v * 64 + lane];
        u[0] += r.x; u[1] += r.y; u[2] += r.z; u[3] += r.w;
      }
    }
    wait_vm<0>();   // this tile's bias (and the control wave's earlier stores)
    const uint2 bias = *reinterpret_cast<const uint2*>(&bias_lds[bslot][2 * lg]);
    const int m = li;
    const int n = (blk + q.tile * G) * 16 + 4 * lg;   // this lane's 4 consecutive outputs
    if (m < M && n < N) {
      float v[4];
      const float b[4] = {bf16_lo(bias.x), bf16_hi(bias.x), bf16_lo(bias.y), bf16_hi(bias.y)};
#pragma unroll
      for (int r = 0; r < 4; ++r)
        v[r] = dual ? act_of<ACT>(g[r]) * u[r] : (l2 ? g[r] + b[r] : act_of<ACT>(g[r] + b[r]));   // b = 0 without a bias
      const uint32_t lo = pack_bf16x2(v[0], v[1]), hi = pack_bf16x2(v[2], v[3]);
      if (LL && !l2) {    // h as two words {bf16 pair, epoch}: the data is its own flag
        const __amdgpu_buffer_rsrc_t rh = make_rsrc(y, (uint32_t)N * 4u);
        st_coherent_b128(rh, (uint32_t)n * 4u, u32x4_t{lo, target, hi, target});
      } else if (TWO && !l2) {   // h: read by every block after the barrier
        const __amdgpu_buffer_rsrc_t rh = make_rsrc(y, (uint32_t)(M * N) * 2u);
        st_coherent_b64(rh, (uint32_t)(m * N + n) * 2u, u32x2_t{lo, hi});
      } else {                   // the output: a plain buffer store (vmcnt only)
        const __amdgpu_buffer_rsrc_t ry = make_rsrc(y, (uint32_t)(M * N) * 2u);
        __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{lo, hi}, ry, (uint32_t)(m * N + n) * 2u, 0, 0);
      }
    }
  };
  // this block's h is complete once the control wave's stores are: raise the flag
  auto ctrl_arrive = [&]() {
    wait_vm<0>();
    if (lane == 0) st_coherent(sync + kSyncFlagWord0 + blk, target);
  };
  // Every control wave reads every block's flag: 4 flags per lane in one
  // 16-byte device-coherent load, so one round trip checks 256 blocks.
  auto ctrl_wait_all = [&]() {
    // whole 16-byte groups (the header's flag area holds a multiple of 4
    // words); flags past the grid are ignored below
    const __amdgpu_buffer_rsrc_t rf = make_rsrc(sync + kSyncFlagWord0, ((uint32_t)G + 3u) / 4u * 16u);
    for (int b0 = 0; b0 < G; b0 += 256) {
      const int f0 = b0 + 4 * lane;
      for (uint32_t spins = 0;; ++spins) {
        const u32x4_t v = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rf, (uint32_t)f0 * 4u, 0, 16 /* sc1 */));
        bool ok = true;
#pragma unroll
        for (int j = 0; j < 4; ++j) ok = ok && (f0 + j >= G || v[j] == target);
        if (__builtin_amdgcn_ballot_w64(!ok) == 0) break;
        if (spins >= kSpinLimit) {
          if (lane == 0)
            __hip_atomic_fetch_add(sync + kSyncTimeoutWord, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    if (blk == 0 && lane == 0) st_coherent(sync + kSyncGenWord, gen_next);
  };
  // LL: read every word of h with device-coherent loads until each carries
  // this call's epoch (one pass when everything has landed: all of a lane's
  // loads are in flight together), and keep the bf16 pairs in h_lds.  Every
  // block owns a layer-1 tile (the launch guarantees it), so once block 0
  // has seen every word, every block has read the generation: only then does
  // it move forward.
  auto ctrl_gather_words = [&]() {
    if constexpr (LL) {
      constexpr int kPer = kLLMaxH / 4 / 64;   // 16-byte pieces (two words) per lane
      const int pieces = (int)(L2.K / 4);       // K of layer 2 = hidden size
      const __amdgpu_buffer_rsrc_t rw = make_rsrc(L2.x, (uint32_t)pieces * 16u);
      uint32_t pend = 0;
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (lane + 64 * i < pieces) pend |= 1u << i;
      for (uint32_t spins = 0;; ++spins) {
        u32x4_t v[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i)
          if (pend & (1u << i))
            v[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                   rw, (uint32_t)(lane + 64 * i) * 16u, 0, 16 /* sc1 */));
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
          if ((pend & (1u << i)) && v[i][1] == target && v[i][3] == target) {
            uint32_t* hw = reinterpret_cast<uint32_t*>(&h_lds[0]) + 2 * (lane + 64 * i);
            hw[0] = v[i][0];
            hw[1] = v[i][2];
            pend &= ~(1u << i);
          }
        }
        if (__builtin_amdgcn_ballot_w64(pend != 0) == 0) break;
        if (spins >= kSpinLimit) {
          if (lane == 0)
            __hip_atomic_fetch_add(sync + kSyncTimeoutWord, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      if (blk == 0 && lane == 0) st_coherent(sync + kSyncGenWord, gen_next);
    }
  };
  // the control wave meets the workers at each of their barriers
  Seg cs = seg_first<TWO>(st);
  Seg bq = cs;                // the tile whose bias is requested next
  int bslot = 0;
  ctrl_fetch_bias(0, bq);
  const int quiet_from = st.total - (R - 1) > 0 ? st.total - (R - 1) : 0;
  int gidx = 0;
  auto ctrl_step = [&]() {
    if (cs.left == 0) seg_next<TWO>(st, cs);
    const bool quiet = gidx > quiet_from;
    if (!quiet) lds_barrier();
    ++gidx;
    if (cs.kind != SEG_END && cs.left == 1) {
      if (quiet) lds_barrier();      // the previous epilogue is done with the partials
      lds_barrier();                 // the workers' partial tiles are in LDS
      const Seg q = cs;
      seg_next<TWO>(st, bq);         // request the next tile's bias
      ctrl_epilogue(q, bslot);
      ctrl_fetch_bias(bslot ^ 1, bq);
      bslot ^= 1;
      if (TWO && !LL && q.kind == SEG_L1 && q.tile == st.nt[0] - 1) ctrl_arrive();
    }
    --cs.left;
  };

  if (TWO && !LL && st.first2 == 0) ctrl_arrive();   // no layer-1 tile: nothing to publish
  for (int g = 0; g < st.first2; ++g) ctrl_step();
  if (LL && st.total > st.first2) {
    ctrl_gather_words();             // every block's h, word by word, into h_lds
    lds_barrier();
    for (int g = st.first2; g < st.total; ++g) ctrl_step();
  } else if (TWO && st.total > st.first2) {
    ctrl_wait_all();                 // entering layer 2: every block's h is complete
    lds_barrier();
    lds_barrier();                   // the workers' h slices are in LDS
    for (int g = st.first2; g < st.total; ++g) ctrl_step();
  }
  wait_vm<0>();
}

struct Occ {
  bool probed = false;
  bool ok = false;
  int cus = 0;
  int per_cu = 0;   // blocks per CU (the LDS ring admits one)
};

std::mutex g_occ_mu;
Occ g_occ[64];

// Residency of the decode kernels on the current device, queried once per
// device with the runtime's occupancy calculator (for the largest-LDS
// variant) and cached.
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
    const bool ok = hipOccupancyMaxActiveBlocksPerMultiprocessor(
                        &o.per_cu, reinterpret_cast<const void*>(&decode_kernel<true, true, 1, false, ACT_GELU_TANH>), kThreads,
                        0) == hipSuccess;
    o.ok = ok && o.cus > 0 && o.per_cu > 0;
  }
  return o;
}

uint32_t mix32(uint32_t v) {
  v ^= v >> 16;
  v *= 0x85EBCA6Bu;
  v ^= v >> 13;
  v *= 0xC2B2AE35u;
  v ^= v >> 16;
  return v;
}

}  // namespace

// A salt per launch: a process-wide counter through a bijective mix, seeded
// from the clock and the process id, so every launch of this process gets a
// different value (for 2^32 launches) and other processes most likely others.
uint32_t next_launch_salt() {
  static const uint32_t seed = mix32((uint32_t)std::chrono::steady_clock::now().time_since_epoch().count() ^
                                     (uint32_t)getpid() * 0x9E3779B1u);
  static std::atomic<uint32_t> counter{0};
  return mix32(seed ^ counter.fetch_add(1u, std::memory_order_relaxed) * 0x27D4EB2Du);
}

namespace {

// One kernel variant on `grid` blocks.  The two-layer form waits for every
// block at its barrier; the grid is capped at one block per CU (the LDS ring
// admits one), so on an otherwise idle device every block is resident.  A
// cooperative launch also refuses a grid that cannot be co-resident, but it
// was measured to add about 18 us to every call (the 4096^3 two-layer forward
// at one token: 36 us against 18 us), twice the whole forward's roofline
// time; so it is opt-in, the plain launch is the default, and a barrier wait
// that gives up is counted in the workspace header for the caller to check.
// With `coop` the launch is cooperative (opt-in, fmlp_set_cooperative_decode):
// the runtime refuses a grid that cannot be resident at once instead of
// letting the barrier time out.
template <bool DUAL1, bool TWO, int MC, bool LL, int ACT>
hipError_t launch_act(unsigned grid, const GemvLayer& L1, const GemvLayer& L2, int M, uint32_t* sync,
                      hipStream_t s, bool coop) {
  uint32_t salt = TWO ? next_launch_salt() : 0u;
  if (coop) {
    GemvLayer a = L1, b = L2;
    void* args[] = {&a, &b, &M, &sync, &salt};
    return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&decode_kernel<DUAL1, TWO, MC, LL, ACT>),
                                      dim3(grid), dim3(kThreads), args, 0, s);
  }
  hipLaunchKernelGGL((decode_kernel<DUAL1, TWO, MC, LL, ACT>), dim3(grid), dim3(kThreads), 0, s, L1, L2, M, sync,
                     salt);
  return hipGetLastError();
}
template <bool DUAL1, bool TWO, int MC, bool LL>
hipError_t launch_variant(unsigned grid, const GemvLayer& L1, const GemvLayer& L2, int M, uint32_t* sync,
                          hipStream_t s, bool coop) {
  switch (L1.act) {
    case ACT_NONE: return launch_act<DUAL1, TWO, MC, LL, ACT_NONE>(grid, L1, L2, M, sync, s, coop);
    case ACT_GELU_ERF: return launch_act<DUAL1, TWO, MC, LL, ACT_GELU_ERF>(grid, L1, L2, M, sync, s, coop);
    case ACT_GELU_TANH: return launch_act<DUAL1, TWO, MC, LL, ACT_GELU_TANH>(grid, L1, L2, M, sync, s, coop);
    case ACT_RELU: return launch_act<DUAL1, TWO, MC, LL, ACT_RELU>(grid, L1, L2, M, sync, s, coop);
    case ACT_SILU: return launch_act<DUAL1, TWO, MC, LL, ACT_SILU>(grid, L1, L2, M, sync, s, coop);
    default: return hipErrorInvalidValue;
  }
}

// activation-row class of M: the rows an LDS stage holds
template <bool DUAL1, bool TWO>
hipError_t launch_mc(unsigned grid, const GemvLayer& L1, const GemvLayer& L2, int M, uint32_t* sync,
                     hipStream_t s, bool coop = false) {
  // word-flag publish of h: one token, h fits h_lds, and every block owns a
  // layer-1 tile (so every block writes words before block 0 can see them all)
  const bool ll = TWO && M == 1 && L2.K <= kLLMaxH && (int64_t)grid <= (L1.N + 15) / 16;
  if (M <= 1 && ll) return launch_variant<DUAL1, TWO, 1, TWO>(grid, L1, L2, M, sync, s, coop);
  if (M <= 1) return launch_variant<DUAL1, TWO, 1, false>(grid, L1, L2, M, sync, s, coop);
  if (M <= 4) return launch_variant<DUAL1, TWO, 4, false>(grid, L1, L2, M, sync, s, coop);
  return launch_variant<DUAL1, TWO, 16, false>(grid, L1, L2, M, sync, s, coop);
}

}  // namespace

hipError_t launch_gemv(const GemvLayer& L, int M, hipStream_t s) {
  if (L.geglu) return hipErrorInvalidValue;   // gate+up runs only in the two-layer kernel
  const int64_t tiles = (L.N + 15) / 16;
  if (tiles <= 0 || M <= 0) return hipSuccess;
  if (M > 16) return hipErrorInvalidValue;
  const Occ o = occ();
  if (!o.ok) return hipErrorInvalidDevice;
  // one layer has no barrier: cap the grid at one resident round of blocks
  const unsigned grid = (unsigned)std::min<int64_t>(tiles, (int64_t)o.cus * o.per_cu);
  return launch_mc<false, false>(grid, L, L, M, nullptr, s);
}

hipError_t launch_gemv2_persistent(const GemvLayer& L1, const GemvLayer& L2, int M, uint32_t* sync,
                                   hipStream_t s, bool cooperative) {
  if (M <= 0) return hipSuccess;
  if (M > 16 || L2.act != ACT_NONE) return hipErrorInvalidValue;   // the second layer has no activation
  const Occ o = occ();
  if (!o.ok) return hipErrorInvalidDevice;
  const int64_t tiles1 = (L1.N + 15) / 16, tiles2 = (L2.N + 15) / 16;
  // every block must be resident at once: the barrier waits for all of them.
  // One block per CU, whatever the occupancy query allows: residency of a
  // second block per CU is not something the barrier may depend on.
  const int64_t cap = std::min<int64_t>((int64_t)o.cus, kDecodeMaxBlocks);
  const unsigned grid = (unsigned)std::min<int64_t>(cap, std::max(tiles1, tiles2));
  if (grid == 0) return hipSuccess;
  if (L1.geglu) return launch_mc<true, true>(grid, L1, L2, M, sync, s, cooperative);
  return launch_mc<false, true>(grid, L1, L2, M, sync, s, cooperative);
}

}  // namespace fmlp
