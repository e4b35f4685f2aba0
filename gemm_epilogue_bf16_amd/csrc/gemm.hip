// Large-token bf16 GEMM with a register epilogue, for gfx950.
//
//   C[rows, N] = epilogue(A[rows, K] . B[N, K]^T),  fp32 accumulate
//
// Both operands are K-contiguous (the weight is read as stored, [out, in]):
// "Profiling in PyTorch (Part 2): From nn.Linear to a Fused MLP", section
// "Where did the transpose go? Kernel layouts and pre-ops".  The epilogue runs
// on the fp32 accumulator in registers and writes only the final tile
// (section "Why are there no separate mul and add kernels?"):
//   GEMM_OUT_BF16        bias add + activation (none / exact GELU / tanh GELU /
//                        ReLU / SiLU)
//   GEMM_OUT_GEGLU       gate and up projections share every A tile; the block
//                        holds matching g and u accumulators and writes only
//                        m = act(g) * u, act = tanh GELU for GeGLU (section
//                        "The fused Triton kernel": the intermediate never
//                        makes an HBM round trip) or another gate activation
//   GEMM_OUT_F32_SCALED  fp32 output scaled per row (expert combine weights;
//                        no scale: 1), optionally split over K into parts
//                        that each write their own copy (summed in order by
//                        the caller: the MoE combine, or the backward's
//                        weight gradients)
//   GEMM_OUT_DACT        backward of a Linear + activation: the forward GEMM
//                        recomputes z = x W^T + b in registers and writes only
//                        dz = dy * act'(z)
//   GEMM_OUT_DGLU        backward of the gated block: the gate+up GEMM
//                        recomputes g and u and, with the incoming dm, writes
//                        m = act(g) * u, dg = dm * u * act'(g) and du = dm * act(g)
//
// Structure: a block computes a BM x BN tile with WAVES_M x WAVES_N waves
// (256 x 256 with 8 waves of 128 x 64 for large inputs: two waves per SIMD,
// so one issues MFMAs while the other waits, each with 128 fp32 accumulators
// in AGPRs).  K advances in stages of BK (64 for the
// large tile: 128-byte LDS rows, two ring slots; 32 for the small one:
// 64-byte rows, four slots).  Stages stream from memory straight into the
// LDS ring with buffer loads that write LDS, R - 1 stages ahead of the MFMAs
// and with no register staging; each wave waits only for its own loads of
// the stage it is about to read, and one workgroup barrier per stage
// publishes the stage and frees the slot the next loads go to.  Each 1 KB
// load instruction fills 1 KB of LDS in lane order, a lane fetching the
// global chunk whose permuted home (swz_a, swz_b below) is its own LDS
// position, so the 16-byte fragment reads are bank-conflict free.  Rows past
// the tile's end and chunks past K are requested out of range and arrive as
// zeros.  The loop is issued in a fixed order: MFMAs of a k-step run from
// registers while the next k-step's fragments are read from LDS and the next
// stage's loads are issued, one such instruction after each MFMA.
// v_mfma_f32_16x16x32_bf16 is fed with the weight as the row operand and the
// activation as the column operand; the weight rows of a fragment pair are
// interleaved so each lane ends with 8 consecutive output columns of one row,
// stored as one 16-byte write.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "common.h"
#include "kernels.h"
#include "lds_dma.h"

namespace fmlp {

namespace {

// LDS layout.  A stage holds BK k of every tile row: rows of BK * 2 bytes
// (CH = BK / 8 chunks of 16 B).  A ds_read_b128 takes four LDS cycles of 16
// lanes (measured on gfx950): the cycle of lane l is set by its half-wave
// (l >> 5) and the parity of its quad index bits ((l >> 2) & 7), and within
// a cycle the lanes must hit distinct 16-byte bank groups (unit index mod 16).
// A fragment read puts k group lg = l >> 4 and row offset li = l & 15 on each
// lane, so a cycle holds two k groups, each with half of the row offsets.
// Chunk c of row r sits at slot c ^ swz(r), with one permutation for
// activation fragments (16 consecutive rows) and one for weight fragments
// (rows interleaved in groups of 4: 8*(l/4) + (l%4)), chosen so every cycle
// of both kinds of read is conflict free:
//   64-byte rows:  q = bits 2-3 (activation) or 3-4 (weight) of r, slot
//                  permutation {0, 2, 3, 1}[q] (the plain q pairs lanes);
//   128-byte rows: bits 1-3 of r (activation), bits 1, 3, 4 (weight).
template <int CH>
__host__ __device__ constexpr int swz_a(int r) {
  if constexpr (CH == 4) return (0x78 >> (2 * ((r >> 2) & 3))) & 3;
  else return (r >> 1) & 7;
}
template <int CH>
__host__ __device__ constexpr int swz_b(int r) {
  if constexpr (CH == 4) return (0x78 >> (2 * ((r >> 3) & 3))) & 3;
  else return ((r >> 1) & 1) | ((r >> 2) & 6);
}

// Weight fragment f of a wave covers tile rows w_lane_row + w_delta(f), with
// the rows permuted so that every lane ends up holding runs of 8 consecutive
// output columns (one 16-byte store each):
//   16x16x32 (M32 = false): the rows of a fragment pair interleave, so lane
//     group g holds columns 8g .. 8g+7 of the pair's 32 columns;
//   32x32x16 (M32 = true): fragment row i (= lane % 32) reads weight row
//     rho(i) = 16 (i >> 4) + 8 ((i >> 2) & 1) + 4 ((i >> 3) & 1) + (i & 3), so
//     the 16 results of lane half h (accumulator registers 0-7 and 8-15) are
//     columns 8h .. 8h+7 and 16+8h .. 16+8h+7 of the fragment's 32.
// With two weight sets, fragments [0, FN/2) read the first and [FN/2, FN) the
// second.
__host__ __device__ constexpr int rho32(int i) {
  return 16 * (i >> 4) + 8 * ((i >> 2) & 1) + 4 * ((i >> 3) & 1) + (i & 3);
}
__host__ __device__ constexpr int w_delta(int f, int FN, int BN, bool dual, bool m32) {
  const int half = FN / 2;
  const int set = dual ? f / half : 0;
  const int fl = dual ? f % half : f;
  return set * (BN / 2) + (m32 ? fl * 32 : (fl >> 1) * 32 + 4 * (fl & 1));
}
__host__ __device__ constexpr int w_lane_row(int wn, int li, int TN, bool dual, bool m32) {
  return wn * (dual ? TN / 2 : TN) + (m32 ? rho32(li) : 8 * (li >> 2) + (li & 3));
}
// The swizzles read only bits 1-4 of a row, so every fragment of a wave has
// the same chunk permutation as its first one and its LDS address is the
// first one's plus a constant.  Checked exhaustively at compile time.
template <int CH, int TM, int TN, int FM, int FN, int BN, int WAVES_M, int WAVES_N, bool DUAL, bool M32>
constexpr bool fragment_swizzle_is_uniform() {
  constexpr int MR = M32 ? 32 : 16;
  for (int li = 0; li < MR; ++li) {
    for (int wm = 0; wm < WAVES_M; ++wm)
      for (int f = 0; f < FM; ++f)
        if (swz_a<CH>(wm * TM + f * MR + li) != swz_a<CH>(wm * TM + li)) return false;
    for (int wn = 0; wn < WAVES_N; ++wn) {
      const int r0 = w_lane_row(wn, li, TN, DUAL, M32);
      for (int f = 0; f < FN; ++f)
        if (swz_b<CH>(r0 + w_delta(f, FN, BN, DUAL, M32)) != swz_b<CH>(r0)) return false;
    }
  }
  return true;
}
// The 32-row fragment reads are bank-conflict free under the measured model
// of a ds_read_b128 (four 16-lane cycles; cycle of lane l: l >> 5 and the
// parity of the bits of (l >> 2) & 7; units within a cycle distinct mod 16):
// checked exhaustively at compile time for both operands' row maps.
template <int CH>
constexpr bool m32_reads_conflict_free(bool weights) {
  if (CH != 8) return false;
  for (int c0 = 0; c0 < CH; c0 += 2)
    for (int base = 0; base < 256; base += 32)
      for (int cyc = 0; cyc < 4; ++cyc) {
        bool seen[16] = {};
        for (int l = 0; l < 64; ++l) {
          const int q = (l >> 2) & 7;
          const int par = (q ^ (q >> 1) ^ (q >> 2)) & 1;
          if (((l >> 5) << 1 | par) != cyc) continue;
          const int i = l & 31;
          const int r = base + (weights ? rho32(i) : i);
          const int c = c0 + (l >> 5);
          const int slot = c ^ (weights ? swz_b<CH>(r) : swz_a<CH>(r));
          const int unit = (r * CH + slot) & 15;
          if (seen[unit]) return false;
          seen[unit] = true;
        }
      }
  return true;
}
static_assert(m32_reads_conflict_free<8>(false) && m32_reads_conflict_free<8>(true),
              "32-row fragment reads of 128-byte rows");

// k-major operand tiles (the backward's contractions over the rows of both
// operands, read without a transpose copy).  A stage holds 64 k-rows of the
// tile's 256 columns: rows of 512 bytes, 32 chunks of 16 B, chunk c of row k
// at slot c ^ kswz(k).  A fragment (16 columns x 32 k) is two transposing
// reads (ds_read_b64_tr_b16): within each 16-lane group, lane 4 r + q points
// at 4 consecutive columns of k-row kbase + r, and lane j gets column group
// j / 4, element j % 4 of all four rows, i.e. 4 consecutive k of one column;
// kbase = 32 ks + 8 (lane / 16) and + 4 give a lane the 8 consecutive k of the
// 16x16x32 operand, in the order the row-major reads give them.  kswz moves
// chunk bits 1-3: the 8 k-rows of a half-wave's read land on 8 distinct chunk
// pairs (an activation fragment's 16 consecutive columns are one chunk pair
// per row), so those reads are conflict free.  A weight fragment keeps the
// pair permutation that gives each lane runs of 8 output columns (16-byte
// stores): its 16 columns are 4 half chunks, all in the same half, so its
// reads take two passes.  (Weight columns kept in order instead, 4-column
// runs with 8-byte stores and conflict-free reads, measured 1 % slower on the
// large backward.)
__host__ __device__ constexpr int kswz(int k) { return 2 * ((k & 7) ^ (((k >> 3) & 1) << 2)); }
typedef short v4i16_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4_t lds_read_tr_pair(uint32_t addr0, uint32_t addr1) {
  typedef __attribute__((address_space(3))) v4i16_t lds_v4;
  const v4i16_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(uintptr_t)addr0);
  const v4i16_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(uintptr_t)addr1);
  u32x4_t r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(a, a, 0, 1));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(a, a, 2, 3));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(b, b, 0, 1));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(b, b, 2, 3));
  return r;
}

// The main loop interleaves MFMAs with loads and LDS reads in a fixed order.
// Instruction selection moves an MFMA builtin freely (it touches no memory),
// so the loop issues them as volatile asm, which keeps its place among the
// other volatile asm (loads into LDS, waits, barriers); the accumulator is
// pinned in AGPRs and updated in place.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void mfma_ordered(f32x4_t& acc, const u32x4_t& a, const u32x4_t& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b) : "memory");
}
// D[32x32] += A[32x16] B[16x32]: lane l supplies row (l % 32) of A and column
// (l % 32) of B, each as 8 consecutive k of k-group l / 32, and receives
// column l % 32 of D, rows 8 (r / 4) + 4 (l / 32) + r % 4 in register r.
__device__ __forceinline__ void mfma_ordered(f32x16_t& acc, const u32x4_t& a, const u32x4_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b) : "memory");
}
// A copy of v the compiler cannot see through: what is computed from it
// stays where it is written instead of being hoisted out of the tile loop and
// kept live (in registers the main loop needs) across it.
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}
// materialise a value in AGPRs at this point of the instruction stream
__device__ __forceinline__ void pin_agpr(f32x4_t& acc) { asm volatile("" : "+a"(acc)); }
__device__ __forceinline__ void pin_agpr(f32x16_t& acc) { asm volatile("" : "+a"(acc)); }
// the same, also ordered after every memory access before it: reads of the
// accumulator cannot be hoisted above the preceding output stores (which
// would have every accumulator copied to VGPRs at once)
__device__ __forceinline__ void pin_agpr_ordered(f32x4_t& acc) { asm volatile("" : "+a"(acc) : : "memory"); }
__device__ __forceinline__ void pin_agpr_ordered(f32x16_t& acc) { asm volatile("" : "+a"(acc) : : "memory"); }
// wait states between the last MFMA of the loop and the first read of its
// accumulators by ordinary code (the hazard check cannot see into asm)
__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }
#pragma clang diagnostic pop

// GACT: the gate activation of a gated (GEMM_OUT_GEGLU, GEMM_OUT_DGLU) kernel,
// or the activation of a GEMM_OUT_DACT kernel, fixed per kernel so each
// carries one epilogue: with several epilogue copies behind a
// runtime switch, the register allocator copied accumulator lanes out of AGPRs
// inside the main loop, a few wait states after the (asm) MFMA that wrote them.
// M32: the wave tile runs on v_mfma_f32_32x32x16_bf16 (32x32 fragments, 16 k
// per MFMA) instead of v_mfma_f32_16x16x32_bf16: half the MFMA instructions
// and half the operand register reads per flop, the same LDS bytes.
// KM: bit 0 A, bit 1 B stored k-major (GemmParams::kmajor).
template <int BM, int BN, int WAVES_M, int WAVES_N, int BK, int R, int OUT, bool GATHER, bool GROUPED,
          int GACT = ACT_NONE, bool M32 = false, int KM = 0>
__global__ void __launch_bounds__(WAVES_M * WAVES_N * 64)
gemm_bf16_kernel(GemmParams p) {
  constexpr int NW = WAVES_M * WAVES_N;
  constexpr int TM = BM / WAVES_M;   // wave tile rows (activation rows)
  constexpr int TN = BN / WAVES_N;   // wave tile width in B-tile rows
  constexpr int MR = M32 ? 32 : 16;  // rows (and columns) of one MFMA's output
  constexpr int KSTEP = M32 ? 16 : 32;   // k per MFMA
  typedef typename std::conditional<M32, f32x16_t, f32x4_t>::type acc_t;
  constexpr int NACC = M32 ? 16 : 4;     // accumulator registers per MFMA tile
  constexpr int FM = TM / MR;
  constexpr int FN = TN / MR;
  constexpr bool DUAL = (OUT == GEMM_OUT_GEGLU || OUT == GEMM_OUT_DGLU);
  constexpr int HALF = FN / 2;       // DUAL: gate fragments [0,HALF), up [HALF,FN)
  constexpr int CH = BK / 8;         // 16-byte chunks per LDS row
  constexpr int KS = BK / KSTEP;     // MFMA k-steps per stage
  constexpr int RPI = 64 / CH;       // rows filled by one 1 KB load instruction
  constexpr int A_INS = BM / (RPI * NW);   // load instructions per wave and stage
  constexpr int B_INS = BN / (RPI * NW);
  constexpr int LOADS = A_INS + B_INS;
  constexpr int SLOT = (BM + BN) * CH;     // 16-byte chunks per ring slot
  constexpr int OUT_N = DUAL ? BN / 2 : BN;   // output columns per block
  static_assert(BK == 32 || BK == 64, "stage depth");
  static_assert(A_INS >= 1 && B_INS >= 1 && BM % (RPI * NW) == 0 && BN % (RPI * NW) == 0, "load mapping");
  static_assert(!DUAL || (BN / 2) % (RPI * NW) == 0, "a load instruction stays in one weight set");
  static_assert(TM % MR == 0 && TN % MR == 0 && FM % 2 == 0, "wave tile");
  static_assert(M32 || (DUAL ? (HALF % 2 == 0) : (FN % 2 == 0)), "fragment pairs");
  static_assert(!DUAL || HALF >= 1, "gate and up fragments");
  static_assert(KS == 1 || KS % 2 == 0, "k-steps per stage");
  static_assert(R >= 2 && LOADS * (R - 2) < 64, "ring depth");
  constexpr bool KMA = (KM & 1) != 0, KMB = (KM & 2) != 0;
  static_assert(KM == 0 || (!DUAL && !GATHER && !GROUPED && !M32 && BM == 256 && BN == 256 && BK == 64 &&
                            WAVES_M == 2 && WAVES_N == 4),
                "k-major operands: 256x256 tiles of 8 waves, 16x16x32 MFMAs, one weight set");

  __shared__ u32x4_t ring[R * SLOT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;

  const int64_t K = p.K, N = p.N;
  const int Kc = (int)K;                       // < 2^22
  const int li = lane & (MR - 1);   // fragment row (weight) / column (activation)
  const int lg = lane / MR;         // k group: 8 consecutive k

  // ---- this block's tiles ----------------------------------------------------
  // The grid is persistent (at most one block per CU).  Logical tiles (in
  // grouped order) are split into one contiguous range per XCD, in
  // proportion to its blocks, and the blocks of an XCD take its range
  // round-robin, so at any time the blocks sharing an L2 work on
  // neighbouring tiles.  Grouped mode counts only the tiles that exist.
  const int tiles_m = GROUPED ? p.tile_off[p.groups] : p.tiles_m;
  // split-K (fp32 output only): every tile appears KSP times, once per part
  // of the K range, each writing its own output copy
  constexpr bool SPLITK = OUT == GEMM_OUT_F32_SCALED;
  const int KSP = SPLITK && p.ksplit > 1 ? p.ksplit : 1;
  const int total = tiles_m * p.tiles_n * KSP;
  const int G = gridDim.x, bid = blockIdx.x;
  const int xcd = bid % kNumXcd, xj = bid / kNumXcd;
  auto blocks_before = [&](int x) {   // blocks on XCDs 0 .. x-1
    const int q = G / kNumXcd, r = G % kNumXcd;
    return x * q + min(x, r);
  };
  const int nbx = blocks_before(xcd + 1) - blocks_before(xcd);
  const int t_lo = (int)((int64_t)total * blocks_before(xcd) / G);
  const int t_hi = (int)((int64_t)total * blocks_before(xcd + 1) / G);
  const int nmine = xj < t_hi - t_lo ? (t_hi - t_lo - xj + nbx - 1) / nbx : 0;
  if (nmine == 0) return;   // block-uniform: no barrier has been reached

  struct Tile {
    int64_t row_begin, row_end, n0;
    int kp;   // part of the K range (split-K)
    const uint16_t* b0;
    const uint16_t* b1;
  };
  auto tile_at = [&](int i) -> Tile {   // this block's i-th tile
    int tm, tn;
    const int lt = t_lo + xj + i * nbx;
    grouped_tile(lt / KSP, tiles_m, p.tiles_n, p.group_m, tm, tn);
    Tile t;
    t.b0 = p.B0;
    t.b1 = p.B1;
    if constexpr (GROUPED) {
      int lo = 0, hi = p.groups;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (p.tile_off[mid] <= tm) lo = mid; else hi = mid;
      }
      t.row_begin = (int64_t)p.group_off[lo] + (int64_t)(tm - p.tile_off[lo]) * BM;
      t.row_end = min(t.row_begin + BM, (int64_t)p.group_off[lo + 1]);
      t.b0 += (int64_t)lo * p.strideB;
      if constexpr (DUAL) t.b1 += (int64_t)lo * p.strideB;
    } else {
      t.row_begin = (int64_t)tm * BM;
      t.row_end = min(t.row_begin + BM, p.M);
    }
    t.n0 = (int64_t)tn * OUT_N;
    t.kp = lt % KSP;
    return t;
  };

  // ---- load descriptors and per-lane offsets (of the tile being issued) -----
  // Load instruction i of this wave fills tile rows RPI * (i * NW + wave) +
  // lane / CH; the lane's LDS position in its row is lane % CH and it fetches
  // the chunk that belongs there.  RPI * NW is a multiple of 32 and the
  // swizzles read bits 1-4 of a row, so that chunk is the same for every load
  // instruction of the lane.  Byte spans fit 31 bits (checked by the caller),
  // so 32-bit offsets suffice and kOutOfRange is past every descriptor's end.
  // A tile's descriptors end at its last valid row, so rows past the end of
  // the activation or weight arrive as zeros with no per-lane test; gathered
  // rows past a group's end get an out-of-range offset once per tile.  Only
  // chunks past K need a mask per stage: they would read the next row.
  static_assert((RPI * NW) % 32 == 0, "one chunk permutation per lane");
  const int ra = RPI * wave + lane / CH;      // tile row of the lane's load 0 (activation and weight)
  const int a_k = 8 * ((lane % CH) ^ swz_a<CH>(ra));   // k of the lane's chunk in a stage
  const int b_k = 8 * ((lane % CH) ^ swz_b<CH>(ra));
  const uint32_t lda2 = (uint32_t)p.lda * 2u;
  const uint32_t K2 = (uint32_t)Kc * 2u;
  // offsets of the lane's load 0 within a tile (load i adds a constant number of rows)
  const uint32_t a_lane = (uint32_t)ra * lda2 + (uint32_t)a_k * 2u;
  const uint32_t b_lane = (uint32_t)ra * K2 + (uint32_t)b_k * 2u;
  // k-major: load i of this wave fills k-rows 16 i + 2 wave + lane / 32 of
  // the stage (2 rows of 512 B per instruction), the lane's slot lane % 32 of
  // its row holding chunk slot ^ kswz(row) (kswz reads row bits 0-3, the same
  // for every i)
  const int kr0 = 2 * wave + (lane >> 5);
  const uint32_t km_chunk = (uint32_t)(((lane & 31) ^ kswz(kr0)) * 16);
  const uint32_t ldb2 = (uint32_t)(KMB ? p.ldb : 0) * 2u;
  const uint32_t a_lane_km = (uint32_t)kr0 * lda2 + km_chunk;
  const uint32_t b_lane_km = (uint32_t)kr0 * ldb2 + km_chunk;
  i32x4_t da, db0, db1;
  uint32_t a_gat[GATHER ? A_INS : 1];   // gather: the lane's source-row offsets in this tile
  auto issue_tile = [&](const Tile& t) {
    const int a_rows_here = (int)(t.row_end - t.row_begin);
    // k-major descriptors end at the operand's last element ((K - 1) ld +
    // width): columns past the width read the next row's (in the operand, and
    // only into accumulators that are never stored), past the last row zeros
    if constexpr (KMA)   // the tile's rows are columns row_begin .. of A [K, lda], p.M wide
      da = make_desc(reinterpret_cast<uint64_t>(p.A + t.row_begin),
                     (uint32_t)((((int64_t)Kc - 1) * p.lda + p.M - t.row_begin) * 2));
    else
      da = GATHER ? make_desc(reinterpret_cast<uint64_t>(p.A), (uint32_t)(p.a_src_rows * p.lda * 2))
                  : make_desc(reinterpret_cast<uint64_t>(p.A + t.row_begin * p.lda), (uint32_t)a_rows_here * lda2);
    const int n_here = (int)min((int64_t)OUT_N, N - t.n0);   // weight rows of each set in this tile
    if constexpr (KMB) {   // the tile's columns are columns n0 .. of B0 [K0, ldb] (and B1 [K - K0, ldb]), N wide
      const int64_t k0rows = p.kb_split > 0 ? p.kb_split : (int64_t)Kc;
      db0 = make_desc(reinterpret_cast<uint64_t>(t.b0 + t.n0), (uint32_t)(((k0rows - 1) * p.ldb + N - t.n0) * 2));
      db1 = p.kb_split > 0 ? make_desc(reinterpret_cast<uint64_t>(t.b1 + t.n0),
                                       (uint32_t)((((int64_t)Kc - p.kb_split - 1) * p.ldb + N - t.n0) * 2))
                           : db0;
    } else {
      db0 = make_desc(reinterpret_cast<uint64_t>(t.b0 + t.n0 * K), (uint32_t)n_here * K2);
      db1 = DUAL ? make_desc(reinterpret_cast<uint64_t>(t.b1 + t.n0 * K), (uint32_t)n_here * K2) : db0;
    }
    if constexpr (GATHER) {
      const int rt = RPI * wave + opaque(lane) / CH;
      const int ak = 8 * ((opaque(lane) % CH) ^ swz_a<CH>(rt));
#pragma unroll
      for (int i = 0; i < A_INS; ++i) {
        const int r = RPI * i * NW + rt;
        const uint32_t src = (uint32_t)p.a_rows[t.row_begin + min(r, a_rows_here - 1)];
        a_gat[i] = r < a_rows_here ? src * lda2 + (uint32_t)ak * 2u : kOutOfRange;
      }
    }
  };
  static_assert(RPI * NW <= BN / 2, "weight row of a load");
  const uint32_t ring_lds = lds_addr(&ring[0]) + (uint32_t)wave * 1024u;
  // Stages of one tile; the loop runs k-steps in pairs (the fragment register
  // sets alternate), so with one k-step per stage an odd count gets one
  // all-zero stage more, which adds nothing.  The block's stream is its
  // tiles' stages back to back: stream stage q is stage q % NS of tile q / NS.
  // Split over K: part kp of a tile takes stages [kp nk / KSP, (kp + 1) nk /
  // KSP) (shares that differ by at most one stage; with one k-step per stage
  // the caller keeps every share even).
  const int nk = (Kc + BK - 1) / BK;
  const int NS = KSP > 1 ? nk / KSP : (KS % 2 == 0 ? nk : (nk + 1) & ~1);   // stages of an unsplit tile
  auto part_first = [&](int kp) { return (int)((int64_t)kp * nk / KSP); };
  auto part_stages = [&](int kp) { return SPLITK ? part_first(kp + 1) - part_first(kp) : NS; };
  int iss_kp = 0;   // K part of the tile whose stages are being issued
  int iss_ns = NS;  // and its stage count
  {
    const Tile t0 = tile_at(0);
    issue_tile(t0);
    iss_kp = t0.kp;
    iss_ns = part_stages(t0.kp);
  }

  // How this wave loads the next stage of its stream (stages are issued once
  // each, in order): the lane's chunks are out of range past K (the k tail,
  // the padding stage) and for stages past the end of the stream; kb is the
  // byte offset of the stage's k range (the loads' soffset).  The first stage
  // of a tile switches the descriptors and offsets over to it.
  int iss_t = 0, iss_s = 0;   // tile and stage within the tile of the next stage issued
  struct StageIssue {
    bool a_in, b_in;
    uint32_t kb;      // soffset of the stage's k range: row-major operands
    uint32_t kb_a;    // A's (its rows past a k-major stage's first)
    uint32_t kb_b;    // B's
    int k0;           // the stage's first k (K when past the end)
    bool b1;          // k-major B: the stage's rows come from B1
  };
  auto stage_begin = [&]() -> StageIssue {
    const bool live = iss_t < nmine;   // block-uniform
    if (live && iss_s == 0 && iss_t > 0) {
      const Tile nt = tile_at(iss_t);
      issue_tile(nt);
      iss_kp = nt.kp;
      iss_ns = part_stages(nt.kp);
    }
    const int ks0 = __builtin_amdgcn_readfirstlane(live ? (SPLITK ? part_first(iss_kp) : 0) + iss_s : 0);   // stage index within K
    const int k0 = live ? ks0 * BK : Kc;
    const uint32_t kb = (uint32_t)ks0 * (BK * 2);
    const bool b1 = KMB && p.kb_split > 0 && k0 >= p.kb_split;   // block-uniform
    const StageIssue st{k0 + a_k < Kc, k0 + b_k < Kc, kb,
                        KMA ? (uint32_t)(ks0 * BK) * lda2 : kb,
                        KMB ? (uint32_t)(ks0 * BK - (b1 ? (int)p.kb_split : 0)) * ldb2 : kb, k0, b1};
    if (++iss_s == iss_ns) {
      iss_s = 0;
      ++iss_t;
    }
    return st;
  };
  // load i (of LOADS) of a stage into the slot at LDS byte address `base`
  auto dma = [&](int i, uint32_t base, const StageIssue& st) {
    if (i < A_INS) {
      if constexpr (KMA) {   // k-rows past K load zeros
        const uint32_t off = a_lane_km + (uint32_t)(16 * i) * lda2;
        asm_load_lds(da, base + (uint32_t)(i * NW) * 1024u, st.k0 + kr0 + 16 * i < Kc ? off : kOutOfRange, st.kb_a);
      } else {
        const uint32_t off = GATHER ? a_gat[GATHER ? i : 0] : a_lane + (uint32_t)(RPI * i * NW) * lda2;
        asm_load_lds(da, base + (uint32_t)(i * NW) * 1024u, st.a_in ? off : kOutOfRange, st.kb_a);
      }
    } else {
      const int b = i - A_INS;
      if constexpr (KMB) {
        const uint32_t off = b_lane_km + (uint32_t)(16 * b) * ldb2;
        asm_load_lds(st.b1 ? db1 : db0, base + (uint32_t)(BM * CH * 16 + b * NW * 1024),
                     st.k0 + kr0 + 16 * b < Kc ? off : kOutOfRange, st.kb_b);
      } else {
        const bool up = DUAL && RPI * (b * NW) >= BN / 2;   // compile-time per i
        const uint32_t off = b_lane + (uint32_t)((RPI * b * NW) % (DUAL ? BN / 2 : BN)) * K2;
        asm_load_lds(up ? db1 : db0, base + (uint32_t)(BM * CH * 16 + b * NW * 1024),
                     st.b_in ? off : kOutOfRange, st.kb_b);
      }
    }
  };
  auto issue_all = [&](int slot) {
    const StageIssue st = stage_begin();
#pragma unroll
    for (int i = 0; i < LOADS; ++i) dma(i, ring_lds + (uint32_t)slot * (SLOT * 16), st);
  };
  // ---- LDS fragment addresses (16-byte units within a slot) -----------------
  // Activation fragment f: rows wm * TM + 16 f + li; weight fragment f: rows
  // w_lane_row + w_delta(f).  One base per k-step, the rest compile-time.
  static_assert(fragment_swizzle_is_uniform<CH, TM, TN, FM, FN, BN, WAVES_M, WAVES_N, DUAL, M32>(),
                "fragment addresses are affine");
  const int wr0 = w_lane_row(wn, li, TN, DUAL, M32);
  int x_idx[KS], w_idx[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int c = ks * (KSTEP / 8) + lg;
    x_idx[ks] = (wm * TM + li) * CH + (c ^ swz_a<CH>(wm * TM + li));
    w_idx[ks] = BM * CH + wr0 * CH + (c ^ swz_b<CH>(wr0));
  }

  acc_t acc[FM][FN];
  // The zeros are pinned into the accumulators here: the loop's MFMAs are
  // asm, so the hazard check cannot see them read a register that a plain
  // write set just before, and the compiler would otherwise sink each write
  // to right before its MFMA.
  auto zero_acc = [&]() {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
#pragma unroll
        for (int r = 0; r < NACC; ++r) acc[i][j][r] = 0.f;
        pin_agpr(acc[i][j]);
      }
  };
  zero_acc();

  // Fragment registers: two sets, alternating by k-step.  Read n of a k-step
  // is x0, w0 .. w(FN-1), x1 .. x(FM-1): the order its MFMAs consume them.
  constexpr int NREADS = FM + FN;
  u32x4_t xf[2][FM], wf[2][FN];
  // k-major: the lane's byte offset in the operand's region for k-step 0,
  // half 0 (k-row 8 (lane / 16) + (lane % 16) / 4) and fragment 0.  The rest
  // are compile-time: k-step 1 is 32 rows on (the swizzle reads row bits 0-3:
  // + 16384 bytes), half 1 is 4 rows on (row bit 2 set: swizzle bit 3 flips,
  // XOR 128, then + 2048), and a fragment XORs chunk bits the lane's own part
  // leaves zero (activation f: 2 f; weight f: 4 (f / 2), plus half chunk
  // f % 2).  One register per operand.
  uint32_t km_x = 0, km_w = 0;
  if constexpr (KM != 0) {
    const int kq = lane >> 4, s16 = lane & 15;
    const int row = 8 * kq + (s16 >> 2);
    km_x = (uint32_t)(row * 512 + (((wm * 16 + ((s16 & 3) >> 1)) ^ kswz(row)) << 4) + ((s16 & 1) << 3));
    km_w = (uint32_t)(BM * CH * 16 + row * 512 + (((wn * 8 + (s16 & 3)) ^ kswz(row)) << 4));
  }
  auto km_pair = [&](const u32x4_t* sl, uint32_t a0, int ks, uint32_t half) -> u32x4_t {
    const uint32_t b = lds_addr(sl) + (uint32_t)(16384 * ks) + half;
    return lds_read_tr_pair(b + a0, b + ((a0 ^ 128u) + 2048u));
  };
  auto frag_x = [&](const u32x4_t* sl, int ks, int f) -> u32x4_t {
    if constexpr (KMA) {
      return km_pair(sl, km_x ^ (uint32_t)(32 * f), ks, 0u);
    } else {
      return sl[x_idx[ks] + f * MR * CH];
    }
  };
  auto frag_w = [&](const u32x4_t* sl, int ks, int f) -> u32x4_t {
    if constexpr (KMB) {   // the pair permutation: columns 32 (f / 2) + 8 g + 4 (f % 2) .. + 3, g = 0..3
      return km_pair(sl, km_w ^ (uint32_t)(64 * (f >> 1)), ks, (uint32_t)(8 * (f & 1)));
    } else {
      return sl[w_idx[ks] + w_delta(f, FN, BN, DUAL, M32) * CH];
    }
  };
  auto frag_read = [&](int n, const u32x4_t* sl, int ks, auto set_c) {
    constexpr int set = decltype(set_c)::value;
    if (n == 0) {
      xf[set][0] = frag_x(sl, ks, 0);
    } else if (n <= FN) {
      wf[set][n - 1] = frag_w(sl, ks, n - 1);
    } else {
      xf[set][n - FN] = frag_x(sl, ks, n - FN);
    }
  };
  auto mfma_t = [&](int t, auto set_c) {   // MFMA t of a k-step: row t / FN, column t % FN
    constexpr int set = decltype(set_c)::value;
    mfma_ordered(acc[t / FN][t % FN], wf[set][t % FN], xf[set][t / FN]);
  };
  using Set0 = std::integral_constant<int, 0>;
  using Set1 = std::integral_constant<int, 1>;

  // ---- epilogue of a finished tile ------------------------------------------
  // Global-address-space accesses: a store through a generic pointer is a flat
  // store, which would also hold lgkmcnt and stall the next tile's fragment
  // reads behind the write.
  typedef __attribute__((address_space(1))) u32x4_t gu32x4_t;
  auto gst16 = [](void* ptr, const u32x4_t& v) { *(gu32x4_t*)ptr = v; };
  auto gld16 = [](const void* ptr) -> u32x4_t { return *(const gu32x4_t*)ptr; };
  // Runs of 8 consecutive output columns a lane holds for activation fragment
  // i, RUNS per weight set (the weight-row permutation above makes them
  // consecutive):
  //   16x16x32: run q is accumulator pair (2q, 2q+1), 4 values each, columns
  //             32 q + 8 lg of the wave's columns;
  //   32x32x16: run q is registers 8 (q % 2) .. +7 of accumulator q / 2,
  //             columns 32 (q / 2) + 16 (q % 2) + 8 lg.
  constexpr int SETF = DUAL ? HALF : FN;   // fragments per weight set
  constexpr int RUNS = M32 ? 2 * SETF : SETF / 2;
  auto run_col = [](int q, int lgv) { return M32 ? (q >> 1) * 32 + 16 * (q & 1) + 8 * lgv : q * 32 + 8 * lgv; };
  auto run_vals = [&](int i, int q, int set, float v[8]) {   // set 0: gate (or the only set), 1: up
    if constexpr (M32) {
      const int f = set * HALF + (q >> 1);
      pin_agpr_ordered(acc[i][f]);
#pragma unroll
      for (int r = 0; r < 8; ++r) v[r] = acc[i][f][8 * (q & 1) + r];
    } else {
      const int f0 = set * HALF + 2 * q;
      pin_agpr_ordered(acc[i][f0]);
      pin_agpr_ordered(acc[i][f0 + 1]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[r] = acc[i][f0][r];
        v[4 + r] = acc[i][f0 + 1][r];
      }
    }
  };
  // The activation is a template argument so each copy of the epilogue is
  // straight-line code (a per-element switch would branch around every value).
  auto epilogue_act = [&](const Tile& t, auto act_c) {
    constexpr int ACT = decltype(act_c)::value;
    const int el = opaque(lane);
    const int li = el & (MR - 1), lg = el / MR;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int64_t lrow = t.row_begin + wm * TM + i * MR + li;
      const bool row_ok = lrow < t.row_end;
      if constexpr (OUT == GEMM_OUT_GEGLU) {
#pragma unroll
        for (int q = 0; q < RUNS; ++q) {
          const int64_t n = t.n0 + wn * (TN / 2) + run_col(q, lg);
          float g[8], u[8], v[8];
          run_vals(i, q, 0, g);
          run_vals(i, q, 1, u);
#pragma unroll
          for (int r = 0; r < 8; ++r) v[r] = act_of<ACT>(g[r]) * u[r];
          if (row_ok && n < N) gst16(static_cast<uint16_t*>(p.C) + lrow * p.ldc + n, pack_bf16x8(v));
        }
      } else if constexpr (OUT == GEMM_OUT_DGLU) {
        // recomputed g and u with the incoming dm: m for the down projection's
        // weight gradient, dg and du for the input and gate/up weight gradients
#pragma unroll
        for (int q = 0; q < RUNS; ++q) {
          const int64_t n = t.n0 + wn * (TN / 2) + run_col(q, lg);
          float g[8], u[8];
          run_vals(i, q, 0, g);
          run_vals(i, q, 1, u);
          if (!(row_ok && n < N)) continue;
          float dm[8];
          unpack_bf16x8(gld16(p.E + lrow * p.lde + n), dm);
          float m[8], dg[8], du[8];
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            float a, da;
            act_and_grad<ACT>(g[r], a, da);
            m[r] = a * u[r];
            dg[r] = dm[r] * u[r] * da;
            du[r] = dm[r] * a;
          }
          gst16(static_cast<uint16_t*>(p.C) + lrow * p.ldc + n, pack_bf16x8(m));
          uint16_t* d2 = static_cast<uint16_t*>(p.C2) + lrow * p.ldc2 + n;
          gst16(d2, pack_bf16x8(dg));
          gst16(d2 + N, pack_bf16x8(du));
        }
      } else {
#pragma unroll
        for (int q = 0; q < RUNS; ++q) {
          const int64_t n = t.n0 + wn * TN + run_col(q, lg);
          float v[8];
          run_vals(i, q, 0, v);
          if (!(row_ok && n < N)) continue;
          if constexpr (OUT == GEMM_OUT_F32_SCALED) {
            const float sc = p.row_scale ? p.row_scale[lrow] : 1.f;
            float* dst = static_cast<float*>(p.C) + (int64_t)t.kp * p.c_kstride + lrow * p.ldc + n;
            u32x4_t lo, hi;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              lo[r] = __float_as_uint(v[r] * sc);
              hi[r] = __float_as_uint(v[4 + r] * sc);
            }
            gst16(dst, lo);
            gst16(dst + 4, hi);
          } else {
            if (p.bias) {
              float b[8];
              unpack_bf16x8(gld16(p.bias + n), b);
#pragma unroll
              for (int r = 0; r < 8; ++r) v[r] += b[r];
            }
            if constexpr (OUT == GEMM_OUT_DACT) {
              // the recomputed pre-activation z: dz = dy * act'(z)
              float dy[8];
              unpack_bf16x8(gld16(p.E + lrow * p.lde + n), dy);
#pragma unroll
              for (int r = 0; r < 8; ++r) {
                float a, da;
                act_and_grad<ACT>(v[r], a, da);
                v[r] = dy[r] * da;
              }
            } else {
#pragma unroll
              for (int r = 0; r < 8; ++r) v[r] = act_of<ACT>(v[r]);
            }
            gst16(static_cast<uint16_t*>(p.C) + lrow * p.ldc + n, pack_bf16x8(v));
          }
        }
      }
    }
  };
  auto epilogue = [&](const Tile& t) {
    mfma_drain();
    if constexpr (OUT == GEMM_OUT_GEGLU || OUT == GEMM_OUT_DGLU || OUT == GEMM_OUT_DACT) {
      epilogue_act(t, std::integral_constant<int, GACT>{});   // the (gate's) activation
    } else if constexpr (OUT == GEMM_OUT_BF16) {
      if (p.act == ACT_GELU_ERF) epilogue_act(t, std::integral_constant<int, ACT_GELU_ERF>{});
      else if (p.act == ACT_GELU_TANH) epilogue_act(t, std::integral_constant<int, ACT_GELU_TANH>{});
      else if (p.act == ACT_RELU) epilogue_act(t, std::integral_constant<int, ACT_RELU>{});
      else if (p.act == ACT_SILU) epilogue_act(t, std::integral_constant<int, ACT_SILU>{});
      else epilogue_act(t, std::integral_constant<int, ACT_NONE>{});
    } else {
      epilogue_act(t, std::integral_constant<int, ACT_NONE>{});
    }
    zero_acc();
  };

  // Prologue: stages 0 .. R-2 in flight, stage 0 published, R-1 issued.
  // Every stage up to the last one read plus R - 1 is issued (past the end
  // they load nothing), so every wait below is the same.
#pragma unroll
  for (int q = 0; q < R - 1; ++q) issue_all(q);
  wait_vm<LOADS * (R - 2)>();
  lds_barrier();
  issue_all(R - 1);
#pragma unroll
  for (int n = 0; n < NREADS; ++n) frag_read(n, ring, 0, Set0{});

  // One k-step (ks of the stage q in slot `slot`), register set CUR.
  //  * Not the stage's last k-step: its MFMAs, each followed by at most one
  //    fragment read of the next k-step (same slot) into the other set.
  //  * The last one: the first half of its MFMAs; hand-off (wait for this
  //    wave's loads of stage q + 1, then a barrier: stage q + 1 is in LDS for
  //    every wave, and every wave has finished reading `slot`); the second
  //    half, each MFMA followed by at most one instruction of the hand-off
  //    stream: the loads of stage q + R into `slot` (the first LNOW of them;
  //    the rest lead the next stage's first k-step), then the fragment reads
  //    of stage q + 1 into the other set.  The matrix core never waits for a
  //    run of memory instructions.  At the end of a tile (LAST) the fragment
  //    reads wait until the epilogue has freed its registers.  After an
  //    epilogue (whose stores count in vmcnt) the hand-off waits for every
  //    access, so no wait count depends on how loads and stores retire
  //    relative to each other.
  //  * Issue priority falls as a wave moves through a stage: 2 from the
  //    hand-off barrier to the end of the hand-off window, 1 through the next
  //    stage's first k-step, 0 up to the next barrier.  Of the two waves on a
  //    SIMD, the one behind gets the issue slots first, and the pair reaches
  //    the next barrier closer together (measured: the 8192/28672 GeGLU at
  //    4096 tokens 3 % faster, the 768/3072 one 2 %; a fixed priority per
  //    wave gained nothing).
  constexpr int NMA = (FM / 2) * FN;          // MFMAs per half k-step
  constexpr int NPRE = NMA;                   // MFMAs of the last k-step before the hand-off
  constexpr int NPOST = 2 * NMA - NPRE;
  static_assert(NPRE >= 1 && NPOST >= 1, "hand-off inside the last k-step");
  // Loads of stage q + R issued in the hand-off window.  With two k-steps per
  // stage half of them go out during the next stage's first k-step instead:
  // every wave reaches the hand-off together, and eight loads each in a
  // quarter of a stage queue behind one another in the address unit (measured
  // 3-4 % faster on the large shapes; a quarter or none in the window is
  // slower again).
  constexpr int LNOW = KS >= 2 ? LOADS / 2 : LOADS;
  StageIssue pend_st{false, false, 0};
  uint32_t pend_base = 0;
  bool pend = false;   // block-uniform: the first stage has none
  bool stored = false;   // an epilogue has stored since the last hand-off
  auto next_slot = [&](int sl) { return sl + 1 == R ? 0 : sl + 1; };
  auto kstep = [&](auto ks_c, int slot, auto cur_c, auto last_c) {
    constexpr int ks = decltype(ks_c)::value;
    constexpr int CUR = decltype(cur_c)::value;
    constexpr bool LAST = decltype(last_c)::value;
    using Nxt = std::integral_constant<int, CUR ^ 1>;
    if constexpr (ks + 1 < KS) {
      const u32x4_t* sl = ring + slot * SLOT;
      // the stage's first k-step leads with the loads deferred from the
      // hand-off window, then every k-step reads the next one's fragments
      constexpr int DEF = ks == 0 ? LOADS - LNOW : 0;
      constexpr int OPS0 = NREADS + DEF;
#pragma unroll
      for (int t = 0; t < 2 * NMA; ++t) {
        mfma_t(t, cur_c);
#pragma unroll
        for (int n = t * OPS0 / (2 * NMA); n < (t + 1) * OPS0 / (2 * NMA); ++n) {
          if (n < DEF) {
            if (pend) dma(LNOW + n, pend_base, pend_st);
          }
          else frag_read(n - DEF, sl, ks + 1, Nxt{});
        }
      }
      if constexpr (ks == 0) __builtin_amdgcn_s_setprio(0);
      return;
    }
    const StageIssue st = stage_begin();   // stage q + R
#pragma unroll
    for (int t = 0; t < NPRE; ++t) mfma_t(t, cur_c);
    if (R > 2 && stored) wait_vm<0>(); else wait_vm<LOADS * (R - 2)>();
    stored = false;
    lds_barrier();
    __builtin_amdgcn_s_setprio(2);
    const uint32_t base = ring_lds + (uint32_t)slot * (SLOT * 16);
    const u32x4_t* sl = ring + next_slot(slot) * SLOT;
    constexpr int OPS = LAST ? LNOW : LNOW + NREADS;
#pragma unroll
    for (int t = 0; t < NPOST; ++t) {
      mfma_t(NPRE + t, cur_c);
#pragma unroll
      for (int n = t * OPS / NPOST; n < (t + 1) * OPS / NPOST; ++n) {
        if (n < LNOW) dma(n, base, st);
        else frag_read(n - LNOW, sl, 0, Nxt{});
      }
    }
    __builtin_amdgcn_s_setprio(1);
    pend_st = st;
    pend_base = base;
    pend = true;
  };
  using Mid = std::false_type;
  using Last = std::true_type;
  // the end of this block's tile ti (its last k-step done): epilogue, then the
  // first fragments of the next tile, from the next slot
  auto tile_end = [&](int ti, int slot) {
    epilogue(tile_at(ti));
    stored = true;
    const u32x4_t* sl = ring + next_slot(slot) * SLOT;
#pragma unroll
    for (int n = 0; n < NREADS; ++n) frag_read(n, sl, 0, Set0{});
  };
  // every k-step of one stage (KS even: the register sets alternate within it)
  auto stage = [&](int slot, auto last_c) {
    auto step = [&](auto self, auto k_c) {
      constexpr int K = decltype(k_c)::value;
      if constexpr (K < KS) {
        kstep(k_c, slot, std::integral_constant<int, K & 1>{},
              std::integral_constant<bool, decltype(last_c)::value && K + 1 == KS>{});
        self(self, std::integral_constant<int, K + 1>{});
      }
    };
    step(step, std::integral_constant<int, 0>{});
  };
  using K0 = std::integral_constant<int, 0>;
  int slot = 0;
  for (int ti = 0; ti < nmine; ++ti) {
    const int ns = SPLITK ? part_stages(tile_at(ti).kp) : NS;
    if constexpr (KS >= 2) {
      for (int q = 0; q < ns - 1; ++q) {
        stage(slot, Mid{});
        slot = next_slot(slot);
      }
      stage(slot, Last{});
    } else {
      for (int q = 0; q < ns - 2; q += 2) {   // ns is even
        kstep(K0{}, slot, Set0{}, Mid{});
        slot = next_slot(slot);
        kstep(K0{}, slot, Set1{}, Mid{});
        slot = next_slot(slot);
      }
      kstep(K0{}, slot, Set0{}, Mid{});
      slot = next_slot(slot);
      kstep(K0{}, slot, Set1{}, Last{});
    }
    tile_end(ti, slot);
    slot = next_slot(slot);
  }
  wait_vm<0>();   // the stages issued past the end (loads of nothing) land before LDS is released
}

template <int BM, int BN, int WM, int WN, int BK, int R, int OUT, bool GATHER, bool GROUPED, int GACT,
          bool M32 = false, int KM = 0>
hipError_t launch_cfg(GemmParams p, hipStream_t s) {
  constexpr int OUT_N = (OUT == GEMM_OUT_GEGLU || OUT == GEMM_OUT_DGLU) ? BN / 2 : BN;
  if (!GROUPED) p.tiles_m = (int)((p.M + BM - 1) / BM);
  p.tiles_n = (int)((p.N + OUT_N - 1) / OUT_N);
  p.group_m = 4;
  const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n *   // grouped: an upper bound
                        ((OUT == GEMM_OUT_F32_SCALED && p.ksplit > 1) ? p.ksplit : 1);
  if (tiles <= 0) return hipSuccess;
  if (tiles > 0x7fffffff || p.cus <= 0) return hipErrorInvalidValue;
  // A 32-k stage tile consumes its stages two at a time, so it needs an even
  // stage count per tile; the parts of a split K range can be odd.
  if (OUT == GEMM_OUT_F32_SCALED && BK < 64 && p.ksplit > 1) return hipErrorInvalidValue;
  if (KM != p.kmajor) return hipErrorInvalidValue;
  if constexpr (KM != 0) {   // the byte spans of k-major operands fit the 31-bit offsets
    if ((KM & 1) && p.K * p.lda * 2 >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    if (KM & 2) {
      if (p.kb_split < 0 || p.kb_split >= p.K || p.kb_split % BK != 0) return hipErrorInvalidValue;
      if (p.kb_split > 0 && p.B1 == nullptr) return hipErrorInvalidValue;
      const int64_t rows = p.kb_split > 0 ? std::max(p.kb_split, p.K - p.kb_split) : p.K;
      if (rows * p.ldb * 2 >= (int64_t(1) << 31) || p.ldb < p.N) return hipErrorInvalidValue;
    }
  } else if (p.kb_split != 0) {
    return hipErrorInvalidValue;
  }
  // persistent: as many blocks as fit on the chip at once, each looping over
  // its tiles
  auto kernel = gemm_bf16_kernel<BM, BN, WM, WN, BK, R, OUT, GATHER, GROUPED, GACT, M32, KM>;
  static const int per_cu = [&] {
    int o = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, kernel, WM * WN * 64, 0) != hipSuccess) o = 1;
    return std::max(o, 1);
  }();
  const int64_t blocks = std::min<int64_t>(tiles, (int64_t)p.cus * per_cu);
  hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(WM * WN * 64), 0, s, p);
  return hipGetLastError();
}

// The 256x256 tile's MFMA shape (see gemm_bf16_kernel's M32).  The 32x32x16
// form halves MFMA instructions and operand register reads, but was measured
// 6 % slower on the large GeGLU (4295-4300 us against 4055-4061 us for the
// 16x16x32 form, same sources and box); 16x16x32 stays the default and the
// 32x32x16 form is built only with -DFMLP_TILE256_M32=1.
#ifndef FMLP_TILE256_M32
#define FMLP_TILE256_M32 0
#endif
constexpr bool kTile256M32 = FMLP_TILE256_M32 != 0;


template <int OUT, bool GATHER, bool GROUPED, int GACT = ACT_NONE>
hipError_t launch_tile(int tile, const GemmParams& p, hipStream_t s) {
  if constexpr ((OUT == GEMM_OUT_GEGLU || OUT == GEMM_OUT_DGLU || OUT == GEMM_OUT_DACT) && GACT == ACT_NONE) {
    // one kernel per (gate) activation
    switch (p.act) {
      case ACT_GELU_TANH: return launch_tile<OUT, GATHER, GROUPED, ACT_GELU_TANH>(tile, p, s);
      case ACT_GELU_ERF: return launch_tile<OUT, GATHER, GROUPED, ACT_GELU_ERF>(tile, p, s);
      case ACT_RELU: return launch_tile<OUT, GATHER, GROUPED, ACT_RELU>(tile, p, s);
      case ACT_SILU: return launch_tile<OUT, GATHER, GROUPED, ACT_SILU>(tile, p, s);
      case ACT_NONE: break;
      default: return hipErrorInvalidValue;
    }
  }
  if constexpr ((OUT == GEMM_OUT_BF16 || OUT == GEMM_OUT_F32_SCALED) && !GATHER && !GROUPED) {
    if (p.kmajor != 0) {   // k-major operands: 256x256 tiles only
      if (tile != TILE_256x256) return hipErrorInvalidValue;
      switch (p.kmajor) {
        case 1: return launch_cfg<256, 256, 2, 4, 64, 2, OUT, false, false, GACT, false, 1>(p, s);
        case 2: return launch_cfg<256, 256, 2, 4, 64, 2, OUT, false, false, GACT, false, 2>(p, s);
        case 3: return launch_cfg<256, 256, 2, 4, 64, 2, OUT, false, false, GACT, false, 3>(p, s);
        default: return hipErrorInvalidValue;
      }
    }
  } else {
    if (p.kmajor != 0) return hipErrorInvalidValue;
  }
  switch (tile) {
    case TILE_128x128: return launch_cfg<128, 128, 2, 2, 32, 4, OUT, GATHER, GROUPED, GACT>(p, s);
    case TILE_256x256: return launch_cfg<256, 256, 2, 4, 64, 2, OUT, GATHER, GROUPED, GACT, kTile256M32>(p, s);
    case TILE_128x192:
      // 4 ring slots of 40 KB: all 160 KB of LDS.  These shapes run about one
      // tile per CU over a long K, bound by the bytes each CU has in flight
      // (the 768/3072 GeGLU's down GEMM: 1.5 % faster forward than 3 slots)
      if constexpr (OUT == GEMM_OUT_BF16 && !GATHER && !GROUPED)
        return launch_cfg<128, 192, 4, 2, 64, 4, OUT, GATHER, GROUPED, GACT>(p, s);
      else
        return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int gemm_tile_bm(int tile) { return tile == TILE_256x256 ? 256 : 128; }
int gemm_tile_bn(int tile) { return tile == TILE_256x256 ? 256 : tile == TILE_128x192 ? 192 : 128; }

hipError_t launch_gemm(int out_kind, bool gather, bool grouped, int tile, GemmParams p,
                       hipStream_t s) {
  if (out_kind == GEMM_OUT_BF16 && !gather && !grouped) return launch_tile<GEMM_OUT_BF16, false, false>(tile, p, s);
  if (out_kind == GEMM_OUT_GEGLU && !gather && !grouped) return launch_tile<GEMM_OUT_GEGLU, false, false>(tile, p, s);
  if (out_kind == GEMM_OUT_GEGLU && gather && grouped) return launch_tile<GEMM_OUT_GEGLU, true, true>(tile, p, s);
  if (out_kind == GEMM_OUT_F32_SCALED && !gather && grouped) return launch_tile<GEMM_OUT_F32_SCALED, false, true>(tile, p, s);
  if (out_kind == GEMM_OUT_F32_SCALED && !gather && !grouped && tile == TILE_256x256)
    return launch_tile<GEMM_OUT_F32_SCALED, false, false>(tile, p, s);
  if (out_kind == GEMM_OUT_DACT && !gather && !grouped && tile != TILE_128x192)
    return launch_tile<GEMM_OUT_DACT, false, false>(tile, p, s);
  if (out_kind == GEMM_OUT_DGLU && !gather && !grouped) return launch_tile<GEMM_OUT_DGLU, false, false>(tile, p, s);
  return hipErrorInvalidValue;
}

}  // namespace fmlp
