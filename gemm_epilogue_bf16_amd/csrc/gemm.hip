// Large-token bf16 GEMM with a register epilogue, for gfx950.
//
//   C[rows, N] = epilogue(A[rows, K] . B[N, K]^T),  fp32 accumulate
//
// Both operands are K-contiguous (the weight is read as stored, [out, in]):
// "Profiling in PyTorch (Part 2): From nn.Linear to a Fused MLP", section
// "Where did the transpose go? Kernel layouts and pre-ops".  The epilogue runs
// on the fp32 accumulator in registers and writes only the final tile
// (section "Why are there no separate mul and add kernels?"):
//   GEMM_OUT_BF16        bias add + activation (none / exact GELU / tanh GELU)
//   GEMM_OUT_GEGLU       gate and up projections share every A tile; the block
//                        holds matching g and u accumulators and writes only
//                        m = gelu_tanh(g) * u (section "The fused Triton kernel":
//                        the intermediate never makes an HBM round trip)
//   GEMM_OUT_F32_SCALED  fp32 output scaled per row (expert combine weights)
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
__device__ __forceinline__ int swz_a(int r) {
  if constexpr (CH == 4) return (0x78 >> (2 * ((r >> 2) & 3))) & 3;
  else return (r >> 1) & 7;
}
template <int CH>
__device__ __forceinline__ int swz_b(int r) {
  if constexpr (CH == 4) return (0x78 >> (2 * ((r >> 3) & 3))) & 3;
  else return ((r >> 1) & 1) | ((r >> 2) & 6);
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
// wait states between the last MFMA of the loop and the first read of its
// accumulators by ordinary code (the hazard check cannot see into asm)
__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }
#pragma clang diagnostic pop

template <int BM, int BN, int WAVES_M, int WAVES_N, int BK, int R, int OUT, bool GATHER, bool GROUPED>
__global__ void __launch_bounds__(WAVES_M * WAVES_N * 64)
gemm_bf16_kernel(GemmParams p) {
  constexpr int NW = WAVES_M * WAVES_N;
  constexpr int TM = BM / WAVES_M;   // wave tile rows (activation rows)
  constexpr int TN = BN / WAVES_N;   // wave tile width in B-tile rows
  constexpr int FM = TM / 16;
  constexpr int FN = TN / 16;
  constexpr bool DUAL = (OUT == GEMM_OUT_GEGLU);
  constexpr int HALF = FN / 2;       // DUAL: gate fragments [0,HALF), up [HALF,FN)
  constexpr int CH = BK / 8;         // 16-byte chunks per LDS row
  constexpr int KS = BK / 32;        // MFMA k-steps per stage
  constexpr int RPI = 64 / CH;       // rows filled by one 1 KB load instruction
  constexpr int A_INS = BM / (RPI * NW);   // load instructions per wave and stage
  constexpr int B_INS = BN / (RPI * NW);
  constexpr int LOADS = A_INS + B_INS;
  constexpr int SLOT = (BM + BN) * CH;     // 16-byte chunks per ring slot
  constexpr int OUT_N = DUAL ? BN / 2 : BN;   // output columns per block
  static_assert(BK == 32 || BK == 64, "stage depth");
  static_assert(A_INS >= 1 && B_INS >= 1 && BM % (RPI * NW) == 0 && BN % (RPI * NW) == 0, "load mapping");
  static_assert(!DUAL || (BN / 2) % (RPI * NW) == 0, "a load instruction stays in one weight set");
  static_assert(TM % 16 == 0 && TN % 16 == 0 && FM % 2 == 0, "wave tile");
  static_assert(DUAL ? (HALF % 2 == 0) : (FN % 2 == 0), "fragment pairs");
  static_assert(R >= 2 && LOADS * (R - 2) < 64, "ring depth");

  __shared__ u32x4_t ring[R * SLOT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;

  // ---- which tile --------------------------------------------------------
  int tm, tn;
  grouped_tile(xcd_remap(blockIdx.x, gridDim.x), p.tiles_m, p.tiles_n, p.group_m, tm, tn);

  int64_t row_begin, row_end;
  const uint16_t* B0 = p.B0;
  const uint16_t* B1 = p.B1;
  if constexpr (GROUPED) {
    const int total = p.tile_off[p.groups];
    if (tm >= total) return;  // block-uniform
    int lo = 0, hi = p.groups;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.tile_off[mid] <= tm) lo = mid; else hi = mid;
    }
    row_begin = (int64_t)p.group_off[lo] + (int64_t)(tm - p.tile_off[lo]) * BM;
    row_end = min(row_begin + BM, (int64_t)p.group_off[lo + 1]);
    B0 += (int64_t)lo * p.strideB;
    if constexpr (DUAL) B1 += (int64_t)lo * p.strideB;
  } else {
    row_begin = (int64_t)tm * BM;
    row_end = min(row_begin + BM, p.M);
  }
  const int64_t n0 = (int64_t)tn * OUT_N;
  const int64_t K = p.K, N = p.N;

  // ---- load descriptors and per-lane offsets -------------------------------
  // Load instruction i of this wave fills tile rows RPI * (i * NW + wave) +
  // lane / CH; the lane's LDS position in its row is lane % CH and it fetches
  // the chunk that belongs there.  Byte spans fit 31 bits (checked by the
  // caller), so kOutOfRange is past every descriptor's end.
  const int jr = lane / CH, jp = lane % CH;
  const int64_t a_rows_here = row_end - row_begin;
  const i32x4_t da = GATHER
      ? make_desc(reinterpret_cast<uint64_t>(p.A), (uint32_t)(p.a_src_rows * p.lda * 2))
      : make_desc(reinterpret_cast<uint64_t>(p.A + row_begin * p.lda), (uint32_t)(a_rows_here * p.lda * 2));
  const int64_t n_here = min((int64_t)OUT_N, N - n0);   // weight rows of each set in this tile
  const i32x4_t db0 = make_desc(reinterpret_cast<uint64_t>(B0 + n0 * K), (uint32_t)(n_here * K * 2));
  const i32x4_t db1 = DUAL ? make_desc(reinterpret_cast<uint64_t>(B1 + n0 * K), (uint32_t)(n_here * K * 2)) : db0;
  uint32_t a_off[A_INS], b_off[B_INS];
  int a_k[A_INS], b_k[B_INS];   // k offset of the lane's chunk within a stage
#pragma unroll
  for (int i = 0; i < A_INS; ++i) {
    const int r = RPI * (i * NW + wave) + jr;
    const int c = jp ^ swz_a<CH>(r);
    a_k[i] = 8 * c;
    if (r < a_rows_here) {
      const int64_t src = GATHER ? (int64_t)p.a_rows[row_begin + r] : (int64_t)r;
      a_off[i] = (uint32_t)(src * p.lda * 2 + c * 16);
    } else {
      a_off[i] = kOutOfRange;
    }
  }
#pragma unroll
  for (int i = 0; i < B_INS; ++i) {
    const int r = RPI * (i * NW + wave) + jr;
    const int c = jp ^ swz_b<CH>(r);
    const int n = DUAL ? r % (BN / 2) : r;
    b_k[i] = 8 * c;
    b_off[i] = n < n_here ? (uint32_t)(n * K * 2 + c * 16) : kOutOfRange;
  }
  const uint32_t ring_lds = lds_addr(&ring[0]) + (uint32_t)wave * 1024u;
  // The loop runs k-steps in pairs (the fragment register sets alternate);
  // with one k-step per stage an odd stage count gets one all-zero stage
  // more, which adds nothing.
  const int Kc = (int)K;                       // < 2^22
  const int nk = (Kc + BK - 1) / BK;
  const int NS = KS == 2 ? nk : (nk + 1) & ~1;

  // This wave's load offsets for stage s: chunks past K (the k tail, the
  // padding stage and the stages issued past the end) are out of range.
  auto stage_offs = [&](int s, uint32_t (&o)[LOADS]) {
    const int k0 = s * BK;
#pragma unroll
    for (int i = 0; i < A_INS; ++i) o[i] = k0 + a_k[i] < Kc ? a_off[i] : kOutOfRange;
#pragma unroll
    for (int i = 0; i < B_INS; ++i) o[A_INS + i] = k0 + b_k[i] < Kc ? b_off[i] : kOutOfRange;
  };
  // load i (of LOADS) of a stage into the slot at LDS byte address `base`
  auto dma = [&](int i, uint32_t base, const uint32_t (&o)[LOADS], uint32_t kb) {
    if (i < A_INS) {
      asm_load_lds(da, base + (uint32_t)(i * NW) * 1024u, o[i], kb);
    } else {
      const int b = i - A_INS;
      const bool up = DUAL && RPI * (b * NW) >= BN / 2;   // compile-time per i
      asm_load_lds(up ? db1 : db0, base + (uint32_t)(BM * CH * 16 + b * NW * 1024), o[i], kb);
    }
  };
  auto issue_all = [&](int s, int slot) {
    uint32_t o[LOADS];
    stage_offs(s, o);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) dma(i, ring_lds + (uint32_t)slot * (SLOT * 16), o, (uint32_t)s * (BK * 2));
  };

  // ---- LDS fragment rows -----------------------------------------------------
  const int li = lane & 15;   // fragment row (weight) / column (activation)
  const int lg = lane >> 4;   // k group: 8 consecutive k
  int x_row[FM], w_row[FN];
#pragma unroll
  for (int f = 0; f < FM; ++f) x_row[f] = wm * TM + f * 16 + li;
#pragma unroll
  for (int f = 0; f < FN; ++f) {
    // interleave the rows of a fragment pair: lane group g ends up holding
    // output columns 8g..8g+7 of the pair's 32 columns
    const int set = DUAL ? f / HALF : 0;
    const int fl = DUAL ? f % HALF : f;
    const int base = set * (BN / 2) + wn * (DUAL ? TN / 2 : TN) + (fl >> 1) * 32;
    w_row[f] = base + 8 * (li >> 2) + 4 * (fl & 1) + (li & 3);
  }

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Fragment registers: two sets, alternating by k-step.  Read n of a k-step
  // is x0, w0 .. w(FN-1), x1 .. x(FM-1): the order its MFMAs consume them.
  constexpr int NREADS = FM + FN;
  u32x4_t xf[2][FM], wf[2][FN];
  auto frag_read = [&](int n, const u32x4_t* sl, int ks, auto set_c) {
    constexpr int set = decltype(set_c)::value;
    const int c = ks * 4 + lg;
    if (n == 0) {
      xf[set][0] = sl[x_row[0] * CH + (c ^ swz_a<CH>(x_row[0]))];
    } else if (n <= FN) {
      const int r = w_row[n - 1];
      wf[set][n - 1] = sl[BM * CH + r * CH + (c ^ swz_b<CH>(r))];
    } else {
      const int r = x_row[n - FN];
      xf[set][n - FN] = sl[r * CH + (c ^ swz_a<CH>(r))];
    }
  };
  auto mfma_t = [&](int t, auto set_c) {   // MFMA t of a k-step: row t / FN, column t % FN
    constexpr int set = decltype(set_c)::value;
    mfma_ordered(acc[t / FN][t % FN], wf[set][t % FN], xf[set][t / FN]);
  };
  using Set0 = std::integral_constant<int, 0>;
  using Set1 = std::integral_constant<int, 1>;

  // Prologue: stages 0 .. R-2 in flight, stage 0 published, R-1 issued.
  // Every stage up to the last one read plus R - 1 is issued (past the end
  // they load nothing), so every wait below is the same.
#pragma unroll
  for (int s = 0; s < R - 1; ++s) issue_all(s, s);
  wait_vm<LOADS * (R - 2)>();
  lds_barrier();
  issue_all(R - 1, R - 1);
#pragma unroll
  for (int n = 0; n < NREADS; ++n) frag_read(n, ring, 0, Set0{});

  // One k-step, register set CUR, of stage s in slot `slot`.
  //  * Not the stage's last k-step: its MFMAs, each followed by at most one
  //    fragment read of the next k-step (same slot) into the other set.
  //  * The last one: the first half of its MFMAs; hand-off (wait for this
  //    wave's loads of stage s + 1, then a barrier: stage s + 1 is in LDS for
  //    every wave, and every wave has finished reading `slot`); the second
  //    half, each MFMA followed by at most one instruction of the hand-off
  //    stream: the loads of stage s + R into `slot`, then the fragment reads
  //    of stage s + 1 into the other set.  The matrix core never waits for a
  //    run of memory instructions.
  constexpr int NMA = (FM / 2) * FN;          // MFMAs per half k-step
  constexpr int NOPS = LOADS + NREADS;
  auto kstep = [&](int s, int ks, int slot, auto cur_c) {
    constexpr int CUR = decltype(cur_c)::value;
    using Nxt = std::integral_constant<int, CUR ^ 1>;
    if (ks + 1 < KS) {
      const u32x4_t* sl = ring + slot * SLOT;
#pragma unroll
      for (int t = 0; t < 2 * NMA; ++t) {
        mfma_t(t, cur_c);
#pragma unroll
        for (int n = t * NREADS / (2 * NMA); n < (t + 1) * NREADS / (2 * NMA); ++n)
          frag_read(n, sl, ks + 1, Nxt{});
      }
      return;
    }
    uint32_t o[LOADS];
    stage_offs(s + R, o);
#pragma unroll
    for (int t = 0; t < NMA; ++t) mfma_t(t, cur_c);
    wait_vm<LOADS * (R - 2)>();
    lds_barrier();
    const uint32_t base = ring_lds + (uint32_t)slot * (SLOT * 16);
    const uint32_t kb = (uint32_t)(s + R) * (BK * 2);
    const u32x4_t* sl = ring + (slot + 1 == R ? 0 : slot + 1) * SLOT;
#pragma unroll
    for (int t = 0; t < NMA; ++t) {
      mfma_t(NMA + t, cur_c);
#pragma unroll
      for (int n = t * NOPS / NMA; n < (t + 1) * NOPS / NMA; ++n) {
        if (n < LOADS) dma(n, base, o, kb);
        else frag_read(n - LOADS, sl, 0, Nxt{});
      }
    }
  };
  int slot = 0;
  if constexpr (KS == 2) {
    for (int s = 0; s < NS; ++s) {
      kstep(s, 0, slot, Set0{});
      kstep(s, 1, slot, Set1{});
      slot = slot + 1 == R ? 0 : slot + 1;
    }
  } else {
    for (int s = 0; s < NS; s += 2) {
      const int s1 = slot + 1 == R ? 0 : slot + 1;
      kstep(s, 0, slot, Set0{});
      kstep(s + 1, 0, s1, Set1{});
      slot = s1 + 1 == R ? 0 : s1 + 1;
    }
  }
  wait_vm<0>();   // the last stages' loads (of nothing) land before LDS is released
  mfma_drain();

  // ---- epilogue -------------------------------------------------------------
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t lrow = row_begin + wm * TM + i * 16 + li;
    const bool row_ok = lrow < row_end;
    if constexpr (OUT == GEMM_OUT_GEGLU) {
#pragma unroll
      for (int q = 0; q < HALF / 2; ++q) {
        const int64_t n = n0 + wn * (TN / 2) + q * 32 + 8 * lg;
        float v[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v[r] = gelu_tanh(acc[i][2 * q][r]) * acc[i][HALF + 2 * q][r];
          v[4 + r] = gelu_tanh(acc[i][2 * q + 1][r]) * acc[i][HALF + 2 * q + 1][r];
        }
        if (row_ok && n < N)
          st16(static_cast<uint16_t*>(p.C) + lrow * p.ldc + n, pack_bf16x8(v));
      }
    } else {
#pragma unroll
      for (int q = 0; q < FN / 2; ++q) {
        const int64_t n = n0 + wn * TN + q * 32 + 8 * lg;
        float v[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v[r] = acc[i][2 * q][r];
          v[4 + r] = acc[i][2 * q + 1][r];
        }
        if (!(row_ok && n < N)) continue;
        if constexpr (OUT == GEMM_OUT_F32_SCALED) {
          const float s = p.row_scale[lrow];
          float* dst = static_cast<float*>(p.C) + lrow * p.ldc + n;
          u32x4_t lo, hi;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            lo[r] = __float_as_uint(v[r] * s);
            hi[r] = __float_as_uint(v[4 + r] * s);
          }
          st16(dst, lo);
          st16(dst + 4, hi);
        } else {
          if (p.bias) {
            float b[8];
            unpack_bf16x8(ld16(p.bias + n), b);
#pragma unroll
            for (int r = 0; r < 8; ++r) v[r] += b[r];
          }
          if (p.act != ACT_NONE) {
#pragma unroll
            for (int r = 0; r < 8; ++r) v[r] = apply_act(v[r], p.act);
          }
          st16(static_cast<uint16_t*>(p.C) + lrow * p.ldc + n, pack_bf16x8(v));
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN, int BK, int R, int OUT, bool GATHER, bool GROUPED>
hipError_t launch_cfg(GemmParams p, hipStream_t s) {
  constexpr int OUT_N = (OUT == GEMM_OUT_GEGLU) ? BN / 2 : BN;
  if (!GROUPED) p.tiles_m = (int)((p.M + BM - 1) / BM);
  p.tiles_n = (int)((p.N + OUT_N - 1) / OUT_N);
  p.group_m = 4;
  const int64_t blocks = (int64_t)p.tiles_m * p.tiles_n;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, BK, R, OUT, GATHER, GROUPED>), dim3((unsigned)blocks),
                     dim3(WM * WN * 64), 0, s, p);
  return hipGetLastError();
}

template <int OUT, bool GATHER, bool GROUPED>
hipError_t launch_tile(int tile, const GemmParams& p, hipStream_t s) {
  switch (tile) {
    case TILE_128x128: return launch_cfg<128, 128, 2, 2, 32, 4, OUT, GATHER, GROUPED>(p, s);
    case TILE_256x256: return launch_cfg<256, 256, 2, 4, 64, 2, OUT, GATHER, GROUPED>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int gemm_tile_bm(int tile) { return tile == TILE_256x256 ? 256 : 128; }
int gemm_tile_bn(int tile) { return tile == TILE_256x256 ? 256 : 128; }

hipError_t launch_gemm(int out_kind, bool gather, bool grouped, int tile, GemmParams p,
                       hipStream_t s) {
  if (out_kind == GEMM_OUT_BF16 && !gather && !grouped) return launch_tile<GEMM_OUT_BF16, false, false>(tile, p, s);
  if (out_kind == GEMM_OUT_GEGLU && !gather && !grouped) return launch_tile<GEMM_OUT_GEGLU, false, false>(tile, p, s);
  if (out_kind == GEMM_OUT_GEGLU && gather && grouped) return launch_tile<GEMM_OUT_GEGLU, true, true>(tile, p, s);
  if (out_kind == GEMM_OUT_F32_SCALED && !gather && grouped) return launch_tile<GEMM_OUT_F32_SCALED, false, true>(tile, p, s);
  return hipErrorInvalidValue;
}

}  // namespace fmlp
