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
// Structure: a block computes a BM x BN tile with WAVES_M x WAVES_N waves.
// K advances in stages of 64; each stage of A and B is copied HBM -> registers
// -> LDS (double buffered, one barrier per stage, the next stage's global loads
// in flight while the current stage feeds the MFMAs).  LDS rows are 128 bytes
// (8 chunks of 16 B), each chunk at an XOR-permuted slot chosen so the 16-byte
// fragment reads of 16 rows are bank-conflict free (swz_a, swz_b below).
// v_mfma_f32_16x16x32_bf16 is fed with the weight as the row operand and the
// activation as the column operand; the weight rows of a fragment pair are
// interleaved so each lane ends with 8 consecutive output columns of one row,
// stored as one 16-byte write.
#include "common.h"
#include "kernels.h"

namespace fmlp {

namespace {

constexpr int kBK = 64;  // k per LDS stage

// LDS rows are 128 bytes (8 chunks of 16 B).  With 64 four-byte banks, two
// rows share a bank line, so a 16-lane fragment read is conflict free when
// (row & 1, slot of the chunk) differs across its 16 rows.  Activation
// fragments read 16 consecutive rows; weight fragments read rows interleaved
// in groups of 4 (8*(l/4) + (l%4)).  Each gets its own chunk permutation.
__device__ __forceinline__ int swz_a(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int swz_b(int r) { return ((r >> 1) & 1) | ((r >> 2) & 6); }

template <int BM, int BN, int WAVES_M, int WAVES_N, int OUT, bool GATHER, bool GROUPED>
__global__ void __launch_bounds__(WAVES_M * WAVES_N * 64)
gemm_bf16_kernel(GemmParams p) {
  constexpr int NT = WAVES_M * WAVES_N * 64;
  constexpr int TM = BM / WAVES_M;   // wave tile rows (activation rows)
  constexpr int TN = BN / WAVES_N;   // wave tile width in B-tile rows
  constexpr int FM = TM / 16;
  constexpr int FN = TN / 16;
  constexpr bool DUAL = (OUT == GEMM_OUT_GEGLU);
  constexpr int HALF = FN / 2;       // DUAL: gate fragments [0,HALF), up [HALF,FN)
  constexpr int ROWS_PER_PASS = NT / 8;
  constexpr int A_IT = BM / ROWS_PER_PASS;
  constexpr int B_IT = BN / ROWS_PER_PASS;
  constexpr int OUT_N = DUAL ? BN / 2 : BN;   // output columns per block
  static_assert(BM % ROWS_PER_PASS == 0 && BN % ROWS_PER_PASS == 0, "load mapping");
  static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile");
  static_assert(DUAL ? (HALF % 2 == 0) : (FN % 2 == 0), "fragment pairs");

  __shared__ u32x4_t sA[2][BM * 8];
  __shared__ u32x4_t sB[2][BN * 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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

  // ---- per-thread global source rows (clamped; k chunk fixed per thread) --
  const int ck = (tid & 7) * 8;           // k offset of this thread's chunk in a stage
  const uint16_t* a_src[A_IT];
  const uint16_t* b_src[B_IT];
  int a_slot[A_IT], b_slot[B_IT];
#pragma unroll
  for (int i = 0; i < A_IT; ++i) {
    const int r = (tid >> 3) + i * ROWS_PER_PASS;
    int64_t lr = row_begin + r;
    if (lr >= row_end) lr = row_end - 1;
    const int64_t src = GATHER ? (int64_t)p.a_rows[lr] : lr;
    a_src[i] = p.A + src * p.lda + ck;
    a_slot[i] = r * 8 + ((tid & 7) ^ swz_a(r));
  }
#pragma unroll
  for (int i = 0; i < B_IT; ++i) {
    const int r = (tid >> 3) + i * ROWS_PER_PASS;
    const uint16_t* base = B0;
    int64_t n = n0 + r;
    if (DUAL && r >= BN / 2) {
      base = B1;
      n = n0 + (r - BN / 2);
    }
    if (n >= N) n = N - 1;
    b_src[i] = base + n * K + ck;
    b_slot[i] = r * 8 + ((tid & 7) ^ swz_b(r));
  }

  u32x4_t ra[A_IT], rb[B_IT];
  auto gload = [&](int kt) {
    const int64_t k0 = (int64_t)kt * kBK;
    const bool ok = (k0 + ck) < K;
#pragma unroll
    for (int i = 0; i < A_IT; ++i) ra[i] = ok ? ld16(a_src[i] + k0) : zero4();
#pragma unroll
    for (int i = 0; i < B_IT; ++i) rb[i] = ok ? ld16(b_src[i] + k0) : zero4();
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_IT; ++i) sA[buf][a_slot[i]] = ra[i];
#pragma unroll
    for (int i = 0; i < B_IT; ++i) sB[buf][b_slot[i]] = rb[i];
  };

  // ---- LDS fragment rows --------------------------------------------------
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

  // Software pipeline: the fragments of the next k-step are read from LDS
  // while the MFMAs of the current one run, and the second k-step's MFMAs
  // straddle the stage barrier (they read registers only), so every phase
  // pairs LDS traffic with MFMA work.
  u32x4_t xf[2][FM], wf[2][FN];
  auto read_frags = [&](int buf, int ks, int set) {
    const int chunk = ks * 4 + lg;
#pragma unroll
    for (int f = 0; f < FM; ++f) xf[set][f] = sA[buf][x_row[f] * 8 + (chunk ^ swz_a(x_row[f]))];
#pragma unroll
    for (int f = 0; f < FN; ++f) wf[set][f] = sB[buf][w_row[f] * 8 + (chunk ^ swz_b(w_row[f]))];
  };
  auto mfmas = [&](int set, int i0, int i1) {
#pragma unroll
    for (int i = i0; i < i1; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = mfma_16x16x32(wf[set][j], xf[set][i], acc[i][j]);
  };

  const int nk = (int)((K + kBK - 1) / kBK);
  gload(0);
  swrite(0);
  __syncthreads();
  read_frags(0, 0, 0);

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) gload(kt + 1);
    read_frags(cur, 1, 1);
    mfmas(0, 0, FM);                 // k-step 0 of this stage
    mfmas(1, 0, FM / 2);             // first half of k-step 1
    if (more) swrite(cur ^ 1);
    __syncthreads();
    if (more) read_frags(cur ^ 1, 0, 0);
    mfmas(1, FM / 2, FM);            // second half of k-step 1
  }

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

template <int BM, int BN, int WM, int WN, int OUT, bool GATHER, bool GROUPED>
hipError_t launch_cfg(GemmParams p, hipStream_t s) {
  constexpr int OUT_N = (OUT == GEMM_OUT_GEGLU) ? BN / 2 : BN;
  if (!GROUPED) p.tiles_m = (int)((p.M + BM - 1) / BM);
  p.tiles_n = (int)((p.N + OUT_N - 1) / OUT_N);
  p.group_m = 8;
  const int64_t blocks = (int64_t)p.tiles_m * p.tiles_n;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, OUT, GATHER, GROUPED>), dim3((unsigned)blocks),
                     dim3(WM * WN * 64), 0, s, p);
  return hipGetLastError();
}

template <int OUT, bool GATHER, bool GROUPED>
hipError_t launch_tile(int tile, const GemmParams& p, hipStream_t s) {
  switch (tile) {
    case TILE_128x128: return launch_cfg<128, 128, 2, 2, OUT, GATHER, GROUPED>(p, s);
    case TILE_256x256: return launch_cfg<256, 256, 2, 2, OUT, GATHER, GROUPED>(p, s);
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
