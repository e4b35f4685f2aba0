// Launch interface of the FP8-weight decode kernel (decode_w8.hip).  Internal
// to the library, like kernels.h; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fmlp {

// One decode layer (M <= 16 tokens) with weights stored as OCP E4M3 codes
// [N, K] and one fp32 scale per row: W[n, k] = s[n] * e4m3(q[n, k]); K % 16 == 0.
// With W1 set it is the gate+up layer y = act(s0 * (x q0^T)) * (s1 * (x q1^T)),
// else y = act(s0 * (x q0^T) + bias).  One launch.
struct W8Layer {
  const uint16_t* x;     // [M, K] bf16
  const uint8_t* W0;     // [N, K] E4M3
  const float* s0;       // [N]
  const uint8_t* W1;     // [N, K] E4M3 (gate+up: the up rows) or nullptr
  const float* s1;       // [N] or nullptr
  const uint16_t* bias;  // [N] or nullptr (ungated only)
  uint16_t* y;           // [M, N] bf16
  int64_t K, N;
  int act;               // Act; for a gated layer, the gate's activation
};

hipError_t launch_decode_w8(const W8Layer& L, int M, hipStream_t s);

// Both layers of a one-token forward in one persistent launch (L1.y is the
// workspace area for h as H / 2 words of 8 bytes {bf16 pair, epoch}; sync is
// the workspace's decode header).  Applies to M == 1, H = L1.N <= 4096 with
// H % 16 == 0, L2.K == H, 2 * L1.K <= 64 KB and a device of at most
// kDecodeMaxBlocks compute units.
bool decode_w8_two_applies(int M, const W8Layer& L1, const W8Layer& L2, int cus);
hipError_t launch_decode_w8_two(const W8Layer& L1, const W8Layer& L2, uint32_t* sync, int cus, hipStream_t s,
                                bool cooperative = false);

}  // namespace fmlp
