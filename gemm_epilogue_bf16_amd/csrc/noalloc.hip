// fmlp_glu for callers that cannot allocate (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc): the workspace is a
// fixed device array of this library instead of a caller's buffer.
//
// Each device the library runs on holds its own copy of `scratch` for the
// life of the process.  Host code never uses the array's name as an address
// (on the host it names a stand-in, not device memory): the first call on a
// device, with that device current, asks the runtime for the array's device
// address once and keeps it; every later call on that device passes that
// address to fmlp_glu as its workspace, so the kernels are exactly the ones
// fmlp_glu runs.  No call allocates.
#include "../../include/fmlp.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace {

constexpr size_t kScratchBytes = FMLP_GLU_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0 && kScratchBytes >= (size_t)fmlp::kWorkspaceHeaderBytes, "scratch size");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Zero the decode header (the first kWorkspaceHeaderBytes) once per device: a
// small fill kernel, not a memset, so that it also replays correctly when the
// first call happens under graph capture.
__global__ void clear_header_kernel(uint32_t* p, int words) {
  for (int i = threadIdx.x; i < words; i += blockDim.x) p[i] = 0u;
}

struct DevScratch {
  bool ready = false;
  void* ptr = nullptr;
};
std::mutex g_mu;
DevScratch g_dev[64];

}  // namespace

namespace fmlp {
fmlp_status record_error(fmlp_status s, const char* msg);   // abi.cpp: fmlp_last_error's text
}

extern "C" fmlp_status fmlp_glu_noalloc(const fmlp_bf16* x, const fmlp_bf16* Wg, const fmlp_bf16* Wu,
                                        const fmlp_bf16* Wd, int gate_act, int64_t M, int64_t D, int64_t H,
                                        fmlp_bf16* y, fmlp_stream stream) {
  const size_t need = fmlp_glu_workspace_size(M, D, H);
  if (need > kScratchBytes)
    return fmlp::record_error(FMLP_E_WORKSPACE,
                              "fmlp_glu_noalloc: this shape needs a workspace larger than the "
                              "FMLP_GLU_NOALLOC_SCRATCH_BYTES the library holds; use fmlp_glu with a workspace");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
    return fmlp::record_error(FMLP_E_DEVICE, "fmlp_glu_noalloc: no usable current HIP device");
  void* ws = nullptr;
  bool first = false;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    DevScratch& d = g_dev[dev];
    if (!d.ready) {
      void* p = nullptr;
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr)
        return fmlp::record_error(FMLP_E_HIP, "fmlp_glu_noalloc: hipGetSymbolAddress(scratch) failed");
      d.ptr = p;
      d.ready = true;
      first = true;
    }
    ws = d.ptr;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (first) {
    hipLaunchKernelGGL(clear_header_kernel, dim3(1), dim3(256), 0, s, static_cast<uint32_t*>(ws),
                       fmlp::kWorkspaceHeaderBytes / 4);
    if (hipGetLastError() != hipSuccess)
      return fmlp::record_error(FMLP_E_HIP, "fmlp_glu_noalloc: clearing the scratch header failed");
  }
  return fmlp_glu(x, Wg, Wu, Wd, gate_act, M, D, H, y, ws, kScratchBytes, stream);
}
