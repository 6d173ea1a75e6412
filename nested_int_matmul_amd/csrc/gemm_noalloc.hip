// mq_gemm_noalloc: the product of mq_gemm for callers that cannot allocate
// device memory (code under graph capture, tight serving loops, harnesses
// that forbid hipMalloc).  The only scratch mq_gemm needs is the fp32
// partial product of each K slice; here it lives in a file-scope device array
// of MQ_GEMM_NOALLOC_MAX_BYTES, one copy per device, which the loader places
// with the code object and the process holds until it ends.
//
// Host code never passes `scratch` itself to a kernel: in host code that name
// is a host-side stand-in, not a device address.  The device address of each
// device's copy comes from hipGetSymbolAddress, taken once per device with
// that device current, and is cached here; kernels receive that address.
#include <mutex>

#include "../../include/mq.h"
#include "mq_internal.h"

namespace {

constexpr size_t kScratchBytes = MQ_GEMM_NOALLOC_MAX_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device (null: not yet taken)

// Device address of the current device's scratch copy, taken on first use.
hipError_t scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

mq_status mq_gemm_noalloc(const uint8_t* packed, int r, const float* alpha, const float* zero,
                          int64_t group, int64_t N, int64_t K, const uint16_t* x, int64_t M,
                          float* y, void* stream) {
  mq_status s = mq::gemm_check(packed, r, alpha, zero, group, N, K, x, M, y);
  if (s != MQ_OK) return s;
  const size_t need = mq::gemm_workspace_bytes(M, N, K, group);
  if (need > kScratchBytes) return MQ_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    hipError_t e = scratch_ptr(&ws);
    if (e != hipSuccess) return mq::record_hip_error(e);
  }
  // mq_gemm checks the device and launches; the partial slices it writes
  // cover all of [S][M][N] before the slice sum reads them, so nothing in
  // the scratch needs clearing between calls
  return mq_gemm(packed, r, alpha, zero, group, N, K, x, M, y, ws, need, stream);
}

}  // extern "C"
