// The router of mq_gemm: the product
//   y[m, n] = sum_k x[m, k] (S(q[n, k], r) - z[n, g]) alpha[n, g]
// ("Matryoshka Quantization" explainer, §3.4, Eq. 6 and the dequantization
// of Eq. 1) for any number of activation rows, sent to the kernel that suits
// M:
//  - M <= 8: the decode kernel (gemv.hip; mq_gemm in abi.hip calls it);
//  - 9 <= M <= 64: the panel kernel (gemm_panel.hip), activations resident
//    in LDS, weights streamed through registers;
//  - M >= 65: gemm_big_kernel (gemm_big.hip), 128-row tiles up to M = 128
//    and 256-row tiles above, with K split when the tiles are few.
// Both GEMM kernels write one fp32 partial per K slice into the caller's
// workspace when they split K, and reduce_slices sums them in slice order.
#include "mq_device.h"
#include "mq_internal.h"

namespace mq {

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t) {
  if (M <= kSkinnyMaxM) return 0;
  if (M <= kPanelMaxM) return panel_workspace_bytes(M, N, K);
  return gemm_big_workspace_bytes(M, N, K);
}

hipError_t launch_gemm(const uint8_t* packed, int r, const float* alpha, const float* zero,
                       int64_t group, int64_t N, int64_t K, const uint16_t* x, int64_t M, float* y,
                       void* workspace, hipStream_t s) {
  if (M <= kPanelMaxM)
    return launch_gemm_panel(packed, r, alpha, zero, group, N, K, x, M, y, workspace, s);
  return launch_gemm_big(packed, r, alpha, zero, group, N, K, x, M, y, workspace, s);
}

}  // namespace mq
