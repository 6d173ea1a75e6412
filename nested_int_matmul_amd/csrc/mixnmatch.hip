// Elementwise steps of a Mix'n'Match layer stack ("Matryoshka Quantization"
// explainer, §3.4 "Mix'n'Match and Interpolative Slicing": one stored int8
// model, a slice precision per layer).  The pages define no layer dataflow;
// the library's is
//   a = bf16(h / sqrt(mean(h^2)));  q,k,v,u,g = W a;  o = W_o bf16(q);
//   d = W_down bf16(u * g);  h = h + o + d.
// The products run in the skinny kernel (its prologue forms bf16(q) and
// bf16(u * g)); these kernels do the normalization and the residual update.
#include "mq_device.h"
#include "mq_internal.h"

namespace mq {

constexpr int kNormThreads = 1024;

// One workgroup per activation row.  Fixed-order reduction (deterministic).
// LOAD: h = x first (bf16 x0, exact in fp32); RESIDUAL: h = h + o + d first.
template <bool RESIDUAL, bool NORM, bool LOAD = false>
__global__ void __launch_bounds__(kNormThreads) norm_kernel(float* __restrict__ h,
                                                            const float* __restrict__ o,
                                                            const float* __restrict__ d,
                                                            uint16_t* __restrict__ a, int H,
                                                            const uint16_t* __restrict__ x0 =
                                                                nullptr) {
  __shared__ float wsum[kNormThreads / 64];
  const int m = blockIdx.x;
  float* hr = h + (int64_t)m * H;
  float ss = 0.f;
  for (int i = threadIdx.x; i < H; i += blockDim.x) {
    float v;
    if (LOAD) {
      v = bf16_to_f32(x0[(int64_t)m * H + i]);
      hr[i] = v;
    } else {
      v = hr[i];
    }
    if (RESIDUAL) {
      v = v + o[(int64_t)m * H + i];
      v = v + d[(int64_t)m * H + i];
      hr[i] = v;
    }
    ss += v * v;
  }
  if (!NORM) return;
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) tot += wsum[w];
  const float rms = sqrtf(tot / (float)H);
  for (int i = threadIdx.x; i < H; i += blockDim.x) {
    a[(int64_t)m * H + i] = (uint16_t)f32_to_bf16_rne(hr[i] / rms);
  }
}

hipError_t launch_rmsnorm_bf16(const float* h, uint16_t* a, int64_t M, int64_t H,
                               hipStream_t stream) {
  hipLaunchKernelGGL((norm_kernel<false, true>), dim3((unsigned)M), dim3(kNormThreads), 0, stream,
                     const_cast<float*>(h), nullptr, nullptr, a, (int)H);
  return hipGetLastError();
}

hipError_t launch_load_rmsnorm_bf16(const uint16_t* x, float* h, uint16_t* a, int64_t M,
                                    int64_t H, hipStream_t stream) {
  hipLaunchKernelGGL((norm_kernel<false, true, true>), dim3((unsigned)M), dim3(kNormThreads), 0,
                     stream, h, nullptr, nullptr, a, (int)H, x);
  return hipGetLastError();
}

hipError_t launch_residual_rmsnorm(float* h, const float* o, const float* d, uint16_t* a,
                                   int64_t M, int64_t H, hipStream_t stream) {
  // a == nullptr: residual update only
  if (a)
    hipLaunchKernelGGL((norm_kernel<true, true>), dim3((unsigned)M), dim3(kNormThreads), 0, stream,
                       h, o, d, a, (int)H);
  else
    hipLaunchKernelGGL((norm_kernel<true, false>), dim3((unsigned)M), dim3(kNormThreads), 0,
                       stream, h, o, d, a, (int)H);
  return hipGetLastError();
}

}  // namespace mq
