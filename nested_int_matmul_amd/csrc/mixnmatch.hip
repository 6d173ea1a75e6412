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

// One workgroup per activation row.  Thread t owns the 4-float vectors
// t, t + 1024, ... (at most VPT of them: H <= 4096 VPT, VPT = 1 or 4 for
// H <= kStackMaxH): they stay in
// registers between the two passes, and all their loads are issued before
// the first is used, so a row costs a few memory latencies rather than one
// per vector.  Fixed-order reduction (deterministic).  LOAD: h = x first
// (bf16 x0, exact in fp32); RESIDUAL: h = h + o + d first.  H is a multiple
// of 64 and every row 16-byte aligned.
template <bool RESIDUAL, bool NORM, bool LOAD, int VPT>
__global__ void __launch_bounds__(kNormThreads) norm_kernel(float* __restrict__ h,
                                                            const float* __restrict__ o,
                                                            const float* __restrict__ d,
                                                            uint16_t* __restrict__ a, int H,
                                                            const uint16_t* __restrict__ x0) {
  __shared__ float wsum[kNormThreads / 64];
  const int m = blockIdx.x, tid = threadIdx.x;
  const int nv = H >> 2;  // 4-float vectors per row
  f32x4* hr = reinterpret_cast<f32x4*>(h + (int64_t)m * H);
  f32x4 keep[VPT];
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int i = tid + j * kNormThreads;
    if (i < nv) {
      f32x4 v;
      if (LOAD) {
        const u32x2 b = reinterpret_cast<const u32x2*>(x0 + (int64_t)m * H)[i];
        v[0] = __uint_as_float(b[0] << 16);
        v[1] = __uint_as_float(b[0] & 0xffff0000u);
        v[2] = __uint_as_float(b[1] << 16);
        v[3] = __uint_as_float(b[1] & 0xffff0000u);
      } else {
        v = hr[i];
      }
      if (RESIDUAL) {
        v = v + reinterpret_cast<const f32x4*>(o + (int64_t)m * H)[i];
        v = v + reinterpret_cast<const f32x4*>(d + (int64_t)m * H)[i];
      }
      keep[j] = v;
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int i = tid + j * kNormThreads;
    if (i < nv) {
      if (LOAD || RESIDUAL) hr[i] = keep[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) ss += keep[j][e] * keep[j][e];
    }
  }
  if (!NORM) return;
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  if ((tid & 63) == 0) wsum[tid >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int w = 0; w < kNormThreads / 64; ++w) tot += wsum[w];
  const float rms = sqrtf(tot / (float)H);
  u32x2* arow = reinterpret_cast<u32x2*>(a + (int64_t)m * H);
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int i = tid + j * kNormThreads;
    if (i < nv) {
      u32x2 b;
      b[0] = f32_to_bf16_rne(keep[j][0] / rms) | (f32_to_bf16_rne(keep[j][1] / rms) << 16);
      b[1] = f32_to_bf16_rne(keep[j][2] / rms) | (f32_to_bf16_rne(keep[j][3] / rms) << 16);
      arow[i] = b;
    }
  }
}

template <bool RESIDUAL, bool NORM, bool LOAD>
static hipError_t launch_norm(float* h, const float* o, const float* d, uint16_t* a, int64_t M,
                              int64_t H, const uint16_t* x0, hipStream_t stream) {
  const int64_t per = (H / 4 + kNormThreads - 1) / kNormThreads;  // vectors per thread
  const dim3 grid((unsigned)M), block(kNormThreads);
  if (per <= 1)
    hipLaunchKernelGGL((norm_kernel<RESIDUAL, NORM, LOAD, 1>), grid, block, 0, stream, h, o, d,
                       a, (int)H, x0);
  else if (per <= 4 && H <= kStackMaxH)
    hipLaunchKernelGGL((norm_kernel<RESIDUAL, NORM, LOAD, 4>), grid, block, 0, stream, h, o, d,
                       a, (int)H, x0);
  else
    return hipErrorInvalidValue;  // H > kStackMaxH is rejected before any launch
  return hipGetLastError();
}

hipError_t launch_rmsnorm_bf16(const float* h, uint16_t* a, int64_t M, int64_t H,
                               hipStream_t stream) {
  return launch_norm<false, true, false>(const_cast<float*>(h), nullptr, nullptr, a, M, H,
                                         nullptr, stream);
}

hipError_t launch_load_rmsnorm_bf16(const uint16_t* x, float* h, uint16_t* a, int64_t M,
                                    int64_t H, hipStream_t stream) {
  return launch_norm<false, true, true>(h, nullptr, nullptr, a, M, H, x, stream);
}

hipError_t launch_residual_rmsnorm(float* h, const float* o, const float* d, uint16_t* a,
                                   int64_t M, int64_t H, hipStream_t stream) {
  // a == nullptr: residual update only
  if (a) return launch_norm<true, true, false>(h, o, d, a, M, H, nullptr, stream);
  return launch_norm<true, false, false>(h, o, d, a, M, H, nullptr, stream);
}

}  // namespace mq
