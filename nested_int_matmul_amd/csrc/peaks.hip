// Measured-peak probes of one gfx950 device (libmq_peaks.so): the ceilings
// the sliced-integer products are compared against next to the vendor
// figures.  A decode product is bound by reading the weights out of HBM, a
// prefill product by the bf16 matrix cores, and every launch pays the
// dispatch cadence of the queue; each probe isolates one of the three.
//
//  - stream_read_kernel: every lane reads 16-byte vectors of a buffer with a
//    grid-stride loop, UNROLL loads in flight, and folds them into one word
//    per workgroup (so the loads are not dead).  Bytes read / time is the
//    achievable HBM read rate for that buffer size.
//  - mfma_loop_kernel: each wave runs CHAINS independent accumulator chains
//    of v_mfma_f32_32x32x16_bf16 on register operands (no memory traffic),
//    enough chains to cover the instruction's dependent-issue latency.
//    Flops / time is the achievable dense bf16 matrix-core rate.
//  - empty_kernel: no work; back-to-back launches give the per-launch
//    cadence that every kernel of a dependent chain pays.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mq_peaks.h"

namespace mqp {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kReadThreads = 256;
constexpr int kUnroll = 8;

__global__ void __launch_bounds__(kReadThreads)
    stream_read_kernel(const u32x4* __restrict__ buf, int64_t n16, uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kReadThreads;
  int64_t i = (int64_t)blockIdx.x * kReadThreads + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= buf[i];
  uint32_t w = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  for (int off = 32; off > 0; off >>= 1) w ^= __shfl_xor(w, off);
  __shared__ uint32_t part[kReadThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = w;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int k = 0; k < kReadThreads / 64; ++k) t ^= part[k];
    sink[blockIdx.x] = t;
  }
}

constexpr int kChains = 4;

__global__ void __launch_bounds__(256) mfma_loop_kernel(float* __restrict__ out, int iters,
                                                        uint32_t seed) {
  // operands from the thread id (never all zero, so nothing folds away)
  const uint32_t v = 0x3F803F80u ^ ((threadIdx.x + seed) & 0x007F007Fu);
  u32x4 raw = {v, v ^ 0x00010001u, v ^ 0x00020002u, v ^ 0x00030003u};
  const bf16x8 a = __builtin_bit_cast(bf16x8, raw);
  const bf16x8 b = __builtin_bit_cast(bf16x8, raw ^ 0x00040004u);
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
#pragma unroll 1
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ void empty_kernel() {}

}  // namespace mqp

extern "C" {

int mqp_stream_read(const void* buf, size_t bytes, int blocks, uint32_t* sink, void* stream) {
  if (!buf || !sink || blocks < 1 || bytes < 16 || (bytes & 15) ||
      (reinterpret_cast<uintptr_t>(buf) & 15))
    return 1;
  hipLaunchKernelGGL(mqp::stream_read_kernel, dim3(blocks), dim3(mqp::kReadThreads), 0,
                     (hipStream_t)stream, static_cast<const mqp::u32x4*>(buf),
                     (int64_t)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int mqp_mfma_loop(float* out, int blocks, int iters, void* stream) {
  if (!out || blocks < 1 || iters < 1) return 1;
  hipLaunchKernelGGL(mqp::mfma_loop_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out,
                     iters, 7u);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

double mqp_mfma_loop_flops(int blocks, int iters) {
  // 4 waves per workgroup, kChains products of 2 * 32 * 32 * 16 flops per iteration
  return (double)blocks * 4.0 * iters * mqp::kChains * 2.0 * 32 * 32 * 16;
}

int mqp_empty(void* stream) {
  hipLaunchKernelGGL(mqp::empty_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
