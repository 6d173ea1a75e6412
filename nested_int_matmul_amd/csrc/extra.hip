// Extra-Precision MatQuant: the slice without the clamp of Eq. 6 (the errata
// Eq. 8 of the "Matryoshka Quantization" explainer, §3.4 "The Bit-Slicing
// Operator") has one more level, 256, reached by the codes
// q >= 256 - 2^(7-r).  The r-bit plane keeps the clamped index; these kernels
// build, per row, the list of the codes at the extra level and add their
// missing 2^(8-r) * alpha * x to a product computed from the plane (the sparse
// addition the explainer's §5 "Critical Assessment" says a kernel would need).
#include "mq_device.h"
#include "mq_internal.h"

namespace mq {

constexpr int kRowWaves = 4;  // rows per 256-thread workgroup (one wave per row)

__device__ __forceinline__ uint32_t over_mask16(const u32x4 v, uint32_t thr) {
  uint32_t m = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w)
#pragma unroll
    for (int b = 0; b < 4; ++b)
      if (((v[w] >> (8 * b)) & 0xffu) >= thr) m |= 1u << (4 * w + b);
  return m;
}

// counts[n] = number of codes of row n at or above thr; one wave per row.
__global__ void __launch_bounds__(64 * kRowWaves) overflow_count_kernel(
    const uint8_t* __restrict__ codes, int N, int K, uint32_t thr, int* __restrict__ counts) {
  const int lane = threadIdx.x & 63;
  for (int n = blockIdx.x * kRowWaves + (threadIdx.x >> 6); n < N; n += gridDim.x * kRowWaves) {
    const uint8_t* row = codes + (int64_t)n * K;
    int c = 0;
    for (int k = lane * 16; k < K; k += 64 * 16)
      c += __popc(over_mask16(*reinterpret_cast<const u32x4*>(row + k), thr));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
    if (lane == 0) counts[n] = c;
  }
}

// row_ptr[n + 1] = counts[0] + ... + counts[n] (in place: counts live at
// row_ptr + 1), row_ptr[0] = 0; one workgroup, chunks of 1024 rows.
__global__ void __launch_bounds__(1024) overflow_scan_kernel(int* __restrict__ row_ptr, int N) {
  __shared__ int part[1024 / 64];
  __shared__ int carry_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) {
    row_ptr[0] = 0;
    carry_s = 0;
  }
  __syncthreads();
  for (int base = 0; base < N; base += 1024) {
    const int i = base + tid;
    int v = i < N ? row_ptr[1 + i] : 0;
    // inclusive scan in the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int u = __shfl_up(v, off);
      if (lane >= off) v += u;
    }
    if (lane == 63) part[wave] = v;
    __syncthreads();
    int before = carry_s;
    for (int w = 0; w < wave; ++w) before += part[w];
    if (i < N) row_ptr[1 + i] = before + v;
    __syncthreads();
    if (tid == 1023) carry_s = before + v;
    __syncthreads();
  }
}

// col_idx[row_ptr[n] ...] = the k of row n's codes at or above thr, increasing
// (16-bit: K <= 65536).
__global__ void __launch_bounds__(64 * kRowWaves) overflow_fill_kernel(
    const uint8_t* __restrict__ codes, int N, int K, uint32_t thr, const int* __restrict__ row_ptr,
    uint16_t* __restrict__ col_idx) {
  const int lane = threadIdx.x & 63;
  for (int n = blockIdx.x * kRowWaves + (threadIdx.x >> 6); n < N; n += gridDim.x * kRowWaves) {
    const uint8_t* row = codes + (int64_t)n * K;
    int out = row_ptr[n];
    for (int k0 = 0; k0 < K; k0 += 64 * 16) {
      const int k = k0 + lane * 16;
      const uint32_t m = k < K ? over_mask16(*reinterpret_cast<const u32x4*>(row + k), thr) : 0u;
      const int c = __popc(m);
      // exclusive prefix of c over the lanes (lane order = k order)
      int incl = c;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int u = __shfl_up(incl, off);
        if (lane >= off) incl += u;
      }
      int pos = out + incl - c;
      uint32_t mm = m;
      while (mm) {
        const int b = __ffs(mm) - 1;
        col_idx[pos++] = (uint16_t)(k + b);
        mm &= mm - 1;
      }
      out += __shfl(incl, 63);
    }
  }
}

// y[m, n] += step * sum over row n's list of alpha[n, k >> gshift] * x[m, k]
// (gshift = 7 for groups of 128; per-channel scales are one alpha per row,
// applied once to the row's sum).  One wave per row, four rows per 256-thread
// workgroup.  A lane takes every 64th entry of its row, eight at a time: the
// eight index loads are issued together, then the gathers (no branch between
// them), so one round trip serves 512 entries of a row.  The 64 lanes are
// then summed in a fixed xor order (deterministic).  Activation rows go in
// blocks of 8; y and the row's scale are read before the list so that their
// latency overlaps.  The kernel is a chain of dependent round trips (row
// bounds, indices, gathers), so one launch takes several matrices (their rows
// concatenated) rather than one launch per matrix.  (A runtime integer
// division for the group index cost more than the rest of the kernel: the
// shift replaces it.)
constexpr int kApplyLanes = 64;
constexpr int kApplyRows = 256 / kApplyLanes;
constexpr int kApplyBatch = 8;

struct ApplyArgs {
  OverflowProblem p[kMaxProblems];
  int count;
  int M;
  float step;
};

template <bool PER_ROW>
__device__ __forceinline__ void apply_rows(const OverflowProblem& P, int n, int M, float step) {
  const int sub = threadIdx.x & (kApplyLanes - 1);
  const int N = P.N, K = P.K;
  const int G = PER_ROW ? 1 : K / 128;
  int b = 0, e = 0;
  if (n < N) {
    b = P.row_ptr[n];
    e = P.row_ptr[n + 1];
  }
  const float* arow = P.alpha + (int64_t)(n < N ? n : 0) * G;
  const float a_row = PER_ROW ? *arow : 1.f;
  for (int m0 = 0; m0 < M; m0 += 8) {
    // this lane's output, read before the list so that its latency overlaps
    const bool writer = n < N && sub < 8 && m0 + sub < M;
    float* yp = P.y + (int64_t)(m0 + (writer ? sub : 0)) * N + (n < N ? n : 0);
    const float y0 = writer ? *yp : 0.f;
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.f;
    for (int j0 = b + sub; j0 < e; j0 += kApplyLanes * kApplyBatch) {
      int k[kApplyBatch];
      float w[kApplyBatch];
#pragma unroll
      for (int u = 0; u < kApplyBatch; ++u) {
        const int j = j0 + u * kApplyLanes;
        k[u] = P.col_idx[j < e ? j : j0];  // j0 < e: a valid entry of the row
        w[u] = j < e ? 1.f : 0.f;
      }
      if (!PER_ROW) {
#pragma unroll
        for (int u = 0; u < kApplyBatch; ++u) w[u] *= arow[k[u] >> 7];
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (m0 + q < M) {
          const uint16_t* xr = P.x + (int64_t)(m0 + q) * K;
#pragma unroll
          for (int u = 0; u < kApplyBatch; ++u) acc[q] += w[u] * bf16_to_f32(xr[k[u]]);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (m0 + q < M) {
#pragma unroll
        for (int off = kApplyLanes / 2; off > 0; off >>= 1) acc[q] += __shfl_xor(acc[q], off);
      }
    }
    if (writer) {
      float v = acc[0];
#pragma unroll
      for (int q = 1; q < 8; ++q) v = sub == q ? acc[q] : v;
      *yp = y0 + step * (a_row * v);
    }
  }
}

__global__ void __launch_bounds__(256) overflow_apply_kernel(const ApplyArgs a) {
  int pi = 0;
#pragma unroll 1
  for (int i = 1; i < a.count; ++i)
    if ((int)blockIdx.x >= a.p[i].tile0) pi = i;
  const OverflowProblem& P = a.p[pi];
  const int n = ((int)blockIdx.x - P.tile0) * kApplyRows + (int)(threadIdx.x / kApplyLanes);
  if (P.group == P.K) apply_rows<true>(P, n, a.M, a.step);
  else apply_rows<false>(P, n, a.M, a.step);
}

static unsigned row_blocks(int64_t N) {
  int64_t b = (N + kRowWaves - 1) / kRowWaves;
  if (b > 65536) b = 65536;
  return (unsigned)(b < 1 ? 1 : b);
}

// r = 8 has no extra level (the threshold 256 is never reached)
static uint32_t extra_threshold(int r) { return r >= 8 ? 256u : 256u - (1u << (7 - r)); }

hipError_t launch_overflow_rows(const uint8_t* codes, int64_t N, int64_t K, int r, int* row_ptr,
                                hipStream_t s) {
  hipLaunchKernelGGL(overflow_count_kernel, dim3(row_blocks(N)), dim3(64 * kRowWaves), 0, s, codes,
                     (int)N, (int)K, extra_threshold(r), row_ptr + 1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(overflow_scan_kernel, dim3(1), dim3(1024), 0, s, row_ptr, (int)N);
  return hipGetLastError();
}

hipError_t launch_overflow_cols(const uint8_t* codes, int64_t N, int64_t K, int r,
                                const int* row_ptr, uint16_t* col_idx, hipStream_t s) {
  hipLaunchKernelGGL(overflow_fill_kernel, dim3(row_blocks(N)), dim3(64 * kRowWaves), 0, s, codes,
                     (int)N, (int)K, extra_threshold(r), row_ptr, col_idx);
  return hipGetLastError();
}

hipError_t launch_overflow_apply(OverflowProblem* probs, int count, int r, int64_t M,
                                 hipStream_t s) {
  ApplyArgs a;
  a.count = count;
  a.M = (int)M;
  a.step = (float)(1 << (8 - r));
  int tile0 = 0;
  for (int i = 0; i < count; ++i) {
    a.p[i] = probs[i];
    a.p[i].tile0 = tile0;
    tile0 += (int)((probs[i].N + kApplyRows - 1) / kApplyRows);
  }
  hipLaunchKernelGGL(overflow_apply_kernel, dim3((unsigned)tile0), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mq
