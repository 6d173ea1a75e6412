// Quantizer (Eq. 1) and slice-and-pack (Eq. 6) kernels.
//
// "Matryoshka Quantization" explainer, §3.4 "Quantization Primitives" (Eq. 1,
// min-max quantization with c = 8) and "The Bit-Slicing Operator" (Eq. 6).
#include "mq_device.h"
#include "mq_internal.h"

namespace mq {

// ---------------------------------------------------------------------------
// mq_quantize: one wavefront per weight vector (group consecutive entries of a
// row).  Min and max are exact; alpha, z and the codes are evaluated in IEEE
// float64 from the stored fp32 alpha and z, in this order:
//   alpha = fp32((max - min) / 255), z = fp32(-min / alpha),
//   q = clamp(floor((w / alpha + z) + 0.5), 0, 255).
// A constant vector takes alpha = 1, z = -min, and so does a vector whose
// fp32 alpha would be zero or subnormal (no usable scale).
// ---------------------------------------------------------------------------
#pragma clang fp contract(off)
// threads per workgroup of these kernels, as a constant (blockDim.x is a
// vector load from the dispatch packet)
constexpr int kPackThreads = 256;

__global__ void __launch_bounds__(256) quantize_kernel(const float* __restrict__ w, int64_t n_vec,
                                                       int group, uint8_t* __restrict__ codes,
                                                       float* __restrict__ alpha,
                                                       float* __restrict__ zero) {
  const int lane = threadIdx.x & 63;
  const int64_t v = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (v >= n_vec) return;
  const float* src = w + v * group;
  float mn = INFINITY, mx = -INFINITY;
  for (int i = lane; i < group; i += 64) {
    float f = src[i];
    mn = fminf(mn, f);
    mx = fmaxf(mx, f);
  }
  for (int off = 32; off > 0; off >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, off));
    mx = fmaxf(mx, __shfl_xor(mx, off));
  }
  float a32 = (float)(((double)mx - (double)mn) / 255.0);
  float z32;
  if (mx == mn || !(a32 >= 0x1p-126f)) {
    // a constant vector, or a range too small for a normal fp32 scale
    a32 = 1.0f;
    z32 = -mn;
  } else {
    z32 = (float)(-(double)mn / (double)a32);
  }
  if (lane == 0) {
    alpha[v] = a32;
    zero[v] = z32;
  }
  const double ad = (double)a32, zd = (double)z32;
  uint8_t* dst = codes + v * group;
  for (int i = lane; i < group; i += 64) {
    double t = (double)src[i] / ad;
    t = t + zd;
    t = t + 0.5;
    double f = floor(t);
    f = f < 0.0 ? 0.0 : (f > 255.0 ? 255.0 : f);
    dst[i] = (uint8_t)(int)f;
  }
}
#pragma clang fp contract(on)

hipError_t launch_quantize(const float* w, int64_t N, int64_t K, int64_t group, uint8_t* codes,
                           float* alpha, float* zero, hipStream_t stream) {
  int64_t n_vec = N * (K / group);
  int64_t blocks = (n_vec + 3) / 4;
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, w, n_vec,
                     (int)group, codes, alpha, zero);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// mq_pack: t = min((q + 2^(7-r)) >> (8-r), 2^r - 1) (t = q for r = 8), i.e.
// round half up of q / 2^(8-r) followed by the clamp of Eq. 6.  Layout: each
// 32-bit word holds 32/r consecutive indices, those at even positions in the
// low 16 bits and those at odd positions in the high 16 bits, the j-th of a
// half in bits [j*r, j*r + r) of that half (so that one AND-OR per register
// yields operand pairs of consecutive k, see mq_device.h).  Rows need no
// special handling: K is a multiple of 64, so the flat packing of the [N, K]
// array is the row-by-row packing.  The loops are grid-strided.
// ---------------------------------------------------------------------------

// The index t = min((q + 2^(7-r)) >> (8-r), 2^r - 1) (Eq. 6, rounding half
// up) of the four bytes of w at once (r = 2, 3, 4, 6): with h = q >> 1,
// (h + 2^(6-r)) >> (7-r) is the same rounded quotient (q + 2^(7-r)) >> (8-r)
// and stays below 256 in every byte, so no carry crosses bytes; the one
// value above 2^r - 1 (2^r itself) is clamped by subtracting its top bit.
template <int R>
__device__ __forceinline__ uint32_t slice4(uint32_t w) {
  constexpr uint32_t ONES = 0x01010101u;
  const uint32_t h = (w >> 1) & 0x7F7F7F7Fu;
  const uint32_t v = ((h + ONES * (1u << (6 - R))) >> (7 - R)) & (ONES * ((2u << R) - 1u));
  return v - ((v >> R) & ONES);
}

// One 16-byte vector of codes (16 consecutive codes of a row) per thread and
// step at r = 2 and 8, so every wave load is one contiguous 1 KiB; two
// adjacent vectors at r = 4, so that each thread stores 16 bytes (measured
// faster than 8-byte stores).  Bytewise for r = 2, 4: a dword d of four indices (one per
// byte) becomes d | d >> (16 - R), whose byte 0 holds the indices of codes 0
// and 2 (code 0 in the low bits) and byte 1 those of codes 1 and 3; byte
// permutes then gather the even codes into the low half of each output word
// and the odd codes into the high half (v_perm_b32: selector values 0-3 pick
// bytes of the second source, 4-7 bytes of the first).  At r = 8 the same
// layout swaps bytes 1 and 2 of every dword (codes 0, 2 low; 1, 3 high).
template <int R>
__global__ void __launch_bounds__(kPackThreads) pack_kernel(const u32x4* __restrict__ codes,
                                                   uint8_t* __restrict__ out, int64_t n_in16) {
  if constexpr (R == 4) {
    for (int64_t i = blockIdx.x * (int64_t)kPackThreads + threadIdx.x; i < n_in16 / 2;
         i += (int64_t)gridDim.x * kPackThreads) {
      const u32x4 in0 = __builtin_nontemporal_load(codes + 2 * i);
      const u32x4 in1 = __builtin_nontemporal_load(codes + 2 * i + 1);
      u32x4 o;
#pragma unroll
      for (int w = 0; w < 4; ++w) {  // codes 8w .. 8w + 7: dwords 2w, 2w + 1 of the pair
        const u32x4& v = w < 2 ? in0 : in1;
        const uint32_t t0 = slice4<4>(v[(2 * w) & 3]), t1 = slice4<4>(v[(2 * w + 1) & 3]);
        o[w] = __builtin_amdgcn_perm(t1 | (t1 >> 12), t0 | (t0 >> 12), 0x05010400u);
      }
      __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(out) + i);
    }
  } else {
    for (int64_t i = blockIdx.x * (int64_t)kPackThreads + threadIdx.x; i < n_in16;
         i += (int64_t)gridDim.x * kPackThreads) {
      const u32x4 in = __builtin_nontemporal_load(codes + i);
      if constexpr (R == 8) {
        u32x4 o;
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = __builtin_amdgcn_perm(in[k], in[k], 0x03010200u);
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(out) + i);
      } else {
        static_assert(R == 2, "byte-aligned precisions only");
        uint32_t tp[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t t = slice4<2>(in[k]);
          tp[k] = t | (t >> 14);
        }
        // 2-bit pairs of two dwords side by side, then their nibbles merged
        const uint32_t u01 = __builtin_amdgcn_perm(tp[1], tp[0], 0x05010400u);
        const uint32_t u23 = __builtin_amdgcn_perm(tp[3], tp[2], 0x05010400u);
        const uint32_t o = __builtin_amdgcn_perm(u23 | (u23 >> 4), u01 | (u01 >> 4), 0x06020400u);
        __builtin_nontemporal_store(o, reinterpret_cast<uint32_t*>(out) + i);
      }
    }
  }
}

// One packed word from dwords of b-bit indices, one index per byte (b = 4:
// 2 dwords, 2: 4 dwords, 1: 8 dwords), in the word layout above: d | d >>
// (16 - b) puts the indices of codes 0 and 2 in byte 0 and of codes 1 and 3
// in byte 1; byte permutes and shifts then merge them, even codes into the
// low half, odd codes into the high half.
__device__ __forceinline__ uint32_t word_of4(const uint32_t* t) {
  return __builtin_amdgcn_perm(t[1] | (t[1] >> 12), t[0] | (t[0] >> 12), 0x05010400u);
}
__device__ __forceinline__ uint32_t word_of2(const uint32_t* t) {
  uint32_t tp[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) tp[k] = t[k] | (t[k] >> 14);
  const uint32_t u01 = __builtin_amdgcn_perm(tp[1], tp[0], 0x05010400u);
  const uint32_t u23 = __builtin_amdgcn_perm(tp[3], tp[2], 0x05010400u);
  return __builtin_amdgcn_perm(u23 | (u23 >> 4), u01 | (u01 >> 4), 0x06020400u);
}
__device__ __forceinline__ uint32_t word_of1(const uint32_t* t) {
  uint32_t v[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {  // 4 indices (2 even, 2 odd) per byte pair -> nibbles
    const uint32_t u = __builtin_amdgcn_perm(t[2 * a + 1] | (t[2 * a + 1] >> 15),
                                             t[2 * a] | (t[2 * a] >> 15), 0x05010400u);
    v[a] = u | (u >> 6);
  }
  const uint32_t w01 = __builtin_amdgcn_perm(v[1], v[0], 0x06020400u);
  const uint32_t w23 = __builtin_amdgcn_perm(v[3], v[2], 0x06020400u);
  return __builtin_amdgcn_perm(w23 | (w23 >> 4), w01 | (w01 >> 4), 0x06020400u);
}

// r = 3 and r = 6: the index t is split into its high bits t >> r_lo (a plane
// of width r - r_lo) and its low bits (width r_lo = 1 or 2), each packed in
// the word layout above; the high plane of all rows comes first, then the low
// plane.  Each thread takes 32 consecutive codes (two 16-byte loads): 4 r_hi
// bytes of the high plane and 4 r_lo bytes of the low plane.
template <int R>
__global__ void __launch_bounds__(kPackThreads) pack_split_kernel(const u32x4* __restrict__ codes,
                                                         uint8_t* __restrict__ out,
                                                         int64_t n_thr, int64_t lo_base) {
  constexpr int RL = R == 6 ? 2 : 1, RH = R - RL;
  constexpr int CODES = 32;  // codes per thread
  constexpr int IN16 = CODES / 16;
  constexpr int HW = RH, LW = RL;  // high- and low-plane words per thread
  for (int64_t i = blockIdx.x * (int64_t)kPackThreads + threadIdx.x; i < n_thr;
       i += (int64_t)gridDim.x * kPackThreads) {
    u32x4 in[IN16];
#pragma unroll
    for (int j = 0; j < IN16; ++j) in[j] = __builtin_nontemporal_load(codes + i * IN16 + j);
    // indices of 4 codes per dword (bytewise), split into high and low fields
    constexpr int DW = CODES / 4;
    uint32_t hi[DW], lo[DW];
#pragma unroll
    for (int k = 0; k < DW; ++k) {
      const uint32_t t = slice4<R>(in[k >> 2][k & 3]);
      hi[k] = (t >> RL) & (0x01010101u * ((1u << RH) - 1u));
      lo[k] = t & (0x01010101u * ((1u << RL) - 1u));
    }
    uint32_t h[HW], l[LW];
#pragma unroll
    for (int w = 0; w < HW; ++w) h[w] = RH == 4 ? word_of4(hi + 2 * w) : word_of2(hi + 4 * w);
#pragma unroll
    for (int w = 0; w < LW; ++w) l[w] = RL == 2 ? word_of2(lo + 4 * w) : word_of1(lo + 8 * w);
    if constexpr (R == 6) {
      const u32x4 hv = {h[0], h[1], h[2], h[3]};
      const u32x2 lv = {l[0], l[1]};
      *reinterpret_cast<u32x4*>(out + i * 16) = hv;
      *reinterpret_cast<u32x2*>(out + lo_base + i * 8) = lv;
    } else {
      const u32x2 hv = {h[0], h[1]};
      *reinterpret_cast<u32x2*>(out + i * 8) = hv;
      *reinterpret_cast<uint32_t*>(out + lo_base + i * 4) = l[0];
    }
  }
}

hipError_t launch_pack(const uint8_t* codes, int64_t N, int64_t K, int r, uint8_t* packed,
                       hipStream_t stream) {
  if (r == 3 || r == 6) {
    const int rh = r == 6 ? 4 : 2;
    const int64_t n_thr = N * K / 32;  // 32 codes per thread
    int64_t blocks = (n_thr + 255) / 256;
    if (blocks > 256 * 64) blocks = 256 * 64;
    if (blocks < 1) blocks = 1;
    const int64_t lo_base = N * K * rh / 8;
    const u32x4* in = reinterpret_cast<const u32x4*>(codes);
    if (r == 6)
      hipLaunchKernelGGL(pack_split_kernel<6>, dim3((unsigned)blocks), dim3(kPackThreads), 0, stream, in,
                         packed, n_thr, lo_base);
    else
      hipLaunchKernelGGL(pack_split_kernel<3>, dim3((unsigned)blocks), dim3(kPackThreads), 0, stream, in,
                         packed, n_thr, lo_base);
    return hipGetLastError();
  }
  const int64_t n16 = N * K / 16;  // input vectors of 16 codes (K % 64 == 0: even)
  int64_t blocks = (n16 + 255) / 256;
  if (blocks > 256 * 64) blocks = 256 * 64;
  if (blocks < 1) blocks = 1;
  const u32x4* in = reinterpret_cast<const u32x4*>(codes);
  uint8_t* out = packed;
  switch (r) {
    case 2:
      hipLaunchKernelGGL(pack_kernel<2>, dim3((unsigned)blocks), dim3(kPackThreads), 0, stream, in, out, n16);
      break;
    case 4:
      hipLaunchKernelGGL(pack_kernel<4>, dim3((unsigned)blocks), dim3(kPackThreads), 0, stream, in, out, n16);
      break;
    default:
      hipLaunchKernelGGL(pack_kernel<8>, dim3((unsigned)blocks), dim3(kPackThreads), 0, stream, in, out, n16);
      break;
  }
  return hipGetLastError();
}

}  // namespace mq
