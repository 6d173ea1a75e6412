// Device-side helpers shared by the gfx950 kernels of libmq.
//
// Operand encoding.  The matrix cores take bf16 operands.  A sliced index t
// (0 <= t < 2^r) is an integer, and the method's dequantized weight is
//   (S(q,r) - z) * alpha = alpha * (2^(8-r) * t - z)
// ("Matryoshka Quantization" explainer, §3.4, Eq. 6 and the dequantization
// alpha*(q - z) of Eq. 1).  The kernels contract x against the exact integer
// and apply alpha, z, 2^(8-r) in fp32 afterwards, so no weight is ever
// rounded to bf16.
//
// For r = 2 and r = 4 the index is turned into a bf16 by placing its bits in
// the top of the mantissa of the bf16 constant 2^r: the result is exactly
// u = 2^r + t (one AND-OR per two values).  The offset folds into the zero
// point: alpha * (2^(8-r) * u - (z + 256)).  For r = 8 the byte is converted
// through fp32 (exact: every integer below 256 is a bf16), u = t.
//
// The order in which one 32-bit word of a packed plane is spread over MFMA
// operand registers is fixed per r; the activations are staged in LDS in the
// same order ("permuted"), so both operands of every product agree on k.
//   r = 4: a word holds 8 indices; operand pairs are (0,4) (1,5) (2,6) (3,7).
//   r = 2: a word holds 16 indices; pairs (j, j+8) for j = 0..7, the first
//          four pairs form one 8-element operand, the last four the next.
//   r = 8: natural order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Word 3 of a raw buffer resource on gfx9: 32-bit dwords, bounds-checked by
// num_records (out-of-range loads return 0).
constexpr uint32_t kBufferWord3 = 0x00020000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           (int)kBufferWord3);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// Offset u - t of the operand encoding, and the zero-point shift it implies.
template <int R>
struct Enc {
  static constexpr float kOffsetShift = (R == 8) ? 0.0f : 256.0f;  // z' = z + shift
  static constexpr float kStep = (float)(1 << (8 - R));            // 2^(8-r)
};

// bf16x2 from a 32-bit word of two bf16 patterns.
__device__ __forceinline__ bf16x8 as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4 v = {a, b, c, d};
  return __builtin_bit_cast(bf16x8, v);
}

// --- r = 4: one word (8 indices) -> one 8-element operand, order 0,4,1,5,2,6,3,7
__device__ __forceinline__ bf16x8 unpack_r4(uint32_t w) {
  const uint32_t m = 0x00780078u, one = 0x41804180u;  // bf16 16.0 in both halves
  uint32_t p0 = ((w << 3) & m) | one;
  uint32_t p1 = ((w >> 1) & m) | one;
  uint32_t p2 = ((w >> 5) & m) | one;
  uint32_t p3 = ((w >> 9) & m) | one;
  return as_bf16x8(p0, p1, p2, p3);
}

// --- r = 2: one word (16 indices) -> two 8-element operands (h = 0, 1)
//     h = 0: order 0,8,1,9,2,10,3,11 ; h = 1: order 4,12,5,13,6,14,7,15
template <int H>
__device__ __forceinline__ bf16x8 unpack_r2(uint32_t w) {
  const uint32_t m = 0x00600060u, one = 0x40804080u;  // bf16 4.0 in both halves
  if (H == 0) {
    uint32_t p0 = ((w << 5) & m) | one;
    uint32_t p1 = ((w << 3) & m) | one;
    uint32_t p2 = ((w << 1) & m) | one;
    uint32_t p3 = ((w >> 1) & m) | one;
    return as_bf16x8(p0, p1, p2, p3);
  } else {
    uint32_t p0 = ((w >> 3) & m) | one;
    uint32_t p1 = ((w >> 5) & m) | one;
    uint32_t p2 = ((w >> 7) & m) | one;
    uint32_t p3 = ((w >> 9) & m) | one;
    return as_bf16x8(p0, p1, p2, p3);
  }
}

// --- r = 8: two words (8 bytes) -> one operand, natural order
__device__ __forceinline__ uint32_t bf16_pair_of_bytes(uint32_t lo, uint32_t hi) {
  // lo, hi < 256: the fp32 value is exact and its upper half is the bf16.
  uint32_t a = __float_as_uint((float)lo);
  uint32_t b = __float_as_uint((float)hi);
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}
__device__ __forceinline__ bf16x8 unpack_r8(uint32_t w0, uint32_t w1) {
  uint32_t p0 = bf16_pair_of_bytes(w0 & 0xffu, (w0 >> 8) & 0xffu);
  uint32_t p1 = bf16_pair_of_bytes((w0 >> 16) & 0xffu, w0 >> 24);
  uint32_t p2 = bf16_pair_of_bytes(w1 & 0xffu, (w1 >> 8) & 0xffu);
  uint32_t p3 = bf16_pair_of_bytes((w1 >> 16) & 0xffu, w1 >> 24);
  return as_bf16x8(p0, p1, p2, p3);
}

// Activation permutation inside a block of PB = (r == 2 ? 16 : 8) values:
// position p of the staged block holds source element perm(p).
template <int R>
struct XPerm {
  static constexpr int PB = (R == 2) ? 16 : 8;
  __device__ __forceinline__ static int src(int p) {
    if (R == 8) return p;
    if (R == 4) return (p >> 1) + ((p & 1) << 2);
    return ((p >> 3) << 2) + ((p >> 1) & 3) + ((p & 1) << 3);
  }
};

// fp32 -> bf16 bits, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

}  // namespace mq
