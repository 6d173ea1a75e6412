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
// For r < 8 the index is turned into a bf16 by placing its bits in the top
// of the mantissa of the bf16 constant 2^r: the result is exactly
// u = 2^r + t (one AND-OR per two values; r = 3 and 6 assemble the bits of
// two planes the same way).  The offset folds into the zero point:
// alpha * (2^(8-r) * u - (z + 256)), the same 256 on the int8 scale for
// every r, so that the fp32 sums the kernels form stay within a small factor
// of the dequantized weights (|S - z| + 256 on the int8 scale).  For r = 8
// the byte is converted through fp32 (exact: every integer below 256 is a
// bf16), u = t.
//
// Plane layout: a 32-bit word holds 32/r consecutive indices, the even-
// positioned ones in its low 16 bits and the odd-positioned ones in its high
// 16 bits.  Shifting the word so that field j of both halves lands under the
// mask puts indices 2j and 2j+1 into the two bf16 halves of one register, so
// unpacked operands come out in natural k order and the activations are used
// as stored.
//   r = 4: a word = one 8-element operand;  r = 2: a word = two operands
//   (elements 0..7, then 8..15);  r = 8: two words = one operand.
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

// Results a kernel writes once and never reads back (GEMM output tiles,
// K-slice partials, summed slices) may be stored at device scope (the sc1
// bit), so that the XCD's L2 writes them through instead of holding them
// dirty until the write-back at the end of the kernel; where that pays is
// measured per kernel.  Whole 16-byte pieces go through a buffer store (a
// relaxed atomic store is at most 8 bytes, and two 8-byte halves written
// through separately measured slower than plain 16-byte stores).  The bits
// stored are the same either way.
constexpr int kCachePolicySc1 = 16;  // the sc1 bit of a vector memory instruction
__device__ __forceinline__ void store_out(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_out16(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0,
                                         kCachePolicySc1);
}

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

// Offset u - t of the operand encoding, and the zero-point shift it implies
// (u * 2^(8-r) = S + shift).
template <int R>
struct Enc {
  static constexpr int kOffset = R == 8 ? 0 : (1 << R);
  static constexpr float kStep = (float)(1 << (8 - R));                 // 2^(8-r)
  static constexpr float kOffsetShift = (float)kOffset * kStep;         // z' = z + shift
};

// bf16x2 from a 32-bit word of two bf16 patterns.
__device__ __forceinline__ bf16x8 as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4 v = {a, b, c, d};
  return __builtin_bit_cast(bf16x8, v);
}

// Constants of the unpack held in registers: gfx9 VOP3 instructions take no
// literal operand, so (w & mask) | magic is one v_and_or_b32 only when mask
// and magic sit in registers.
struct UnpackK {
  uint32_t m4, one4, m2, one2;
  __device__ __forceinline__ static UnpackK make() {
    UnpackK k{0x00780078u, 0x41804180u, 0x00600060u, 0x40804080u};
    asm volatile("" : "+v"(k.m4), "+v"(k.one4), "+v"(k.m2), "+v"(k.one2));
    return k;
  }
};

// Written in C (not inline asm) so that the compiler sees the write and keeps
// the wait states between it and a matrix instruction that reads the result
// or read the register before; with m and o in registers it is one
// v_and_or_b32.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
  return (a & m) | o;
}

// --- r = 4: one word (8 indices) -> one 8-element operand, order 0,4,1,5,2,6,3,7
//     (bf16 16.0 in both halves; 16 + t)
__device__ __forceinline__ bf16x8 unpack_r4(uint32_t w, const UnpackK& k) {
  uint32_t p0 = and_or(w << 3, k.m4, k.one4);
  uint32_t p1 = and_or(w >> 1, k.m4, k.one4);
  uint32_t p2 = and_or(w >> 5, k.m4, k.one4);
  uint32_t p3 = and_or(w >> 9, k.m4, k.one4);
  return as_bf16x8(p0, p1, p2, p3);
}
__device__ __forceinline__ bf16x8 unpack_r4(uint32_t w) { return unpack_r4(w, UnpackK::make()); }

// --- r = 2: one word (16 indices) -> two 8-element operands (h = 0, 1)
//     h = 0: order 0,8,1,9,2,10,3,11 ; h = 1: order 4,12,5,13,6,14,7,15
//     (bf16 4.0 in both halves; 4 + t)
template <int H>
__device__ __forceinline__ bf16x8 unpack_r2(uint32_t w, const UnpackK& k) {
  if (H == 0) {
    uint32_t p0 = and_or(w << 5, k.m2, k.one2);
    uint32_t p1 = and_or(w << 3, k.m2, k.one2);
    uint32_t p2 = and_or(w << 1, k.m2, k.one2);
    uint32_t p3 = and_or(w >> 1, k.m2, k.one2);
    return as_bf16x8(p0, p1, p2, p3);
  } else {
    uint32_t p0 = and_or(w >> 3, k.m2, k.one2);
    uint32_t p1 = and_or(w >> 5, k.m2, k.one2);
    uint32_t p2 = and_or(w >> 7, k.m2, k.one2);
    uint32_t p3 = and_or(w >> 9, k.m2, k.one2);
    return as_bf16x8(p0, p1, p2, p3);
  }
}
template <int H>
__device__ __forceinline__ bf16x8 unpack_r2(uint32_t w) { return unpack_r2<H>(w, UnpackK::make()); }

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}
// --- r = 8: two words (8 bytes) -> one operand.  A word holds elements
//     (e0, e2) in bytes 0, 1 and (e1, e3) in bytes 2, 3.
__device__ __forceinline__ uint32_t bf16_pair_of_bytes(uint32_t lo, uint32_t hi) {
  // lo, hi < 256: the fp32 value is exact and its upper half is the bf16.
  uint32_t a = __float_as_uint((float)lo);
  uint32_t b = __float_as_uint((float)hi);
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}
__device__ __forceinline__ bf16x8 unpack_r8(uint32_t w0, uint32_t w1) {
  uint32_t p0 = bf16_pair_of_bytes(w0 & 0xffu, (w0 >> 16) & 0xffu);
  uint32_t p1 = bf16_pair_of_bytes((w0 >> 8) & 0xffu, w0 >> 24);
  uint32_t p2 = bf16_pair_of_bytes(w1 & 0xffu, (w1 >> 16) & 0xffu);
  uint32_t p3 = bf16_pair_of_bytes((w1 >> 8) & 0xffu, w1 >> 24);
  return as_bf16x8(p0, p1, p2, p3);
}

// --- r = 6 and r = 3: the index is stored as two planes (high bits t >> r_lo
//     in the word layout of width r - r_lo, low bits in that of width r_lo).
//     The two fields are assembled at mantissa bits [7 - r, 7) of each half
//     under the bf16 constant 2^r (64 or 8), whose mantissa step there is 1:
//     u = 2^r + t, exact.
struct UnpackK36 {
  uint32_t mhi6, mlo6, one6, mhi3, mlo3, one3;
  __device__ __forceinline__ static UnpackK36 make() {
    UnpackK36 k{0x00780078u, 0x00060006u, 0x42804280u, 0x00600060u, 0x00100010u, 0x41004100u};
    asm volatile("" : "+v"(k.mhi6), "+v"(k.mlo6), "+v"(k.one6), "+v"(k.mhi3), "+v"(k.mlo3),
                 "+v"(k.one3));
    return k;
  }
};

__device__ __forceinline__ uint32_t shift_signed(uint32_t w, int s) {  // s > 0: right
  return s >= 0 ? (w >> s) : (w << (-s));
}

// r = 6, operand i (elements 8i .. 8i+7 of a lane's 32): hi = the 4-bit word
// of those 8 elements, lo = the 2-bit word of elements 16*(i/2) .. +16.
// Register j holds elements 2j, 2j+1: the low field (bits 2j' of the r = 2
// layout) goes to bits 1..2, the high field (bits 4j of the r = 4 layout) to
// bits 3..6, under 64.
__device__ __forceinline__ bf16x8 unpack_r6(uint32_t hi, uint32_t lo, int i_odd,
                                            const UnpackK36& k) {
  uint32_t p[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t l = and_or(shift_signed(lo, 2 * j + 8 * i_odd - 1), k.mlo6, k.one6);
    p[j] = and_or(shift_signed(hi, 4 * j - 3), k.mhi6, l);
  }
  return as_bf16x8(p[0], p[1], p[2], p[3]);
}
// r = 3, operand i of a lane's 32 elements: hi = the 2-bit word of elements
// 16*(i/2) .. +16, lo = the 1-bit word of the lane's 32 elements.  The low
// bit goes to bit 4, the two high bits to bits 5..6, under 8.
__device__ __forceinline__ bf16x8 unpack_r3(uint32_t hi, uint32_t lo, int i,
                                            const UnpackK36& k) {
  uint32_t p[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t l = and_or(shift_signed(lo, 4 * i + j - 4), k.mlo3, k.one3);
    p[j] = and_or(shift_signed(hi, 2 * (4 * (i & 1) + j) - 5), k.mhi3, l);
  }
  return as_bf16x8(p[0], p[1], p[2], p[3]);
}

// Per-step weight loads of a lane: one bounds-checked load (r = 2, 4, 8) or
// one from each plane of a split (r = 3, 6); `words` flattens them.
template <int R, int V>
struct LoadT;
template <int R>
struct LoadT<R, 16> {
  typedef u32x4 T;
  static constexpr int NW = 4;
  __device__ __forceinline__ static T load(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t) {
    return buf_load16(r, off);
  }
  __device__ __forceinline__ static void words(const T& t, uint32_t* d) {
    d[0] = t[0]; d[1] = t[1]; d[2] = t[2]; d[3] = t[3];
  }
};
template <int R>
struct LoadT<R, 8> {
  typedef u32x2 T;
  static constexpr int NW = 2;
  __device__ __forceinline__ static T load(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t) {
    return buf_load8(r, off);
  }
  __device__ __forceinline__ static void words(const T& t, uint32_t* d) {
    d[0] = t[0]; d[1] = t[1];
  }
};
struct Split6 {  // 16 high bytes (32 four-bit fields) + 8 low bytes (32 two-bit fields)
  u32x4 h;
  u32x2 l;
};
struct Split3 {  // 8 high bytes (32 two-bit fields) + 4 low bytes (32 one-bit fields)
  u32x2 h;
  uint32_t l;
};
template <>
struct LoadT<6, 0> {
  typedef Split6 T;
  static constexpr int NW = 6;
  __device__ __forceinline__ static T load(__amdgpu_buffer_rsrc_t r, uint32_t oh, uint32_t ol) {
    T t;
    t.h = buf_load16(r, oh);
    t.l = buf_load8(r, ol);
    return t;
  }
  __device__ __forceinline__ static void words(const T& t, uint32_t* d) {
    d[0] = t.h[0]; d[1] = t.h[1]; d[2] = t.h[2]; d[3] = t.h[3];
    d[4] = t.l[0]; d[5] = t.l[1];
  }
};
template <>
struct LoadT<3, 0> {
  typedef Split3 T;
  static constexpr int NW = 3;
  __device__ __forceinline__ static T load(__amdgpu_buffer_rsrc_t r, uint32_t oh, uint32_t ol) {
    T t;
    t.h = buf_load8(r, oh);
    t.l = buf_load4(r, ol);
    return t;
  }
  __device__ __forceinline__ static void words(const T& t, uint32_t* d) {
    d[0] = t.h[0]; d[1] = t.h[1];
    d[2] = t.l;
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
