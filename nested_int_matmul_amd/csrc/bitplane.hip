// Bit-plane storage: one stored copy of the 8-bit codes, kept as eight planes
// of one bit each, serves every precision r = 1..8 without repacking.
//
// Slicing from planes ("Matryoshka Quantization" explainer, §3.4 "The
// Bit-Slicing Operator"): the index of Eq. 6 is the integer part of
// q / 2^(8-r) (the r most significant bits h, planes 8-r .. 7) plus the first
// discarded bit c (plane 7-r: rounding half up), clamped to 2^r - 1.  The
// clamp matters only where h is all ones and c = 1; the unclamped form (the
// errata Eq. 8, "Extra-Precision MatQuant") keeps the extra level 2^r.  A
// server at r reads r + 1 planes ((r + 1)/8 of the bytes; all 8 at r = 8).
//
// Storage (uint8 [8][N][K/8], plane p = bit p of q): each plane row is cut
// into 512-code superblocks of 64 bytes = 16 little-endian words; word 4s + G
// holds, at bit 16h + i, the bit of code 128G + 32s + 2i + h (s, G in 0..3,
// i in 0..15, h in 0..1).  K is a multiple of 512.
//
// Product (decode, M <= 8), design for gfx950:
//  - A wave owns 16 rows and a range of superblocks; per superblock each lane
//    loads 16 bytes (words 4s .. 4s+3, s = lane / 16) of its row from each
//    plane it needs, through bounds-checked buffer loads kept DEPTH
//    superblocks ahead.  The loads of a wave cover 16 rows x 64 contiguous
//    bytes per plane.
//  - The index t = h + c is formed bit-sliced on whole words (32 codes per
//    operation): a ripple carry through the h planes, with c dropped where h
//    is all ones unless the unclamped slice is asked for.
//  - Word G of a lane covers 32 codes of group G (128 codes); the four lane
//    slots together cover the group, so one v_mfma_f32_16x16x32_bf16 never
//    mixes groups.  The t-planes become exact bf16 operands by a bit
//    transpose: delta swaps turn planes 0-3 (and 4-7 when present) into
//    4-bit indices, nibble q of word a holding the code at word position
//    4q + a (codes 8q + 2a and 8q + 2a + 1 of the 32 for nibbles q and
//    q + 4).  Low nibbles go on mantissa bits 3..6 under bf16 16 (u = 16 + n),
//    high nibbles under bf16 256 (u = 256 + 16 n).  Operand a pairs with
//    activation dwords 4q + a, so four products (eight above four planes)
//    cover the 32 codes whatever r is.
//    A group's products accumulate into one fp32 accumulator that starts at
//    minus the group's offset (16 or 272 times the group's sum of x), so it
//    holds the group's sum of x * t; at the group's end it is folded into the
//    row total (with the group's alpha and z when group = 128).
//  - Activations are staged in LDS in natural order (buffer-to-LDS loads);
//    the same pass forms the sum of x per group of 128.
//  - Waves that share a row block split the superblocks; their results are
//    summed in LDS in a fixed order (deterministic).
#include "mq_device.h"
#include "mq_internal.h"

namespace mq {
namespace bp {

constexpr int kWaves = 8;     // waves per workgroup
constexpr int kSuper = 512;   // codes of a row per superblock (one step)
constexpr int kXPad = 8;      // bf16 elements of padding per staged activation row

template <int R, bool EXTRA>
struct Bp {
  static constexpr int PL = R < 8 ? R + 1 : 8;                   // planes read
  static constexpr int FIRST = R < 8 ? 7 - R : 0;                // lowest plane read
  static constexpr int PT = R < 8 ? (EXTRA ? R + 1 : R) : 8;     // planes of t
  static constexpr int DEPTH = PL <= 2 ? 4 : (PL <= 3 ? 3 : 2);  // superblocks in flight
  static constexpr float STEP = (float)(1 << (8 - R));           // 2^(8-r)
};

// (w & mask) | magic, written in C so that the compiler sees every write and
// keeps the wait states the matrix cores need between an operand's last
// write and its read (and between that read and the operand's next write).
// With mask and magic in vector registers the pair is one v_and_or_b32.
__device__ __forceinline__ uint32_t and_or_c(uint32_t w, uint32_t m, uint32_t o) {
  return (w & m) | o;
}

// Delta swap: the bit blocks of width s at odd block positions of a trade
// places with the blocks at even positions of b.
__device__ __forceinline__ void delta_swap(uint32_t& a, uint32_t& b, int sh, uint32_t m) {
  const uint32_t d = ((a >> sh) ^ b) & m;
  b ^= d;
  a ^= d << sh;
}

// Four bit-sliced words (bit p of word j = bit j of the index of the code at
// word position p) -> four words of 4-bit indices: nibble q of word a holds
// the index bits of the code at position 4q + a.
__device__ __forceinline__ void transpose4(uint32_t& w0, uint32_t& w1, uint32_t& w2,
                                           uint32_t& w3) {
  delta_swap(w0, w1, 1, 0x55555555u);
  delta_swap(w2, w3, 1, 0x55555555u);
  delta_swap(w0, w2, 2, 0x33333333u);
  delta_swap(w1, w3, 2, 0x33333333u);
}

// Nibbles q and q + 4 of w on mantissa bits 3..6 of the two halves under the
// bf16 constant `one` (16: unit 1, u = 16 + n; 256: unit 16, u = 256 + 16 n),
// for q = 0..3: both exact.
__device__ __forceinline__ bf16x8 nibble_operand(uint32_t w, uint32_t m4, uint32_t one) {
  return as_bf16x8(and_or_c(w << 3, m4, one), and_or_c(w >> 1, m4, one),
                   and_or_c(w >> 5, m4, one), and_or_c(w >> 9, m4, one));
}

struct Args {
  const uint8_t* planes;
  const float* alpha;
  const float* zero;
  const uint16_t* x;
  float* y;
  int N, K, group, M, kc, ks;
};

template <int R, bool GROUPED, bool EXTRA>
__global__ void __launch_bounds__(64 * kWaves) bp_gemv_kernel(const Args P) {
  using C = Bp<R, EXTRA>;
  extern __shared__ __align__(16) unsigned char smem[];
  const int M = P.M, K = P.K, N = P.N, KS = P.ks;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int rbpw = kWaves / KS;
  const int rb0 = (int)blockIdx.x * rbpw;

  const int kc = P.kc;
  const int xstride = kc + kXPad;
  const int gpc = kc / 128;  // groups per chunk
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);                       // [M][xstride]
  float* sxs = reinterpret_cast<float*>(smem + (size_t)M * xstride * 2);  // [M][gpc] sum of x
  float* sxt = sxs + M * gpc;            // [M] total of x
  float* red = sxt + kSkinnyMaxM;        // [kWaves * 16][M]

  const uint32_t rowb = (uint32_t)K / 8;
  const uint32_t plane_bytes = (uint32_t)N * rowb;
  const int G = K / P.group;
  const int rbl = wave / KS, ks = wave % KS;
  const int row0 = (rb0 + rbl) * 16;
  const int col = lane & 15, slot = lane >> 4;
  const int n_ld = row0 + col;
  const __amdgpu_buffer_rsrc_t pr = make_rsrc(P.planes, 8u * plane_bytes);
  // the lane's bytes of its row in the lowest plane read; rows past N read zeros
  const uint32_t row_off = n_ld < N ? (uint32_t)C::FIRST * plane_bytes + (uint32_t)n_ld * rowb +
                                          (uint32_t)slot * 16u
                                    : 0x80000000u;

  // per-channel epilogue operands: thread t writes row rr = t % rows_wg
  const int rows_wg = rbpw * 16;
  const int ep_rr = threadIdx.x % rows_wg;
  float ep_a = 0.f, ep_b = 0.f;
  if (!GROUPED) {
    const int n = rb0 * 16 + ep_rr;
    if (n < N) {
      const float a = P.alpha[n], z = P.zero[n];
      ep_a = a * C::STEP;
      ep_b = a * z;
    }
  }
  if (threadIdx.x < kSkinnyMaxM) sxt[threadIdx.x] = 0.f;

  // nibble operands: mask of mantissa bits 3..6 and the bf16 constants 16, 256
  uint32_t m4n = 0x00780078u, one16 = 0x41804180u, one256 = 0x43804380u;
  asm volatile("" : "+v"(m4n), "+v"(one16), "+v"(one256));

  const int xcol = col < M ? col : M - 1;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(P.x, (uint32_t)((int64_t)M * K * 2));
  const __amdgpu_buffer_rsrc_t ar = make_rsrc(P.alpha, (uint32_t)((int64_t)N * G * 4));
  const __amdgpu_buffer_rsrc_t zr = make_rsrc(P.zero, (uint32_t)((int64_t)N * G * 4));
  f32x4 tot = {0.f, 0.f, 0.f, 0.f};
  const int nchunks = (K + kc - 1) / kc;

#pragma unroll 1
  for (int c = 0; c < nchunks; ++c) {
    const int ck0 = c * kc;
    const int clen = min(kc, K - ck0);
    const int csteps = clen / kSuper;
    const int lo = __builtin_amdgcn_readfirstlane(csteps * ks / KS);
    const int hi = __builtin_amdgcn_readfirstlane(csteps * (ks + 1) / KS);
    const uint32_t cbase = row_off + (uint32_t)(ck0 / 8);
    auto loff = [&](int st) __attribute__((always_inline)) -> uint32_t {
      return (st < hi && row_off != 0x80000000u) ? cbase + (uint32_t)st * 64u : 0x80000000u;
    };
    u32x4 buf[C::DEPTH][C::PL];
    __syncthreads();
    // ---- stage x[:, ck0 : ck0 + clen): one 1 KiB piece per wave instruction
    {
      const int pieces = clen / 512;
      for (int pc = wave; pc < M * pieces; pc += kWaves) {
        const int m = pc / pieces, j = pc - m * pieces;
        const int k = ck0 + j * 512 + lane * 8;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            xr, (__attribute__((address_space(3))) void*)(xs + (size_t)m * xstride + j * 512), 16,
            (uint32_t)((m * K + k) * 2), 0, 0, 0);
      }
    }
    // ---- first superblocks of this wave, behind the staging loads
#pragma unroll
    for (int d = 0; d < C::DEPTH; ++d)
#pragma unroll
      for (int pl = 0; pl < C::PL; ++pl) {
        const uint32_t o = loff(lo + d);
        buf[d][pl] = buf_load16(pr, o == 0x80000000u ? o : o + (uint32_t)pl * plane_bytes);
      }
    __syncthreads();
    // ---- per group of 128: sum of x
    {
      const int bpr = clen / 8;
      const int total = M * bpr;
      const uint32_t ones = 0x3F803F80u;
      for (int b0 = 0; b0 < total; b0 += (64 * kWaves)) {
        const int b = b0 + threadIdx.x;
        float s = 0.f;
        int m = 0, kb = 0;
        if (b < total) {
          m = b / bpr;
          kb = (b - m * bpr) * 8;
          const u32x4 w4 = *reinterpret_cast<const u32x4*>(xs + (size_t)m * xstride + kb);
#pragma unroll
          for (int q = 0; q < 4; ++q) s += dot2_bf16(w4[q], ones, 0.f);
        }
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) s += __shfl_xor(s, off);
        if (b < total && (kb % 128) == 0) sxs[m * gpc + kb / 128] = s;
      }
    }
    __syncthreads();
    if (!GROUPED) {
      for (int m = wave; m < M; m += kWaves) {
        float s = 0.f;
        for (int gi = lane; gi < clen / 128; gi += 64) s += sxs[m * gpc + gi];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
        if (lane == 0) sxt[m] += s;
      }
    }

    // ---- stream this wave's superblocks
    const uint16_t* xrow = xs + (size_t)xcol * xstride + slot * 32;
#pragma unroll 1
    for (int base = lo; base < hi; base += C::DEPTH) {
#pragma unroll
      for (int d = 0; d < C::DEPTH; ++d) {
        const int st = base + d;
        if (st < hi) {
#pragma unroll
          for (int Gi = 0; Gi < 4; ++Gi) {
            // the index planes of word Gi (bit-sliced, 32 codes per word)
            uint32_t t[C::PT];
            if constexpr (R == 8) {
#pragma unroll
              for (int j = 0; j < 8; ++j) t[j] = buf[d][j][Gi];
            } else {
              uint32_t cy = buf[d][0][Gi];
              if constexpr (!EXTRA) {
                uint32_t all = buf[d][1][Gi];
#pragma unroll
                for (int j = 1; j < R; ++j) all &= buf[d][1 + j][Gi];
                cy &= ~all;
              }
#pragma unroll
              for (int j = 0; j < R; ++j) {
                const uint32_t h = buf[d][1 + j][Gi];
                t[j] = h ^ cy;
                cy = h & cy;
              }
              if constexpr (EXTRA) t[R] = cy;
            }
            const int gl = st * 4 + Gi;  // group in the chunk
            const uint16_t* xp = xrow + st * kSuper + Gi * 128;
            // the t-planes transposed into 4-bit indices (planes 0-3, and
            // 4-7 when there are more than four): word a then holds, in
            // nibbles q and q + 4, the codes of word positions 4q + a and
            // 4q + 16 + a, i.e. codes 8q + 2a and 8q + 2a + 1 of the 32.
            // Operand a pairs them with activation dwords 4q + a.
            uint32_t lo[4], hi[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              lo[j] = j < C::PT ? t[j] : 0u;
              hi[j] = j + 4 < C::PT ? t[j + 4] : 0u;
            }
            transpose4(lo[0], lo[1], lo[2], lo[3]);
            if constexpr (C::PT > 4) transpose4(hi[0], hi[1], hi[2], hi[3]);
            // u = 16 + (t & 15) [+ 256 + 16 (t >> 4)]: start at minus the offsets
            const float gsx = sxs[xcol * gpc + gl];
            const float off = C::PT > 4 ? 272.f : 16.f;
            f32x4 part;
#pragma unroll
            for (int i = 0; i < 4; ++i) part[i] = -off * gsx;
            u32x4 xv[4];
#pragma unroll
            for (int mu = 0; mu < 4; ++mu) xv[mu] = *reinterpret_cast<const u32x4*>(xp + 8 * mu);
#pragma unroll
            for (int a = 0; a < 4; ++a) {
              const bf16x8 xa = as_bf16x8(xv[0][a], xv[1][a], xv[2][a], xv[3][a]);
              part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(nibble_operand(lo[a], m4n, one16),
                                                             xa, part, 0, 0, 0);
              if constexpr (C::PT > 4)
                part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    nibble_operand(hi[a], m4n, one256), xa, part, 0, 0, 0);
            }
            if constexpr (GROUPED) {
              const int g = ck0 / 128 + gl;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int n = row0 + 4 * slot + i;
                const uint32_t aoff = (n < N) ? (uint32_t)(n * G + g) * 4u : 0x80000000u;
                const float ga = __uint_as_float(buf_load4(ar, aoff));
                const float gz = __uint_as_float(buf_load4(zr, aoff));
                tot[i] = tot[i] + (ga * C::STEP) * part[i] - (ga * gz) * gsx;
              }
            } else {
#pragma unroll
              for (int i = 0; i < 4; ++i) tot[i] += part[i];
            }
          }
        }
        // refill this slot after its last use
        const uint32_t o = loff(st + C::DEPTH);
#pragma unroll
        for (int pl = 0; pl < C::PL; ++pl)
          buf[d][pl] = buf_load16(pr, o == 0x80000000u ? o : o + (uint32_t)pl * plane_bytes);
      }
    }
  }

  // ---- sum the K splits in a fixed order, then write y
  __syncthreads();
  if (col < M) {
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(wave * 16 + 4 * slot + i) * M + col] = tot[i];
  }
  __syncthreads();
  {
    const int rr = ep_rr;
    const int rbl2 = rr >> 4, row = rr & 15;
    const int n = rb0 * 16 + rr;
    const int mstep = (64 * kWaves) / rows_wg;
    if (n < N) {
      for (int m = threadIdx.x / rows_wg; m < M; m += mstep) {
        float s = 0.f;
        for (int k2 = 0; k2 < KS; ++k2) s += red[((rbl2 * KS + k2) * 16 + row) * M + m];
        if (!GROUPED) s = ep_a * s - ep_b * sxt[m];
        P.y[(int64_t)m * N + n] = s;
      }
    }
  }
}

// delta swap: exchange the bits of x under m with the bits sh above them
__device__ __forceinline__ uint32_t dswap(uint32_t x, int sh, uint32_t m) {
  const uint32_t t = (x ^ (x >> sh)) & m;
  return x ^ t ^ (t << sh);
}
// 8 x 8 bit transpose of 8 bytes (lo: rows 0-3, hi: rows 4-7, row k = byte
// k): afterwards byte j holds bit j of every row, row k at bit k.  Swaps of
// 1-bit, 2-bit and 4-bit blocks; the last one crosses the two dwords.
__device__ __forceinline__ void transpose8x8(uint32_t& lo, uint32_t& hi) {
  lo = dswap(lo, 7, 0x00AA00AAu);
  hi = dswap(hi, 7, 0x00AA00AAu);
  lo = dswap(lo, 14, 0x0000CCCCu);
  hi = dswap(hi, 14, 0x0000CCCCu);
  const uint32_t t = (lo ^ (hi << 4)) & 0xF0F0F0F0u;
  lo ^= t;
  hi ^= t >> 4;
}

// codes [N][K] -> planes [8][N][K/8]; one thread per output word of a row
// (32 codes: 128G + 32s + 0..31 of a superblock), one word per plane.  Bit
// 16h + i of plane p's word is bit p of code 2i + h: byte permutes
// (v_perm_b32: selector values 0-3 pick bytes of the second source, 4-7 of
// the first) split the even codes from the odd ones, an 8 x 8 bit transpose
// of each group of 8 gives one byte per plane, and a 4 x 4 byte transpose
// places the four bytes of each plane (even codes 0-14, 16-30, odd codes
// 1-15, 17-31).
constexpr int kPackThreads = 256;  // (a constant: blockDim.x is a vector load from the dispatch packet)
__global__ void __launch_bounds__(kPackThreads) pack_bitplanes_kernel(const uint8_t* __restrict__ codes,
                                                             int N, int K,
                                                             uint8_t* __restrict__ planes) {
  const int64_t wpr = K / 32;
  const int64_t total = (int64_t)N * wpr;
  const int64_t plane_words = total;
  uint32_t* out = reinterpret_cast<uint32_t*>(planes);
  for (int64_t t = (int64_t)blockIdx.x * kPackThreads + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * kPackThreads) {
    const int64_t n = t / wpr;
    const int wi = (int)(t - n * wpr);
    const int sb = wi >> 4, s = (wi >> 2) & 3, g = wi & 3;
    const uint8_t* src = codes + n * K + sb * kSuper + 128 * g + 32 * s;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(src);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(src + 16);
    const uint32_t dw[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    // E[j]: even codes 8j .. 8j + 6 of dwords 2j, 2j + 1; O[j]: the odd ones
    uint32_t E[4], O[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      E[j] = __builtin_amdgcn_perm(dw[2 * j + 1], dw[2 * j], 0x06040200u);
      O[j] = __builtin_amdgcn_perm(dw[2 * j + 1], dw[2 * j], 0x07050301u);
    }
    transpose8x8(E[0], E[1]);  // even codes 0-14: byte p = plane p
    transpose8x8(E[2], E[3]);  // even codes 16-30
    transpose8x8(O[0], O[1]);  // odd codes 1-15
    transpose8x8(O[2], O[3]);  // odd codes 17-31
    uint32_t w[8];
#pragma unroll
    for (int half = 0; half < 2; ++half) {  // planes 4 half .. 4 half + 3
      const uint32_t a = __builtin_amdgcn_perm(E[2 + half], E[half], 0x05010400u);
      const uint32_t b = __builtin_amdgcn_perm(E[2 + half], E[half], 0x07030602u);
      const uint32_t c = __builtin_amdgcn_perm(O[2 + half], O[half], 0x05010400u);
      const uint32_t d = __builtin_amdgcn_perm(O[2 + half], O[half], 0x07030602u);
      w[4 * half + 0] = __builtin_amdgcn_perm(c, a, 0x05040100u);
      w[4 * half + 1] = __builtin_amdgcn_perm(c, a, 0x07060302u);
      w[4 * half + 2] = __builtin_amdgcn_perm(d, b, 0x05040100u);
      w[4 * half + 3] = __builtin_amdgcn_perm(d, b, 0x07060302u);
    }
#pragma unroll
    for (int p = 0; p < 8; ++p) out[p * plane_words + t] = w[p];
  }
}

template <int R, bool GROUPED, bool EXTRA>
static hipError_t launch_r(const Args& a, unsigned tiles, size_t lds, hipStream_t s) {
  // the LDS limit is raised once per process (a function-local static is
  // initialized exactly once, also when several host threads launch)
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)bp_gemv_kernel<R, GROUPED, EXTRA>, hipFuncAttributeMaxDynamicSharedMemorySize,
      160 * 1024);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((bp_gemv_kernel<R, GROUPED, EXTRA>), dim3(tiles), dim3(64 * kWaves), lds, s,
                     a);
  return hipGetLastError();
}

template <bool GROUPED, bool EXTRA>
static hipError_t launch_g(int r, const Args& a, unsigned tiles, size_t lds, hipStream_t s) {
  switch (r) {
    case 1: return launch_r<1, GROUPED, EXTRA>(a, tiles, lds, s);
    case 2: return launch_r<2, GROUPED, EXTRA>(a, tiles, lds, s);
    case 3: return launch_r<3, GROUPED, EXTRA>(a, tiles, lds, s);
    case 4: return launch_r<4, GROUPED, EXTRA>(a, tiles, lds, s);
    case 5: return launch_r<5, GROUPED, EXTRA>(a, tiles, lds, s);
    case 6: return launch_r<6, GROUPED, EXTRA>(a, tiles, lds, s);
    case 7: return launch_r<7, GROUPED, EXTRA>(a, tiles, lds, s);
    default: return launch_r<8, GROUPED, false>(a, tiles, lds, s);
  }
}

}  // namespace bp

hipError_t launch_pack_bitplanes(const uint8_t* codes, int64_t N, int64_t K, uint8_t* planes,
                                 hipStream_t s) {
  const int64_t total = N * (K / 32);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(bp::pack_bitplanes_kernel, dim3((unsigned)blocks), dim3(bp::kPackThreads), 0, s, codes,
                     (int)N, (int)K, planes);
  return hipGetLastError();
}

hipError_t launch_gemv_bitplanes(const uint8_t* planes, int r, bool extra, const float* alpha,
                                 const float* zero, int64_t group, int64_t N, int64_t K,
                                 const uint16_t* x, int64_t M, float* y, hipStream_t s) {
  bp::Args a;
  a.planes = planes;
  a.alpha = alpha;
  a.zero = zero;
  a.x = x;
  a.y = y;
  a.N = (int)N;
  a.K = (int)K;
  a.group = (int)group;
  a.M = (int)M;
  // activation chunk: at most 32 KiB of staged bf16, a multiple of 512 codes
  int kc = (int)((16384 / M) / bp::kSuper * bp::kSuper);
  if (kc < bp::kSuper) kc = bp::kSuper;
  if (kc > K) kc = (int)K;
  a.kc = kc;
  // split of the superblocks among the waves of a row block: enough waves in
  // flight to cover the memory latency, at least two superblocks per wave
  const int rblocks = (int)((N + 15) / 16);
  const int steps = (int)(K / bp::kSuper);
  int ks = 1;
  while (ks < bp::kWaves && rblocks * ks < 4096 && steps / (ks * 2) >= 2) ks *= 2;
  a.ks = ks;
  const int rbpw = bp::kWaves / ks;
  const unsigned tiles = (unsigned)((rblocks + rbpw - 1) / rbpw);
  const int gpc = kc / 128;
  const size_t lds = (size_t)M * (kc + bp::kXPad) * 2 + (size_t)(M * gpc + kSkinnyMaxM) * 4 +
                     (size_t)bp::kWaves * 16 * M * 4;
  const bool grouped = group != K;
  const bool ex = extra && r < 8;
  if (grouped)
    return ex ? bp::launch_g<true, true>(r, a, tiles, lds, s)
              : bp::launch_g<true, false>(r, a, tiles, lds, s);
  return ex ? bp::launch_g<false, true>(r, a, tiles, lds, s)
            : bp::launch_g<false, false>(r, a, tiles, lds, s);
}

}  // namespace mq
