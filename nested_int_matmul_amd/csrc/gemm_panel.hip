// Small-batch product (9 <= M <= 64 activation rows) against r-bit planes:
//   y[m, n] = sum_k x[m, k] (S(q[n, k], r) - z[n, g]) alpha[n, g]
// ("Matryoshka Quantization" explainer, §3.4: Eq. 6 slicing, Eq. 1
// dequantization).  At these M the product still streams the planes out of
// HBM (every packed byte is used M times, on the matrix cores).
//
// Design (gfx950, v_mfma_f32_16x16x32_bf16, A = weights, B = activations):
//  - A workgroup owns a panel of 256 weight rows (8 waves x two 16-row
//    blocks) and a slice of K of at most 1024 codes; or, at M <= 16, a panel
//    of 64 rows (four 16-row blocks x two halves of the slice) and a slice of
//    up to 4096 codes, which at K <= 4096 is all of K.  The activations of
//    the slice (all M rows, padded to 16 * MB) are brought into LDS once with
//    buffer-to-LDS loads; the per-128 sums of x are formed from LDS.
//  - Four lanes share a weight row and load 16 contiguous packed bytes each
//    per step, so one load instruction reads 64 contiguous bytes of each of
//    16 rows (measured: 32-byte row pieces per instruction stream HBM at
//    about two thirds of the rate of 64-byte pieces).  The bytes go straight
//    into registers (every row has one reader), DEPTH steps ahead of use,
//    and are unpacked into exact bf16 integers (mq_device.h); one unpacked
//    operand feeds MB matrix-core products (16 activation rows each).
//    r = 3 and 6 (a high-bit and a low-bit plane) take 32 codes per lane per
//    step from both planes and assemble u = 2^r + t in the same registers.
//  - r = 2 with groups of 128: a step (256 codes of a row) spans two groups,
//    lanes 0-31 holding the first and lanes 32-63 the second; half of each
//    lane's words are exchanged with the lane 32 away (v_permlane32_swap) so
//    that every product takes codes of one group only.
//  - alpha and z of the panel's groups are staged in LDS with the
//    activations; group-128 scales are applied at each group end in fp32
//    (y += alpha 2^(8-r) P_g - alpha (z + shift) sum_g x), per-channel scales
//    once at the end.
//  - The two halves of a 64-row panel's slice are summed in LDS, the first
//    half's sums then the second's.  When K is split over several
//    workgroups, each writes its fp32 partial tile to the workspace and a
//    second kernel sums the slices in a fixed order (deterministic).
#include <algorithm>

#include "mq_device.h"
#include "mq_internal.h"

namespace mq {

namespace panel {

constexpr int kKSlice = 1024;          // codes of K per workgroup when K is split over workgroups
constexpr int kKFull = 4096;           // codes of K per workgroup of the 64-row panels (M <= 16)
constexpr int kXPadE = 8;              // bf16 padding per staged activation row
constexpr int kNW = 8;                 // waves per workgroup

// Workgroup shapes (K in slices over blockIdx.y; when there are several,
// reduce_slices sums the partials in slice order):
//  - 8 waves x two 16-row blocks = 256 weight rows, slices of kKSlice codes;
//  - M <= 16: 4 row blocks x 2 halves of the slice = 64 weight rows, slices
//    of kKFull codes (one slice up to K = 4096); the two halves are summed
//    in LDS (fixed order).
template <int KSL, int RBW, int KH>
struct Shape {
  static constexpr int WPK = kNW / KH;         // waves per part of K
  static constexpr int ROWS_WG = WPK * RBW * 16;  // weight rows per workgroup
  static constexpr int GPS = KSL / 128;        // groups of 128 per slice
};

template <int R, bool GROUPED>
struct Pc {
  // r = 3 and 6: a high-bit and a low-bit plane (rows of the high plane, then
  // rows of the low plane), 32 codes per lane per step from each
  static constexpr bool SPLIT = (R == 3 || R == 6);
  static constexpr int RL = R == 6 ? 2 : 1, RH = R - RL;  // split: plane widths
  static constexpr int CPL = SPLIT ? 32 : 16 * 8 / R;    // codes per lane per step
  static constexpr int STEP = 4 * CPL;      // codes per row per step (four lanes)
  static constexpr int MFMAS = CPL / 8;     // 32-deep products per step per operand pair
  static constexpr bool SWAP = (R == 2 && GROUPED);      // two groups per step
  static constexpr int SPG = STEP >= 128 ? 1 : 128 / STEP;  // steps per group (r = 8: 2)
  using LD = LoadT<R, SPLIT ? 0 : 16>;      // one lane's loads of a step
};
// weight loads in flight per lane and row block: 4 steps (or the wave's
// whole share when shorter).  With the refills issued on every trip the wait
// at the loop head is exact, and 4 measured best: at M = 16 against 8,
// 14336 x 4096 r = 2 10.3 -> 9.4 us and 4096 x 14336 r = 4 / 2 13.1 -> 12.4 /
// 12.2 -> 11.2 us; at M = 64, r = 4, 24.4 -> 23.2 us (2, 3, 6 and 12 no
// better)
template <int R, bool GROUPED, int KSL, int KH>
constexpr int depth() {
  using C = Pc<R, GROUPED>;
  return KSL / (C::STEP * KH) < 4 ? KSL / (C::STEP * KH) : 4;
}

struct Args {
  const uint8_t* packed;
  const float* alpha;
  const float* zero;
  const uint16_t* x;
  float* y;     // output [M, N] (one K slice) or the partial slices [S][M][N]
  int M, N, K, G;
  int ksl;      // codes per K slice: <= the shape's KSL, a multiple of 512 when K is split
};

__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void lds_dma4(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)lds, 4, voff, 0, 0, 0);
}

template <int R>
__device__ __forceinline__ bf16x8 unpack_b(const uint32_t* d, int i, const UnpackK& k,
                                           const UnpackK36& k36) {
  if (R == 4) return unpack_r4(d[i], k);
  if (R == 2) return (i & 1) ? unpack_r2<1>(d[i >> 1], k) : unpack_r2<0>(d[i >> 1], k);
  if (R == 6) return unpack_r6(d[i], d[4 + (i >> 1)], i & 1, k36);  // 4 high, 2 low words
  if (R == 3) return unpack_r3(d[i >> 1], d[2], i, k36);             // 2 high, 1 low word
  return unpack_r8(d[2 * i], d[2 * i + 1]);
}

template <int R, int MB, bool GROUPED, int KSL, int RBW, int KH>
__global__ void __launch_bounds__(64 * kNW) panel_kernel(const Args a) {
  using C = Pc<R, GROUPED>;
  using S = Shape<KSL, RBW, KH>;
  constexpr int ROWS = 16 * MB;   // staged activation rows
  constexpr int DEPTH = depth<R, GROUPED, KSL, KH>();
  constexpr int ROWS_WG = S::ROWS_WG, GPS = S::GPS;
  extern __shared__ __align__(16) unsigned char smem[];

  // the wave index is uniform: in a scalar register, the loop bounds below
  // and every branch on them are scalar
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, slot = lane >> 4;
  const int wrow = wave % S::WPK, kh = wave / S::WPK;  // row group and part of K of this wave
  const int M = a.M, N = a.N, K = a.K, G = a.G;
  const int ksl = min(a.ksl, KSL);  // (bounded by KSL in the code, so that loops over the
                                    //  slice's groups keep a known trip count)
  const int k0 = (int)blockIdx.y * ksl;
  const int klen = min(ksl, K - k0);
  const int ngl = (klen + 127) >> 7;              // groups of 128 in the slice
  const int steps = (klen + C::STEP - 1) / C::STEP;
  // this wave's steps: all of the slice, or one of KH parts in whole groups
  int s0 = 0, s1 = steps;
  if (KH > 1) {
    const int units = steps / C::SPG;
    s0 = (units * kh / KH) * C::SPG;
    s1 = (units * (kh + 1) / KH) * C::SPG;
  }
  constexpr int xstride = KSL + kXPadE;           // elements

  // the small arrays first, so that their reads take immediate offsets (under
  // 64 KiB), the staged activations after them
  float* azs = reinterpret_cast<float*>(smem);  // [2][GPS][ROWS_WG] (staged as [2][ROWS_WG][GPS])
  float* sxs = azs + 2 * ROWS_WG * GPS;         // [ngl][ROWS]
  float* red = sxs + GPS * ROWS;  // KH = 2: [WPK][64][RBW][MB][4] second half's sums
  uint16_t* xs = reinterpret_cast<uint16_t*>(red + (KH == 2 ? S::WPK * 64 * RBW * MB * 4 : 0));
  // [ROWS][xstride]

  const int n0 = (int)blockIdx.x * ROWS_WG;
  const int rowbytes = K * R / 8;
  const uint32_t plane = (uint32_t)((int64_t)N * rowbytes);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.packed, plane);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, (uint32_t)((int64_t)M * K * 2));

  // The loads are issued in the order the workgroup needs them: the staged
  // activations and group scales (which the first barrier waits for), then
  // the weights (which it does not).  Every loop here is unrolled, so no
  // wait is placed before a load is issued.
  // ---- activations of the slice: 1 KiB pieces (512 codes) of each row,
  //      one per wave instruction; rows past M and columns past K read zeros
  constexpr int PPR = KSL / 512;  // pieces per row
#pragma unroll
  for (int q = 0; q < ROWS * PPR / kNW; ++q) {
    const int pc = wave + q * kNW;
    const int m = pc / PPR, j = pc % PPR;
    const int k = k0 + j * 512 + lane * 8;
    const uint32_t off =
        (m < M && k < k0 + klen) ? (uint32_t)(((int64_t)m * K + k) * 2) : 0x80000000u;
    lds_dma16(xr, xs + (size_t)m * xstride + j * 512, off);
  }
  // ---- group-128 scales of the panel staged in LDS as
  //      [alpha | zero][row][group of the slice] by 4-byte buffer-to-LDS
  //      loads (entries past N or past the slice read zeros)
  if (GROUPED) {
    const __amdgpu_buffer_rsrc_t ar = make_rsrc(a.alpha, (uint32_t)((int64_t)N * G * 4));
    const __amdgpu_buffer_rsrc_t zr = make_rsrc(a.zero, (uint32_t)((int64_t)N * G * 4));
    const int g0 = k0 >> 7;
#pragma unroll
    for (int e = 0; e < ROWS_WG * GPS / (64 * kNW); ++e) {
      const int base = (wave + e * kNW) * 64;  // ROWS_WG rows x GPS groups, one entry per lane
      const int idx = base + lane;
      const int rr = idx / GPS, gg = idx % GPS;
      const int nn = n0 + rr;
      const uint32_t off =
          (nn < N && gg < ngl) ? (uint32_t)(((int64_t)nn * G + g0 + gg) * 4) : 0x80000000u;
      lds_dma4(ar, azs + base, off);
      lds_dma4(zr, azs + ROWS_WG * GPS + base, off);
    }
  }

  // every wave has issued its activation and scale loads before any wave
  // issues weight loads, so that the staged data (cache hits) is not queued
  // behind weight requests to HBM (no wait here: the loads stay in flight);
  // measured at M = 16: 12.7 -> 12.0 us (14336 x 4096, r = 4)
  __builtin_amdgcn_s_barrier();

  // ---- the first DEPTH weight loads of both row blocks
  // split planes: the lane's high-plane bytes, and its low-plane bytes after
  // all N rows of the high plane
  constexpr int WH = C::SPLIT ? C::RH : R;  // bits per code in the (high) plane
  const uint32_t hrow = (uint32_t)(K * WH / 8), lrow = (uint32_t)(K * C::RL / 8);
  uint32_t base_hi[RBW], base_lo[RBW];
#pragma unroll
  for (int b = 0; b < RBW; ++b) {
    const int n = n0 + wrow * RBW * 16 + b * 16 + col;  // weight row this lane loads
    const uint32_t kb = (uint32_t)((k0 + slot * C::CPL) * WH / 8);
    base_hi[b] = n < N ? (uint32_t)n * hrow + kb : plane;
    base_lo[b] = n < N ? (uint32_t)N * hrow + (uint32_t)n * lrow +
                             (uint32_t)((k0 + slot * C::CPL) * C::RL / 8)
                       : plane;
  }
  auto loff = [&](int b, int st) -> uint32_t {
    return st < s1 ? base_hi[b] + (uint32_t)(st * (C::STEP * WH / 8)) : 0x80000000u;
  };
  auto loff_lo = [&](int b, int st) -> uint32_t {
    return st < s1 ? base_lo[b] + (uint32_t)(st * (C::STEP * C::RL / 8)) : 0x80000000u;
  };
  using LD = typename C::LD;
  typename LD::T buf[RBW][DEPTH];
#pragma unroll
  for (int j = 0; j < DEPTH; ++j)
#pragma unroll
    for (int b = 0; b < RBW; ++b) buf[b][j] = LD::load(wr, loff(b, s0 + j), loff_lo(b, s0 + j));

  // per-channel scales of this lane's output rows (needed at the end only;
  // issued after the weights so that no wait before the loop covers them)
  float pa[RBW][4], pz[RBW][4];
  if (!GROUPED) {
#pragma unroll
    for (int b = 0; b < RBW; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int n = n0 + wrow * RBW * 16 + b * 16 + 4 * slot + e;
        const int nc = n < N ? n : N - 1;
        pa[b][e] = a.alpha[nc];
        pz[b][e] = a.zero[nc];
      }
  }
  __syncthreads();

  // ---- group factors: alpha 2^(8-r) and -alpha (z + shift), transposed to
  //      [group][row] so that a lane's four consecutive output rows are one
  //      16-byte read.  Each wave instruction takes 64 rows on a diagonal of
  //      the groups (row rbase + lane, group (lane / Q + c) mod GPS): its reads
  //      of the [row][group] layout fall on 64 distinct banks, its writes on
  //      64 consecutive words.  All reads are done before a barrier, the
  //      writes after it (the transpose is in place).
  constexpr int kTr = ROWS_WG * GPS / (64 * kNW);  // entries per thread
  static_assert(ROWS_WG * GPS == kTr * 64 * kNW && 64 % GPS == 0 && ROWS_WG % 64 == 0,
                "the diagonal transpose covers the panel's scales exactly");
  float tav[kTr], tnb[kTr];
  int tdst[kTr];
  if (GROUPED) {
    constexpr int Q = 64 / GPS;
#pragma unroll
    for (int k = 0; k < kTr; ++k) {
      const int q = wave + k * kNW;
      const int r = (q / GPS) * 64 + lane, g = (lane / Q + q % GPS) % GPS;
      const float al = azs[r * GPS + g], ze = azs[ROWS_WG * GPS + r * GPS + g];
      tav[k] = al * Enc<R>::kStep;
      tnb[k] = -al * (ze + Enc<R>::kOffsetShift);
      tdst[k] = g * ROWS_WG + r;
    }
  }

  // ---- per-128 sums of the staged activations: one thread per (row,
  //      group) sums its 16 chunks of 8 in order (no cross-lane reduction;
  //      consecutive lanes take consecutive rows, whose 16-byte reads fall
  //      on distinct banks)
  {
    const uint32_t ones = 0x3F803F80u;
    for (int t = tid; t < ROWS * ngl; t += 64 * kNW) {
      const int m = t % ROWS, gl = t / ROWS;
      const uint16_t* p = xs + (size_t)m * xstride + gl * 128;
      u32x4 w[16];
#pragma unroll
      for (int c = 0; c < 16; ++c) w[c] = *reinterpret_cast<const u32x4*>(p + c * 8);
      float sp = 0.f;
#pragma unroll
      for (int c = 0; c < 16; ++c)
#pragma unroll
        for (int q = 0; q < 4; ++q) sp = dot2_bf16(w[c][q], ones, sp);
      sxs[gl * ROWS + m] = sp;
    }
  }
  if (GROUPED) {
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kTr; ++k) {
      azs[tdst[k]] = tav[k];
      azs[ROWS_WG * GPS + tdst[k]] = tnb[k];
    }
  }
  __syncthreads();

  // ---- stream the slice
  const UnpackK uk = UnpackK::make();
  UnpackK36 uk36;
  if constexpr (C::SPLIT) uk36 = UnpackK36::make();
  // accumulators: lane holds rows 4 * slot + e of each 16-row block, for
  // activation row mb * 16 + col; per-channel: acc only; group-128: part
  // collects one group (two at r = 2: part and part2), acc the scaled sum
  f32x4 acc[RBW][MB], part[RBW][MB], part2[RBW][MB];
#pragma unroll
  for (int b = 0; b < RBW; ++b)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[b][mb][e] = 0.f;
        part[b][mb][e] = 0.f;
        part2[b][mb][e] = 0.f;
      }
  // this lane's activation column offset within a step: the codes it
  // multiplies are those of its own 16-byte piece (slot * CPL ...), or at
  // r = 2 with groups, after the exchange, the first group's codes at xa_sw
  // (products 0-3) and the second group's 128 codes later (products 4-7)
  const int xa_sw = slot < 2 ? 64 * slot + 32 : 64 * (slot - 2);
  const uint16_t* xa = xs + (size_t)col * xstride + (C::SWAP ? xa_sw : slot * C::CPL);

  // group end: acc += alpha 2^(8-r) * P - alpha (z + shift) * sum_g x for
  // the lane's four rows of each block (both factors formed once above),
  // then the group's products restart
  auto group_end = [&](int gl, f32x4 (&p)[RBW][MB]) {
    if (gl < ngl) {
#pragma unroll
      for (int b = 0; b < RBW; ++b) {
        const float* azr = azs + gl * ROWS_WG + wrow * RBW * 16 + b * 16 + 4 * slot;
        // alpha 2^(8-r) and -alpha (z + shift) of the lane's four rows
        const f32x4 av = *reinterpret_cast<const f32x4*>(azr);
        const f32x4 nb = *reinterpret_cast<const f32x4*>(azr + ROWS_WG * GPS);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const float sx = sxs[gl * ROWS + mb * 16 + col];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[b][mb][e] = fmaf(av[e], p[b][mb][e], fmaf(nb[e], sx, acc[b][mb][e]));
        }
      }
    }
#pragma unroll
    for (int b = 0; b < RBW; ++b)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) p[b][mb][e] = 0.f;
  };

#pragma unroll 1
  for (int base = s0; base < s1; base += DEPTH) {
#pragma unroll
    for (int j = 0; j < DEPTH; ++j) {
      const int st = base + j;
      if (st < s1) {
        uint32_t d[RBW][LD::NW];
#pragma unroll
        for (int b = 0; b < RBW; ++b) {
          LD::words(buf[b][j], d[b]);
          if constexpr (C::SWAP) {
            // after the exchange words 0-1 hold first-group codes and words
            // 2-3 second-group codes in every lane
            const auto s02 = __builtin_amdgcn_permlane32_swap(d[b][2], d[b][0], false, false);
            const auto s13 = __builtin_amdgcn_permlane32_swap(d[b][3], d[b][1], false, false);
            d[b][0] = s02[0];
            d[b][1] = s13[0];
            d[b][2] = s02[1];
            d[b][3] = s13[1];
          }
        }
        const uint16_t* xp = xa + st * C::STEP;
#pragma unroll
        for (int i = 0; i < C::MFMAS; ++i) {
          bf16x8 xv[MB];
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            const int xo = C::SWAP ? 8 * (i & 3) + 128 * (i >> 2) : 8 * i;
            xv[mb] = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const u32x4*>(xp + (size_t)mb * 16 * xstride + xo));
          }
#pragma unroll
          for (int b = 0; b < RBW; ++b) {
            const bf16x8 w = unpack_b<R>(d[b], i, uk, uk36);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
              if (!GROUPED)
                acc[b][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w, xv[mb], acc[b][mb], 0, 0, 0);
              else if (C::SWAP && i >= 4)
                part2[b][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w, xv[mb], part2[b][mb], 0, 0, 0);
              else
                part[b][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w, xv[mb], part[b][mb], 0, 0, 0);
            }
          }
        }
        if constexpr (GROUPED) {
          if constexpr (C::SWAP) {
            group_end(2 * st, part);
            group_end(2 * st + 1, part2);
          } else if ((j % C::SPG) == C::SPG - 1) {
            group_end(st / C::SPG, part);
          }
        }
      }
      // refill this slot after its last use; past the wave's steps the
      // offset points past the plane (zeros, no memory traffic), so every
      // trip issues the same loads and the waits stay exact across trips
#pragma unroll
      for (int b = 0; b < RBW; ++b)
        buf[b][j] = LD::load(wr, loff(b, st + DEPTH), loff_lo(b, st + DEPTH));
    }
  }

  // ---- two parts of K: the second half's sums go through LDS and are
  //      added to the first's (fixed order); the first half's waves store
  if constexpr (KH == 2) {
    float* rw = red + (size_t)(wrow * 64 + lane) * RBW * MB * 4;
    if (kh == 1) {
#pragma unroll
      for (int b = 0; b < RBW; ++b)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          *reinterpret_cast<f32x4*>(rw + (b * MB + mb) * 4) = acc[b][mb];
    }
    __syncthreads();
    if (kh == 1) return;
#pragma unroll
    for (int b = 0; b < RBW; ++b)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[b][mb] += *reinterpret_cast<const f32x4*>(rw + (b * MB + mb) * 4);
  }

  // ---- epilogue: lane holds rows n = row block + 4 * slot + e (e = 0..3)
  //      of activation row m = mb * 16 + col
  float* out = a.y + (size_t)blockIdx.y * M * N;
  const bool vec = (N & 3) == 0;
  // device-scope (write-through) stores of the tile: measured faster at
  // M = 64 for r <= 6 (14336 x 4096 r = 4 / 2 / 3: 23.1-23.5 / 24.9 / 28.2 ->
  // 22.0-22.4 / 22.5 / 26.2-26.5 us with the slice sum), slower at r = 8 and
  // at M = 32 (27.8-28.5 -> 28.8-29.1 us; 16.0 -> 16.5 us), where plain
  // stores are kept
  constexpr bool kWriteThrough = R < 8 && MB == 4;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    // the block's 16 output rows from its first row at column n0: at most
    // 16 N floats (N <= 2^25, so under 2^31 bytes)
    const __amdgpu_buffer_rsrc_t orr =
        make_rsrc(out + (size_t)mb * 16 * N + n0, (uint32_t)(16 * (int64_t)N * 4));
    const int m = mb * 16 + col;
    if (m >= M) continue;
    float tot = 0.f;
    if (!GROUPED) {
      for (int gl = 0; gl < ngl; ++gl) tot += sxs[gl * ROWS + m];
    }
#pragma unroll
    for (int b = 0; b < RBW; ++b) {
      const int nb0 = n0 + wrow * RBW * 16 + b * 16 + 4 * slot;
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        v[e] = GROUPED ? acc[b][mb][e]
                       : pa[b][e] * Enc<R>::kStep * acc[b][mb][e] -
                             pa[b][e] * (pz[b][e] + Enc<R>::kOffsetShift) * tot;
      float* o = out + (size_t)m * N + nb0;
      if (vec && nb0 + 3 < N) {
        if (kWriteThrough) store_out16(orr, (uint32_t)((col * (int64_t)N + nb0 - n0) * 4), v);
        else *reinterpret_cast<f32x4*>(o) = v;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (nb0 + e < N) o[e] = v[e];
      }
    }
  }
}

// y = sum over S slices of the partial tiles, in slice order.  16-byte
// vectors only when every slice starts 16-byte aligned (count % 4 == 0).  The
// slices of an element are loaded kReduceBatch at a time, all issued before
// the first is added (a slice per memory latency otherwise), and added in
// slice order.
constexpr int kReduceBatch = 8;

constexpr int kReduceThreads = 256;  // (a constant: blockDim.x is a vector load)
__global__ void __launch_bounds__(kReduceThreads) reduce_slices(const float* __restrict__ part,
                                                     float* __restrict__ y, int64_t count,
                                                     int S) {
  const int64_t stride = (int64_t)gridDim.x * kReduceThreads;
  const int64_t n4 = (count & 3) ? 0 : count >> 2;
  const f32x4* p4 = reinterpret_cast<const f32x4*>(part);
  for (int64_t i0 = (int64_t)blockIdx.x * kReduceThreads; i0 < n4; i0 += stride) {
    // this trip's kReduceThreads vectors from a uniform base
    const int64_t i = i0 + threadIdx.x;
    if (i >= n4) break;
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(y + 4 * i0, kReduceThreads * 16);
    f32x4 v = p4[i];
    for (int s0 = 1; s0 < S; s0 += kReduceBatch) {
      f32x4 t[kReduceBatch];
#pragma unroll
      for (int b = 0; b < kReduceBatch; ++b)
        if (s0 + b < S) t[b] = p4[(int64_t)(s0 + b) * n4 + i];
#pragma unroll
      for (int b = 0; b < kReduceBatch; ++b)
        if (s0 + b < S) v += t[b];
    }
    store_out16(yr, (uint32_t)threadIdx.x * 16, v);
  }
  for (int64_t i = (n4 << 2) + (int64_t)blockIdx.x * kReduceThreads + threadIdx.x; i < count;
       i += stride) {
    float v = part[i];
    for (int s0 = 1; s0 < S; s0 += kReduceBatch) {
      float t[kReduceBatch];
#pragma unroll
      for (int b = 0; b < kReduceBatch; ++b)
        if (s0 + b < S) t[b] = part[(int64_t)(s0 + b) * count + i];
#pragma unroll
      for (int b = 0; b < kReduceBatch; ++b)
        if (s0 + b < S) v += t[b];
    }
    store_out(y + i, v);
  }
}

}  // namespace panel

// ---------------------------------------------------------------------------
// Host planning
// ---------------------------------------------------------------------------

struct PanelPlan {
  int slices, panels;
  int ksl;    // codes per slice: the slices of a split are equal (multiples of 512)
  bool wide;  // 64-row panels over slices of kKFull codes (halves of a slice summed in LDS)
};

// At M <= 16 the activations of kKFull codes fit in LDS, so a workgroup can
// take a 64-row panel over a slice of up to 4096 codes, in whole 512-code
// pieces: at N >= 12288 and K <= 4096 that is all of K (no partial slices,
// no second launch), at the 4096-wide down projection (K = 14336) four
// slices instead of fourteen.  It is used when its workgroups fill the chip
// (192 or more); otherwise 256-row panels over slices of kKSlice codes.
static PanelPlan plan_panel(int64_t M, int64_t N, int64_t K) {
  PanelPlan p;
  using W = panel::Shape<panel::kKFull, 1, 2>;
  const int64_t wpanels = (N + W::ROWS_WG - 1) / W::ROWS_WG;
  const int64_t wslices = (K + panel::kKFull - 1) / panel::kKFull;
  p.wide = M <= 16 && K % 512 == 0 && wpanels * wslices >= 192;
  if (p.wide) {
    p.panels = (int)wpanels;
    p.slices = (int)wslices;
    p.ksl = panel::kKFull;
  } else {
    using S = panel::Shape<panel::kKSlice, 2, 1>;
    p.panels = (int)((N + S::ROWS_WG - 1) / S::ROWS_WG);
    // K slice: the largest the activations allow in LDS at M = 64 (1024
    // codes): longer workgroups and fewer partial slices measured faster
    // than more, shorter ones at the Mistral shapes (M = 16 and 64)
    p.slices = (int)((K + panel::kKSlice - 1) / panel::kKSlice);
    p.ksl = panel::kKSlice;
  }
  // equal slices, so that no workgroup streams a longer K than the others
  // (14336 in four slices of 3584, not 3 x 4096 + 2048); each a multiple of
  // 512 codes (whole activation pieces and groups), at most the shape's
  if (p.slices > 1) {
    const int64_t per = (K + p.slices - 1) / p.slices;
    p.ksl = (int)std::min<int64_t>((per + 511) / 512 * 512, p.ksl);
  }
  return p;
}

size_t panel_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const PanelPlan p = plan_panel(M, N, K);
  return p.slices > 1 ? (size_t)p.slices * M * N * 4 : 0;
}

template <int R, int MB, bool GROUPED, int KSL, int RBW, int KH>
static hipError_t launch_panel_t(const panel::Args& a, const PanelPlan& p, hipStream_t s) {
  using namespace panel;
  using S = Shape<KSL, RBW, KH>;
  const size_t lds = (size_t)16 * MB * (KSL + kXPadE) * 2 + (size_t)S::GPS * 16 * MB * 4 +
                     (size_t)2 * S::ROWS_WG * S::GPS * 4 +
                     (KH == 2 ? (size_t)S::WPK * 64 * RBW * MB * 4 * 4 : 0);
  // the LDS limit is raised once per process (a function-local static is
  // initialized exactly once, also when several host threads launch)
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)panel_kernel<R, MB, GROUPED, KSL, RBW, KH>,
      hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((panel_kernel<R, MB, GROUPED, KSL, RBW, KH>), dim3(p.panels, p.slices),
                     dim3(64 * kNW), lds, s, a);
  return hipGetLastError();
}

// activation rows in blocks of 16: 1, 2 or 4 blocks (33 <= M <= 48 takes 4)
template <int R>
static hipError_t launch_panel_r(const panel::Args& a, const PanelPlan& p, bool grouped,
                                 hipStream_t s) {
  using namespace panel;
  if (p.wide)
    return grouped ? launch_panel_t<R, 1, true, kKFull, 1, 2>(a, p, s)
                   : launch_panel_t<R, 1, false, kKFull, 1, 2>(a, p, s);
  if (a.M <= 16)
    return grouped ? launch_panel_t<R, 1, true, kKSlice, 2, 1>(a, p, s)
                   : launch_panel_t<R, 1, false, kKSlice, 2, 1>(a, p, s);
  if (a.M <= 32)
    return grouped ? launch_panel_t<R, 2, true, kKSlice, 2, 1>(a, p, s)
                   : launch_panel_t<R, 2, false, kKSlice, 2, 1>(a, p, s);
  return grouped ? launch_panel_t<R, 4, true, kKSlice, 2, 1>(a, p, s)
                 : launch_panel_t<R, 4, false, kKSlice, 2, 1>(a, p, s);
}

hipError_t launch_gemm_panel(const uint8_t* packed, int r, const float* alpha, const float* zero,
                             int64_t group, int64_t N, int64_t K, const uint16_t* x, int64_t M,
                             float* y, void* workspace, hipStream_t s) {
  const PanelPlan p = plan_panel(M, N, K);
  panel::Args a;
  a.packed = packed;
  a.alpha = alpha;
  a.zero = zero;
  a.x = x;
  a.y = p.slices > 1 ? static_cast<float*>(workspace) : y;
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  a.G = (int)(K / group);
  a.ksl = p.ksl;
  const bool grouped = group != K;
  hipError_t e;
  switch (r) {
    case 2: e = launch_panel_r<2>(a, p, grouped, s); break;
    case 3: e = launch_panel_r<3>(a, p, grouped, s); break;
    case 4: e = launch_panel_r<4>(a, p, grouped, s); break;
    case 6: e = launch_panel_r<6>(a, p, grouped, s); break;
    default: e = launch_panel_r<8>(a, p, grouped, s); break;
  }
  if (e != hipSuccess || p.slices == 1) return e;
  return launch_reduce_slices(static_cast<const float*>(workspace), y, M * N, p.slices, s);
}

hipError_t launch_reduce_slices(const float* part, float* y, int64_t count, int S, hipStream_t s) {
  const int blocks = (int)std::min<int64_t>((count / 4 + 255) / 256 + 1, 2048);
  hipLaunchKernelGGL(panel::reduce_slices, dim3(blocks), dim3(panel::kReduceThreads), 0, s, part, y, count, S);
  return hipGetLastError();
}

}  // namespace mq
