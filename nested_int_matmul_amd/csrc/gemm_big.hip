// Batched product (M >= 65 activation rows, up to prefill sizes) against
// r-bit planes on bf16 matrix cores:
//   y[m, n] = sum_g alpha[n, g] * (2^(8-r) * sum_{k in g} x[m, k] u[n, k]
//                                   - (z[n, g] + shift) * sum_{k in g} x[m, k])
// with u the exact bf16 operand of the index t (mq_device.h), which equals
// sum_k x[m, k] (S(q[n, k], r) - z[n, g]) alpha[n, g]
// ("Matryoshka Quantization" explainer, §3.4: Eq. 6 and Eq. 1).
//
// Tiling (gfx950, v_mfma_f32_32x32x16_bf16, A = activations, B = weights):
//  - a workgroup of 8 waves computes a BM x 256 tile of y (BM = 256, or 128
//    up to M = 128, where a 256-row tile would be half padding); each wave
//    owns a BM/2 (m) x 64 (n) sub-tile = BM/64 x 2 blocks of 32 x 32 (128 or
//    64 fp32 accumulators per lane);
//  - each K iteration covers 64 codes: the activation tile (BM x 64 bf16) and
//    the packed weight tile (256 rows x 64 codes) are brought into LDS with
//    buffer-to-LDS loads, double-buffered, one barrier per iteration; the
//    activation and weight tiles are XOR-swizzled in 16-byte chunks so that
//    the operand reads of 16 consecutive rows hit distinct banks;
//  - one accumulator set carries all groups: at the end of group g it holds
//    C_g = P_g + (running total) / a_g in units of 1/a_g (a_g = alpha * 2^(8-r));
//    the group's zero-point term is subtracted in those units and the set is
//    rescaled to the next group's units by alpha_g / alpha_{g+1}
//    (two VALU operations per accumulator per group, and the accumulator
//    stays centred, which keeps fp32 cancellation small);
//  - the per-group row sums of x come from the staged tiles (v_dot2);
//  - the scales and zero points reach LDS in windows of 4 groups (16 bytes
//    of a column per lane), double-buffered: read per group from global
//    memory, each column's value is a cache line of its own (columns are G
//    floats apart);
//  - r = 3 and 6 stage a high-plane and a low-plane sub-tile per iteration
//    and assemble u = 2^r + t from both (8-byte low rows at r = 3 go through
//    4-byte buffer-to-LDS loads);
//  - tiles are mapped to XCDs so that the workgroups of one XCD share
//    activation rows (its L2 keeps them);
//  - when the tiles alone leave CUs idle (few rows of y or of n, e.g. a
//    4096-wide down projection), K is split over blockIdx.y into slices of
//    whole groups; each slice ends in absolute units with its own last
//    group's scale, and the slices are summed in slice order afterwards.
#include "mq_device.h"
#include "mq_internal.h"

namespace mq {

namespace big {

constexpr int BN = 256, BK = 64;
constexpr int WAVES = 8, THREADS = 64 * WAVES;
constexpr int NB = 2;  // 32x32 blocks per wave along n
// BM = 256 or 128 rows per tile (the 128-row tiles for small M)
template <int R, int BM>
struct Cfg {
  static constexpr int MB = BM / 64;          // 32x32 blocks per wave along m (2 m-waves)
  static constexpr int XT_BYTES = BM * BK * 2;  // staged activation tile
  // r = 3 and 6: a high-bit plane (rows of K * RH / 8 bytes) followed by a
  // low-bit plane (rows of K * RL / 8 bytes); staged as two sub-tiles
  static constexpr bool SPLIT = (R == 3 || R == 6);
  static constexpr int RL = SPLIT ? (R == 6 ? 2 : 1) : 0, RH = R - RL;
  static constexpr int WROW = BK * RH / 8;  // (high-)plane bytes per weight row per iteration
  static constexpr int WLOW = BK * RL / 8;  // low-plane bytes per weight row per iteration
  static constexpr int LO_OFF = BN * WROW;  // low sub-tile within a stage
  static constexpr int WT_BYTES = BN * (WROW + WLOW);
  static constexpr int LDS = 2 * XT_BYTES + 2 * WT_BYTES + BM * 4;
  // group-128 scales: + [2 windows][alpha, zero][BN columns][4 groups] fp32
  static constexpr int LDS_GROUPED = LDS + 2 * 2 * BN * 4 * 4;
};

// LDS swizzles (16-byte chunks).  Operand reads serve 16 lanes per cycle
// (256 bytes); both swizzles keep those lanes on distinct banks, and also the
// 8-lane groups of a 128-byte cycle.
//  - activations, row r (128 bytes): logical chunk c sits at c ^ xsw(r);
//  - packed weights, row r (WROW bytes = CPR chunks: 2 at r = 4 and 6, 4 at
//    r = 8): chunk c sits at c ^ wsw(r) (one-chunk rows: no swizzle).
__device__ __forceinline__ int xsw(int r) { return (r & 7) ^ ((r >> 3) & 1); }
template <int CPR>
__device__ __forceinline__ int wsw(int r) {
  return CPR == 2 ? ((r >> 2) ^ (r >> 3)) & 1 : CPR == 4 ? ((r >> 1) ^ (r >> 2)) & 3 : 0;
}

__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void lds_dma4(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)lds, 4, voff, 0, 0, 0);
}

template <int R, bool GROUPED, int BM>
__global__ void __launch_bounds__(THREADS)
    gemm_big_kernel(const uint8_t* __restrict__ packed, const float* __restrict__ alpha,
                    const float* __restrict__ zero, const uint16_t* __restrict__ x,
                    float* __restrict__ y, int M, int N, int K, int group, int mt, int nt,
                    int its) {
  using C = Cfg<R, BM>;
  constexpr int MB = C::MB, XT_BYTES = C::XT_BYTES;
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* xs0 = smem;                                  // [2][BM][128 B] swizzled
  unsigned char* ws0 = smem + 2 * XT_BYTES;                   // [2][BN][WROW]
  float* sxg = reinterpret_cast<float*>(smem + 2 * XT_BYTES + 2 * C::WT_BYTES);  // [BM]

  // the wave index is uniform: in a scalar register, the staging addresses
  // derived from it (and the LDS bases of buffer-to-LDS loads) stay scalar
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;

  // ---- tile of this workgroup: the workgroups of one XCD (id % 8) walk
  //      consecutive tiles in m-major order so that they share activations
  int t = blockIdx.x;
  const int T = mt * nt;
  if ((T & 7) == 0) t = (t & 7) * (T >> 3) + (t >> 3);
  const int m0 = (t / nt) * BM, n0 = (t % nt) * BN;

  const int rowbytes = K * R / 8;
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(packed, (uint32_t)((int64_t)N * rowbytes));
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)((int64_t)M * K * 2));
  const int G = K / group;
  const int iters = K / BK;
  constexpr int IPG = 128 / BK;  // iterations per group of 128 (grouped)
  // this workgroup's K slice: iterations [ib, ie) (its is a multiple of
  // IPG); slice blockIdx.y of a split writes partial [blockIdx.y][M][N]
  const int ib = (int)blockIdx.y * its;
  const int ie = min(iters, ib + its);
  y += (int64_t)blockIdx.y * M * N;
  const UnpackK uk = UnpackK::make();
  UnpackK36 uk36;
  if constexpr (C::SPLIT) uk36 = UnpackK36::make();
  const int hrow = K * C::RH / 8, lrow = K * C::RL / 8;  // plane row bytes (high, low)

  // ---- group scales (grouped): window w = groups [4w, 4w + 4) into LDS
  //      buffer w & 1; waves 0-3 bring alpha, waves 4-7 the zero points, 64
  //      columns each.  Columns past N take the last row (never stored);
  //      groups past G read beyond the row (or 0 past the array) and are
  //      never used.
  float* sw = reinterpret_cast<float*>(smem + 2 * XT_BYTES + 2 * C::WT_BYTES + BM * 4);
  const __amdgpu_buffer_rsrc_t ar = make_rsrc(alpha, (uint32_t)((int64_t)N * G * 4));
  const __amdgpu_buffer_rsrc_t zr = make_rsrc(zero, (uint32_t)((int64_t)N * G * 4));
  auto stage_scales = [&](int w) {
    const int n = min(n0 + (wave & 3) * 64 + lane, N - 1);
    const uint32_t off = (uint32_t)(((int64_t)n * G + 4 * w) * 4);
    float* dst = sw + (w & 1) * (2 * BN * 4) + (wave >> 2) * (BN * 4) + (wave & 3) * 256;
    if (wave < 4) lds_dma16(ar, dst, off);
    else lds_dma16(zr, dst, off);
  };

  // ---- per-iteration staging (buffer-to-LDS, 1 KiB per wave instruction)
  auto stage = [&](int it, int buf) {
    const int k0 = it * BK;
    unsigned char* xs = xs0 + buf * XT_BYTES;
#pragma unroll
    for (int q = 0; q < BM * 128 / 1024 / WAVES; ++q) {
      const int rb = (wave * (BM * 128 / 1024 / WAVES) + q) * 8;  // first row of this piece
      const int row = rb + (lane >> 3);
      const int c = (lane & 7) ^ xsw(row);                        // logical 16-byte chunk
      const int m = m0 + row;
      const uint32_t off = m < M ? (uint32_t)(((int64_t)m * K + k0 + c * 8) * 2) : 0x80000000u;
      lds_dma16(xr, xs + rb * 128, off);
    }
    unsigned char* ws = ws0 + buf * C::WT_BYTES;
    constexpr int WPIECES = BN * C::WROW / 1024;
    for (int q = wave; q < WPIECES; q += WAVES) {
      const int byte = q * 1024 + lane * 16;
      const int row = byte / C::WROW;
      const int col = (((byte % C::WROW) >> 4) ^ wsw<C::WROW / 16>(row)) << 4;  // logical chunk here
      const int n = n0 + row;
      const uint32_t off =
          n < N ? (uint32_t)n * (uint32_t)hrow + (uint32_t)(k0 * C::RH / 8 + col) : 0x80000000u;
      lds_dma16(wr, ws + q * 1024, off);
    }
    if constexpr (C::SPLIT) {
      // low-plane sub-tile [BN][WLOW]: 16-byte rows (r = 6) one per lane;
      // 8-byte rows (r = 3) as 4-byte pieces, 256 bytes per wave instruction
      constexpr int PIECE = C::WLOW >= 16 ? 1024 : 256;
      for (int q = wave; q < BN * C::WLOW / PIECE; q += WAVES) {
        const int byte = q * PIECE + lane * (PIECE / 64);
        const int row = byte / C::WLOW, col = byte % C::WLOW;
        const int n = n0 + row;
        const uint32_t off = n < N ? (uint32_t)N * hrow + (uint32_t)n * lrow +
                                         (uint32_t)(k0 * C::RL / 8 + col)
                                   : 0x80000000u;
        if constexpr (PIECE == 1024) lds_dma16(wr, ws + C::LO_OFF + q * PIECE, off);
        else lds_dma4(wr, ws + C::LO_OFF + q * PIECE, off);
      }
    }
  };

  f32x16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int l32 = lane & 31, s = lane >> 5;
  // per-lane weight columns and their scales for the current group
  int ncol[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) ncol[j] = n0 + wn * 64 + j * 32 + l32;
  // columns past N read the last row's scales (unconditional loads; those
  // outputs are not stored)
  int nld[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) nld[j] = ncol[j] < N ? ncol[j] : N - 1;
  auto scale = [&](int j, int g) -> float { return alpha[(int64_t)nld[j] * G + g]; };
  auto zraw = [&](int j, int g) -> float { return zero[(int64_t)nld[j] * G + g]; };

  // row sums of x: RPW rows per wave; thread (row = RPW * wave + lane % RPW,
  // part = lane / RPW) sums CPT 16-byte chunks (8 codes each) per iteration
  constexpr int RPW = BM / WAVES, CPT = 8 / (64 / RPW);
  const int srow = wave * RPW + lane % RPW, spart = lane / RPW;
  float srun = 0.f;
  const uint32_t ones = 0x3F803F80u;

  // factors of the next group transition (zero-point term and rescale),
  // formed at each group's last iteration from the LDS scale window
  float cz[NB], rho[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    cz[j] = 0.f;
    rho[j] = 1.f;
  }

  // the first group's update reads these (cz = 0): keep them finite
  if (GROUPED && spart == 0) sxg[srow] = 0.f;
  if (GROUPED) {
    // the slice's first window; and the next one when the slice starts
    // inside a window (the loop issues a window only at a window's start)
    const int gb = ib / IPG;
    stage_scales(gb >> 2);
    if ((gb & 3) != 0 && 4 * ((gb >> 2) + 1) < G) stage_scales((gb >> 2) + 1);
  }
  stage(ib, ib & 1);
  // one trip of the outer loop = one group of 128 codes = IPG iterations
#pragma unroll 1
  for (int it0 = ib; it0 < ie; it0 += IPG) {
#pragma unroll
    for (int it2 = 0; it2 < IPG; ++it2) {
      const int it = it0 + it2;
      if (!GROUPED && it >= ie) break;  // per-channel K may end mid-pair
      const int buf = it & 1;
      __syncthreads();  // staging of `it` complete (vmcnt waited by the compiler), buf^1 free
      // raw scales of the group ending with this trip and of the next one,
      // read from LDS before this iteration's staging is issued
      float a0n[NB], a1n[NB], z0n[NB];
      const bool prep = GROUPED && it2 == IPG - 1 && it + 1 < ie;
      if (prep) {
        const int g = it / IPG;
        const float* w0 = sw + ((g >> 2) & 1) * (2 * BN * 4) + (g & 3);
        const float* w1 = sw + (((g + 1) >> 2) & 1) * (2 * BN * 4) + ((g + 1) & 3);
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int col = wn * 64 + j * 32 + l32;
          a0n[j] = w0[col * 4];
          z0n[j] = w0[BN * 4 + col * 4];
          a1n[j] = w1[col * 4];
        }
      }
      if (it + 1 < ie) stage(it + 1, buf ^ 1);
      // the next scale window, at the start of a window: its buffer was last
      // read before this iteration's barrier, and it is first needed at the
      // window's last group end
      if (GROUPED && it2 == 0 && ((it0 / IPG) & 3) == 0 && it0 / IPG + 4 < G)
        stage_scales(it0 / IPG / 4 + 1);

      // ---- row sums of this tile's activations
      {
        const unsigned char* xs = xs0 + buf * XT_BYTES;
        float sp = 0.f;
#pragma unroll
        for (int c4 = 0; c4 < CPT; ++c4) {
          const int c = spart * CPT + c4;
          const u32x4 w = *reinterpret_cast<const u32x4*>(xs + srow * 128 + ((c ^ xsw(srow)) * 16));
#pragma unroll
          for (int e = 0; e < 4; ++e) sp = dot2_bf16(w[e], ones, sp);
        }
#pragma unroll
        for (int off = RPW; off < 64; off <<= 1) sp += __shfl_xor(sp, off);
        srun += sp;
        if (GROUPED && it2 == IPG - 1) {
          if (spart == 0) sxg[srow] = srun;
          srun = 0.f;
        }
      }

      // ---- 4 k-steps of MFMAs; on the first iteration of a group (after the
      //      first), each block first takes the previous group's zero-point
      //      term and moves to this group's units (cz = 0, rho = 1 before)
      const unsigned char* xs = xs0 + buf * XT_BYTES;
      const unsigned char* ws = ws0 + buf * C::WT_BYTES;
      // this lane's packed words of the iteration (its 32 codes) per n-block:
      // 4R bytes, or for split planes 4 RH high bytes then 4 RL low bytes
      uint32_t wv[NB][R];
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int wrow = wn * 64 + j * 32 + l32;
        const unsigned char* p = ws + wrow * C::WROW;
        if (C::RH == 2) {
          const u32x2 v = *reinterpret_cast<const u32x2*>(p + s * 8);
          wv[j][0] = v[0]; wv[j][1] = v[1];
        } else {
#pragma unroll
          for (int h = 0; h < C::RH / 4; ++h) {
            const int c = s * (C::RH / 4) + h;  // logical chunk
            const u32x4 v =
                *reinterpret_cast<const u32x4*>(p + ((c ^ wsw<C::WROW / 16>(wrow)) << 4));
            wv[j][4 * h + 0] = v[0]; wv[j][4 * h + 1] = v[1];
            wv[j][4 * h + 2] = v[2]; wv[j][4 * h + 3] = v[3];
          }
        }
        if constexpr (C::SPLIT) {
          const unsigned char* pl = ws + C::LO_OFF + wrow * C::WLOW;
          if (C::RL == 2) {
            const u32x2 v = *reinterpret_cast<const u32x2*>(pl + s * 8);
            wv[j][4] = v[0]; wv[j][5] = v[1];
          } else {
            wv[j][2] = *reinterpret_cast<const uint32_t*>(pl + s * 4);
          }
        }
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        bf16x8 a[MB], b[NB];
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          const int row = wm * (MB * 32) + i * 32 + l32;
          const int c = 4 * s + kk;
          const u32x4 v = *reinterpret_cast<const u32x4*>(xs + row * 128 + ((c ^ xsw(row)) * 16));
          a[i] = __builtin_bit_cast(bf16x8, v);
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          if (R == 4) b[j] = unpack_r4(wv[j][kk], uk);
          else if (R == 2) b[j] = (kk & 1) ? unpack_r2<1>(wv[j][kk >> 1], uk)
                                           : unpack_r2<0>(wv[j][kk >> 1], uk);
          else if (R == 6) b[j] = unpack_r6(wv[j][kk], wv[j][4 + (kk >> 1)], kk & 1, uk36);
          else if (R == 3) b[j] = unpack_r3(wv[j][kk >> 1], wv[j][2], kk, uk36);
          else b[j] = unpack_r8(wv[j][2 * kk], wv[j][2 * kk + 1]);
        }
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          f32x4 sv[4];
          if (GROUPED && it2 == 0 && kk == 0) {
#pragma unroll
            for (int eq = 0; eq < 4; ++eq)
              sv[eq] = *reinterpret_cast<const f32x4*>(sxg + wm * (MB * 32) + i * 32 + eq * 8 + s * 4);
          }
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            if (GROUPED && it2 == 0 && kk == 0) {
#pragma unroll
              for (int e = 0; e < 16; ++e) {
                const float av0 = acc[i][j][e];
                acc[i][j][e] = rho[j] * (av0 - cz[j] * sv[e >> 2][e & 3]);
              }
            }
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
          }
        }
      }
      if (prep) {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          cz[j] = (z0n[j] + Enc<R>::kOffsetShift) * (1.0f / Enc<R>::kStep);
          rho[j] = a0n[j] / a1n[j];
        }
      }
    }
  }

  // ---- epilogue: last group's (or the only group's) zero-point term and scale
  if (!GROUPED && spart == 0) sxg[srow] = srun;
  __syncthreads();
  const int glast = GROUPED ? ie / IPG - 1 : 0;  // the slice's last group
  float av[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    cz[j] = (zraw(j, glast) + Enc<R>::kOffsetShift) * (1.0f / Enc<R>::kStep);
    av[j] = scale(j, glast) * Enc<R>::kStep;
  }
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int eq = 0; eq < 4; ++eq) {
      const int row = wm * (MB * 32) + i * 32 + eq * 8 + s * 4;
      const f32x4 sv = *reinterpret_cast<const f32x4*>(sxg + row);
#pragma unroll
      for (int e3 = 0; e3 < 4; ++e3) {
        const int m = m0 + row + e3;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          if (ncol[j] >= N) continue;
          const float v = av[j] * (acc[i][j][eq * 4 + e3] - cz[j] * sv[e3]);
          store_out(y + (int64_t)m * N + ncol[j], v);
        }
      }
    }
}

}  // namespace big

// Tile height: 128 rows up to kBig128MaxM rows of x (fewer padded rows and
// twice the tiles), 256 above.  Measured at the Mistral shapes: 128-row
// tiles take 65 <= M <= 128 25-35% faster than a 128 x 128 register-staged
// kernel did, and gain nothing over 256-row tiles from M = 160.
constexpr int kBig128MaxM = 128;
static int big_rows(int64_t M) { return M <= kBig128MaxM ? 128 : 256; }

// K split: while the tiles fill fewer than kBigTarget CUs (one workgroup
// each) and every slice keeps at least kBigMinIters iterations (whole groups)
constexpr int kBigTarget = 256, kBigMinIters = 8;

struct BigPlan {
  int bm, mt, nt, slices, its;
};

static BigPlan plan_big(int64_t M, int64_t N, int64_t K) {
  using namespace big;
  BigPlan p;
  p.bm = big_rows(M);
  p.mt = (int)((M + p.bm - 1) / p.bm);
  p.nt = (int)((N + BN - 1) / BN);
  const int iters = (int)(K / BK);
  int s = 1;
  while ((int64_t)p.mt * p.nt * s * 2 <= kBigTarget && iters / (s * 2) >= kBigMinIters) s *= 2;
  const int ipg = 128 / BK;
  p.its = ((iters + s - 1) / s + ipg - 1) / ipg * ipg;
  p.slices = (iters + p.its - 1) / p.its;
  return p;
}

size_t gemm_big_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const BigPlan p = plan_big(M, N, K);
  return p.slices > 1 ? (size_t)p.slices * M * N * 4 : 0;
}

template <int R, int BM>
static hipError_t launch_big_t(const BigPlan& p, const uint8_t* packed, const float* alpha,
                               const float* zero, int64_t group, int64_t N, int64_t K,
                               const uint16_t* x, int64_t M, float* out, hipStream_t s) {
  using namespace big;
  using C = Cfg<R, BM>;
  const bool grouped = group != K;
  // the LDS limit is raised once per process and kernel (function-local
  // statics are initialized exactly once, also when several host threads launch)
  static const hipError_t attr_g = hipFuncSetAttribute(
      (const void*)gemm_big_kernel<R, true, BM>, hipFuncAttributeMaxDynamicSharedMemorySize,
      C::LDS_GROUPED);
  static const hipError_t attr_c = hipFuncSetAttribute(
      (const void*)gemm_big_kernel<R, false, BM>, hipFuncAttributeMaxDynamicSharedMemorySize,
      C::LDS);
  if (attr_g != hipSuccess) return attr_g;
  if (attr_c != hipSuccess) return attr_c;
  dim3 grid((unsigned)(p.mt * p.nt), (unsigned)p.slices), block(THREADS);
  if (grouped)
    hipLaunchKernelGGL((gemm_big_kernel<R, true, BM>), grid, block, C::LDS_GROUPED, s, packed,
                       alpha, zero, x, out, (int)M, (int)N, (int)K, (int)group, p.mt, p.nt,
                       p.its);
  else
    hipLaunchKernelGGL((gemm_big_kernel<R, false, BM>), grid, block, C::LDS, s, packed, alpha,
                       zero, x, out, (int)M, (int)N, (int)K, (int)group, p.mt, p.nt, p.its);
  return hipGetLastError();
}

template <int R>
static hipError_t launch_big_r(const uint8_t* packed, const float* alpha, const float* zero,
                               int64_t group, int64_t N, int64_t K, const uint16_t* x, int64_t M,
                               float* y, void* workspace, hipStream_t s) {
  const BigPlan p = plan_big(M, N, K);
  float* out = p.slices > 1 ? static_cast<float*>(workspace) : y;
  hipError_t e = p.bm == 128
                     ? launch_big_t<R, 128>(p, packed, alpha, zero, group, N, K, x, M, out, s)
                     : launch_big_t<R, 256>(p, packed, alpha, zero, group, N, K, x, M, out, s);
  if (e != hipSuccess || p.slices == 1) return e;
  return launch_reduce_slices(out, y, M * N, p.slices, s);
}

hipError_t launch_gemm_big(const uint8_t* packed, int r, const float* alpha, const float* zero,
                           int64_t group, int64_t N, int64_t K, const uint16_t* x, int64_t M,
                           float* y, void* workspace, hipStream_t s) {
  switch (r) {
    case 2: return launch_big_r<2>(packed, alpha, zero, group, N, K, x, M, y, workspace, s);
    case 4: return launch_big_r<4>(packed, alpha, zero, group, N, K, x, M, y, workspace, s);
    case 3: return launch_big_r<3>(packed, alpha, zero, group, N, K, x, M, y, workspace, s);
    case 6: return launch_big_r<6>(packed, alpha, zero, group, N, K, x, M, y, workspace, s);
    default: return launch_big_r<8>(packed, alpha, zero, group, N, K, x, M, y, workspace, s);
  }
}

}  // namespace mq
