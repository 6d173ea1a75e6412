// Small-batch product (9 <= M <= 64 activation rows) against r-bit planes:
//   y[m, n] = sum_k x[m, k] (S(q[n, k], r) - z[n, g]) alpha[n, g]
// ("Matryoshka Quantization" explainer, §3.4: Eq. 6 slicing, Eq. 1
// dequantization).  At these M the product still streams the planes out of
// HBM (every packed byte is used M times, on the matrix cores).
//
// Design (gfx950, v_mfma_f32_32x32x16_bf16, A = activations, B = weights):
//  - A workgroup owns a panel of 32 * NW weight rows (one 32-row block per
//    wave) and a slice of K of at most 1024 codes.  The activations of that
//    slice (all M rows, padded to 32 * MB) are brought into LDS once with
//    buffer-to-LDS loads; the per-128 sums of x are formed from LDS.
//  - Each lane streams 16 contiguous packed bytes of one weight row per step
//    straight into registers (no LDS for weights: every row has one reader),
//    DEPTH steps ahead of use, and unpacks them into exact bf16 integers
//    (mq_device.h).  One unpacked operand feeds MB matrix-core products.
//    r = 3 and 6 (a high-bit and a low-bit plane) take 32 codes per lane per
//    step from both planes and assemble u = 2^r + t in the same registers.
//  - alpha and z of the panel's groups are staged in LDS with the
//    activations; group-128 scales are applied at each group end in fp32
//    (y += alpha 2^(8-r) P_g - alpha (z + shift) sum_g x), per-channel scales
//    once at the end.
//  - When K is split over several workgroups, each writes its fp32 partial
//    tile to the workspace and a second kernel sums the slices in a fixed
//    order (deterministic).
#include <algorithm>

#include "mq_device.h"
#include "mq_internal.h"

namespace mq {

namespace panel {

constexpr int kKSlice = 1024;     // codes of K per workgroup (activations resident in LDS)
constexpr int kXPadE = 8;         // bf16 padding per staged activation row

template <int R>
struct Pc {
  // r = 3 and 6: a high-bit and a low-bit plane (rows of the high plane, then
  // rows of the low plane), 32 codes per lane per step from each
  static constexpr bool SPLIT = (R == 3 || R == 6);
  static constexpr int RL = R == 6 ? 2 : 1, RH = R - RL;  // split: plane widths
  static constexpr int CPL = SPLIT ? 32 : 16 * 8 / R;    // codes per lane per step
  static constexpr int STEP = 2 * CPL;      // codes per row per step (two lane slots)
  static constexpr int MFMAS = CPL / 8;     // 16-deep products per step per m-block
  static constexpr int SPG = 128 / STEP;    // steps per group of 128
  static constexpr int STEPS = kKSlice / STEP;  // steps of a full slice
  // weight loads in flight per lane: the whole slice at r = 2 (8 steps),
  // 16 steps at r = 4 (the whole slice) and r = 8; 8 for the split planes
  // (their two loads per step take 6 or 3 registers each)
  static constexpr int DEPTH = SPLIT ? 8 : (STEPS < 16 ? STEPS : 16);
  using LD = LoadT<R, SPLIT ? 0 : 16>;      // one lane's loads of a step
};

struct Args {
  const uint8_t* packed;
  const float* alpha;
  const float* zero;
  const uint16_t* x;
  float* y;     // output [M, N] (one K slice) or the partial slices [S][M][N]
  int M, N, K, G;
  int kslice;   // codes of K per workgroup (kKSlice)
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

template <int R, int MB, int NW, bool GROUPED>
__global__ void __launch_bounds__(64 * NW) panel_kernel(const Args a) {
  using C = Pc<R>;
  constexpr int ROWS = 32 * MB;
  extern __shared__ __align__(16) unsigned char smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, s = lane >> 5;
  const int M = a.M, N = a.N, K = a.K, G = a.G;
  constexpr int DEPTH = C::DEPTH;
  const int k0 = (int)blockIdx.y * kKSlice;
  const int klen = min(kKSlice, K - k0);
  const int ngl = (klen + 127) >> 7;              // groups of 128 in the slice
  const int steps = (klen + C::STEP - 1) / C::STEP;
  constexpr int xstride = kKSlice + kXPadE;       // elements

  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);                              // [ROWS][xstride]
  float* sxs = reinterpret_cast<float*>(smem + (size_t)ROWS * xstride * 2);      // [ngl][ROWS]
  float* azs = sxs + (kKSlice / 128) * ROWS;                                     // [2][NW*32][8]

  const int n0 = (int)blockIdx.x * NW * 32;
  const int n = n0 + wave * 32 + l32;  // weight row of this lane
  const int rowbytes = K * R / 8;
  const uint32_t plane = (uint32_t)((int64_t)N * rowbytes);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.packed, plane);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, (uint32_t)((int64_t)M * K * 2));

  // The loads are issued in the order the workgroup needs them: the staged
  // activations and group scales (which the first barrier waits for), then
  // the weights (which it does not).  Every loop here is unrolled, so no
  // wait is placed before a load is issued.
  // ---- activations of the slice: two 1 KiB pieces (512 codes) per row,
  //      one per wave instruction; rows past M and columns past K read zeros
#pragma unroll
  for (int q = 0; q < ROWS * 2 / NW; ++q) {
    const int pc = wave + q * NW;
    const int m = pc >> 1, j = pc & 1;
    const int k = k0 + j * 512 + lane * 8;
    const uint32_t off = (m < M && k < K) ? (uint32_t)(((int64_t)m * K + k) * 2) : 0x80000000u;
    lds_dma16(xr, xs + (size_t)m * xstride + j * 512, off);
  }
  // ---- scales of the panel: group-128 ones staged in LDS as
  //      [alpha | zero][row][group of the slice] by 4-byte buffer-to-LDS
  //      loads (entries past N or past the slice read zeros); per-channel
  //      ones in registers (needed at the end only)
  float pa = 0.f, pz = 0.f;
  if (GROUPED) {
    const __amdgpu_buffer_rsrc_t ar = make_rsrc(a.alpha, (uint32_t)((int64_t)N * G * 4));
    const __amdgpu_buffer_rsrc_t zr = make_rsrc(a.zero, (uint32_t)((int64_t)N * G * 4));
    const int g0 = k0 >> 7;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int base = (wave + e * NW) * 64;  // NW*32 rows x 8 groups, one entry per lane
      const int idx = base + lane;
      const int rr = idx >> 3, gg = idx & 7;
      const int nn = n0 + rr;
      const uint32_t off =
          (nn < N && gg < ngl) ? (uint32_t)(((int64_t)nn * G + g0 + gg) * 4) : 0x80000000u;
      lds_dma4(ar, azs + base, off);
      lds_dma4(zr, azs + NW * 32 * 8 + base, off);
    }
  } else {
    const int nc = n < N ? n : N - 1;
    pa = a.alpha[nc];
    pz = a.zero[nc];
  }

  // ---- the first DEPTH weight loads
  // split planes: the lane's high-plane bytes, and its low-plane bytes after
  // all N rows of the high plane
  constexpr int WH = C::SPLIT ? C::RH : R;  // bits per code in the (high) plane
  const uint32_t hrow = (uint32_t)(K * WH / 8), lrow = (uint32_t)(K * C::RL / 8);
  const uint32_t row_off = n < N ? (uint32_t)n * hrow : plane;
  const uint32_t base_off = row_off + (uint32_t)((k0 + s * C::CPL) * WH / 8);
  const uint32_t base_lo = n < N ? (uint32_t)N * hrow + (uint32_t)n * lrow +
                                       (uint32_t)((k0 + s * C::CPL) * C::RL / 8)
                                 : plane;
  auto loff = [&](int st) -> uint32_t {
    return st < steps ? base_off + (uint32_t)(st * (C::STEP * WH / 8)) : 0x80000000u;
  };
  auto loff_lo = [&](int st) -> uint32_t {
    return st < steps ? base_lo + (uint32_t)(st * (C::STEP * C::RL / 8)) : 0x80000000u;
  };
  using LD = typename C::LD;
  typename LD::T buf[DEPTH];
#pragma unroll
  for (int j = 0; j < DEPTH; ++j) buf[j] = LD::load(wr, loff(j), loff_lo(j));
  __syncthreads();

  // ---- per-128 sums of the staged activations: one thread per (row,
  //      group) sums its 16 chunks of 8 in order (no cross-lane reduction;
  //      consecutive lanes take consecutive rows, whose 16-byte reads fall
  //      on distinct banks)
  {
    const uint32_t ones = 0x3F803F80u;
    for (int t = tid; t < ROWS * ngl; t += 64 * NW) {
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
  __syncthreads();

  // ---- stream the slice
  const UnpackK uk = UnpackK::make();
  UnpackK36 uk36;
  if constexpr (C::SPLIT) uk36 = UnpackK36::make();
  f32x16 acc[MB], part[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      acc[mb][e] = 0.f;
      part[mb][e] = 0.f;
    }
  const uint16_t* xa = xs + (size_t)l32 * xstride + s * C::CPL;
  const float* az_row = azs + (wave * 32 + l32) * 8;
  // group-128: each group's products accumulate onto -cz * sum_g x, with
  // cz = (z + shift) / 2^(8-r), so that at the group's end
  // part = sum_g x u - cz sum_g x and y += alpha 2^(8-r) part
  auto start_group = [&](int gl) {
    const float cz = (az_row[NW * 32 * 8 + gl] + Enc<R>::kOffsetShift) * (1.0f / Enc<R>::kStep);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int eq = 0; eq < 4; ++eq) {
        const f32x4 sv =
            *reinterpret_cast<const f32x4*>(sxs + gl * ROWS + mb * 32 + eq * 8 + s * 4);
#pragma unroll
        for (int e3 = 0; e3 < 4; ++e3) part[mb][eq * 4 + e3] = -cz * sv[e3];
      }
  };
  if (GROUPED) start_group(0);

#pragma unroll 1
  for (int base = 0; base < steps; base += DEPTH) {
#pragma unroll
    for (int j = 0; j < DEPTH; ++j) {
      const int st = base + j;
      if (st < steps) {
        uint32_t d[LD::NW];
        LD::words(buf[j], d);
        const uint16_t* xp = xa + st * C::STEP;
#pragma unroll
        for (int i = 0; i < C::MFMAS; ++i) {
          const bf16x8 b = unpack_b<R>(d, i, uk, uk36);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            const u32x4 v =
                *reinterpret_cast<const u32x4*>(xp + (size_t)mb * 32 * xstride + 8 * i);
            const bf16x8 av = __builtin_bit_cast(bf16x8, v);
            if (GROUPED) {
              part[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b, part[mb], 0, 0, 0);
            } else {
              acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b, acc[mb], 0, 0, 0);
            }
          }
        }
        if (GROUPED && (j % C::SPG) == C::SPG - 1) {
          const int gl = st / C::SPG;
          const float av = az_row[gl] * Enc<R>::kStep;
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[mb][e] = fmaf(av, part[mb][e], acc[mb][e]);
          start_group(gl + 1 < ngl ? gl + 1 : gl);
        }
      }
      // refill this slot after its last use (while steps remain)
      if (st + DEPTH < steps) buf[j] = LD::load(wr, loff(st + DEPTH), loff_lo(st + DEPTH));
    }
  }

  // ---- epilogue: lane holds column n, rows mb*32 + eq*8 + s*4 + e3
  float* out = a.y + (size_t)blockIdx.y * M * N;
  if (n < N) {
    float ep_a = 0.f, ep_b = 0.f;
    if (!GROUPED) {
      ep_a = pa * Enc<R>::kStep;
      ep_b = pa * (pz + Enc<R>::kOffsetShift);
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int eq = 0; eq < 4; ++eq) {
        f32x4 tot = {0.f, 0.f, 0.f, 0.f};
        if (!GROUPED) {
          for (int gl = 0; gl < ngl; ++gl)
            tot += *reinterpret_cast<const f32x4*>(sxs + gl * ROWS + mb * 32 + eq * 8 + s * 4);
        }
#pragma unroll
        for (int e3 = 0; e3 < 4; ++e3) {
          const int m = mb * 32 + eq * 8 + s * 4 + e3;
          if (m < M) {
            const float v = GROUPED ? acc[mb][eq * 4 + e3]
                                    : ep_a * acc[mb][eq * 4 + e3] - ep_b * tot[e3];
            out[(size_t)m * N + n] = v;
          }
        }
      }
  }
}

// y = sum over S slices of the partial tiles, in slice order.  16-byte
// vectors only when every slice starts 16-byte aligned (count % 4 == 0).
__global__ void __launch_bounds__(256) reduce_slices(const float* __restrict__ part,
                                                     float* __restrict__ y, int64_t count,
                                                     int S) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t n4 = (count & 3) ? 0 : count >> 2;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    f32x4 v = reinterpret_cast<const f32x4*>(part)[i];
    for (int sl = 1; sl < S; ++sl) v += reinterpret_cast<const f32x4*>(part + sl * count)[i];
    reinterpret_cast<f32x4*>(y)[i] = v;
  }
  for (int64_t i = (n4 << 2) + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
       i += stride) {
    float v = part[i];
    for (int sl = 1; sl < S; ++sl) v += part[sl * count + i];
    y[i] = v;
  }
}

}  // namespace panel

// ---------------------------------------------------------------------------
// Host planning
// ---------------------------------------------------------------------------

struct PanelPlan {
  int nw, kslice, slices, panels;
};

static PanelPlan plan_panel(int64_t M, int64_t N, int64_t K) {
  (void)M;
  PanelPlan p;
  p.nw = 8;
  p.panels = (int)((N + 32 * p.nw - 1) / (32 * p.nw));
  // K slice: the largest the activations allow in LDS (1024 codes): longer
  // workgroups and fewer partial slices measured faster than more, shorter
  // ones at the Mistral shapes (M = 16 and 64)
  p.kslice = panel::kKSlice;
  p.slices = (int)((K + p.kslice - 1) / p.kslice);
  return p;
}

size_t panel_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const PanelPlan p = plan_panel(M, N, K);
  return p.slices > 1 ? (size_t)p.slices * M * N * 4 : 0;
}

template <int R, int MB, bool GROUPED>
static hipError_t launch_panel_t(const panel::Args& a, const PanelPlan& p, hipStream_t s) {
  constexpr int NW = 8;
  const size_t lds = (size_t)32 * MB * (p.kslice + panel::kXPadE) * 2 +
                     (size_t)(panel::kKSlice / 128) * 32 * MB * 4 + (size_t)2 * NW * 32 * 8 * 4;
  // the LDS limit is raised once per process (a function-local static is
  // initialized exactly once, also when several host threads launch)
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)panel::panel_kernel<R, MB, NW, GROUPED>,
      hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((panel::panel_kernel<R, MB, NW, GROUPED>), dim3(p.panels, p.slices),
                     dim3(64 * NW), lds, s, a);
  return hipGetLastError();
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
  a.kslice = p.kslice;
  const bool grouped = group != K;
  const int mb = M > 32 ? 2 : 1;
  hipError_t e;
  switch (r * 4 + (mb - 1) * 2 + (grouped ? 1 : 0)) {
    case 8: e = launch_panel_t<2, 1, false>(a, p, s); break;
    case 9: e = launch_panel_t<2, 1, true>(a, p, s); break;
    case 10: e = launch_panel_t<2, 2, false>(a, p, s); break;
    case 11: e = launch_panel_t<2, 2, true>(a, p, s); break;
    case 12: e = launch_panel_t<3, 1, false>(a, p, s); break;
    case 13: e = launch_panel_t<3, 1, true>(a, p, s); break;
    case 14: e = launch_panel_t<3, 2, false>(a, p, s); break;
    case 15: e = launch_panel_t<3, 2, true>(a, p, s); break;
    case 16: e = launch_panel_t<4, 1, false>(a, p, s); break;
    case 17: e = launch_panel_t<4, 1, true>(a, p, s); break;
    case 18: e = launch_panel_t<4, 2, false>(a, p, s); break;
    case 19: e = launch_panel_t<4, 2, true>(a, p, s); break;
    case 24: e = launch_panel_t<6, 1, false>(a, p, s); break;
    case 25: e = launch_panel_t<6, 1, true>(a, p, s); break;
    case 26: e = launch_panel_t<6, 2, false>(a, p, s); break;
    case 27: e = launch_panel_t<6, 2, true>(a, p, s); break;
    case 32: e = launch_panel_t<8, 1, false>(a, p, s); break;
    case 33: e = launch_panel_t<8, 1, true>(a, p, s); break;
    case 34: e = launch_panel_t<8, 2, false>(a, p, s); break;
    default: e = launch_panel_t<8, 2, true>(a, p, s); break;
  }
  if (e != hipSuccess || p.slices == 1) return e;
  return launch_reduce_slices(static_cast<const float*>(workspace), y, M * N, p.slices, s);
}

hipError_t launch_reduce_slices(const float* part, float* y, int64_t count, int S, hipStream_t s) {
  const int blocks = (int)std::min<int64_t>((count / 4 + 255) / 256 + 1, 2048);
  hipLaunchKernelGGL(panel::reduce_slices, dim3(blocks), dim3(256), 0, s, part, y, count, S);
  return hipGetLastError();
}

}  // namespace mq
