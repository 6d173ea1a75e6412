// Batched product against r-bit planes on bf16 matrix cores: the router of
// mq_gemm (M <= 8 decode kernel, 9..64 panel kernel, 65..127 at r = 2, 4, 8
// the tiled kernel below, everything else the prefill kernel).
//
//   y[m, n] = sum_g alpha[n, g] * (2^(8-r) * sum_{k in g} x[m, k] t[n, k]
//                                   - z[n, g] * sum_{k in g} x[m, k])
// which is sum_k x[m, k] (S(q[n, k], r) - z[n, g]) alpha[n, g] with
// S = t * 2^(8-r) ("Matryoshka Quantization" explainer, §3.4, Eq. 6 and the
// dequantization of Eq. 1).  The integer index (plus the encoding offset of
// mq_device.h) is contracted exactly in bf16 x bf16 -> fp32; alpha, 2^(8-r)
// and z are applied in fp32 once per group of 128 (or once at the end for
// per-channel scales).
//
// Tiling (gfx950, v_mfma_f32_32x32x16_bf16): A = activations (32 rows of m x
// 16 k), B = unpacked weights (16 k x 32 rows of n), D = y tile [m][n].  A
// workgroup of 4 waves computes a BM x BN tile; each K iteration covers 128
// codes (one scale group): the activation tile (bf16, natural order) and the
// packed weight tile are staged in LDS, the next tile's global loads are
// issued before the current tile's MFMAs.  Every group is folded into fp32
// totals in absolute units, so a run of K iterations is an additive partial:
// when the tiles alone leave CUs idle (few rows of n, long K), K is split over
// blockIdx.z and the slices are summed in slice order by a second kernel.
#include <algorithm>

#include "mq_device.h"
#include "mq_internal.h"

namespace mq {

constexpr int kBK = 128;     // codes per K iteration (one group of 128)
constexpr int kXsPad = 8;    // bf16 padding per staged activation row

template <int R, int MB, int NB, int WM, int WN>
struct Gm {
  static constexpr int BM = 32 * MB * WM;
  static constexpr int BN = 32 * NB * WN;
  static constexpr int THREADS = 64 * WM * WN;
  static constexpr int XS = kBK + kXsPad;         // staged x row stride (elements)
  static constexpr int WROW = kBK * R / 8;        // packed bytes per row per iteration
  static constexpr int WS = WROW + 16;            // staged weight row stride (bytes)
  // x tile loads: BM rows x 128 codes = BM * 16 vectors of 8 bf16
  static constexpr int XV = BM * 16 / THREADS;    // 16-byte vectors per thread
  static constexpr int WV = BN * WROW / 16 / THREADS;  // 16-byte packed vectors per thread
  static_assert(XV >= 1 && (BM * 16) % THREADS == 0, "x tile split");
  static_assert((BN * WROW / 16) % THREADS == 0 && WV >= 1, "w tile split");
};

// Position in the staged activation tile of the 8 values that lane
// slot s feeds at k-step kk (16 codes per k-step), and the packed byte offset
// of the matching weight word(s).
template <int R>
__device__ __forceinline__ int xpos(int kk, int s) {
  return R == 2 ? 32 * (kk >> 1) + 16 * s + 8 * (kk & 1) : 16 * kk + 8 * s;
}
template <int R>
__device__ __forceinline__ int wbyte(int kk, int s) {
  return R == 2 ? 8 * (kk >> 1) + 4 * s : (R == 4 ? 8 * kk + 4 * s : 16 * kk + 8 * s);
}

template <int R, int MB, int NB, int WM, int WN, bool GROUPED>
__global__ void __launch_bounds__(64 * WM * WN)
    gemm_kernel(const uint8_t* __restrict__ packed, const float* __restrict__ alpha,
                const float* __restrict__ zero, const uint16_t* __restrict__ x,
                float* __restrict__ y, int M, int N, int K, int group, int its) {
  using C = Gm<R, MB, NB, WM, WN>;
  __shared__ __align__(16) uint16_t xs[C::BM * C::XS];
  __shared__ __align__(16) uint8_t ws[C::BN * C::WS];
  __shared__ float sxg[C::BM];   // per-group sums of x (this iteration)
  __shared__ float sxh[C::BM * 2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int m0 = blockIdx.y * C::BM, n0 = blockIdx.x * C::BN;
  const int G = K / group;
  const int rowbytes = K * R / 8;
  const uint32_t plane = (uint32_t)((int64_t)N * rowbytes);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(packed, plane);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)((int64_t)M * K * 2));
  // this workgroup's K iterations [it0, it1) (slice blockIdx.z of its each);
  // a split writes slice z of the partial tiles [S][M][N]
  const int iters = (K + kBK - 1) / kBK;
  const int it0 = (int)blockIdx.z * its;
  const int it1 = min(iters, it0 + its);
  y += (int64_t)blockIdx.z * M * N;

  // ---- per-thread staging assignment
  // x: thread covers XV consecutive 16-byte vectors of one row
  const int xvec0 = tid * C::XV;             // first vector index in [0, BM*16)
  const int xrow = xvec0 / 16, xcol = (xvec0 % 16) * 8;
  const bool xrow_ok = (m0 + xrow) < M;
  const uint32_t xoff_row = xrow_ok ? (uint32_t)((m0 + xrow) * K) * 2u : 0xffffffffu;
  // w: thread covers WV vectors of 16 packed bytes
  auto wvec_off = [&](int v, int it) -> uint32_t {
    const int vid = tid * C::WV + v;
    const int row = vid / (C::WROW / 16), cb = (vid % (C::WROW / 16)) * 16;
    const int n = n0 + row;
    if (n >= N) return 0xffffffffu;
    return (uint32_t)n * (uint32_t)rowbytes + (uint32_t)(it * C::WROW + cb);
  };

  const int l32 = lane & 31, s = lane >> 5;
  const int am0 = wm * MB * 32, bn0 = wn * NB * 32;

  u32x4 xreg[C::XV], wreg[C::WV];
  float ga[NB], gz[NB];  // grouped: scale and zero point of the loaded group
  auto gload = [&](int it) {
#pragma unroll
    for (int v = 0; v < C::XV; ++v) {
      const int k = it * kBK + xcol + 8 * v;
      const uint32_t off = (xrow_ok && k < K) ? xoff_row + (uint32_t)k * 2u : 0xffffffffu;
      xreg[v] = buf_load16(xr, off);
    }
#pragma unroll
    for (int v = 0; v < C::WV; ++v) wreg[v] = buf_load16(wr, wvec_off(v, it));
    if (GROUPED) {  // group == 128 == kBK: iteration it is group it
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int n = min(n0 + bn0 + 32 * j + (lane & 31), N - 1);
        ga[j] = alpha[(int64_t)n * G + it];
        gz[j] = zero[(int64_t)n * G + it];
      }
    }
  };
  float xsum_run = 0.f;  // per-channel: running sum of this thread's x values
  auto lstore = [&]() {
    // activations: stored as loaded (natural k order), summed
    float s = 0.f;
    const uint32_t ones = 0x3F803F80u;
    u32x4* dst = reinterpret_cast<u32x4*>(xs + xrow * C::XS + xcol);
#pragma unroll
    for (int v = 0; v < C::XV; ++v) {
      dst[v] = xreg[v];
#pragma unroll
      for (int e = 0; e < 4; ++e) s = dot2_bf16(xreg[v][e], ones, s);
    }
    // threads of one row: 16 / XV of them; reduce their sums
    constexpr int TPR = 16 / C::XV;
#pragma unroll
    for (int off = 1; off < TPR; off <<= 1) s += __shfl_xor(s, off);
    if ((tid % TPR) == 0) sxg[xrow] = s;
    xsum_run += s;
#pragma unroll
    for (int v = 0; v < C::WV; ++v) {
      const int vid = tid * C::WV + v;
      const int row = vid / (C::WROW / 16), cb = (vid % (C::WROW / 16)) * 16;
      *reinterpret_cast<u32x4*>(ws + row * C::WS + cb) = wreg[v];
    }
  };

  f32x16 part[MB][NB], tot[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        part[i][j][e] = 0.f;
        tot[i][j][e] = 0.f;
      }


  gload(it0);
#pragma unroll 1
  for (int it = it0; it < it1; ++it) {
    __syncthreads();
    lstore();
    float ca[NB], cz[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      ca[j] = ga[j];
      cz[j] = gz[j];
    }
    __syncthreads();
    if (it + 1 < it1) gload(it + 1);

#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      bf16x8 a[MB], b[NB];
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(xs + (am0 + 32 * i + l32) * C::XS +
                                                        xpos<R>(kk, s));
        a[i] = __builtin_bit_cast(bf16x8, w);
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const uint8_t* wp = ws + (bn0 + 32 * j + l32) * C::WS + wbyte<R>(kk, s);
        if (R == 4) {
          b[j] = unpack_r4(*reinterpret_cast<const uint32_t*>(wp));
        } else if (R == 2) {
          const uint32_t w = *reinterpret_cast<const uint32_t*>(wp);
          b[j] = (kk & 1) ? unpack_r2<1>(w) : unpack_r2<0>(w);
        } else {
          const u32x2 w = *reinterpret_cast<const u32x2*>(wp);
          b[j] = unpack_r8(w[0], w[1]);
        }
      }
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
          part[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], part[i][j], 0, 0, 0);
    }

    if (GROUPED) {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        // columns past N fold clamped scales; they are never stored
        const float av = ca[j] * Enc<R>::kStep;
        const float bv = ca[j] * (cz[j] + Enc<R>::kOffsetShift);
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int mrow = am0 + 32 * i + 8 * (e >> 2) + 4 * s + (e & 3);
            tot[i][j][e] = tot[i][j][e] + av * part[i][j][e] - bv * sxg[mrow];
            part[i][j][e] = 0.f;
          }
      }
    }
  }

  // ---- epilogue
  if (!GROUPED) {
    constexpr int TPR = 16 / C::XV;
    __syncthreads();
    if ((tid % TPR) == 0) sxh[xrow] = 0.f;
    __syncthreads();
    // xsum_run of the TPR threads of a row were already reduced per iteration
    if ((tid % TPR) == 0) sxh[xrow] = xsum_run;
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int n = n0 + bn0 + 32 * j + l32;
    if (n >= N) continue;
    float av = 0.f, bv = 0.f;
    if (!GROUPED) {
      av = alpha[n] * Enc<R>::kStep;
      bv = alpha[n] * (zero[n] + Enc<R>::kOffsetShift);
    }
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int mrow = am0 + 32 * i + 8 * (e >> 2) + 4 * s + (e & 3);
        const int m = m0 + mrow;
        if (m >= M) continue;
        float v;
        if (GROUPED) {
          v = tot[i][j][e];
        } else {
          v = av * part[i][j][e] - bv * sxh[mrow];
        }
        y[(int64_t)m * N + n] = v;
      }
  }
}

// 64 < M < 128 (r = 2, 4, 8): 128 x 128 tiles of 4 waves.  K is split while
// the tiles fill fewer than the target number of workgroups (measured best:
// 512 with per-channel scales, 256 with group-128 scales, whose per-group
// folds cost more per iteration) and every slice keeps at least
// kTiledMinIters iterations.
constexpr int kTiledBM = 128, kTiledBN = 128;
constexpr int kTiledTargetChannel = 512, kTiledTargetGroup = 256, kTiledMinIters = 4;

struct TiledPlan {
  int gx, gy, slices, its;
};

static TiledPlan plan_tiled(int64_t M, int64_t N, int64_t K, int64_t group) {
  const int target = group == K ? kTiledTargetChannel : kTiledTargetGroup;
  TiledPlan p;
  p.gx = (int)((N + kTiledBN - 1) / kTiledBN);
  p.gy = (int)((M + kTiledBM - 1) / kTiledBM);
  const int iters = (int)((K + kBK - 1) / kBK);
  int s = 1;
  while ((int64_t)p.gx * p.gy * s * 2 <= target && iters / (s * 2) >= kTiledMinIters) s *= 2;
  p.its = (iters + s - 1) / s;
  p.slices = (iters + p.its - 1) / p.its;
  return p;
}

// From M = 128 the prefill kernel (256 x 256 tiles, buffer-to-LDS staging,
// its own K split) measured faster at the Mistral shapes; below, the
// 128-row tiles waste fewer rows.
constexpr int kTiledMaxM = 127;
static bool tiled_route(int64_t M) { return M > kPanelMaxM && M <= kTiledMaxM; }

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t group) {
  if (M <= kSkinnyMaxM) return 0;
  if (M <= kPanelMaxM) return panel_workspace_bytes(M, N, K);
  const size_t big = gemm_big_workspace_bytes(M, N, K);
  if (!tiled_route(M)) return big;
  // r is not an argument: 64 < M < 128 takes the tiled kernel at r = 2, 4, 8
  // and the prefill kernel at r = 3, 6; the workspace covers both
  const TiledPlan p = plan_tiled(M, N, K, group);
  return std::max(big, p.slices > 1 ? (size_t)p.slices * M * N * 4 : (size_t)0);
}

template <int R>
static hipError_t launch_r(const uint8_t* packed, const float* alpha, const float* zero,
                           int64_t group, int64_t N, int64_t K, const uint16_t* x, int64_t M,
                           float* y, void* workspace, hipStream_t s) {
  using C = Gm<R, 2, 2, 2, 2>;
  static_assert(C::BM == kTiledBM && C::BN == kTiledBN, "tile of the plan");
  const TiledPlan p = plan_tiled(M, N, K, group);
  float* out = p.slices > 1 ? static_cast<float*>(workspace) : y;
  dim3 grid((unsigned)p.gx, (unsigned)p.gy, (unsigned)p.slices);
  if (group == K)
    hipLaunchKernelGGL((gemm_kernel<R, 2, 2, 2, 2, false>), grid, dim3(C::THREADS), 0, s, packed,
                       alpha, zero, x, out, (int)M, (int)N, (int)K, (int)group, p.its);
  else
    hipLaunchKernelGGL((gemm_kernel<R, 2, 2, 2, 2, true>), grid, dim3(C::THREADS), 0, s, packed,
                       alpha, zero, x, out, (int)M, (int)N, (int)K, (int)group, p.its);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.slices == 1) return e;
  return launch_reduce_slices(out, y, M * N, p.slices, s);
}

hipError_t launch_gemm(const uint8_t* packed, int r, const float* alpha, const float* zero,
                       int64_t group, int64_t N, int64_t K, const uint16_t* x, int64_t M, float* y,
                       void* workspace, hipStream_t s) {
  if (M <= kPanelMaxM)
    return launch_gemm_panel(packed, r, alpha, zero, group, N, K, x, M, y, workspace, s);
  // M >= 128, and the split planes (r = 3, 6) above the small batch: the
  // prefill kernel, whose partial tiles cover any M
  if (!tiled_route(M) || split_precision(r))
    return launch_gemm_big(packed, r, alpha, zero, group, N, K, x, M, y, workspace, s);
  switch (r) {
    case 2: return launch_r<2>(packed, alpha, zero, group, N, K, x, M, y, workspace, s);
    case 4: return launch_r<4>(packed, alpha, zero, group, N, K, x, M, y, workspace, s);
    default: return launch_r<8>(packed, alpha, zero, group, N, K, x, M, y, workspace, s);
  }
}

}  // namespace mq
