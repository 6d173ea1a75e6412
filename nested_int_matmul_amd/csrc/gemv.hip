// Decode-shaped product (M <= 8 activation rows) against r-bit planes.
//
//   y[m, n] = sum_k x[m, k] * (S(q[n, k], r) - z[n, g]) * alpha[n, g]
// ("Matryoshka Quantization" explainer, §3.4: Eq. 6 slicing, Eq. 1
// dequantization; decode time is set by moving the weights out of HBM, §2).
//
// Design (gfx950):
//  - The product is streaming: every packed byte is read once.  A wavefront
//    owns a block of 16 weight rows and a slice of K; each lane loads 16 (or
//    8) contiguous packed bytes of one row per step through a bounds-checked
//    buffer load (rows past N and bytes past the plane read as zero).
//  - The bytes are unpacked in registers into exact bf16 integers (see
//    mq_device.h) and multiplied on the matrix cores with
//    v_mfma_f32_16x16x32_bf16: A = 16 weight rows x 32 k, B = 32 k x 16
//    activation columns (only the first M are non-zero), fp32 accumulation.
//  - The activations are staged once per workgroup in LDS, in the per-r
//    permuted order that matches the unpacked operand layout, in chunks of
//    `kc` codes; the same pass forms the per-128 sums of x used by the
//    zero-point term.
//  - alpha, 2^(8-r) and the zero point are applied in fp32: per group of 128
//    when group == 128, once at the end for per-channel scales.
//  - Waves that share a row block split K; their partial results are summed
//    in LDS in a fixed order (deterministic), then written as fp32.
//  - One launch can carry up to 8 independent problems (grouped GEMV).
#include "mq_device.h"
#include "mq_internal.h"

namespace mq {

template <int R, bool GROUPED>
struct Sk {
  static constexpr int V = (R == 2 && GROUPED) ? 8 : 16;  // bytes per lane per step
  static constexpr int CPL = V * 8 / R;                   // codes per lane per step
  static constexpr int STEP = 4 * CPL;                    // codes per row per step
  static constexpr int MFMAS = CPL / 8;                   // MFMAs per step
  static constexpr int SPG = GROUPED ? 128 / STEP : 1;    // steps per group of 128
  static constexpr int PB = XPerm<R>::PB;                 // staging block (values)
};

constexpr int kXPad = 8;  // bf16 elements of padding per staged activation row

template <int R>
__device__ __forceinline__ bf16x8 unpack_op(const uint32_t* d, int i) {
  if (R == 4) return unpack_r4(d[i]);
  if (R == 2) return (i & 1) ? unpack_r2<1>(d[i >> 1]) : unpack_r2<0>(d[i >> 1]);
  return unpack_r8(d[2 * i], d[2 * i + 1]);
}

// Load PB activation values of row m starting at column k (k < K, PB | K),
// round to bf16 if needed; returns bf16 bits in v[0..PB).
template <int PB>
__device__ __forceinline__ void load_x_block(const SkinnyProblem& p, int m, int k, uint32_t* v) {
  const int64_t base = (int64_t)m * p.K + k;
  if (p.xmode == kXBf16) {
    const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.x0) + base);
#pragma unroll
    for (int j = 0; j < PB / 8; ++j) {
      u32x4 w = src[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[8 * j + 2 * e] = w[e] & 0xffffu;
        v[8 * j + 2 * e + 1] = w[e] >> 16;
      }
    }
  } else {
    const f32x4* a = reinterpret_cast<const f32x4*>(static_cast<const float*>(p.x0) + base);
    const f32x4* b = reinterpret_cast<const f32x4*>(static_cast<const float*>(p.x1) + base);
#pragma unroll
    for (int j = 0; j < PB / 4; ++j) {
      f32x4 f = a[j];
      if (p.xmode == kXF32Prod) {
        f32x4 g = b[j];
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = f[e] * g[e];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * j + e] = f32_to_bf16_rne(f[e]);
    }
  }
}

template <int R, bool GROUPED>
__global__ void __launch_bounds__(1024) skinny_kernel(const SkinnyArgs args) {
  using C = Sk<R, GROUPED>;
  extern __shared__ __align__(16) unsigned char smem[];

  // ---- locate this workgroup's problem and row blocks
  int pi = 0;
#pragma unroll 1
  for (int i = 1; i < args.count; ++i)
    if ((int)blockIdx.x >= args.p[i].tile0) pi = i;
  const SkinnyProblem& P = args.p[pi];
  const int M = args.M;
  const int K = P.K, N = P.N;
  const int KS = P.ks;
  const int waves = blockDim.x >> 6;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rb0 = ((int)blockIdx.x - P.tile0) * P.rbpw;

  const int kc = args.kc;             // codes per chunk
  const int xstride = kc + kXPad;     // staged row stride (bf16 elements)
  const int g_per_chunk = kc / 128;
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);                        // [M][xstride]
  float* sxs = reinterpret_cast<float*>(smem + (size_t)M * xstride * 2);   // [M][g_per_chunk]
  float* sxt = sxs + M * g_per_chunk;                                      // [M] per-channel total
  float* red = sxt + kSkinnyMaxM;                                          // [waves*16][M]

  const int rowbytes = K * R / 8;
  const uint32_t plane_bytes = (uint32_t)((int64_t)N * rowbytes);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(P.packed, plane_bytes);
  const int G = K / P.group;
  const __amdgpu_buffer_rsrc_t ar = make_rsrc(P.alpha, (uint32_t)((int64_t)N * G * 4));
  const __amdgpu_buffer_rsrc_t zr = make_rsrc(P.zero, (uint32_t)((int64_t)N * G * 4));

  const int rbl = wave / KS, ks = wave % KS;
  const int row0 = (rb0 + rbl) * 16;
  const int col = lane & 15, slot = lane >> 4;
  const int n_ld = row0 + col;  // row this lane loads (A operand row)
  // rows past N: point the load past the plane so it returns zeros
  const uint32_t row_off = (n_ld < N) ? (uint32_t)n_ld * (uint32_t)rowbytes : plane_bytes;

  const int Kpad = ((K + 255) / 256) * 256;
  const int nchunks = (Kpad + kc - 1) / kc;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};  // per-channel: raw sum; grouped: running scaled total
  f32x4 part = {0.f, 0.f, 0.f, 0.f};
  if (!GROUPED && threadIdx.x < kSkinnyMaxM) sxt[threadIdx.x] = 0.f;

#pragma unroll 1
  for (int c = 0; c < nchunks; ++c) {
    const int ck0 = c * kc;
    const int clen = min(kc, Kpad - ck0);
    __syncthreads();
    // ---- stage x[:, ck0 : ck0 + clen) permuted, and per-128 sums
    {
      constexpr int PB = C::PB;
      const int bpr = clen / PB;  // blocks per row in this chunk
      const int total = M * bpr;
      for (int b0 = 0; b0 < total; b0 += blockDim.x) {
        const int b = b0 + threadIdx.x;
        uint32_t v[PB];
        float s = 0.f;
        int m = 0, kb = 0;
        if (b < total) {
          m = b / bpr;
          kb = (b - m * bpr) * PB;
          if (ck0 + kb < K) {
            load_x_block<PB>(P, m, ck0 + kb, v);
          } else {
#pragma unroll
            for (int e = 0; e < PB; ++e) v[e] = 0;
          }
#pragma unroll
          for (int e = 0; e < PB; ++e) s += bf16_to_f32(v[e]);
          uint32_t outw[PB / 2];
#pragma unroll
          for (int q = 0; q < PB / 2; ++q)
            outw[q] = v[XPerm<R>::src(2 * q)] | (v[XPerm<R>::src(2 * q + 1)] << 16);
          u32x4* dst = reinterpret_cast<u32x4*>(xs + (size_t)m * xstride + kb);
#pragma unroll
          for (int q = 0; q < PB / 8; ++q) {
            u32x4 w4 = {outw[4 * q], outw[4 * q + 1], outw[4 * q + 2], outw[4 * q + 3]};
            dst[q] = w4;
          }
        }
        // sum over the 128 / PB consecutive blocks of one group of 128
#pragma unroll
        for (int off = 1; off < 128 / PB; off <<= 1) s += __shfl_xor(s, off);
        if (b < total && (kb % 128) == 0) sxs[m * g_per_chunk + kb / 128] = s;
      }
    }
    __syncthreads();
    if (!GROUPED && wave < M) {
      float s = 0.f;
      for (int gi = lane; gi < clen / 128; gi += 64) s += sxs[wave * g_per_chunk + gi];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
      if (lane == 0) sxt[wave] += s;
    }

    // ---- stream this wave's share of the chunk's steps
    const int csteps = clen / C::STEP;
    int lo, hi;
    {
      const int units = csteps / C::SPG;
      lo = (units * ks / KS) * C::SPG;
      hi = (units * (ks + 1) / KS) * C::SPG;
    }
    const uint16_t* xrow = xs + (size_t)col * xstride + slot * C::CPL;
    const bool xon = col < M;
#pragma unroll 2
    for (int st = lo; st < hi; ++st) {
      const uint32_t off = row_off + (uint32_t)((ck0 + st * C::STEP) * R / 8 + slot * C::V);
      uint32_t d[C::V / 4];
      if (C::V == 16) {
        u32x4 w = buf_load16(wr, off);
        d[0] = w[0]; d[1] = w[1]; d[2] = w[2]; d[3] = w[3];
      } else {
        u32x2 w = buf_load8(wr, off);
        d[0] = w[0]; d[1] = w[1];
      }
      float ga[4], gb[4], gsx = 0.f;
      const bool gend = GROUPED && ((st + 1) % C::SPG == 0);
      if (gend) {
        const int g = (ck0 + (st + 1) * C::STEP) / 128 - 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = row0 + 4 * slot + i;
          const uint32_t aoff = (n < N) ? (uint32_t)(n * G + g) * 4u : 0xffffffffu;
          ga[i] = __uint_as_float(buf_load4(ar, aoff));
          gb[i] = __uint_as_float(buf_load4(zr, aoff));
        }
        if (xon) gsx = sxs[col * g_per_chunk + (g - ck0 / 128)];
      }
#pragma unroll
      for (int i = 0; i < C::MFMAS; ++i) {
        bf16x8 a = unpack_op<R>(d, i);
        bf16x8 bx;
        if (xon) {
          u32x4 w = *reinterpret_cast<const u32x4*>(xrow + st * C::STEP + 8 * i);
          bx = __builtin_bit_cast(bf16x8, w);
        } else {
          u32x4 w = {0u, 0u, 0u, 0u};
          bx = __builtin_bit_cast(bf16x8, w);
        }
        part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bx, part, 0, 0, 0);
      }
      if (gend) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float av = ga[i] * Enc<R>::kStep;
          const float bv = ga[i] * (gb[i] + Enc<R>::kOffsetShift);
          acc[i] = acc[i] + av * part[i] - bv * gsx;
          part[i] = 0.f;
        }
      }
    }
  }
  if (!GROUPED) acc = part;

  // ---- cross-wave reduction (fixed order) and epilogue
  __syncthreads();
  if (col < M) {
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(wave * 16 + 4 * slot + i) * M + col] = acc[i];
  }
  __syncthreads();
  const int rows_wg = P.rbpw * 16;
  for (int t = threadIdx.x; t < rows_wg * M; t += blockDim.x) {
    const int m = t / rows_wg, rr = t - m * rows_wg;
    const int rbl2 = rr >> 4, row = rr & 15;
    const int n = (rb0 + rbl2) * 16 + row;
    if (n >= N) continue;
    float s = 0.f;
    for (int k2 = 0; k2 < KS; ++k2) s += red[((rbl2 * KS + k2) * 16 + row) * M + m];
    if (!GROUPED) {
      const float a = P.alpha[n];
      const float z = P.zero[n];
      s = (a * Enc<R>::kStep) * s - (a * (z + Enc<R>::kOffsetShift)) * sxt[m];
    }
    P.y[(int64_t)m * N + n] = s;
  }
  (void)waves;
}

// ---------------------------------------------------------------------------
// Host planning
// ---------------------------------------------------------------------------
static int step_codes(int r, bool grouped) {
  const int V = (r == 2 && grouped) ? 8 : 16;
  return 4 * V * 8 / r;
}

template <int R, bool GROUPED>
static hipError_t launch_t(const SkinnyArgs& a, int waves, size_t lds, hipStream_t s) {
  static bool attr_set = false;  // benign race: idempotent attribute call
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)skinny_kernel<R, GROUPED>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  int tiles = a.p[a.count - 1].tile0 + a.p[a.count - 1].tiles;
  hipLaunchKernelGGL((skinny_kernel<R, GROUPED>), dim3(tiles), dim3(64 * waves), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_skinny(SkinnyArgs& args, int r, bool grouped, hipStream_t stream) {
  const int waves = 16;
  const int M = args.M;
  const int step = step_codes(r, grouped);
  // activation chunk: at most 64 KiB of staged bf16, a multiple of 256 codes
  int kmax = 0;
  for (int i = 0; i < args.count; ++i) kmax = args.p[i].K > kmax ? args.p[i].K : kmax;
  const int kpad_max = ((kmax + 255) / 256) * 256;
  int kc = (32768 / M) / 256 * 256;
  if (kc > kpad_max) kc = kpad_max;
  args.kc = kc;
  int tile0 = 0;
  for (int i = 0; i < args.count; ++i) {
    SkinnyProblem& p = args.p[i];
    const int kpad = ((p.K + 255) / 256) * 256;
    // steps (in units of groups when grouped) each wave gets
    const int units = grouped ? kpad / 128 : kpad / step;
    int ks = 1;
    while (ks < waves && units / (ks * 2) >= 4) ks *= 2;
    p.ks = ks;
    p.rbpw = waves / ks;
    const int rblocks = (p.N + 15) / 16;
    p.tiles = (rblocks + p.rbpw - 1) / p.rbpw;
    p.tile0 = tile0;
    tile0 += p.tiles;
  }
  const int gpc = kc / 128;
  const size_t lds = (size_t)M * (kc + kXPad) * 2 + (size_t)(M * gpc + kSkinnyMaxM) * 4 +
                     (size_t)waves * 16 * M * 4;
  switch (r * 2 + (grouped ? 1 : 0)) {
    case 4: return launch_t<2, false>(args, waves, lds, stream);
    case 5: return launch_t<2, true>(args, waves, lds, stream);
    case 8: return launch_t<4, false>(args, waves, lds, stream);
    case 9: return launch_t<4, true>(args, waves, lds, stream);
    case 16: return launch_t<8, false>(args, waves, lds, stream);
    default: return launch_t<8, true>(args, waves, lds, stream);
  }
}

}  // namespace mq
