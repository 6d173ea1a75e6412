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
//    buffer load (rows past N and bytes past the plane read as zero).  Loads
//    run DEPTH steps ahead of use in a rolling register buffer, and the first
//    DEPTH are issued before the activations are staged, so the two memory
//    latencies overlap.
//  - The bytes are unpacked in registers into exact bf16 integers (see
//    mq_device.h) and multiplied on the matrix cores with
//    v_mfma_f32_16x16x32_bf16: A = 16 weight rows x 32 k, B = 32 k x 16
//    activation columns (only the first M are non-zero), fp32 accumulation.
//  - The activations are staged once per workgroup in LDS as stored (the
//    plane layout makes unpacked operands come out in natural k order), in
//    chunks of `kc` codes; the same pass forms the sums of x and of
//    offset * x used by the zero-point and encoding-offset terms: per group
//    of 128 for group-128 scales, only the chunk's totals per activation row
//    for per-channel scales.
//  - alpha, 2^(8-r) and the zero point are applied in fp32: per group of 128
//    when group == 128, once at the end for per-channel scales (whose alpha
//    and z are fetched at kernel start).
//  - Waves that share a row block split K (while each keeps at least 16 load
//    steps); their partial results are summed in LDS in a fixed order
//    (deterministic), then written as fp32.
//  - One launch can carry up to 16 independent problems (grouped GEMV), each
//    at its own r; a problem may pair two matrices of one shape that share x
//    (alternate row blocks of a workgroup), which can also write bf16 of the
//    elementwise product of the two outputs.
#include "mq_device.h"
#include "mq_internal.h"

namespace mq {

template <int R, bool GROUPED, bool LEAN = false>
struct Sk {
  // r = 3 and r = 6 planes are split in a high-bit and a low-bit plane
  static constexpr bool SPLIT = (R == 3 || R == 6);
  static constexpr int RL = R == 6 ? 2 : 1;               // split: low-plane width
  static constexpr int RH = R - RL;                       // split: high-plane width
  static constexpr int V = (R == 2 && GROUPED) ? 8 : 16;  // bytes per lane per step
  static constexpr int CPL = SPLIT ? 32 : V * 8 / R;      // codes per lane per step
  static constexpr int HB = CPL * RH / 8, LB = CPL * RL / 8;  // split: bytes per lane per step
  static constexpr int STEP = 4 * CPL;                    // codes per row per step
  static constexpr int MFMAS = CPL / 8;                   // MFMAs per step
  static constexpr int SPG = GROUPED ? 128 / STEP : 1;    // steps per group of 128
  static constexpr int PB = 8;                            // staging block (values)
  // loads in flight per lane: 8, and 4 at r = 2 (measured on the Gemma MLP
  // launch at r = 2: 15.0 against 16.6 us with 8; r = 4 and 8 unchanged or
  // slower with 4).  LEAN (per-channel launches whose LDS leaves room for six
  // workgroups per CU): 6 at r = 4, which brings the kernel from 88 to 76
  // VGPRs, so six waves fit per SIMD instead of five (a lone 14336 x 3584
  // matrix at r = 4: 9.4 -> 8.6 us).  Where the staged activations allow only
  // five workgroups per CU anyway, 8 keeps more bytes in flight (the Gemma
  // nine-product launch was 0.4 us slower with 6).  The split precisions
  // (two planes per step) take 4: 88 instead of 120 VGPRs per-channel (five
  // waves per SIMD instead of four), 124 instead of 160 with groups; the
  // Gemma MLP at r = 6 / 3 went from 34.6-36.5 / 30.7-31.2 to 33.4-33.8 /
  // 29.1 us (6 measured in between).
  static constexpr int DEPTH = R == 2 ? 4 : (R == 4 && LEAN) ? 6 : SPLIT ? 4 : 8;
};

constexpr int kXPad = 8;          // bf16 elements of padding per staged activation row
constexpr int kSkinnyWaves = 4;   // waves per workgroup
// threads per workgroup, as a constant: blockDim.x is read from the dispatch
// packet with a vector load, and waiting for that load would also wait for
// every weight load issued before it
constexpr int kSkinnyThreads = 64 * kSkinnyWaves;
constexpr int kSkinnyFillTiles = 256;  // workgroups a launch should have (one per CU)

template <int R>
__device__ __forceinline__ bf16x8 unpack_op(const uint32_t* d, int i, const UnpackK& k,
                                            const UnpackK36& k36) {
  if (R == 4) return unpack_r4(d[i], k);
  if (R == 2) return (i & 1) ? unpack_r2<1>(d[i >> 1], k) : unpack_r2<0>(d[i >> 1], k);
  if (R == 6) return unpack_r6(d[i], d[4 + (i >> 1)], i & 1, k36);  // 4 high, 2 low words
  if (R == 3) return unpack_r3(d[i >> 1], d[2], i, k36);             // 2 high, 1 low word
  return unpack_r8(d[2 * i], d[2 * i + 1]);
}

constexpr int kStageBatch = 2;    // fp32 activation loads in flight per thread while staging

// Load 8 activation values of row m starting at column k (k < K, 8 | K) as
// four words of bf16 pairs, rounding fp32 sources to bf16 (nearest even).
__device__ __forceinline__ u32x4 load_x8(const SkinnyProblem& p, int m, int k) {
  const int64_t base = (int64_t)m * p.K + k;
  if (p.xmode == kXBf16)
    return *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.x0) + base);
  const f32x4* a = reinterpret_cast<const f32x4*>(static_cast<const float*>(p.x0) + base);
  const f32x4* b = reinterpret_cast<const f32x4*>(static_cast<const float*>(p.x1) + base);
  uint32_t v[8];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    f32x4 f = a[j];
    if (p.xmode == kXF32Prod) {
      f32x4 g = b[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) f[e] = f[e] * g[e];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) v[4 * j + e] = f32_to_bf16_rne(f[e]);
  }
  u32x4 w = {v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16)};
  return w;
}

// Activation of a gated MLP's gate output: identity, SiLU g * sigmoid(g), or
// GELU in its tanh form g/2 * (1 + tanh(z)), z = sqrt(2/pi) * (g + 0.044715 g^3),
// evaluated as g / (1 + exp(-2z)) (the same function): 1 + tanh(z) cancels
// where tanh(z) is near -1, and in fp32 loses most of its digits there.
__device__ __forceinline__ float gate_act(float g, int act) {
  if (act == kActSilu) return g / (1.f + expf(-g));
  if (act == kActGeluTanh) {
    const float z = 0.7978845608028654f * (g + 0.044715f * g * g * g);
    return g / (1.f + expf(-2.f * z));
  }
  return g;
}

// One workgroup's share of problem pi, at slice precision R.
template <int R, bool GROUPED, bool LEAN = false>
__device__ __forceinline__ void skinny_body(const SkinnyArgs& args, const int pi) {
  using C = Sk<R, GROUPED, LEAN>;
  using LD = LoadT<R, C::SPLIT ? 0 : C::V>;
  extern __shared__ __align__(16) unsigned char smem[];
  const SkinnyProblem& P = args.p[pi];
  const int M = args.M;
  const int K = P.K, N = P.N;
  const int KS = P.ks;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  // a pair: the workgroup's row blocks alternate between the two matrices
  // (even: first, odd: second) over rbpw / 2 distinct 16-row blocks
  const bool paired = P.y2 != nullptr;
  const int rb0 = ((int)blockIdx.x - P.tile0) * (paired ? P.rbpw / 2 : P.rbpw);

  const int kc = args.kc;             // codes per chunk
  const int xstride = kc + kXPad;     // staged row stride (bf16 elements)
  const int g_per_chunk = kc / 128;
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);                        // [M][xstride]
  float* sxs = reinterpret_cast<float*>(smem + (size_t)M * xstride * 2);   // [M][g_per_chunk]
  float* sxos = sxs + M * g_per_chunk;      // [M][g_per_chunk] sums of offset * x
  float* sxt = sxos + M * g_per_chunk;      // [M] per-channel total of x
  float* sxot = sxt + kSkinnyMaxM;          // [M] per-channel total of offset * x
  float* red = sxot + kSkinnyMaxM;          // [waves*16][M]
  float* fin = red + kSkinnyWaves * 16 * M;  // [rows_wg][M] results (pairs)

  const int rowbytes = K * R / 8;
  const uint32_t plane_bytes = (uint32_t)((int64_t)N * rowbytes);
  const int G = K / P.group;

  const int rbl = wave / KS, ks = wave % KS;
  const int sel = paired ? (rbl & 1) : 0;  // which matrix this wave streams
  const int row0 = (rb0 + (paired ? rbl >> 1 : rbl)) * 16;
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(sel ? P.packed2 : P.packed, plane_bytes);
  const float* alpha_w = sel ? P.alpha2 : P.alpha;
  const float* zero_w = sel ? P.zero2 : P.zero;
  const int col = lane & 15, slot = lane >> 4;
  const int n_ld = row0 + col;  // row this lane loads (A operand row)
  // rows past N: point the load past the plane so it returns zeros
  // split planes: rows of the high plane, then rows of the low plane
  const uint32_t hrow = (uint32_t)(K * C::RH / 8), lrow = (uint32_t)(K * C::RL / 8);
  const uint32_t row_off =
      (n_ld < N) ? (uint32_t)n_ld * (C::SPLIT ? hrow : (uint32_t)rowbytes) : plane_bytes;
  const uint32_t row_off_lo =
      (n_ld < N) ? (uint32_t)N * hrow + (uint32_t)n_ld * lrow : plane_bytes;

  // per-channel epilogue operands, fetched now: thread t writes row
  // rr = t % rows_wg of the tile, for m = t / rows_wg, + kSkinnyThreads / rows_wg, ...
  const int rows_wg = P.rbpw * 16;
  const int ep_rr = threadIdx.x % rows_wg;
  float ep_a = 0.f, ep_b = 0.f;
  // virtual row block of the epilogue row: for a pair, even blocks are the
  // first matrix's and odd blocks the second's
  auto ep_sel = [&]() __attribute__((always_inline)) { return paired ? ((ep_rr >> 4) & 1) : 0; };
  auto ep_n = [&]() __attribute__((always_inline)) {
    return (rb0 + (paired ? ep_rr >> 5 : ep_rr >> 4)) * 16 + (ep_rr & 15);
  };
  if (!GROUPED) {
    const int n = ep_n();
    if (n < N) {
      const int ep_sel = paired ? ((ep_rr >> 4) & 1) : 0;
      const float a = (ep_sel ? P.alpha2 : P.alpha)[n], z = (ep_sel ? P.zero2 : P.zero)[n];
      ep_a = a * Enc<R>::kStep;
      ep_b = a * z;
    }
  }

  const int Kpad = ((K + 511) / 512) * 512;
  const int nchunks = (Kpad + kc - 1) / kc;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};  // per-channel: raw sum; grouped: running scaled total
  f32x4 part = {0.f, 0.f, 0.f, 0.f};
  if (!GROUPED && threadIdx.x < kSkinnyMaxM) {
    sxt[threadIdx.x] = 0.f;
    sxot[threadIdx.x] = 0.f;
  }
  const UnpackK uk = UnpackK::make();
  UnpackK36 uk36;
  if constexpr (C::SPLIT) uk36 = UnpackK36::make();
  // all lanes read activations: columns past M duplicate column M - 1 (ignored)
  const int xcol = col < M ? col : M - 1;

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(P.x0, (uint32_t)((int64_t)M * K * 2));
  const __amdgpu_buffer_rsrc_t ar = make_rsrc(alpha_w, (uint32_t)((int64_t)N * G * 4));
  const __amdgpu_buffer_rsrc_t zr = make_rsrc(zero_w, (uint32_t)((int64_t)N * G * 4));

#pragma unroll 1
  for (int c = 0; c < nchunks; ++c) {
    const int ck0 = c * kc;
    const int clen = min(kc, Kpad - ck0);
    const int csteps = clen / C::STEP;
    int lo, hi;
    {
      const int units = csteps / C::SPG;
      lo = __builtin_amdgcn_readfirstlane((units * ks / KS) * C::SPG);
      hi = __builtin_amdgcn_readfirstlane((units * (ks + 1) / KS) * C::SPG);
    }
    // offsets of step st for this lane; steps past the range read past the
    // plane (bounds check returns zeros), so the loop has no branches
    const uint32_t cbase =
        C::SPLIT ? row_off + (uint32_t)((ck0 + slot * C::CPL) * C::RH / 8)
                 : row_off + (uint32_t)(ck0 * R / 8 + slot * C::V);
    const uint32_t cbase_lo = row_off_lo + (uint32_t)((ck0 + slot * C::CPL) * C::RL / 8);
    auto loff = [&](int st) -> uint32_t {
      return st < hi ? cbase + (uint32_t)(st * (C::STEP * (C::SPLIT ? C::RH : R) / 8))
                     : 0x80000000u;
    };
    auto loff_lo = [&](int st) -> uint32_t {
      return st < hi ? cbase_lo + (uint32_t)(st * (C::STEP * C::RL / 8)) : 0x80000000u;
    };
    typename LD::T buf[C::DEPTH];
    // nothing in flight when the chunk starts: the previous chunk's last
    // refills (past its steps) must land before their registers are reused.
    // Said explicitly here, the compiler's own wait for them (which, placed
    // after the staging loads, also waited for the activations before the
    // first weight load) goes away, and the weights are issued behind the
    // staging as intended.  vmcnt(0); expcnt and lgkmcnt at their maximum.
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
    // ---- stage x[:, ck0 : ck0 + clen) as stored, then form the per-128 sums
    //      of x and of offset * x (v_dot2 against constant bf16 pairs).
    constexpr int PB = C::PB;
    if (P.xmode == kXBf16) {
      // bf16 activations: buffer-to-LDS loads, one 1 KiB piece per wave
      // instruction; columns past K read as zeros through the bounds check.
      const int pieces = clen / 512;  // per row
      for (int pc = wave; pc < M * pieces; pc += kSkinnyWaves) {
        const int m = pc / pieces, j = pc - m * pieces;
        const int k = ck0 + j * 512 + lane * 8;
        const uint32_t off = k < K ? (uint32_t)((m * K + k) * 2) : 0x80000000u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            xr, (__attribute__((address_space(3))) void*)(xs + (size_t)m * xstride + j * 512), 16,
            off, 0, 0, 0);
      }
    } else {
      // fp32 sources (rounded to bf16 on the way): through registers, up to
      // kStageBatch loads in flight per thread
      const int bpr = clen / PB;
      const int total = M * bpr;
      const int nthr = kSkinnyThreads;
      for (int b0 = 0; b0 < total; b0 += kStageBatch * nthr) {
        u32x4 w4[kStageBatch];
#pragma unroll
        for (int j = 0; j < kStageBatch; ++j) {
          const int b = b0 + j * nthr + threadIdx.x;
          u32x4 z4 = {0u, 0u, 0u, 0u};
          w4[j] = z4;
          if (b < total) {
            const int m = b / bpr;
            const int kb = (b - m * bpr) * PB;
            if (ck0 + kb < K) w4[j] = load_x8(P, m, ck0 + kb);
          }
        }
#pragma unroll
        for (int j = 0; j < kStageBatch; ++j) {
          const int b = b0 + j * nthr + threadIdx.x;
          if (b < total) {
            const int m = b / bpr;
            const int kb = (b - m * bpr) * PB;
            *reinterpret_cast<u32x4*>(xs + (size_t)m * xstride + kb) = w4[j];
          }
        }
      }
    }
    // ---- first DEPTH weight loads of this chunk, issued behind the staging
    //      loads so that waiting for the activations does not wait for them
#pragma unroll
    for (int j = 0; j < C::DEPTH; ++j) buf[j] = LD::load(wr, loff(lo + j), loff_lo(lo + j));
    __syncthreads();
    if constexpr (GROUPED) {
      // per group of 128: sum of x and of offset * x, one thread per
      // (row, group) summing its 16 blocks of 8 in order (no cross-lane
      // reduction)
      const int gl_n = clen / 128;
      const uint32_t ones = 0x3F803F80u;
      for (int t = threadIdx.x; t < M * gl_n; t += kSkinnyThreads) {
        const int m = t / gl_n, gl = t - m * gl_n;
        const uint16_t* p = xs + (size_t)m * xstride + gl * 128;
        u32x4 w4[16];
#pragma unroll
        for (int c = 0; c < 16; ++c) w4[c] = *reinterpret_cast<const u32x4*>(p + c * PB);
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < 16; ++c)
#pragma unroll
          for (int q = 0; q < 4; ++q) s = dot2_bf16(w4[c][q], ones, s);
        sxs[m * g_per_chunk + gl] = s;
        sxos[m * g_per_chunk + gl] = (float)Enc<R>::kOffset * s;
      }
      __syncthreads();  // the streaming loop reads other threads' group sums
    } else {
      // per-channel scales need only the chunk's totals per activation row:
      // each thread sums its blocks of 8, then one reduction per row (the
      // per-group sums and their lane shuffles are not formed at all)
      const int bpr = clen / PB;
      const uint32_t ones = 0x3F803F80u;
      float* part_s = sxs;   // [waves] partial sums (sxs is free per-channel)
      for (int m = 0; m < M; ++m) {
        float s = 0.f;
        for (int bi = threadIdx.x; bi < bpr; bi += kSkinnyThreads) {
          const u32x4 w4 = *reinterpret_cast<const u32x4*>(xs + (size_t)m * xstride + bi * PB);
#pragma unroll
          for (int q = 0; q < 4; ++q) s = dot2_bf16(w4[q], ones, s);
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
        if (lane == 0) part_s[wave] = s;
        __syncthreads();
        if (threadIdx.x == 0) {
          float ts = 0.f;
          for (int w = 0; w < kSkinnyWaves; ++w) ts += part_s[w];
          sxt[m] += ts;
          sxot[m] += (float)Enc<R>::kOffset * ts;
        }
        __syncthreads();
      }
    }

    // ---- stream this wave's share of the chunk's steps
    const uint16_t* xrow = xs + (size_t)xcol * xstride + slot * C::CPL;
#pragma unroll 1
    for (int base = lo; base < hi; base += C::DEPTH) {
#pragma unroll
      for (int j = 0; j < C::DEPTH; ++j) {
        const int st = base + j;
        uint32_t d[LD::NW];
        LD::words(buf[j], d);
        const uint16_t* xp = xrow + st * C::STEP;
        if (st < hi) {
        if constexpr (GROUPED) {
          {
#pragma unroll
            for (int i = 0; i < C::MFMAS; ++i) {
              const u32x4 w = *reinterpret_cast<const u32x4*>(xp + 8 * i);
              part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(unpack_op<R>(d, i, uk, uk36),
                                                             __builtin_bit_cast(bf16x8, w), part,
                                                             0, 0, 0);
            }
            if ((st + 1) % C::SPG == 0) {
              const int g = (ck0 + (st + 1) * C::STEP) / 128 - 1;
              const float gsx = sxs[xcol * g_per_chunk + (g - ck0 / 128)];
              const float gsxo = sxos[xcol * g_per_chunk + (g - ck0 / 128)];
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int n = row0 + 4 * slot + i;
                const uint32_t aoff = (n < N) ? (uint32_t)(n * G + g) * 4u : 0x80000000u;
                const float ga = __uint_as_float(buf_load4(ar, aoff));
                const float gb = __uint_as_float(buf_load4(zr, aoff));
                const float av = ga * Enc<R>::kStep;
                const float bv = ga * gb;
                acc[i] = acc[i] + av * (part[i] - gsxo) - bv * gsx;
                part[i] = 0.f;
              }
            }
          }
        } else {
#pragma unroll
          for (int i = 0; i < C::MFMAS; ++i) {
            const u32x4 w = *reinterpret_cast<const u32x4*>(xp + 8 * i);
            part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(unpack_op<R>(d, i, uk, uk36),
                                                           __builtin_bit_cast(bf16x8, w), part,
                                                           0, 0, 0);
          }
        }
        }
        // refill this slot after its last use, so the buffer stays in place
        buf[j] = LD::load(wr, loff(st + C::DEPTH), loff_lo(st + C::DEPTH));
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
  const int mstep = kSkinnyThreads / rows_wg;
  {
    const int rr = ep_rr;
    const int rbl2 = rr >> 4, row = rr & 15;
    const int n = ep_n();
    float* yo = ep_sel() ? P.y2 : P.y;
    if (n < N) {
      for (int m = threadIdx.x / rows_wg; m < M; m += mstep) {
        float s = 0.f;
        for (int k2 = 0; k2 < KS; ++k2) s += red[((rbl2 * KS + k2) * 16 + row) * M + m];
        if (!GROUPED) s = ep_a * (s - sxot[m]) - ep_b * sxt[m];
        yo[(int64_t)m * N + n] = s;
        if (paired) fin[rr * M + m] = s;
        else if (P.ybf) P.ybf[(int64_t)m * N + n] = (uint16_t)f32_to_bf16_rne(s);
      }
    }
  }
  if (paired && P.ybf) {
    // bf16(first * act(second)) for the rows of this workgroup
    __syncthreads();
    const int half = rows_wg / 2;  // distinct rows
    for (int t = threadIdx.x; t < half * M; t += kSkinnyThreads) {
      const int j = t % half, m = t / half;
      const int rr1 = ((j >> 4) * 2) * 16 + (j & 15), rr2 = rr1 + 16;
      const int n = (rb0 + (j >> 4)) * 16 + (j & 15);
      if (n < N) {
        const float v = fin[rr1 * M + m] * gate_act(fin[rr2 * M + m], P.act);
        P.ybf[(int64_t)m * N + n] = (uint16_t)f32_to_bf16_rne(v);
      }
    }
  }
}

// The problems of a launch may differ in r (one launch can serve several
// precisions of one stored model); each workgroup runs its problem's body.
// The byte-aligned precisions (2, 4, 8) and the split ones (3, 6) are two
// kernels, so that the registers of one set do not limit the other's occupancy.
// Cache warm-up workgroup w of n: reads its own contiguous share of
// warm[0, bytes) (a multiple of 64 KiB; the shares past the end are empty)
// with buffer-to-LDS loads into one KiB of LDS that nothing reads (no
// registers held, and the loads cannot be dropped), all in flight at once,
// then waits for them before the workgroup's LDS is released.  Contiguous
// shares measured 1% faster on the Mistral-7B stack than 4 KiB pieces
// interleaved over the workgroups, which gained nothing.
__device__ __forceinline__ void warm_body(const uint8_t* warm, uint32_t bytes, int w, int n) {
  extern __shared__ __align__(16) unsigned char smem[];
  const __amdgpu_buffer_rsrc_t r = make_rsrc(warm, bytes);
  const uint32_t share = ((bytes + (uint32_t)n - 1) / (uint32_t)n + 65535u) & ~65535u;
  const uint32_t beg = (uint32_t)w * share;
  for (uint32_t off = beg + threadIdx.x * 16; off < beg + share; off += kSkinnyThreads * 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)smem, 16,
                                             off, 0, 0, 0);
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
}

template <bool GROUPED, bool SPLIT, bool LEAN>
__device__ __forceinline__ void skinny_dispatch(const SkinnyArgs& args) {
  if ((int)blockIdx.x >= args.tiles) {
    warm_body(args.warm, args.warm_bytes, (int)blockIdx.x - args.tiles, args.warm_wgs);
    return;
  }
  int pi = 0;
#pragma unroll 1
  for (int i = 1; i < args.count; ++i)
    if ((int)blockIdx.x >= args.p[i].tile0) pi = i;
  const int r = args.p[pi].r;
  if constexpr (SPLIT) {
    if (r == 6) skinny_body<6, GROUPED>(args, pi);
    else skinny_body<3, GROUPED>(args, pi);
  } else {
    if (r == 8) skinny_body<8, GROUPED, LEAN>(args, pi);
    else if (r == 4) skinny_body<4, GROUPED, LEAN>(args, pi);
    else skinny_body<2, GROUPED, LEAN>(args, pi);
  }
}

template <bool GROUPED, bool SPLIT>
__global__ void __launch_bounds__(kSkinnyThreads) skinny_kernel(const SkinnyArgs args) {
  skinny_dispatch<GROUPED, SPLIT, false>(args);
}

// per-channel scales, r in {2, 4, 8}, short enough activation chunks for six
// workgroups per CU: the same body with fewer registers (Sk::DEPTH)
__global__ void __launch_bounds__(kSkinnyThreads) skinny_lean_kernel(const SkinnyArgs args) {
  skinny_dispatch<false, false, true>(args);
}

// ---------------------------------------------------------------------------
// Host planning
// ---------------------------------------------------------------------------
static int step_codes(int r, bool grouped) {
  if (r == 3 || r == 6) return Sk<6, false>::STEP;  // 32 codes per lane for both
  const int V = (r == 2 && grouped) ? 8 : 16;
  return 4 * V * 8 / r;
}

template <bool GROUPED, bool SPLIT, bool LEAN>
static hipError_t launch_t(const SkinnyArgs& a, size_t lds, hipStream_t s) {
  const void* fn = LEAN ? (const void*)skinny_lean_kernel : (const void*)skinny_kernel<GROUPED, SPLIT>;
  // the LDS limit is raised once per process (a function-local static is
  // initialized exactly once, also when several host threads launch)
  static const hipError_t attr =
      hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (attr != hipSuccess) return attr;
  const int wgs = a.tiles + (a.warm && a.warm_bytes ? a.warm_wgs : 0);
  if constexpr (LEAN)
    hipLaunchKernelGGL(skinny_lean_kernel, dim3(wgs), dim3(kSkinnyThreads), lds, s, a);
  else
    hipLaunchKernelGGL((skinny_kernel<GROUPED, SPLIT>), dim3(wgs), dim3(kSkinnyThreads), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_skinny(SkinnyArgs& args, bool grouped, hipStream_t stream) {
  const int waves = kSkinnyWaves;
  const int M = args.M;
  // activation chunk: at most 64 KiB of staged bf16, a multiple of 512 codes
  int kmax = 0;
  for (int i = 0; i < args.count; ++i) kmax = args.p[i].K > kmax ? args.p[i].K : kmax;
  const int kpad_max = ((kmax + 511) / 512) * 512;
  int kc = (32768 / M) / 512 * 512;
  if (kc > kpad_max) kc = kpad_max;
  args.kc = kc;
  // split of K: at least ~16 load steps per wave (on the Gemma MLP launch of
  // nine products, 16 to 24 measured about 7% faster than 12 or 8; above 24
  // a single-r launch no longer fills the chip)
  int steps_per_wave[kMaxProblems];
  for (int i = 0; i < args.count; ++i) {
    SkinnyProblem& p = args.p[i];
    const int step = step_codes(p.r, grouped);
    const int kpad = ((p.K + 511) / 512) * 512;
    const int steps = kpad / step;
    const int spg = grouped ? 128 / step : 1;
    const int units = steps / spg;
    int ks = 1;
    // a pair needs two row blocks (one per matrix) per workgroup
    const int ks_max = p.y2 ? waves / 2 : waves;
    while (ks < ks_max && (units / (ks * 2)) * spg >= 16) ks *= 2;
    p.ks = ks;
    p.rbpw = waves / ks;
    const int rblocks = (p.N + 15) / 16 * (p.y2 ? 2 : 1);
    p.tiles = (rblocks + p.rbpw - 1) / p.rbpw;
    steps_per_wave[i] = steps / ks;
  }
  // balance: the waves of one precision should carry about the same number
  // of steps, or the longer ones set the launch's tail (at r = 2 the rule
  // above leaves the 14336-long down projection 28 steps per wave against 14
  // for up and gate; splitting it to 14 took that launch from 18.0 to
  // 17.0 us).  Problems at different r keep their own lengths: the launch
  // runs the longest first.
  for (int i = 0; i < args.count; ++i) {
    SkinnyProblem& p = args.p[i];
    int tmin = 1 << 30;
    for (int j = 0; j < args.count; ++j)
      if (args.p[j].r == p.r && steps_per_wave[j] < tmin) tmin = steps_per_wave[j];
    const int step = step_codes(p.r, grouped);
    const int steps = ((p.K + 511) / 512) * 512 / step;
    const int spg = grouped ? 128 / step : 1;
    const int ks_max = p.y2 ? waves / 2 : waves;
    while (p.ks < ks_max && 2 * steps_per_wave[i] > 3 * tmin &&
           ((steps / spg) / (p.ks * 2)) * spg >= 8) {
      p.ks *= 2;
      p.rbpw = waves / p.ks;
      const int rblocks = (p.N + 15) / 16 * (p.y2 ? 2 : 1);
      p.tiles = (rblocks + p.rbpw - 1) / p.rbpw;
      steps_per_wave[i] = steps / p.ks;
    }
  }
  // fill: a launch with fewer workgroups than CUs (a lone 14336-long down
  // projection at r = 2 gets 112) splits the K of its longest problem further
  // while every wave keeps at least 4 load steps (r = 2 down alone: 13.4 ->
  // about 9 us; a lone 14336 x 3584 matrix at r = 2, 224 -> 448 workgroups of
  // 7 steps per wave: 9.0 -> 8.2 us)
  for (;;) {
    int tiles = 0, best = -1;
    for (int i = 0; i < args.count; ++i) tiles += args.p[i].tiles;
    if (tiles >= kSkinnyFillTiles) break;
    for (int i = 0; i < args.count; ++i) {
      const SkinnyProblem& p = args.p[i];
      const int steps = ((p.K + 511) / 512) * 512 / step_codes(p.r, grouped);
      const int spg = grouped ? 128 / step_codes(p.r, grouped) : 1;
      const int ks_max = p.y2 ? waves / 2 : waves;
      if (p.ks < ks_max && ((steps / spg) / (p.ks * 2)) * spg >= 4 &&
          (best < 0 || steps_per_wave[i] > steps_per_wave[best]))
        best = i;
    }
    if (best < 0) break;
    SkinnyProblem& p = args.p[best];
    p.ks *= 2;
    p.rbpw = waves / p.ks;
    const int rblocks = (p.N + 15) / 16 * (p.y2 ? 2 : 1);
    p.tiles = (rblocks + p.rbpw - 1) / p.rbpw;
    steps_per_wave[best] = ((p.K + 511) / 512) * 512 / step_codes(p.r, grouped) / p.ks;
  }
  // longest workgroups first: they start early and the short ones fill in
  for (int i = 1; i < args.count; ++i)
    for (int j = i; j > 0 && steps_per_wave[j] > steps_per_wave[j - 1]; --j) {
      SkinnyProblem t = args.p[j];
      args.p[j] = args.p[j - 1];
      args.p[j - 1] = t;
      int u = steps_per_wave[j];
      steps_per_wave[j] = steps_per_wave[j - 1];
      steps_per_wave[j - 1] = u;
    }
  int tile0 = 0;
  for (int i = 0; i < args.count; ++i) {
    args.p[i].tile0 = tile0;
    tile0 += args.p[i].tiles;
  }
  args.tiles = tile0;
  if (args.warm_wgs < 0) args.warm_wgs = 0;
  const int gpc = kc / 128;
  const size_t lds = (size_t)M * (kc + kXPad) * 2 +
                     (size_t)(2 * M * gpc + 2 * kSkinnyMaxM) * 4 + (size_t)2 * waves * 16 * M * 4;
  const bool split = args.p[0].r == 3 || args.p[0].r == 6;
  if (split)
    return grouped ? launch_t<true, true, false>(args, lds, stream)
                   : launch_t<false, true, false>(args, lds, stream);
  if (grouped) return launch_t<true, false, false>(args, lds, stream);
  // six workgroups per CU fit the 160 KiB of LDS (in 512-byte units)
  const bool lean = 6 * ((lds + 511) / 512 * 512) <= 160 * 1024;
  return lean ? launch_t<false, false, true>(args, lds, stream)
              : launch_t<false, false, false>(args, lds, stream);
}

}  // namespace mq
