// C ABI of libmq: argument validation, status codes, dispatch to the gfx950
// kernels.  Nothing is enqueued unless every argument is valid.
#include <atomic>
#include <cstring>

#include "../../include/mq.h"
#include "mq_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

mq_status hip_fail(hipError_t e) {
  g_last_hip_error = (int)e;
  return MQ_ERR_HIP;
}

// Per-device cache of "is gfx950" (0 unknown, 1 yes, 2 no).
std::atomic<int> g_dev_ok[64];

mq_status check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= 64) return MQ_ERR_DEVICE;
  int s = g_dev_ok[dev].load(std::memory_order_relaxed);
  if (s == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e);
    s = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_dev_ok[dev].store(s, std::memory_order_relaxed);
  }
  return s == 1 ? MQ_OK : MQ_ERR_DEVICE;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_r(int r) { return r == 2 || r == 3 || r == 4 || r == 6 || r == 8; }

constexpr int64_t kMaxK = 65536;
constexpr int64_t kMaxPlaneBytes = (int64_t)1 << 31;
// Mix'n'Match stack: bytes at the head of the next layer's q plane that a
// layer's second launch warms into the last-level cache, and the workgroups
// that read them, 64 KiB each (on the 32-layer Mistral-7B stack: 1321 to
// 1307 us per token; 4 and 8 MiB gained less, 10 MiB and more cost time)
constexpr uint64_t kStackWarmBytes = (uint64_t)6 << 20;
constexpr int kWarmWorkgroups = 96;

// a * b > lim for a, b >= 1, without forming the product (sizes come from
// the caller unchecked and may be anywhere in int64)
bool mul_gt(int64_t a, int64_t b, int64_t lim) { return a > lim / b; }

// Shape checks shared by the products.
mq_status check_matrix(int64_t N, int64_t K, int64_t group, int r) {
  if (!valid_r(r)) return MQ_ERR_PRECISION;
  if (N < 1 || K < 64 || K % 64 != 0 || K > kMaxK) return MQ_ERR_SHAPE;
  if (mul_gt(N, K, kMaxPlaneBytes)) return MQ_ERR_SHAPE;
  if (!(group == K || (group == 128 && K % 128 == 0))) return MQ_ERR_GROUP;
  return MQ_OK;
}

mq_status check_product(const uint8_t* packed, int r, const float* alpha, const float* zero,
                        int64_t group, int64_t N, int64_t K, const void* x, const float* y) {
  if (!packed || !alpha || !zero || !x || !y) return MQ_ERR_NULL;
  mq_status s = check_matrix(N, K, group, r);
  if (s != MQ_OK) return s;
  if (!aligned16(packed) || !aligned16(x) || !aligned16(y)) return MQ_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(alpha) & 3u) || (reinterpret_cast<uintptr_t>(zero) & 3u))
    return MQ_ERR_ALIGN;
  return MQ_OK;
}

mq_status skinny_run(mq::SkinnyArgs& a, bool grouped, hipStream_t stream) {
  hipError_t e = mq::launch_skinny(a, grouped, stream);
  return e == hipSuccess ? MQ_OK : hip_fail(e);
}

// One launch per (scale granularity, precision set) present among the problems.
// warm, warm_bytes: optional cache warm-up carried by the first of these launches.
mq_status run_mixed(mq::SkinnyProblem* probs, int count, int64_t M, hipStream_t s,
                    const uint8_t* warm = nullptr, uint32_t warm_bytes = 0) {
  for (int pass = 0; pass < 4; ++pass) {
    const bool grouped = (pass & 1) != 0, split = (pass & 2) != 0;
    mq::SkinnyArgs a;
    std::memset(&a, 0, sizeof a);
    a.M = (int)M;
    a.warm = warm;
    a.warm_bytes = warm_bytes;
    a.warm_wgs = kWarmWorkgroups;
    for (int i = 0; i < count; ++i)
      if ((probs[i].group != probs[i].K) == grouped && mq::split_precision(probs[i].r) == split)
        a.p[a.count++] = probs[i];
    if (a.count == 0) continue;
    mq_status st = skinny_run(a, grouped, s);
    if (st != MQ_OK) return st;
    warm = nullptr;
  }
  return MQ_OK;
}

// Validate every problem, then launch them (one launch per granularity and
// precision set present).
mq_status gemv_products(const mq_gemv_problem* problems, const int* r, int count, int64_t M,
                        hipStream_t stream) {
  if (M < 1 || M > mq::kSkinnyMaxM) return MQ_ERR_SHAPE;
  for (int i = 0; i < count; ++i) {
    const mq_gemv_problem& p = problems[i];
    mq_status s = check_product(p.packed, r[i], p.alpha, p.zero, p.group, p.N, p.K, p.x, p.y);
    if (s != MQ_OK) return s;
  }
  mq_status s = check_device();
  if (s != MQ_OK) return s;
  mq::SkinnyProblem probs[mq::kMaxProblems];
  for (int i = 0; i < count; ++i) {
    const mq_gemv_problem& p = problems[i];
    probs[i] = mq::SkinnyProblem{p.packed, p.alpha, p.zero, p.x, nullptr, p.y, (int)p.N,
                                 (int)p.K, (int)p.group, mq::kXBf16, r[i], 0, 0, 0, 0};
  }
  return run_mixed(probs, count, M, stream);
}

}  // namespace

extern "C" {

const char* mq_status_string(int status) {
  switch (status) {
    case MQ_OK: return "MQ_OK";
    case MQ_ERR_NULL: return "MQ_ERR_NULL: a required pointer is NULL";
    case MQ_ERR_SHAPE: return "MQ_ERR_SHAPE: a size is out of range";
    case MQ_ERR_PRECISION: return "MQ_ERR_PRECISION: r must be 2, 3, 4, 6 or 8";
    case MQ_ERR_GROUP: return "MQ_ERR_GROUP: group must be K or 128 (with K % 128 == 0)";
    case MQ_ERR_ALIGN: return "MQ_ERR_ALIGN: a pointer is not suitably aligned";
    case MQ_ERR_WORKSPACE: return "MQ_ERR_WORKSPACE: workspace missing or too small";
    case MQ_ERR_DEVICE: return "MQ_ERR_DEVICE: the current device is not a gfx950";
    case MQ_ERR_HIP: return "MQ_ERR_HIP: a HIP runtime call failed";
    default: return "unknown mq_status";
  }
}

int mq_last_hip_error(void) { return g_last_hip_error; }

const char* mq_version(void) { return "mq 0.1 gfx950"; }

size_t mq_packed_bytes(int64_t N, int64_t K, int r) {
  if (!valid_r(r) || N < 0 || K < 0) return 0;
  if (N > 0 && K > 0 && mul_gt(N, K, (int64_t)1 << 56)) return 0;
  return (size_t)(N * K * r / 8);
}

mq_status mq_quantize(const float* w, int64_t N, int64_t K, int64_t group, uint8_t* codes,
                      float* alpha, float* zero, void* stream) {
  if (!w || !codes || !alpha || !zero) return MQ_ERR_NULL;
  if (N < 1 || K < 1 || mul_gt(N, K, kMaxPlaneBytes)) return MQ_ERR_SHAPE;
  if (!(group == K || (group == 128 && K % 128 == 0))) return MQ_ERR_GROUP;
  if ((reinterpret_cast<uintptr_t>(w) & 3u) || (reinterpret_cast<uintptr_t>(alpha) & 3u) ||
      (reinterpret_cast<uintptr_t>(zero) & 3u))
    return MQ_ERR_ALIGN;
  mq_status s = check_device();
  if (s != MQ_OK) return s;
  hipError_t e = mq::launch_quantize(w, N, K, group, codes, alpha, zero, (hipStream_t)stream);
  return e == hipSuccess ? MQ_OK : hip_fail(e);
}

mq_status mq_pack(const uint8_t* codes, int64_t N, int64_t K, int r, uint8_t* packed,
                  void* stream) {
  if (!codes || !packed) return MQ_ERR_NULL;
  if (!valid_r(r)) return MQ_ERR_PRECISION;
  if (N < 1 || K < 64 || K % 64 != 0 || mul_gt(N, K, kMaxPlaneBytes)) return MQ_ERR_SHAPE;
  if (!aligned16(codes) || !aligned16(packed)) return MQ_ERR_ALIGN;
  mq_status s = check_device();
  if (s != MQ_OK) return s;
  hipError_t e = mq::launch_pack(codes, N, K, r, packed, (hipStream_t)stream);
  return e == hipSuccess ? MQ_OK : hip_fail(e);
}

mq_status mq_gemv(const uint8_t* packed, int r, const float* alpha, const float* zero,
                  int64_t group, int64_t N, int64_t K, const uint16_t* x, int64_t M, float* y,
                  void* stream) {
  mq_status s = check_product(packed, r, alpha, zero, group, N, K, x, y);
  if (s != MQ_OK) return s;
  if (M < 1 || M > mq::kSkinnyMaxM) return MQ_ERR_SHAPE;
  s = check_device();
  if (s != MQ_OK) return s;
  mq::SkinnyArgs a;
  std::memset(&a, 0, sizeof a);
  a.count = 1;
  a.M = (int)M;
  a.p[0] = mq::SkinnyProblem{packed, alpha, zero, x, nullptr, y, (int)N, (int)K, (int)group,
                             mq::kXBf16, r, 0, 0, 0, 0};
  return skinny_run(a, group != K, (hipStream_t)stream);
}

mq_status mq_gemv_grouped(const mq_gemv_problem* problems, int count, int r, int64_t M,
                          void* stream) {
  if (!problems) return MQ_ERR_NULL;
  if (count < 1 || count > mq::kMaxProblems) return MQ_ERR_SHAPE;
  int rs[mq::kMaxProblems];
  for (int i = 0; i < count; ++i) rs[i] = r;
  return gemv_products(problems, rs, count, M, (hipStream_t)stream);
}

mq_status mq_gemv_mixed(const mq_gemv_problem* problems, const int* r, int count, int64_t M,
                        void* stream) {
  if (!problems || !r) return MQ_ERR_NULL;
  if (count < 1 || count > mq::kMaxProblems) return MQ_ERR_SHAPE;
  return gemv_products(problems, r, count, M, (hipStream_t)stream);
}

size_t mq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t group) {
  // 0 for shapes mq_gemm refuses (the planners assume valid shapes)
  if (check_matrix(N, K, group, 8) != MQ_OK) return 0;
  if (M < 1 || mul_gt(M, K, (int64_t)1 << 30) || mul_gt(M, N, (int64_t)1 << 31)) return 0;
  return mq::gemm_workspace_bytes(M, N, K, group);
}

}  // extern "C"

namespace mq {

mq_status record_hip_error(hipError_t e) { return hip_fail(e); }

mq_status gemm_check(const uint8_t* packed, int r, const float* alpha, const float* zero,
                     int64_t group, int64_t N, int64_t K, const uint16_t* x, int64_t M,
                     const float* y) {
  mq_status s = check_product(packed, r, alpha, zero, group, N, K, x, y);
  if (s != MQ_OK) return s;
  if (M < 1 || mul_gt(M, K, (int64_t)1 << 30) || mul_gt(M, N, (int64_t)1 << 31)) return MQ_ERR_SHAPE;
  return MQ_OK;
}

}  // namespace mq

extern "C" {

mq_status mq_gemm(const uint8_t* packed, int r, const float* alpha, const float* zero,
                  int64_t group, int64_t N, int64_t K, const uint16_t* x, int64_t M, float* y,
                  void* workspace, size_t workspace_bytes, void* stream) {
  mq_status s = mq::gemm_check(packed, r, alpha, zero, group, N, K, x, M, y);
  if (s != MQ_OK) return s;
  const size_t need = mq::gemm_workspace_bytes(M, N, K, group);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MQ_ERR_WORKSPACE;
  s = check_device();
  if (s != MQ_OK) return s;
  if (M <= mq::kSkinnyMaxM) return mq_gemv(packed, r, alpha, zero, group, N, K, x, M, y, stream);
  hipError_t e = mq::launch_gemm(packed, r, alpha, zero, group, N, K, x, M, y, workspace,
                                 (hipStream_t)stream);
  return e == hipSuccess ? MQ_OK : hip_fail(e);
}

// ---------------------------------------------------------------- Extra precision

mq_status mq_overflow_rows(const uint8_t* codes, int64_t N, int64_t K, int r, int32_t* row_ptr,
                           void* stream) {
  if (!codes || !row_ptr) return MQ_ERR_NULL;
  if (!valid_r(r)) return MQ_ERR_PRECISION;
  if (N < 1 || K < 64 || K % 64 != 0 || K > kMaxK || mul_gt(N, K, kMaxPlaneBytes - 1)) return MQ_ERR_SHAPE;
  if (!aligned16(codes) || (reinterpret_cast<uintptr_t>(row_ptr) & 3u)) return MQ_ERR_ALIGN;
  mq_status s = check_device();
  if (s != MQ_OK) return s;
  hipError_t e = mq::launch_overflow_rows(codes, N, K, r, row_ptr, (hipStream_t)stream);
  return e == hipSuccess ? MQ_OK : hip_fail(e);
}

mq_status mq_overflow_cols(const uint8_t* codes, int64_t N, int64_t K, int r,
                           const int32_t* row_ptr, uint16_t* col_idx, void* stream) {
  if (!codes || !row_ptr || !col_idx) return MQ_ERR_NULL;
  if (!valid_r(r)) return MQ_ERR_PRECISION;
  if (N < 1 || K < 64 || K % 64 != 0 || K > kMaxK || mul_gt(N, K, kMaxPlaneBytes - 1)) return MQ_ERR_SHAPE;
  if (!aligned16(codes) || (reinterpret_cast<uintptr_t>(row_ptr) & 3u) ||
      (reinterpret_cast<uintptr_t>(col_idx) & 1u))
    return MQ_ERR_ALIGN;
  mq_status s = check_device();
  if (s != MQ_OK) return s;
  hipError_t e = mq::launch_overflow_cols(codes, N, K, r, row_ptr, col_idx, (hipStream_t)stream);
  return e == hipSuccess ? MQ_OK : hip_fail(e);
}

// ---- bit-plane storage

static mq_status check_bitplane_shape(int64_t N, int64_t K) {
  if (N < 1 || K < 512 || K % 512 != 0 || K > kMaxK || mul_gt(N, K, kMaxPlaneBytes))
    return MQ_ERR_SHAPE;
  return MQ_OK;
}

size_t mq_bitplanes_bytes(int64_t N, int64_t K) {
  return check_bitplane_shape(N, K) == MQ_OK ? (size_t)(N * K) : 0;
}

mq_status mq_pack_bitplanes(const uint8_t* codes, int64_t N, int64_t K, uint8_t* planes,
                            void* stream) {
  if (!codes || !planes) return MQ_ERR_NULL;
  mq_status s = check_bitplane_shape(N, K);
  if (s != MQ_OK) return s;
  if (!aligned16(codes) || !aligned16(planes)) return MQ_ERR_ALIGN;
  s = check_device();
  if (s != MQ_OK) return s;
  hipError_t e = mq::launch_pack_bitplanes(codes, N, K, planes, (hipStream_t)stream);
  return e == hipSuccess ? MQ_OK : hip_fail(e);
}

mq_status mq_gemv_bitplanes(const uint8_t* planes, int r, int extra, const float* alpha,
                            const float* zero, int64_t group, int64_t N, int64_t K,
                            const uint16_t* x, int64_t M, float* y, void* stream) {
  if (!planes || !alpha || !zero || !x || !y) return MQ_ERR_NULL;
  if (r < 1 || r > 8) return MQ_ERR_PRECISION;
  if (extra != 0 && extra != 1) return MQ_ERR_PRECISION;
  mq_status s = check_bitplane_shape(N, K);
  if (s != MQ_OK) return s;
  if (M < 1 || M > mq::kSkinnyMaxM) return MQ_ERR_SHAPE;
  if (!(group == K || group == 128)) return MQ_ERR_GROUP;
  if (!aligned16(planes) || !aligned16(x) || !aligned16(y)) return MQ_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(alpha) & 3u) || (reinterpret_cast<uintptr_t>(zero) & 3u))
    return MQ_ERR_ALIGN;
  s = check_device();
  if (s != MQ_OK) return s;
  hipError_t e = mq::launch_gemv_bitplanes(planes, r, extra != 0, alpha, zero, group, N, K, x, M,
                                           y, (hipStream_t)stream);
  return e == hipSuccess ? MQ_OK : hip_fail(e);
}

static mq_status check_overflow_apply(const int32_t* row_ptr, const uint16_t* col_idx, int r,
                                       const float* alpha, int64_t group, int64_t N, int64_t K,
                                       const uint16_t* x, int64_t M, const float* y) {
  if (!row_ptr || !col_idx || !alpha || !x || !y) return MQ_ERR_NULL;
  if (!valid_r(r)) return MQ_ERR_PRECISION;
  if (N < 1 || K < 64 || K % 64 != 0 || K > kMaxK || mul_gt(N, K, kMaxPlaneBytes - 1))
    return MQ_ERR_SHAPE;
  if (!(group == K || (group == 128 && K % 128 == 0))) return MQ_ERR_GROUP;
  if (M < 1 || mul_gt(M, K, (int64_t)1 << 30) || mul_gt(M, N, (int64_t)1 << 31)) return MQ_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(row_ptr) & 3u) || (reinterpret_cast<uintptr_t>(col_idx) & 1u) ||
      (reinterpret_cast<uintptr_t>(alpha) & 3u) || (reinterpret_cast<uintptr_t>(x) & 1u) ||
      (reinterpret_cast<uintptr_t>(y) & 3u))
    return MQ_ERR_ALIGN;
  return MQ_OK;
}

mq_status mq_overflow_apply(const int32_t* row_ptr, const uint16_t* col_idx, int r,
                            const float* alpha, int64_t group, int64_t N, int64_t K,
                            const uint16_t* x, int64_t M, float* y, void* stream) {
  mq_overflow_problem p{row_ptr, col_idx, alpha, x, y, N, K, group};
  return mq_overflow_apply_grouped(&p, 1, r, M, stream);
}

mq_status mq_overflow_apply_grouped(const mq_overflow_problem* problems, int count, int r,
                                    int64_t M, void* stream) {
  if (!problems) return MQ_ERR_NULL;
  if (count < 1 || count > mq::kMaxProblems) return MQ_ERR_SHAPE;
  for (int i = 0; i < count; ++i) {
    const mq_overflow_problem& p = problems[i];
    const mq_status st =
        check_overflow_apply(p.row_ptr, p.col_idx, r, p.alpha, p.group, p.N, p.K, p.x, M, p.y);
    if (st != MQ_OK) return st;
  }
  mq_status s = check_device();
  if (s != MQ_OK) return s;
  mq::OverflowProblem probs[mq::kMaxProblems];
  for (int i = 0; i < count; ++i) {
    const mq_overflow_problem& p = problems[i];
    probs[i] = mq::OverflowProblem{p.row_ptr, p.col_idx, p.alpha, p.x, p.y, (int)p.N, (int)p.K,
                                   (int)p.group, 0};
  }
  hipError_t e = mq::launch_overflow_apply(probs, count, r, M, (hipStream_t)stream);
  return e == hipSuccess ? MQ_OK : hip_fail(e);
}

// ---------------------------------------------------------------- Mix'n'Match

namespace {

struct StackDims {
  int64_t H, Hkv, F;
};

// MQ_OK, or the status check_product would return for this linear's shape,
// precision, group and pointer alignment (MQ_ERR_SHAPE on a shape mismatch)
mq_status linear_ok(const mq_linear& l, int64_t n, int64_t k, int r) {
  if (!l.packed || !l.alpha || !l.zero) return MQ_ERR_NULL;
  if (l.N != n || l.K != k) return MQ_ERR_SHAPE;
  mq_status s = check_matrix(l.N, l.K, l.group, r);
  if (s != MQ_OK) return s;
  if (!aligned16(l.packed)) return MQ_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(l.alpha) & 3u) || (reinterpret_cast<uintptr_t>(l.zero) & 3u))
    return MQ_ERR_ALIGN;
  return MQ_OK;
}

mq_status check_stack(const mq_layer* layers, int n_layers, int64_t M, StackDims* d) {
  if (!layers) return MQ_ERR_NULL;
  if (n_layers < 1 || M < 1 || M > mq::kSkinnyMaxM) return MQ_ERR_SHAPE;
  const int64_t H = layers[0].q.N, Hkv = layers[0].k.N, F = layers[0].up.N;
  if (H > mq::kStackMaxH) return MQ_ERR_SHAPE;  // the norm holds a row in registers
  for (int i = 0; i < n_layers; ++i) {
    const mq_layer& L = layers[i];
    const mq_linear* all[7] = {&L.q, &L.k, &L.v, &L.o, &L.up, &L.gate, &L.down};
    for (const mq_linear* l : all)
      if (!l->packed || !l->alpha || !l->zero) return MQ_ERR_NULL;
    if (!valid_r(L.r)) return MQ_ERR_PRECISION;
    const int64_t want[7][2] = {{H, H}, {Hkv, H}, {Hkv, H}, {H, H}, {F, H}, {F, H}, {H, F}};
    for (int j = 0; j < 7; ++j) {
      const mq_status s = linear_ok(*all[j], want[j][0], want[j][1], L.r);
      if (s != MQ_OK) return s;
    }
  }
  d->H = H;
  d->Hkv = Hkv;
  d->F = F;
  return MQ_OK;
}

size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

// a, q, k, v, u, g, o, d, bf16(q), bf16(u * g)
constexpr int kStackBuffers = 10;

void stack_offsets(const StackDims& d, int64_t M, size_t* off, size_t* total) {
  size_t o = 0;
  const size_t sizes[kStackBuffers] = {
      (size_t)(M * d.H * 2),   (size_t)(M * d.H * 4), (size_t)(M * d.Hkv * 4),
      (size_t)(M * d.Hkv * 4), (size_t)(M * d.F * 4), (size_t)(M * d.F * 4),
      (size_t)(M * d.H * 4),   (size_t)(M * d.H * 4), (size_t)(M * d.H * 2),
      (size_t)(M * d.F * 2)};
  for (int i = 0; i < kStackBuffers; ++i) {
    off[i] = o;
    o += up256(sizes[i]);
  }
  *total = o;
}

// Run the problems of one launch, split by scale granularity.
mq::SkinnyProblem prob(const mq_linear& l, int r, const void* x0, const void* x1, int xmode,
                       float* y) {
  return mq::SkinnyProblem{l.packed, l.alpha, l.zero, x0, x1, y, (int)l.N, (int)l.K,
                           (int)l.group, xmode, r, 0, 0, 0, 0};
}

}  // namespace

size_t mq_mixnmatch_workspace_bytes(const mq_layer* layers, int n_layers, int64_t M) {
  StackDims d;
  if (check_stack(layers, n_layers, M, &d) != MQ_OK) return 0;
  size_t off[kStackBuffers], total;
  stack_offsets(d, M, off, &total);
  return total;
}

mq_status mq_mixnmatch_workspace_offsets(const mq_layer* layers, int n_layers, int64_t M,
                                         size_t* offsets) {
  if (!offsets) return MQ_ERR_NULL;
  StackDims d;
  mq_status s = check_stack(layers, n_layers, M, &d);
  if (s != MQ_OK) return s;
  size_t total;
  stack_offsets(d, M, offsets, &total);
  return MQ_OK;
}

namespace {

// The layer loop of both stack entry points.  x == nullptr: h holds the
// residual stream on entry; else h = x (bf16) first.
mq_status run_stack(const mq_layer* layers, int n_layers, const uint16_t* x, float* h, int64_t M,
                    void* workspace, size_t workspace_bytes, hipStream_t st) {
  StackDims d;
  mq_status s = check_stack(layers, n_layers, M, &d);
  if (s != MQ_OK) return s;
  if (!h) return MQ_ERR_NULL;
  if (!aligned16(h) || (x && !aligned16(x))) return MQ_ERR_ALIGN;
  size_t off[kStackBuffers], total;
  stack_offsets(d, M, off, &total);
  if (!workspace || workspace_bytes < total) return MQ_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return MQ_ERR_ALIGN;
  s = check_device();
  if (s != MQ_OK) return s;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  uint16_t* a = reinterpret_cast<uint16_t*>(ws + off[0]);
  float* q = reinterpret_cast<float*>(ws + off[1]);
  float* k = reinterpret_cast<float*>(ws + off[2]);
  float* v = reinterpret_cast<float*>(ws + off[3]);
  float* u = reinterpret_cast<float*>(ws + off[4]);
  float* g = reinterpret_cast<float*>(ws + off[5]);
  float* o = reinterpret_cast<float*>(ws + off[6]);
  float* dd = reinterpret_cast<float*>(ws + off[7]);
  uint16_t* qb = reinterpret_cast<uint16_t*>(ws + off[8]);
  uint16_t* ugb = reinterpret_cast<uint16_t*>(ws + off[9]);

  hipError_t e = x ? mq::launch_load_rmsnorm_bf16(x, h, a, M, d.H, st)
                   : mq::launch_rmsnorm_bf16(h, a, M, d.H, st);
  if (e != hipSuccess) return hip_fail(e);
  for (int i = 0; i < n_layers; ++i) {
    const mq_layer& L = layers[i];
    // first launch: q (with its bf16 copy), k, v and, when up and gate share
    // a scale granularity, the up/gate pair in the same workgroups, which
    // also writes bf16(up * gate); the second launch then reads bf16 inputs
    const bool pair = L.up.group == L.gate.group;
    mq::SkinnyProblem p1[5] = {prob(L.q, L.r, a, nullptr, mq::kXBf16, q),
                               prob(L.k, L.r, a, nullptr, mq::kXBf16, k),
                               prob(L.v, L.r, a, nullptr, mq::kXBf16, v),
                               prob(L.up, L.r, a, nullptr, mq::kXBf16, u),
                               prob(L.gate, L.r, a, nullptr, mq::kXBf16, g)};
    p1[0].ybf = qb;
    if (pair) {
      p1[3].packed2 = L.gate.packed;
      p1[3].alpha2 = L.gate.alpha;
      p1[3].zero2 = L.gate.zero;
      p1[3].y2 = g;
      p1[3].ybf = ugb;
    }
    s = run_mixed(p1, pair ? 4 : 5, M, st);
    if (s != MQ_OK) return s;
    mq::SkinnyProblem p2[2] = {prob(L.o, L.r, qb, nullptr, mq::kXBf16, o),
                               pair ? prob(L.down, L.r, ugb, nullptr, mq::kXBf16, dd)
                                    : prob(L.down, L.r, u, g, mq::kXF32Prod, dd)};
    // this launch (about a third of the layer's bytes, on fewer workgroups
    // than the CUs hold) also warms the head of the next layer's q plane
    const uint8_t* warm = nullptr;
    uint32_t warm_bytes = 0;
    if (i + 1 < n_layers) {
      const mq_linear& nq = layers[i + 1].q;
      const uint64_t qb = (uint64_t)nq.N * (uint64_t)nq.K * (uint64_t)layers[i + 1].r / 8;
      warm = nq.packed;
      warm_bytes = (uint32_t)(qb < kStackWarmBytes ? qb : kStackWarmBytes);
    }
    s = run_mixed(p2, 2, M, st, warm, warm_bytes);
    if (s != MQ_OK) return s;
    // the last layer leaves its own input a in the workspace
    e = mq::launch_residual_rmsnorm(h, o, dd, i + 1 < n_layers ? a : nullptr, M, d.H, st);
    if (e != hipSuccess) return hip_fail(e);
  }
  return MQ_OK;
}

}  // namespace

mq_status mq_mixnmatch_forward(const mq_layer* layers, int n_layers, const uint16_t* x,
                               int64_t M, float* h_out, void* workspace, size_t workspace_bytes,
                               void* stream) {
  if (!x) return MQ_ERR_NULL;
  return run_stack(layers, n_layers, x, h_out, M, workspace, workspace_bytes,
                   (hipStream_t)stream);
}

mq_status mq_mixnmatch_forward_inplace(const mq_layer* layers, int n_layers, float* h,
                                       int64_t M, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  return run_stack(layers, n_layers, nullptr, h, M, workspace, workspace_bytes,
                   (hipStream_t)stream);
}

// ---- decode MLP block

size_t mq_mlp_workspace_bytes(int64_t M, int64_t F) {
  if (M < 1 || M > mq::kSkinnyMaxM || F < 1 || F > kMaxPlaneBytes) return 0;
  return 2 * up256((size_t)(M * F * 4)) + up256((size_t)(M * F * 2));
}

mq_status mq_mlp_decode(const mq_linear* up, const mq_linear* gate, const mq_linear* down, int r,
                        int act, const uint16_t* x, int64_t M, float* y, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (!up || !gate || !down || !x || !y) return MQ_ERR_NULL;
  if (!up->packed || !up->alpha || !up->zero || !gate->packed || !gate->alpha || !gate->zero ||
      !down->packed || !down->alpha || !down->zero)
    return MQ_ERR_NULL;
  if (!valid_r(r) || act < mq::kActIdentity || act > mq::kActGeluTanh) return MQ_ERR_PRECISION;
  if (M < 1 || M > mq::kSkinnyMaxM) return MQ_ERR_SHAPE;
  const int64_t F = up->N, H = up->K;
  for (const mq_status s0 :
       {linear_ok(*up, F, H, r), linear_ok(*gate, F, H, r), linear_ok(*down, H, F, r)})
    if (s0 != MQ_OK) return s0;
  if (up->group != gate->group) return MQ_ERR_GROUP;
  if (!aligned16(x) || !aligned16(y)) return MQ_ERR_ALIGN;
  const size_t need = mq_mlp_workspace_bytes(M, F);
  if (!workspace || workspace_bytes < need) return MQ_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return MQ_ERR_ALIGN;
  mq_status s = check_device();
  if (s != MQ_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  const size_t fb = up256((size_t)(M * F * 4));
  float* u = reinterpret_cast<float*>(ws);
  float* g = reinterpret_cast<float*>(ws + fb);
  uint16_t* a = reinterpret_cast<uint16_t*>(ws + 2 * fb);
  // up and gate in one launch (rows paired in each workgroup, x read once),
  // writing bf16(u * act(g)); then down from that bf16 copy
  mq::SkinnyProblem p1 = prob(*up, r, x, nullptr, mq::kXBf16, u);
  p1.packed2 = gate->packed;
  p1.alpha2 = gate->alpha;
  p1.zero2 = gate->zero;
  p1.y2 = g;
  p1.ybf = a;
  p1.act = act;
  s = run_mixed(&p1, 1, M, st);
  if (s != MQ_OK) return s;
  mq::SkinnyProblem p2 = prob(*down, r, a, nullptr, mq::kXBf16, y);
  return run_mixed(&p2, 1, M, st);
}

}  // extern "C"
