// Internal launcher interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mq.h"

namespace mq {

// How a skinny-kernel problem reads its activations.
enum XMode : int {
  kXBf16 = 0,     // x: bf16 bits [M, K]
  kXF32 = 1,      // x0: fp32 [M, K], rounded to bf16 (nearest even) on load
  kXF32Prod = 2,  // x0 * x1 (fp32 product), rounded to bf16 on load
};

constexpr int kMaxProblems = 16;
constexpr int kSkinnyMaxM = 8;
constexpr int kPanelMaxM = 64;  // mq_gemm: rows served by the small-batch kernel

struct SkinnyProblem {
  const uint8_t* packed;
  const float* alpha;
  const float* zero;
  const void* x0;
  const void* x1;
  float* y;
  int N, K, group, xmode;
  int r;         // slice precision of this problem (2, 3, 4, 6 or 8)
  int ks;        // waves sharing one 16-row block (split of K)
  int rbpw;      // 16-row blocks per workgroup (rbpw * ks == waves per workgroup)
  int tiles;     // workgroups of this problem
  int tile0;     // first workgroup index of this problem
  // optional: a second matrix of the same shape, precision and scales layout
  // on the same x (its rows are computed by the same workgroups), and a
  // bf16 copy of the output: bf16(y) alone, bf16(y * act(y2)) for a pair
  const uint8_t* packed2;
  const float* alpha2;
  const float* zero2;
  float* y2;
  uint16_t* ybf;
  int act;       // pair only: activation of the second output (kActIdentity, ...)
};

enum GateAct { kActIdentity = 0, kActSilu = 1, kActGeluTanh = 2 };


struct SkinnyArgs {
  SkinnyProblem p[kMaxProblems];
  int count;
  int M;
  int kc;        // activation codes staged per chunk (multiple of every step size)
  int tiles;     // workgroups of the products (set by launch_skinny)
  // optional cache warm-up: warm_wgs further workgroups read warm[0, warm_bytes)
  // (weights a later launch streams first) and discard it, so that the later
  // launch finds those bytes in the last-level cache; they run in this
  // launch's ramp and tail, when its own loads leave HBM idle
  const uint8_t* warm;
  uint32_t warm_bytes;
  int warm_wgs;
};

// Host-side planning + launch of the skinny (M <= 8) kernel.  `probs` hold the
// pointers, shapes and r; tiling fields are filled in here.  All problems of
// one launch share the scale granularity (grouped or per-channel) and the
// precision set: {2, 4, 8} or {3, 6} (split planes).
hipError_t launch_skinny(SkinnyArgs& args, bool grouped, hipStream_t stream);
inline bool split_precision(int r) { return r == 3 || r == 6; }

hipError_t launch_quantize(const float* w, int64_t N, int64_t K, int64_t group, uint8_t* codes,
                           float* alpha, float* zero, hipStream_t stream);
hipError_t launch_pack(const uint8_t* codes, int64_t N, int64_t K, int r, uint8_t* packed,
                       hipStream_t stream);

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t group);
size_t panel_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_panel(const uint8_t* packed, int r, const float* alpha, const float* zero,
                             int64_t group, int64_t N, int64_t K, const uint16_t* x, int64_t M,
                             float* y, void* workspace, hipStream_t s);
// y = sum over S partial [count] slices of `part`, in slice order.
hipError_t launch_reduce_slices(const float* part, float* y, int64_t count, int S, hipStream_t s);
hipError_t launch_gemm_big(const uint8_t* packed, int r, const float* alpha, const float* zero,
                           int64_t group, int64_t N, int64_t K, const uint16_t* x, int64_t M,
                           float* y, void* workspace, hipStream_t s);
// partial slices of the prefill kernel's K split (0 when it does not split)
size_t gemm_big_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm(const uint8_t* packed, int r, const float* alpha, const float* zero,
                       int64_t group, int64_t N, int64_t K, const uint16_t* x, int64_t M, float* y,
                       void* workspace, hipStream_t stream);
// Records e as this thread's last HIP error (mq_last_hip_error); returns MQ_ERR_HIP.
mq_status record_hip_error(hipError_t e);
// Argument checks of mq_gemm other than the workspace and the device.
mq_status gemm_check(const uint8_t* packed, int r, const float* alpha, const float* zero,
                     int64_t group, int64_t N, int64_t K, const uint16_t* x, int64_t M,
                     const float* y);

// Extra-Precision lists and the sparse addition.
hipError_t launch_overflow_rows(const uint8_t* codes, int64_t N, int64_t K, int r, int* row_ptr,
                                hipStream_t s);
hipError_t launch_overflow_cols(const uint8_t* codes, int64_t N, int64_t K, int r,
                                const int* row_ptr, uint16_t* col_idx, hipStream_t s);
// One matrix's lists, scales, activations and output for the sparse addition.
struct OverflowProblem {
  const int* row_ptr;
  const uint16_t* col_idx;
  const float* alpha;
  const uint16_t* x;
  float* y;
  int N, K, group;
  int tile0;  // first workgroup of this matrix (set by the launcher)
};
// The sparse addition for `count` (<= kMaxProblems) matrices at precision r
// and M activation rows, in one launch.
hipError_t launch_overflow_apply(OverflowProblem* probs, int count, int r, int64_t M,
                                 hipStream_t s);

// Mix'n'Match helpers.  The norm keeps a row in registers: H <= kStackMaxH.
constexpr int64_t kStackMaxH = 16384;
hipError_t launch_rmsnorm_bf16(const float* h, uint16_t* a, int64_t M, int64_t H,
                               hipStream_t stream);
// h = x (bf16, exact in fp32), then a = bf16(h / rms(h))
hipError_t launch_load_rmsnorm_bf16(const uint16_t* x, float* h, uint16_t* a, int64_t M,
                                    int64_t H, hipStream_t stream);
hipError_t launch_residual_rmsnorm(float* h, const float* o, const float* d, uint16_t* a,
                                   int64_t M, int64_t H, hipStream_t stream);

// Bit-plane storage (bitplane.hip).
hipError_t launch_pack_bitplanes(const uint8_t* codes, int64_t N, int64_t K, uint8_t* planes,
                                 hipStream_t s);
hipError_t launch_gemv_bitplanes(const uint8_t* planes, int r, bool extra, const float* alpha,
                                 const float* zero, int64_t group, int64_t N, int64_t K,
                                 const uint16_t* x, int64_t M, float* y, hipStream_t s);

}  // namespace mq
