// Argument sweep of the C ABI under host AddressSanitizer and
// UndefinedBehaviorSanitizer (built and run by tests/test_abi_sanitize.py on a
// machine without a GPU).  Every entry point is called with null, misaligned,
// out-of-range and extreme arguments; each call must return an mq_status
// without touching memory it was not given (the sanitizers abort the process
// otherwise).  Valid-looking calls stop at the device check (no GPU), so no
// kernel is ever launched and the dummy addresses are never dereferenced.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "mq.h"

namespace {

int g_calls = 0, g_bad = 0;

void expect_status(int s, const char* what) {
  ++g_calls;
  if (s < MQ_OK || s > MQ_ERR_HIP) {
    std::printf("%s: status %d out of range\n", what, s);
    ++g_bad;
  }
}

void expect(int s, int want, const char* what) {
  ++g_calls;
  if (s != want) {
    std::printf("%s: status %d, expected %d\n", what, s, want);
    ++g_bad;
  }
}

}  // namespace

int main() {
  // dummy device addresses: aligned and misaligned, never dereferenced
  auto* P16 = reinterpret_cast<uint8_t*>(0x10000);
  auto* P1 = reinterpret_cast<uint8_t*>(0x10001);
  const float* F16 = reinterpret_cast<const float*>(0x10000);
  float* Y16 = reinterpret_cast<float*>(0x10000);
  const uint16_t* X16 = reinterpret_cast<const uint16_t*>(0x10000);
  const int64_t big[] = {0, 1, 63, 64, 65, 128, 4096, 65536, 65600, (int64_t)1 << 31,
                         (int64_t)1 << 40, INT64_MAX, -1, INT64_MIN};
  const int rs[] = {-1, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 64};

  for (int64_t N : big)
    for (int64_t K : big) {
      for (int r : rs) {
        expect_status((int)mq_packed_bytes(N, K, r) >= 0, "packed_bytes");
        expect_status(mq_pack(P16, N, K, r, P16, nullptr), "pack");
        for (int64_t g : {K, (int64_t)128, (int64_t)0, (int64_t)-128}) {
          expect_status(mq_gemv(P16, r, F16, F16, g, N, K, X16, 1, Y16, nullptr), "gemv");
          expect_status(mq_gemm(P16, r, F16, F16, g, N, K, X16, 17, Y16, nullptr, 0, nullptr),
                        "gemm");
          expect_status(mq_gemm_noalloc(P16, r, F16, F16, g, N, K, X16, 300, Y16, nullptr),
                        "gemm_noalloc");
          expect_status(mq_gemv_bitplanes(P16, r, 0, F16, F16, g, N, K, X16, 2, Y16, nullptr),
                        "gemv_bitplanes");
          expect_status(mq_overflow_apply(reinterpret_cast<const int32_t*>(P16),
                                          reinterpret_cast<const uint16_t*>(P16), r, F16, g, N, K,
                                          X16, 3, Y16, nullptr),
                        "overflow_apply");
        }
        expect_status(mq_overflow_rows(P16, N, K, r, reinterpret_cast<int32_t*>(P16), nullptr),
                      "overflow_rows");
      }
      for (int64_t M : big) {
        (void)mq_gemm_workspace_bytes(M, N, K, 128);
        (void)mq_gemm_workspace_bytes(M, N, K, K);
        (void)mq_mlp_workspace_bytes(M, N);
        expect_status(mq_gemm(P16, 4, F16, F16, 128, N, K, X16, M, Y16, P16, 1 << 20, nullptr),
                      "gemm M");
      }
      (void)mq_bitplanes_bytes(N, K);
      expect_status(mq_quantize(F16, N, K, 128, P16, Y16, Y16, nullptr), "quantize");
      expect_status(mq_pack_bitplanes(P16, N, K, P16, nullptr), "pack_bitplanes");
    }

  // specific refusals, checked exactly
  expect(mq_gemv(nullptr, 4, F16, F16, 64, 4, 64, X16, 1, Y16, nullptr), MQ_ERR_NULL, "gemv null");
  expect(mq_gemv(P16, 5, F16, F16, 64, 4, 64, X16, 1, Y16, nullptr), MQ_ERR_PRECISION, "gemv r");
  expect(mq_gemv(P1, 4, F16, F16, 64, 4, 64, X16, 1, Y16, nullptr), MQ_ERR_ALIGN, "gemv align");
  expect(mq_gemv(P16, 4, F16, F16, 64, (int64_t)1 << 40, 65536, X16, 1, Y16, nullptr),
         MQ_ERR_SHAPE, "gemv N*K overflow");
  expect(mq_gemv(P16, 4, F16, F16, 64, INT64_MAX, 64, X16, 1, Y16, nullptr), MQ_ERR_SHAPE,
         "gemv huge N");

  // grouped and mixed launches: counts, null arrays and per-problem checks
  std::vector<mq_gemv_problem> probs(17);
  for (auto& p : probs) p = mq_gemv_problem{P16, F16, F16, X16, Y16, 64, 64, 64};
  int rr[17];
  for (int i = 0; i < 17; ++i) rr[i] = rs[i % 12];
  for (int c : {-1, 0, 1, 5, 16, 17})
    for (int64_t M : {(int64_t)0, (int64_t)1, (int64_t)8, (int64_t)9, INT64_MAX}) {
      expect_status(mq_gemv_grouped(probs.data(), c, 4, M, nullptr), "gemv_grouped");
      expect_status(mq_gemv_mixed(probs.data(), rr, c, M, nullptr), "gemv_mixed");
    }
  expect(mq_gemv_grouped(nullptr, 2, 4, 1, nullptr), MQ_ERR_NULL, "grouped null");
  expect(mq_gemv_mixed(probs.data(), nullptr, 2, 1, nullptr), MQ_ERR_NULL, "mixed null r");

  // Mix'n'Match stacks and the MLP block: inconsistent shapes, bad r, sizes
  mq_linear lin{P16, F16, F16, 64, 64, 64};
  mq_layer L{4, lin, lin, lin, lin, lin, lin, lin};
  std::vector<mq_layer> layers(3, L);
  for (int n : {-1, 0, 1, 3})
    for (int64_t M : {(int64_t)0, (int64_t)1, (int64_t)8, (int64_t)9, INT64_MAX}) {
      (void)mq_mixnmatch_workspace_bytes(layers.data(), n, M);
      size_t off[10];
      expect_status(mq_mixnmatch_workspace_offsets(layers.data(), n, M, off), "offsets");
      expect_status(mq_mixnmatch_forward(layers.data(), n, X16, M, Y16, P16, 1 << 20, nullptr),
                    "mixnmatch_forward");
      expect_status(mq_mixnmatch_forward_inplace(layers.data(), n, Y16, M, P16, 1 << 20, nullptr),
                    "mixnmatch_forward_inplace");
    }
  layers[1].down = mq_linear{P16, F16, F16, 64, 65, 65};
  expect(mq_mixnmatch_forward(layers.data(), 3, X16, 1, Y16, P16, 1 << 20, nullptr), MQ_ERR_SHAPE,
         "stack bad down");
  layers[1].down = lin;
  layers[2].r = 7;
  expect(mq_mixnmatch_forward(layers.data(), 3, X16, 1, Y16, P16, 1 << 20, nullptr),
         MQ_ERR_PRECISION, "stack bad r");
  expect(mq_mixnmatch_forward(nullptr, 3, X16, 1, Y16, P16, 1 << 20, nullptr), MQ_ERR_NULL,
         "stack null");
  for (int r : rs)
    for (int act : {-1, 0, 1, 2, 3})
      for (int64_t M : {(int64_t)0, (int64_t)1, (int64_t)8, (int64_t)9})
        expect_status(mq_mlp_decode(&lin, &lin, &lin, r, act, X16, M, Y16, P16, 1 << 20, nullptr),
                      "mlp_decode");
  expect(mq_mlp_decode(nullptr, &lin, &lin, 4, 0, X16, 1, Y16, P16, 1 << 20, nullptr), MQ_ERR_NULL,
         "mlp null");

  for (int s = -2; s < 12; ++s) (void)mq_status_string(s);
  (void)mq_version();
  (void)mq_last_hip_error();

  std::printf("abi sweep: %d calls, %d unexpected\n", g_calls, g_bad);
  return g_bad == 0 ? 0 : 1;
}
