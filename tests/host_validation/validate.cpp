// Host-side argument validation of every libmxq entry point, built with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host code only and
// run where no GPU is visible.  Device pointers are fake addresses that no
// call may dereference: every case either fails a host-side check (its
// expected status) or reaches the launch, which fails without a device
// (MXQ_ERR_HIP).  Extreme sizes probe the launchers' 64-bit size arithmetic,
// where an overflow is undefined behaviour and stops the run.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "mxq.h"

static int g_fail = 0, g_n = 0;

#define EXPECT(call, want)                                                               \
  do {                                                                                   \
    ++g_n;                                                                               \
    const int got_ = (call);                                                             \
    if (got_ != (want)) {                                                                \
      ++g_fail;                                                                          \
      std::printf("FAIL line %d: %s -> %d, expected %d\n", __LINE__, #call, got_, (int)(want)); \
    }                                                                                    \
  } while (0)

int main() {
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) == hipSuccess && ndev > 0) {
    std::printf("skipped: a GPU is visible (these calls pass fake device addresses)\n");
    return 0;
  }
  const int64_t BIG = INT64_C(1) << 62, HUGE_ = INT64_MAX;
  uint8_t* P = reinterpret_cast<uint8_t*>(uintptr_t(4096));   // never dereferenced
  uint16_t* X = reinterpret_cast<uint16_t*>(P);
  float* Fp = reinterpret_cast<float*>(P);
  int64_t* O = reinterpret_cast<int64_t*>(P);
  const int HIP = MXQ_ERR_HIP;

  // ---- row-wise MX quantization ----
  EXPECT(mx_quantize_rowwise(X, -1, 32, 32, P, 32, P, 1, nullptr), MXQ_ERR_SHAPE);
  EXPECT(mx_quantize_rowwise(X, 4, 40, 40, P, 48, P, 2, nullptr), MXQ_ERR_SHAPE);
  EXPECT(mx_quantize_rowwise(nullptr, 4, 32, 32, P, 32, P, 1, nullptr), MXQ_ERR_NULL);
  EXPECT(mx_quantize_rowwise(X, 4, 32, 36, P, 32, P, 1, nullptr), MXQ_ERR_ALIGN);
  EXPECT(mx_quantize_rowwise(X + 1, 4, 32, 32, P, 32, P, 1, nullptr), MXQ_ERR_ALIGN);
  EXPECT(mx_quantize_rowwise(nullptr, 0, 32, 32, nullptr, 32, nullptr, 1, nullptr), MXQ_OK);
  EXPECT(mx_quantize_rowwise(X, 4, 32, 32, P, 32, P, 1, nullptr), HIP);
  EXPECT(mx_quantize_rowwise(X, BIG, 64, 64, P, 64, P, 2, nullptr), MXQ_ERR_SHAPE);
  EXPECT(mx_quantize_rowwise(X, HUGE_, HUGE_ / 32 * 32, HUGE_, P, HUGE_, P, HUGE_, nullptr),
         MXQ_ERR_ALIGN);                                      // odd strides fail first
  EXPECT(mx_quantize_rowwise(X, HUGE_, 1 << 16, 1 << 16, P, 1 << 16, P, 1 << 11, nullptr),
         MXQ_ERR_SHAPE);
  EXPECT(mx_quantize_rowwise(X, 1 << 20, 1 << 16, 1 << 16, P, 1 << 16, P, 1 << 11, nullptr),
         HIP);                                                // 2^36 elements, row by row
  // ---- row-wise, several matrices in one launch ----
  {
    const mxq_rowwise_item good{X, 4, 32, 32, P, 32, P, 1};
    const mxq_rowwise_item bad_k{X, 4, 40, 40, P, 48, P, 2};
    const mxq_rowwise_item odd{X + 1, 4, 32, 32, P, 32, P, 1};
    const mxq_rowwise_item empty{nullptr, 0, 32, 32, nullptr, 32, nullptr, 1};
    const mxq_rowwise_item huge{X, HUGE_, 1 << 16, 1 << 16, P, 1 << 16, P, 1 << 11};
    // 2^23 strided rows of 2^16: 2^30 segments each, so two pass 2^31 together
    const mxq_rowwise_item half{X, INT64_C(1) << 23, 1 << 16, (1 << 16) + 8, P, 1 << 16, P,
                                1 << 11};
    const mxq_rowwise_item five[5] = {good, good, good, good, good};
    EXPECT(mx_quantize_rowwise_batch(five, 0, nullptr), MXQ_ERR_SHAPE);
    EXPECT(mx_quantize_rowwise_batch(five, 5, nullptr), MXQ_ERR_SHAPE);
    EXPECT(mx_quantize_rowwise_batch(nullptr, 1, nullptr), MXQ_ERR_NULL);
    const mxq_rowwise_item a[2] = {good, bad_k}, b2[2] = {odd, good}, c[2] = {empty, empty};
    const mxq_rowwise_item d[2] = {good, huge}, e[2] = {half, half}, f[3] = {empty, half, good};
    EXPECT(mx_quantize_rowwise_batch(a, 2, nullptr), MXQ_ERR_SHAPE);
    EXPECT(mx_quantize_rowwise_batch(b2, 2, nullptr), MXQ_ERR_ALIGN);
    EXPECT(mx_quantize_rowwise_batch(c, 2, nullptr), MXQ_OK);   // nothing to launch
    EXPECT(mx_quantize_rowwise_batch(d, 2, nullptr), MXQ_ERR_SHAPE);
    EXPECT(mx_quantize_rowwise_batch(e, 2, nullptr), MXQ_ERR_SHAPE);
    EXPECT(mx_quantize_rowwise_batch(f, 3, nullptr), HIP);
    EXPECT(mx_quantize_rowwise_batch(five, 4, nullptr), HIP);
  }
  // ---- column-wise / dual ----
  EXPECT(mx_quantize_colwise(X, 64, 20, 24, nullptr, 0, P, 64, 64, P, 2, nullptr, nullptr),
         MXQ_ERR_SHAPE);
  EXPECT(mx_quantize_colwise(X, 64, 32, 32, O, 4, P, 160, 160, P, 16, O, nullptr), MXQ_ERR_SHAPE);
  EXPECT(mx_quantize_colwise(X, 64, 32, 32, O, 4, P, 192, 192, P, 16, O, nullptr), HIP);
  EXPECT(mx_quantize_colwise(X, HUGE_, 32, 32, O, 4, P, 256, 256, P, 16, O, nullptr),
         MXQ_ERR_SHAPE);
  EXPECT(mx_quantize_colwise(X, 64, HUGE_ / 8 * 8, HUGE_, nullptr, 0, P, 64, 64, P, 16, nullptr,
                             nullptr), MXQ_ERR_ALIGN);
  EXPECT(mx_quantize_colwise(X, 64, HUGE_ / 8 * 8, HUGE_ / 8 * 8, nullptr, 0, P, 64, 64, P, 16,
                             nullptr, nullptr), MXQ_ERR_SHAPE);      // too many column tiles
  EXPECT(mx_quantize_dual(X, 64, 32, 32, O, 4, P, 32, P, 16, P, 160, 160, P, 16, O, nullptr),
         MXQ_ERR_SHAPE);
  EXPECT(mx_quantize_dual(X, 64, 32, 32, O, 4, P, 32, P, 16, P, 192, 192, P, 16, O, nullptr), HIP);
  EXPECT(mx_quantize_dual(X, HUGE_, 32, 32, O, 4, P, 32, P, 16, P, 256, 256, P, 16, O, nullptr),
         MXQ_ERR_SHAPE);
  EXPECT(mx_quantize_dual(X, 64, 32, 32, O, 0, P, 32, P, 16, P, 192, 192, P, 16, O, nullptr),
         MXQ_ERR_SHAPE);
  // ---- dual-axis, several matrices in one launch ----
  {
    const mxq_dual_item good{X, 64, 32, 32, O, 4, P, 32, P, 16, P, 192, 192, P, 16, O};
    const mxq_dual_item small_cap{X, 64, 32, 32, O, 4, P, 32, P, 16, P, 160, 160, P, 16, O};
    const mxq_dual_item no_groups{X, 64, 32, 32, O, 0, P, 32, P, 16, P, 192, 192, P, 16, O};
    const mxq_dual_item odd{X + 1, 64, 32, 32, O, 4, P, 32, P, 16, P, 192, 192, P, 16, O};
    const mxq_dual_item null_qt{X, 64, 32, 32, O, 4, P, 32, P, 16, nullptr, 192, 192, P, 16, O};
    const mxq_dual_item empty{nullptr, 0, 0, 0, nullptr, 0, nullptr, 0, nullptr, 0, nullptr, 0,
                              0, nullptr, 0, nullptr};
    // 2^38 output columns of one K chunk: 2^31 column tiles
    const mxq_dual_item huge{nullptr, 0, 256, 256, nullptr, 0, nullptr, 256, nullptr, 8, P,
                             INT64_C(1) << 38, INT64_C(1) << 38, P, INT64_C(1) << 33, nullptr};
    // 2^30 workgroups each, so two pass 2^31 together
    const mxq_dual_item half{nullptr, 0, 256, 256, nullptr, 0, nullptr, 256, nullptr, 8, P,
                             INT64_C(1) << 37, INT64_C(1) << 37, P, INT64_C(1) << 32, nullptr};
    const mxq_dual_item five[5] = {good, good, good, good, good};
    EXPECT(mx_quantize_dual_batch(five, 0, nullptr), MXQ_ERR_SHAPE);
    EXPECT(mx_quantize_dual_batch(five, 5, nullptr), MXQ_ERR_SHAPE);
    EXPECT(mx_quantize_dual_batch(nullptr, 1, nullptr), MXQ_ERR_NULL);
    const mxq_dual_item a[2] = {good, small_cap}, b2[2] = {odd, good}, c[2] = {empty, empty};
    const mxq_dual_item d[2] = {good, huge}, e[2] = {half, half}, f[3] = {empty, half, good};
    const mxq_dual_item g2[2] = {good, no_groups}, h2[2] = {null_qt, good};
    EXPECT(mx_quantize_dual_batch(a, 2, nullptr), MXQ_ERR_SHAPE);
    EXPECT(mx_quantize_dual_batch(b2, 2, nullptr), MXQ_ERR_ALIGN);
    EXPECT(mx_quantize_dual_batch(c, 2, nullptr), MXQ_OK);      // nothing to launch
    EXPECT(mx_quantize_dual_batch(d, 2, nullptr), MXQ_ERR_SHAPE);
    EXPECT(mx_quantize_dual_batch(e, 2, nullptr), MXQ_ERR_SHAPE);
    EXPECT(mx_quantize_dual_batch(g2, 2, nullptr), MXQ_ERR_SHAPE);
    EXPECT(mx_quantize_dual_batch(h2, 2, nullptr), MXQ_ERR_NULL);
    EXPECT(mx_quantize_dual_batch(f, 3, nullptr), HIP);
    EXPECT(mx_quantize_dual_batch(five, 4, nullptr), HIP);
  }
  // ---- per-tensor and per-group ----
  EXPECT(fp8_quantize_per_tensor(X, -5, P, Fp, P, 4096, nullptr), MXQ_ERR_SHAPE);
  EXPECT(fp8_quantize_per_tensor(X, 100, P, Fp, P, 4, nullptr), MXQ_ERR_WORKSPACE);
  EXPECT(fp8_quantize_per_tensor(X, 100, P, Fp, P, 4096, nullptr), HIP);
  EXPECT(fp8_quantize_per_tensor(X, HUGE_, P, Fp, P, 4096, nullptr), HIP);
  EXPECT(fp8_quantize_per_tensor_amax(X, -5, Fp, P, Fp, nullptr), MXQ_ERR_SHAPE);
  EXPECT(fp8_quantize_per_tensor_amax(X, 100, nullptr, P, Fp, nullptr), MXQ_ERR_NULL);
  EXPECT(fp8_quantize_per_tensor_amax(X, 100, Fp, P, nullptr, nullptr), MXQ_ERR_NULL);
  EXPECT(fp8_quantize_per_tensor_amax(nullptr, 100, Fp, P, Fp, nullptr), MXQ_ERR_NULL);
  EXPECT(fp8_quantize_per_tensor_amax(X + 1, 100, Fp, P, Fp, nullptr), MXQ_ERR_ALIGN);
  EXPECT(fp8_quantize_per_tensor_amax(nullptr, 0, Fp, nullptr, Fp, nullptr), HIP);
  EXPECT(fp8_quantize_per_tensor_amax(X, 100, Fp, P, Fp, nullptr), HIP);
  EXPECT(fp8_quantize_per_tensor_amax(X, HUGE_, Fp, P, Fp, nullptr), HIP);
  const size_t ws = mxq_workspace_size(MXQ_WS_PER_GROUP, 64, 4, 0, 0);
  EXPECT((int)(ws == (64 + 4) * 4), 1);
  EXPECT((int)(mxq_workspace_size(MXQ_WS_PER_GROUP, -1, 4, 0, 0) == 0), 1);
  EXPECT((int)(mxq_workspace_size(MXQ_WS_PER_TENSOR, 0, 0, 0, 0) == 0), 1);
  EXPECT(fp8_quantize_per_group(X, 64, 32, 32, O, 4, P, 32, Fp, P, ws, nullptr), HIP);
  EXPECT(fp8_quantize_per_group(X, 64, 32, 32, O, 4, P, 32, Fp, P, ws - 4, nullptr),
         MXQ_ERR_WORKSPACE);
  EXPECT(fp8_quantize_per_group(X, HUGE_, 32, 32, O, 4, P, 32, Fp, P, ws, nullptr),
         MXQ_ERR_WORKSPACE);
  EXPECT(fp8_quantize_per_group_noalloc(X, 262144, 32, 32, O, 1, P, 32, Fp, nullptr),
         MXQ_ERR_SHAPE);
  EXPECT(fp8_quantize_per_group_noalloc(X, HUGE_, 32, 32, O, 1, P, 32, Fp, nullptr),
         MXQ_ERR_SHAPE);
  EXPECT(fp8_quantize_per_group_noalloc(X, 64, 32, 32, nullptr, 4, P, 32, Fp, nullptr),
         MXQ_ERR_NULL);
  EXPECT(fp8_quantize_per_group_noalloc(X, 64, 32, 32, O, 4, P, 32, Fp, nullptr), HIP);
  EXPECT(fp8_quantize_per_group_colwise(X, 64, 32, 32, O, 4, P, 160, 160, Fp, O, P, ws, nullptr),
         MXQ_ERR_SHAPE);
  EXPECT(fp8_quantize_per_group_colwise(X, 64, 32, 32, O, 4, P, 192, 192, Fp, O, P, ws, nullptr),
         HIP);
  EXPECT(fp8_quantize_per_group_dual(X, 64, 32, 32, O, 4, nullptr, P, 32, P, 160, 160, Fp, O, P,
                                     ws, nullptr), MXQ_ERR_SHAPE);
  EXPECT(fp8_quantize_per_group_dual(X, HUGE_, 32, 32, O, 4, nullptr, P, 32, P, 256, 256, Fp, O,
                                     P, ws, nullptr), MXQ_ERR_SHAPE);
  // ---- blockwise ----
  EXPECT(fp8_quantize_blockwise_act(X, 8, 96, 96, P, 96, Fp, 1, nullptr), MXQ_ERR_SHAPE);
  EXPECT(fp8_quantize_blockwise_act(X, 8, 128, 128, P, 128, Fp, 1, nullptr), HIP);
  EXPECT(fp8_quantize_blockwise_act(X, HUGE_, 128, 128, P, 128, Fp, 1, nullptr), MXQ_ERR_SHAPE);
  EXPECT(fp8_quantize_blockwise_weight(X, 200, 256, 256, P, 256, Fp, 1, nullptr), MXQ_ERR_SHAPE);
  EXPECT(fp8_quantize_blockwise_weight(X, HUGE_, 256, 256, P, 256, Fp, 2, nullptr), MXQ_ERR_SHAPE);
  // ---- GEMMs ----
  for (int acc = 0; acc < 2; ++acc) {
    EXPECT(mx_gemm(P, P, 32, 1, P, P, 32, 1, 4, 4, 33, P, 4, 0, acc, nullptr), MXQ_ERR_SHAPE);
    EXPECT(mx_gemm(P, P, 32, 1, P, P, 32, 1, 4, 4, 32, P, 4, 0, acc, nullptr), HIP);
    EXPECT(mx_gemm(P, P, 32, 1, P, P, 32, 1, HUGE_, HUGE_, 32, P, HUGE_, 0, acc, nullptr),
           MXQ_ERR_SHAPE);
    EXPECT(mx_gemm(P, P, HUGE_ / 32 * 32, HUGE_, P, P, HUGE_ / 32 * 32, HUGE_, 4, 4,
                   HUGE_ / 32 * 32, P, 4, 0, acc, nullptr), MXQ_ERR_SHAPE);
    EXPECT(fp8_gemm_per_tensor(P, Fp, 32, P, Fp, 32, 4, 4, 32, P, 4, 1, acc, nullptr), HIP);
    EXPECT(fp8_gemm_per_tensor_amax(P, Fp, 32, P, Fp, 32, 4, 4, 32, P, 4, 1, acc, nullptr,
                                    nullptr), MXQ_ERR_NULL);
    EXPECT(fp8_gemm_per_tensor_amax(P, Fp, 32, P, Fp, 32, 4, 4, 32, P, 4, 1, acc,
                                    reinterpret_cast<float*>(P + 2), nullptr), MXQ_ERR_ALIGN);
    EXPECT(fp8_gemm_per_tensor_amax(P, Fp, 32, P, Fp, 32, 4, 4, 33, P, 4, 1, acc, Fp, nullptr),
           MXQ_ERR_SHAPE);
    EXPECT(fp8_gemm_per_tensor_amax(P, Fp, 32, P, Fp, 32, 0, 4, 32, P, 4, 1, acc, Fp, nullptr),
           HIP);                                              // clears the amax: a launch
    EXPECT(fp8_gemm_per_tensor_amax(P, Fp, 32, P, Fp, 32, 4, 4, 32, P, 4, 1, acc, Fp, nullptr),
           HIP);
    EXPECT(fp8_gemm_per_tensor(P, Fp, 32, P, Fp, 32, HUGE_, HUGE_, 32, P, HUGE_, 1, acc, nullptr),
           MXQ_ERR_SHAPE);
    EXPECT(mx_grouped_gemm(P, P, 32, 1, P, P, 32, 1, 256, 8, O, 4, 8, 8, 32, P, 8, 0, acc, nullptr),
           HIP);
    EXPECT(mx_grouped_gemm(P, P, 32, 1, P, P, 32, 1, 256, 8, O, 4, HUGE_, 8, 32, P, 8, 0, acc,
                           nullptr), MXQ_ERR_SHAPE);
    EXPECT(mx_grouped_gemm(P, P, 32, 1, P, P, 32, 1, HUGE_ / 16 * 16, HUGE_, O, 4, 8, 8, 32, P, 8,
                           0, acc, nullptr), HIP);
    EXPECT(mx_grouped_gemm_wgrad(P, P, 32, 1, P, P, 32, 1, O, 2, 8, 8, P, 8, 0, acc, nullptr), HIP);
    EXPECT(mx_grouped_gemm_wgrad(P, P, 32, 1, P, P, 32, 1, O, 256, HUGE_, HUGE_, P, HUGE_, 0, acc,
                                 nullptr), MXQ_ERR_SHAPE);
    EXPECT(fp8_grouped_gemm_per_group(P, Fp, 32, P, Fp, 32, 256, O, 4, 8, 8, 32, P, 8, 0, acc,
                                      nullptr), HIP);
    EXPECT(fp8_grouped_gemm_wgrad_per_group(P, Fp, 32, P, Fp, 32, O, 2, 8, 8, P, 8, 0, acc,
                                            nullptr), HIP);
    EXPECT(fp8_grouped_gemm_wgrad_per_group(P, Fp, 32, P, Fp, 32, O, 2, HUGE_, HUGE_, P, HUGE_, 0,
                                            acc, nullptr), MXQ_ERR_SHAPE);
  }
  EXPECT(mx_gemm(P, P, 32, 1, P, P, 32, 1, 4, 4, 32, P, 4, 0, 7, nullptr), MXQ_ERR_ARG);
  EXPECT(fp8_gemm_blockwise(P, Fp, 128, 1, P, Fp, 128, 1, 4, 4, 128, P, 4, 0, 1, nullptr),
         MXQ_ERR_ARG);
  EXPECT(fp8_gemm_blockwise(P, Fp, 128, 1, P, Fp, 128, 1, 4, 4, 128, P, 4, 0, 0, nullptr), HIP);
  EXPECT(fp8_gemm_blockwise(P, Fp, 128, 1, P, Fp, 128, 1, HUGE_, HUGE_, 128, P, HUGE_, 0, 0,
                            nullptr), MXQ_ERR_SHAPE);
  // ---- fused producers ----
  EXPECT(mx_grouped_gemm_swiglu(P, P, 32, 16, P, P, 32, 16, 4096, 2048, O, 4, 64, 64, 32, P, 128,
                                P, 64, P, 16, P, 256, P, 16, 256, O, nullptr), HIP);
  EXPECT(mx_grouped_gemm_swiglu(P, P, 32, 16, P, P, 32, 16, 4096, 2048, O, 4, 64, 64, 32, P, 128,
                                P, 64, P, 16, P, 160, P, 16, 160, O, nullptr), MXQ_ERR_SHAPE);
  EXPECT(mx_grouped_gemm_swiglu(P, P, 32, 16, P, P, 32, 16, 4096, 2048, O, 4, HUGE_, 64, 32, P,
                                128, P, 64, P, 16, P, 256, P, 16, 256, O, nullptr), MXQ_ERR_SHAPE);
  EXPECT(fp8_grouped_gemm_per_group_swiglu(P, Fp, 32, P, Fp, 32, 4096, O, 4, 64, 64, 32, P, 128,
                                           X, 64, Fp, nullptr), HIP);
  EXPECT(fp8_grouped_gemm_per_group_swiglu(P, Fp, 32, P, Fp, 32, 4096, O, 4, HUGE_, 64, 32, P,
                                           128, X, 64, Fp, nullptr), MXQ_ERR_SHAPE);
  // ---- helpers ----
  EXPECT(mxq_validate_offsets(nullptr, 4, 10, nullptr), MXQ_ERR_NULL);
  EXPECT(mxq_validate_offsets(O, 4, 10, nullptr), HIP);
  EXPECT((int)(std::strcmp(mxq_status_string(MXQ_ERR_HIP), "HIP runtime error") == 0), 1);
  std::printf("%d cases, %d failed\n", g_n, g_fail);
  return g_fail ? 1 : 0;
}
