// Host-side helpers of the libmxq C ABI: status strings, version, and the
// debug validator for device-side group offsets.

#include <vector>

#include "mxq.h"

extern "C" const char* mxq_status_string(int status) {
  switch (status) {
    case MXQ_OK: return "ok";
    case MXQ_ERR_NULL: return "null pointer";
    case MXQ_ERR_SHAPE: return "bad shape or size";
    case MXQ_ERR_ALIGN: return "misaligned pointer or leading dimension";
    case MXQ_ERR_ARG: return "bad enum argument";
    case MXQ_ERR_WORKSPACE: return "workspace too small";
    case MXQ_ERR_HIP: return "HIP runtime error";
    case MXQ_ERR_OFFSETS: return "invalid group offsets";
    default: return "unknown status";
  }
}

extern "C" int mxq_version(void) { return 1 * 10000 + 0 * 100 + 0; }

extern "C" int mxq_validate_offsets(const int64_t* offsets, int32_t E, int64_t M,
                                    hipStream_t stream) {
  if (!offsets) return MXQ_ERR_NULL;
  if (E < 1 || M < 0) return MXQ_ERR_SHAPE;
  std::vector<int64_t> h((size_t)E + 1);
  if (hipMemcpyAsync(h.data(), offsets, h.size() * sizeof(int64_t), hipMemcpyDeviceToHost,
                     stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return MXQ_ERR_HIP;
  if (h[0] != 0 || h[E] != M) return MXQ_ERR_OFFSETS;
  for (int32_t e = 0; e < E; ++e)
    if (h[e + 1] < h[e]) return MXQ_ERR_OFFSETS;
  return MXQ_OK;
}
