// Stand-alone paged KV-cache update (rpa_update_kv_cache); rpa_forward runs
// the same code inside its planning launch.
#include <algorithm>

#include "scatter.h"

namespace rpa {
namespace {

constexpr int kThreads = 256;
constexpr int kTargetWGs = 1024;      // spread small batches over the chip

template <typename IN, typename C>
__global__ __launch_bounds__(kThreads) void scatter_kernel(ScatterParams p, int tpw) {
  scatter_body<IN, C, kThreads>(p, tpw, blockIdx.x);
}

}  // namespace

hipError_t launch_scatter(const ScatterParams& p, rpa_dtype in_dt, rpa_dtype cache_dt,
                          hipStream_t s) {
  if (p.T <= 0) return hipSuccess;
  const int tpw = std::min(8, std::max(1, (p.T + kTargetWGs - 1) / kTargetWGs));
  dim3 grid((p.T + tpw - 1) / tpw), block(kThreads);
  if (trace_active() && trace_launch("scatter_kernel", grid.x, kThreads, 0, s)) return hipSuccess;
  if (in_dt == RPA_F32 && cache_dt == RPA_F32) {
    scatter_kernel<float, float><<<grid, block, 0, s>>>(p, tpw);
  } else if (in_dt == RPA_BF16 && cache_dt == RPA_BF16) {
    scatter_kernel<uint16_t, uint16_t><<<grid, block, 0, s>>>(p, tpw);
  } else if (in_dt == RPA_BF16 && cache_dt == RPA_FP8_E4M3) {
    scatter_kernel<uint16_t, uint8_t><<<grid, block, 0, s>>>(p, tpw);
  } else if (in_dt == RPA_FP8_E4M3 && cache_dt == RPA_FP8_E4M3) {
    scatter_kernel<uint8_t, uint8_t><<<grid, block, 0, s>>>(p, tpw);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rpa
