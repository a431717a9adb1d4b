// The first launch of rpa_forward: workgroup 0 plans the attention kernels
// (plan.h) while the other workgroups, when the call brings new K/V tokens,
// write them into the paged cache (scatter.h).  The two parts touch disjoint
// memory and neither reads the other's output, so one launch serves both.
#include <algorithm>
#include <cstdio>

#include "plan.h"
#include "scatter.h"

namespace rpa {
namespace {

template <typename IN, typename C>
__global__ __launch_bounds__(kPlanThreads) void prep_kernel(PlanParams pp, ScatterParams sp,
                                                            int tpw) {
  extern __shared__ int32_t s_seq_rows[];           // planner tables (plan_lds_words)
  if (blockIdx.x == 0) plan_body(pp, s_seq_rows);
  else scatter_body<IN, C, kPlanThreads>(sp, tpw, blockIdx.x - 1);
}

constexpr int kTargetScatterWGs = 256;

}  // namespace

hipError_t launch_prep(const PlanParams& pp, const ScatterParams* sp, rpa_dtype in_dt,
                       rpa_dtype cache_dt, hipStream_t s) {
  const size_t lds = (size_t)plan_lds_words(pp.max_num_seqs) * sizeof(int32_t);
  ScatterParams p = {};
  int tpw = 1;
  unsigned grid = 1;
  if (sp && sp->T > 0) {
    p = *sp;
    tpw = std::min(kScatterRowsMax,
                   std::max(1, (p.T + kTargetScatterWGs - 1) / kTargetScatterWGs));
    grid = 1u + (unsigned)((p.T + tpw - 1) / tpw);
  } else {
    in_dt = cache_dt = RPA_BF16;                    // planner only
  }
  if (trace_active()) {
    char nm[96];
    std::snprintf(nm, sizeof nm, "prep_kernel<%s,%s>(plan%s, rows_per_wg=%d)",
                  in_dt == RPA_F32 ? "f32" : in_dt == RPA_BF16 ? "bf16" : "fp8",
                  cache_dt == RPA_F32 ? "f32" : cache_dt == RPA_BF16 ? "bf16" : "fp8",
                  grid > 1 ? "+scatter" : "", tpw);
    if (trace_launch(nm, grid, kPlanThreads, lds, s)) return hipSuccess;
  }
  if (in_dt == RPA_F32 && cache_dt == RPA_F32) {
    prep_kernel<float, float><<<grid, kPlanThreads, lds, s>>>(pp, p, tpw);
  } else if (in_dt == RPA_BF16 && cache_dt == RPA_BF16) {
    prep_kernel<uint16_t, uint16_t><<<grid, kPlanThreads, lds, s>>>(pp, p, tpw);
  } else if (in_dt == RPA_BF16 && cache_dt == RPA_FP8_E4M3) {
    prep_kernel<uint16_t, uint8_t><<<grid, kPlanThreads, lds, s>>>(pp, p, tpw);
  } else if (in_dt == RPA_FP8_E4M3 && cache_dt == RPA_FP8_E4M3) {
    prep_kernel<uint8_t, uint8_t><<<grid, kPlanThreads, lds, s>>>(pp, p, tpw);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rpa
