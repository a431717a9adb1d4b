// Stand-ins for the kernel launchers of librpa.so, for the host-only
// sanitizer build of the C ABI's host code (rpa_api.cpp): each reports its
// launch to the trace hooks like the real launcher and launches nothing.
// Together with host_checks.cpp this exercises argument validation,
// workspace layout, tracing and error strings under ASan / UBSan on a machine
// with no GPU.
#include "rpa_internal.h"

namespace rpa {

namespace {
hipError_t stub(const char* name, unsigned grid, unsigned block, hipStream_t s) {
  if (trace_active()) (void)trace_launch(name, grid, block, 0, s);
  return hipSuccess;
}
}  // namespace

bool prefill_supported(const rpa_desc& d) {
  return d.q_dtype == RPA_BF16 && (d.cache_dtype == RPA_BF16 || d.cache_dtype == RPA_FP8_E4M3) &&
         (d.head_dim == 64 || d.head_dim == 128);
}
int row_waves(rpa_dtype, rpa_dtype, int, int, int, int, bool) { return 2048; }
hipError_t launch_scatter(const ScatterParams& p, rpa_dtype, rpa_dtype, hipStream_t s) {
  return stub("scatter_kernel", (unsigned)p.T, 256, s);
}
hipError_t launch_prep(const PlanParams& pp, const ScatterParams* sp, rpa_dtype, rpa_dtype,
                       hipStream_t s) {
  return stub(sp ? "prep_kernel(plan+scatter)" : "prep_kernel(plan)", 1 + (sp ? sp->T : 0),
              kPlanThreads, s);
}
hipError_t launch_rows(const AttnParams& p, rpa_dtype, rpa_dtype, hipStream_t s) {
  return stub("row_kernel", (unsigned)p.lay.max_chunks, 256, s);
}
hipError_t launch_merge(const AttnParams& p, rpa_dtype, hipStream_t s) {
  return stub("merge_kernel", (unsigned)p.lay.max_merge_rows, 256, s);
}
hipError_t launch_prefill(const AttnParams& p, rpa_dtype, rpa_dtype, hipStream_t s) {
  return stub("prefill_kernel", (unsigned)p.lay.max_pf_items, 256, s);
}
hipError_t launch_slot_mapping(const SlotMapParams& p, hipStream_t s) {
  return stub("slot_mapping_kernel", (unsigned)p.T, 256, s);
}
hipError_t launch_validate(const ValidateParams&, hipStream_t s) {
  return stub("validate", 1, 256, s);
}
hipError_t launch_copy_blocks(const CopyBlocksParams& p, hipStream_t s) {
  return stub("copy_blocks_kernel", (unsigned)p.num_pairs, 256, s);
}
hipError_t launch_reshape_and_cache(const ReshapeParams& p, rpa_dtype, rpa_dtype, hipStream_t s) {
  return stub("reshape_cache_kernel", (unsigned)p.T, 256, s);
}

}  // namespace rpa
