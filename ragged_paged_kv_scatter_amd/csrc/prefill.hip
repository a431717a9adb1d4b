// Prefill / mixed-chunk kernel (MFMA).  Placeholder until the MFMA tile kernel
// lands: every sequence is served by the row kernel.
#include "rpa_internal.h"

namespace rpa {

bool prefill_supported(const rpa_desc&) { return false; }

hipError_t launch_prefill(const AttnParams&, rpa_dtype, rpa_dtype, hipStream_t) {
  return hipSuccess;
}

}  // namespace rpa
