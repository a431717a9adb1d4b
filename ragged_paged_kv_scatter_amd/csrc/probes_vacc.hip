// rpa_probe_mix with the MFMA accumulators in VGPRs (include/rpa_probes.h):
// this file is compiled with -mllvm --amdgpu-mfma-vgpr-form (see build.py),
// the form the attention kernels' MFMAs take because their VALU code reads
// the accumulators.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rpa_probes.h"

namespace {

constexpr int kT = 256;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#include "probes_mix.h"

}  // namespace

extern "C" int rpa_probe_mix_vgpr_acc(float* sink, int64_t* clocks, int nv, int exp, int iters,
                                      int blocks, void* stream) {
  return launch_mix(sink, clocks, nv, exp, iters, blocks, stream);
}
