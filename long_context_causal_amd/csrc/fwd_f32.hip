// fwd_f32.hip -- the fp32 forward kernel and its launcher.
#include "fwd_f32.hpp"
#include "launch.hpp"

namespace gqa {

static_assert(kRowsF32 == kRowsPerWave, "host plan and kernel disagree on rows per wave");

hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(fwd_f32_kernel<kWavesF32>, dim3((unsigned)p.n_qb * (unsigned)p.G), dim3(kWavesF32 * 64), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace gqa
