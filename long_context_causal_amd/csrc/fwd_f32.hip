// fwd_f32.hip -- the fp32 forward kernel and its launcher.
#include "fwd_f32.hpp"
#include "launch.hpp"

namespace gqa {

static_assert(kRowsF32 == kRowsPerWave, "host plan and kernel disagree on rows per wave");
static_assert(kTileKeysF32 == kBkF, "host plan and kernel disagree on the key tile");

hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t stream) {
  const unsigned splits = p.n_split > 1 ? (unsigned)p.n_split : 1u;
  hipLaunchKernelGGL(fwd_f32_kernel<kWavesF32>, dim3((unsigned)p.n_qb * (unsigned)p.G * splits), dim3(kWavesF32 * 64), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace gqa
