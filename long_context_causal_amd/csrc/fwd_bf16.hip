// fwd_bf16.hip -- the bf16 forward kernel and its launcher.
#include "fwd_bf16.hpp"
#include "launch.hpp"

namespace gqa {

static_assert(kWavesBf16 == kWavesB && kRowsBf16 == kRowsB, "host plan and kernel disagree on the workgroup shape");

hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)p.n_qb * (unsigned)p.G), block(kWavesB * 64);
  if (p.seg_q != nullptr)
    hipLaunchKernelGGL(fwd_bf16_kernel<true>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(fwd_bf16_kernel<false>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace gqa
