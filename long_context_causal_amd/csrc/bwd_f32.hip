// bwd_f32.hip -- the fp32 backward kernels and their launcher.
#include "bwd_f32.hpp"
#include "launch.hpp"

namespace gqa {

static_assert(kBwdWavesDQ == kWavesDQ && kBwdRowsDQ == kRowsDQ && kBwdKeysDKV == kKeysBlockDKV,
              "host plan and kernels disagree on the backward work shapes");

hipError_t launch_bwd_f32(const BwdParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(bwd_dq_f32_kernel, dim3((unsigned)p.f.n_qb * (unsigned)p.f.G), dim3(kWavesDQ * 64), 0, stream,
                     p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_dkv_f32_kernel, dim3((unsigned)p.n_kb * (unsigned)p.BH), dim3(kWavesDKV * 64), 0, stream,
                     p);
  return hipGetLastError();
}

}  // namespace gqa
