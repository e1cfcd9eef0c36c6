// bwd_h16.hip -- the 16-bit-input (bf16, fp16) backward kernels and their launchers.
#include "bwd_h16.hpp"
#include "launch.hpp"

namespace gqa {

static_assert(kBwdWavesDQH == kWavesH && kBwdRowsDQH == kRowsDQH && kBwdKeysDKVH == kKeysBlockDKVH,
              "host plan and kernels disagree on the 16-bit backward work shapes");

template <typename E>
static hipError_t launch_bwd_h16(const BwdParams& p, hipStream_t stream) {
  const dim3 block(kWavesH * 64);
  const dim3 gq((unsigned)p.f.n_qb * (unsigned)p.f.G), gk((unsigned)p.n_kb * (unsigned)p.BH);
  if (p.f.seg_q != nullptr) hipLaunchKernelGGL((bwd_dq_h16_kernel<E, true>), gq, block, 0, stream, p);
  else hipLaunchKernelGGL((bwd_dq_h16_kernel<E, false>), gq, block, 0, stream, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.f.seg_q != nullptr) hipLaunchKernelGGL((bwd_dkv_h16_kernel<E, true>), gk, block, 0, stream, p);
  else hipLaunchKernelGGL((bwd_dkv_h16_kernel<E, false>), gk, block, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t stream) { return launch_bwd_h16<__bf16>(p, stream); }
hipError_t launch_bwd_f16(const BwdParams& p, hipStream_t stream) { return launch_bwd_h16<_Float16>(p, stream); }

}  // namespace gqa
