// fwd_h16.hip -- the 16-bit-input (bf16, fp16) forward kernels and their launchers.
#include "fwd_h16.hpp"
#include "launch.hpp"

namespace gqa {

static_assert(kWavesH16 == kWavesB && kRowsH16 == kRowsB, "host plan and kernel disagree on the workgroup shape");
static_assert(kTileKeysH16 == kBkB, "host plan and kernel disagree on the key tile");

template <typename E>
static hipError_t launch_h16(const FwdParams& p, hipStream_t stream) {
  const unsigned splits = p.n_split > 1 ? (unsigned)p.n_split : 1u;
  const dim3 grid((unsigned)p.n_qb * (unsigned)p.G * splits), block(kWavesB * 64);
  if (p.seg_q != nullptr)
    hipLaunchKernelGGL((fwd_h16_kernel<E, true>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((fwd_h16_kernel<E, false>), grid, block, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t stream) { return launch_h16<__bf16>(p, stream); }
hipError_t launch_fwd_f16(const FwdParams& p, hipStream_t stream) { return launch_h16<_Float16>(p, stream); }

}  // namespace gqa
