// decode_h16.hip -- the short-query-block (decoding) forward kernels for
// 16-bit inputs and their launchers.
#include "decode_h16.hpp"
#include "launch.hpp"

namespace gqa {

static_assert(kDecodeBlockRows == kDecBlockRows, "host plan and kernel disagree on the row block");
static_assert(kTileKeysDec == kDecBk, "host plan and kernel disagree on the key tile");

template <typename E>
static hipError_t launch_dec(const FwdParams& p, hipStream_t stream) {
  const unsigned splits = p.n_split > 1 ? (unsigned)p.n_split : 1u;
  const dim3 grid(splits * (unsigned)p.n_qb * (unsigned)p.G), block(kDecWaves * 64);
  hipLaunchKernelGGL((decode_h16_kernel<E>), grid, block, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_decode_bf16(const FwdParams& p, hipStream_t stream) { return launch_dec<__bf16>(p, stream); }
hipError_t launch_decode_f16(const FwdParams& p, hipStream_t stream) { return launch_dec<_Float16>(p, stream); }

}  // namespace gqa
