// decode_f32.hip -- the short-query-block (decoding) forward kernel for fp32
// inputs and its launcher.
#include "decode_f32.hpp"
#include "launch.hpp"

namespace gqa {

static_assert(kDecodeBlockRows == kDecFBlockRows, "host plan and kernel disagree on the row block");
static_assert(kTileKeysDecF32 == kDecFBk, "host plan and kernel disagree on the key tile");

hipError_t launch_decode_f32(const FwdParams& p, hipStream_t stream) {
  const unsigned splits = p.n_split > 1 ? (unsigned)p.n_split : 1u;
  const dim3 grid(splits * (unsigned)p.n_qb * (unsigned)p.G), block(kDecFWaves * 64);
  // at most 16 packed rows per KV head (then p.n_qb = 1): the 4 waves split d
  if ((int64_t)p.n_rep * p.Lq <= kDecFRows)
    hipLaunchKernelGGL(decode_f32_kernel<true>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(decode_f32_kernel<false>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace gqa
