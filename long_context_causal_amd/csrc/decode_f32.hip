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
  // packed rows per KV head: at most 16 or 32 (then p.n_qb = ceil(R / 64) = 1,
  // the one block of 16 or 32 rows) take 4 or 2 parts of d
  const int64_t R = (int64_t)p.n_rep * p.Lq;
  if (R <= kDecFRows)
    hipLaunchKernelGGL(decode_f32_kernel<4>, grid, block, 0, stream, p);
  else if (R <= 2 * kDecFRows)
    hipLaunchKernelGGL(decode_f32_kernel<2>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(decode_f32_kernel<1>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace gqa
