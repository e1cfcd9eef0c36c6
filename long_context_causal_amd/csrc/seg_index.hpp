// seg_index.hpp -- the id-range index of a segment-id array: for each block of
// kSegBlk consecutive ids of a batch row, their minimum and maximum. The
// forward and backward kernels classify their tiles from it instead of from
// the ids (one eighth of the bytes per workgroup), so a caller whose ids stay
// the same over many calls (every layer of one packed batch) reads the ids
// once.
#pragma once
#include "common.hpp"

namespace gqa {

// One thread per entry of idx[B][nblk]; entry j of row b covers ids
// [16 j, min(16 j + 16, L)) of that row.
__global__ __launch_bounds__(256) void seg_index_kernel(const int32_t* seg, int64_t L, int64_t nblk, int64_t total,
                                                        SegBlk* idx) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int64_t b = i / nblk, j = i - b * nblk;
  const int32_t* row = seg + b * L + j * kSegBlk;
  const int n = (int)min((int64_t)kSegBlk, L - j * kSegBlk);
  int lo = row[0], hi = row[0];
  if (n == kSegBlk) {
#pragma unroll
    for (int x = 1; x < kSegBlk; ++x) {
      lo = min(lo, row[x]);
      hi = max(hi, row[x]);
    }
  } else {
    for (int x = 1; x < n; ++x) {
      lo = min(lo, row[x]);
      hi = max(hi, row[x]);
    }
  }
  idx[i] = SegBlk{lo, hi};
}

}  // namespace gqa
