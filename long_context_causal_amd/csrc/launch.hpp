// launch.hpp -- launchers of the forward and backward kernels, each defined in
// the translation unit of its kernel (fwd_f32.hip, fwd_h16.hip, bwd_f32.hip,
// bwd_h16.hip)
// so that each kernel is compiled with its own code-generation flags.
#pragma once
#include <hip/hip_runtime.h>

#include "common.hpp"

namespace gqa {

// Workgroup shapes the host plan needs: waves per workgroup and query rows per wave.
constexpr int kWavesF32 = 4, kRowsF32 = 32;
constexpr int kWavesH16 = 4, kRowsH16 = 32;  // bf16 and fp16
// Keys per tile of the forward kernels (the unit of a split-KV range).
constexpr int kTileKeysF32 = 32, kTileKeysH16 = 64;

// Enqueue one forward launch (grid = p.n_qb * p.G workgroups, times p.n_split
// for a split-KV launch); returns hipGetLastError() after the launch.
hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t stream);
hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t stream);
hipError_t launch_fwd_f16(const FwdParams& p, hipStream_t stream);

// Short query blocks (decoding) with no segment ids: query positions below
// which a decode kernel serves a launch, its packed rows per workgroup and keys
// per tile (the unit of its split-KV ranges: 32 for 16-bit inputs, 16 for
// fp32). Grid: n_split x p.n_qb row blocks x p.G (= B * Hkv); p.n_qb =
// ceil(n_rep Lq / 64).
constexpr int kDecodeMaxLq = 32, kDecodeBlockRows = 64, kTileKeysDec = 32, kTileKeysDecF32 = 16;
hipError_t launch_decode_bf16(const FwdParams& p, hipStream_t stream);
hipError_t launch_decode_f16(const FwdParams& p, hipStream_t stream);
hipError_t launch_decode_f32(const FwdParams& p, hipStream_t stream);

// Backward: waves per workgroup and query rows per wave of the dQ kernel, keys
// per workgroup of the dK/dV kernel (host plan).
constexpr int kBwdWavesDQ = 8, kBwdRowsDQ = 16, kBwdKeysDKV = 64;

// Enqueue the dQ kernel (grid p.f.n_qb * p.f.G) then the dK/dV kernel (grid
// p.n_kb * p.BH) on `stream`; returns the first launch error.
hipError_t launch_bwd_f32(const BwdParams& p, hipStream_t stream);

// 16-bit backward: 4 waves x 32 query rows (dQ kernel), 128 keys per dK/dV workgroup.
constexpr int kBwdWavesDQH = 4, kBwdRowsDQH = 32, kBwdKeysDKVH = 128;
hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t stream);
hipError_t launch_bwd_f16(const BwdParams& p, hipStream_t stream);

}  // namespace gqa
