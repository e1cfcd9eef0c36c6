// gqa_attn.hip -- host side of libgqa_attn.so: argument checks, launch plan
// and kernel launches behind the C ABI declared in include/gqa_attn.h.
#include "gqa_attn.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "common.hpp"
#include "launch.hpp"
#include "merge.hpp"
#include "seg_index.hpp"

namespace {

bool misaligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) != 0; }

// [lo, lo + n) and [lo2, lo2 + n2) overlap?
bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

// Query heads per key/value head the library takes (any count from 1 to this).
constexpr int64_t kMaxRep = 64;

// Query heads of one group that a workgroup's waves share out: the largest of
// W, W / 2, ... that divides n_rep (W = 4: 4, 2 or 1), so that the waves split
// evenly into heads x position blocks and the group into whole head chunks.
int64_t heads_per_workgroup(int64_t n_rep, int64_t W) {
  int64_t h = W;
  while (n_rep % h != 0) h >>= 1;
  return h;
}

// Launches the short-block (decode) kernels serve, for every input type: no
// segment ids, fewer than 32 query positions, and key counts whose tile ends
// stay below 2^31 (their tile arithmetic is 32-bit).
bool decode_shape(int64_t Lq, int64_t Lk, bool seg) {
  return !seg && Lq < gqa::kDecodeMaxLq && Lk < ((int64_t)1 << 31) - 64;
}

// Keys per tile of the decode kernel of an input type.
int64_t decode_tile_keys(int dtype) { return dtype == GQA_F32 ? gqa::kTileKeysDecF32 : gqa::kTileKeysDec; }

// split-KV: the most splits one launch takes, and the workgroup count the
// recommended split count aims at: one per compute unit (the forward kernels'
// LDS use admits one workgroup per CU; measured on 16 decode rows over 60,926
// keys, 64 splits = 256 workgroups ran in 51 us against 63 us for 128)
constexpr int kMaxSplits = 1024;
constexpr int64_t kSplitTargetWorkgroups = 256;

}  // namespace

// The library is built with hidden visibility; these are its only exports.
#define GQA_API extern "C" __attribute__((visibility("default")))

// Argument checks and launch plan shared by the forward entry points.
static int fwd_plan(gqa::FwdParams& p, const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                    int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D, int64_t q_offset,
                    const int32_t* seg_q, const int32_t* seg_k, int causal, int dtype) {
  if (!q || !k || !v || !o || !lse) return GQA_ERR_NULL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Lq <= 0 || Lk <= 0 || D <= 0) return GQA_ERR_SHAPE;
  if (Hq % Hkv != 0 || q_offset < 0 || q_offset > ((int64_t)1 << 62)) return GQA_ERR_SHAPE;
  if ((seg_q == nullptr) != (seg_k == nullptr)) return GQA_ERR_SHAPE;
  if (D != gqa::kD || (dtype != GQA_F32 && dtype != GQA_BF16 && dtype != GQA_F16)) return GQA_ERR_UNSUPPORTED;
  const int64_t n_rep = Hq / Hkv;
  if (n_rep > kMaxRep || Lq >= ((int64_t)1 << 31) || Lk >= ((int64_t)1 << 31) || B * Hkv >= ((int64_t)1 << 24))
    return GQA_ERR_UNSUPPORTED;
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16) || misaligned(lse, 4) ||
      misaligned(seg_q, 4) || misaligned(seg_k, 4))
    return GQA_ERR_ALIGN;
  const int64_t es = dtype == GQA_F32 ? 4 : 2;
  const int64_t qo_bytes = B * Hq * Lq * D * es, kv_bytes = B * Hkv * Lk * D * es, lse_bytes = B * Hq * Lq * 4;
  if (overlap(o, qo_bytes, q, qo_bytes) || overlap(o, qo_bytes, k, kv_bytes) || overlap(o, qo_bytes, v, kv_bytes) ||
      overlap(lse, lse_bytes, o, qo_bytes) || overlap(lse, lse_bytes, q, qo_bytes) ||
      overlap(lse, lse_bytes, k, kv_bytes) || overlap(lse, lse_bytes, v, kv_bytes))
    return GQA_ERR_ALIAS;
  // every workgroup reads the ids while earlier ones already write o and lse
  if (seg_q && (overlap(o, qo_bytes, seg_q, B * Lq * 4) || overlap(o, qo_bytes, seg_k, B * Lk * 4) ||
                overlap(lse, lse_bytes, seg_q, B * Lq * 4) || overlap(lse, lse_bytes, seg_k, B * Lk * 4)))
    return GQA_ERR_ALIAS;

  const int W = dtype == GQA_F32 ? gqa::kWavesF32 : gqa::kWavesH16;
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.seg_q = seg_q; p.seg_k = seg_k;
  p.Lq = Lq; p.Lk = Lk; p.q_offset = q_offset;
  p.Hq = (int)Hq; p.Hkv = (int)Hkv; p.n_rep = (int)n_rep;
  p.hpc = (int)heads_per_workgroup(n_rep, W);
  p.ppc = (W / p.hpc) * (dtype == GQA_F32 ? gqa::kRowsF32 : gqa::kRowsH16);
  const int64_t n_qb = (Lq + p.ppc - 1) / p.ppc;
  const int64_t G = B * Hkv * (n_rep / p.hpc);
  if (n_qb * G >= ((int64_t)1 << 31)) return GQA_ERR_UNSUPPORTED;
  p.n_qb = (int)n_qb;
  p.G = (int)G;
  p.causal = causal ? 1 : 0;
  p.scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
  p.n_split = 1;
  p.part_rows = B * Hq * Lq;
  p.decode = 0;
  if (decode_shape(Lq, Lk, seg_q != nullptr)) {
    // row blocks of 64 packed (head, position) rows per KV head
    p.decode = 1;
    p.n_qb = (int)((n_rep * Lq + gqa::kDecodeBlockRows - 1) / gqa::kDecodeBlockRows);
    p.G = (int)(B * Hkv);
  }
  return GQA_OK;
}

static hipError_t launch_fwd(const gqa::FwdParams& p, int dtype, hipStream_t s) {
  if (p.decode)
    return dtype == GQA_F32    ? gqa::launch_decode_f32(p, s)
           : dtype == GQA_BF16 ? gqa::launch_decode_bf16(p, s)
                               : gqa::launch_decode_f16(p, s);
  return dtype == GQA_F32    ? gqa::launch_fwd_f32(p, s)
         : dtype == GQA_BF16 ? gqa::launch_fwd_bf16(p, s)
                             : gqa::launch_fwd_f16(p, s);
}

// Keys per tile of the kernel a plan launches (the unit of a split-KV range).
static int64_t plan_tile_keys(const gqa::FwdParams& p, int dtype) {
  return p.decode ? decode_tile_keys(dtype) : dtype == GQA_F32 ? gqa::kTileKeysF32 : gqa::kTileKeysH16;
}

// Key tiles per split and the number of (non-empty) splits for a requested count.
static void split_shape(int64_t Lk, int64_t tile, int n_split, int* split_tiles, int* n_eff) {
  const int64_t n_tiles = (Lk + tile - 1) / tile;
  const int64_t st = (n_tiles + n_split - 1) / n_split;
  *split_tiles = (int)st;
  *n_eff = (int)((n_tiles + st - 1) / st);
}

GQA_API int gqa_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                            int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                            int64_t q_offset, const int32_t* seg_q, const int32_t* seg_k,
                            int causal, int dtype, void* stream) {
  gqa::FwdParams p{};
  const int rc = fwd_plan(p, q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, q_offset, seg_q, seg_k, causal, dtype);
  if (rc != GQA_OK) return rc;
  (void)hipGetLastError();
  return launch_fwd(p, dtype, (hipStream_t)stream) == hipSuccess ? GQA_OK : GQA_ERR_LAUNCH;
}

// Index rows of a sequence of L ids.
static int64_t seg_index_blocks(int64_t L) { return (L + gqa::kSegBlk - 1) / gqa::kSegBlk; }

GQA_API int64_t gqa_attn_seg_index_bytes(int64_t B, int64_t L) {
  if (B <= 0 || L <= 0) return 0;
  return B * seg_index_blocks(L) * (int64_t)sizeof(gqa::SegBlk);
}

GQA_API int gqa_attn_seg_index(const int32_t* seg, int64_t B, int64_t L, void* index, int64_t index_bytes,
                               void* stream) {
  if (!seg || !index) return GQA_ERR_NULL;
  if (B <= 0 || L <= 0) return GQA_ERR_SHAPE;
  if (L >= ((int64_t)1 << 31) || B >= ((int64_t)1 << 24)) return GQA_ERR_UNSUPPORTED;
  if (misaligned(seg, 4) || misaligned(index, 8)) return GQA_ERR_ALIGN;
  const int64_t need = gqa_attn_seg_index_bytes(B, L);
  if (index_bytes < need) return GQA_ERR_WORKSPACE;
  if (overlap(index, need, seg, B * L * 4)) return GQA_ERR_ALIAS;
  const int64_t nblk = seg_index_blocks(L), total = B * nblk;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  hipLaunchKernelGGL(gqa::seg_index_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, seg, L, nblk,
                     total, (gqa::SegBlk*)index);
  return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_LAUNCH;
}

// Checks of the optional id-range indexes of an indexed call: each only
// beside segment ids, 8-byte aligned, and apart from every output.
static int index_checks(const void* seg_q, const void* seg_q_index, const void* seg_k_index, int64_t B, int64_t Lq,
                        int64_t Lk, const void* const* outs, const int64_t* out_n, int n_out) {
  if (!seg_q && (seg_q_index || seg_k_index)) return GQA_ERR_SHAPE;
  if (misaligned(seg_q_index, 8) || misaligned(seg_k_index, 8)) return GQA_ERR_ALIGN;
  const int64_t qn = gqa_attn_seg_index_bytes(B, Lq), kn = gqa_attn_seg_index_bytes(B, Lk);
  for (int a = 0; a < n_out; ++a)
    if ((seg_q_index && overlap(outs[a], out_n[a], seg_q_index, qn)) ||
        (seg_k_index && overlap(outs[a], out_n[a], seg_k_index, kn)))
      return GQA_ERR_ALIAS;
  return GQA_OK;
}

GQA_API int gqa_attn_fwd_indexed(const void* q, const void* k, const void* v, void* o, float* lse,
                                 int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                                 int64_t q_offset, const int32_t* seg_q, const int32_t* seg_k,
                                 const void* seg_q_index, const void* seg_k_index,
                                 int causal, int dtype, void* stream) {
  gqa::FwdParams p{};
  const int rc = fwd_plan(p, q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, q_offset, seg_q, seg_k, causal, dtype);
  if (rc != GQA_OK) return rc;
  const int64_t es = dtype == GQA_F32 ? 4 : 2;
  const void* outs[2] = {o, lse};
  const int64_t out_n[2] = {B * Hq * Lq * D * es, B * Hq * Lq * 4};
  const int ri = index_checks(seg_q, seg_q_index, seg_k_index, B, Lq, Lk, outs, out_n, 2);
  if (ri != GQA_OK) return ri;
  p.seg_q_idx = (const gqa::SegBlk*)seg_q_index;
  p.seg_k_idx = (const gqa::SegBlk*)seg_k_index;
  (void)hipGetLastError();
  return launch_fwd(p, dtype, (hipStream_t)stream) == hipSuccess ? GQA_OK : GQA_ERR_LAUNCH;
}

GQA_API int gqa_attn_split_count(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int dtype) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Lq <= 0 || Lk <= 0 || Hq % Hkv != 0) return 1;
  const int64_t n_rep = Hq / Hkv;
  const int W = dtype == GQA_F32 ? gqa::kWavesF32 : gqa::kWavesH16;
  const int64_t hpc = heads_per_workgroup(n_rep, W);
  const int64_t ppc = (W / hpc) * (dtype == GQA_F32 ? gqa::kRowsF32 : gqa::kRowsH16);
  // workgroups of one split (for short blocks, those of the decode kernel: the
  // count assumes no segment ids)
  const bool dec = decode_shape(Lq, Lk, false);
  const int64_t base = dec ? ((n_rep * Lq + gqa::kDecodeBlockRows - 1) / gqa::kDecodeBlockRows) * B * Hkv
                           : ((Lq + ppc - 1) / ppc) * B * Hkv * (n_rep / hpc);
  const int64_t tile = dec ? decode_tile_keys(dtype) : dtype == GQA_F32 ? gqa::kTileKeysF32 : gqa::kTileKeysH16;
  const int64_t n_tiles = (Lk + tile - 1) / tile;
  // aim at one workgroup per compute unit, each split at least 4 tiles long
  int64_t n = (kSplitTargetWorkgroups + base - 1) / base;
  n = n < n_tiles / 4 ? n : n_tiles / 4;
  n = n < kMaxSplits ? n : kMaxSplits;
  return (int)(n < 1 ? 1 : n);
}

GQA_API int64_t gqa_attn_split_workspace(int64_t B, int64_t Hq, int64_t Lq, int64_t D, int n_split) {
  if (B <= 0 || Hq <= 0 || Lq <= 0 || D <= 0 || n_split < 1) return 0;
  return (int64_t)n_split * B * Hq * Lq * (D + 1) * 4;
}

// The split-KV launch pair on a workspace that the caller (gqa_attn_fwd_split)
// or the library (gqa_attn_fwd_split_noalloc) provides. `p` is a checked plan.
static int fwd_split_run(gqa::FwdParams& p, const void* q, const void* k, const void* v, void* o, float* lse,
                         int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                         const int32_t* seg_q, const int32_t* seg_k, int dtype, int split_tiles, int n_eff,
                         void* workspace, int64_t workspace_bytes, hipStream_t s) {
  // workspace: fp32 partial O [n_eff][rows][D], then lse parts [n_eff][rows]
  const int64_t rows = B * Hq * Lq;
  const int64_t need = (int64_t)n_eff * rows * (D + 1) * 4;
  if (!workspace) return GQA_ERR_NULL;
  if (workspace_bytes < need) return GQA_ERR_WORKSPACE;
  if (misaligned(workspace, 16)) return GQA_ERR_ALIGN;
  const int64_t es = dtype == GQA_F32 ? 4 : 2;
  const int64_t qo = rows * D * es, kv = B * Hkv * Lk * D * es;
  if (overlap(workspace, need, q, qo) || overlap(workspace, need, k, kv) || overlap(workspace, need, v, kv) ||
      overlap(workspace, need, o, qo) || overlap(workspace, need, lse, rows * 4) ||
      (seg_q && overlap(workspace, need, seg_q, B * Lq * 4)) || (seg_k && overlap(workspace, need, seg_k, B * Lk * 4)))
    return GQA_ERR_ALIAS;
  if ((int64_t)n_eff * p.n_qb * p.G >= ((int64_t)1 << 31) || rows >= ((int64_t)1 << 31)) return GQA_ERR_UNSUPPORTED;
  p.n_split = n_eff;
  p.split_tiles = split_tiles;
  p.o_part = (float*)workspace;
  p.lse_part = (float*)workspace + n_eff * rows * D;
  (void)hipGetLastError();
  if (launch_fwd(p, dtype, s) != hipSuccess) return GQA_ERR_LAUNCH;
  const dim3 grid((unsigned)rows);  // one workgroup per row (rows < 2^31, checked above)
  if (dtype == GQA_F32)
    hipLaunchKernelGGL(gqa::merge_splits_kernel<float>, grid, dim3(256), 0, s, p.o_part, p.lse_part, n_eff,
                       (float*)o, lse, rows);
  else if (dtype == GQA_BF16)
    hipLaunchKernelGGL(gqa::merge_splits_kernel<__bf16>, grid, dim3(256), 0, s, p.o_part, p.lse_part, n_eff,
                       (__bf16*)o, lse, rows);
  else
    hipLaunchKernelGGL(gqa::merge_splits_kernel<_Float16>, grid, dim3(256), 0, s, p.o_part, p.lse_part, n_eff,
                       (_Float16*)o, lse, rows);
  return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_LAUNCH;
}

GQA_API int gqa_attn_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                                  int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                                  int64_t q_offset, const int32_t* seg_q, const int32_t* seg_k,
                                  int causal, int dtype, int n_split, void* workspace, int64_t workspace_bytes,
                                  void* stream) {
  gqa::FwdParams p{};
  const int rc = fwd_plan(p, q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, q_offset, seg_q, seg_k, causal, dtype);
  if (rc != GQA_OK) return rc;
  if (n_split < 1 || n_split > kMaxSplits) return GQA_ERR_UNSUPPORTED;
  int split_tiles, n_eff;
  split_shape(Lk, plan_tile_keys(p, dtype), n_split, &split_tiles, &n_eff);
  hipStream_t s = (hipStream_t)stream;
  if (n_eff <= 1) {
    (void)hipGetLastError();
    return launch_fwd(p, dtype, s) == hipSuccess ? GQA_OK : GQA_ERR_LAUNCH;
  }
  return fwd_split_run(p, q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, seg_q, seg_k, dtype, split_tiles, n_eff, workspace,
                       workspace_bytes, s);
}

// ---------------------------------------------------------------------------
// Allocation-free split-KV forward. Its partial results live in `scratch`, a
// file-scope device array: every GPU the library runs on holds one copy (the
// runtime places it when the code object loads on that device) until the
// process ends. Host code never uses the array's name as an address (on the
// host it names a stand-in): the device address of each GPU's copy comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// is passed to the kernels like the caller's workspace in gqa_attn_fwd_split.
// All calls on one GPU share its copy, so calls that overlap in time on one
// GPU race; nothing in it needs to start at zero.
// ---------------------------------------------------------------------------
namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kScratchDevices];  // device address of `scratch` per device (null until taken)
}  // namespace

static __device__ __align__(256) unsigned char scratch[GQA_NOALLOC_SCRATCH_BYTES];

// Device address of the current device's copy of `scratch` (taken on the first
// call on that device).
static int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return GQA_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return GQA_ERR_LAUNCH;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return GQA_OK;
}

GQA_API int gqa_attn_fwd_split_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                       int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                                       int64_t q_offset, const int32_t* seg_q, const int32_t* seg_k,
                                       int causal, int dtype, int n_split, void* stream) {
  gqa::FwdParams p{};
  const int rc = fwd_plan(p, q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, q_offset, seg_q, seg_k, causal, dtype);
  if (rc != GQA_OK) return rc;
  if (n_split < 0 || n_split > kMaxSplits) return GQA_ERR_UNSUPPORTED;
  const int64_t row_bytes = B * Hq * Lq * (D + 1) * 4;  // one split's partials
  if (n_split == 0) {
    // the recommended count, lowered to what the scratch holds
    n_split = gqa_attn_split_count(B, Hq, Hkv, Lq, Lk, dtype);
    const int64_t fit = GQA_NOALLOC_SCRATCH_BYTES / row_bytes;
    if (n_split > fit) n_split = fit < 1 ? 1 : (int)fit;
  }
  int split_tiles, n_eff;
  split_shape(Lk, plan_tile_keys(p, dtype), n_split, &split_tiles, &n_eff);
  hipStream_t s = (hipStream_t)stream;
  if (n_eff <= 1) {
    (void)hipGetLastError();
    return launch_fwd(p, dtype, s) == hipSuccess ? GQA_OK : GQA_ERR_LAUNCH;
  }
  if ((int64_t)n_eff * row_bytes > GQA_NOALLOC_SCRATCH_BYTES) return GQA_ERR_WORKSPACE;
  void* ws = nullptr;
  const int rs = scratch_address(&ws);
  if (rs != GQA_OK) return rs;
  return fwd_split_run(p, q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, seg_q, seg_k, dtype, split_tiles, n_eff, ws,
                       GQA_NOALLOC_SCRATCH_BYTES, s);
}

static int bwd_run(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv, float* delta,
                   int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                   int64_t q_offset, const int32_t* seg_q, const int32_t* seg_k,
                   const void* seg_q_index, const void* seg_k_index, int causal, int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !delta) return GQA_ERR_NULL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Lq <= 0 || Lk <= 0 || D <= 0) return GQA_ERR_SHAPE;
  if (Hq % Hkv != 0 || q_offset < 0 || q_offset > ((int64_t)1 << 62)) return GQA_ERR_SHAPE;
  if ((seg_q == nullptr) != (seg_k == nullptr)) return GQA_ERR_SHAPE;
  if (D != gqa::kD || (dtype != GQA_F32 && dtype != GQA_BF16 && dtype != GQA_F16)) return GQA_ERR_UNSUPPORTED;
  const int64_t n_rep = Hq / Hkv;
  if (n_rep > kMaxRep || Lq > ((int64_t)1 << 21) || Lk > ((int64_t)1 << 21) || B * Hkv >= ((int64_t)1 << 24))
    return GQA_ERR_UNSUPPORTED;
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16) || misaligned(dout, 16) ||
      misaligned(dq, 16) || misaligned(dk, 16) || misaligned(dv, 16) || misaligned(lse, 4) ||
      misaligned(delta, 4) || misaligned(seg_q, 4) || misaligned(seg_k, 4))
    return GQA_ERR_ALIGN;
  const int64_t es = dtype == GQA_F32 ? 4 : 2;
  const int64_t qo = B * Hq * Lq * D * es, kv = B * Hkv * Lk * D * es, rl = B * Hq * Lq * 4;
  const void* ins[8] = {q, k, v, o, lse, dout, seg_q, seg_k};
  const int64_t in_n[8] = {qo, kv, kv, qo, rl, qo, seg_q ? B * Lq * 4 : 0, seg_k ? B * Lk * 4 : 0};
  const void* outs[4] = {dq, dk, dv, delta};
  const int64_t out_n[4] = {qo, kv, kv, rl};
  for (int a = 0; a < 4; ++a) {
    for (int i = 0; i < 8; ++i)
      if (in_n[i] > 0 && overlap(outs[a], out_n[a], ins[i], in_n[i])) return GQA_ERR_ALIAS;
    for (int b2 = a + 1; b2 < 4; ++b2)
      if (overlap(outs[a], out_n[a], outs[b2], out_n[b2])) return GQA_ERR_ALIAS;
  }
  const int ri = index_checks(seg_q, seg_q_index, seg_k_index, B, Lq, Lk, outs, out_n, 4);
  if (ri != GQA_OK) return ri;

  gqa::BwdParams bp{};
  gqa::FwdParams& p = bp.f;
  p.q = q; p.k = k; p.v = v; p.o = const_cast<void*>(o); p.lse = const_cast<float*>(lse);
  p.seg_q = seg_q; p.seg_k = seg_k;
  p.seg_q_idx = (const gqa::SegBlk*)seg_q_index;
  p.seg_k_idx = (const gqa::SegBlk*)seg_k_index;
  p.Lq = Lq; p.Lk = Lk; p.q_offset = q_offset;
  p.Hq = (int)Hq; p.Hkv = (int)Hkv; p.n_rep = (int)n_rep;
  // work shapes: dQ kernel waves x rows per wave, keys per dK/dV workgroup
  const bool h16 = dtype != GQA_F32;
  const int wq = h16 ? gqa::kBwdWavesDQH : gqa::kBwdWavesDQ;
  const int rq = h16 ? gqa::kBwdRowsDQH : gqa::kBwdRowsDQ;
  const int kb = h16 ? gqa::kBwdKeysDKVH : gqa::kBwdKeysDKV;
  p.hpc = (int)heads_per_workgroup(n_rep, 4);
  p.ppc = (wq / p.hpc) * rq;
  const int64_t n_qb = (Lq + p.ppc - 1) / p.ppc;
  const int64_t G = B * Hkv * (n_rep / p.hpc);
  const int64_t n_kb = (Lk + kb - 1) / kb;
  if (n_qb * G >= ((int64_t)1 << 31) || n_kb * B * Hkv >= ((int64_t)1 << 31)) return GQA_ERR_UNSUPPORTED;
  p.n_qb = (int)n_qb;
  p.G = (int)G;
  p.causal = causal ? 1 : 0;
  p.scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
  bp.dout = dout; bp.dq = dq; bp.dk = dk; bp.dv = dv; bp.delta = delta;
  bp.n_kb = (int)n_kb;
  bp.BH = (int)(B * Hkv);

  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  const hipError_t e = dtype == GQA_F32    ? gqa::launch_bwd_f32(bp, s)
                       : dtype == GQA_BF16 ? gqa::launch_bwd_bf16(bp, s)
                                           : gqa::launch_bwd_f16(bp, s);
  return e == hipSuccess ? GQA_OK : GQA_ERR_LAUNCH;
}

GQA_API int gqa_attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv, float* delta,
                         int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                         int64_t q_offset, const int32_t* seg_q, const int32_t* seg_k,
                         int causal, int dtype, void* stream) {
  return bwd_run(q, k, v, o, lse, dout, dq, dk, dv, delta, B, Hq, Hkv, Lq, Lk, D, q_offset, seg_q, seg_k, nullptr,
                 nullptr, causal, dtype, stream);
}

GQA_API int gqa_attn_bwd_indexed(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                 const void* dout, void* dq, void* dk, void* dv, float* delta,
                                 int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                                 int64_t q_offset, const int32_t* seg_q, const int32_t* seg_k,
                                 const void* seg_q_index, const void* seg_k_index,
                                 int causal, int dtype, void* stream) {
  return bwd_run(q, k, v, o, lse, dout, dq, dk, dv, delta, B, Hq, Hkv, Lq, Lk, D, q_offset, seg_q, seg_k,
                 seg_q_index, seg_k_index, causal, dtype, stream);
}

GQA_API int gqa_attn_merge(const void* o1, const float* lse1, const void* o2, const float* lse2,
                              void* o, float* lse, int64_t rows, int64_t D, int dtype, void* stream) {
  if (!o1 || !lse1 || !o2 || !lse2 || !o || !lse) return GQA_ERR_NULL;
  if (rows <= 0 || D <= 0) return GQA_ERR_SHAPE;
  if (D % 8 != 0 || (dtype != GQA_F32 && dtype != GQA_BF16 && dtype != GQA_F16) || rows >= ((int64_t)1 << 33))
    return GQA_ERR_UNSUPPORTED;
  if (misaligned(o1, 16) || misaligned(o2, 16) || misaligned(o, 16) || misaligned(lse1, 4) ||
      misaligned(lse2, 4) || misaligned(lse, 4))
    return GQA_ERR_ALIGN;
  const int64_t ob = rows * D * (dtype == GQA_F32 ? 4 : 2), lb = rows * 4;
  // outputs may be exactly an input (in place) but must not partially overlap one
  if ((o != o1 && overlap(o, ob, o1, ob)) || (o != o2 && overlap(o, ob, o2, ob)) ||
      (lse != lse1 && overlap(lse, lb, lse1, lb)) || (lse != lse2 && overlap(lse, lb, lse2, lb)) ||
      overlap(o, ob, lse, lb) || overlap(o, ob, lse1, lb) || overlap(o, ob, lse2, lb) ||
      overlap(lse, lb, o1, ob) || overlap(lse, lb, o2, ob))
    return GQA_ERR_ALIAS;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (dtype == GQA_F32)
    hipLaunchKernelGGL(gqa::merge_kernel<float>, grid, dim3(256), 0, s, (const float*)o1, lse1, (const float*)o2,
                       lse2, (float*)o, lse, rows, D);
  else if (dtype == GQA_BF16)
    hipLaunchKernelGGL(gqa::merge_kernel<__bf16>, grid, dim3(256), 0, s, (const __bf16*)o1, lse1,
                       (const __bf16*)o2, lse2, (__bf16*)o, lse, rows, D);
  else
    hipLaunchKernelGGL(gqa::merge_kernel<_Float16>, grid, dim3(256), 0, s, (const _Float16*)o1, lse1,
                       (const _Float16*)o2, lse2, (_Float16*)o, lse, rows, D);
  return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_LAUNCH;
}

GQA_API const char* gqa_attn_strerror(int code) {
  switch (code) {
    case GQA_OK: return "success";
    case GQA_ERR_NULL: return "a required pointer is NULL";
    case GQA_ERR_SHAPE: return "invalid shape: non-positive extent, Hq not a multiple of Hkv, negative q_offset, "
                               "only one segment-id array, or an id index without segment ids";
    case GQA_ERR_UNSUPPORTED: return "unsupported: D must be 256, dtype F32, BF16 or F16, Hq/Hkv at most 64, "
                                     "lengths below 2^31 (backward: at most 2^21)";
    case GQA_ERR_ALIGN: return "misaligned pointer: tensors need 16-byte alignment, lse and segment ids 4-byte";
    case GQA_ERR_LAUNCH: return "kernel launch failed";
    case GQA_ERR_ALIAS: return "output overlaps an input";
    case GQA_ERR_WORKSPACE: return "workspace smaller than gqa_attn_split_workspace() for the split count "
                                   "(allocation-free call: the partials exceed GQA_NOALLOC_SCRATCH_BYTES; "
                                   "id index: smaller than gqa_attn_seg_index_bytes())";
    default: return "unknown status code";
  }
}

GQA_API int gqa_attn_version(void) { return (1 << 16) | 8; }
