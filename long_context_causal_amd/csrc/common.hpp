// common.hpp -- device-side pieces shared by the gfx950 attention kernels:
// vector types, the work decode (which query block and head group a workgroup
// owns), the per-workgroup segment scan that decides which key tiles are
// visible, and small lane-exchange helpers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kD = 256;             // head dimension the kernels are built for
constexpr float kInvSqrtD = 0.0625f;  // 1/sqrt(kD), exact
static_assert(kD == 256, "kInvSqrtD is 1/sqrt(256)");
constexpr int kRowsPerWave = 32;    // query rows (one head, 32 positions) per wave

// Id range (min, max) of one block of kSegBlk consecutive segment ids: the
// entry type of the index that gqa_attn_seg_index writes.
constexpr int kSegBlk = 16;
struct SegBlk {
  int32_t lo, hi;
};

// Arguments of one forward launch (passed by value).
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* seg_q;
  const int32_t* seg_k;
  // optional id-range indexes of seg_q / seg_k (SegBlk per 16 entries, rows of
  // ceil(L / 16) per batch; null: the kernels scan the ids themselves)
  const SegBlk* seg_q_idx;
  const SegBlk* seg_k_idx;
  int64_t Lq, Lk, q_offset;
  int Hq, Hkv, n_rep;
  int hpc;        // query heads per workgroup (a divisor of n_rep)
  int ppc;        // query positions per workgroup
  int n_qb;       // number of position blocks
  int G;          // B * Hkv * (n_rep / hpc): independent head groups per position block
  int causal;
  float scale_log2;  // log2(e) / sqrt(D): scores go straight to the base-2 domain
  // Split-KV (n_split > 1): the grid is n_split x (n_qb * G); split s takes the
  // key tiles [s split_tiles, (s + 1) split_tiles) (in the kernel's own tile
  // size) and writes its normalised partial O (fp32) and lse to
  // o_part[s][row][D] and lse_part[s][row] (row over B * Hq * Lq) instead of o, lse.
  int n_split;
  int split_tiles;
  int64_t part_rows;  // B * Hq * Lq: the rows of one split's part
  float* o_part;
  float* lse_part;
  // Host plan only: the launch goes to the short-block (decode) kernel, whose
  // grid is n_split x n_qb row blocks of 64 packed rows x G = B * Hkv.
  int decode;
};

// Arguments of one backward launch pair (passed by value to both kernels).
struct BwdParams {
  FwdParams f;   // q, k, v, o, lse, ids, shape; plan (hpc, ppc, n_qb, G) of the dQ kernel
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* delta;  // [B, Hq, Lq]: written by the dQ kernel, read by the dK/dV kernel
  int n_kb;      // key blocks per key/value head (dK/dV kernel)
  int BH;        // B * Hkv
};

// Which (batch, kv head, head chunk, position block) a workgroup owns.
// Block ids run over position blocks from the last (most keys under a causal
// mask) to the first, and over head groups fastest. Workgroups are handed to
// the 8 XCDs round-robin by id, so with 4 (or 8) head groups every XCD works on
// one kv head and its K/V stream stays in that XCD's L2.
struct Work {
  int b, kvh, h0, qb;
  int64_t p0;
  int split;  // key split of a split-KV launch (0 otherwise)
};

__device__ __forceinline__ Work decode_work(const FwdParams& p) {
  const int base = p.n_qb * p.G;
  const int i = (int)blockIdx.x % base;
  Work w;
  w.split = (int)blockIdx.x / base;
  w.qb = p.n_qb - 1 - i / p.G;
  const int gi = i % p.G;
  const int nhc = p.n_rep / p.hpc;
  const int hc = gi % nhc;
  const int rest = gi / nhc;
  w.kvh = rest % p.Hkv;
  w.b = rest / p.Hkv;
  w.h0 = w.kvh * p.n_rep + hc * p.hpc;
  w.p0 = (int64_t)w.qb * p.ppc;
  return w;
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// max / sum of a value with the same value in lane l ^ 32.
__device__ __forceinline__ float xor32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// max / sum of a value over the 4 lanes l % 16 + 16 j (j = 0..3): the lanes
// of one query row in the 16x16 product layouts (the decode kernels).
__device__ __forceinline__ float xor16_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float row4_max(float x) { return xor32_max(xor16_max(x)); }
__device__ __forceinline__ float row4_sum(float x) { return xor32_sum(xor16_sum(x)); }

__device__ __forceinline__ int wave_min_i(int x) {
  for (int s = 32; s >= 1; s >>= 1) x = min(x, __shfl_xor(x, s));
  return x;
}
__device__ __forceinline__ int wave_max_i(int x) {
  for (int s = 32; s >= 1; s >>= 1) x = max(x, __shfl_xor(x, s));
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}
__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// The same wait as a builtin, which the compiler's own wait insertion sees: after
// the loads a kernel makes before its main loop (Q, K held in registers), so
// that the compiler places no vmcnt wait for them inside the loop, where the
// counter also counts the loop's async tile copies and such a wait would hold
// the wave until the next tile's copies land. (gfx9 encoding: vmcnt 0,
// expcnt 7, lgkmcnt 15.)
__device__ __forceinline__ void wait_vm0_known() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Async global -> LDS copies through a buffer resource (MUBUF with the LDS
// bit): lane l's 16 (or 4) bytes from the resource base + voff land at LDS
// byte lds + 16 l (or 4 l); the resource and lds must be the same in every
// lane of the wave. The resource bounds the read, and lanes whose offset falls
// at or past its size read zeros, so a tile that runs past the end of a tensor
// needs no clamping. Resource words: 48-bit base address (stride 0), size in
// bytes, and the format word of a raw 32-bit buffer on this family.
// The copies are issued through inline asm on purpose: the compiler then does
// not treat them as LDS stores whose completion every later LDS read must wait
// for, which would serialise the prefetch ring. Completion is ensured by the
// explicit s_waitcnt vmcnt waits and workgroup barriers of the kernels. The
// instruction writes no VGPR; M0 (the LDS base) is set in the same asm block,
// one wait state ahead.
typedef __attribute__((ext_vector_type(4))) int rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return rsrc_t{(int)(uint32_t)a, (int)(uint32_t)(a >> 32), (int)bytes, 0x00020000};
}
// lds: LDS byte address of the wave's 1 KB (or 256 B) destination. It and the
// resource words go through readfirstlane: they are wave-uniform, and this
// keeps them in SGPRs even where the compiler has placed a uniform value in
// VGPRs (inside a branch on the lane index, for one); where they already are
// in SGPRs the compiler drops the readfirstlane.
__device__ __forceinline__ rsrc_t uniform_rsrc(rsrc_t r) {
  return rsrc_t{__builtin_amdgcn_readfirstlane(r[0]), __builtin_amdgcn_readfirstlane(r[1]),
                __builtin_amdgcn_readfirstlane(r[2]), __builtin_amdgcn_readfirstlane(r[3])};
}
__device__ __forceinline__ void buf2lds16(rsrc_t rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(uniform_rsrc(rsrc)) : "memory");
}
// The same with the LDS address lds + imm, imm a constant once the caller is
// inlined and unrolled: the add writes M0 directly (one scalar instruction
// per copy instead of an add and a move). The add also sets SCC (its carry),
// hence the clobber: without it the compiler may keep a carry live across the
// block, between the two halves of a 64-bit address add, and the high half
// then loses it.
__device__ __forceinline__ void buf2lds16_imm(rsrc_t rsrc, uint32_t voff, uint32_t lds, uint32_t imm) {
  asm volatile("s_add_u32 m0, %0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(uniform_rsrc(rsrc)), "i"(imm)
               : "memory", "scc");
}
// The 4-byte copy takes its resource words through readfirstlane, a VALU
// write of SGPRs that a vector-memory read of them must trail by 5 wait
// states; the compiler inserts those only before loads it can see, so the
// block brings its own (the M0 move and s_nop 3). The 16-byte copies pass
// their resource as it is; tests/test_asm_hazards.py checks the compiled
// kernels for a VALU-written SGPR within 5 wait states of any copy.
__device__ __forceinline__ void buf2lds4(rsrc_t rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 3\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(uniform_rsrc(rsrc)) : "memory");
}

// ---------------------------------------------------------------------------
// Segment classification. With segment ids, a key tile is visible to the
// workgroup when the id range of its keys meets the id range of the
// workgroup's query rows, and "full" (no element mask needed for the segment
// part) when both ranges are the same single id. The ranges are exact for any
// ids and tight for sorted (packed) ids. The state is two bits per group of
// 2^shift consecutive tiles, shift the smallest that fits the tile count into
// kSegGroups groups: one tile per bit up to 32,768 tiles (2M keys in 64-key
// tiles), then groups of 2, 4, ... tiles, so the metadata is a fixed 8 KB of
// LDS at any length and never grows as (L / tile)^2 (the block-mask tables of
// splash attention do, and overflowed at 1M tokens: maxtext pull request 4929,
// problem statement). A group is visible if any of its tiles is; a tile of a
// visible group that holds no visible key is processed with the element mask
// and contributes nothing.
// ---------------------------------------------------------------------------
constexpr int kSegGroups = 32768;  // bits per map (visible, full)
struct SegBits {
  unsigned vis[kSegGroups / 32];
  unsigned full[kSegGroups / 32];
  int qmin, qmax;
};

// log2 of the tiles per group for a map of n_tiles tiles.
__device__ __forceinline__ int seg_shift(int n_tiles) {
  int s = 0;
  while (((int64_t)(n_tiles - 1) >> s) >= kSegGroups) ++s;
  return s;
}

// Min and max over each aligned group of `lanes` lanes (a power of two,
// 1..64); every lane of a group ends with its group's values. The steps pair
// lane l with l ^ 1 and l ^ 2 (quad permutes), then with its mirror in the
// half row and in the row (after the earlier steps those hold the values of
// l ^ 4 and l ^ 8), then l ^ 16 and l ^ 32 (row swaps).
__device__ __forceinline__ void group_minmax(int& lo, int& hi, int lanes) {
  if (lanes >= 2) { lo = min(lo, __builtin_amdgcn_mov_dpp(lo, 0xB1, 0xF, 0xF, false));
                    hi = max(hi, __builtin_amdgcn_mov_dpp(hi, 0xB1, 0xF, 0xF, false)); }
  if (lanes >= 4) { lo = min(lo, __builtin_amdgcn_mov_dpp(lo, 0x4E, 0xF, 0xF, false));
                    hi = max(hi, __builtin_amdgcn_mov_dpp(hi, 0x4E, 0xF, 0xF, false)); }
  if (lanes >= 8) { lo = min(lo, __builtin_amdgcn_mov_dpp(lo, 0x141, 0xF, 0xF, false));
                    hi = max(hi, __builtin_amdgcn_mov_dpp(hi, 0x141, 0xF, 0xF, false)); }
  if (lanes >= 16) { lo = min(lo, __builtin_amdgcn_mov_dpp(lo, 0x140, 0xF, 0xF, false));
                     hi = max(hi, __builtin_amdgcn_mov_dpp(hi, 0x140, 0xF, 0xF, false)); }
  if (lanes >= 32) {
    const auto a = __builtin_amdgcn_permlane16_swap((unsigned)lo, (unsigned)lo, false, false);
    const auto b = __builtin_amdgcn_permlane16_swap((unsigned)hi, (unsigned)hi, false, false);
    lo = min((int)a[0], (int)a[1]);
    hi = max((int)b[0], (int)b[1]);
  }
  if (lanes >= 64) {
    const auto a = __builtin_amdgcn_permlane32_swap((unsigned)lo, (unsigned)lo, false, false);
    const auto b = __builtin_amdgcn_permlane32_swap((unsigned)hi, (unsigned)hi, false, false);
    lo = min((int)a[0], (int)a[1]);
    hi = max((int)b[0], (int)b[1]);
  }
}

typedef __attribute__((ext_vector_type(4), aligned(4))) int i32x4_a4;  // 4-byte aligned 16-byte load

// The bits at lanes 0, 4, 8, ..., 60 of a wave mask, packed into bits 0..15.
__device__ __forceinline__ unsigned pack_quads(uint64_t m) {
  m &= 0x1111111111111111ull;
  m = (m | (m >> 3)) & 0x0303030303030303ull;
  m = (m | (m >> 6)) & 0x000F000F000F000Full;
  m = (m | (m >> 12)) & 0x000000FF000000FFull;
  m = (m | (m >> 24)) & 0xFFFFull;
  return (unsigned)m;
}

// Classifies the tiles of the scanned side for one workgroup. `own` are the
// ids of the workgroup's own entries [own0, own0 + own_n) of a sequence of
// own_len (entries past the end are ignored); the scanned side `other`
// (other_len entries) is cut into tiles of BT entries, tiles [0, n_tiles);
// groups wholly below tile t_first are left invisible (the caller never
// visits them). sh = seg_shift(n_tiles).
// Layout of the reads: a batch is 16 consecutive tiles, tile 16 b + q read by
// the four lanes of quad q, each lane 16 contiguous bytes of each 16-entry
// chunk of the tile, so a load instruction covers 64 contiguous bytes per tile
// and 16 tiles; 16 loads per lane are in flight, then the tile ranges come
// from two quad steps. With one tile per map bit the 16 tiles' bits of a
// batch come from one ballot; larger groups reduce further across lanes (and
// across batches) and set their bits with LDS atomics. Each wave owns a
// contiguous run of map words.
// First part of both scans: the id range of the own entries into sb.qmin /
// sb.qmax, and the map words of n_tiles tiles cleared; returns the word count.
template <int NT>
__device__ int seg_scan_begin(SegBits& sb, int sh, const int32_t* own, int64_t own0, int own_n, int64_t own_len,
                              int n_tiles) {
  const int tid = threadIdx.x, lane = lane_id();
  if (tid == 0) { sb.qmin = INT32_MAX; sb.qmax = INT32_MIN; }
  __syncthreads();
  {
    int lo = INT32_MAX, hi = INT32_MIN;
    for (int i = tid; i < own_n; i += NT) {
      const int64_t x = own0 + i;
      if (x < own_len) { const int s = own[x]; lo = min(lo, s); hi = max(hi, s); }
    }
    lo = wave_min_i(lo);
    hi = wave_max_i(hi);
    if (lane == 0) { atomicMin(&sb.qmin, lo); atomicMax(&sb.qmax, hi); }
  }
  const int n_groups = (int)(((int64_t)n_tiles - 1) >> sh) + 1;
  const int n_words = (n_groups + 31) >> 5;
  for (int wd = tid; wd < n_words; wd += NT) { sb.vis[wd] = 0u; sb.full[wd] = 0u; }
  __syncthreads();
  return n_words;
}

template <int NT, int BT>
__device__ void seg_scan_ids(SegBits& sb, int sh, const int32_t* own, int64_t own0, int own_n, int64_t own_len,
                             const int32_t* other, int64_t other_len, int n_tiles, int t_first = 0) {
  static_assert(BT == 16 || BT == 32 || BT == 64, "tiles of 16, 32 or 64 entries");
  constexpr int W = NT / 64;
  constexpr int kCh = BT / 16;     // 16-entry chunks per tile: loads per batch
  constexpr int kNB = 16 / kCh;    // batches per pass (16 loads per lane in flight)
  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  const int q = lane >> 2, r = lane & 3;
  const int n_words = seg_scan_begin<NT>(sb, sh, own, own0, own_n, own_len, n_tiles);
  const int qmin = sb.qmin, qmax = sb.qmax;
  const int64_t lim = min(other_len, (int64_t)n_tiles * BT);  // entries past it count as absent
  const int w_first = min(n_words, (min(t_first, n_tiles) >> sh) >> 5);
  const int per_wave = (n_words - w_first + W - 1) / W;
  const int wb = w_first + wave * per_wave, we = min(n_words, wb + per_wave);
  if (lim < 4) {
    // fewer than 4 entries (one tile, one group): the first lane classifies them
    if (tid == 0) {
      int lo = INT32_MAX, hi = INT32_MIN;
      for (int64_t x = 0; x < lim; ++x) { lo = min(lo, other[x]); hi = max(hi, other[x]); }
      if (lo <= qmax && hi >= qmin) sb.vis[0] = 1u;
      if (lo == hi && qmin == qmax && lo == qmin) sb.full[0] = 1u;
    }
  } else if (wb < we) {
    const int64_t tb = (int64_t)wb << (5 + sh), te = min((int64_t)n_tiles, (int64_t)we << (5 + sh));
    const int gq = sh < 4 ? 4 << sh : 64;   // lanes per group within a batch (16 tiles = 64 lanes)
    const int nbg = sh > 4 ? 1 << (sh - 4) : 1;  // batches per group
    unsigned vword = 0u, fword = 0u;
    int bg = 0, lo_acc = INT32_MAX, hi_acc = INT32_MIN;
    constexpr int64_t kPass = 16 * kNB;  // tiles per pass
    // the 16 loads of the pass at tile t0 (windows past lim pulled back to end at it)
    auto load = [&](i32x4_a4* vv, int64_t t0) {
#pragma unroll
      for (int b = 0; b < kNB; ++b)
#pragma unroll
        for (int j = 0; j < kCh; ++j) {
          const int64_t x = (t0 + 16 * b + q) * BT + 16 * j + 4 * r;
          vv[b * kCh + j] = *(const i32x4_a4*)(other + (x + 4 <= lim ? x : lim - 4));
        }
    };
    auto process = [&](i32x4_a4* vv, int64_t t0) {
      // one statement that takes every loaded value of the pass: all 16 loads
      // are issued before it and waited for once
      asm volatile("" : "+v"(vv[0]), "+v"(vv[1]), "+v"(vv[2]), "+v"(vv[3]), "+v"(vv[4]), "+v"(vv[5]),
                   "+v"(vv[6]), "+v"(vv[7]), "+v"(vv[8]), "+v"(vv[9]), "+v"(vv[10]), "+v"(vv[11]),
                   "+v"(vv[12]), "+v"(vv[13]), "+v"(vv[14]), "+v"(vv[15]));
#pragma unroll
      for (int b = 0; b < kNB; ++b) {
        const int64_t tbat = t0 + 16 * b;
        if (tbat >= te) break;  // uniform
        int lo = INT32_MAX, hi = INT32_MIN;
#pragma unroll
        for (int j = 0; j < kCh; ++j) {
          const int64_t x = (tbat + q) * BT + 16 * j + 4 * r;
          const int64_t d = x + 4 <= lim ? 0 : x - (lim - 4);  // window entries below this lane's own
          const i32x4_a4 v = vv[b * kCh + j];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            lo = c >= d ? min(lo, v[c]) : lo;
            hi = c >= d ? max(hi, v[c]) : hi;
          }
        }
        // the quad's tile: lanes l ^ 1 and l ^ 2
        lo = min(lo, __builtin_amdgcn_mov_dpp(lo, 0xB1, 0xF, 0xF, false));
        hi = max(hi, __builtin_amdgcn_mov_dpp(hi, 0xB1, 0xF, 0xF, false));
        lo = min(lo, __builtin_amdgcn_mov_dpp(lo, 0x4E, 0xF, 0xF, false));
        hi = max(hi, __builtin_amdgcn_mov_dpp(hi, 0x4E, 0xF, 0xF, false));
        if (sh == 0) {
          // one tile per bit: the batch's 16 bits from one ballot (all four
          // lanes of a quad agree), half a map word
          const bool v_ok = lo <= hi && lo <= qmax && hi >= qmin;
          const bool f_ok = lo <= hi && lo == hi && qmin == qmax && lo == qmin;
          const int half = (int)(tbat >> 4) & 1;
          vword |= pack_quads(__builtin_amdgcn_ballot_w64(v_ok)) << (16 * half);
          fword |= pack_quads(__builtin_amdgcn_ballot_w64(f_ok)) << (16 * half);
          if (half == 1 || tbat + 16 >= te) {
            if (lane == 0) { sb.vis[tbat >> 5] = vword; sb.full[tbat >> 5] = fword; }
            vword = fword = 0u;
          }
        } else {
          // groups of 2^sh tiles: gq lanes of this batch (and nbg batches)
          group_minmax(lo, hi, gq);
          lo_acc = min(lo_acc, lo);
          hi_acc = max(hi_acc, hi);
          if (++bg < nbg && tbat + 16 < te) continue;  // the range's last group may be cut short
          bg = 0;
          lo = lo_acc;
          hi = hi_acc;
          lo_acc = INT32_MAX;
          hi_acc = INT32_MIN;
          if ((lane & (gq - 1)) == 0 && lo <= hi) {
            const int gi = (int)((tbat + q) >> sh);
            if (lo <= qmax && hi >= qmin) atomicOr(&sb.vis[gi >> 5], 1u << (gi & 31));
            if (lo == hi && qmin == qmax && lo == qmin) atomicOr(&sb.full[gi >> 5], 1u << (gi & 31));
          }
        }
      }
    };
    i32x4_a4 vv[16];
    for (int64_t t0 = tb; t0 < te; t0 += kPass) {
      load(vv, t0);
      process(vv, t0);
    }
  }
  __syncthreads();
}

// The same classification from an id-range index of the scanned side
// (SegBlk per kSegBlk entries, nblk = ceil(other_len / kSegBlk) entries) in
// place of its ids: a tile's range is the range of its BT / kSegBlk index
// entries, which is the range of its ids, so the map comes out bit for bit as
// seg_scan_ids makes it, from 1/8 of the bytes. Layout of the reads: a batch
// is 64 consecutive tiles, one per lane; 4 batches per pass, their entries
// loaded together (addresses clamped into the index, entries past its end
// taken as empty).
template <int NT, int BT>
__device__ void seg_scan_index(SegBits& sb, int sh, const int32_t* own, int64_t own0, int own_n, int64_t own_len,
                               const SegBlk* other, int64_t other_len, int n_tiles, int t_first = 0) {
  static_assert(BT == 16 || BT == 32 || BT == 64, "tiles of 16, 32 or 64 entries");
  constexpr int W = NT / 64;
  constexpr int kE = BT / kSegBlk;  // index entries per tile
  constexpr int kB = 4;             // batches of 64 tiles per pass
  const int lane = lane_id(), wave = wave_id();
  const int n_words = seg_scan_begin<NT>(sb, sh, own, own0, own_n, own_len, n_tiles);
  const int qmin = sb.qmin, qmax = sb.qmax;
  const int64_t nblk = (other_len + kSegBlk - 1) / kSegBlk;
  const int w_first = min(n_words, (min(t_first, n_tiles) >> sh) >> 5);
  const int per_wave = (n_words - w_first + W - 1) / W;
  const int wb = w_first + wave * per_wave, we = min(n_words, wb + per_wave);
  if (wb < we) {
    const int64_t tb = (int64_t)wb << (5 + sh), te = min((int64_t)n_tiles, (int64_t)we << (5 + sh));
    const int gq = sh < 6 ? 1 << sh : 64;        // lanes per group within a batch
    const int nbg = sh > 6 ? 1 << (sh - 6) : 1;  // batches per group
    int bg = 0, lo_acc = INT32_MAX, hi_acc = INT32_MIN;
    for (int64_t t0 = tb; t0 < te; t0 += 64 * kB) {
      SegBlk e[kB][kE];
#pragma unroll
      for (int b = 0; b < kB; ++b)
#pragma unroll
        for (int i = 0; i < kE; ++i) {
          const int64_t blk = (t0 + 64 * b + lane) * kE + i;
          e[b][i] = other[blk < nblk ? blk : nblk - 1];
        }
#pragma unroll
      for (int b = 0; b < kB; ++b) {
        const int64_t tbat = t0 + 64 * b;
        if (tbat >= te) break;  // uniform
        const int64_t t = tbat + lane;
        int lo = INT32_MAX, hi = INT32_MIN;
#pragma unroll
        for (int i = 0; i < kE; ++i) {
          const bool ok = t < te && t * kE + i < nblk;
          lo = ok ? min(lo, e[b][i].lo) : lo;
          hi = ok ? max(hi, e[b][i].hi) : hi;
        }
        if (sh == 0) {
          // one tile per bit: the batch's 64 bits from one ballot, two map
          // words (the second only while it is this wave's)
          const uint64_t vm = __builtin_amdgcn_ballot_w64(lo <= hi && lo <= qmax && hi >= qmin);
          const uint64_t fm = __builtin_amdgcn_ballot_w64(lo <= hi && lo == hi && qmin == qmax && lo == qmin);
          const int wd = (int)(tbat >> 5);
          if (lane == 0) {
            sb.vis[wd] = (unsigned)vm;
            sb.full[wd] = (unsigned)fm;
            if (wd + 1 < we) {
              sb.vis[wd + 1] = (unsigned)(vm >> 32);
              sb.full[wd + 1] = (unsigned)(fm >> 32);
            }
          }
        } else {
          // groups of 2^sh tiles: gq lanes of this batch (and nbg batches)
          group_minmax(lo, hi, gq);
          lo_acc = min(lo_acc, lo);
          hi_acc = max(hi_acc, hi);
          if (++bg < nbg && tbat + 64 < te) continue;  // the range's last group may be cut short
          bg = 0;
          lo = lo_acc;
          hi = hi_acc;
          lo_acc = INT32_MAX;
          hi_acc = INT32_MIN;
          if ((lane & (gq - 1)) == 0 && lo <= hi) {
            const int gi = (int)(t >> sh);
            if (lo <= qmax && hi >= qmin) atomicOr(&sb.vis[gi >> 5], 1u << (gi & 31));
            if (lo == hi && qmin == qmax && lo == qmin) atomicOr(&sb.full[gi >> 5], 1u << (gi & 31));
          }
        }
      }
    }
  }
  __syncthreads();
}

// Scans of the forward, the dQ kernel (key tiles) and the dK/dV kernel (row
// tiles): from the index where the call brings one, else from the ids.
template <int NT, int BT>
__device__ __forceinline__ void seg_scan_any(SegBits& sb, int sh, const int32_t* own, int64_t own0, int own_n,
                                             int64_t own_len, const int32_t* other, const SegBlk* other_idx,
                                             int64_t other_len, int n_tiles, int t_first = 0) {
  if (other_idx)
    seg_scan_index<NT, BT>(sb, sh, own, own0, own_n, own_len, other_idx, other_len, n_tiles, t_first);
  else
    seg_scan_ids<NT, BT>(sb, sh, own, own0, own_n, own_len, other, other_len, n_tiles, t_first);
}

// The forward's use: own = the workgroup's query rows, scanned = key tiles of BK.
template <int W, int BK>
__device__ void seg_scan(SegBits& sb, int sh, const FwdParams& p, const Work& w, int n_tiles) {
  const int64_t nblk = (p.Lk + kSegBlk - 1) / kSegBlk;
  seg_scan_any<W * 64, BK>(sb, sh, p.seg_q + (int64_t)w.b * p.Lq, w.p0, p.ppc, p.Lq, p.seg_k + (int64_t)w.b * p.Lk,
                           p.seg_k_idx ? p.seg_k_idx + (int64_t)w.b * nblk : nullptr, p.Lk, n_tiles);
}

// The searches below run on every lane of the wave with the same arguments
// (the kernels call them where control flow is wave-uniform): lane l reads map
// word w0 + l (or w1 - l), so one LDS read and one ballot cover 64 words
// (2,048 groups), and the word that holds the answer comes over from its lane
// into a scalar register (v_readlane). The tile index derived from it then
// feeds scalar address arithmetic: the tile copies take their buffer resource
// from SGPRs written by scalar instructions, never straight from a VALU
// write, which a copy would have to trail by 5 wait states. A serial walk
// word by word took one LDS round trip per 32 groups, thousands of cycles for
// a workgroup far into a long sequence.

// First group in [g, ng) whose bit in `bits` is `val` (ng if none).
__device__ __forceinline__ int seg_find(const unsigned* bits, int g, int ng, bool val) {
  const int lane = lane_id();
  const int wg = g >> 5, wlast = (ng - 1) >> 5;
  for (int w0 = wg; w0 <= wlast; w0 += 64) {
    const int wi = w0 + lane;
    unsigned w = 0u;
    if (wi <= wlast) {
      w = bits[wi];
      if (!val) w = ~w;
      if (wi == wg) w &= ~0u << (g & 31);  // groups below g
    }
    const uint64_t m = __builtin_amdgcn_ballot_w64(w != 0u);
    if (m) {
      const int l = __builtin_ctzll(m);
      const unsigned wf = (unsigned)__builtin_amdgcn_readlane((int)w, l);
      const int r = ((w0 + l) << 5) + __builtin_ctz(wf);
      return r < ng ? r : ng;
    }
  }
  return ng;
}

// Last group in [glo, g] whose bit in `bits` is set (glo - 1 if none).
__device__ __forceinline__ int seg_find_last(const unsigned* bits, int g, int glo) {
  const int lane = lane_id();
  const int wg = g >> 5, wlo = glo >> 5;
  for (int w1 = wg; w1 >= wlo; w1 -= 64) {
    const int wi = w1 - lane;
    unsigned w = 0u;
    if (wi >= wlo) {
      w = bits[wi];
      if (wi == wg) w &= (2u << (g & 31)) - 1u;  // groups above g
    }
    const uint64_t m = __builtin_amdgcn_ballot_w64(w != 0u);
    if (m) {
      const int l = __builtin_ctzll(m);
      const unsigned wf = (unsigned)__builtin_amdgcn_readlane((int)w, l);
      const int r = ((w1 - l) << 5) + 31 - __builtin_clz(wf);
      return r >= glo ? r : glo - 1;
    }
  }
  return glo - 1;
}

// First tile >= t of a visible group (n_tiles if none): t itself when its
// group is visible, else the first tile of the next visible group.
__device__ __forceinline__ int seg_next(const SegBits& sb, int sh, int t, int n_tiles) {
  if (t >= n_tiles) return n_tiles;
  const int g0 = t >> sh, ng = ((n_tiles - 1) >> sh) + 1;
  const int r = seg_find(sb.vis, g0, ng, true);
  if (r >= ng) return n_tiles;
  return r == g0 ? t : min(n_tiles, r << sh);
}

// Last tile <= t and >= lo of a visible group (lo - 1 if none): t itself when
// its group is visible, else the last tile of the previous visible group.
__device__ __forceinline__ int seg_prev(const SegBits& sb, int sh, int t, int lo) {
  if (t < lo) return lo - 1;
  const int g0 = t >> sh, glo = lo >> sh;
  const int r = seg_find_last(sb.vis, g0, glo);
  if (r < glo) return lo - 1;
  return r == g0 ? t : ((r + 1) << sh) - 1;
}

// The first run of set bits of a map (vis or full) at or after tile t, in
// tiles: [lo, hi), lo >= t; lo = hi = n_tiles if there is none. A kernel that
// visits tiles in increasing order keeps the run and reads the map again only
// once it has passed the run's end.
__device__ __forceinline__ void seg_run(const unsigned* bits, int sh, int t, int n_tiles, int& lo, int& hi) {
  const int ng = ((n_tiles - 1) >> sh) + 1;
  const int gs = seg_find(bits, t >> sh, ng, true);
  if (gs >= ng) {
    lo = hi = n_tiles;
    return;
  }
  const int gz = seg_find(bits, gs, ng, false);
  lo = max(t, gs << sh);
  hi = min(n_tiles, gz << sh);
}

// Is every key of tile t's group of the workgroup's single query id?
__device__ __forceinline__ bool seg_full_tile(const SegBits& sb, int sh, int t) {
  const int g = t >> sh;
  return (sb.full[g >> 5] >> (g & 31)) & 1u;
}

}  // namespace gqa
