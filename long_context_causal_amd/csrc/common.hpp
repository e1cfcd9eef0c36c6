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
constexpr int kMaxSegTiles = 16384; // key tiles a workgroup can classify for segment skipping

// Arguments of one forward launch (passed by value).
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* seg_q;
  const int32_t* seg_k;
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
// keeps them in SGPRs even where the compiler cannot prove that (inside a
// branch on the lane index, for one).
__device__ __forceinline__ rsrc_t uniform_rsrc(rsrc_t r) {
  return rsrc_t{__builtin_amdgcn_readfirstlane(r[0]), __builtin_amdgcn_readfirstlane(r[1]),
                __builtin_amdgcn_readfirstlane(r[2]), __builtin_amdgcn_readfirstlane(r[3])};
}
__device__ __forceinline__ void buf2lds16(rsrc_t rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rsrc) : "memory");
}
// The same with the LDS address lds + imm, imm a constant once the caller is
// inlined and unrolled: the add writes M0 directly (one scalar instruction
// per copy instead of an add and a move). The add also sets SCC (its carry),
// hence the clobber: without it the compiler may keep a carry live across the
// block, between the two halves of a 64-bit address add, and the high half
// then loses it.
__device__ __forceinline__ void buf2lds16_imm(rsrc_t rsrc, uint32_t voff, uint32_t lds, uint32_t imm) {
  asm volatile("s_add_u32 m0, %0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rsrc), "i"(imm) : "memory", "scc");
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
// Segment scan. With segment ids, a key tile is visible to the workgroup when
// the id range of its keys meets the id range of the workgroup's query rows; it
// is "full" (no element mask needed for the segment part) when both ranges are
// the same single id. Ranges are exact for any ids and tight for sorted
// (packed) ids, and the per-tile state is two bits, so the metadata grows with
// L / tile, never with (L / tile)^2.
// ---------------------------------------------------------------------------
struct SegBits {
  unsigned vis[kMaxSegTiles / 32];
  unsigned full[kMaxSegTiles / 32];
  int qmin, qmax;
};

// Generic form: `own` are the ids of this workgroup's own entries [own0,
// own0 + own_n) of a sequence of own_len (entries past the end are ignored);
// the scanned side `other` (other_len entries) is cut into tiles of BT.
template <int NT, int BT>
__device__ void seg_scan_ids(SegBits& sb, const int32_t* own, int64_t own0, int own_n, int64_t own_len,
                             const int32_t* other, int64_t other_len, int n_tiles) {
  constexpr int W = NT / 64;
  constexpr int KPL = BT < 32 ? BT : 32;  // consecutive entries each lane reduces per pass
  constexpr int LPT = BT / KPL;           // lanes that share one tile
  static_assert(BT % KPL == 0, "tile must be a whole number of lane chunks");
  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  const int words = (n_tiles + 31) >> 5;
  for (int i = tid; i < words; i += NT) { sb.vis[i] = 0u; sb.full[i] = 0u; }
  if (tid == 0) { sb.qmin = INT32_MAX; sb.qmax = INT32_MIN; }
  __syncthreads();
  // id range of this workgroup's own entries
  {
    int lo = INT32_MAX, hi = INT32_MIN;
    for (int r = tid; r < own_n; r += NT) {
      const int64_t i = own0 + r;
      if (i < own_len) { const int s = own[i]; lo = min(lo, s); hi = max(hi, s); }
    }
    lo = wave_min_i(lo);
    hi = wave_max_i(hi);
    if (lane == 0) { atomicMin(&sb.qmin, lo); atomicMax(&sb.qmax, hi); }
  }
  __syncthreads();
  const int qmin = sb.qmin, qmax = sb.qmax;
  const int64_t n_other = (int64_t)n_tiles * BT;
  for (int64_t base = (int64_t)wave * 64 * KPL; base < n_other; base += (int64_t)W * 64 * KPL) {
    const int64_t k0 = base + (int64_t)lane * KPL;
    int v[KPL];
#pragma unroll
    for (int e = 0; e < KPL; ++e) v[e] = (k0 + e < other_len) ? other[k0 + e] : qmin;
    int lo = INT32_MAX, hi = INT32_MIN;
    const int nvalid = (int)max((int64_t)0, min((int64_t)KPL, other_len - k0));
#pragma unroll
    for (int e = 0; e < KPL; ++e) {
      if (e < nvalid) { lo = min(lo, v[e]); hi = max(hi, v[e]); }
    }
#pragma unroll
    for (int s = 1; s < LPT; s <<= 1) {
      lo = min(lo, __shfl_xor(lo, s));
      hi = max(hi, __shfl_xor(hi, s));
    }
    const int64_t t = k0 / BT;
    if ((lane % LPT) == 0 && t < n_tiles && lo <= hi) {
      if (lo <= qmax && hi >= qmin) atomicOr(&sb.vis[t >> 5], 1u << (t & 31));
      if (lo == hi && qmin == qmax && lo == qmin) atomicOr(&sb.full[t >> 5], 1u << (t & 31));
    }
  }
  __syncthreads();
}

// The forward's use: own = the workgroup's query rows, scanned = key tiles of BK.
template <int W, int BK>
__device__ void seg_scan(SegBits& sb, const FwdParams& p, const Work& w, int n_tiles) {
  seg_scan_ids<W * 64, BK>(sb, p.seg_q + (int64_t)w.b * p.Lq, w.p0, p.ppc, p.Lq, p.seg_k + (int64_t)w.b * p.Lk,
                           p.Lk, n_tiles);
}

// First visible tile index >= t (n_tiles if none).
__device__ __forceinline__ int seg_next(const SegBits& sb, int t, int n_tiles) {
  while (t < n_tiles) {
    unsigned m = sb.vis[t >> 5] >> (t & 31);
    if (m) return t + __builtin_ctz(m);
    t = (t | 31) + 1;
  }
  return n_tiles;
}

// Last visible tile index <= t and >= lo (lo - 1 if none).
__device__ __forceinline__ int seg_prev(const SegBits& sb, int t, int lo) {
  while (t >= lo) {
    const unsigned m = sb.vis[t >> 5] << (31 - (t & 31));
    if (m) {
      const int r = t - __builtin_clz(m);
      return r >= lo ? r : lo - 1;
    }
    t = (t & ~31) - 1;
  }
  return lo - 1;
}

}  // namespace gqa
