// fwd_bf16.hpp -- causal grouped-query attention forward, bf16 inputs, fp32
// accumulation, on gfx950 bf16 MFMA (v_mfma_f32_32x32x16_bf16).
//
// One workgroup = 4 waves, one per SIMD. For Hq/Hkv = 4 the workgroup owns the
// 4 query heads of one KV head x 32 positions; each wave owns one head and 32
// query rows. Q stays in VGPRs (64 per lane) and the O^T accumulator in AGPRs
// (128 per lane). Key tiles of 32 keys flow HBM -> LDS through a 4-stage ring
// (async global_load_lds, two tiles in flight ahead of use), each tile read by
// all 4 waves, so every K/V byte fetched serves each query head of the group;
// K/V are never repeated per head.
//
// The 32-row MFMA tile matters on this chip: an LDS fragment of 1 KB (32 keys
// x 16 d of K, or 32 d x 16 keys of V) feeds a 32x32x16 product, so the LDS
// bytes read per flop are half those of 16-row tiles and the LDS stays below
// the matrix core's rate.
//
// Per wave and key tile j (scores of tile j already in registers, with their
// row max folded into the running max):
//   A: S^T(j+1) = K(j+1) Q^T (A operand = K from LDS, B operand = Q; a lane
//      holds one query row, lane % 32, and 16 of the 32 keys) interleaved with
//      P = exp2(...) of tile j rounded to bf16 (RNE), l from the unrounded p
//      (for lse) and lr from the rounded P (for O, so O is an exact convex
//      combination of V rows);
//   B: O^T += V^T P^T (A operand = V^T through the transposing LDS read
//      ds_read_b64_tr_b16, B operand = P straight from the S^T registers)
//      interleaved with the mask and row max of tile j+1 and the lazy update
//      of the running max (it moves only when a row's maximum grows by more
//      than 8 in log2 units, so O and l are rescaled rarely and p <= 2^8).
// Masks (diagonal, ragged tail, segment boundaries) are applied only to the
// tiles that need them. O^T keeps one query row per lane, so the rescale and
// the final 1/lr are lane-local.
#pragma once
#include "common.hpp"

namespace gqa {

constexpr int kWavesB = 4;                  // waves per workgroup (one per SIMD)
constexpr int kRowsB = 32;                  // query rows per wave
constexpr int kBkB = 32;                    // keys per LDS tile
constexpr int kStagesB = 4;                 // LDS ring depth
constexpr int kTileBytesB = kBkB * kD * 2;  // 16 KB per K or V tile
constexpr int kCopiesB = 2 * kTileBytesB / 1024 / kWavesB;  // 16-byte-per-lane copies per wave and tile
constexpr float kLazy = 8.0f;               // lazy-rescale threshold (log2 units)

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// LDS image of a bf16 tile: 512-byte key rows of 32 16-byte chunks; chunk c of
// key k is stored at chunk c ^ swz_k(k) in K tiles and c ^ swz_v(k) in V tiles.
// LDS has 64 banks of 4 bytes (16 chunks). A K read (16 B per lane) serves 16
// lanes per clock, 16 consecutive keys at one chunk: an XOR by k % 16 puts them
// on 16 different chunks. A transposing V read (8 B per lane) serves 32 lanes
// per clock, 4 consecutive keys x 64 bytes (4 chunks) of d: an XOR by
// 4 (k % 4) puts the 4 keys on 4 different chunk quads.
__device__ __forceinline__ int swz_k(int key) { return key & 15; }
__device__ __forceinline__ int swz_v(int key) { return (key & 3) << 2; }

struct SmemB {
  __attribute__((aligned(16))) char k[kStagesB][kTileBytesB];
  __attribute__((aligned(16))) char v[kStagesB][kTileBytesB];
  __attribute__((aligned(16))) int segk[kStagesB][kBkB];
  SegBits bits;
};

__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  bf16x2 r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return __builtin_bit_cast(unsigned, r);
}

typedef __attribute__((address_space(3))) const char lds_cchar;

// Per-lane parts of the tile-copy and LDS-read addresses; the rest of each
// address is uniform or a compile-time immediate.
struct LanesB {
  uint32_t ldk[4];  // K copy it: byte offset (within the tile) of this lane's 16 bytes of block 4 wave + it
  uint32_t ldv[4];  // the same for V
  lds_cchar* k[8];  // K read, d chunk c (16 d), c % 8 = j: + 256 (c / 8)
  lds_cchar* v[4];  // V read, d block n (32 d), n % 4 = j: + 256 (n / 4) + 8192 h + 4096 jj
  // kbase/vbase: LDS byte addresses of the K and V ring regions (folded in, so a
  // read is one of these VGPRs plus a compile-time immediate)
  __device__ __forceinline__ void init(int wave, int lane, lds_cchar* kbase, lds_cchar* vbase) {
    const int l32 = lane & 31, g = lane >> 5;
    // copy block b = 4 wave + it (1 KB) holds keys 2 b and 2 b + 1; lane l
    // writes LDS chunk l % 32 of key 2 b + g, i.e. global chunk (l % 32) ^ swz(key)
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int blk = 4 * wave + it, key = 2 * blk + g;
      ldk[it] = (uint32_t)blk * 1024u + (uint32_t)g * 512u + ((uint32_t)(l32 ^ swz_k(key)) << 4);
      ldv[it] = (uint32_t)blk * 1024u + (uint32_t)g * 512u + ((uint32_t)(l32 ^ swz_v(key)) << 4);
    }
    // K read: key l32, chunk 2c + g
#pragma unroll
    for (int j = 0; j < 8; ++j) k[j] = kbase + l32 * 512 + (((2 * j + g) ^ swz_k(l32)) << 4);
    // V read (transposing, groups of 16 lanes): lane group q = lane / 16 takes
    // d half q % 2 and key quad q / 2; lane s of the group supplies key
    // 4 (q / 2) + s / 4 (+ 16 h + 8 jj) and d 32 n + 16 (q % 2) + 4 (s % 4) .. + 3.
    // Chunk 4 n + 2 (q % 2) + (s % 4) / 2 of a key with k % 4 = i is stored at
    // (4 n + ...) ^ 4 i = 4 (n ^ i) + ...
    const int q = lane >> 4, s = lane & 15, i = s >> 2;
    const int kr = 4 * (q >> 1) + i;
    const int cw = 2 * (q & 1) + ((s & 3) >> 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = vbase + kr * 512 + ((4 * (j ^ i) + cw) << 4) + ((s & 1) << 3);
  }
};

// Async copy of one key tile (keys 32t .. 32t+31) of K, V and the key
// segment ids into an LDS stage, issued piecewise between the products so the
// vector-memory pipe (which takes a CU's 32 KB per tile at about 64 bytes per
// clock) never stalls a wave's issue. Wave w copies the 1 KB blocks
// 4w .. 4w+3 (2 key rows each) of K and of V; the buffer resources end at Lk,
// so keys past it read as zeros (finite data that the mask removes).
struct TileCopy {
  rsrc_t rk, rv, rs;  // K, V, segment ids from the tile start
  uint32_t k_lds;     // LDS byte addresses of the stage's K, V and id regions
  uint32_t v_lds;
  uint32_t s_lds;
  __device__ __forceinline__ void k(const LanesB& ln, int it, int wave) const {
    buf2lds16(rk, ln.ldk[it], k_lds + (uint32_t)(4 * wave + it) * 1024u);
  }
  __device__ __forceinline__ void v(const LanesB& ln, int it, int wave) const {
    buf2lds16(rv, ln.ldv[it], v_lds + (uint32_t)(4 * wave + it) * 1024u);
  }
  __device__ __forceinline__ void seg(int wave, int lane) const {
    if (wave == kWavesB - 1) {  // uniform
      if (lane < kBkB) buf2lds4(rs, (uint32_t)lane * 4u, s_lds);
    }
  }
};

// LDS byte addresses of stage 0 of the K, V and id rings (taken once; a
// stage's address is these plus a multiple of its size).
struct RingBase {
  uint32_t k, v, s;
};

__device__ __forceinline__ TileCopy tile_copy(const RingBase& rb, int st, const char* kb, const char* vb,
                                              const int32_t* skb, int64_t t, int64_t Lk) {
  const int64_t keys = min((int64_t)kBkB, Lk - t * kBkB);  // >= 1 for every tile that is copied
  TileCopy c;
  c.rk = make_rsrc(kb + t * kTileBytesB, (uint32_t)keys * (kD * 2));
  c.rv = make_rsrc(vb + t * kTileBytesB, (uint32_t)keys * (kD * 2));
  c.rs = make_rsrc(skb != nullptr ? skb + t * kBkB : nullptr, skb != nullptr ? (uint32_t)keys * 4u : 0u);
  c.k_lds = rb.k + (uint32_t)st * kTileBytesB;
  c.v_lds = rb.v + (uint32_t)st * kTileBytesB;
  c.s_lds = rb.s + (uint32_t)st * (kBkB * 4);
  return c;
}

// The whole tile at once (prologue).
__device__ __forceinline__ void load_tile_b(const RingBase& rb, int st, const char* kb, const char* vb,
                                            const int32_t* skb, int64_t t, int64_t Lk, int wave, int lane,
                                            const LanesB& ln) {
  const TileCopy c = tile_copy(rb, st, kb, vb, skb, t, Lk);
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    c.k(ln, it, wave);
    c.v(ln, it, wave);
  }
  if (skb != nullptr) c.seg(wave, lane);
}

typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((address_space(3))) const i32x4 lds_i32x4;

// Online-softmax state of the wave's rows (per lane: its row). l sums the
// unrounded p (for lse), lr the bf16-rounded P that the PV product uses.
struct RowState {
  float m;      // running max, base-2 scaled domain (-inf before any visible key)
  float m_use;  // m, or 0 while m is -inf (so exp2(-inf - m_use) = 0)
  float l;      // this lane's partial sum of p (its 16 of every 32 keys)
  float lr;     // the same over the rounded P
};

// Element mask of one tile: lane holds keys key0 + 8 j + 4 g + i (s[4 j + i])
// of row `row`; segk_lane points at the stage's key ids + 4 g.
__device__ __forceinline__ void mask_tile(f32x16& s, int64_t key0, int g, int64_t Lk, int causal, int64_t lim,
                                          bool seg_elem, lds_cchar* segk_lane, int sq) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int kk = 8 * j + 4 * g;
    i32x4 ids = {0, 0, 0, 0};
    if (seg_elem) ids = *(lds_i32x4*)(segk_lane + 32 * j);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t key = key0 + kk + i;
      bool vis = key < Lk;
      if (causal) vis = vis && key <= lim;
      if (seg_elem) vis = vis && ids[i] == sq;
      s[4 * j + i] = vis ? s[4 * j + i] : -INFINITY;
    }
  }
}

// The lazy update of the running max from a tile's row max mx (raw scores;
// -inf for a fully masked row). Returns the per-lane rescale factor alpha (1
// where the max did not move).
__device__ __forceinline__ float lazy_max_update(float mx, RowState& rs, float sl2) {
  const float mxs = mx * sl2;
  const bool need = mxs > rs.m + kLazy;
  const float m_new = need ? mxs : rs.m;
  const float alpha = need ? fast_exp2(rs.m - m_new) : 1.f;
  rs.m = m_new;
  rs.m_use = (m_new == -INFINITY) ? 0.f : m_new;
  return alpha;
}

// Row max of a tile (the lanes l and l ^ 32 share a row) and the lazy update.
__device__ __forceinline__ float softmax_max(const f32x16& s, RowState& rs, float sl2) {
  float mx = fmaxf(s[0], s[1]);
#pragma unroll
  for (int r = 2; r < 16; ++r) mx = fmaxf(mx, s[r]);
  return lazy_max_update(xor32_max(mx), rs, sl2);
}

// One step of the exps: P for scores s[2u], s[2u+1] as one bf16 pair (the
// PV B operand of key half h takes pairs 4 h .. 4 h + 3) and the sums.
__device__ __forceinline__ void exp_pair(const f32x16& s, int u, float sl2, float m_use, unsigned* pk, float& lsum,
                                         float& lrsum) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  const float a = fast_exp2(fmaf(s[2 * u], sl2, -m_use));
  const float b = fast_exp2(fmaf(s[2 * u + 1], sl2, -m_use));
  pk[u] = pack_bf16(a, b);
  lsum += a + b;
  lrsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[u]), ones, lrsum, false);
}

// V^T fragment for d block n (32 d) and key half h: keys 16 h + 4 g + 0..3
// then 16 h + 8 + 4 g + 0..3 (g = lane / 32), d 32 n + lane % 32.
__device__ __forceinline__ bf16x8 v_frag(int n, int h, lds_cchar* const* vb) {
  lds_cchar* a = vb[n & 3] + ((n >> 2) * 256 + h * 8192);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)a);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a + 4096));
  const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
  return __builtin_bit_cast(bf16x8, u32x4{lo2[0], lo2[1], hi2[0], hi2[1]});
}

// The exps of one tile, software-pipelined over the products that hide them:
// at slot e the argument of score e is formed, the exp of score e - 1 taken
// and score e - 2 summed (and paired and rounded), so no VALU instruction waits
// on the result of the one before it (the wave issues in order, and an exp
// result takes several cycles); slots 16 and 17 drain the pipeline. P pairs
// 0..3 (key half 0) are complete after slot 9, pairs 4..7 after slot 17.
struct ExpPipe {
  float t[16], x[16];
  float lsum = 0.f, lrsum = 0.f;
  __device__ __forceinline__ void slot(int e, const f32x16& s, float sl2, float m_use, unsigned* pk) {
    if (e < 16) t[e] = fmaf(s[e], sl2, -m_use);
    if (e >= 1 && e <= 16) x[e - 1] = fast_exp2(t[e - 1]);
    if (e >= 2) {
      const int f = e - 2;
      lsum += x[f];
      if (f & 1) {
        const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
        pk[f >> 1] = pack_bf16(x[f - 1], x[f]);
        lrsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[f >> 1]), ones, lrsum, false);
      }
    }
  }
};

// Each product and the work placed beside it form one scheduling segment
// (the compiler's scheduling barrier keeps the segments in source order, so
// the exps stay spread over the products instead of bunching up).
#define GQA_SEGMENT_END() __builtin_amdgcn_sched_barrier(0)

// V fragments of phase B kept in flight (an LDS read takes several products'
// time under load); the first kVPre are read during phase A.
constexpr int kVPre = 6;

// Phase A: S^T(next) = K Q^T for the tile in ring stage st (16 MFMAs over
// D = 256, a dependent chain; K fragments read three MFMAs ahead) with slots
// 0..15 of the current tile's exps, and the K part of the tile copy three
// ahead (a CU's vector-memory pipe takes about 64 bytes per clock, so the
// copies are spread too).
__device__ __forceinline__ void phase_a(int st, const bf16x8* qf, const LanesB& ln, f32x16& s_nxt,
                                        const f32x16& s_cur, float sl2, float m_use, unsigned* pk, ExpPipe& ep,
                                        const TileCopy& tc, int wave, lds_cchar* const* vb, bf16x8* vf) {
  lds_cchar* kb[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) kb[j] = ln.k[j] + st * kTileBytesB;
  auto kfrag = [&](int c) { return *(lds_bf16x8*)(kb[c & 7] + (c >> 3) * 256); };
  bf16x8 kf[3];
#pragma unroll
  for (int c = 0; c < 3; ++c) kf[c] = kfrag(c);
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    s_nxt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[c % 3], qf[c], c == 0 ? f32x16{} : s_nxt, 0, 0, 0);
    if (c + 3 < 16) kf[c % 3] = kfrag(c + 3);
    ep.slot(c, s_cur, sl2, m_use, pk);
    if ((c & 3) == 1) tc.k(ln, c >> 2, wave);
    if (c >= 16 - kVPre) vf[c - (16 - kVPre)] = v_frag(c - (16 - kVPre), 0, vb);  // first PV fragments
    GQA_SEGMENT_END();
  }
  // Anchor the slot results in this block: their users lie past the mask
  // branch, and the compiler would otherwise sink the exps down to them.
  asm volatile("" ::"v"(pk[0]), "v"(pk[1]), "v"(pk[2]), "v"(pk[3]), "v"(pk[4]), "v"(pk[5]), "v"(pk[6]),
               "v"(ep.t[15]), "v"(ep.x[14]), "v"(ep.lsum), "v"(ep.lrsum));
}

// QK alone (the first tile of a row block).
__device__ __forceinline__ void qk_only(int st, const bf16x8* qf, const LanesB& ln, f32x16& s) {
  lds_cchar* kb[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) kb[j] = ln.k[j] + st * kTileBytesB;
  auto kfrag = [&](int c) { return *(lds_bf16x8*)(kb[c & 7] + (c >> 3) * 256); };
  bf16x8 kf[3];
#pragma unroll
  for (int c = 0; c < 3; ++c) kf[c] = kfrag(c);
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[c % 3], qf[c], c == 0 ? f32x16{} : s, 0, 0, 0);
    if (c + 3 < 16) kf[c % 3] = kfrag(c + 3);
  }
}

// O^T *= alpha where some row's max moved. The products stay in AGPRs, where
// the PV products keep O (the empty asm pins them there; without it the
// compiler keeps O in VGPRs around the loop and copies it into AGPRs before
// every PV product).
__device__ __forceinline__ void rescale(f32x16* acc, RowState& rs, float alpha) {
  if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      acc[n] *= alpha;
      asm volatile("" : "+a"(acc[n]));
    }
  }
  rs.l *= alpha;
  rs.lr *= alpha;
}

// Wait until at most one tile's worth (8 copies) of this wave's async copies
// is outstanding (copies complete in issue order; the wave that also copies
// segment ids issues one more per tile, which only makes the wait stricter).
__device__ __forceinline__ void wait_one_tile_outstanding() {
  static_assert(kCopiesB == 8, "the vmcnt immediate assumes 8 copies per tile");
  asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
}

// Everything one workgroup's wave needs inside the tile loop.
template <bool SEG>
struct Bf16Wave {
  const FwdParams& p;
  SmemB& sm;
  LanesB ln;
  bf16x8 qf[16];
  f32x16 acc[8];
  f32x16 s_cur;
  RowState rs;
  const char* kb;
  const char* vb;
  const int32_t* skb;
  int64_t pw, lim;
  int wave, lane, g, sq, n_tiles;
  bool use_bits;
  int cur, nxt, nn;  // visible tiles: being finished, QK this step, in flight
  RingBase rb;

  __device__ __forceinline__ Bf16Wave(const FwdParams& p_, SmemB& sm_) : p(p_), sm(sm_) {}

  __device__ __forceinline__ int next_tile(int t) const {
    if (t >= n_tiles) return n_tiles;
    if constexpr (SEG) return use_bits ? seg_next(sm.bits, t + 1, n_tiles) : t + 1;
    return t + 1;
  }
  // Tiles past the last visible one are still copied (the last tile again, into
  // a stage that is never read), so every step waits for the same copy count.
  __device__ __forceinline__ void load(int st, int t) {
    load_tile_b(rb, st, kb, vb, SEG ? skb : nullptr, min(t, n_tiles - 1), p.Lk, wave, lane, ln);
  }
  __device__ __forceinline__ TileCopy copier(int st, int t) {
    return tile_copy(rb, st, kb, vb, SEG ? skb : nullptr, min(t, n_tiles - 1), p.Lk);
  }
  __device__ __forceinline__ bool full_bit(int t) const {
    return SEG && use_bits && ((sm.bits.full[t >> 5] >> (t & 31)) & 1u);
  }
  __device__ __forceinline__ void mask_if_needed(f32x16& s, int t, int st) {
    const int64_t k0 = (int64_t)t * kBkB;
    const bool seg_elem = SEG && !full_bit(t);
    if (seg_elem || k0 + kBkB > p.Lk || (p.causal && k0 + kBkB - 1 > p.q_offset + pw))
      mask_tile(s, k0, g, p.Lk, p.causal, lim, seg_elem, (lds_cchar*)sm.segk[st] + 16 * g, sq);
  }

  // Phase B: O^T += V^T P^T for the tile in stage st (16 MFMAs, V fragments
  // read three MFMAs ahead) with the last exp slots of this tile, the row max
  // of the next scores s_nxt (masked first where needed) spread over the
  // products, the lazy update of the running max, and the V part of the tile
  // copy. Returns alpha.
  __device__ __forceinline__ float phase_b(int st1, f32x16& s_nxt, unsigned* pk, ExpPipe& ep, const TileCopy& tc,
                                           lds_cchar* const* vb, bf16x8* vf) {
    const float sl2 = p.scale_log2;
    const float m_cur = rs.m_use;
    mask_if_needed(s_nxt, nxt, st1);
    const bf16x8 p0 = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
    bf16x8 p1;
    float mx = -INFINITY, alpha = 1.f;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      if (u == 8) p1 = __builtin_bit_cast(bf16x8, u32x4{pk[4], pk[5], pk[6], pk[7]});
      acc[u & 7] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[u % kVPre], u < 8 ? p0 : p1, acc[u & 7], 0, 0, 0);
      if (u + kVPre < 16) vf[u % kVPre] = v_frag((u + kVPre) & 7, (u + kVPre) >> 3, vb);
      if (u < 2) ep.slot(16 + u, s_cur, sl2, m_cur, pk);
      if (u >= 2 && u < 10) mx = fmaxf(mx, fmaxf(s_nxt[2 * (u - 2)], s_nxt[2 * (u - 2) + 1]));
      if (u == 11) mx = xor32_max(mx);
      if (u == 13) alpha = lazy_max_update(mx, rs, sl2);
      if ((u & 3) == 1) tc.v(ln, u >> 2, wave);
      if (SEG && u == 3) tc.seg(wave, lane);
      GQA_SEGMENT_END();
    }
    rs.l += ep.lsum;
    rs.lr += ep.lrsum;
    return alpha;
  }

  // The last tile: its exps, then its PV product.
  __device__ __forceinline__ void finish(int st) {
    unsigned pk[8];
    float lsum = 0.f, lrsum = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) exp_pair(s_cur, u, p.scale_log2, rs.m_use, pk, lsum, lrsum);
    rs.l += lsum;
    rs.lr += lrsum;
    lds_cchar* vb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) vb[j] = ln.v[j] + st * kTileBytesB;
    const bf16x8 p0 = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
    const bf16x8 p1 = __builtin_bit_cast(bf16x8, u32x4{pk[4], pk[5], pk[6], pk[7]});
#pragma unroll
    for (int u = 0; u < 16; ++u)
      acc[u & 7] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_frag(u & 7, u >> 3, vb), u < 8 ? p0 : p1,
                                                           acc[u & 7], 0, 0, 0);
  }

  // One step with `cur` in stage st: returns false after finishing the last tile.
  __device__ __forceinline__ bool step(int st) {
    if (nxt >= n_tiles) {
      finish(st);
      return false;
    }
    const int st1 = (st + 1) & 3, st3 = (st + 3) & 3;
    wait_one_tile_outstanding();  // tile nxt has landed (nn may still be in flight)
    __syncthreads();              // ... for every wave; and stage st3 is free
    const int n3 = next_tile(nn);
    const TileCopy tc = copier(st3, n3);
    unsigned pk[8];
    ExpPipe ep;
    f32x16 s_nxt;
    lds_cchar* vb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) vb[j] = ln.v[j] + st * kTileBytesB;
    bf16x8 vf[kVPre];
    phase_a(st1, qf, ln, s_nxt, s_cur, p.scale_log2, rs.m_use, pk, ep, tc, wave, vb, vf);
    const float alpha = phase_b(st1, s_nxt, pk, ep, tc, vb, vf);
    rescale(acc, rs, alpha);
    s_cur = s_nxt;
    cur = nxt;
    nxt = nn;
    nn = n3;
    return true;
  }
};

template <bool SEG>
__global__ __launch_bounds__(kWavesB * 64) void fwd_bf16_kernel(FwdParams p) {
  __shared__ SmemB sm;
  Bf16Wave<SEG> wv(p, sm);
  const Work w = decode_work(p);
  wv.wave = wave_id();
  wv.lane = lane_id();
  const int l32 = wv.lane & 31;
  wv.g = wv.lane >> 5;
  const int h = w.h0 + wv.wave % p.hpc;
  wv.pw = w.p0 + (int64_t)(wv.wave / p.hpc) * kRowsB;  // first row of this wave
  const int64_t row = wv.pw + l32;
  const int64_t row_c = min(row, p.Lq - 1);

  const int64_t p_end = min(w.p0 + (int64_t)p.ppc, p.Lq);
  const int64_t kv_end = p.causal ? min(p.Lk, p.q_offset + p_end) : p.Lk;
  wv.n_tiles = (int)((kv_end + kBkB - 1) / kBkB);

  wv.use_bits = SEG && wv.n_tiles <= kMaxSegTiles;
  if (SEG && wv.use_bits) seg_scan<kWavesB, kBkB>(sm.bits, p, w, wv.n_tiles);

  const int64_t kv_head = (int64_t)w.b * p.Hkv + w.kvh;
  wv.kb = (const char*)p.k + kv_head * p.Lk * kD * 2;
  wv.vb = (const char*)p.v + kv_head * p.Lk * kD * 2;
  wv.skb = SEG ? p.seg_k + (int64_t)w.b * p.Lk : nullptr;
  wv.sq = SEG ? p.seg_q[(int64_t)w.b * p.Lq + row_c] : 0;
  wv.lim = p.q_offset + row;  // last key this row may see (causal)

  // Q in registers, B-operand layout: lane holds Q[row][16 c + 8 g .. + 7].
  const int64_t hq = ((int64_t)w.b * p.Hq + h) * p.Lq;
  {
    const bf16x8* qr = (const bf16x8*)((const char*)p.q + (hq + row_c) * kD * 2);
#pragma unroll
    for (int c = 0; c < 16; ++c) wv.qf[c] = qr[2 * c + wv.g];
  }
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    wv.acc[n] = f32x16{};
    asm volatile("" : "+a"(wv.acc[n]));
  }
  wv.rs = RowState{-INFINITY, 0.f, 0.f, 0.f};
  wv.ln.init(wv.wave, wv.lane, (lds_cchar*)sm.k[0], (lds_cchar*)sm.v[0]);
  wv.rb = RingBase{lds_addr(sm.k[0]), lds_addr(sm.v[0]), lds_addr(sm.segk[0])};

  wv.cur = SEG && wv.use_bits ? seg_next(sm.bits, 0, wv.n_tiles) : 0;
  if (wv.cur < wv.n_tiles) {
    wv.nxt = wv.next_tile(wv.cur);
    wv.nn = wv.next_tile(wv.nxt);
    wv.load(0, wv.cur);
    wv.load(1, wv.nxt);
    wv.load(2, wv.nn);
    asm volatile("s_waitcnt vmcnt(16)" ::: "memory");  // tile cur has landed
    __syncthreads();
    qk_only(0, wv.qf, wv.ln, wv.s_cur);
    wv.mask_if_needed(wv.s_cur, wv.cur, 0);
    (void)softmax_max(wv.s_cur, wv.rs, p.scale_log2);  // nothing accumulated yet: no rescale
    for (int st = 0; wv.step(st); st = (st + 1) & 3) {
    }
  }

  // epilogue: O = acc / lr (bf16), lse = ln2 (m + log2 l); lane holds
  // O[row][32 n + 8 j + 4 g + i] in acc[n][4 j + i]
#pragma unroll
  for (int n = 0; n < 8; ++n) asm volatile("" : "+a"(wv.acc[n]));
  const float l_tot = xor32_sum(wv.rs.l);
  const float lr_tot = xor32_sum(wv.rs.lr);
  if (row < p.Lq) {
    const float inv = lr_tot > 0.f ? 1.f / lr_tot : 0.f;
    char* op = (char*)p.o + (hq + row) * kD * 2;
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x2 val = {pack_bf16(wv.acc[n][4 * j] * inv, wv.acc[n][4 * j + 1] * inv),
                           pack_bf16(wv.acc[n][4 * j + 2] * inv, wv.acc[n][4 * j + 3] * inv)};
        *(u32x2*)(op + (32 * n + 8 * j + 4 * wv.g) * 2) = val;
      }
    if (wv.g == 0)
      p.lse[hq + row] = l_tot > 0.f ? (wv.rs.m_use + log2f(l_tot)) * 0.69314718055994530942f : -INFINITY;
  }
}

}  // namespace gqa
