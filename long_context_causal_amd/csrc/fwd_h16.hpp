// fwd_h16.hpp -- causal grouped-query attention forward for 16-bit inputs
// (bf16 or fp16), fp32 accumulation, on gfx950 MFMA (v_mfma_f32_32x32x16_bf16
// / _f16). The element type only changes the products' opcode and the
// conversions to it (round to nearest even); the layouts are the same.
//
// One workgroup = 4 waves, one per SIMD. For Hq/Hkv = 4 the workgroup owns the
// 4 query heads of one KV head x 32 positions; each wave owns one head and 32
// query rows. Q stays in VGPRs (64 per lane) and the O^T accumulator in AGPRs
// (128 per lane). Key tiles of 64 keys flow HBM -> LDS once per workgroup and
// are read by all 4 waves, so every K/V byte fetched serves each query head of
// the group; K/V are never repeated per head.
//
// The 32-row MFMA tile matters on this chip: an LDS fragment of 1 KB (32 keys
// x 16 d of K, or 32 d x 16 keys of V) feeds a 32x32x16 product, so the LDS
// bytes read per flop are half those of 16-row tiles and the LDS stays below
// the matrix core's rate.
//
// Per wave and step i (visible tile #i: its scores already in registers, with
// their row max folded into the running max):
//   A: S^T(#i+1) = K(#i+1) Q^T (A operand = K from LDS, B operand = Q; a lane
//      holds one query row, lane % 32, and 32 of the 64 keys) interleaved with
//      P = exp2(...) of tile #i rounded to bf16 (RNE), l from the unrounded p
//      (for lse) and lr from the rounded P (for O, so O is an exact convex
//      combination of V rows);
//   B: O^T += V^T P^T of tile #i (A operand = V^T through the transposing LDS
//      read ds_read_b64_tr_b16, B operand = P straight from the S^T registers)
//      interleaved with the mask and row max of tile #i+1 and the lazy update
//      of the running max (it moves only when a row's maximum grows by more
//      than 8 in log2 units, so O and l are rescaled rarely and p <= 2^8).
// K of a tile is read only in phase A one step ahead, V only in phase B of its
// own step, so K and V have rings of their own, two stages each: in step i
// the copies of K(#i+2) and V(#i+1) refill the stages that K(#i) and V(#i-1)
// left, and one workgroup barrier per step covers both. The copies are spread
// between the products (a CU's vector-memory pipe takes about 64 bytes per
// clock, and a wave issues in order). Masks (diagonal, ragged tail, segment
// boundaries) are applied only to the tiles that need them. O^T keeps one
// query row per lane, so the rescale and the final 1/lr are lane-local.
#pragma once
#include "common.hpp"
#include "elem16.hpp"

namespace gqa {

constexpr int kWavesB = 4;                  // waves per workgroup (one per SIMD)
constexpr int kRowsB = 32;                  // query rows per wave
constexpr int kBkB = 64;                    // keys per LDS tile
constexpr int kTileBytesB = kBkB * kD * 2;  // 32 KB per K or V tile
constexpr int kCopiesB = kTileBytesB / 1024 / kWavesB;  // 1 KB copies per wave for the K (or V) part of a tile
constexpr float kLazy = 8.0f;               // lazy-rescale threshold (log2 units)
constexpr int kVPre = 6;                    // V fragments in flight in phase B (the first read in phase A)

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
  __attribute__((aligned(16))) char k[2][kTileBytesB];
  __attribute__((aligned(16))) char v[2][kTileBytesB];
  __attribute__((aligned(16))) int segk[2][kBkB];  // key segment ids, staged with K
  SegBits bits;
};

typedef __attribute__((address_space(3))) const char lds_cchar;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((address_space(3))) const i32x4 lds_i32x4;

// Per-lane parts of the tile-copy and LDS-read addresses; the rest of each
// address is uniform or a compile-time immediate.
struct LanesB {
  uint32_t ldk[kCopiesB];  // K copy it: byte offset (within the tile) of this lane's 16 bytes of block 8 wave + it
  uint32_t ldv[kCopiesB];  // the same for V
  lds_cchar* k[8];         // K read, d chunk c (16 d), c % 8 = j: + 256 (c / 8) + 16384 (key half)
  lds_cchar* v[4];         // V read, d block n (32 d), n % 4 = j: + 256 (n / 4) + 8192 (key quarter) + 4096 jj
  // kbase/vbase: LDS byte addresses of the K and V rings (folded in, so a read
  // is one of these VGPRs plus a compile-time immediate)
  __device__ __forceinline__ void init(int wave, int lane, lds_cchar* kbase, lds_cchar* vbase) {
    const int l32 = lane & 31, g = lane >> 5;
    // copy block b = 8 wave + it (1 KB) holds keys 2 b and 2 b + 1; lane l
    // writes LDS chunk l % 32 of key 2 b + g, i.e. global chunk (l % 32) ^ swz(key)
#pragma unroll
    for (int it = 0; it < kCopiesB; ++it) {
      const int blk = kCopiesB * wave + it, key = 2 * blk + g;
      ldk[it] = (uint32_t)blk * 1024u + (uint32_t)g * 512u + ((uint32_t)(l32 ^ swz_k(key)) << 4);
      ldv[it] = (uint32_t)blk * 1024u + (uint32_t)g * 512u + ((uint32_t)(l32 ^ swz_v(key)) << 4);
    }
    // K read: key l32 (+ 32 per key half), chunk 2c + g
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

// LDS byte addresses of the K, V and id rings (taken once; a stage's address is
// these plus a multiple of its size).
struct RingBase {
  uint32_t k, v, s;
};

// Async copy of one part (K with its key segment ids, or V) of key tile t
// (keys 64t .. 64t+63) into an LDS stage. Wave w copies the 1 KB blocks
// 8w .. 8w+7 (2 key rows each). The buffer resource ends at Lk, so keys past it
// read as zeros (finite data that the mask removes); a resource of size 0 (no
// tile) writes only zeros.
struct PartCopy {
  rsrc_t r, rs;    // rows (K or V) and key ids from the tile start
  uint32_t lds;    // LDS stage
  uint32_t s_lds;  // LDS stage of the ids
  __device__ __forceinline__ void rows(const uint32_t* ld, int it, int wave) const {
    buf2lds16_imm(r, ld[it], lds + (uint32_t)(kCopiesB * wave) * 1024u, (uint32_t)it * 1024u);
  }
  __device__ __forceinline__ void ids(int wave, int lane) const {
    if (wave == kWavesB - 1) buf2lds4(rs, (uint32_t)lane * 4u, s_lds);  // uniform branch; 64 ids
  }
};

// Key counts in 32 bits: Lk < 2^31 (the entry point checks it), and a valid
// tile starts below Lk. The tile's byte offset needs 64 bits.
__device__ __forceinline__ PartCopy part_copy(uint32_t lds, uint32_t s_lds, const char* base, const int32_t* skb,
                                              int t, bool valid, int64_t Lk) {
  const uint32_t rem = (uint32_t)Lk - (uint32_t)t * (uint32_t)kBkB;
  const uint32_t keys = valid ? min(rem, (uint32_t)kBkB) : 0u;
  const uint64_t tv = valid ? (uint64_t)(uint32_t)t : 0u;
  PartCopy c;
  c.r = make_rsrc(base + tv * kTileBytesB, keys * (kD * 2));
  c.rs = make_rsrc(skb != nullptr ? skb + tv * kBkB : nullptr, skb != nullptr ? keys * 4u : 0u);
  c.lds = lds;
  c.s_lds = s_lds;
  return c;
}

// V^T fragment for d block n (32 d) and key quarter h (16 keys) of a stage
// whose read bases are vb[]: keys 16 h + 4 g + 0..3 then 16 h + 8 + 4 g + 0..3
// (g = lane / 32), d 32 n + lane % 32.
template <typename V8>
__device__ __forceinline__ V8 v_frag(int n, int h, lds_cchar* const* vb) {
  lds_cchar* a = vb[n & 3] + ((n >> 2) * 256 + h * 8192);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)a);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a + 4096));
  const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
  return __builtin_bit_cast(V8, u32x4{lo2[0], lo2[1], hi2[0], hi2[1]});
}

// Online-softmax state of the wave's rows (per lane: its row). l sums the
// unrounded p (for lse), lr the bf16-rounded P that the PV product uses.
struct RowState {
  float m;      // running max, base-2 scaled domain (-inf before any visible key)
  float m_use;  // m, or 0 while m is -inf (so exp2(-inf - m_use) = 0)
  float l;      // this lane's partial sum of p (its 32 of every 64 keys)
  float lr;     // the same over the rounded P
};

// Element mask of one 32-key half of a tile: lane holds keys key0 + 8 j + 4 g + i
// (s[4 j + i]) of row `row`; segk_lane points at the half's key ids + 4 g.
__device__ __forceinline__ void mask_half(float* s, int64_t key0, int g, int64_t Lk, int causal, int64_t lim,
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

// Max of a tile's 32 scores in this lane (the lanes l and l ^ 32 share a row:
// the row max is xor32_max of it).
__device__ __forceinline__ float lane_max(const float* s) {
  float mx = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; ++r) mx = fmaxf(fmaxf(mx, s[r]), s[16 + r]);
  return mx;
}

// The exps of one tile (32 scores per lane), software-pipelined over the
// products that hide them: at slot e the argument of score e is formed, the
// exp of score e - 1 taken and score e - 2 summed (and paired and rounded), so
// no VALU instruction waits on the result of the one before it (the wave
// issues in order, and an exp result takes several cycles); slots 32 and 33
// drain the pipeline. Score e is s[e] (s[16 j + r] is element r of key half
// j); P pair f / 2 goes to pk, and key quarter h of the PV product takes
// pk[4 h .. 4 h + 3].
template <typename E>
struct ExpPipe {
  float t[32], x[32];
  float lsum = 0.f, lrsum = 0.f;
  __device__ __forceinline__ void slot(int e, const float* s, float sl2, float m_use, unsigned* pk) {
    if (e < 32) t[e] = fmaf(s[e], sl2, -m_use);
    if (e >= 1 && e <= 32) x[e - 1] = fast_exp2(t[e - 1]);
    if (e >= 2) {
      const int f = e - 2;
      lsum += x[f];
      if (f & 1) {
        pk[f >> 1] = Elem<E>::pack(x[f - 1], x[f]);
        lrsum = Elem<E>::sum2(pk[f >> 1], lrsum);
      }
    }
  }
};

// Each product and the work placed beside it form one scheduling segment (the
// compiler's scheduling barrier keeps the segments in source order, so the
// exps stay spread over the products instead of bunching up).
#define GQA_SEGMENT_END() __builtin_amdgcn_sched_barrier(0)

// QK product q (0..31) of a tile: key half q % 2, d chunk q / 2 (16 d); the
// two halves are independent chains, interleaved. K fragments are read three
// products ahead from a stage whose read bases are kb[].
template <typename V8>
__device__ __forceinline__ V8 k_frag(int q, lds_cchar* const* kb) {
  typedef __attribute__((address_space(3))) const V8 lds_v8;
  const int j = q & 1, c = q >> 1;
  return *(lds_v8*)(kb[c & 7] + ((c >> 3) * 256 + j * 16384));
}

// Phase A: S^T(next) = K Q^T for the tile in K stage kst (32 MFMAs over
// D = 256, two key halves) with slots 0..31 of the current tile's exps, the
// tile copies (K of the tile two ahead, V of the tile one ahead: early
// enough that they land before the next barrier), and the first V fragments
// of phase B (already resident). Q stays in AGPRs, where the products read it
// (the empty asm pins it there; the VGPRs go to the scores, P and fragments).
template <typename E>
__device__ __forceinline__ void phase_a(int kst, typename Elem<E>::v8* qf, const LanesB& ln, f32x16* s_nxt,
                                        const float* s_cur, float sl2, float m_use, unsigned* pk, ExpPipe<E>& ep,
                                        const PartCopy& kc, const PartCopy& vc, int wave, lds_cchar* const* vb,
                                        typename Elem<E>::v8* vf) {
  typedef typename Elem<E>::v8 V8;
  lds_cchar* kb[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) kb[j] = ln.k[j] + kst * kTileBytesB;
  V8 kf[3];
#pragma unroll
  for (int q = 0; q < 3; ++q) kf[q] = k_frag<V8>(q, kb);
#pragma unroll
  for (int q = 0; q < 32; ++q) {
    const int j = q & 1, c = q >> 1;
    if (j == 0) asm volatile("" : "+a"(qf[c]));
    s_nxt[j] = Elem<E>::mfma(kf[q % 3], qf[c], c == 0 ? f32x16{} : s_nxt[j]);
    if (q + 3 < 32) kf[q % 3] = k_frag<V8>(q + 3, kb);
    ep.slot(q, s_cur, sl2, m_use, pk);
    if ((q & 3) == 1) kc.rows(ln.ldk, q >> 2, wave);
    if ((q & 3) == 3) vc.rows(ln.ldv, q >> 2, wave);
    if (q >= 32 - kVPre) vf[q - (32 - kVPre)] = v_frag<V8>(q - (32 - kVPre), 0, vb);
    GQA_SEGMENT_END();
  }
  // Anchor the slot results in this block: their users lie past the mask
  // branch, and the compiler would otherwise sink the exps down to them.
  asm volatile("" ::"v"(pk[0]), "v"(pk[1]), "v"(pk[2]), "v"(pk[3]), "v"(pk[4]), "v"(pk[5]), "v"(pk[6]),
               "v"(pk[7]), "v"(pk[8]), "v"(pk[9]), "v"(pk[10]), "v"(pk[11]), "v"(pk[12]), "v"(pk[13]),
               "v"(pk[14]), "v"(ep.t[31]), "v"(ep.x[30]), "v"(ep.lsum), "v"(ep.lrsum));
}

// QK alone (the first tile of a row block).
template <typename E>
__device__ __forceinline__ void qk_only(int kst, const typename Elem<E>::v8* qf, const LanesB& ln, f32x16* s) {
  typedef typename Elem<E>::v8 V8;
  lds_cchar* kb[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) kb[j] = ln.k[j] + kst * kTileBytesB;
  V8 kf[3];
#pragma unroll
  for (int q = 0; q < 3; ++q) kf[q] = k_frag<V8>(q, kb);
#pragma unroll
  for (int q = 0; q < 32; ++q) {
    const int j = q & 1, c = q >> 1;
    s[j] = Elem<E>::mfma(kf[q % 3], qf[c], c == 0 ? f32x16{} : s[j]);
    if (q + 3 < 32) kf[q % 3] = k_frag<V8>(q + 3, kb);
  }
}

// O^T *= alpha where some row's max moved. The products stay in AGPRs, where
// the PV products keep O (the empty asm pins them there; without it the
// compiler keeps O in VGPRs around the loop and copies it into AGPRs before
// every PV product).
__device__ __forceinline__ void rescale(f32x16* acc, RowState& rs, float alpha) {
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0, 0)) {
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      acc[n] *= alpha;
      asm volatile("" : "+a"(acc[n]));
    }
  }
  rs.l *= alpha;
  rs.lr *= alpha;
}

// Everything one workgroup's wave needs inside the tile loop.
template <typename E, bool SEG>
struct H16Wave {
  typedef typename Elem<E>::v8 V8;
  const FwdParams& p;
  SmemB& sm;
  LanesB ln;
  RingBase rb;
  V8 qf[16];
  f32x16 acc[8];
  float s_cur[32];  // scores of the tile being finished, in VGPRs (see phase_b)
  RowState rs;
  const char* kb;
  const char* vb;
  const int32_t* skb;
  int64_t pw, lim;
  int wave, lane, g, sq, n_tiles;
  int sh;  // log2 of the key tiles per segment-map group
  int cur, nxt, nn;  // visible tiles: being finished, QK this step, next after that
  bool f_nxt, f_nn;  // their segment state: every key of the workgroup's one query id (no id mask)
  int vr_lo, vr_hi;  // the run of visible tiles at or after the last lookup
  int fr_lo, fr_hi;  // the run of full tiles at or after the last lookup

  __device__ __forceinline__ H16Wave(const FwdParams& p_, SmemB& sm_) : p(p_), sm(sm_) {}

  // The first visible tile after t (n_tiles if none). Calls come in increasing
  // t; the map is read only past the end of the current run.
  __device__ __forceinline__ int next_tile(int t) {
    const int u = t + 1;
    if (u >= n_tiles) return n_tiles;
    if constexpr (SEG) {
      if (u >= vr_hi) seg_run(sm.bits.vis, sh, u, n_tiles, vr_lo, vr_hi);
      return max(u, vr_lo);
    }
    return u;
  }
  // Is tile t full (no id mask needed)? Calls come in increasing t.
  __device__ __forceinline__ bool is_full(int t) {
    if constexpr (SEG) {
      if (t >= n_tiles) return false;
      if (t >= fr_hi) seg_run(sm.bits.full, sh, t, n_tiles, fr_lo, fr_hi);
      return t >= fr_lo;
    }
    return true;
  }
  __device__ __forceinline__ PartCopy k_copy(int st, int t) const {
    return part_copy(rb.k + (uint32_t)st * kTileBytesB, rb.s + (uint32_t)st * (kBkB * 4), kb, SEG ? skb : nullptr,
                     t, t < n_tiles, p.Lk);
  }
  __device__ __forceinline__ PartCopy v_copy(int st, int t) const {
    return part_copy(rb.v + (uint32_t)st * kTileBytesB, 0u, vb, nullptr, t, t < n_tiles, p.Lk);
  }
  // Masks the 32 scores per lane of tile t (s[16 j + r]: element r of key
  // half j; `full`: its segment state) where some key of the tile is hidden
  // from some row of the wave; returns whether it did.
  __device__ __forceinline__ bool mask_if_needed(float* s, int t, bool full, int st) {
    const int64_t k0 = (int64_t)t * kBkB;
    const bool seg_elem = SEG && !full;
    if (__builtin_expect(seg_elem || k0 + kBkB > p.Lk || (p.causal && k0 + kBkB - 1 > p.q_offset + pw), 0)) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
        mask_half(s + 16 * j, k0 + 32 * j, g, p.Lk, p.causal, lim, seg_elem,
                  (lds_cchar*)sm.segk[st] + 128 * j + 16 * g, sq);
      return true;
    }
    return false;
  }

  // Phase B: O^T += V^T P^T for the tile whose V fragments vf[] start in
  // flight (32 MFMAs: 4 key quarters x 8 d blocks, fragments read kVPre
  // products ahead) with the last exp slots of this tile, the row max of the
  // next scores s_nxt spread over the products, and the lazy update of the
  // running max. Returns alpha. The max pass is the one read of the scores
  // from the products' AGPRs: two per product, pinned in VGPRs and returned
  // in sn (the next step's exps take them from there). Where the tile needs a
  // mask (ids in K stage kst1), it applies to those VGPR copies and the lane
  // max is taken again: masking the AGPRs first would put all 32 reads in one
  // run at the start of the phase, the products starved behind them.
  __device__ __forceinline__ float phase_b(int kst1, const f32x16* s_nxt, unsigned* pk, ExpPipe<E>& ep,
                                           lds_cchar* const* vbs, V8* vf, float* sn) {
    const float sl2 = p.scale_log2;
    const float m_cur = rs.m_use;
    float mx = -INFINITY, alpha = 1.f;
    auto product = [&](int u) {
      const int n = u & 7, h = u >> 3;
      const V8 ph = __builtin_bit_cast(V8, u32x4{pk[4 * h], pk[4 * h + 1], pk[4 * h + 2], pk[4 * h + 3]});
      acc[n] = Elem<E>::mfma(vf[u % kVPre], ph, acc[n]);
      if (u + kVPre < 32) vf[u % kVPre] = v_frag<V8>((u + kVPre) & 7, (u + kVPre) >> 3, vbs);
      if (u < 2) ep.slot(32 + u, s_cur, sl2, m_cur, pk);
      if (u >= 2 && u < 18) {
        const int r = u - 2;
        float a0 = s_nxt[0][r], a1 = s_nxt[1][r];
        asm volatile("" : "+v"(a0), "+v"(a1));
        sn[r] = a0;
        sn[16 + r] = a1;
        mx = fmaxf(fmaxf(mx, a0), a1);
      }
      // a "next" tile past the range (the last step's, also the tile after a
      // key split) holds the zeros of its copy, no scores: its max stays -inf
      if (u == 19) mx = nxt < n_tiles ? xor32_max(mx) : -INFINITY;
      if (u == 21) alpha = lazy_max_update(mx, rs, sl2);
      GQA_SEGMENT_END();
    };
    // the mask sits between two unrolled loops, not inside one: inside, its
    // code (the segment-id form is large) counts in every iteration before
    // u == 18 is folded, and the loop would stay rolled
#pragma unroll
    for (int u = 0; u < 19; ++u) product(u);
    if (mask_if_needed(sn, nxt, f_nxt, kst1)) mx = lane_max(sn);
#pragma unroll
    for (int u = 19; u < 32; ++u) product(u);
    rs.l += ep.lsum;
    rs.lr += ep.lrsum;
    return alpha;
  }

  // One step with tile `cur` in stages (K, V) = i % 2. The step of the last
  // tile runs like the others: its "next" tile is past the end, copied as
  // zeros and fully masked (-inf scores leave the running max, and with it O,
  // unchanged), which costs one tile's QK products per workgroup and keeps a
  // single loop body.
  __device__ __forceinline__ void step(int i) {
    const int st = i & 1, st1 = st ^ 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // K(nxt) and V(cur), copied last step, have landed
    __syncthreads();                                    // ... for every wave; K stage st and V stage st1 are free
    const int n3 = next_tile(nn);
    const bool f3 = is_full(n3);
    const PartCopy kc = k_copy(st, nn);   // K(#i+2) into K(#i)'s stage
    const PartCopy vc = v_copy(st1, nxt);  // V(#i+1) into V(#i-1)'s stage
    // the key ids of K(#i+2), where that tile needs them (not full), go out
    // here rather than among the products: phase A is then the same code with
    // and without segment ids
    if (__builtin_expect(SEG && !f_nn, 0)) kc.ids(wave, lane);
    unsigned pk[16];
    ExpPipe<E> ep;
    f32x16 s_nxt[2];
    lds_cchar* vbs[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) vbs[j] = ln.v[j] + st * kTileBytesB;
    V8 vf[kVPre];
    phase_a<E>(st1, qf, ln, s_nxt, s_cur, p.scale_log2, rs.m_use, pk, ep, kc, vc, wave, vbs, vf);
    float sn[32];
    const float alpha = phase_b(st1, s_nxt, pk, ep, vbs, vf, sn);
    rescale(acc, rs, alpha);
#pragma unroll
    for (int r = 0; r < 32; ++r) s_cur[r] = sn[r];
    cur = nxt;
    nxt = nn;
    nn = n3;
    f_nxt = f_nn;
    f_nn = f3;
  }
};

template <typename E, bool SEG>
__global__ __launch_bounds__(kWavesB * 64) void fwd_h16_kernel(FwdParams p) {
  typedef typename Elem<E>::v8 V8;
  __shared__ SmemB sm;
  H16Wave<E, SEG> wv(p, sm);
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

  // Q of the lane's row, B-operand layout: Q[row][16 c + 8 g .. + 7] (loads
  // issued here, first, so that their latency passes during the segment scan)
  const int64_t hq = ((int64_t)w.b * p.Hq + h) * p.Lq;
  {
    const V8* qr = (const V8*)((const char*)p.q + (hq + row_c) * kD * 2);
#pragma unroll
    for (int c = 0; c < 16; ++c) wv.qf[c] = qr[2 * c + wv.g];
  }

  wv.sh = SEG ? seg_shift(wv.n_tiles) : 0;
  if (SEG) seg_scan<kWavesB, kBkB>(sm.bits, wv.sh, p, w, wv.n_tiles);
  // tiles [t_lo, n_tiles): all of them, or this workgroup's key split (tiles
  // at or past the new n_tiles count as past the end)
  const bool split = p.n_split > 1;
  const int t_lo = split ? w.split * p.split_tiles : 0;
  if (split) wv.n_tiles = min(wv.n_tiles, t_lo + p.split_tiles);

  const int64_t kv_head = (int64_t)w.b * p.Hkv + w.kvh;
  wv.kb = (const char*)p.k + kv_head * p.Lk * kD * 2;
  wv.vb = (const char*)p.v + kv_head * p.Lk * kD * 2;
  wv.skb = SEG ? p.seg_k + (int64_t)w.b * p.Lk : nullptr;
  wv.sq = SEG ? p.seg_q[(int64_t)w.b * p.Lq + row_c] : 0;
  wv.lim = p.q_offset + row;  // last key this row may see (causal)

#pragma unroll
  for (int n = 0; n < 8; ++n) {
    wv.acc[n] = f32x16{};
    asm volatile("" : "+a"(wv.acc[n]));
  }
  wv.rs = RowState{-INFINITY, 0.f, 0.f, 0.f};
  wv.ln.init(wv.wave, wv.lane, (lds_cchar*)sm.k[0], (lds_cchar*)sm.v[0]);
  wv.rb = RingBase{lds_addr(sm.k[0]), lds_addr(sm.v[0]), lds_addr(sm.segk[0])};

  wv.vr_lo = wv.vr_hi = wv.fr_lo = wv.fr_hi = 0;
  wv.cur = wv.next_tile(t_lo - 1);
  if (wv.cur < wv.n_tiles) {
    wv.nxt = wv.next_tile(wv.cur);
    wv.nn = wv.next_tile(wv.nxt);
    const bool f_cur = wv.is_full(wv.cur);
    wv.f_nxt = wv.is_full(wv.nxt);
    wv.f_nn = wv.is_full(wv.nn);
    // K(#0), K(#1) and V(#0) into stages 0, 1 and 0 (V(#1) is copied in step 0)
    const PartCopy k0 = wv.k_copy(0, wv.cur), k1 = wv.k_copy(1, wv.nxt), v0 = wv.v_copy(0, wv.cur);
#pragma unroll
    for (int it = 0; it < kCopiesB; ++it) {
      k0.rows(wv.ln.ldk, it, wv.wave);
      k1.rows(wv.ln.ldk, it, wv.wave);
      v0.rows(wv.ln.ldv, it, wv.wave);
    }
    if (SEG) {
      if (!f_cur) k0.ids(wv.wave, wv.lane);
      if (!wv.f_nxt) k1.ids(wv.wave, wv.lane);
    }
    // Q pinned in AGPRs (its 16 loads went out before the segment scan and the
    // tile copies; one statement takes them all, so they are waited for once,
    // together with the copies)
    asm volatile("" : "+a"(wv.qf[0]), "+a"(wv.qf[1]), "+a"(wv.qf[2]), "+a"(wv.qf[3]), "+a"(wv.qf[4]),
                 "+a"(wv.qf[5]), "+a"(wv.qf[6]), "+a"(wv.qf[7]), "+a"(wv.qf[8]), "+a"(wv.qf[9]),
                 "+a"(wv.qf[10]), "+a"(wv.qf[11]), "+a"(wv.qf[12]), "+a"(wv.qf[13]), "+a"(wv.qf[14]),
                 "+a"(wv.qf[15]));
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    f32x16 s0[2];
    qk_only<E>(0, wv.qf, wv.ln, s0);
    // into VGPRs, as phase_b leaves the scores of every later tile (a
    // loop-carried value that enters in AGPRs would go round them each step)
    float sc[32];
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      sc[r] = s0[r >> 4][r & 15];
      asm volatile("" : "+v"(sc[r]));
    }
    wv.mask_if_needed(sc, wv.cur, f_cur, 0);
    (void)lazy_max_update(xor32_max(lane_max(sc)), wv.rs, p.scale_log2);  // nothing accumulated yet: no rescale
#pragma unroll
    for (int r = 0; r < 32; ++r) wv.s_cur[r] = sc[r];
    for (int i = 0; wv.cur < wv.n_tiles; ++i) wv.step(i);
  }

  // epilogue: O = acc / lr (in E), lse = ln2 (m + log2 l); lane holds
  // O[row][32 n + 8 j + 4 g + i] in acc[n][4 j + i]
#pragma unroll
  for (int n = 0; n < 8; ++n) asm volatile("" : "+a"(wv.acc[n]));
  const float l_tot = xor32_sum(wv.rs.l);
  const float lr_tot = xor32_sum(wv.rs.lr);
  if (row < p.Lq) {
    const float inv = lr_tot > 0.f ? 1.f / lr_tot : 0.f;
    const float lse = l_tot > 0.f ? (wv.rs.m_use + log2f(l_tot)) * 0.69314718055994530942f : -INFINITY;
    if (split) {
      // a split writes its normalised part in fp32 (the merge rounds once) and its lse
      float* op = p.o_part + ((int64_t)w.split * p.part_rows + hq + row) * kD;
#pragma unroll
      for (int n = 0; n < 8; ++n)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *(f32x4*)(op + 32 * n + 8 * j + 4 * wv.g) = f32x4{wv.acc[n][4 * j] * inv, wv.acc[n][4 * j + 1] * inv,
                                                              wv.acc[n][4 * j + 2] * inv, wv.acc[n][4 * j + 3] * inv};
      if (wv.g == 0) p.lse_part[(int64_t)w.split * p.part_rows + hq + row] = lse;
    } else {
      char* op = (char*)p.o + (hq + row) * kD * 2;
#pragma unroll
      for (int n = 0; n < 8; ++n)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x2 val = {Elem<E>::pack(wv.acc[n][4 * j] * inv, wv.acc[n][4 * j + 1] * inv),
                             Elem<E>::pack(wv.acc[n][4 * j + 2] * inv, wv.acc[n][4 * j + 3] * inv)};
          *(u32x2*)(op + (32 * n + 8 * j + 4 * wv.g) * 2) = val;
        }
      if (wv.g == 0) p.lse[hq + row] = lse;
    }
  }
}

}  // namespace gqa
