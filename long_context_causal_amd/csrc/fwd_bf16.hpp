// fwd_bf16.hpp -- causal grouped-query attention forward, bf16 inputs, fp32
// accumulation, on gfx950 bf16 MFMA (v_mfma_f32_16x16x32_bf16).
//
// One workgroup = 8 waves, two per SIMD, so one wave's softmax (VALU) runs
// while the other wave's products occupy the matrix core. For Hq/Hkv = 4 the
// workgroup owns the 4 query heads of one KV head x 32 positions; each wave
// owns one head and 16 query rows (16-row MFMA tiles keep a wave's registers,
// O^T 64 + Q 32 per lane, within the 256 that two waves per SIMD allow). Key
// tiles of 32 keys flow HBM -> LDS through a 4-stage ring (async
// global_load_lds, two tiles in flight ahead of use), each tile read by all 8
// waves, so every K/V byte fetched serves each query head of the group; K/V
// are never repeated per head.
//
// Per wave and key tile j:
//   row max of tile j (exchanges between lanes l, l ^ 16, l ^ 32) and the lazy
//      rescale of the running max (it moves only when a row's maximum grows
//      by more than 8 in log2 units, so O and l are rescaled rarely and
//      p <= 2^8);
//   A: S^T(j+1) = K(j+1) Q^T (A operand = K from LDS, B operand = Q kept in
//      registers; a lane holds one query row, lane % 16, and 8 of the 32 keys)
//      interleaved with P = exp2(...) of tile j rounded to bf16 (RNE), l from
//      the unrounded p (for lse) and lr from the rounded P (for O, so O is an
//      exact convex combination of V rows);
//   B: O^T += V^T P^T (A operand = V^T through the transposing LDS read
//      ds_read_b64_tr_b16, B operand = P straight from the S^T registers).
// Masks (diagonal, ragged tail, segment boundaries) are applied only to the
// tiles that need them. O^T keeps one query row per lane, so the rescale and
// the final 1/lr are lane-local.
#pragma once
#include "common.hpp"

namespace gqa {

constexpr int kWavesB = 8;                  // waves per workgroup
constexpr int kRowsB = 16;                  // query rows per wave
constexpr int kBkB = 32;                    // keys per LDS tile
constexpr int kStagesB = 4;                 // LDS ring depth
constexpr int kTileBytesB = kBkB * kD * 2;  // 16 KB per K or V tile
constexpr float kLazy = 8.0f;               // lazy-rescale threshold (log2 units)

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// LDS image of a bf16 tile: 512-byte key rows of 32 16-byte chunks; chunk c of
// key k is stored at chunk c ^ swz_k(k) in K tiles and c ^ swz_v(k) in V tiles.
// LDS has 64 banks of 4 bytes. The K reads (16 consecutive keys at one chunk,
// lanes 16G..16G+15 at chunk 4c + G) are conflict-free with an XOR by k % 16;
// the transposing V reads (8 keys x one aligned pair of chunks per 32 lanes)
// are conflict-free with swz_v = 2 (k % 8) + (k / 8) % 2, which sends 8
// consecutive keys to 8 different chunk pairs. Both swizzles were checked with
// the SQ_LDS_BANK_CONFLICT counter on gfx950.
__device__ __forceinline__ int swz_k(int key) { return key & 15; }
__device__ __forceinline__ int swz_v(int key) { return ((key & 7) << 1) | ((key >> 3) & 1); }

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

// Per-lane parts of the tile-copy and LDS-read addresses; the rest of each
// address is uniform or a compile-time immediate.
typedef __attribute__((address_space(3))) const char lds_cchar;

struct LanesB {
  uint32_t ldk;    // copy: this lane's 16 bytes within a 1 KB block of 2 key rows (K tile)
  uint32_t ldv;    // the same for the V tile
  lds_cchar* k[4];   // K read, d chunk c (32 d each), c % 4 = j, keys 16 b + l16: + 256 (c / 4) + 8192 b
  lds_cchar* v[8];   // V read, d block n (16 d), n % 8 = j, keys 4G..: + 256 (n / 8); keys 16 + 4G..: + 8192 more
                     // (swz_v(k + 16) = swz_v(k))
  // kbase/vbase: LDS byte addresses of the K and V ring regions (folded in, so a
  // read is one of these VGPRs plus a compile-time immediate)
  __device__ __forceinline__ void init(int wave, int lane, lds_cchar* kbase, lds_cchar* vbase) {
    const int l16 = lane & 15, G = lane >> 4, g = lane >> 5;
    ldk = (uint32_t)g * 512u + ((uint32_t)((lane & 31) ^ swz_k(2 * wave + g)) << 4);
    ldv = (uint32_t)g * 512u + ((uint32_t)((lane & 31) ^ swz_v(2 * wave + g)) << 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) k[j] = kbase + l16 * 512 + (((4 * j + G) ^ swz_k(l16)) << 4);
    const int kr = 4 * G + (l16 >> 2);               // key of this lane's copy within a 16-key block
    const int h = (l16 & 3) >> 1;                     // 16-byte chunk within the 32 bytes of a d block
    const int in = (l16 & 1) << 3;                    // 8-byte half of the chunk
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v[j] = vbase + kr * 512 + (((2 * j + h) ^ swz_v(kr)) << 4) + in;
    }
  }
};

// Async copy of key tile t (keys 32t .. 32t+31) of K, V and the key segment
// ids into LDS stage `st`. Wave w copies the 1 KB blocks w and w + 8 (2 key
// rows each) of K and of V. Keys past Lk re-read row Lk-1 (finite data that
// the mask removes), so no read leaves the tensors.
__device__ __forceinline__ void load_tile_b(SmemB& sm, int st, const char* kb, const char* vb, const int32_t* skb,
                                            int64_t t, int64_t Lk, int wave, int lane, const LanesB& ln) {
  const char* kt = kb + t * kTileBytesB;
  const char* vt = vb + t * kTileBytesB;
  const int last = (int)min((int64_t)(kBkB - 1), Lk - 1 - t * kBkB);  // last valid key within the tile
  if (last == kBkB - 1) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int blk = wave + kWavesB * it;
      g2lds16(kt, ln.ldk + (uint32_t)blk * 1024u, sm.k[st] + blk * 1024);
      g2lds16(vt, ln.ldv + (uint32_t)blk * 1024u, sm.v[st] + blk * 1024);
    }
  } else {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int blk = wave + kWavesB * it;
      uint32_t offk = ln.ldk + (uint32_t)blk * 1024u, offv = ln.ldv + (uint32_t)blk * 1024u;
      const int kk = (int)(offk >> 9);  // the same key row for both
      if (kk > last) {
        offk = ((uint32_t)last << 9) | (offk & 511u);
        offv = ((uint32_t)last << 9) | (offv & 511u);
      }
      g2lds16(kt, offk, sm.k[st] + blk * 1024);
      g2lds16(vt, offv, sm.v[st] + blk * 1024);
    }
  }
  if (skb != nullptr && wave == kWavesB - 1 && lane < kBkB)
    g2lds4((const char*)(skb + t * kBkB), (uint32_t)min(lane, last) * 4u, sm.segk[st]);
}

typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// K fragment u = 2 c + b (16-key block b, 32-d chunk c) of a tile whose
// per-lane read bases (LanesB::k plus the stage offset) are kb[].
__device__ __forceinline__ bf16x8 k_frag(int u, lds_cchar* const* kb) {
  const int b = u & 1, c = u >> 1;
  return *(lds_bf16x8*)(kb[c & 3] + (b * 8192 + (c >> 2) * 256));
}

// S^T = K Q^T for the tile in ring stage st: two 16-key blocks, each 8 MFMAs
// over D = 256, alternating between the blocks; K fragments read three MFMAs ahead.
__device__ __forceinline__ void qk_tile(int st, const bf16x8* qf, const LanesB& ln, f32x4* s) {
  lds_cchar* kb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) kb[j] = ln.k[j] + st * kTileBytesB;
  s[0] = f32x4{};
  s[1] = f32x4{};
  bf16x8 kf[3];
#pragma unroll
  for (int u = 0; u < 3; ++u) kf[u] = k_frag(u, kb);
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    s[u & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[u % 3], qf[u >> 1], s[u & 1], 0, 0, 0);
    if (u + 3 < 16) kf[u % 3] = k_frag(u + 3, kb);
  }
}

typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((address_space(3))) const i32x4 lds_i32x4;

// Element mask of one tile: lane holds keys key0 + 16 b + 4G + r (s[b][r]) of
// row `row`. segk_lane points at this lane's 4 key ids (keys 4G..) in the stage.
__device__ __forceinline__ void mask_tile(f32x4* s, int64_t key0, int G, int64_t Lk, int causal, int64_t lim,
                                          bool seg_elem, lds_cchar* segk_lane, int sq) {
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int kk = 16 * b + 4 * G;
    i32x4 ids = {0, 0, 0, 0};
    if (seg_elem) ids = *(lds_i32x4*)(segk_lane + 64 * b);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t key = key0 + kk + r;
      bool vis = key < Lk;
      if (causal) vis = vis && key <= lim;
      if (seg_elem) vis = vis && ids[r] == sq;
      s[b][r] = vis ? s[b][r] : -INFINITY;
    }
  }
}

// max over the 4 lanes l, l ^ 16, l ^ 32, l ^ 48 that share a query row
__device__ __forceinline__ float row_max4(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  return xor32_max(x);
}
__device__ __forceinline__ float row_sum4(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  return xor32_sum(x);
}

// Online-softmax state of the wave's rows (per lane: its row). l sums the
// unrounded p (for lse), lr the bf16-rounded P that the PV product uses.
struct RowState {
  float m;   // running max, base-2 scaled domain (-inf before any visible key)
  float l;   // this lane's partial sum of p (its 8 of every 32 keys)
  float lr;  // the same over the rounded P
};

// Softmax, first part: row max and the lazy update of the running max.
// Returns the per-lane rescale factor alpha (1 where the max did not move).
__device__ __forceinline__ float softmax_max(const f32x4* s, RowState& rs, float sl2, float& m_use) {
  float mx = fmaxf(fmaxf(s[0][0], s[0][1]), s[0][2]);
  mx = fmaxf(fmaxf(mx, s[0][3]), s[1][0]);
  mx = fmaxf(fmaxf(mx, s[1][1]), s[1][2]);
  mx = fmaxf(mx, s[1][3]);
  mx = row_max4(mx);
  const float mxs = mx * sl2;
  const bool need = mxs > rs.m + kLazy;
  const float m_new = need ? mxs : rs.m;
  const float alpha = need ? fast_exp2(rs.m - m_new) : 1.f;
  rs.m = m_new;
  m_use = (m_new == -INFINITY) ? 0.f : m_new;
  return alpha;
}

// Softmax, second part: P = exp2(s * scale - m) as bf16 pairs in the order of
// the PV B operand (keys 4G..4G+3 of block 0, then of block 1) and the row sums.
__device__ __forceinline__ void softmax_exp(const f32x4* s, RowState& rs, unsigned* pk, float sl2, float m_use,
                                            float alpha) {
  float lsum = 0.f, lrsum = 0.f;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = fast_exp2(fmaf(s[i >> 1][2 * (i & 1)], sl2, -m_use));
    const float b = fast_exp2(fmaf(s[i >> 1][2 * (i & 1) + 1], sl2, -m_use));
    pk[i] = pack_bf16(a, b);
    lsum += a + b;
    lrsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[i]), ones, lrsum, false);
  }
  rs.l = fmaf(rs.l, alpha, lsum);
  rs.lr = fmaf(rs.lr, alpha, lrsum);
}

// V^T fragment for d block n (16 d) of a tile with per-lane read bases vb[]:
// keys 4G..4G+3 and 16+4G..16+4G+3.
__device__ __forceinline__ bf16x8 v_frag(int n, lds_cchar* const* vb) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb[n & 7] + ((n >> 3) * 256)));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb[n & 7] + (8192 + (n >> 3) * 256)));
  const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
  return __builtin_bit_cast(bf16x8, u32x4{lo2[0], lo2[1], hi2[0], hi2[1]});
}

// O^T += V^T P^T for the tile in ring stage st: 16 d blocks, V fragments read
// three MFMAs ahead.
__device__ __forceinline__ void pv_tile(int st, f32x4* acc, const unsigned* pk, const LanesB& ln) {
  lds_cchar* vb[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) vb[j] = ln.v[j] + st * kTileBytesB;
  const bf16x8 pf = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
  bf16x8 vf[3];
#pragma unroll
  for (int n = 0; n < 3; ++n) vf[n] = v_frag(n, vb);
#pragma unroll
  for (int n = 0; n < 16; ++n) {
    acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[n % 3], pf, acc[n], 0, 0, 0);
    if (n + 3 < 16) vf[n % 3] = v_frag(n + 3, vb);
  }
}

__device__ __forceinline__ void rescale_if_needed(f32x4* acc, float alpha) {
  if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
    for (int n = 0; n < 16; ++n) acc[n] *= alpha;
  }
}

// Wait until at most `n` tiles' worth (4 copies per wave per tile) of this
// wave's async copies are outstanding (copies complete in issue order).
__device__ __forceinline__ void wait_tiles(int tiles_outstanding) {
  if (tiles_outstanding >= 2) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else if (tiles_outstanding == 1) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int W>
__global__ __launch_bounds__(W * 64) void fwd_bf16_kernel(FwdParams p) {
  static_assert(W == kWavesB, "the copy pattern assumes 8 waves");
  __shared__ SmemB sm;
  const Work w = decode_work(p);
  const int wave = wave_id(), lane = lane_id();
  const int l16 = lane & 15, G = lane >> 4;
  const int h = w.h0 + wave % p.hpc;
  const int64_t pw = w.p0 + (int64_t)(wave / p.hpc) * kRowsB;  // first row of this wave
  const int64_t row = pw + l16;
  const int64_t row_c = min(row, p.Lq - 1);

  const int64_t p_end = min(w.p0 + (int64_t)p.ppc, p.Lq);
  const int64_t kv_end = p.causal ? min(p.Lk, p.q_offset + p_end) : p.Lk;
  const int n_tiles = (int)((kv_end + kBkB - 1) / kBkB);

  const bool seg = p.seg_q != nullptr;
  const bool use_bits = seg && n_tiles <= kMaxSegTiles;
  if (use_bits) seg_scan<W, kBkB>(sm.bits, p, w, n_tiles);

  const int64_t kv_head = (int64_t)w.b * p.Hkv + w.kvh;
  const char* kb = (const char*)p.k + kv_head * p.Lk * kD * 2;
  const char* vb = (const char*)p.v + kv_head * p.Lk * kD * 2;
  const int32_t* skb = seg ? p.seg_k + (int64_t)w.b * p.Lk : nullptr;
  const int sq = seg ? p.seg_q[(int64_t)w.b * p.Lq + row_c] : 0;
  const int64_t lim = p.q_offset + row;  // last key this row may see (causal)

  // Q in registers, B-operand layout: lane holds Q[row][32c + 8G .. 32c + 8G + 7].
  const int64_t hq = ((int64_t)w.b * p.Hq + h) * p.Lq;
  bf16x8 qf[8];
  {
    const bf16x8* qr = (const bf16x8*)((const char*)p.q + (hq + row_c) * kD * 2);
#pragma unroll
    for (int c = 0; c < 8; ++c) qf[c] = qr[4 * c + G];
  }

  f32x4 acc[16];
#pragma unroll
  for (int n = 0; n < 16; ++n) acc[n] = f32x4{};
  RowState rs = {-INFINITY, 0.f, 0.f};
  const float sl2 = p.scale_log2;
  LanesB ln;
  ln.init(wave, lane, (lds_cchar*)sm.k[0], (lds_cchar*)sm.v[0]);

  auto full_bit = [&](int t) -> bool { return use_bits && ((sm.bits.full[t >> 5] >> (t & 31)) & 1u); };
  auto next_tile = [&](int t) -> int {
    if (t >= n_tiles) return n_tiles;
    return use_bits ? seg_next(sm.bits, t + 1, n_tiles) : t + 1;
  };
  lds_cchar* segk_lane = (lds_cchar*)sm.segk[0] + 16 * G;
  auto mask_if_needed = [&](f32x4* s, int t, int st) {
    const int64_t k0 = (int64_t)t * kBkB;
    const bool seg_elem = seg && !full_bit(t);
    if (seg_elem || k0 + kBkB > p.Lk || (p.causal && k0 + kBkB - 1 > p.q_offset + pw))
      mask_tile(s, k0, G, p.Lk, p.causal, lim, seg_elem, segk_lane + st * (kBkB * 4), sq);
  };

  // visible tiles in order: cur (being finished), nxt (QK this step), nn and n3 (in flight)
  int cur = use_bits ? seg_next(sm.bits, 0, n_tiles) : 0;
  if (cur < n_tiles) {
    int nxt = next_tile(cur), nn = next_tile(nxt);
    load_tile_b(sm, 0, kb, vb, skb, cur, p.Lk, wave, lane, ln);
    if (nxt < n_tiles) load_tile_b(sm, 1, kb, vb, skb, nxt, p.Lk, wave, lane, ln);
    if (nn < n_tiles) load_tile_b(sm, 2, kb, vb, skb, nn, p.Lk, wave, lane, ln);
    wait_tiles((nxt < n_tiles) + (nn < n_tiles));
    __syncthreads();
    f32x4 s_cur[2];
    qk_tile(0, qf, ln, s_cur);
    mask_if_needed(s_cur, cur, 0);
    int i = 0;  // ring stage of `cur`
    while (nxt < n_tiles) {
      wait_tiles(nn < n_tiles);  // tile nxt has landed (nn may still be in flight)
      __syncthreads();           // ... for every wave; and stage (i + 3) % 4 is free
      const int n3 = next_tile(nn);
      if (n3 < n_tiles) load_tile_b(sm, (i + 3) & 3, kb, vb, skb, n3, p.Lk, wave, lane, ln);
      const int s1 = (i + 1) & 3;
      float m_use;
      const float alpha = softmax_max(s_cur, rs, sl2, m_use);
      rescale_if_needed(acc, alpha);
      // A: QK of the next tile interleaved with this tile's exps
      unsigned pk[4];
      f32x4 s_nxt[2];
      qk_tile(s1, qf, ln, s_nxt);
      softmax_exp(s_cur, rs, pk, sl2, m_use, alpha);
      // B: PV of this tile
      pv_tile(i, acc, pk, ln);
      mask_if_needed(s_nxt, nxt, s1);
      s_cur[0] = s_nxt[0];
      s_cur[1] = s_nxt[1];
      cur = nxt;
      nxt = nn;
      nn = n3;
      i = s1;
    }
    float m_use;
    const float alpha = softmax_max(s_cur, rs, sl2, m_use);
    rescale_if_needed(acc, alpha);
    unsigned pk[4];
    softmax_exp(s_cur, rs, pk, sl2, m_use, alpha);
    pv_tile(i, acc, pk, ln);
  }

  // epilogue: O = acc / lr (bf16), lse = ln2 (m + log2 l); lane holds O[row][16 n + 4G + r]
  const float l_tot = row_sum4(rs.l);
  const float lr_tot = row_sum4(rs.lr);
  if (row < p.Lq) {
    const float inv = lr_tot > 0.f ? 1.f / lr_tot : 0.f;
    char* op = (char*)p.o + (hq + row) * kD * 2;
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      const u32x2 val = {pack_bf16(acc[n][0] * inv, acc[n][1] * inv), pack_bf16(acc[n][2] * inv, acc[n][3] * inv)};
      *(u32x2*)(op + (16 * n + 4 * G) * 2) = val;
    }
    if (G == 0) {
      const float m_use = (rs.m == -INFINITY) ? 0.f : rs.m;
      p.lse[hq + row] = l_tot > 0.f ? (m_use + log2f(l_tot)) * 0.69314718055994530942f : -INFINITY;
    }
  }
}

}  // namespace gqa
