// fwd_bf16.hpp -- causal grouped-query attention forward, bf16 inputs, fp32
// accumulation, on gfx950 bf16 MFMA (v_mfma_f32_32x32x16_bf16).
//
// One workgroup = 4 waves (one per SIMD). For Hq/Hkv = 4 the workgroup owns
// the 4 query heads of one KV head x 32 positions; each wave owns one head and
// 32 query rows. Key tiles of 32 keys flow HBM -> LDS through a 4-stage ring
// (async global_load_lds, two tiles in flight ahead of use), each tile read by
// all 4 waves, so every K/V byte fetched serves each query head of the group;
// K/V are never repeated per head.
//
// Per wave and key tile j, software-pipelined:
//   row max of tile j (one exchange between lanes l and l ^ 32) and the lazy
//      rescale of the running max (it moves only when a row's maximum grows
//      by more than 8 in log2 units, so O and l are rescaled rarely and
//      p <= 2^8);
//   A: S^T(j+1) = K(j+1) Q^T on the matrix core (A operand = K from LDS,
//      B operand = Q kept in registers; a lane holds one query row, lane % 32,
//      and 16 of the 32 keys) while the VALU computes P = exp2(...) of tile j
//      rounded to bf16 (RNE), l from the unrounded p (for lse) and lr from the
//      rounded P (for O, so O is an exact convex combination of V rows);
//   B: O^T += V^T P^T (A operand = V^T through the transposing LDS read
//      ds_read_b64_tr_b16, B operand = P straight from the S^T registers).
// Masks (diagonal, ragged tail, segment boundaries) are applied only to the
// tiles that need them. O^T keeps one query row per lane, so the rescale and
// the final 1/lr are lane-local.
#pragma once
#include "common.hpp"

namespace gqa {

constexpr int kBkB = 32;                    // keys per LDS tile (one MFMA block)
constexpr int kStagesB = 4;                 // LDS ring depth
constexpr int kTileBytesB = kBkB * kD * 2;  // 16 KB per K or V tile
constexpr int kLoadsB = 2 * (kTileBytesB / 1024) / 4;  // 16-byte-per-lane copies per wave per tile (4 waves)
constexpr float kLazy = 8.0f;               // lazy-rescale threshold (log2 units)

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// LDS image of a bf16 tile: 512-byte key rows of 32 16-byte chunks; chunk c of
// key k is stored at chunk c ^ swz16(k). LDS has 64 banks of 4 bytes; a
// 16-byte read is served 16 lanes per clock and the transposing 8-byte read 32
// lanes per clock. swz16 maps any 16 consecutive keys to 16 different values,
// so the K reads (16 consecutive keys, one column) hit 16 different 16-byte
// bank groups; within any 4 consecutive keys its top two bits differ, so the
// transposing V reads (4 keys x 4 chunks per 32 lanes) hit 16 different groups
// too. Both access patterns are conflict-free.
__device__ __forceinline__ int swz16(int key) { return ((key & 3) << 2) | ((key >> 2) & 3); }

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
struct LanesB {
  uint32_t ld[2];  // copy: lane's chunk in 1 KB block (2 key rows); block b = wave + 4 it uses ld[it & 1]
  uint32_t k[8];   // K read of chunk 2c + g, c % 8 = j, key l32: + 256 (c / 8)
  uint32_t v[8];   // V transposing read, d block n % 4 = j (v[j]) and the keys 8 higher (v[4 + j]): + 256 (n / 4)
  __device__ __forceinline__ void init(int wave, int lane) {
    const int l32 = lane & 31, g = lane >> 5, G16 = lane >> 4, i16 = lane & 15;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int kk = 2 * wave + 8 * j + g;  // key row of this lane's copy (mod 16 is what matters)
      ld[j] = (uint32_t)g * 512u + ((uint32_t)((lane & 31) ^ swz16(kk)) << 4);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) k[j] = (uint32_t)l32 * 512u + ((uint32_t)((2 * j + g) ^ swz16(l32)) << 4);
    const int kk0 = 4 * (G16 >> 1) + (i16 >> 2);           // key within a 16-key chunk (0..7)
    const int z = 2 * (G16 & 1) + ((i16 & 3) >> 1);         // 16-byte chunk within a 32-d block (0..3)
    const uint32_t in = (uint32_t)(i16 & 1) << 3;           // 8-byte half of the chunk
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = (uint32_t)kk0 * 512u + ((uint32_t)((4 * j + z) ^ swz16(kk0)) << 4) + in;
      v[4 + j] = (uint32_t)(kk0 + 8) * 512u + ((uint32_t)((4 * j + z) ^ swz16(kk0 + 8)) << 4) + in;
    }
  }
};

// Async copy of key tile t (keys 32t .. 32t+31) of K, V and the key segment
// ids into LDS stage `st`. Wave w copies the 1 KB blocks w, w+4, w+8, w+12
// (2 key rows each) of K and of V. Keys past Lk re-read row Lk-1 (finite data
// that the mask removes), so no read leaves the tensors.
__device__ __forceinline__ void load_tile_b(SmemB& sm, int st, const char* kb, const char* vb, const int32_t* skb,
                                            int64_t t, int64_t Lk, int wave, int lane, const LanesB& ln) {
  const char* kt = kb + t * kTileBytesB;
  const char* vt = vb + t * kTileBytesB;
  if ((t + 1) * kBkB <= Lk) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int blk = wave + 4 * it;
      const uint32_t off = ln.ld[it & 1] + (uint32_t)blk * 1024u;
      g2lds16(kt, off, sm.k[st] + blk * 1024);
      g2lds16(vt, off, sm.v[st] + blk * 1024);
    }
  } else {
    const int last = (int)(Lk - 1 - t * kBkB);  // last valid key within the tile
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int blk = wave + 4 * it;
      const uint32_t off = ln.ld[it & 1] + (uint32_t)blk * 1024u;
      const int kk = (int)(off >> 9);
      const uint32_t src = kk <= last ? off : ((uint32_t)last << 9) | (off & 511u);
      g2lds16(kt, src, sm.k[st] + blk * 1024);
      g2lds16(vt, src, sm.v[st] + blk * 1024);
    }
  }
  if (skb != nullptr && wave == 3 && lane < kBkB) {
    const int64_t last = Lk - 1 - t * kBkB;
    g2lds4((const char*)(skb + t * kBkB), (uint32_t)min((int64_t)lane, last) * 4u, sm.segk[st]);
  }
}

// S^T = K Q^T for the tile in LDS at Ks (32 keys x 256 d), K fragments read
// four MFMAs ahead.
__device__ __forceinline__ f32x16 qk_tile(const char* Ks, const bf16x8* qf, const LanesB& ln) {
  f32x16 s = {};
  bf16x8 kf[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) kf[c] = *(const bf16x8*)(Ks + ln.k[c & 7] + (c >> 3) * 256);
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[c & 3], qf[c], s, 0, 0, 0);
    if (c + 4 < 16) kf[c & 3] = *(const bf16x8*)(Ks + ln.k[(c + 4) & 7] + ((c + 4) >> 3) * 256);
  }
  return s;
}

// Element mask of one tile: lane holds keys key0 + 8(r/4) + 4g + r%4 of row `row`.
__device__ __forceinline__ void mask_tile(f32x16& s, int64_t key0, int g, int64_t Lk, int causal, int64_t lim,
                                          bool seg_elem, const int* segk, int sq) {
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) {
    const int kk = 8 * r4 + 4 * g;
    int4 ids = {0, 0, 0, 0};
    if (seg_elem) ids = *(const int4*)(segk + kk);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t key = key0 + kk + e;
      bool vis = key < Lk;
      if (causal) vis = vis && key <= lim;
      const int id = e == 0 ? ids.x : e == 1 ? ids.y : e == 2 ? ids.z : ids.w;
      if (seg_elem) vis = vis && id == sq;
      s[4 * r4 + e] = vis ? s[4 * r4 + e] : -INFINITY;
    }
  }
}

// Online-softmax state of the wave's 32 rows (per lane: its row). l sums the
// unrounded p (for lse), lr the bf16-rounded P that the PV product uses.
struct RowState {
  float m;   // running max, base-2 scaled domain (-inf before any visible key)
  float l;   // this lane's partial sum of p (its 16 of every 32 keys)
  float lr;  // the same over the rounded P
};

// Softmax, first part: row max (one exchange between lanes l and l ^ 32) and
// the lazy update of the running max. Returns the per-lane rescale factor
// alpha (1 where the lane's max did not move) and sets m_use for the exps.
__device__ __forceinline__ float softmax_max(const f32x16& s, RowState& rs, float sl2, float& m_use) {
  float mx = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
  for (int r = 3; r < 15; r += 2) mx = fmaxf(fmaxf(mx, s[r]), s[r + 1]);
  mx = fmaxf(mx, s[15]);
  mx = xor32_max(mx);
  const float mxs = mx * sl2;
  const bool need = mxs > rs.m + kLazy;
  const float m_new = need ? mxs : rs.m;
  const float alpha = need ? fast_exp2(rs.m - m_new) : 1.f;
  rs.m = m_new;
  m_use = (m_new == -INFINITY) ? 0.f : m_new;
  return alpha;
}

// Softmax, second part (no branches): P = exp2(s * scale - m) rounded to bf16
// pairs, and the row sums of the unrounded and of the rounded values.
__device__ __forceinline__ void softmax_exp(const f32x16& s, RowState& rs, unsigned* pk, float sl2, float m_use,
                                            float alpha) {
  float lsum = 0.f, lrsum = 0.f;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float a = fast_exp2(fmaf(s[2 * i], sl2, -m_use));
    const float b = fast_exp2(fmaf(s[2 * i + 1], sl2, -m_use));
    pk[i] = pack_bf16(a, b);
    lsum += a + b;
    lrsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[i]), ones, lrsum, false);
  }
  rs.l = fmaf(rs.l, alpha, lsum);
  rs.lr = fmaf(rs.lr, alpha, lrsum);
}

// V^T fragment m of a tile (16-key chunk m / 8, d block m % 8): two
// transposing reads of 4 bf16 each.
__device__ __forceinline__ bf16x8 v_frag(const char* Vs, int m, const LanesB& ln) {
  const char* Vc = Vs + 16 * (m >> 3) * 512;
  const int n = m & 7;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(Vc + ln.v[n & 3] + (n >> 2) * 256));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(Vc + ln.v[4 + (n & 3)] + (n >> 2) * 256));
  const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
  return __builtin_bit_cast(bf16x8, u32x4{lo2[0], lo2[1], hi2[0], hi2[1]});
}

// O^T += V^T P^T for the tile in LDS at Vs, V fragments read three MFMAs ahead.
__device__ __forceinline__ void pv_tile(f32x16* acc, const char* Vs, const unsigned* pk, const LanesB& ln) {
  const bf16x8 pf0 = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
  const bf16x8 pf1 = __builtin_bit_cast(bf16x8, u32x4{pk[4], pk[5], pk[6], pk[7]});
  bf16x8 vf[3];
#pragma unroll
  for (int m = 0; m < 3; ++m) vf[m] = v_frag(Vs, m, ln);
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    acc[m & 7] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[m % 3], m < 8 ? pf0 : pf1, acc[m & 7], 0, 0, 0);
    if (m + 3 < 16) vf[m % 3] = v_frag(Vs, m + 3, ln);
  }
}

__device__ __forceinline__ void rescale_if_needed(f32x16* acc, float alpha) {
  if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[n] *= alpha;
  }
}

// Wait until at most `n` of this wave's async copies are outstanding (copies
// complete in issue order); n is 0, 1 or 2 tiles' worth.
__device__ __forceinline__ void wait_tiles(int tiles_outstanding) {
  if (tiles_outstanding >= 2) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  else if (tiles_outstanding == 1) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}
static_assert(kLoadsB == 8, "wait_tiles assumes 8 copies per wave per tile");

template <int W>
__global__ __launch_bounds__(W * 64) void fwd_bf16_kernel(FwdParams p) {
  static_assert(W == 4, "the copy pattern assumes 4 waves");
  __shared__ SmemB sm;
  const Work w = decode_work(p);
  const int wave = wave_id(), lane = lane_id();
  const int l32 = lane & 31, g = lane >> 5;
  const int h = w.h0 + wave % p.hpc;
  const int64_t pw = w.p0 + (int64_t)(wave / p.hpc) * kRowsPerWave;  // first row of this wave
  const int64_t row = pw + l32;
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

  // Q in registers, B-operand layout: lane holds Q[row][16c + 8g .. 16c + 8g + 7].
  const int64_t hq = ((int64_t)w.b * p.Hq + h) * p.Lq;
  bf16x8 qf[16];
  {
    const bf16x8* qr = (const bf16x8*)((const char*)p.q + (hq + row_c) * kD * 2);
#pragma unroll
    for (int c = 0; c < 16; ++c) qf[c] = qr[2 * c + g];
  }

  f32x16 acc[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) acc[n] = f32x16{};
  RowState rs = {-INFINITY, 0.f, 0.f};
  const float sl2 = p.scale_log2;
  LanesB ln;
  ln.init(wave, lane);

  // which tiles of this wave's rows need an element mask
  auto needs_mask = [&](int t) -> bool {
    const int64_t k0 = (int64_t)t * kBkB;
    const bool seg_full = !seg || (use_bits && ((sm.bits.full[t >> 5] >> (t & 31)) & 1u));
    return !seg_full || k0 + kBkB > p.Lk || (p.causal && k0 + kBkB - 1 > p.q_offset + pw);
  };
  auto seg_elem = [&](int t) -> bool {
    return seg && !(use_bits && ((sm.bits.full[t >> 5] >> (t & 31)) & 1u));
  };
  auto next_tile = [&](int t) -> int {
    if (t >= n_tiles) return n_tiles;
    return use_bits ? seg_next(sm.bits, t + 1, n_tiles) : t + 1;
  };

  // visible tiles in order: cur (being finished), nxt (QK this iteration), nn, n3 (in flight)
  int cur = use_bits ? seg_next(sm.bits, 0, n_tiles) : 0;
  if (cur < n_tiles) {
    int nxt = next_tile(cur), nn = next_tile(nxt);
    load_tile_b(sm, 0, kb, vb, skb, cur, p.Lk, wave, lane, ln);
    if (nxt < n_tiles) load_tile_b(sm, 1, kb, vb, skb, nxt, p.Lk, wave, lane, ln);
    if (nn < n_tiles) load_tile_b(sm, 2, kb, vb, skb, nn, p.Lk, wave, lane, ln);
    wait_tiles((nxt < n_tiles) + (nn < n_tiles));
    __syncthreads();
    f32x16 s_cur = qk_tile(sm.k[0], qf, ln);
    if (needs_mask(cur)) mask_tile(s_cur, (int64_t)cur * kBkB, g, p.Lk, p.causal, lim, seg_elem(cur), sm.segk[0], sq);
    int i = 0;  // ring position of `cur`
    while (nxt < n_tiles) {
      wait_tiles(nn < n_tiles);  // tile nxt has landed (nn may still be in flight)
      __syncthreads();           // ... for every wave; and stage (i + 3) % 4 is free
      const int n3 = next_tile(nn);
      if (n3 < n_tiles) load_tile_b(sm, (i + 3) & 3, kb, vb, skb, n3, p.Lk, wave, lane, ln);
      const int s1 = (i + 1) & 3;
      // softmax max of this tile and the (rare) rescale of O, ahead of the overlapped block
      float m_use;
      const float alpha = softmax_max(s_cur, rs, sl2, m_use);
      rescale_if_needed(acc, alpha);
      // A: QK of the next tile on the matrix core while the VALU runs this tile's exps
      unsigned pk[8];
      f32x16 s_nxt = qk_tile(sm.k[s1], qf, ln);
      softmax_exp(s_cur, rs, pk, sl2, m_use, alpha);
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // 4 VALU
      }
      // B: PV of this tile
      pv_tile(acc, sm.v[i & 3], pk, ln);
      if (needs_mask(nxt))
        mask_tile(s_nxt, (int64_t)nxt * kBkB, g, p.Lk, p.causal, lim, seg_elem(nxt), sm.segk[s1], sq);
      s_cur = s_nxt;
      cur = nxt;
      nxt = nn;
      nn = n3;
      i = (i + 1) & 3;
    }
    float m_use;
    const float alpha = softmax_max(s_cur, rs, sl2, m_use);
    rescale_if_needed(acc, alpha);
    unsigned pk[8];
    softmax_exp(s_cur, rs, pk, sl2, m_use, alpha);
    pv_tile(acc, sm.v[i & 3], pk, ln);
  }

  // epilogue: O = acc / lr (bf16), lse = ln2 (m + log2 l)
  if (row < p.Lq) {
    const float l_tot = xor32_sum(rs.l);
    const float lr_tot = xor32_sum(rs.lr);
    const float inv = lr_tot > 0.f ? 1.f / lr_tot : 0.f;
    char* op = (char*)p.o + (hq + row) * kD * 2;
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = 32 * n + 8 * r4 + 4 * g;
        const u32x2 val = {pack_bf16(acc[n][4 * r4] * inv, acc[n][4 * r4 + 1] * inv),
                           pack_bf16(acc[n][4 * r4 + 2] * inv, acc[n][4 * r4 + 3] * inv)};
        *(u32x2*)(op + d0 * 2) = val;
      }
    if (g == 0) {
      const float m_use = (rs.m == -INFINITY) ? 0.f : rs.m;
      p.lse[hq + row] = l_tot > 0.f ? (m_use + log2f(l_tot)) * 0.69314718055994530942f : -INFINITY;
    }
  } else {
    // keep the exchange lockstep for lanes past Lq (their values are unused)
    (void)xor32_sum(rs.l);
  }
}

}  // namespace gqa
