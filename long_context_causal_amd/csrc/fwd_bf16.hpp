// fwd_bf16.hpp -- causal grouped-query attention forward, bf16 inputs, fp32
// accumulation, on gfx950 bf16 MFMA (v_mfma_f32_32x32x16_bf16).
//
// One workgroup = 4 waves (one per SIMD). For Hq/Hkv = 4 the workgroup owns
// the 4 query heads of one KV head x (32 NB) positions; each wave owns one head
// and NB blocks of 32 rows. Key tiles of 64 keys are copied HBM -> LDS once per
// workgroup (async global_load_lds, double-buffered) and read by all 4 waves,
// so each K/V byte fetched serves every query head of the group; K/V are never
// repeated per head. Every K or V fragment read from LDS feeds NB MFMAs.
//
// Per wave and 32-key sub-block:
//   S^T = K Q^T  (A operand = K from LDS, B operand = Q kept in registers):
//        a lane holds one query row (lane % 32) and 16 of the 32 keys,
//   mask only on diagonal / ragged / segment-boundary sub-blocks,
//   online softmax in base 2 with a lazy rescale: the running max moves only
//        when a row's new maximum exceeds it by more than 8 (log2 units), so
//        O and l are rescaled rarely and p <= 2^8 stays far from overflow,
//   P rounded to bf16 (RNE) and the row sum l taken from the same rounded P,
//   O^T += V^T P^T (A operand = V^T through the transposing LDS read
//        ds_read_b64_tr_b16, B operand = P straight from the S^T registers).
// O^T keeps one query row per lane, so the rescale and the final 1/l are
// lane-local; the row max needs one exchange between lanes l and l ^ 32.
#pragma once
#include "common.hpp"

namespace gqa {

constexpr int kBkB = 64;                    // keys per LDS tile
constexpr int kTileBytesB = kBkB * kD * 2;  // 32 KB per K or V tile
constexpr int kBlocksB = 1;                 // 32-row blocks per wave
constexpr float kLazy = 8.0f;               // lazy-rescale threshold (log2 units)

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// Byte offset of (key, 16-byte chunk) in a bf16 tile: 512-byte rows, chunks
// XOR-swizzled by key % 8 so 8 consecutive keys at one column use 8 different
// bank groups (both the K reads and the transposing V reads are conflict-free).
__device__ __forceinline__ uint32_t swz_b(int key, int chunk16) {
  return (uint32_t)key * 512u + ((uint32_t)(chunk16 ^ (key & 7)) << 4);
}

struct SmemB {
  __attribute__((aligned(16))) char k[2][kTileBytesB];
  __attribute__((aligned(16))) char v[2][kTileBytesB];
  __attribute__((aligned(16))) int segk[2][kBkB];
  SegBits bits;
};

__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  bf16x2 r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return __builtin_bit_cast(unsigned, r);
}

// Per-lane byte offsets (within a tile of the global tensor) of the 16-byte
// chunks this lane copies: the LDS image of a tile is written 1 KB per wave
// instruction, lane l landing at byte 16 l of its block, and the swizzle is
// applied by choosing which global chunk each lane fetches.
template <int W>
struct TileLanesB {
  uint32_t off[32 / W];
  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int it = 0; it < 32 / W; ++it) {
      const int s = (wave + W * it) * 64 + lane;
      const int kk = s >> 5;
      off[it] = (uint32_t)kk * 512u + ((uint32_t)((s & 31) ^ (kk & 7)) << 4);
    }
  }
};

// Async copy of key tile t of K, V (and the key segment ids) into LDS stage
// `st`. A tile that runs past Lk re-reads row Lk-1 for its missing keys
// (finite data that the mask removes), so no read leaves the tensors.
template <int W>
__device__ __forceinline__ void load_tile_b(SmemB& sm, int st, const char* kb, const char* vb, const int32_t* skb,
                                            int64_t t, int64_t Lk, int wave, int lane, const TileLanesB<W>& tl) {
  const char* kt = kb + t * kTileBytesB;
  const char* vt = vb + t * kTileBytesB;
  if ((t + 1) * kBkB <= Lk) {
#pragma unroll
    for (int it = 0; it < 32 / W; ++it) {
      const int blk = wave + W * it;
      g2lds16(kt + tl.off[it], (lds_void*)(sm.k[st] + blk * 1024));
      g2lds16(vt + tl.off[it], (lds_void*)(sm.v[st] + blk * 1024));
    }
  } else {
    const uint32_t last = (uint32_t)(Lk - 1 - t * kBkB);  // last valid key within the tile
#pragma unroll
    for (int it = 0; it < 32 / W; ++it) {
      const int blk = wave + W * it;
      const uint32_t kk = tl.off[it] >> 9;
      const uint32_t off = (kk <= last ? tl.off[it] : (last << 9) | (tl.off[it] & 511u));
      g2lds16(kt + off, (lds_void*)(sm.k[st] + blk * 1024));
      g2lds16(vt + off, (lds_void*)(sm.v[st] + blk * 1024));
    }
  }
  if (skb != nullptr && wave == W - 1) {
    const int64_t key = min(t * kBkB + lane, Lk - 1);
    g2lds4(skb + key, (lds_void*)sm.segk[st]);
  }
}

// Online-softmax state of one 32-row block. Two row sums are kept: lr sums the
// bf16-rounded P that the PV product actually uses (so O = sum P~ V / sum P~ is
// an exact convex combination of the V rows with the rounded weights), and l
// sums the unrounded p, which the log-sum-exp needs.
struct RowState {
  float m;   // running max, base-2 scaled domain (-inf before any visible key)
  float l;   // this lane's partial sum of p (its 16 of every 32 keys)
  float lr;  // the same over the bf16-rounded p
};

// Mask, max, lazy rescale and P for one 32-row block and one 32-key sub-block.
// s: S^T registers (lane: row `row`, keys kbase + 8(r/4) + 4g + r%4).
__device__ __forceinline__ void softmax_block(f32x16& s, RowState& rs, f32x16* acc, unsigned* pk, bool need_mask,
                                              int64_t key0, int g, int64_t Lk, int causal, int64_t lim,
                                              bool seg_elem, const int* segk_sub, int sq, float sl2) {
  if (need_mask) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int kk = 8 * r4 + 4 * g;
      int4 ids = {0, 0, 0, 0};
      if (seg_elem) ids = *(const int4*)(segk_sub + kk);
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
  float mx = s[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
  mx = xor32_max(mx);
  const float mxs = mx * sl2;
  if (__builtin_amdgcn_ballot_w64(mxs > rs.m + kLazy)) {
    const float m_new = fmaxf(rs.m, mxs);
    const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(rs.m - m_new);
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[n] *= alpha;
    rs.l *= alpha;
    rs.lr *= alpha;
    rs.m = m_new;
  }
  const float m_use = (rs.m == -INFINITY) ? 0.f : rs.m;
  float lsum = 0.f, lrsum = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float a = fast_exp2(fmaf(s[2 * i], sl2, -m_use));
    const float b = fast_exp2(fmaf(s[2 * i + 1], sl2, -m_use));
    pk[i] = pack_bf16(a, b);
    lsum += a + b;
    lrsum += __uint_as_float(pk[i] << 16) + __uint_as_float(pk[i] & 0xffff0000u);
  }
  rs.l += lsum;
  rs.lr += lrsum;
}

// O = acc / lr (bf16) and lse = ln2 (m + log2 l) for one 32-row block.
__device__ __forceinline__ void epilogue_block(const f32x16* acc, const RowState& rs, char* o_row, float* lse_ptr,
                                               int g) {
  const float l_tot = xor32_sum(rs.l);
  const float lr_tot = xor32_sum(rs.lr);
  const float inv = lr_tot > 0.f ? 1.f / lr_tot : 0.f;
#pragma unroll
  for (int n = 0; n < 8; ++n)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d0 = 32 * n + 8 * r4 + 4 * g;
      const u32x2 val = {pack_bf16(acc[n][4 * r4] * inv, acc[n][4 * r4 + 1] * inv),
                         pack_bf16(acc[n][4 * r4 + 2] * inv, acc[n][4 * r4 + 3] * inv)};
      *(u32x2*)(o_row + d0 * 2) = val;
    }
  if (g == 0) {
    const float m_use = (rs.m == -INFINITY) ? 0.f : rs.m;
    *lse_ptr = l_tot > 0.f ? (m_use + log2f(l_tot)) * 0.69314718055994530942f : -INFINITY;
  }
}

// NB = number of 32-row blocks per wave (rows per wave = 32 NB).
template <int W, int NB>
__global__ __launch_bounds__(W * 64) void fwd_bf16_kernel(FwdParams p) {
  __shared__ SmemB sm;
  const Work w = decode_work(p);
  const int wave = wave_id(), lane = lane_id();
  const int l32 = lane & 31, g = lane >> 5;
  const int h = w.h0 + wave % p.hpc;
  const int64_t pw = w.p0 + (int64_t)(wave / p.hpc) * (32 * NB);  // first row of this wave
  int64_t row[NB], row_c[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    row[j] = pw + 32 * j + l32;
    row_c[j] = min(row[j], p.Lq - 1);
  }

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
  int sq[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) sq[j] = seg ? p.seg_q[(int64_t)w.b * p.Lq + row_c[j]] : 0;

  // Q in registers, B-operand layout: lane holds Q[row][16c + 8g .. 16c + 8g + 7].
  bf16x8 qf[NB][16];
  const int64_t hq = ((int64_t)w.b * p.Hq + h) * p.Lq;
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const bf16x8* qr = (const bf16x8*)((const char*)p.q + (hq + row_c[j]) * kD * 2);
#pragma unroll
    for (int c = 0; c < 16; ++c) qf[j][c] = qr[2 * c + g];
  }

  f32x16 acc[NB][8];
  RowState rs[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[j][n] = f32x16{};
    rs[j] = RowState{-INFINITY, 0.f, 0.f};
  }
  const float sl2 = p.scale_log2;
  TileLanesB<W> tl;
  tl.init(wave, lane);
  const int G16 = lane >> 4, i16 = lane & 15;

  int t = use_bits ? seg_next(sm.bits, 0, n_tiles) : 0;
  int st = 0;
  if (t < n_tiles) load_tile_b<W>(sm, 0, kb, vb, skb, t, p.Lk, wave, lane, tl);
  while (t < n_tiles) {
    const int tn = use_bits ? seg_next(sm.bits, t + 1, n_tiles) : t + 1;
    wait_vm0();
    __syncthreads();
    if (tn < n_tiles) load_tile_b<W>(sm, st ^ 1, kb, vb, skb, tn, p.Lk, wave, lane, tl);
    const bool seg_full = !seg || (use_bits && ((sm.bits.full[t >> 5] >> (t & 31)) & 1u));
    const char* Ks = sm.k[st];
    const char* Vs = sm.v[st];
#pragma unroll 1
    for (int sb = 0; sb < 2; ++sb) {
      const int kbase = sb * 32;
      const int64_t k0 = (int64_t)t * kBkB + kbase;
      // the last block holds the latest rows: if none of them sees a key here, no block does
      if (k0 >= p.Lk || (p.causal && k0 > p.q_offset + pw + 32 * NB - 1)) continue;
      const bool tail = k0 + 32 > p.Lk;

      // S^T = K Q^T over D = 256; each K fragment feeds every row block
      f32x16 s[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) s[j] = f32x16{};
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const bf16x8 a = *(const bf16x8*)(Ks + swz_b(kbase + l32, 2 * c + g));
#pragma unroll
        for (int j = 0; j < NB; ++j) s[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[j][c], s[j], 0, 0, 0);
      }
      unsigned pk[NB][8];
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const bool need_mask = !seg_full || tail || (p.causal && k0 + 31 > p.q_offset + pw + 32 * j);
        softmax_block(s[j], rs[j], acc[j], pk[j], need_mask, k0, g, p.Lk, p.causal, p.q_offset + row[j],
                      !seg_full, sm.segk[st] + kbase, sq[j], sl2);
      }
      // O^T += V^T P^T, two 16-key chunks; each V fragment feeds every row block
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        bf16x8 pf[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j)
          pf[j] = __builtin_bit_cast(bf16x8, u32x4{pk[j][4 * c], pk[j][4 * c + 1], pk[j][4 * c + 2], pk[j][4 * c + 3]});
        const int kk0 = kbase + 16 * c + 4 * (G16 >> 1) + (i16 >> 2);
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          const int d0 = 32 * n + 16 * (G16 & 1) + 4 * (i16 & 3);
          const uint32_t off_in = (uint32_t)(d0 & 7) << 1;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4*)(Vs + swz_b(kk0, d0 >> 3) + off_in));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4*)(Vs + swz_b(kk0 + 8, d0 >> 3) + off_in));
          const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
          const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{lo2[0], lo2[1], hi2[0], hi2[1]});
#pragma unroll
          for (int j = 0; j < NB; ++j) acc[j][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[j], acc[j][n], 0, 0, 0);
        }
      }
    }
    t = tn;
    st ^= 1;
  }

#pragma unroll
  for (int j = 0; j < NB; ++j)
    if (row[j] < p.Lq) epilogue_block(acc[j], rs[j], (char*)p.o + (hq + row[j]) * kD * 2, p.lse + hq + row[j], g);
}

}  // namespace gqa
