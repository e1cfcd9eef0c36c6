// fwd_f32.hpp -- causal grouped-query attention forward, fp32 inputs and
// output, full-fp32 products on gfx950 MFMA (v_mfma_f32_32x32x2_f32; no
// reduced-precision variant, matching the pages' fp32 runs with TF32 off).
//
// One workgroup = 4 waves, one per SIMD: Q (128 VGPRs per lane) and the O^T
// accumulator (128) stay in registers. For Hq/Hkv = 4 the workgroup owns the 4
// query heads of one KV head x 32 positions. Key tiles of 32 keys (32 KB each
// for K and V) are copied HBM -> LDS once per workgroup with async
// global_load_lds, double-buffered, and shared by the 4 heads.
//
// The data flow matches the bf16 kernel: S^T = K Q^T leaves one query row per
// lane (16 of the 32 keys in registers), the base-2 online softmax with a lazy
// rescale runs lane-locally plus one lane-pair exchange for the row max, and
// O^T += V^T P^T takes P straight from the S^T registers. The fp32 MFMA takes
// one element per lane per operand, so V needs no transposing read: lanes
// 0-31 read 32 consecutive d of one key row.
#pragma once
#include "common.hpp"

namespace gqa {

constexpr int kBkF = 32;                    // keys per LDS tile
constexpr int kTileBytesF = kBkF * kD * 4;  // 32 KB per K or V tile
constexpr float kLazyF = 8.0f;

// LDS image of an fp32 tile: 1 KB key rows of 64 16-byte chunks; chunk c of key
// k is stored at chunk c ^ swzk_f(k) in K tiles and c ^ swzv_f(k) in V tiles.
// The K reads are 16-byte reads of 16 consecutive keys at one chunk per clock:
// an XOR by k % 16 spreads them over all 64 banks. The V reads are 4-byte
// reads of 32 consecutive d (8 chunks) of two keys 4 apart per clock: swzv_f
// puts key bit 2 into chunk bit 3 so the two keys use different halves of the
// banks (and permutes within the 8 chunks by k % 8).
__device__ __forceinline__ int swzk_f(int key) { return key & 15; }
__device__ __forceinline__ int swzv_f(int key) { return (((key >> 2) & 1) << 3) | (key & 7); }

struct SmemF {
  __attribute__((aligned(16))) char k[2][kTileBytesF];
  __attribute__((aligned(16))) char v[2][kTileBytesF];
  __attribute__((aligned(16))) int segk[2][kBkF];
  SegBits bits;
};

// Per-lane pieces of the swizzled LDS addresses, precomputed once so the
// inner loops use a few VGPRs plus immediate offsets.
struct LanesF {
  uint32_t ldk[4];    // K copy of key row w + 4 it, it % 4 = j: (lane ^ swzk_f(row)) * 16
  uint32_t ldv[2];    // V copy of key row w + 4 it, it % 2 = j: (lane ^ swzv_f(row)) * 16
  uint32_t kq[8];     // K read of chunk 2c + g, c % 8 = j, key l32: + 256 (c / 8)
  uint32_t vq[2][4];  // V read of key step tt (tt % 4 = j), d block n: vq[n % 2][j] + 8192 (tt / 4) + 128 n
  __device__ __forceinline__ void init(int wave, int lane) {
    const int l32 = lane & 31, g = lane >> 5;
#pragma unroll
    for (int j = 0; j < 4; ++j) ldk[j] = (uint32_t)(lane ^ swzk_f(wave + 4 * j)) << 4;
#pragma unroll
    for (int j = 0; j < 2; ++j) ldv[j] = (uint32_t)(lane ^ swzv_f(wave + 4 * j)) << 4;
#pragma unroll
    for (int j = 0; j < 8; ++j) kq[j] = (uint32_t)l32 * 1024u + ((uint32_t)((2 * j + g) ^ swzk_f(l32)) << 4);
    // V key kk = 8 (tt / 4) + 4 g + j has swzv_f(kk) = 8 g + 4 g + j, so chunk
    // (8 n + l32 / 4) ^ swzv_f(kk) = 8 (n ^ g) + ((l32 / 4) ^ (4 g + j))
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t base = (uint32_t)(4 * g + j) * 1024u + ((uint32_t)((l32 >> 2) ^ (4 * g + j)) << 4) +
                            ((uint32_t)(l32 & 3) << 2);
      vq[0][j] = base + 128u * (uint32_t)g;  // even n: 8 (n ^ g) = 8 n + 8 g
      vq[1][j] = base - 128u * (uint32_t)g;  // odd n:  8 (n ^ g) = 8 n - 8 g
    }
  }
};

// Async copy of key tile t into LDS stage `st`: wave w copies key rows
// w, w + W, ... (1 KB each, lane l fetching the global chunk that the swizzle
// places at its position). Missing keys past Lk re-read row Lk-1.
template <int W>
__device__ __forceinline__ void load_tile_f(SmemF& sm, int st, const char* kb, const char* vb, const int32_t* skb,
                                            int64_t t, int64_t Lk, int wave, int lane, const LanesF& ln) {
  static_assert(W == 4, "the lane patterns assume 4 waves");
  const char* kt = kb + t * kTileBytesF;
  const char* vt = vb + t * kTileBytesF;
  const int64_t last = Lk - 1 - t * kBkF;  // last valid key within the tile (>= 0)
#pragma unroll
  for (int it = 0; it < kBkF / W; ++it) {
    const int kk = wave + W * it;
    const uint32_t src = (uint32_t)(kk <= last ? kk : (int)last) * 1024u;
    g2lds16(kt, src + ln.ldk[it & 3], sm.k[st] + kk * 1024);
    g2lds16(vt, src + ln.ldv[it & 1], sm.v[st] + kk * 1024);
  }
  if (skb != nullptr && wave == W - 1 && lane < kBkF) {
    g2lds4((const char*)(skb + t * kBkF), (uint32_t)min((int64_t)lane, last) * 4u, sm.segk[st]);
  }
}

template <int W>
__global__ __launch_bounds__(W * 64) void fwd_f32_kernel(FwdParams p) {
  __shared__ SmemF sm;
  const Work w = decode_work(p);
  const int wave = wave_id(), lane = lane_id();
  const int l32 = lane & 31, g = lane >> 5;
  const int h = w.h0 + wave % p.hpc;
  const int64_t pw = w.p0 + (int64_t)(wave / p.hpc) * kRowsPerWave;
  const int64_t row = pw + l32;
  const int64_t row_c = min(row, p.Lq - 1);

  const int64_t p_end = min(w.p0 + (int64_t)p.ppc, p.Lq);
  const int64_t kv_end = p.causal ? min(p.Lk, p.q_offset + p_end) : p.Lk;
  const int n_tiles = (int)((kv_end + kBkF - 1) / kBkF);

  const bool seg = p.seg_q != nullptr;
  const bool use_bits = seg && n_tiles <= kMaxSegTiles;
  if (use_bits) seg_scan<W, kBkF>(sm.bits, p, w, n_tiles);
  // tiles [t_lo, t_hi): all of them, or this workgroup's key split
  const bool split = p.n_split > 1;
  const int t_lo = split ? w.split * p.split_tiles : 0;
  const int t_hi = split ? min(n_tiles, t_lo + p.split_tiles) : n_tiles;

  const int64_t kv_head = (int64_t)w.b * p.Hkv + w.kvh;
  const char* kb = (const char*)p.k + kv_head * p.Lk * kD * 4;
  const char* vb = (const char*)p.v + kv_head * p.Lk * kD * 4;
  const int32_t* skb = seg ? p.seg_k + (int64_t)w.b * p.Lk : nullptr;
  const int sq = seg ? p.seg_q[(int64_t)w.b * p.Lq + row_c] : 0;

  // Q in registers: lane holds Q[row][8c + 4g + e], e = 0..3.
  f32x4 qf[32];
  const int64_t hq = ((int64_t)w.b * p.Hq + h) * p.Lq;
  {
    const f32x4* qr = (const f32x4*)((const char*)p.q + (hq + row_c) * kD * 4);
#pragma unroll
    for (int c = 0; c < 32; ++c) qf[c] = qr[2 * c + g];
  }
  wait_vm0_known();

  f32x16 acc[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) acc[n] = f32x16{};
  float m_run = -INFINITY, l_part = 0.f;
  const float sl2 = p.scale_log2;

  int t = use_bits ? seg_next(sm.bits, t_lo, t_hi) : t_lo;
  int st = 0;
  LanesF ln;
  ln.init(wave, lane);
  if (t < t_hi) load_tile_f<W>(sm, 0, kb, vb, skb, t, p.Lk, wave, lane, ln);
  while (t < t_hi) {
    const int tn = use_bits ? seg_next(sm.bits, t + 1, t_hi) : t + 1;
    wait_vm0();
    __syncthreads();
    if (tn < t_hi) load_tile_f<W>(sm, st ^ 1, kb, vb, skb, tn, p.Lk, wave, lane, ln);
    const int64_t k0 = (int64_t)t * kBkF;
    if (!(p.causal && k0 > p.q_offset + pw + 31)) {
      const bool seg_full = !seg || (use_bits && ((sm.bits.full[t >> 5] >> (t & 31)) & 1u));
      const bool need_mask = !seg_full || k0 + kBkF > p.Lk || (p.causal && k0 + kBkF - 1 > p.q_offset + pw);
      const char* Ks = sm.k[st];
      const char* Vs = sm.v[st];

      // S^T = K Q^T: MFMA (c, e) contracts d = 8c + e (lanes 0-31) and 8c + 4 + e (lanes 32-63).
      // K fragments are read two steps ahead of their MFMAs.
      f32x16 s = {};
      f32x4 kf0 = *(const f32x4*)(Ks + ln.kq[0]);
      f32x4 kf1 = *(const f32x4*)(Ks + ln.kq[1]);
#pragma unroll
      for (int c = 0; c < 32; ++c) {
        const f32x4 a = kf0;
        kf0 = kf1;
        if (c + 2 < 32) kf1 = *(const f32x4*)(Ks + ln.kq[(c + 2) & 7] + ((c + 2) >> 3) * 256);
#pragma unroll
        for (int e = 0; e < 4; ++e) s = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], qf[c][e], s, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      // lane holds keys k0 + 8(r/4) + 4g + r%4 of its row
      if (need_mask) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int kk = 8 * r4 + 4 * g;
          int4 ids = {0, 0, 0, 0};
          if (!seg_full) ids = *(const int4*)(sm.segk[st] + kk);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int64_t key = k0 + kk + e;
            bool vis = key < p.Lk;
            if (p.causal) vis = vis && key <= p.q_offset + row;
            const int id = e == 0 ? ids.x : e == 1 ? ids.y : e == 2 ? ids.z : ids.w;
            if (!seg_full) vis = vis && id == sq;
            s[4 * r4 + e] = vis ? s[4 * r4 + e] : -INFINITY;
          }
        }
      }
      float mx = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
      mx = xor32_max(mx);
      const float mxs = mx * sl2;
      if (__builtin_amdgcn_ballot_w64(mxs > m_run + kLazyF)) {
        const float m_new = fmaxf(m_run, mxs);
        const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run - m_new);
#pragma unroll
        for (int n = 0; n < 8; ++n) acc[n] *= alpha;
        l_part *= alpha;
        m_run = m_new;
      }
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      float pr[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        pr[r] = fast_exp2(fmaf(s[r], sl2, -m_use));
        l_part += pr[r];
      }
      // O^T += V^T P^T: MFMA tt contracts key 8(tt/4) + 4g + tt%4 (P register tt).
      // The 8 V values of key step tt (one per d block) are read one step ahead.
      float vcur[8], vnxt[8];
#pragma unroll
      for (int n = 0; n < 8; ++n) vcur[n] = *(const float*)(Vs + ln.vq[n & 1][0] + n * 128);
#pragma unroll
      for (int tt = 0; tt < 16; ++tt) {
        if (tt + 1 < 16) {
          const int u = tt + 1;
#pragma unroll
          for (int n = 0; n < 8; ++n) vnxt[n] = *(const float*)(Vs + ln.vq[n & 1][u & 3] + (u >> 2) * 8192 + n * 128);
        }
#pragma unroll
        for (int n = 0; n < 8; ++n) acc[n] = __builtin_amdgcn_mfma_f32_32x32x2f32(vcur[n], pr[tt], acc[n], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int n = 0; n < 8; ++n) vcur[n] = vnxt[n];
      }
    }
    t = tn;
    st ^= 1;
  }

  const float l_tot = xor32_sum(l_part);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (row < p.Lq) {
    // a split writes its normalised part and its lse to the split's slots
    float* obase = split ? p.o_part + (int64_t)w.split * p.part_rows * kD : (float*)p.o;
    float* lbase = split ? p.lse_part + (int64_t)w.split * p.part_rows : p.lse;
    float* op = obase + (hq + row) * kD;
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = 32 * n + 8 * r4 + 4 * g;
        *(f32x4*)(op + d0) = f32x4{acc[n][4 * r4] * inv, acc[n][4 * r4 + 1] * inv, acc[n][4 * r4 + 2] * inv,
                                   acc[n][4 * r4 + 3] * inv};
      }
    if (g == 0) {
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      lbase[hq + row] = l_tot > 0.f ? (m_use + log2f(l_tot)) * 0.69314718055994530942f : -INFINITY;
    }
  }
}

}  // namespace gqa
