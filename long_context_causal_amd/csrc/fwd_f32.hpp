// fwd_f32.hpp -- causal grouped-query attention forward, fp32 inputs and
// output, full-fp32 products on gfx950 MFMA (v_mfma_f32_32x32x2_f32; no
// reduced-precision variant, matching the pages' fp32 runs with TF32 off).
//
// One workgroup = 4 waves, one per SIMD. For Hq/Hkv = 4 the workgroup owns the
// 4 query heads of one KV head x 32 positions; each wave owns one head and 32
// query rows. Key tiles of 32 keys (32 KB each for K and V) are copied HBM ->
// LDS once per workgroup with async buffer loads and shared by the 4 heads.
// Q (128 registers per lane) lives in AGPRs, read by the score products in
// place; the O^T accumulator (128), the scores and P live in VGPRs.
//
// S^T = K Q^T leaves one query row per lane (16 of the 32 keys in registers),
// the base-2 online softmax with a lazy rescale runs lane-locally plus one
// lane-pair exchange for the row max, and O^T += V^T P^T takes P straight from
// the S^T registers. The fp32 MFMA takes one element per lane per operand, so
// V needs no transposing read: lanes 0-31 read 32 consecutive d of one key row.
//
// The loop is software-pipelined over tiles, so the matrix cores never wait
// for the softmax. Step i:
//   phase A: the 128 score products of the next tile, with the 16 exps of
//            the current tile spread between them, and the tile copies;
//   phase B: the 128 PV products of the current tile, with the mask and row
//            max of the next tile's scores spread between them;
//   after:   the lazy update of the running max. The max moves only when a
//            row's maximum grows by more than 8 in log2 units. Then O and l
//            are rescaled, rarely.
// K and V have two-stage rings of their own. In step i the copies of K(#i+2)
// and V(#i+1) refill the stages that K(#i) and V(#i-1) left, and one barrier
// per step covers both.
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
  __attribute__((aligned(16))) int segk[2][2 * kBkF];  // key ids of a K stage (the upper half takes the copy's spill)
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

// Async copy of one part (K with its key segment ids, or V) of key tile t
// (keys 32t .. 32t+31) into an LDS stage. Wave w copies the key rows w + 4 it,
// it = 0..7 (1 KB each; lane l fetches the 16-byte chunk that the swizzle
// places at its position). The buffer resource ends at Lk, so keys past it
// read as zeros (finite data that the mask removes); a resource of size 0 (no
// tile) writes only zeros.
struct PartCopyF {
  rsrc_t r, rs;    // rows (K or V) and key ids from the tile start
  uint32_t lds;    // LDS stage
  uint32_t s_lds;  // LDS stage of the ids
  __device__ __forceinline__ void row(int it, int wave, uint32_t lane_off) const {
    const uint32_t kk = (uint32_t)(wave + 4 * it);
    buf2lds16(r, kk * 1024u + lane_off, lds + kk * 1024u);
  }
  // the tile's 32 ids (lanes 32-63 read zeros into the stage's upper half)
  __device__ __forceinline__ void ids(int wave, int lane) const {
    if (wave == 3) buf2lds4(rs, (uint32_t)lane * 4u, s_lds);  // uniform branch
  }
};

__device__ __forceinline__ PartCopyF part_copy_f(uint32_t lds, uint32_t s_lds, const char* base, const int32_t* skb,
                                                 int64_t t, bool valid, int64_t Lk) {
  const int64_t keys = valid ? min((int64_t)kBkF, Lk - t * kBkF) : 0;
  PartCopyF c;
  c.r = make_rsrc(base + (valid ? t * kTileBytesF : 0), (uint32_t)keys * 1024u);
  c.rs = make_rsrc(skb != nullptr ? skb + (valid ? t * kBkF : 0) : nullptr, skb != nullptr ? (uint32_t)keys * 4u : 0u);
  c.lds = lds;
  c.s_lds = s_lds;
  return c;
}

// Each product and the work placed beside it form one scheduling segment.
#define GQA_SEGMENT_END_F() __builtin_amdgcn_sched_barrier(0)

template <int W>
__global__ __launch_bounds__(W * 64) void fwd_f32_kernel(FwdParams p) {
  static_assert(W == 4, "the lane patterns assume 4 waves");
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
  const int sh = seg ? seg_shift(n_tiles) : 0;
  if (seg) seg_scan<W, kBkF>(sm.bits, sh, p, w, n_tiles);
  // tiles [t_lo, t_hi): all of them, or this workgroup's key split
  const bool split = p.n_split > 1;
  const int t_lo = split ? w.split * p.split_tiles : 0;
  const int t_hi = split ? min(n_tiles, t_lo + p.split_tiles) : n_tiles;

  const int64_t kv_head = (int64_t)w.b * p.Hkv + w.kvh;
  const char* kb = (const char*)p.k + kv_head * p.Lk * kD * 4;
  const char* vb = (const char*)p.v + kv_head * p.Lk * kD * 4;
  const int32_t* skb = seg ? p.seg_k + (int64_t)w.b * p.Lk : nullptr;
  const int sq = seg ? p.seg_q[(int64_t)w.b * p.Lq + row_c] : 0;
  const int64_t lim = p.q_offset + row;  // last key this row may see (causal)

  // Q: lane holds Q[row][8c + 4g + e], e = 0..3, in AGPRs (the empty asm
  // statements keep it there; the products read it in place).
  f32x4 qf[32];
  const int64_t hq = ((int64_t)w.b * p.Hq + h) * p.Lq;
  {
    const f32x4* qr = (const f32x4*)((const char*)p.q + (hq + row_c) * kD * 4);
#pragma unroll
    for (int c = 0; c < 32; ++c) qf[c] = qr[2 * c + g];
  }
  wait_vm0_known();
#pragma unroll
  for (int c = 0; c < 32; ++c) asm volatile("" : "+a"(qf[c]));

  f32x16 acc[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) acc[n] = f32x16{};
  float m_run = -INFINITY, l_part = 0.f;
  const float sl2 = p.scale_log2;

  LanesF ln;
  ln.init(wave, lane);
  const uint32_t kbase = lds_addr(sm.k[0]), vbase = lds_addr(sm.v[0]), sbase = lds_addr(sm.segk[0]);

  // the first visible tile after t (t_hi if none) and the segment state
  // (full: no id mask) of tile t; both are asked in increasing t, and the map
  // is read only past the end of the run found last
  int vr_lo = 0, vr_hi = 0, fr_lo = 0, fr_hi = 0;
  auto next_tile = [&](int t) -> int {
    const int u = t + 1;
    if (u >= t_hi) return t_hi;
    if (!seg) return u;
    if (u >= vr_hi) seg_run(sm.bits.vis, sh, u, t_hi, vr_lo, vr_hi);
    return max(u, vr_lo);
  };
  auto is_full = [&](int t) -> bool {
    if (!seg) return true;
    if (t >= t_hi) return false;
    if (t >= fr_hi) seg_run(sm.bits.full, sh, t, t_hi, fr_lo, fr_hi);
    return t >= fr_lo;
  };
  auto k_copy = [&](int st, int t) {
    return part_copy_f(kbase + (uint32_t)st * kTileBytesF, sbase + (uint32_t)st * (2 * kBkF * 4), kb, skb, t,
                       t < t_hi, p.Lk);
  };
  auto v_copy = [&](int st, int t) {
    return part_copy_f(vbase + (uint32_t)st * kTileBytesF, 0u, vb, nullptr, t, t < t_hi, p.Lk);
  };
  // element mask of tile t's scores (its ids in K stage st), where the tile needs one
  auto mask_if_needed = [&](f32x16& s, int t, bool seg_full, int st) {
    const int64_t k0 = (int64_t)t * kBkF;
    if (seg_full && k0 + kBkF <= p.Lk && !(p.causal && k0 + kBkF - 1 > p.q_offset + pw)) return;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int kk = 8 * r4 + 4 * g;
      int4 ids = {0, 0, 0, 0};
      if (!seg_full) ids = *(const int4*)(sm.segk[st] + kk);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t key = k0 + kk + e;
        bool vis = key < p.Lk;
        if (p.causal) vis = vis && key <= lim;
        const int id = e == 0 ? ids.x : e == 1 ? ids.y : e == 2 ? ids.z : ids.w;
        if (!seg_full) vis = vis && id == sq;
        s[4 * r4 + e] = vis ? s[4 * r4 + e] : -INFINITY;
      }
    }
  };
  // the lazy update of the running max from a tile's row max (raw scores)
  auto lazy_update = [&](float mx) {
    const float mxs = xor32_max(mx) * sl2;
    if (__builtin_amdgcn_ballot_w64(mxs > m_run + kLazyF)) {
      const float m_new = fmaxf(m_run, mxs);
      const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run - m_new);
#pragma unroll
      for (int n = 0; n < 8; ++n) acc[n] *= alpha;
      l_part *= alpha;
      m_run = m_new;
    }
  };

  int cur = next_tile(t_lo - 1);
  if (cur < t_hi) {
    int nxt = next_tile(cur), nn = next_tile(nxt);
    const bool f_cur = is_full(cur);
    bool f_nxt = is_full(nxt), f_nn = is_full(nn);
    // K(#0), K(#1) and V(#0) into stages 0, 1 and 0 (V(#1) is copied in step 0)
    {
      const PartCopyF k0 = k_copy(0, cur), k1 = k_copy(1, nxt), v0 = v_copy(0, cur);
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        k0.row(it, wave, ln.ldk[it & 3]);
        k1.row(it, wave, ln.ldk[it & 3]);
        v0.row(it, wave, ln.ldv[it & 1]);
      }
      if (!f_cur) k0.ids(wave, lane);
      if (!f_nxt) k1.ids(wave, lane);
    }
    wait_vm0();
    __syncthreads();
    f32x16 s_cur = {};
    {
      const char* Ks = sm.k[0];
#pragma unroll
      for (int c = 0; c < 32; ++c) {
        const f32x4 a = *(const f32x4*)(Ks + ln.kq[c & 7] + (c >> 3) * 256);
#pragma unroll
        for (int e = 0; e < 4; ++e) s_cur = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], qf[c][e], s_cur, 0, 0, 0);
      }
    }
    mask_if_needed(s_cur, cur, f_cur, 0);
    {
      float mx = s_cur[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s_cur[r]);
      lazy_update(mx);  // nothing accumulated yet
    }

    for (int i = 0; cur < t_hi; ++i) {
      const int st = i & 1, st1 = st ^ 1;
      wait_vm0();       // K(nxt) and V(cur), copied last step, have landed
      __syncthreads();  // ... for every wave; K stage st and V stage st1 are free
      const int n3 = next_tile(nn);
      const bool f3 = is_full(n3);
      const PartCopyF kc = k_copy(st, nn);   // K(#i+2) into K(#i)'s stage
      const PartCopyF vc = v_copy(st1, nxt);  // V(#i+1) into V(#i-1)'s stage
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;

      // phase A: S^T(nxt) = K Q^T from K stage st1; the exps of s_cur at every
      // other chunk; the copies between the chunks
      float pr[16];
      float lsum = 0.f;
      f32x16 s_nxt = {};
      {
        const char* Ks = sm.k[st1];
        f32x4 kf0 = *(const f32x4*)(Ks + ln.kq[0]);
        f32x4 kf1 = *(const f32x4*)(Ks + ln.kq[1]);
#pragma unroll
        for (int c = 0; c < 32; ++c) {
          const f32x4 a = kf0;
          kf0 = kf1;
          if (c + 2 < 32) kf1 = *(const f32x4*)(Ks + ln.kq[(c + 2) & 7] + ((c + 2) >> 3) * 256);
          asm volatile("" : "+a"(qf[c]));
#pragma unroll
          for (int e = 0; e < 4; ++e) s_nxt = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], qf[c][e], s_nxt, 0, 0, 0);
          if ((c & 1) == 0) {
            const int r = c >> 1;
            pr[r] = fast_exp2(fmaf(s_cur[r], sl2, -m_use));
            lsum += pr[r];
          }
          if ((c & 3) == 1) kc.row(c >> 2, wave, ln.ldk[(c >> 2) & 3]);
          if ((c & 3) == 3) vc.row(c >> 2, wave, ln.ldv[(c >> 2) & 1]);
          if (c == 2 && !f_nn) kc.ids(wave, lane);  // the tile needs its key ids
          GQA_SEGMENT_END_F();
        }
      }
      l_part += lsum;

      // phase B: O^T += V^T P^T from V stage st (MFMA tt contracts key
      // 8 (tt / 4) + 4 g + tt % 4, P register tt; the 8 V values of key step
      // tt are read one step ahead), with the mask and row max of s_nxt
      mask_if_needed(s_nxt, nxt, f_nxt, st1);
      float mx = -INFINITY;
      {
        const char* Vs = sm.v[st];
        float vcur[8], vnxt[8];
#pragma unroll
        for (int n = 0; n < 8; ++n) vcur[n] = *(const float*)(Vs + ln.vq[n & 1][0] + n * 128);
#pragma unroll
        for (int tt = 0; tt < 16; ++tt) {
          if (tt + 1 < 16) {
            const int u = tt + 1;
#pragma unroll
            for (int n = 0; n < 8; ++n)
              vnxt[n] = *(const float*)(Vs + ln.vq[n & 1][u & 3] + (u >> 2) * 8192 + n * 128);
          }
#pragma unroll
          for (int n = 0; n < 8; ++n) acc[n] = __builtin_amdgcn_mfma_f32_32x32x2f32(vcur[n], pr[tt], acc[n], 0, 0, 0);
          mx = fmaxf(mx, s_nxt[tt]);
          GQA_SEGMENT_END_F();
#pragma unroll
          for (int n = 0; n < 8; ++n) vcur[n] = vnxt[n];
        }
      }
      // a "next" tile past the range (the last step's, also the tile after a
      // key split) holds the zeros of its copy, no scores: its max stays -inf
      lazy_update(nxt < t_hi ? mx : -INFINITY);
      s_cur = s_nxt;
      cur = nxt;
      nxt = nn;
      nn = n3;
      f_nxt = f_nn;
      f_nn = f3;
    }
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
