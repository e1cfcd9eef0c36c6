// bwd_f32.hpp -- backward of the causal grouped-query attention, fp32 inputs
// and gradients, full-fp32 products (v_mfma_f32_16x16x4_f32).
//
// Two kernels, no atomics (so the result is deterministic):
//  * dQ kernel, over query blocks: recomputes S^T = K Q^T and dP^T = V dO^T for
//    its rows, forms dS^T = P^T (dP^T - delta) and accumulates dQ^T += K^T dS^T.
//    It also computes delta_i = dO_i . O_i for its rows and writes it out.
//  * dK/dV kernel, over key blocks (after the dQ kernel, which wrote delta):
//    recomputes S = Q K^T and dP = dO V^T for every query row and head that
//    sees its keys, and accumulates dV^T += dO^T P and dK^T += Q^T dS, summing
//    over the query heads of the key/value head (the GQA reduction).
//
// MFMA 16x16x4 f32 layouts (lane l, g = l / 16, m = l % 16): A operand
// A[m][k = g], B operand B[k = g][n = m], result D[4 g + r][m], r = 0..3. A
// contraction index may be assigned to lanes in any order as long as A and B
// agree, so each lane reads 16-byte chunks (4 consecutive d) and the outputs of
// one product feed the next as operands without moving between lanes:
//  * d-contractions (S, dP): step (c, e) contracts d = 16 c + 4 g + e;
//  * key/row contractions (dQ, dK, dV): step (kb, r) contracts the entry
//    4 g + r of 16-entry block kb, which is exactly where the previous
//    product's result left it in register r;
//  * output d-blocks n = 4 a + b hold d = 64 a + 4 m + b, so one 16-byte read
//    of chunk 16 a + m serves the four blocks b = 0..3.
// LDS tiles are 1 KB rows of 64 16-byte chunks; chunk c of row x is stored at
// chunk c ^ (x % 16). Both read shapes are then conflict-free: 16 rows x one
// chunk (the S / dP operands) and one row x 16 chunks (the dQ / dK / dV ones).
#pragma once
#include "common.hpp"

namespace gqa {

constexpr int kWavesDQ = 8;      // dQ kernel: 2 waves per SIMD
constexpr int kRowsDQ = 16;      // query rows per wave
constexpr int kBkDQ = 32;        // keys per LDS tile
constexpr int kWavesDKV = 4;     // dK/dV kernel: 1 wave per SIMD
constexpr int kKeysDKV = 16;     // keys per wave
constexpr int kRowsDKV = 16;     // query rows per LDS tile
constexpr int kKeysBlockDKV = kWavesDKV * kKeysDKV;

__device__ __forceinline__ f32x4 mfma16(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// LDS byte offset of chunk c of row x in a swizzled 1 KB-row tile.
__device__ __forceinline__ uint32_t swz_off(int x, int c) { return (uint32_t)x * 1024u + ((uint32_t)(c ^ (x & 15)) << 4); }

// Per-lane offsets of the two read shapes (m = lane % 16, g = lane / 16):
//  dcon[j]: row m, chunk 4 c + g for c % 4 = j; chunk c adds 256 (c / 4)
//  rowc[r]: row 4 g + r, chunk 16 a + m; a adds 256 a
struct LanesBwdF {
  uint32_t dcon[4];
  uint32_t rowc[4];
  __device__ __forceinline__ void init(int lane) {
    const int m = lane & 15, g = lane >> 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) dcon[j] = swz_off(m, 4 * j + g);
#pragma unroll
    for (int r = 0; r < 4; ++r) rowc[r] = swz_off(4 * g + r, m);
  }
};

// ---------------------------------------------------------------------------
// dQ kernel
// ---------------------------------------------------------------------------
struct SmemDQ {
  __attribute__((aligned(16))) char k[2][kBkDQ * 1024];
  __attribute__((aligned(16))) char v[2][kBkDQ * 1024];
  __attribute__((aligned(16))) int segk[2][kBkDQ];
  SegBits bits;
};

// Async copy of key tile t (K, V and key ids) into stage st. Wave w copies key
// rows w, w + 8, w + 16, w + 24; lane l fetches the global chunk that the
// swizzle stores at chunk l. Keys past Lk read zeros (buffer bound).
__device__ __forceinline__ void dq_copy(SmemDQ& sm, int st, rsrc_t rk, rsrc_t rv, rsrc_t rs, bool seg, int64_t t,
                                        int wave, int lane) {
#pragma unroll
  for (int it = 0; it < kBkDQ / kWavesDQ; ++it) {
    const int kk = wave + kWavesDQ * it;
    const uint32_t src = (uint32_t)(t * kBkDQ + kk) * 1024u + ((uint32_t)(lane ^ (kk & 15)) << 4);
    buf2lds16(rk, src, lds_addr(sm.k[st] + kk * 1024));
    buf2lds16(rv, src, lds_addr(sm.v[st] + kk * 1024));
  }
  // lane l writes id slot l: only the first kBkDQ lanes take part
  if (seg && wave == kWavesDQ - 1 && lane < kBkDQ)
    buf2lds4(rs, (uint32_t)(t * kBkDQ + lane) * 4u, lds_addr(sm.segk[st]));
}

__global__ __launch_bounds__(kWavesDQ * 64) void bwd_dq_f32_kernel(BwdParams bp) {
  __shared__ SmemDQ sm;
  const FwdParams& p = bp.f;
  const Work w = decode_work(p);
  const int wave = wave_id(), lane = lane_id();
  const int m = lane & 15, g = lane >> 4;
  const int h = w.h0 + wave % p.hpc;
  const int64_t pw = w.p0 + (int64_t)(wave / p.hpc) * kRowsDQ;
  const int64_t row = pw + m;
  const int64_t row_c = min(row, p.Lq - 1);

  const int64_t p_end = min(w.p0 + (int64_t)p.ppc, p.Lq);
  const int64_t kv_end = p.causal ? min(p.Lk, p.q_offset + p_end) : p.Lk;
  const int n_tiles = (int)((kv_end + kBkDQ - 1) / kBkDQ);

  const bool seg = p.seg_q != nullptr;
  const int sh = seg ? seg_shift(n_tiles) : 0;
  if (seg) seg_scan<kWavesDQ, kBkDQ>(sm.bits, sh, p, w, n_tiles);

  const int64_t kv_head = (int64_t)w.b * p.Hkv + w.kvh;
  const rsrc_t rk = make_rsrc((const char*)p.k + kv_head * p.Lk * kD * 4, (uint32_t)(p.Lk * kD * 4));
  const rsrc_t rv = make_rsrc((const char*)p.v + kv_head * p.Lk * kD * 4, (uint32_t)(p.Lk * kD * 4));
  const rsrc_t rs = make_rsrc(seg ? (const void*)(p.seg_k + (int64_t)w.b * p.Lk) : (const void*)p.k,
                              seg ? (uint32_t)(p.Lk * 4) : 0u);
  const int sq = seg ? p.seg_q[(int64_t)w.b * p.Lq + row_c] : 0;

  // Q and dO of the lane's row: chunk 4 c + g (d = 16 c + 4 g + e); delta = dO . O.
  const int64_t hq = ((int64_t)w.b * p.Hq + h) * p.Lq;
  f32x4 qf[16], df[16];
  float delta;
  {
    const f32x4* qr = (const f32x4*)((const char*)p.q + (hq + row_c) * kD * 4);
    const f32x4* dr = (const f32x4*)((const char*)bp.dout + (hq + row_c) * kD * 4);
    const f32x4* orow = (const f32x4*)((const char*)p.o + (hq + row_c) * kD * 4);
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      qf[c] = qr[4 * c + g];
      df[c] = dr[4 * c + g];
      const f32x4 ov = orow[4 * c + g];
      acc = fmaf(df[c][0], ov[0], acc);
      acc = fmaf(df[c][1], ov[1], acc);
      acc = fmaf(df[c][2], ov[2], acc);
      acc = fmaf(df[c][3], ov[3], acc);
    }
    acc += __shfl_xor(acc, 16);
    acc += __shfl_xor(acc, 32);
    delta = acc;
    if (g == 0 && row < p.Lq) bp.delta[hq + row] = delta;
  }
  const float lse = p.lse[hq + row_c];
  const float lse2 = lse == -INFINITY ? 0.f : lse * 1.4426950408889634f;
  wait_vm0_known();
  const float sl2 = p.scale_log2;

  f32x4 acc[16];
#pragma unroll
  for (int n = 0; n < 16; ++n) acc[n] = f32x4{};

  LanesBwdF ln;
  ln.init(lane);
  int t = seg ? seg_next(sm.bits, sh, 0, n_tiles) : 0;
  int st = 0;
  if (t < n_tiles) dq_copy(sm, 0, rk, rv, rs, seg, t, wave, lane);
  while (t < n_tiles) {
    const int tn = seg ? seg_next(sm.bits, sh, t + 1, n_tiles) : t + 1;
    wait_vm0();
    __syncthreads();
    if (tn < n_tiles) dq_copy(sm, st ^ 1, rk, rv, rs, seg, tn, wave, lane);
    const int64_t k0 = (int64_t)t * kBkDQ;
    if (!(p.causal && k0 > p.q_offset + pw + kRowsDQ - 1)) {
      const bool seg_full = !seg || seg_full_tile(sm.bits, sh, t);
      const bool need_mask = !seg_full || k0 + kBkDQ > p.Lk || (p.causal && k0 + kBkDQ - 1 > p.q_offset + pw);
      const char* Ks = sm.k[st];
      const char* Vs = sm.v[st];
      // S^T and dP^T, 2 blocks of 16 keys: lane holds key 16 kb + 4 g + r of its row
      f32x4 s[2], dp[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x4{};
        dp[kb] = f32x4{};
#pragma unroll
        for (int c = 0; c < 16; ++c) {
          const f32x4 kf = *(const f32x4*)(Ks + ln.dcon[c & 3] + (c >> 2) * 256 + kb * 16384);
          const f32x4 vf = *(const f32x4*)(Vs + ln.dcon[c & 3] + (c >> 2) * 256 + kb * 16384);
#pragma unroll
          for (int e = 0; e < 4; ++e) s[kb] = mfma16(kf[e], qf[c][e], s[kb]);
#pragma unroll
          for (int e = 0; e < 4; ++e) dp[kb] = mfma16(vf[e], df[c][e], dp[kb]);
        }
      }
      // dS^T = P^T (dP^T - delta), P^T = exp2(S^T log2(e)/sqrt(D) - lse log2(e))
      float ds[2][4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        int4 ids = {0, 0, 0, 0};
        if (need_mask && !seg_full) ids = *(const int4*)(sm.segk[st] + 16 * kb + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float pv = fast_exp2(fmaf(s[kb][r], sl2, -lse2));
          if (need_mask) {
            const int64_t key = k0 + 16 * kb + 4 * g + r;
            bool vis = key < p.Lk;
            if (p.causal) vis = vis && key <= p.q_offset + row;
            const int id = r == 0 ? ids.x : r == 1 ? ids.y : r == 2 ? ids.z : ids.w;
            if (!seg_full) vis = vis && id == sq;
            pv = vis ? pv : 0.f;
          }
          ds[kb][r] = pv * (dp[kb][r] - delta);
        }
      }
      // dQ^T += K^T dS^T: step (kb, r) contracts key 16 kb + 4 g + r
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const f32x4 kf = *(const f32x4*)(Ks + ln.rowc[r] + a * 256 + kb * 16384);
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[4 * a + b] = mfma16(kf[b], ds[kb][r], acc[4 * a + b]);
          }
    }
    t = tn;
    st ^= 1;
  }

  // lane holds dQ^T[d = 64 a + 16 g + 4 r + b][row] in acc[4 a + b][r]
  if (row < p.Lq) {
    const float sc = kInvSqrtD;
    float* dqr = (float*)bp.dq + (hq + row) * kD;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *(f32x4*)(dqr + 64 * a + 16 * g + 4 * r) =
            f32x4{acc[4 * a][r] * sc, acc[4 * a + 1][r] * sc, acc[4 * a + 2][r] * sc, acc[4 * a + 3][r] * sc};
  }
}

// ---------------------------------------------------------------------------
// dK/dV kernel
// ---------------------------------------------------------------------------
struct SmemDKV {
  __attribute__((aligned(16))) char v[kKeysBlockDKV * 1024];  // V of the block's keys, for the whole kernel
  __attribute__((aligned(16))) char q[2][kRowsDKV * 1024];
  __attribute__((aligned(16))) char d[2][kRowsDKV * 1024];
  __attribute__((aligned(16))) float lse[2][kRowsDKV];
  __attribute__((aligned(16))) float delta[2][kRowsDKV];
  __attribute__((aligned(16))) int segq[2][kRowsDKV];
  SegBits bits;
};

// Async copy of query tile (rows i0.., head h) into stage st: the Q and dO
// rows (wave w copies rows w, w + 4, w + 8, w + 12) and, in a separate call
// (wave 0, lanes 0..15), the lse, delta and row ids. Rows past Lq read zeros.
// With live == false the descriptors have size 0: the copy then takes no
// branch and writes zeros into the idle stage.
__device__ __forceinline__ void dkv_copy_rows(SmemDKV& sm, int st, const BwdParams& bp, int b, int h, int64_t i0,
                                              int wave, int lane, bool live = true) {
  const FwdParams& p = bp.f;
  const int64_t hq = ((int64_t)b * p.Hq + h) * p.Lq;
  const uint32_t nb = live ? (uint32_t)(p.Lq * kD * 4) : 0u;
  const rsrc_t rq = make_rsrc((const char*)p.q + hq * kD * 4, nb);
  const rsrc_t rd = make_rsrc((const char*)bp.dout + hq * kD * 4, nb);
#pragma unroll
  for (int it = 0; it < kRowsDKV / kWavesDKV; ++it) {
    const int rr = wave + kWavesDKV * it;
    const uint32_t src = (uint32_t)(i0 + rr) * 1024u + ((uint32_t)(lane ^ (rr & 15)) << 4);
    buf2lds16(rq, src, lds_addr(sm.q[st] + rr * 1024));
    buf2lds16(rd, src, lds_addr(sm.d[st] + rr * 1024));
  }
}
__device__ __forceinline__ void dkv_copy_rowdata(SmemDKV& sm, int st, const BwdParams& bp, int b, int h,
                                                 int64_t i0, int wave, int lane) {
  const FwdParams& p = bp.f;
  // lane l writes slot l: only the first kRowsDKV lanes take part
  if (wave == 0 && lane < kRowsDKV) {
    const int64_t hq = ((int64_t)b * p.Hq + h) * p.Lq;
    const uint32_t off = (uint32_t)(i0 + lane) * 4u, nb = (uint32_t)(p.Lq * 4);
    buf2lds4(make_rsrc(p.lse + hq, nb), off, lds_addr(sm.lse[st]));
    buf2lds4(make_rsrc(bp.delta + hq, nb), off, lds_addr(sm.delta[st]));
    if (p.seg_q != nullptr) buf2lds4(make_rsrc(p.seg_q + (int64_t)b * p.Lq, nb), off, lds_addr(sm.segq[st]));
  }
}

__global__ __launch_bounds__(kWavesDKV * 64) void bwd_dkv_f32_kernel(BwdParams bp) {
  __shared__ SmemDKV sm;
  const FwdParams& p = bp.f;
  // block ids: key blocks from the first (most rows under a causal mask) to the
  // last, (batch, kv head) fastest so each XCD keeps to one kv head
  const int kbk = blockIdx.x / bp.BH;
  const int bh = blockIdx.x % bp.BH;
  const int kvh = bh % p.Hkv, b = bh / p.Hkv;
  const int wave = wave_id(), lane = lane_id();
  const int m = lane & 15, g = lane >> 4;
  const int64_t j0 = (int64_t)kbk * kKeysBlockDKV;
  const int64_t kw0 = j0 + (int64_t)wave * kKeysDKV;
  const int64_t key = kw0 + m;
  const int64_t key_c = min(key, p.Lk - 1);

  // query rows that can see the block: i >= j0 - q_offset under a causal mask
  const int64_t r_first = p.causal ? max((int64_t)0, j0 - p.q_offset) : 0;
  const int rb0 = (int)(r_first / kRowsDKV);
  const int n_rb = (int)((p.Lq + kRowsDKV - 1) / kRowsDKV);

  const bool seg = p.seg_q != nullptr;
  const int sh = seg ? seg_shift(n_rb) : 0;
  // the row ids' index, where the call brings one (rows of ceil(Lq / 16) entries per batch)
  const SegBlk* qix = p.seg_q_idx ? p.seg_q_idx + (int64_t)b * ((p.Lq + kSegBlk - 1) / kSegBlk) : nullptr;
  if (seg)
    seg_scan_any<kWavesDKV * 64, kRowsDKV>(sm.bits, sh, p.seg_k + (int64_t)b * p.Lk, j0, kKeysBlockDKV, p.Lk,
                                           p.seg_q + (int64_t)b * p.Lq, qix, p.Lq, n_rb, rb0);
  const int sk = seg ? p.seg_k[(int64_t)b * p.Lk + key_c] : 0;

  // K of the lane's key in registers: chunk 4 c + g (d = 16 c + 4 g + e). V of
  // the block's 64 keys in LDS (swizzled rows; keys past Lk read zeros): the
  // registers hold K, the dK and dV accumulators and the operand rings.
  const int64_t kv_head = (int64_t)b * p.Hkv + kvh;
  f32x4 kf[16];
  {
    const f32x4* kr = (const f32x4*)((const char*)p.k + (kv_head * p.Lk + key_c) * kD * 4);
#pragma unroll
    for (int c = 0; c < 16; ++c) kf[c] = kr[4 * c + g];
    const rsrc_t rv = make_rsrc((const char*)p.v + kv_head * p.Lk * kD * 4, (uint32_t)(p.Lk * kD * 4));
#pragma unroll
    for (int it = 0; it < kKeysBlockDKV / kWavesDKV; ++it) {
      const int kk = wave + kWavesDKV * it;
      buf2lds16(rv, (uint32_t)(j0 + kk) * 1024u + ((uint32_t)(lane ^ (kk & 15)) << 4), lds_addr(sm.v + kk * 1024));
    }
  }
  wait_vm0_known();
  f32x4 dka[16], dva[16];
#pragma unroll
  for (int n = 0; n < 16; ++n) {
    dka[n] = f32x4{};
    dva[n] = f32x4{};
  }
  const float sl2 = p.scale_log2;
  const int n_rep = p.n_rep;
  const int h0 = kvh * n_rep;
  const char* Vs = sm.v + wave * kKeysDKV * 1024;

  LanesBwdF ln;
  ln.init(lane);
  // tiles (rb, hh), hh fastest, row blocks from the last down to rb0: every
  // key block starts at the last rows, so the workgroups that run together on
  // an XCD (one kv head) stream the same Q / dO tiles at about the same time
  // and share them in that XCD's L2.
  int rb = seg ? seg_prev(sm.bits, sh, n_rb - 1, rb0) : n_rb - 1;
  int hh = 0;
  int st = 0;
  if (rb >= rb0) {
    dkv_copy_rows(sm, 0, bp, b, h0, (int64_t)rb * kRowsDKV, wave, lane);
    dkv_copy_rowdata(sm, 0, bp, b, h0, (int64_t)rb * kRowsDKV, wave, lane);
  }
  while (rb >= rb0) {
    int rbn = rb, hhn = hh + 1;
    if (hhn == n_rep) {
      hhn = 0;
      rbn = seg ? seg_prev(sm.bits, sh, rb - 1, rb0) : rb - 1;
    }
    wait_vm0();
    __syncthreads();
    if (rbn >= rb0) {
      dkv_copy_rows(sm, st ^ 1, bp, b, h0 + hhn, (int64_t)rbn * kRowsDKV, wave, lane);
      dkv_copy_rowdata(sm, st ^ 1, bp, b, h0 + hhn, (int64_t)rbn * kRowsDKV, wave, lane);
    }
    const int64_t i0 = (int64_t)rb * kRowsDKV;
    if (!(p.causal && kw0 > p.q_offset + i0 + kRowsDKV - 1)) {
      const bool seg_full = !seg || seg_full_tile(sm.bits, sh, rb);
      const bool need_mask =
          !seg_full || i0 + kRowsDKV > p.Lq || (p.causal && kw0 + kKeysDKV - 1 > p.q_offset + i0);
      const char* Qs = sm.q[st];
      const char* Ds = sm.d[st];
      // row data of the tile, read now so that the softmax step does not wait for it
      const f32x4 lse4 = *(const f32x4*)(&sm.lse[st][4 * g]);
      const f32x4 del4 = *(const f32x4*)(&sm.delta[st][4 * g]);
      int4 ids = {sk, sk, sk, sk};
      if (!seg_full) ids = *(const int4*)(&sm.segq[st][4 * g]);
      // mask limits in 32 bits: row 4 g + r of the tile sees the lane's key iff
      // 4 g + r >= lim (causal) and 4 g + r < nrow (rows past Lq)
      const int lim = (p.causal && need_mask) ? (int)max((int64_t)-1, min((int64_t)kRowsDKV, key - p.q_offset - i0)) : -1;
      const int nrow = (int)min((int64_t)kRowsDKV, p.Lq - i0);
      // S = Q K^T and dP = dO V^T: lane holds row 4 g + r of its key. With one
      // wave per SIMD nothing else hides the LDS latency, so the operand reads
      // run two steps ahead of their products (a ring of three).
      f32x4 s = {}, dp = {};
      f32x4 qa[3], da[3], va[3];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        qa[c] = *(const f32x4*)(Qs + ln.dcon[c & 3] + (c >> 2) * 256);
        da[c] = *(const f32x4*)(Ds + ln.dcon[c & 3] + (c >> 2) * 256);
        va[c] = *(const f32x4*)(Vs + ln.dcon[c & 3] + (c >> 2) * 256);
      }
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        if (c + 2 < 16) {
          const int u = c + 2;
          qa[u % 3] = *(const f32x4*)(Qs + ln.dcon[u & 3] + (u >> 2) * 256);
          da[u % 3] = *(const f32x4*)(Ds + ln.dcon[u & 3] + (u >> 2) * 256);
          va[u % 3] = *(const f32x4*)(Vs + ln.dcon[u & 3] + (u >> 2) * 256);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s = mfma16(qa[c % 3][e], kf[c][e], s);
          dp = mfma16(da[c % 3][e], va[c % 3][e], dp);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // the first two operand pairs of the dV / dK products, read while the
      // last S and dP products finish
      f32x4 qb[3], db[3];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        db[u] = *(const f32x4*)(Ds + ln.rowc[u >> 2] + (u & 3) * 256);
        qb[u] = *(const f32x4*)(Qs + ln.rowc[u >> 2] + (u & 3) * 256);
      }
      float pr[4], ds[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float l2 = lse4[r] == -INFINITY ? 0.f : lse4[r] * 1.4426950408889634f;
        float pv = fast_exp2(fmaf(s[r], sl2, -l2));
        // branch-free: lim = -1, nrow = 16 and ids = sk when no mask is needed
        const int ri = 4 * g + r;
        const int id = r == 0 ? ids.x : r == 1 ? ids.y : r == 2 ? ids.z : ids.w;
        pv = (ri < nrow && ri >= lim && id == sk) ? pv : 0.f;
        pr[r] = pv;
        ds[r] = pv * (dp[r] - del4[r]);
      }
      __builtin_amdgcn_sched_barrier(0);
      // dV^T += dO^T P and dK^T += Q^T dS: step u = 4 r + a contracts row 4 g + r
      // for d-blocks 4 a .. 4 a + 3
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        if (u + 2 < 16) {
          const int w2 = u + 2;
          db[w2 % 3] = *(const f32x4*)(Ds + ln.rowc[w2 >> 2] + (w2 & 3) * 256);
          qb[w2 % 3] = *(const f32x4*)(Qs + ln.rowc[w2 >> 2] + (w2 & 3) * 256);
        }
        const int r = u >> 2, a = u & 3;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          dva[4 * a + bb] = mfma16(db[u % 3][bb], pr[r], dva[4 * a + bb]);
          dka[4 * a + bb] = mfma16(qb[u % 3][bb], ds[r], dka[4 * a + bb]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    rb = rbn;
    hh = hhn;
    st ^= 1;
  }
  wait_vm0();  // the V copy is still in flight when no row sees the block

  // lane holds dK^T[d = 64 a + 16 g + 4 r + b][key] in dka[4 a + b][r]
  if (key < p.Lk) {
    const float sc = kInvSqrtD;
    float* dkr = (float*)bp.dk + (kv_head * p.Lk + key) * kD;
    float* dvr = (float*)bp.dv + (kv_head * p.Lk + key) * kD;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d0 = 64 * a + 16 * g + 4 * r;
        *(f32x4*)(dkr + d0) = f32x4{dka[4 * a][r] * sc, dka[4 * a + 1][r] * sc, dka[4 * a + 2][r] * sc,
                                    dka[4 * a + 3][r] * sc};
        *(f32x4*)(dvr + d0) = f32x4{dva[4 * a][r], dva[4 * a + 1][r], dva[4 * a + 2][r], dva[4 * a + 3][r]};
      }
  }
}

}  // namespace gqa
