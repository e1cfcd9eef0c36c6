// bwd_h16.hpp -- backward of the causal grouped-query attention for 16-bit
// inputs (bf16 or fp16): dQ, dK, dV in the input type, fp32 accumulation, on
// gfx950 32x32x16 MFMA. The same two-kernel split as the fp32 backward (no
// atomics): a dQ kernel over query blocks that also writes delta = dO . O, then
// a dK/dV kernel over key blocks that sums the query heads of each key/value
// head in registers.
//
// MFMA 32x32x16 layouts (lane l, l32 = l % 32, g = l / 32): A operand
// A[l32][k = 8 g .. 8 g + 7], B operand B[k = 8 g .. 8 g + 7][l32], result
// register r at row 8 (r / 4) + 4 g + r % 4, column l32. A contraction index
// may be assigned to the k slots in any order as long as A and B agree:
//  * d-contractions (scores, dP): step c contracts d = 16 c + 8 g .. + 7, a
//    16-byte chunk of a row;
//  * key / row contractions (dQ, dK, dV): quarter h of a 32-entry block
//    contracts entries 16 h + 4 g + 0..3 and 16 h + 8 + 4 g + 0..3, which is
//    where the score product left them (registers 8 h .. 8 h + 7); the other
//    operand then needs 4 consecutive rows of one d per lane, which the
//    transposing LDS read ds_read_b64_tr_b16 delivers.
// Why 32-row (32-key) waves: the 16-bit products run 16 times faster than the
// fp32 ones while the LDS bandwidth is the same, and a 32x32x16 product takes
// a 1 KB LDS fragment for twice the flops of a 16x16x32 one.
//
// LDS rows are 512 bytes (32 chunks of 16 B); chunk c of row x is stored at
// c ^ swz16(x), swz16(x) = 4 (x % 4) + (x / 4) % 4. The row reads (16
// consecutive rows at one chunk per clock) and the transposing reads (4
// consecutive rows x 4 chunks per clock) are both conflict-free under it, so
// one tile serves both read shapes.
#pragma once
#include "common.hpp"
#include "elem16.hpp"

namespace gqa {

constexpr int kWavesH = 4;                              // both kernels: one wave per SIMD
constexpr int kRowsDQH = 32;                            // dQ kernel: query rows per wave
constexpr int kBkH = 64;                                // dQ kernel: keys per LDS tile
constexpr int kKeysDKVH = 32;                           // dK/dV kernel: keys per wave
constexpr int kKeysBlockDKVH = kWavesH * kKeysDKVH;     // keys per dK/dV workgroup
constexpr int kRowsDKVH = 32;                           // dK/dV kernel: query rows per LDS tile
constexpr int kRowB16 = kD * 2;                         // bytes per 16-bit row

typedef __attribute__((address_space(3))) const char lds_c16;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4b;
typedef __attribute__((ext_vector_type(4))) int i32x4b;

__device__ __forceinline__ int swz16(int x) { return ((x & 3) << 2) | ((x >> 2) & 3); }

// Per-lane read pointers into one swizzled region (set once per region):
//  row[j]: row l32, chunk 2 c + g for c % 8 = j; chunk c adds 256 (c / 8),
//          row block (32 rows) b adds 16384 b;
//  tr[hi][j]: transposing read of rows 4 g' + 0..3 (+ 8 for hi) at d block n
//          (32 d) with n % 4 = j; n / 4 adds 256, row quarter h adds 8192 h.
// For the transposing read, the 16-lane group q = l / 16 covers rows
// 4 (q / 2) + 0..3 and d half q % 2; lane s of the group supplies row
// 4 (q / 2) + s / 4 and d 32 n + 16 (q % 2) + 4 (s % 4) .. + 3, and after the
// transpose lane s holds column s of the group's 4 x 16 block: lane l gets
// d 32 n + l32 of rows 4 g + 0..3.
struct Ptrs16 {
  lds_c16* row[8];
  lds_c16* tr[2][4];
  __device__ __forceinline__ void init(lds_c16* base, int lane) {
    const int l32 = lane & 31, g = lane >> 5;
#pragma unroll
    for (int j = 0; j < 8; ++j) row[j] = base + l32 * kRowB16 + (((2 * j + g) ^ swz16(l32)) << 4);
    const int q = lane >> 4, s = lane & 15, i = s >> 2;
    const int cw = 2 * (q & 1) + ((s & 3) >> 1);
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int rw = 4 * (q >> 1) + i + 8 * hi;  // row within the quarter
      const int a = (rw >> 2) & 3;
#pragma unroll
      for (int j = 0; j < 4; ++j) tr[hi][j] = base + rw * kRowB16 + ((4 * (j ^ i) + (cw ^ a)) << 4) + ((s & 1) << 3);
    }
  }
};

// Row fragment: chunk 2 c + g of row l32 of row block rb, at byte offset `off` from the region.
template <typename V8>
__device__ __forceinline__ V8 row_frag(const Ptrs16& pt, int c, int rb, uint32_t off) {
  typedef __attribute__((address_space(3))) const V8 lds_v8;
  return *(lds_v8*)(pt.row[c & 7] + (off + (c >> 3) * 256 + rb * 32 * kRowB16));
}
// Transposed fragment of d block n over row quarter h (rows 16 h + 4 g + 0..3
// then 16 h + 8 + 4 g + 0..3), at byte offset `off` from the region.
template <typename V8>
__device__ __forceinline__ V8 tr_frag(const Ptrs16& pt, int n, int h, uint32_t off) {
  const uint32_t o = off + (n >> 2) * 256 + h * 16 * kRowB16;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4b*)(pt.tr[0][n & 3] + o));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4b*)(pt.tr[1][n & 3] + o));
  const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
  return __builtin_bit_cast(V8, u32x4{lo2[0], lo2[1], hi2[0], hi2[1]});
}

// Async copy of rows [r0, r0 + 2 * nblk) of a 16-bit tensor region into a
// swizzled LDS region: block b (1 KB, rows 2 b and 2 b + 1) goes to
// lds + 1024 b; lane l writes chunk l % 32 of row 2 b + l / 32, i.e. fetches
// global chunk (l % 32) ^ swz16(row). The resource bounds the rows: rows past
// it read zeros.
struct Copy16 {
  rsrc_t r;
  uint32_t lds;
  __device__ __forceinline__ void block(int b, int lane) const {
    const int row = 2 * b + (lane >> 5);
    const uint32_t src = (uint32_t)row * kRowB16 + ((uint32_t)((lane & 31) ^ swz16(row)) << 4);
    buf2lds16(r, src, lds + (uint32_t)b * 1024u);
  }
};

// ---------------------------------------------------------------------------
// dQ kernel: 4 waves x 32 query rows (one head each, like the forward);
// 64-key tiles, K and V double-buffered in LDS.
// ---------------------------------------------------------------------------
struct SmemDQH {
  __attribute__((aligned(16))) char k[2][kBkH * kRowB16];
  __attribute__((aligned(16))) char v[2][kBkH * kRowB16];
  __attribute__((aligned(16))) int segk[2][kBkH];
  SegBits bits;
};

template <typename E, bool SEG>
__global__ __launch_bounds__(kWavesH * 64) void bwd_dq_h16_kernel(BwdParams bp) {
  typedef typename Elem<E>::v8 V8;
  __shared__ SmemDQH sm;
  const FwdParams& p = bp.f;
  const Work w = decode_work(p);
  const int wave = wave_id(), lane = lane_id();
  const int l32 = lane & 31, g = lane >> 5;
  const int h = w.h0 + wave % p.hpc;
  const int64_t pw = w.p0 + (int64_t)(wave / p.hpc) * kRowsDQH;
  const int64_t row = pw + l32;
  const int64_t row_c = min(row, p.Lq - 1);

  const int64_t p_end = min(w.p0 + (int64_t)p.ppc, p.Lq);
  const int64_t kv_end = p.causal ? min(p.Lk, p.q_offset + p_end) : p.Lk;
  const int n_tiles = (int)((kv_end + kBkH - 1) / kBkH);
  const int sh = SEG ? seg_shift(n_tiles) : 0;
  if (SEG) seg_scan<kWavesH, kBkH>(sm.bits, sh, p, w, n_tiles);

  const int64_t kv_head = (int64_t)w.b * p.Hkv + w.kvh;
  const char* kbase = (const char*)p.k + kv_head * p.Lk * kRowB16;
  const char* vbase = (const char*)p.v + kv_head * p.Lk * kRowB16;
  const int32_t* skb = SEG ? p.seg_k + (int64_t)w.b * p.Lk : nullptr;
  const int sq = SEG ? p.seg_q[(int64_t)w.b * p.Lq + row_c] : 0;

  // Q and dO of the lane's row (B-operand layout: chunk 2 c + g); delta = dO . O
  const int64_t hq = ((int64_t)w.b * p.Hq + h) * p.Lq;
  V8 qf[16], df[16];
  float delta;
  {
    const V8* qr = (const V8*)((const char*)p.q + (hq + row_c) * kRowB16);
    const V8* dr = (const V8*)((const char*)bp.dout + (hq + row_c) * kRowB16);
    const V8* orow = (const V8*)((const char*)p.o + (hq + row_c) * kRowB16);
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      qf[c] = qr[2 * c + g];
      df[c] = dr[2 * c + g];
      const u32x4 du = __builtin_bit_cast(u32x4, df[c]), ou = __builtin_bit_cast(u32x4, orow[2 * c + g]);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = Elem<E>::dot2(du[e], ou[e], acc);
    }
    delta = xor32_sum(acc);
    if (g == 0 && row < p.Lq) bp.delta[hq + row] = delta;
  }
  const float lse = p.lse[hq + row_c];
  const float lse2 = lse == -INFINITY ? 0.f : lse * 1.4426950408889634f;
  const float sl2 = p.scale_log2;
  wait_vm0_known();

  f32x16 acc[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    acc[n] = f32x16{};
    asm volatile("" : "+a"(acc[n]));
  }
  Ptrs16 pk0, pv0;  // K and V stage 0 (stage 1 adds the stage size)
  pk0.init((lds_c16*)sm.k[0], lane);
  pv0.init((lds_c16*)sm.v[0], lane);
  const uint32_t kst_lds = lds_addr(sm.k[0]), vst_lds = lds_addr(sm.v[0]), sst_lds = lds_addr(sm.segk[0]);
  constexpr uint32_t kStage = kBkH * kRowB16;

  auto copy_of = [&](int t, int st, bool valid, Copy16& ck, Copy16& cv, rsrc_t& rs) {
    const int64_t keys = valid ? min((int64_t)kBkH, p.Lk - (int64_t)t * kBkH) : 0;
    const int64_t off = valid ? (int64_t)t * kBkH * kRowB16 : 0;
    ck.r = make_rsrc(kbase + off, (uint32_t)keys * kRowB16);
    ck.lds = kst_lds + (uint32_t)st * kStage;
    cv.r = make_rsrc(vbase + off, (uint32_t)keys * kRowB16);
    cv.lds = vst_lds + (uint32_t)st * kStage;
    rs = make_rsrc(SEG ? (const void*)(skb + (valid ? (int64_t)t * kBkH : 0)) : (const void*)kbase,
                   SEG ? (uint32_t)keys * 4u : 0u);
  };

  int t = SEG ? seg_next(sm.bits, sh, 0, n_tiles) : 0;
  int st = 0;
  if (t < n_tiles) {
    Copy16 ck, cv;
    rsrc_t rs;
    copy_of(t, 0, true, ck, cv, rs);
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      ck.block(8 * wave + it, lane);
      cv.block(8 * wave + it, lane);
    }
    if (SEG && wave == kWavesH - 1) buf2lds4(rs, (uint32_t)lane * 4u, sst_lds);
  }
  while (t < n_tiles) {
    const int tn = SEG ? seg_next(sm.bits, sh, t + 1, n_tiles) : t + 1;
    wait_vm0();
    __syncthreads();
    Copy16 ck, cv;
    rsrc_t rs;
    copy_of(tn, st ^ 1, tn < n_tiles, ck, cv, rs);
    if (SEG && wave == kWavesH - 1) buf2lds4(rs, (uint32_t)lane * 4u, sst_lds + (uint32_t)(st ^ 1) * (kBkH * 4));
    const int64_t k0 = (int64_t)t * kBkH;
    const uint32_t so = (uint32_t)st * kStage;

    // mask of the tile in 32 bits: key 32 j + 8 (r / 4) + 4 g + r % 4 of the
    // tile is visible to the lane's row iff it is below kl (causal and Lk) and
    // (with ids) its id equals the row's
    const bool seg_elem = SEG && !seg_full_tile(sm.bits, sh, t);
    const int64_t kend = p.causal ? min(p.Lk, p.q_offset + row + 1) : p.Lk;
    const int kl = (int)max((int64_t)0, min((int64_t)kBkH, kend - k0));

    // S^T = K Q^T, two key halves (2 chains of 16 products); lane holds key
    // 32 j + 8 (r / 4) + 4 g + r % 4 of its row. K fragments two steps ahead;
    // the K copies of the next tile spread over the steps.
    f32x16 s[2], dp[2];
    {
      V8 kr[3][2];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < 2; ++j) kr[u][j] = row_frag<V8>(pk0, u, j, so);
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        if (c + 2 < 16) {
#pragma unroll
          for (int j = 0; j < 2; ++j) kr[(c + 2) % 3][j] = row_frag<V8>(pk0, c + 2, j, so);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) s[j] = Elem<E>::mfma(kr[c % 3][j], qf[c], c == 0 ? f32x16{} : s[j]);
        if ((c & 1) == 0) ck.block(8 * wave + (c >> 1), lane);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // dP^T = V dO^T (2 chains of 16) with P^T = exp2(S^T log2(e)/sqrt(D) -
    // lse log2(e)) formed beside them, one score per product (score e is
    // s[e / 16][e % 16]); the V copies of the next tile spread over the steps;
    // key ids of the 4-key group of a score read one group ahead.
    float pv[32];
    {
      V8 vr[3][2];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < 2; ++j) vr[u][j] = row_frag<V8>(pv0, u, j, so);
      i32x4b id4[2];
      id4[0] = i32x4b{sq, sq, sq, sq};
      if (seg_elem) id4[0] = *(const i32x4b*)(&sm.segk[st][4 * g]);
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        if (c + 2 < 16) {
#pragma unroll
          for (int j = 0; j < 2; ++j) vr[(c + 2) % 3][j] = row_frag<V8>(pv0, c + 2, j, so);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          dp[j] = Elem<E>::mfma(vr[c % 3][j], df[c], c == 0 ? f32x16{} : dp[j]);
          const int e = 2 * c + j, je = e >> 4, re = e & 15, grp = e >> 2;
          if ((e & 3) == 1 && grp + 1 < 8) {
            const int gn = grp + 1;  // group gn: half gn / 4, registers 4 (gn % 4) ..
            id4[gn & 1] = i32x4b{sq, sq, sq, sq};
            if (seg_elem) id4[gn & 1] = *(const i32x4b*)(&sm.segk[st][32 * (gn >> 2) + 8 * (gn & 3) + 4 * g]);
          }
          const int rk = 32 * je + 8 * (re >> 2) + 4 * g + (re & 3);
          float sv = s[je][re];
          asm volatile("" : "+v"(sv));  // the score's VGPR copy, taken at its slot
          const float x = fast_exp2(fmaf(sv, sl2, -lse2));
          pv[e] = (rk < kl && id4[grp & 1][re & 3] == sq) ? x : 0.f;
        }
        if ((c & 1) == 1) cv.block(8 * wave + (c >> 1), lane);
        __builtin_amdgcn_sched_barrier(0);
      }
      // S keeps AGPRs of its own through the loop (dP's products do not
      // reuse them)
      asm volatile("" ::"a"(s[0]), "a"(s[1]));
    }
    // dS^T = P^T (dP^T - delta), packed in pairs; key quarter h in dsk[4 h ..].
    // Quarter 0 before the dQ products; quarters 1-3 beside the products of
    // the quarter before (one pair every other product), each pair's dP read
    // out of the AGPRs at its slot. Formed all at once, the 32 reads and the
    // VALU work left the matrix core idle before the first dQ product.
    unsigned dsk[16];
    auto ds_pair = [&](int f) {  // pair f: scores 2 f and 2 f + 1
      const int e = 2 * f;
      float d0 = dp[e >> 4][e & 15], d1 = dp[e >> 4][(e + 1) & 15];
      asm volatile("" : "+v"(d0), "+v"(d1));
      dsk[f] = Elem<E>::pack(pv[e] * (d0 - delta), pv[e + 1] * (d1 - delta));
    };
#pragma unroll
    for (int f = 0; f < 4; ++f) ds_pair(f);
    __builtin_amdgcn_sched_barrier(0);

    // dQ^T += K^T dS^T: 4 key quarters x 8 d blocks; K^T fragments through the
    // transposing read, two products ahead
    V8 kt[3];
    kt[0] = tr_frag<V8>(pk0, 0, 0, so);
    kt[1] = tr_frag<V8>(pk0, 1, 0, so);
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      if (u + 2 < 32) kt[(u + 2) % 3] = tr_frag<V8>(pk0, (u + 2) & 7, (u + 2) >> 3, so);
      const int n = u & 7, hq4 = u >> 3;
      const V8 b = __builtin_bit_cast(V8, u32x4{dsk[4 * hq4], dsk[4 * hq4 + 1], dsk[4 * hq4 + 2], dsk[4 * hq4 + 3]});
      acc[n] = Elem<E>::mfma(kt[u % 3], b, acc[n]);
      if (u < 24 && (u & 1) == 0) ds_pair(4 * (hq4 + 1) + ((u & 7) >> 1));
      __builtin_amdgcn_sched_barrier(0);
    }
    t = tn;
    st ^= 1;
  }

  // dQ = acc / sqrt(D) in E: lane holds dQ[row][32 n + 8 j + 4 g + i] in acc[n][4 j + i]
#pragma unroll
  for (int n = 0; n < 8; ++n) asm volatile("" : "+a"(acc[n]));
  if (row < p.Lq) {
    char* qp = (char*)bp.dq + (hq + row) * kRowB16;
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x2 val = {Elem<E>::pack(acc[n][4 * j] * kInvSqrtD, acc[n][4 * j + 1] * kInvSqrtD),
                           Elem<E>::pack(acc[n][4 * j + 2] * kInvSqrtD, acc[n][4 * j + 3] * kInvSqrtD)};
        *(u32x2*)(qp + (32 * n + 8 * j + 4 * g) * 2) = val;
      }
  }
}

// ---------------------------------------------------------------------------
// dK/dV kernel: 4 waves x 32 keys of one key/value head; K in registers, V of
// the 128 keys in LDS; 32-row tiles of Q, dO (one query head each),
// double-buffered, walked from the last rows down; dK^T, dV^T in AGPRs.
// ---------------------------------------------------------------------------
struct SmemDKVH {
  __attribute__((aligned(16))) char v[kKeysBlockDKVH * kRowB16];
  __attribute__((aligned(16))) char q[2][kRowsDKVH * kRowB16];
  __attribute__((aligned(16))) char d[2][kRowsDKVH * kRowB16];
  __attribute__((aligned(16))) float lse[2][64];    // 64 slots (one per lane of the copy), 32 used
  __attribute__((aligned(16))) float delta[2][64];
  __attribute__((aligned(16))) int segq[2][64];
  SegBits bits;
};

template <typename E, bool SEG>
__global__ __launch_bounds__(kWavesH * 64) void bwd_dkv_h16_kernel(BwdParams bp) {
  typedef typename Elem<E>::v8 V8;
  __shared__ SmemDKVH sm;
  const FwdParams& p = bp.f;
  const int kbk = blockIdx.x / bp.BH;
  const int bh = blockIdx.x % bp.BH;
  const int kvh = bh % p.Hkv, b = bh / p.Hkv;
  const int wave = wave_id(), lane = lane_id();
  const int l32 = lane & 31, g = lane >> 5;
  const int64_t j0 = (int64_t)kbk * kKeysBlockDKVH;
  const int64_t kw0 = j0 + (int64_t)wave * kKeysDKVH;
  const int64_t key = kw0 + l32;
  const int64_t key_c = min(key, p.Lk - 1);

  const int64_t r_first = p.causal ? max((int64_t)0, j0 - p.q_offset) : 0;
  const int rb0 = (int)(r_first / kRowsDKVH);
  const int n_rb = (int)((p.Lq + kRowsDKVH - 1) / kRowsDKVH);
  const int sh = SEG ? seg_shift(n_rb) : 0;
  // the row ids' index, where the call brings one (rows of ceil(Lq / 16) entries per batch)
  const SegBlk* qix = p.seg_q_idx ? p.seg_q_idx + (int64_t)b * ((p.Lq + kSegBlk - 1) / kSegBlk) : nullptr;
  if (SEG)
    seg_scan_any<kWavesH * 64, kRowsDKVH>(sm.bits, sh, p.seg_k + (int64_t)b * p.Lk, j0, kKeysBlockDKVH, p.Lk,
                                          p.seg_q + (int64_t)b * p.Lq, qix, p.Lq, n_rb, rb0);
  const int sk = SEG ? p.seg_k[(int64_t)b * p.Lk + key_c] : 0;

  // K of the lane's key (B-operand layout: chunk 2 c + g); V of the block's
  // 128 keys into LDS (keys past Lk read zeros)
  const int64_t kv_head = (int64_t)b * p.Hkv + kvh;
  V8 kf[16];
  {
    const V8* kr = (const V8*)((const char*)p.k + (kv_head * p.Lk + key_c) * kRowB16);
#pragma unroll
    for (int c = 0; c < 16; ++c) kf[c] = kr[2 * c + g];
    const int64_t nkeys = max((int64_t)0, min((int64_t)kKeysBlockDKVH, p.Lk - j0));
    Copy16 cvb;
    cvb.r = make_rsrc((const char*)p.v + (kv_head * p.Lk + j0) * kRowB16, (uint32_t)nkeys * kRowB16);
    cvb.lds = lds_addr(sm.v);
#pragma unroll
    for (int it = 0; it < 16; ++it) cvb.block(16 * wave + it, lane);
  }
  wait_vm0_known();
  f32x16 dka[8], dva[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    dka[n] = f32x16{};
    dva[n] = f32x16{};
    asm volatile("" : "+a"(dka[n]), "+a"(dva[n]));
  }
  const float sl2 = p.scale_log2;
  const int n_rep = p.n_rep;
  const int h0 = kvh * n_rep;

  Ptrs16 pq0, pd0, pvw;
  pq0.init((lds_c16*)sm.q[0], lane);
  pd0.init((lds_c16*)sm.d[0], lane);
  pvw.init((lds_c16*)(sm.v + wave * kKeysDKVH * kRowB16), lane);
  const uint32_t q_lds = lds_addr(sm.q[0]), d_lds = lds_addr(sm.d[0]);
  constexpr uint32_t kStage = kRowsDKVH * kRowB16;

  // Q, dO rows of tile (rows i0.., head hh) for stage st: 16 blocks of 1 KB per
  // tensor, 4 per wave each; lse, delta and row ids by wave 0 (64 lanes, 64
  // slots, 32 used). live == false: size-0 resources, zeros into the idle stage.
  auto rows_of = [&](int hh, int64_t i0, int st, bool live, Copy16& cq, Copy16& cd) {
    const int64_t hq = ((int64_t)b * p.Hq + h0 + hh) * p.Lq;
    const int64_t nrows = live ? max((int64_t)0, p.Lq - i0) : 0;
    const uint32_t nb = (uint32_t)min(nrows, (int64_t)kRowsDKVH) * kRowB16;
    const int64_t off = live ? (hq + i0) * kRowB16 : 0;
    cq.r = make_rsrc((const char*)p.q + off, nb);
    cq.lds = q_lds + (uint32_t)st * kStage;
    cd.r = make_rsrc((const char*)bp.dout + off, nb);
    cd.lds = d_lds + (uint32_t)st * kStage;
  };
  auto rowdata = [&](int hh, int64_t i0, int st) {
    const int64_t hq = ((int64_t)b * p.Hq + h0 + hh) * p.Lq;
    const uint32_t off = (uint32_t)(i0 + lane) * 4u, nb = (uint32_t)(p.Lq * 4);
    buf2lds4(make_rsrc(p.lse + hq, nb), off, lds_addr(sm.lse[st]));
    buf2lds4(make_rsrc(bp.delta + hq, nb), off, lds_addr(sm.delta[st]));
    if (SEG) buf2lds4(make_rsrc(p.seg_q + (int64_t)b * p.Lq, nb), off, lds_addr(sm.segq[st]));
  };

  int rb = SEG ? seg_prev(sm.bits, sh, n_rb - 1, rb0) : n_rb - 1;
  int hh = 0;
  int st = 0;
  if (rb >= rb0) {
    Copy16 cq, cd;
    rows_of(0, (int64_t)rb * kRowsDKVH, 0, true, cq, cd);
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      cq.block(4 * wave + it, lane);
      cd.block(4 * wave + it, lane);
    }
    if (wave == 0) rowdata(0, (int64_t)rb * kRowsDKVH, 0);
  }
  while (rb >= rb0) {
    int rbn = rb, hhn = hh + 1;
    if (hhn == n_rep) {
      hhn = 0;
      rbn = SEG ? seg_prev(sm.bits, sh, rb - 1, rb0) : rb - 1;
    }
    const bool have_next = rbn >= rb0;
    wait_vm0();
    __syncthreads();
    if (have_next && wave == 0) rowdata(hhn, (int64_t)rbn * kRowsDKVH, st ^ 1);
    Copy16 cq, cd;
    rows_of(hhn, (int64_t)rbn * kRowsDKVH, st ^ 1, have_next, cq, cd);
    const int64_t i0 = (int64_t)rb * kRowsDKVH;
    const uint32_t so = (uint32_t)st * kStage;

    // mask limits of the tile (32-bit): row ri of the tile sees the lane's key
    // iff lim <= ri < nrow and (with ids) the row's id equals the key's
    const bool seg_elem = SEG && !seg_full_tile(sm.bits, sh, rb);
    const bool need_mask = seg_elem || i0 + kRowsDKVH > p.Lq || (p.causal && kw0 + kKeysDKVH - 1 > p.q_offset + i0);
    const int lim = (p.causal && need_mask)
                        ? (int)max((int64_t)-1, min((int64_t)kRowsDKVH, key - p.q_offset - i0))
                        : -1;
    const int nrow = (int)min((int64_t)kRowsDKVH, p.Lq - i0);

    // S = Q K^T (16 products, one chain): lane holds row 8 (r / 4) + 4 g + r % 4
    // of its key. Q fragments two steps ahead; the next tile's copies spread
    // over the steps.
    f32x16 s, dp;
    {
      V8 qr[3];
      qr[0] = row_frag<V8>(pq0, 0, 0, so);
      qr[1] = row_frag<V8>(pq0, 1, 0, so);
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        if (c + 2 < 16) qr[(c + 2) % 3] = row_frag<V8>(pq0, c + 2, 0, so);
        s = Elem<E>::mfma(qr[c % 3], kf[c], c == 0 ? f32x16{} : s);
        // steps 4 k: Q block k of this wave; steps 4 k + 2: dO block k
        if ((c & 3) == 0) cq.block(4 * wave + (c >> 2), lane);
        if ((c & 3) == 2) cd.block(4 * wave + (c >> 2), lane);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // dP = dO V^T (16 products) with P = exp2(S log2(e)/sqrt(D) - lse log2(e))
    // formed beside them (P needs only S): register r at step r. The lse (and
    // ids) of the 4 rows of register group r / 4 are read one group ahead.
    float pv[16];
    {
      V8 dr[3], vr[3];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        dr[u] = row_frag<V8>(pd0, u, 0, so);
        vr[u] = row_frag<V8>(pvw, u, 0, 0);
      }
      f32x4 l4[2];
      i32x4b id4[2];
      l4[0] = *(const f32x4*)(&sm.lse[st][4 * g]);
      id4[0] = i32x4b{sk, sk, sk, sk};
      if (seg_elem) id4[0] = *(const i32x4b*)(&sm.segq[st][4 * g]);
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        if (c + 2 < 16) {
          dr[(c + 2) % 3] = row_frag<V8>(pd0, c + 2, 0, so);
          vr[(c + 2) % 3] = row_frag<V8>(pvw, c + 2, 0, 0);
        }
        if ((c & 3) == 1 && c < 12) {
          const int j = (c >> 2) + 1;
          l4[j & 1] = *(const f32x4*)(&sm.lse[st][8 * j + 4 * g]);
          id4[j & 1] = i32x4b{sk, sk, sk, sk};
          if (seg_elem) id4[j & 1] = *(const i32x4b*)(&sm.segq[st][8 * j + 4 * g]);
        }
        dp = Elem<E>::mfma(dr[c % 3], vr[c % 3], c == 0 ? f32x16{} : dp);
        {
          const int j = c >> 2, i = c & 3, ri = 8 * j + 4 * g + i;
          const float lv = l4[j & 1][i];
          const float l2 = lv == -INFINITY ? 0.f : lv * 1.4426950408889634f;
          const float x = fast_exp2(fmaf(s[c], sl2, -l2));
          pv[c] = (ri < nrow && ri >= lim && id4[j & 1][i] == sk) ? x : 0.f;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // dS = P (dP - delta); P and dS packed in pairs, row quarter h in pk/dk[4 h ..]
    unsigned pk[8], dk[8];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const f32x4 d4 = *(const f32x4*)(&sm.delta[st][8 * r4 + 4 * g]);
      float dsv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) dsv[i] = pv[4 * r4 + i] * (dp[4 * r4 + i] - d4[i]);
      pk[2 * r4] = Elem<E>::pack(pv[4 * r4], pv[4 * r4 + 1]);
      pk[2 * r4 + 1] = Elem<E>::pack(pv[4 * r4 + 2], pv[4 * r4 + 3]);
      dk[2 * r4] = Elem<E>::pack(dsv[0], dsv[1]);
      dk[2 * r4 + 1] = Elem<E>::pack(dsv[2], dsv[3]);
    }
    __builtin_amdgcn_sched_barrier(0);

    // dV^T += dO^T P and dK^T += Q^T dS: 2 row quarters x 8 d blocks each;
    // dO^T and Q^T through the transposing read, one step ahead
    V8 dt[2], qt[2];
    dt[0] = tr_frag<V8>(pd0, 0, 0, so);
    qt[0] = tr_frag<V8>(pq0, 0, 0, so);
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      if (u + 1 < 16) {
        dt[(u + 1) & 1] = tr_frag<V8>(pd0, (u + 1) & 7, (u + 1) >> 3, so);
        qt[(u + 1) & 1] = tr_frag<V8>(pq0, (u + 1) & 7, (u + 1) >> 3, so);
      }
      const int n = u & 7, hq4 = u >> 3;
      const V8 pb = __builtin_bit_cast(V8, u32x4{pk[4 * hq4], pk[4 * hq4 + 1], pk[4 * hq4 + 2], pk[4 * hq4 + 3]});
      const V8 db = __builtin_bit_cast(V8, u32x4{dk[4 * hq4], dk[4 * hq4 + 1], dk[4 * hq4 + 2], dk[4 * hq4 + 3]});
      dva[n] = Elem<E>::mfma(dt[u & 1], pb, dva[n]);
      dka[n] = Elem<E>::mfma(qt[u & 1], db, dka[n]);
      __builtin_amdgcn_sched_barrier(0);
    }
    rb = rbn;
    hh = hhn;
    st ^= 1;
  }
  wait_vm0();  // the V copy is still in flight when no row sees the block

  // lane holds dK^T[d = 32 n + 8 j + 4 g + i][key] in dka[n][4 j + i]
#pragma unroll
  for (int n = 0; n < 8; ++n) asm volatile("" : "+a"(dka[n]), "+a"(dva[n]));
  if (key < p.Lk) {
    char* kp = (char*)bp.dk + (kv_head * p.Lk + key) * kRowB16;
    char* vp = (char*)bp.dv + (kv_head * p.Lk + key) * kRowB16;
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d0 = 32 * n + 8 * j + 4 * g;
        const u32x2 kv = {Elem<E>::pack(dka[n][4 * j] * kInvSqrtD, dka[n][4 * j + 1] * kInvSqrtD),
                          Elem<E>::pack(dka[n][4 * j + 2] * kInvSqrtD, dka[n][4 * j + 3] * kInvSqrtD)};
        const u32x2 vv = {Elem<E>::pack(dva[n][4 * j], dva[n][4 * j + 1]),
                          Elem<E>::pack(dva[n][4 * j + 2], dva[n][4 * j + 3])};
        *(u32x2*)(kp + d0 * 2) = kv;
        *(u32x2*)(vp + d0 * 2) = vv;
      }
  }
}

}  // namespace gqa
