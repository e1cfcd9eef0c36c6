// decode_h16.hpp -- causal grouped-query attention forward for short query
// blocks (decoding: fewer than 32 positions) over long key sequences, 16-bit
// inputs (bf16 or fp16), fp32 accumulation, on the 16x16x32 MFMA of gfx950.
// The arithmetic is that of the long-block kernel (fwd_h16.hpp): scores in the
// base-2 domain, online softmax with the lazy rescale, P rounded to the input
// type (RNE) for the PV product, l from the unrounded p for the lse.
//
// The query rows of one KV head (its n_rep heads x Lq positions) are packed
// into blocks of 64: row rr of a block is head rr / Lq of the group at
// position rr % Lq. Heads are stored one after another and positions in
// order, so a block is one contiguous run of rows of Q (and of O). One
// workgroup = 4 waves x 16 rows = one block, over one key range (a split).
// Per key tile of 32 keys a wave forms S^T = K Q^T (2 key halves x 8 d slices
// of 16x16x32 products), the softmax of its 16 rows, and O^T += V^T P^T
// (16 d blocks, one 32-key product each). The 16-row product fits these rows:
// the 32-row tiles of the long-block kernel would be half empty at 16
// positions. Every K/V byte copied into LDS serves all query heads of the
// group.
//
// The work is bound by the K/V stream from HBM (1 KB per key, read once), and
// the bytes a compute unit keeps in flight set its share of the bandwidth. A
// ring of 5 LDS stages of one tile each (K then V, 32 KB: all 160 KB of LDS)
// keeps the copies of 4 tiles in flight per workgroup while the 5th is
// computed, with one workgroup barrier per tile. Q arrives by the same kind of
// copy into the 5th stage, issued with the first tiles' copies so that one
// wait covers both; once every wave holds its Q in registers (a second
// barrier, in the first step only) that stage joins the ring.
#pragma once
#include "common.hpp"
#include "elem16.hpp"

namespace gqa {

constexpr int kDecWaves = 4;                        // waves per workgroup
constexpr int kDecRows = 16;                        // query rows per wave
constexpr int kDecBlockRows = kDecWaves * kDecRows;  // 64 packed rows per workgroup
constexpr int kDecBk = 32;                          // keys per tile
constexpr int kDecStages = 5;                       // LDS ring depth (tiles)
constexpr int kDecPart = kDecBk * kD * 2;           // 16 KB: the K (or V) part of a tile
constexpr int kDecStage = 2 * kDecPart;             // 32 KB: K then V
constexpr int kDecCopies = kDecPart / 1024 / kDecWaves;        // 1 KB copies per wave per part (4)
constexpr int kDecQCopies = kDecBlockRows * kD * 2 / 1024 / kDecWaves;  // per wave for Q (8)
// copies a wave issues per tile; the wait at the top of a step leaves the
// last three tiles' copies in flight
constexpr int kDecTileCopies = 2 * kDecCopies;
static_assert(kDecTileCopies * (kDecStages - 2) == 24, "the s_waitcnt immediates below assume 24");
static_assert(kDecBlockRows * kD * 2 == kDecStage, "Q of a row block fills one stage");
constexpr float kDecLazy = 8.0f;  // lazy-rescale threshold (log2 units), as in the long-block kernel

// LDS image: 512-byte rows (keys, or Q rows) of 32 chunks of 16 bytes. K and Q
// store chunk c of row r at c ^ (r % 16): a 16-byte-per-lane read of 16 rows
// at one chunk (16 lanes per clock) then meets all 64 banks once. V stores
// chunk c of key k at c ^ 2 (k % 8): a transposing read (32 lanes per clock)
// takes 8 keys x 32 bytes at one d offset, and the XOR puts the 8 keys' 32
// bytes in 8 different bank groups.
__device__ __forceinline__ int dec_swz_k(int row) { return row & 15; }
__device__ __forceinline__ int dec_swz_v(int key) { return (key & 7) << 1; }

struct DecSmem {
  __attribute__((aligned(16))) char stage[kDecStages][kDecStage];  // Q first lands in the last one
};

template <typename E>
struct Dec16;
template <>
struct Dec16<__bf16> {
  static __device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct Dec16<_Float16> {
  static __device__ __forceinline__ f32x4 mfma(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

typedef __attribute__((address_space(3))) const char dec_lds_cchar;
typedef __attribute__((address_space(3))) s16x4 dec_lds_s16x4;

template <typename E>
__global__ __launch_bounds__(kDecWaves * 64) void decode_h16_kernel(FwdParams p) {
  typedef typename Elem<E>::v8 V8;
  typedef __attribute__((address_space(3))) const V8 lds_v8;
  __shared__ DecSmem sm;
  const int wave = wave_id(), lane = lane_id();
  const int r16 = lane & 15, g = lane >> 4, hi = lane >> 5;

  // which (batch, KV head), row block and key split this workgroup owns
  const int n_split = p.n_split > 1 ? p.n_split : 1;
  const int split = (int)blockIdx.x % n_split;
  const int rest = (int)blockIdx.x / n_split;
  const int rb = rest % p.n_qb;
  const int bh = rest / p.n_qb;
  const int b = bh / p.Hkv, kvh = bh % p.Hkv;
  // packed rows of the group (n_rep <= 64 heads x Lq < 32 positions: 32-bit)
  const int R = p.n_rep * (int)p.Lq;
  const int row0 = rb * kDecBlockRows;  // first packed row of the block
  const int64_t grow0 = ((int64_t)b * p.Hq + (int64_t)kvh * p.n_rep) * p.Lq;  // global row of packed row 0

  // this lane's row (wave rows 16 wave .. + 15) and its last visible key
  const int rr = row0 + wave * kDecRows + r16;
  const bool row_ok = rr < R;
  const int64_t pos = row_ok ? (int64_t)(rr % (int)p.Lq) : 0;
  const int64_t kv_end = p.causal ? min(p.Lk, p.q_offset + p.Lq) : p.Lk;
  const int lim = (int)(p.causal ? min(p.q_offset + pos, p.Lk - 1) : p.Lk - 1);
  // tiles from this key on hold a key hidden from some row (causal or past Lk)
  const int mask_from = (int)(p.causal ? min(p.q_offset, p.Lk - 1) : p.Lk - 1);
  const int n_tiles = (int)((kv_end + kDecBk - 1) / kDecBk);
  const int t_lo = p.n_split > 1 ? split * p.split_tiles : 0;
  const int t_hi = p.n_split > 1 ? min(n_tiles, t_lo + p.split_tiles) : n_tiles;
  const int n = max(0, t_hi - t_lo);

  const int64_t kv_head = (int64_t)b * p.Hkv + kvh;
  const char* kbase = (const char*)p.k + kv_head * p.Lk * (kD * 2);
  const char* vbase = (const char*)p.v + kv_head * p.Lk * (kD * 2);

  // per-lane copy offsets: block 4 wave + it of a part holds rows 2 blk, 2 blk + 1;
  // lane l writes LDS chunk l % 32 of row 2 blk + l / 32 with global chunk (l % 32) ^ swz
  uint32_t ldk[kDecCopies], ldv[kDecCopies], ldq[kDecQCopies];
#pragma unroll
  for (int it = 0; it < kDecCopies; ++it) {
    const int key = 2 * (kDecCopies * wave + it) + hi;
    ldk[it] = (uint32_t)key * 512u + ((uint32_t)((lane & 31) ^ dec_swz_k(key)) << 4);
    ldv[it] = (uint32_t)key * 512u + ((uint32_t)((lane & 31) ^ dec_swz_v(key)) << 4);
  }
#pragma unroll
  for (int it = 0; it < kDecQCopies; ++it) {
    const int row = 2 * (kDecQCopies * wave + it) + hi;
    ldq[it] = (uint32_t)row * 512u + ((uint32_t)((lane & 31) ^ dec_swz_k(row)) << 4);
  }
  const uint32_t lds_stage0 = lds_addr(sm.stage[0]);

  // Copies of tile t (absolute) into stage st; a tile past this split's range
  // (or Lk) copies from a resource of size 0, which writes zeros, so every
  // step issues the same number of copies and the wait count stays fixed.
  auto copy_tile = [&](int st, int t) {
    const bool valid = t < t_hi;
    const uint32_t keys = valid ? min((uint32_t)p.Lk - (uint32_t)t * kDecBk, (uint32_t)kDecBk) : 0u;
    const uint64_t off = valid ? (uint64_t)(uint32_t)t * kDecPart : 0u;
    const rsrc_t rk = make_rsrc(kbase + off, keys * (kD * 2));
    const rsrc_t rv = make_rsrc(vbase + off, keys * (kD * 2));
    const uint32_t dst = lds_stage0 + (uint32_t)st * kDecStage + (uint32_t)(kDecCopies * wave) * 1024u;
#pragma unroll
    for (int it = 0; it < kDecCopies; ++it) {
      buf2lds16_imm(rk, ldk[it], dst, (uint32_t)it * 1024u);
      buf2lds16_imm(rv, ldv[it], dst + kDecPart, (uint32_t)it * 1024u);
    }
  };

  // Q of the block (rows past the group's end read as zeros) into the last
  // stage, then tiles 0..3 into stages 0..3
  dec_lds_cchar* const qlds = (dec_lds_cchar*)sm.stage[kDecStages - 1];
  {
    const int rows = min(kDecBlockRows, R - row0);
    const rsrc_t rq = make_rsrc((const char*)p.q + (grow0 + row0) * (kD * 2), (uint32_t)rows * (kD * 2));
    const uint32_t dst = lds_addr(sm.stage[kDecStages - 1]) + (uint32_t)(kDecQCopies * wave) * 1024u;
#pragma unroll
    for (int it = 0; it < kDecQCopies; ++it) buf2lds16_imm(rq, ldq[it], dst, (uint32_t)it * 1024u);
  }
#pragma unroll
  for (int j = 0; j < kDecStages - 1; ++j) copy_tile(j, t_lo + j);

  // LDS read addresses. K (and Q): row r16 (+16 for the second key half),
  // chunk 4 kk + g of d slice kk (32 d), stored at chunk (4 kk + g) ^ r16 =
  // 16 (kk / 4) + ((4 (kk % 4) + g) ^ r16). V (transposing read, 16-lane
  // group g, lane s = r16): key 4 g + s / 4 (+16), d 16 n + 4 (s % 4) .. + 3
  // of d block n, at byte 32 (n ^ x) + 8 (s % 4) of the key row (x = key % 8),
  // = 256 (n / 8) + 32 ((n % 8) ^ x) + 8 (s % 4).
  dec_lds_cchar* const st0 = (dec_lds_cchar*)sm.stage[0];
  dec_lds_cchar* kr[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) kr[j] = st0 + r16 * 512 + (((4 * j + g) ^ r16) << 4);
  const int vkey = 4 * g + (r16 >> 2), vx = vkey & 7;
  dec_lds_cchar* vr[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) vr[j] = st0 + kDecPart + vkey * 512 + ((j ^ vx) << 5) + ((r16 & 3) << 3);

  asm volatile("s_waitcnt vmcnt(24)" ::: "memory");  // this wave's Q and tile-0 copies have landed
  __syncthreads();                                    // ... and every wave's

  // Q^T as the B operand: lane holds Q[row 16 wave + r16][32 kk + 8 g .. + 7]
  V8 qf[8];
  {
    dec_lds_cchar* qb = qlds + (wave * kDecRows) * 512;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qf[kk] = *(lds_v8*)(qb + r16 * 512 + ((kk >> 2) << 8) + (((4 * (kk & 3) + g) ^ r16) << 4));
    // every wave's Q is in registers before the first copy into its stage
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __syncthreads();
  }

  const float sl2 = p.scale_log2;
  float m = -INFINITY, m_use = 0.f, l = 0.f, lr = 0.f;
  f32x4 acc[16];
#pragma unroll
  for (int nb = 0; nb < 16; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int i = 0, st = 0; i < n; ++i, st = st == kDecStages - 1 ? 0 : st + 1) {
    if (i > 0) {
      asm volatile("s_waitcnt vmcnt(24)" ::: "memory");  // tile i's copies have landed
      __syncthreads();  // ... for every wave; the stage of tile i - 1 is free
    }
    copy_tile(st == 0 ? kDecStages - 1 : st - 1, t_lo + i + kDecStages - 1);
    const int t = t_lo + i;
    const int so = st * kDecStage;

    // All 16 K fragments of the tile are read before the first product and
    // waited for once (one LDS latency per tile instead of one per product:
    // with one wave per SIMD nothing else would hide it).
    V8 kf[16];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      dec_lds_cchar* a = kr[kk & 3] + so + ((kk >> 2) << 8);
      kf[2 * kk] = *(lds_v8*)a;
      kf[2 * kk + 1] = *(lds_v8*)(a + 16 * 512);
    }
    asm volatile("" : "+v"(kf[0]), "+v"(kf[1]), "+v"(kf[2]), "+v"(kf[3]), "+v"(kf[4]), "+v"(kf[5]), "+v"(kf[6]),
                 "+v"(kf[7]), "+v"(kf[8]), "+v"(kf[9]), "+v"(kf[10]), "+v"(kf[11]), "+v"(kf[12]), "+v"(kf[13]),
                 "+v"(kf[14]), "+v"(kf[15]));
    // S^T = K Q^T: sa holds keys 4 g + 0..3, sb keys 16 + 4 g + 0..3 of row r16
    f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      sa = Dec16<E>::mfma(kf[2 * kk], qf[kk], sa);
      sb = Dec16<E>::mfma(kf[2 * kk + 1], qf[kk], sb);
    }
    // the V fragments (d block nb: keys 4 g + 0..3 then 16 + 4 g + 0..3) do not
    // depend on P: their reads go out now and land during the softmax
    V8 vf[16];
#pragma unroll
    for (int nb = 0; nb < 16; ++nb) {
      dec_lds_cchar* a = vr[nb & 7] + so + ((nb >> 3) << 8);
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((dec_lds_s16x4*)a);
      const s16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((dec_lds_s16x4*)(a + 16 * 512));
      const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), up2 = __builtin_bit_cast(u32x2, up);
      vf[nb] = __builtin_bit_cast(V8, u32x4{lo2[0], lo2[1], up2[0], up2[1]});
    }
    if (t * kDecBk + kDecBk - 1 > mask_from) {
      const int k0 = t * kDecBk + 4 * g;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sa[e] = k0 + e <= lim ? sa[e] : -INFINITY;
        sb[e] = k0 + 16 + e <= lim ? sb[e] : -INFINITY;
      }
    }
    // row max over the 4 lanes of the row, then the lazy update (the running
    // max moves only when a row's max grows by more than 8 in log2 units)
    float mx = fmaxf(fmaxf(fmaxf(sa[0], sa[1]), fmaxf(sa[2], sa[3])), fmaxf(fmaxf(sb[0], sb[1]), fmaxf(sb[2], sb[3])));
    mx = row4_max(mx) * sl2;
    if (mx > m + kDecLazy) {
      const float alpha = fast_exp2(m - mx);  // 0 while m is -inf
      m = mx;
      m_use = mx;
#pragma unroll
      for (int nb = 0; nb < 16; ++nb) acc[nb] *= alpha;
      l *= alpha;
      lr *= alpha;
    }
    // P = exp2(s sl2 - m), rounded to E for the product; l from the unrounded p
    float pa[4], pb[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pa[e] = fast_exp2(fmaf(sa[e], sl2, -m_use));
      pb[e] = fast_exp2(fmaf(sb[e], sl2, -m_use));
    }
    l += ((pa[0] + pa[1]) + (pa[2] + pa[3])) + ((pb[0] + pb[1]) + (pb[2] + pb[3]));
    const unsigned p0 = Elem<E>::pack(pa[0], pa[1]), p1 = Elem<E>::pack(pa[2], pa[3]);
    const unsigned p2 = Elem<E>::pack(pb[0], pb[1]), p3 = Elem<E>::pack(pb[2], pb[3]);
    lr = Elem<E>::sum2(p3, Elem<E>::sum2(p2, Elem<E>::sum2(p1, Elem<E>::sum2(p0, lr))));
    const V8 pv = __builtin_bit_cast(V8, u32x4{p0, p1, p2, p3});

    // O^T += V^T P^T (16 d blocks)
    asm volatile("" : "+v"(vf[0]), "+v"(vf[1]), "+v"(vf[2]), "+v"(vf[3]), "+v"(vf[4]), "+v"(vf[5]), "+v"(vf[6]),
                 "+v"(vf[7]), "+v"(vf[8]), "+v"(vf[9]), "+v"(vf[10]), "+v"(vf[11]), "+v"(vf[12]), "+v"(vf[13]),
                 "+v"(vf[14]), "+v"(vf[15]));
#pragma unroll
    for (int nb = 0; nb < 16; ++nb) acc[nb] = Dec16<E>::mfma(vf[nb], pv, acc[nb]);
  }
  // the zero copies of the tiles past the range are still in flight
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // epilogue: lane holds O[row r16][16 nb + 4 g + e] in acc[nb][e]
  const float l_tot = row4_sum(l), lr_tot = row4_sum(lr);
  if (row_ok) {
    const float inv = lr_tot > 0.f ? 1.f / lr_tot : 0.f;
    const float lse = l_tot > 0.f ? (m_use + log2f(l_tot)) * 0.69314718055994530942f : -INFINITY;
    const int64_t grow = grow0 + rr;
    if (p.n_split > 1) {
      float* op = p.o_part + ((int64_t)split * p.part_rows + grow) * kD + 4 * g;
#pragma unroll
      for (int nb = 0; nb < 16; ++nb) *(f32x4*)(op + 16 * nb) = acc[nb] * inv;
      if (g == 0) p.lse_part[(int64_t)split * p.part_rows + grow] = lse;
    } else {
      char* op = (char*)p.o + (grow * kD + 4 * g) * 2;
#pragma unroll
      for (int nb = 0; nb < 16; ++nb)
        *(u32x2*)(op + 32 * nb) = u32x2{Elem<E>::pack(acc[nb][0] * inv, acc[nb][1] * inv),
                                        Elem<E>::pack(acc[nb][2] * inv, acc[nb][3] * inv)};
      if (g == 0) p.lse[grow] = lse;
    }
  }
}

}  // namespace gqa
