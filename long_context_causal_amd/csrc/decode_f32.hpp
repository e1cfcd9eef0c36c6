// decode_f32.hpp -- causal grouped-query attention forward for short query
// blocks (decoding: fewer than 32 positions) over long key sequences, fp32
// inputs and fp32 arithmetic throughout, on the 16x16x4 fp32 MFMA of gfx950.
// This is the serving step of an fp32 model over a long state, which meets
// the same grouped-query fallback (kev PR 202, "Not in this PR"). The
// arithmetic is that of the fp32 long-block kernel (fwd_f32.hpp): scores in
// the base-2 domain, online softmax with the lazy rescale, P kept in fp32 for
// the PV product.
//
// Rows are packed as in the 16-bit decode kernel: the n_rep heads x Lq
// positions of one KV head form blocks (row rr of a block is head rr / Lq of
// the group at position rr % Lq; a block is one contiguous run of rows of Q
// and of O). One workgroup = one block over one key range (a split); its 4
// waves hold 16-row blocks, each over all of d or over a half or a quarter of
// it (NDP below). Per key tile of 16 keys and 16 rows over all of d, S^T =
// K Q^T takes 64 products of 16 keys x 16 rows x 4 d, and O^T += V^T P^T
// 64 more (4 key steps x 16 d blocks). The long-block kernel's 32-row tiles
// over 32 positions of 4 heads would leave most rows empty at these lengths:
// it streams K and V at about 2 TB/s here.
//
// Operand layouts (16x16x4 fp32 product: A lane l = row l % 16, k l / 16; B
// lane l = column l % 16, k l / 16; D lane l = rows 4 (l / 16) + e, column
// l % 16). A lane (r16 = l % 16, g = l / 16) owns query row r16 of its wave.
//   QK: product kk = 4 b + c contracts d = 16 b + 4 g + c over the lanes'
//       k index g, so one 16-byte LDS read of key r16 at d 16 b + 4 g gives
//       the A operands of 4 products, and Q (64 registers) is held as
//       Q[r16][16 b + 4 g .. + 3] for b = 0..15.
//   S^T: the lane holds keys 4 g + e (e = 0..3) of row r16.
//   PV: key step e contracts keys 4 g + e, whose P the lane holds already
//       (its own S^T value). D block nb = 4 a + c has row m at d
//       64 a + 4 m + c, so one 16-byte read of key 4 g + e at d 64 a + 4 m
//       gives the A operands of 4 blocks; the lane's O^T values then sit at
//       d = 64 a + 16 g + 4 e + c (block 4 a + c, element e).
//
// LDS: a ring of 5 stages of one tile each (K then V, 16 keys x 1 KB each:
// 32 KB; all 160 KB) and one workgroup barrier per tile. In step i the V reads
// of tile i go out between the score products and the K reads of tile i + 1
// between the PV products (so neither waits for the LDS), while tiles i + 2 ..
// i + 4 are in flight. Q (up to 64 rows x 1 KB) arrives by the same kind of
// copy into the last two stages, issued before the first three tiles' copies so
// that one wait covers Q and tiles 0 and 1; once every wave holds its Q in
// registers (a second barrier) those two stages take tiles 3 and 4.
#pragma once
#include "common.hpp"

namespace gqa {

constexpr int kDecFWaves = 4;                          // waves per workgroup
constexpr int kDecFRows = 16;                          // query rows per wave
constexpr int kDecFBlockRows = kDecFWaves * kDecFRows;  // 64 packed rows per workgroup
constexpr int kDecFBk = 16;                            // keys per tile
constexpr int kDecFStages = 5;                         // LDS ring depth (tiles)
constexpr int kDecFRow = kD * 4;                       // 1 KB: one key row
constexpr int kDecFPart = kDecFBk * kDecFRow;          // 16 KB: the K (or V) part of a tile
constexpr int kDecFStage = 2 * kDecFPart;              // 32 KB: K then V
constexpr int kDecFCopies = kDecFBk / kDecFWaves;      // 1 KB copies (one key row each) per wave per part
// copies a wave issues per tile; the wait at the top of step i leaves the
// copies of tiles i + 2 and i + 3 in flight
constexpr int kDecFTileCopies = 2 * kDecFCopies;
static_assert(kDecFTileCopies * (kDecFStages - 3) == 16, "the s_waitcnt immediates below assume 16");
// before the loop: Q, then tiles 0..2; the first wait leaves tile 2 in flight
static_assert(kDecFTileCopies == 8, "the first s_waitcnt immediate below assumes 8");
static_assert(kDecFBlockRows * kDecFRow == 2 * kDecFStage, "Q of a row block fills the last two stages");
constexpr float kDecFLazy = 8.0f;  // lazy-rescale threshold (log2 units), as in the long-block kernel

// LDS image: 1 KB key rows of 64 chunks of 16 bytes; chunk c of key r is
// stored at (c & ~15) | ((c & 15) ^ (r % 16)). A 16-byte-per-lane read of 16
// keys at one chunk (the K read) and one of 16 chunks of one key (the V read)
// then each meet all 64 banks once per 16 lanes.
__device__ __forceinline__ uint32_t decf_chunk(int c, int key) {
  return (uint32_t)((c & ~15) | ((c & 15) ^ (key & 15)));
}

struct DecFSmem {
  __attribute__((aligned(16))) char stage[kDecFStages][kDecFStage];
};

typedef __attribute__((address_space(3))) const char decf_lds_cchar;
typedef __attribute__((address_space(3))) const f32x4 decf_lds_f32x4;

// NDP (d parts: 1, 2 or 4): the 4 waves form 4 / NDP row blocks of 16 rows
// times NDP parts of d, and a workgroup holds 64 / NDP packed rows. With
// NDP > 1 the waves of one row block each form their part's partial S^T (64 /
// NDP products per tile), the partials meet through the LDS (each of those
// waves adds them in the same order, so they hold the same S^T and the same
// softmax state), and each wave forms O^T for its part of d (64 / NDP
// products). The launch takes NDP = 4 for groups of at most 16 rows (one
// decode position of a 4-head group), 2 for at most 32, else 1: with NDP = 1
// such groups would leave waves idle while each live wave carried all 128
// products of every tile. The exchange uses the current stage's K part,
// whose K every wave read into registers in the step before.
template <int NDP>
__global__ __launch_bounds__(kDecFWaves * 64) void decode_f32_kernel(FwdParams p) {
  static_assert(NDP == 1 || NDP == 2 || NDP == 4, "1, 2 or 4 parts of d");
  __shared__ DecFSmem sm;
  constexpr int kBlockRows = kDecFBlockRows / NDP;  // packed rows per workgroup
  constexpr int kQCopies = kBlockRows / kDecFWaves;  // 1 KB Q row copies per wave
  constexpr int kQ = 16 / NDP;                       // 16-byte Q (and K, and V) reads per lane per tile
  constexpr int kNA = 4 / NDP;                       // 64-d groups a of O^T per wave
  const int wave = wave_id(), lane = lane_id();
  const int r16 = lane & 15, g = lane >> 4;
  const int dq = wave % NDP;  // this wave's part of d: 16-d blocks kQ dq .. + kQ - 1
  const int rbw = wave / NDP;  // this wave's row block (16 rows) in the workgroup

  // which (batch, KV head), row block and key split this workgroup owns
  const int n_split = p.n_split > 1 ? p.n_split : 1;
  const int split = (int)blockIdx.x % n_split;
  const int rest = (int)blockIdx.x / n_split;
  const int rb = rest % p.n_qb;
  const int bh = rest / p.n_qb;
  const int b = bh / p.Hkv, kvh = bh % p.Hkv;
  // packed rows of the group (n_rep <= 64 heads x Lq < 32 positions: 32-bit)
  const int R = p.n_rep * (int)p.Lq;
  const int row0 = rb * kBlockRows;
  const int64_t grow0 = ((int64_t)b * p.Hq + (int64_t)kvh * p.n_rep) * p.Lq;  // global row of packed row 0

  // this lane's row (row r16 of the wave's row block) and its last visible
  // key; a row past the group's end (its Q reads as zeros) writes nothing
  const int rw = rbw * kDecFRows + r16;  // row within the workgroup's block
  const int rr = row0 + rw;
  const bool row_ok = rr < R;
  const int64_t pos = row_ok ? (int64_t)(rr % (int)p.Lq) : 0;
  const int64_t kv_end = p.causal ? min(p.Lk, p.q_offset + p.Lq) : p.Lk;
  const int lim = (int)(p.causal ? min(p.q_offset + pos, p.Lk - 1) : p.Lk - 1);
  // tiles from this key on hold a key hidden from some row (causal or past Lk)
  const int mask_from = (int)(p.causal ? min(p.q_offset, p.Lk - 1) : p.Lk - 1);
  const int n_tiles = (int)((kv_end + kDecFBk - 1) / kDecFBk);
  const int t_lo = p.n_split > 1 ? split * p.split_tiles : 0;
  const int t_hi = p.n_split > 1 ? min(n_tiles, t_lo + p.split_tiles) : n_tiles;
  const int n = max(0, t_hi - t_lo);

  const int64_t kv_head = (int64_t)b * p.Hkv + kvh;
  const char* kbase = (const char*)p.k + kv_head * p.Lk * kDecFRow;
  const char* vbase = (const char*)p.v + kv_head * p.Lk * kDecFRow;

  // per-lane copy offsets: copy it of this wave, in either part, is key row
  // kDecFCopies wave + it (of Q: row kQCopies wave + it); lane l writes its
  // LDS chunk l, fetched from the global chunk stored there
  uint32_t ldo[kDecFCopies], ldq[kQCopies];
#pragma unroll
  for (int it = 0; it < kDecFCopies; ++it) {
    const int key = kDecFCopies * wave + it;
    ldo[it] = (uint32_t)key * kDecFRow + (decf_chunk(lane, key) << 4);
  }
#pragma unroll
  for (int it = 0; it < kQCopies; ++it) {
    const int row = kQCopies * wave + it;
    ldq[it] = (uint32_t)row * kDecFRow + (decf_chunk(lane, row) << 4);
  }
  const uint32_t lds_stage0 = lds_addr(sm.stage[0]);
  const uint32_t lds_q = lds_addr(sm.stage[kDecFStages - 2]);

  // Copies of tile t (absolute) into stage st; a tile past this split's range
  // (or Lk) copies from a resource of size 0, which writes zeros, so every
  // step issues the same number of copies and the wait count stays fixed.
  auto copy_tile = [&](int st, int t) {
    const bool valid = t < t_hi;
    const uint32_t keys = valid ? min((uint32_t)p.Lk - (uint32_t)t * kDecFBk, (uint32_t)kDecFBk) : 0u;
    const uint64_t off = valid ? (uint64_t)(uint32_t)t * kDecFPart : 0u;
    const rsrc_t rk = make_rsrc(kbase + off, keys * kDecFRow);
    const rsrc_t rv = make_rsrc(vbase + off, keys * kDecFRow);
    const uint32_t dst = lds_stage0 + (uint32_t)st * kDecFStage + (uint32_t)(kDecFCopies * wave) * kDecFRow;
#pragma unroll
    for (int it = 0; it < kDecFCopies; ++it) {
      buf2lds16_imm(rk, ldo[it], dst, (uint32_t)it * kDecFRow);
      buf2lds16_imm(rv, ldo[it], dst + kDecFPart, (uint32_t)it * kDecFRow);
    }
  };
  // Q of the block (rows past the group's end read as zeros) into the last
  // two stages (the first 64 / NDP KB of them), then tiles 0..2 into stages
  // 0..2
  {
    const int rows = min(kBlockRows, R - row0);
    const rsrc_t rq = make_rsrc((const float*)p.q + (grow0 + row0) * kD, (uint32_t)rows * kDecFRow);
    const uint32_t dst = lds_q + (uint32_t)(kQCopies * wave) * kDecFRow;
#pragma unroll
    for (int it = 0; it < kQCopies; ++it) buf2lds16_imm(rq, ldq[it], dst, (uint32_t)it * kDecFRow);
  }
#pragma unroll
  for (int j = 0; j < kDecFStages - 2; ++j) copy_tile(j, t_lo + j);

  // LDS read addresses (stage 0; a stage adds st * 32 KB). K: key r16, 16-d
  // block bb (= kQ dq + j), chunk 4 bb + g at 256 (bb / 4) + 16 ((4 (bb % 4) +
  // g) ^ r16). V, key step e, 64-d group a (= kNA dq + j % kNA): key 4 g + e,
  // chunk 16 a + r16 at 256 a + 16 (r16 ^ (4 g + e)).
  decf_lds_cchar* const st0 = (decf_lds_cchar*)sm.stage[0];
  decf_lds_cchar* kr[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) kr[j] = st0 + r16 * kDecFRow + (((4 * j + g) ^ r16) << 4);
  decf_lds_cchar* vr[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int key = 4 * g + e;
    vr[e] = st0 + kDecFPart + key * kDecFRow + ((r16 ^ key) << 4) + ((kNA * dq) << 8);
  }
  // byte offset of 16-d block bb = kQ dq + j in a 1 KB row, without the XOR part
  auto kblk = [&](int j) { return ((kQ * dq + j) >> 2) << 8; };

  asm volatile("s_waitcnt vmcnt(8)" ::: "memory");  // this wave's Q, tile-0 and tile-1 copies have landed
  __syncthreads();                                   // ... and every wave's

  // a wave whose 16 rows all lie past the group's end takes part in the
  // copies and barriers only
  const bool live = row0 + rbw * kDecFRows < R;
  // Q as the B operand: qf[j] = Q[row rw][16 bb + 4 g .. + 3] (bb = kQ dq + j),
  // held in AGPRs (read there by the score products); K of tile 0 into kf
  f32x4 qf[kQ], kf[kQ];
  {
    decf_lds_cchar* qb = (decf_lds_cchar*)sm.stage[kDecFStages - 2] + rw * kDecFRow;
#pragma unroll
    for (int j = 0; j < kQ; ++j) {
      qf[j] = *(decf_lds_f32x4*)(qb + kblk(j) + (((4 * (j & 3) + g) ^ r16) << 4));
      kf[j] = *(decf_lds_f32x4*)(kr[j & 3] + kblk(j));
    }
    // every wave's Q is in registers before the first copy into those stages
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kQ; ++j) asm volatile("" : "+a"(qf[j]));
  }

  const float sl2 = p.scale_log2;
  float m = -INFINITY, m_use = 0.f, l = 0.f;
  f32x4 acc[4 * kNA];
#pragma unroll
  for (int nb = 0; nb < 4 * kNA; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Step i: K of tile i is in kf (read during step i - 1); the V reads of tile
  // i go out between the score products, the K reads of tile i + 1 between
  // the PV products. Tiles i and i + 1 have landed at the top of the step;
  // i + 2 .. i + 4 are in flight.
  for (int i = 0, st = 0; i < n; ++i, st = st == kDecFStages - 1 ? 0 : st + 1) {
    if (i > 0) {
      asm volatile("s_waitcnt vmcnt(16)" ::: "memory");  // tile i + 1's copies have landed
      __syncthreads();  // ... for every wave; the stage of tile i - 1 is free
    }
    if (i == 0) copy_tile(kDecFStages - 2, t_lo + kDecFStages - 2);  // tile 3 into the other Q stage
    copy_tile(st == 0 ? kDecFStages - 1 : st - 1, t_lo + i + kDecFStages - 1);
    const int t = t_lo + i;
    const int so = st * kDecFStage;
    const int so1 = (st == kDecFStages - 1 ? 0 : st + 1) * kDecFStage;
    // (every wave, live or not, reaches the exchange barrier below)
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    f32x4 vf[kQ];
    if (live) {
      // S^T = K Q^T over this wave's part of d: s[e] is key 4 g + e of row
      // r16, summed as four chains (one per d offset c) added at the end; V
      // read j (key step j / kNA, 64-d group kNA dq + j % kNA) goes out before
      // score block j
      f32x4 s4[4] = {};
#pragma unroll
      for (int j = 0; j < kQ; ++j) {
        vf[j] = *(decf_lds_f32x4*)(vr[j / kNA] + so + ((j % kNA) << 8));
#pragma unroll
        for (int c = 0; c < 4; ++c)
          s4[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[j][c], qf[j][c], s4[c], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      s = (s4[0] + s4[1]) + (s4[2] + s4[3]);
    }
    if (NDP > 1) {
      // the parts' partial sums meet in the K part of this tile's stage (every
      // wave read that K in the step before); the waves of a row block add
      // them in part order
      float* const xw = (float*)sm.stage[st];
      *(f32x4*)(xw + (wave * 64 + lane) * 4) = s;
      __syncthreads();
      f32x4 part[NDP];
#pragma unroll
      for (int w = 0; w < NDP; ++w)
        part[w] = w == dq ? s : *(const f32x4*)(xw + ((rbw * NDP + w) * 64 + lane) * 4);
      s = part[0];
#pragma unroll
      for (int w = 1; w < NDP; ++w) s += part[w];
    }
    if (!live) continue;
    if (t * kDecFBk + kDecFBk - 1 > mask_from) {
      const int k0 = t * kDecFBk + 4 * g;
#pragma unroll
      for (int e = 0; e < 4; ++e) s[e] = k0 + e <= lim ? s[e] : -INFINITY;
    }
    // row max over the 4 lanes of the row, then the lazy update (the running
    // max moves only when a row's max grows by more than 8 in log2 units)
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = row4_max(mx) * sl2;
    if (mx > m + kDecFLazy) {
      const float alpha = fast_exp2(m - mx);  // 0 while m is -inf
      m = mx;
      m_use = mx;
#pragma unroll
      for (int nb = 0; nb < 4 * kNA; ++nb) acc[nb] *= alpha;
      l *= alpha;
    }
    float pe[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) pe[e] = fast_exp2(fmaf(s[e], sl2, -m_use));
    l += (pe[0] + pe[1]) + (pe[2] + pe[3]);
    __builtin_amdgcn_sched_barrier(0);

    // O^T += V^T P^T: key step e = j / kNA, d block 4 (kNA dq + j % kNA) + c
    // (acc[4 (j % kNA) + c]); K read j of tile i + 1 goes out before PV group j
#pragma unroll
    for (int j = 0; j < kQ; ++j) {
      kf[j] = *(decf_lds_f32x4*)(kr[j & 3] + so1 + kblk(j));
      const int e = j / kNA, al = j % kNA;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc[4 * al + c] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf[j][c], pe[e], acc[4 * al + c], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // the zero copies of the tiles past the range are still in flight
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // epilogue: lane holds O[row][64 a + 16 g + 4 e + c] (a = kNA dq + al) in
  // acc[4 al + c][e]
  const float l_tot = row4_sum(l);
  if (row_ok && live) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float lse = l_tot > 0.f ? (m_use + log2f(l_tot)) * 0.69314718055994530942f : -INFINITY;
    const int64_t grow = grow0 + rr;
    float* op = p.n_split > 1 ? p.o_part + ((int64_t)split * p.part_rows + grow) * kD : (float*)p.o + grow * kD;
#pragma unroll
    for (int al = 0; al < kNA; ++al)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        *(f32x4*)(op + 64 * (kNA * dq + al) + 16 * g + 4 * e) =
            f32x4{acc[4 * al][e] * inv, acc[4 * al + 1][e] * inv, acc[4 * al + 2][e] * inv, acc[4 * al + 3][e] * inv};
    if (g == 0 && dq == 0) {
      if (p.n_split > 1)
        p.lse_part[(int64_t)split * p.part_rows + grow] = lse;
      else
        p.lse[grow] = lse;
    }
  }
}

}  // namespace gqa
