/*
 * gqa_attn.h -- C ABI of the MI355X (gfx950) exact causal grouped-query
 * attention forward with memory linear in sequence length.
 *
 * The operation. For every batch b, query head h and query row i:
 *     s_j   = (q[b,h,i,:] . k[b,g,j,:]) / sqrt(D)     for every visible key j
 *     o     = sum_j softmax(s)_j v[b,g,j,:]
 *     lse   = ln sum_j exp(s_j)
 * with g = h / (Hq/Hkv): contiguous groups of query heads share one key/value
 * head, the sharing of 16 query heads over 4 key/value heads (system1-omni
 * issue 27, "The closest planned or implemented model"; kev pull request 202,
 * "Why fp32 fell to the L x L kernel", where the L x L math path computes the
 * same attention by materialising the score matrix, and "The change", where
 * repeating K/V per query head gives the same result with memory linear in L).
 * Key j is visible to query row i iff
 *     (!causal || j <= q_offset + i)  &&  (seg_q == NULL || seg_q[b,i] == seg_k[b,j]).
 * q_offset places the queries at positions q_offset.. of the key sequence: a
 * branch whose positions restart at the state length S uses q_offset = S
 * (system1-omni issue 27, "Three differences from Cua-S1 that matter", item 3).
 * Segment ids are separate for queries and keys, NULL meaning one segment
 * (maxtext pull request 4929: with constant ids the segmented and the
 * non-segmented kernels give the same result). A row with no visible key gets
 * o = 0 and lse = -inf.
 *
 * Layouts (all contiguous, row-major, element offsets fit int64):
 *   q, o  [B, Hq,  Lq, D]   in `dtype`
 *   k, v  [B, Hkv, Lk, D]   in `dtype`
 *   lse   [B, Hq,  Lq]      fp32, natural log
 *   seg_q [B, Lq], seg_k [B, Lk]  int32 (any values; sorted ids skip more work)
 * All pointers are device pointers on the current HIP device. Accumulation is
 * fp32; bf16 and fp16 outputs are rounded to nearest even, and so are the
 * softmax weights that enter the P V product in those types. fp32 inputs use
 * full-fp32 matrix instructions (no reduced-precision products). fp16 is the
 * other half-width input type that the same fast path serves (kev pull request
 * 202, "The change": bf16 and fp16 calls keep the fused kernels).
 *
 * Ownership and threading. The caller allocates every buffer. The library
 * allocates no device memory (its code object holds one static array of
 * GQA_NOALLOC_SCRATCH_BYTES per GPU, used only by gqa_attn_fwd_split_noalloc,
 * placed by the HIP runtime when the code object loads), keeps no pointer
 * after returning and never synchronises: work is enqueued on `stream` (a hipStream_t; NULL is the
 * default stream) and outputs are valid once the stream reaches that point.
 * Every element of o and lse is written. o must not overlap q, k or v.
 * Calls are reentrant and deterministic (same inputs give the same bits).
 *
 * Errors. Arguments are checked before any HIP call; on an error nothing is
 * enqueued and outputs are untouched. A launch failure returns
 * GQA_ERR_LAUNCH. gqa_attn_strerror names every code.
 */
#ifndef GQA_ATTN_H
#define GQA_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum gqa_dtype { GQA_F32 = 0, GQA_BF16 = 1, GQA_F16 = 2 };

enum gqa_status {
  GQA_OK = 0,
  GQA_ERR_NULL = 1,        /* q, k, v, o or lse is NULL */
  GQA_ERR_SHAPE = 2,       /* an extent <= 0, Hq % Hkv != 0, q_offset < 0, exactly one segment pointer NULL,
                              or an id index without segment ids */
  GQA_ERR_UNSUPPORTED = 3, /* D != 256, dtype not F32/BF16/F16, Hq/Hkv above 64, or Lq/Lk >= 2^31
                              (backward: Lq/Lk > 2^21) */
  GQA_ERR_ALIGN = 4,       /* q, k, v, o not 16-byte aligned, lse/seg not 4-byte aligned, or an id index
                              not 8-byte aligned */
  GQA_ERR_LAUNCH = 5,      /* the HIP runtime reported an error at launch */
  GQA_ERR_ALIAS = 6,       /* o overlaps q, k or v (or, for merge, partially overlaps an input) */
  GQA_ERR_WORKSPACE = 7    /* split-KV workspace smaller than gqa_attn_split_workspace() requires,
                              or an id index buffer smaller than gqa_attn_seg_index_bytes() */
};

/*
 * Attention forward (the operation above). Shapes as above; D must be 256.
 * `stream` is a hipStream_t passed as void*. Returns a gqa_status. Calls with
 * fewer than 32 query positions and no segment ids (decoding) run on kernels
 * of their own that pack a key/value head's query heads x positions into
 * 16-row products; their results equal the other kernels' up to the order of
 * the fp32 sums.
 */
int gqa_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                 int64_t q_offset, const int32_t* seg_q, const int32_t* seg_k,
                 int causal, int dtype, void* stream);

/*
 * Log-sum-exp merge of two attention results over disjoint key sets of the
 * same query rows into the result over their union:
 *     M = max(lse1, lse2),  w_x = exp(lse_x - M),
 *     o = (w1 o1 + w2 o2) / (w1 + w2),  lse = M + ln(w1 + w2);
 * both lse = -inf gives o = 0, lse = -inf. This joins the prefix part and the
 * causal suffix part of a shared-prefix branch (system1-omni issue 27, "Three
 * differences from Cua-S1 that matter", item 3: one state, then a branch per
 * question). o1, o2, o: [rows, D] in `dtype`; lse1, lse2, lse: [rows] fp32.
 * o may be exactly o1 or o2 and lse exactly lse1 or lse2 (in place); partial
 * overlaps are rejected. D must be a positive multiple of 8.
 */
int gqa_attn_merge(const void* o1, const float* lse1, const void* o2, const float* lse2,
                   void* o, float* lse, int64_t rows, int64_t D, int dtype, void* stream);

/*
 * Attention backward: the gradients of a scalar loss with respect to q, k and
 * v, given its gradient `dout` with respect to o. The pages train at these
 * lengths (kev pull request 202, the title of the change: states of 64k tokens
 * are trained and served; system1-omni issue 27, "The closest planned or
 * implemented model": the model trains end to end), so this is the chain rule
 * through the forward above. With p_ij = exp(s_ij - lse_i) over the visible
 * keys:
 *     delta_i = sum_d dout[i,d] o[i,d]          (= sum_j p_ij dp_ij)
 *     dp_ij   = dout_i . v_j,   ds_ij = p_ij (dp_ij - delta_i)
 *     dq_i    = (1/sqrt(D)) sum_j ds_ij k_j
 *     dk_j    = (1/sqrt(D)) sum_{h,i} ds_ij q_i,   dv_j = sum_{h,i} p_ij dout_i
 * where the dk/dv sums run over every query head h of the key/value head's
 * group (grouped-query attention reduces the gradient over the heads that share
 * a key/value head) and over the rows i that see key j.
 *
 * Inputs: q, k, v as for the forward; o and lse are the forward's outputs for
 * the same arguments (or, for a key set split into parts, the merged o and lse
 * of the whole: each part's call then yields that part's dk, dv and its share
 * of dq, and the dq of the parts add up); dout [B,Hq,Lq,D] in `dtype`.
 * Outputs: dq [B,Hq,Lq,D], dk and dv [B,Hkv,Lk,D] in `dtype`, and
 * delta [B,Hq,Lq] fp32 (written, then read by the second kernel; a caller
 * buffer so that the library allocates nothing). Every element of the outputs
 * is written (rows with no visible key get dq = 0; keys no row sees get
 * dk = dv = 0). Outputs must not overlap any input or each other.
 * Same shape rules as the forward, plus Lq, Lk <= 2^21. Accumulation is fp32;
 * for bf16 and fp16 inputs the gradients are rounded to nearest even, and so
 * are P and dS where they enter a product in that type.
 * Deterministic: no atomics; dq comes from one kernel over query blocks, dk and
 * dv from one over key blocks. Returns a gqa_status; GQA_ERR_NULL when any
 * pointer but the segment ids is NULL.
 */
int gqa_attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv, float* delta,
                 int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                 int64_t q_offset, const int32_t* seg_q, const int32_t* seg_k,
                 int causal, int dtype, void* stream);

/*
 * Id-range index of a segment-id array, for callers that run many calls over
 * the same ids (every layer's forward and backward of one packed batch). With
 * ids, each workgroup of gqa_attn_fwd and gqa_attn_bwd finds the key (or row)
 * tiles it must visit by reading every id up to its causal end. The index
 * holds, for each block of 16 consecutive ids of a batch row, their minimum
 * and maximum (int32 pairs, row-major [B][ceil(L / 16)][2]); the *_indexed
 * calls classify the tiles from it, from one eighth of the bytes, and give
 * results identical bit for bit to the calls without it. The same role as the
 * per-block mask metadata that splash attention builds ahead of its kernel
 * (maxtext pull request 4929, the problem statement: fwd_mask_info.data_next,
 * block_mask, mask_next, the kernel's prefetched operands), but linear in L.
 *
 * gqa_attn_seg_index_bytes: the index size in bytes for B rows of L ids
 * (0 for a non-positive extent).
 * gqa_attn_seg_index: writes the index of seg [B, L] (device, int32) into
 * `index` (device, 8-byte aligned, at least gqa_attn_seg_index_bytes(B, L)
 * bytes, not overlapping seg); enqueued on `stream`. Errors: GQA_ERR_NULL,
 * GQA_ERR_SHAPE (B or L <= 0), GQA_ERR_UNSUPPORTED (L >= 2^31 or B >= 2^24),
 * GQA_ERR_ALIGN, GQA_ERR_WORKSPACE (index too small), GQA_ERR_ALIAS; nothing is
 * enqueued on an error.
 */
int64_t gqa_attn_seg_index_bytes(int64_t B, int64_t L);
int gqa_attn_seg_index(const int32_t* seg, int64_t B, int64_t L, void* index, int64_t index_bytes, void* stream);

/*
 * gqa_attn_fwd and gqa_attn_bwd with the indexes of seg_q (over Lq) and seg_k
 * (over Lk) from gqa_attn_seg_index, written on this stream or complete before
 * the call. Either index may be NULL (its ids are then scanned as in the plain
 * call); both must be NULL without segment ids (else GQA_ERR_SHAPE). The
 * forward reads the key index; the backward's dQ kernel the key index, its
 * dK/dV kernel the row index. An index that does not match its ids gives
 * unspecified results (the ids themselves still mask every element the tile
 * classification lets through). Indexes must be 8-byte aligned (else
 * GQA_ERR_ALIGN) and must not overlap an output (else GQA_ERR_ALIAS). Other
 * arguments, outputs and errors as the plain calls.
 */
int gqa_attn_fwd_indexed(const void* q, const void* k, const void* v, void* o, float* lse,
                         int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                         int64_t q_offset, const int32_t* seg_q, const int32_t* seg_k,
                         const void* seg_q_index, const void* seg_k_index,
                         int causal, int dtype, void* stream);
int gqa_attn_bwd_indexed(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv, float* delta,
                         int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                         int64_t q_offset, const int32_t* seg_q, const int32_t* seg_k,
                         const void* seg_q_index, const void* seg_k_index,
                         int causal, int dtype, void* stream);

/*
 * Split-KV forward: the same operation and outputs as gqa_attn_fwd (equal up
 * to the order of the fp32 sums), for short query blocks over long key
 * sequences (decoding after a long state; one question's branch over the
 * shared prefix, system1-omni issue 27, "Three differences from Cua-S1 that
 * matter", item 3), where gqa_attn_fwd would launch too few workgroups to fill
 * the GPU. The key range is cut into n_split consecutive ranges of whole key
 * tiles. Calls with fewer than 32 query positions and no segment ids
 * (decoding) run on kernels of their own that pack the group's heads x
 * positions into 16-row products: 16-key tiles for fp32 inputs, 32 keys for
 * 16-bit inputs. Other calls: 32 keys for fp32 inputs, 64 keys for 16-bit
 * inputs. One launch computes every (query block, head group, range) and
 * writes a normalised partial o (fp32) and its lse into `workspace`, and a
 * second kernel combines the parts with the log-sum-exp merge of
 * gqa_attn_merge, over n_split parts, then rounds o once to `dtype`.
 * n_split in [1, 1024]; fewer ranges than n_split are used when Lk has fewer
 * key tiles; n_split = 1 is gqa_attn_fwd (workspace unused, may be NULL).
 * workspace: device memory of at least gqa_attn_split_workspace(B, Hq, Lq, D,
 * n_split) bytes, 16-byte aligned, not overlapping any argument; its contents
 * on entry do not matter and on return are unspecified. Errors as for
 * gqa_attn_fwd, plus GQA_ERR_NULL (no workspace) and GQA_ERR_WORKSPACE (too
 * small); nothing is enqueued on an error.
 */
int gqa_attn_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                       int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                       int64_t q_offset, const int32_t* seg_q, const int32_t* seg_k,
                       int causal, int dtype, int n_split, void* workspace, int64_t workspace_bytes,
                       void* stream);

/*
 * Split-KV forward that allocates nothing and takes no workspace: for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc). Same operation, arguments
 * and result as gqa_attn_fwd_split with the same n_split (the same kernels on
 * the same split), but the partial results go to a static device array of
 * GQA_NOALLOC_SCRATCH_BYTES that the library's code object holds on each GPU
 * it runs on, placed by the HIP runtime when the code object loads there and
 * kept until the process ends. The call itself makes no allocation.
 * n_split: 0 picks gqa_attn_split_count()'s count, lowered to what the array
 * holds; 1 .. 1024 as in gqa_attn_fwd_split, and GQA_ERR_WORKSPACE when
 * n_split * B * Hq * Lq * (D + 1) * 4 bytes of partials exceed the array
 * (checked before any HIP call; nothing is enqueued). Every call on one GPU
 * uses that GPU's single array: calls whose work overlaps in time on one GPU
 * (other streams, other host threads) race and must be ordered by the caller.
 * GQA_ERR_LAUNCH also when the runtime cannot report the array's address.
 */
#define GQA_NOALLOC_SCRATCH_BYTES (64ll << 20)
int gqa_attn_fwd_split_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                               int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                               int64_t q_offset, const int32_t* seg_q, const int32_t* seg_k,
                               int causal, int dtype, int n_split, void* stream);

/* Bytes of workspace gqa_attn_fwd_split needs for n_split ranges:
 * n_split * B * Hq * Lq * (D + 1) * 4. Returns 0 for invalid arguments. */
int64_t gqa_attn_split_workspace(int64_t B, int64_t Hq, int64_t Lq, int64_t D, int n_split);

/* A split count for gqa_attn_fwd_split that fills the GPU (about one
 * workgroup per compute unit, each range at least 4 key tiles), from the
 * shape alone; 1 when gqa_attn_fwd already launches enough workgroups. */
int gqa_attn_split_count(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int dtype);

/* Static description of a status code (never NULL). */
const char* gqa_attn_strerror(int code);

/* ABI version: (major << 16) | minor. */
int gqa_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GQA_ATTN_H */
