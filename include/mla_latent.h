/*
 * mla_latent.h -- C ABI of the matrix-absorbed MLA decode path on MI355X (gfx950).
 *
 * The four compute entry points follow the order of the absorbed decode:
 *
 *   mla_absorb_q       q~ = W_UK^T q_nope              ("MLA in full detail", Step 2:
 *                                                       fold W_UK into the query)
 *   mla_decode_latent  attention of all query heads against one shared paged
 *                      latent cache of [c (512) || k_pe (64)] rows; score
 *                      (q~ . c + q_pe . k_pe) * scale, softmax over the key
 *                      axis, output the softmax-weighted sum of the 512-wide
 *                      latents, optionally as split-KV partial states
 *                                                      (same page, Step 3: attend
 *                                                       against the latent directly;
 *                                                       M5.8 0x05 paged address
 *                                                       translation; M5.8 0x08 lse output)
 *   mla_merge_splits   exact log-sum-exp merge of the split partials
 *                                                      (M5.8 0x0C sequence-split merge;
 *                                                       mlxcel Stage 2 merge contract)
 *   mla_unabsorb_out   out = W_UV latent                ("MLA in full detail", Step 4:
 *                                                       fold W_UV into the output)
 *
 * mla_merge_unabsorb takes the last two in one kernel (split partials in, out
 * and lse out; the merged latent never goes to memory).
 *
 * and, for multi-step decoding, mla_append_cache (the new tokens' cache rows
 * written at their paged positions before the decode that reads them); for
 * sparse (top-k) attention, mla_decode_sparse (bf16 rows) and
 * mla_decode_sparse_fp8 (FP8 rows) in place of mla_decode_latent.
 * The same function in the Normal (per-head up-projected) association order,
 * for comparison, is a separate library: mla_normal.h / libmla_normal.so.
 *
 * "M5.8" is the page "M5.8 - Multi-Head Latent Attention: Latent KV State,
 * Weight Absorption, and FlashMLA"; "mlxcel" is its "MLA absorbed decode" page.
 *
 * Conventions for every entry point:
 *  - Tensor arguments are DEVICE pointers to caller-owned, row-major, contiguous
 *    memory.  bf16 tensors are passed as uint16_t storage of bfloat16 values.
 *    Tensor pointers must be 16-byte aligned; int32 index arrays and fp32 lse
 *    arrays 4-byte aligned.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Calls
 *    validate host-side scalars and pointers, enqueue their kernels on `stream`
 *    and return; they never synchronise, never allocate device memory and keep
 *    no state between calls -- except mla_validate_inputs (synchronous, for
 *    debugging) and mla_decode_latent_noalloc (a device array of its own per
 *    GPU, whose address it keeps per device).
 *    Calls on different streams that share no output or workspace buffer may
 *    run concurrently.
 *  - The return value is MLA_OK or a negative mla_status.  On a negative return
 *    nothing has been enqueued, except MLA_ERR_LAUNCH, which reports a failed
 *    kernel launch (hipGetLastError) after validation passed.
 *  - Device-resident index data (block tables, sequence lengths) is trusted by
 *    the compute entry points: an out-of-range entry is undefined behaviour.
 *    mla_validate_inputs checks it (synchronously) for callers that need that.
 *
 * Fixed geometry of this library: kv_lora_rank r = 512, rope width d_R = 64,
 * d_nope = d_V = 128.  H (query heads) is 1..128, T (query tokens per
 * sequence: 1 for plain decode, a few for multi-token decode, up to a
 * prefill-sized block when comparing with the Normal path) is 1..1024,
 * page_size is a multiple of 16 in [16, 1024].
 */
#ifndef MLA_LATENT_H
#define MLA_LATENT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL = -1,          /* a required pointer is NULL */
  MLA_ERR_ALIGN = -2,         /* a pointer is not 16-byte aligned */
  MLA_ERR_SHAPE = -3,         /* a size is out of range or sizes disagree */
  MLA_ERR_UNSUPPORTED = -4,   /* geometry outside what this library implements */
  MLA_ERR_WORKSPACE = -5,     /* workspace or partial buffers too small / missing */
  MLA_ERR_LAUNCH = -6,        /* a kernel launch failed */
  MLA_ERR_INVALID_INDEX = -7, /* (mla_validate_inputs) bad block-table entry or length */
  MLA_ERR_DEVICE = -8         /* HIP runtime error while querying the device */
} mla_status;

typedef enum { MLA_BF16 = 0, MLA_F32 = 1 } mla_dtype;

/* Absorb: q_lat[b,t,h,c] = sum_{n<d_nope} q_nope[b,t,h,n] * W_UK[h,n,c], accumulated
 * in fp32 and rounded to bf16 (nearest-even).
 *   q_nope  [B,T,H,d_nope] bf16        w_uk [H,d_nope,r] bf16
 *   q_lat   [B,T,H,r]      bf16 (out)
 * Source: "MLA in full detail", Step 2 (the bmm [N,B,P] x [N,P,L] -> [N,B,L]);
 * M5.8 0x04 "Batched absorption trace" (einsum bhqn,hnc->bhqc; W_UK [H,d_N,d_c]). */
int mla_absorb_q(const uint16_t* q_nope, const uint16_t* w_uk, uint16_t* q_lat, int B, int T,
                 int H, int d_nope, int r, void* stream);

/* Sizes the caller must provide for mla_decode_latent with `num_splits`:
 *   *workspace_bytes  -- bytes of the `workspace` argument (0 unless num_splits == 0);
 *   *max_total_splits -- rows of part_out / part_lse (0 when num_splits == 1).
 * num_splits: 1 = no split; S > 1 = every sequence cut into S chunks (see
 * mla_decode_latent); 0 = automatic, chosen on the device from the sequence
 * lengths: with U = compute units / ceil(T*H/128) work units available at once,
 * the chunk c is the smallest multiple of page_size, at least 256 tokens, with
 *     sum_b clamp(ceil(L_b / c), 1, 128) <= U
 * (every sequence one chunk when B >= U); sequence b is cut into
 * S_b = clamp(ceil(L_b / c), 1, 128) chunks of ceil(ceil(L_b/S_b)/page_size)
 * * page_size tokens (split_indptr[b+1] - split_indptr[b] = S_b).
 * Queries the current HIP device (compute-unit count) when num_splits == 0. */
int mla_decode_workspace_size(int B, int T, int H, int r, int max_seqlen, int page_size,
                              int num_splits, size_t* workspace_bytes, int* max_total_splits);

/* Absorbed latent attention over a paged cache.
 *   q_lat       [B,T,H,r]    bf16   absorbed query (mla_absorb_q)
 *   q_pe        [B,T,H,d_R]  bf16   rope part of the query, already rotated
 *   kv_cache    [num_blocks,page_size,r+d_R] bf16; row = [c (r) || k_pe (d_R)], one
 *               latent KV head shared by all query heads (1152-byte rows)
 *   block_table [B,max_blocks_per_seq] int32: physical block of each logical page;
 *               logical token j of sequence b is row block_table[b, j/page_size] *
 *               page_size + j%page_size (M5.8 0x05).  Entries at or past
 *               ceil(seqlens[b]/page_size) are never read.
 *   seqlens     [B] int32: visible rows per sequence, INCLUDING the T current
 *               rows; T <= seqlens[b] <= max_seqlen.  Query t of sequence b sees
 *               keys j <= seqlens[b] - T + t (causal over the current rows;
 *               M5.8 0x05: a query at position p sees p + 1 rows).
 *   softmax_scale  the caller passes 1/sqrt(d_nope + d_R) = 1/sqrt(192)
 *               ("MLA in full detail", numpy parity script: the scale of the
 *               original 192-wide key is kept).
 *   num_splits  1: single pass, writes out_latent and lse.
 *               S > 1: sequence b is cut into S contiguous chunks of
 *               ceil(ceil(seqlens[b]/S)/page_size)*page_size tokens (trailing
 *               chunks may be empty); chunk s writes its partial state to row
 *               split_indptr[b] + s of part_out / part_lse.
 *               0: automatic split counts (see mla_decode_workspace_size).
 *               When out_latent is given and B*ceil(T*H/128) work units already
 *               reach the CU count, the automatic rule gives every sequence
 *               one chunk and the call runs unsplit: out_latent and lse are
 *               written directly, the partial buffers and split_indptr are not
 *               touched.
 *   workspace   device scratch of the size reported by mla_decode_workspace_size
 *               (the automatic mode's work list); may be NULL when that size is 0.
 *               Contents on entry are ignored.
 *   part_out    [max_total_splits,T,H,r] f32 or bf16 (part_dtype): partial outputs,
 *               each divided by its own softmax denominator (mlxcel Stage 2
 *               contract).  bf16 halves the partial traffic; the values are
 *               convex combinations of cache rows, so their rounding error is
 *               relative (2^-9) and the merge weights are exact fp32.
 *   part_lse    [max_total_splits,T,H] f32: natural-log LSE of each partial;
 *               -inf for an empty chunk (whose part_out row is zero)
 *   split_indptr [B+1] int32 (out): first partial row of each sequence
 *   out_latent  [B,T,H,r] bf16 or f32 (out_dtype).  With num_splits == 1 it
 *               receives the result.  With num_splits != 1 it may be NULL (the
 *               caller runs mla_merge_splits later); when non-NULL the
 *               partials are merged on the device before the call returns
 *               (stream order) and out_latent / lse receive the merged result.
 *   lse         [B,T,H] f32 natural-log LSE of each query row; nullable.
 * Returns MLA_ERR_WORKSPACE when num_splits != 1 and part_out, part_lse or
 * split_indptr is missing, or the workspace is missing or smaller than
 * mla_decode_workspace_size reports. */
int mla_decode_latent(const uint16_t* q_lat, const uint16_t* q_pe, const uint16_t* kv_cache,
                      int num_blocks, int page_size, const int32_t* block_table,
                      int max_blocks_per_seq, const int32_t* seqlens, int B, int T, int H, int r,
                      int d_R, int max_seqlen, float softmax_scale, int num_splits,
                      void* workspace, size_t workspace_bytes, void* part_out,
                      mla_dtype part_dtype, float* part_lse, int32_t* split_indptr,
                      void* out_latent, mla_dtype out_dtype, float* lse, void* stream);

/* mla_decode_latent over a cache of FP8 rows (M5.8 0x0B, "Exact 656-byte FP8
 * row"): every argument and result as there, except
 *   kv_cache    [num_blocks,page_size,656] bytes, 16-byte aligned; row =
 *               bytes [0,512) the E4M3 codes (OCP encoding, the one called
 *               E4M3FN) of latent columns 0..511, bytes [512,528) four
 *               little-endian fp32 scales, scale g covering columns
 *               [128g, 128g+128), bytes [528,656) the 64 bf16 rope values.
 * The latent is dequantized to bf16 in the kernel, c = bf16(code * scale)
 * (the product formed in fp32, then rounded to nearest even), and the
 * attention runs in bf16 as for bf16 rows.  The pages give the three
 * segments and their sizes, not their order; the order above is the one
 * they are listed in.  Codes of rows no query may see are never converted
 * into a result (NaN codes or scales there are harmless). */
int mla_decode_latent_fp8(const uint16_t* q_lat, const uint16_t* q_pe, const uint8_t* kv_cache,
                          int num_blocks, int page_size, const int32_t* block_table,
                          int max_blocks_per_seq, const int32_t* seqlens, int B, int T, int H, int r,
                          int d_R, int max_seqlen, float softmax_scale, int num_splits,
                          void* workspace, size_t workspace_bytes, void* part_out,
                          mla_dtype part_dtype, float* part_lse, int32_t* split_indptr,
                          void* out_latent, mla_dtype out_dtype, float* lse, void* stream);

/* Split count of mla_decode_sparse: num_splits > 0 is returned as is; 0 picks
 * S = clamp(floor(CUs / (B*T*ceil(H/128))), 1, ceil(topk/256)) (and at most
 * 128), enough work units for every CU with chunks of at least 256 entries.
 * The split partial buffers of mla_decode_sparse hold B*T*S rows. */
int mla_sparse_split_count(int B, int T, int H, int topk, int num_splits, int* splits);

/* mla_decode_latent without caller scratch, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Arguments and results are those of
 * mla_decode_latent with out_latent required (the merged result is written);
 * the automatic plan's work list, split_indptr and the split partials (bf16,
 * with their f32 lse) live in a device array of 64 MiB that the library holds
 * on every GPU it runs on until the process ends.  No allocation and no
 * allocating library routine is called; the first call on a device resolves
 * that device's array address (hipGetSymbolAddress) and keeps it.
 *   num_splits  1: as mla_decode_latent (no scratch); S > 1 or 0 (automatic):
 *               split decode + merge through the array.
 * Limit: the plan (256 + 16 * rows bytes), split table (4 * (B + 1)), partial
 * lse (4 * rows * T * H) and bf16 partials (1024 * rows * T * H), each rounded
 * up to 256 bytes, must fit in 64 MiB, rows = max_total_splits of
 * mla_decode_workspace_size for the same arguments (on the headline geometry,
 * B = 64, H = 128, the automatic mode needs 42 MB); beyond it the call returns
 * MLA_ERR_WORKSPACE and enqueues nothing.  MLA_ERR_DEVICE if the current device
 * cannot be queried.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents: calls that overlap on one GPU (other streams or host threads) race
 * on it and must be serialised by the caller. */
int mla_decode_latent_noalloc(const uint16_t* q_lat, const uint16_t* q_pe, const uint16_t* kv_cache,
                              int num_blocks, int page_size, const int32_t* block_table, int max_blocks_per_seq,
                              const int32_t* seqlens, int B, int T, int H, int r, int d_R, int max_seqlen,
                              float softmax_scale, int num_splits, void* out_latent, mla_dtype out_dtype,
                              float* lse, void* stream);

/* Sparse (top-k) absorbed latent attention.  Query token (b, t) -- all H heads
 * -- attends to the cache rows listed in its index row, without a causal mask:
 *   indices     [B,T,topk] int32: physical row ids page * page_size + offset of
 *               the pool (no block table is read); entries past the valid
 *               prefix are never used (any value).  A repeated id counts once
 *               per occurrence.  Ids outside [0, num_blocks*page_size) inside
 *               the valid prefix are undefined behaviour (clamped into the
 *               pool, so never read outside it).
 *   topk_length [B] int32, nullable: valid prefix of the index rows of sequence
 *               b (clamped to [0, topk]); NULL means all topk entries.  A row
 *               with no valid entry gives out_latent 0 and lse -inf.
 *   q_lat, q_pe, kv_cache, softmax_scale, out_latent, out_dtype, lse: as for
 *               mla_decode_latent (kv_cache of at most 2^32 - 1 rows).
 *   num_splits  S from mla_sparse_split_count (0 = automatic): with S > 1 the
 *               valid prefix of every index row is cut into S chunks of
 *               ceil(ceil(n/S)/32)*32 entries; partial rows follow the
 *               mla_decode_latent layout over the B*T query tokens
 *               (part_out [B*T*S,H,r], part_lse [B*T*S,H], split_indptr
 *               [B*T+1]; merge over B*T "sequences" of one token each).
 * Source: M5.8 0x0B "Sparse indices are physical execution metadata" (the
 * index layout, physical ids, valid-prefix lengths) and 0x08 (sparse mode of
 * the runtime ABI: no causal mask).  The score, softmax and value sum are
 * those of mla_decode_latent over the selected rows. */
int mla_decode_sparse(const uint16_t* q_lat, const uint16_t* q_pe, const uint16_t* kv_cache,
                      int num_blocks, int page_size, const int32_t* indices, int topk,
                      const int32_t* topk_length, int B, int T, int H, int r, int d_R,
                      float softmax_scale, int num_splits, void* part_out, mla_dtype part_dtype,
                      float* part_lse, int32_t* split_indptr, void* out_latent, mla_dtype out_dtype,
                      float* lse, void* stream);

/* mla_decode_sparse over a pool of FP8 rows (the row layout of
 * mla_decode_latent_fp8: 512 E4M3 codes, four fp32 scales, 64 bf16 rope
 * values; 656 bytes, kv_cache 16-byte aligned): every argument and result as
 * for mla_decode_sparse, the selected rows dequantized to bf16 in the kernel
 * as mla_decode_latent_fp8 does (c = bf16(code * scale), nearest even).
 * Source: M5.8 0x0B ("Exact 656-byte FP8 row"; sparse indices are physical
 * execution metadata) and 0x08 (the checked sparse decode path reads the FP8
 * cache). */
int mla_decode_sparse_fp8(const uint16_t* q_lat, const uint16_t* q_pe, const uint8_t* kv_cache,
                          int num_blocks, int page_size, const int32_t* indices, int topk,
                          const int32_t* topk_length, int B, int T, int H, int r, int d_R,
                          float softmax_scale, int num_splits, void* part_out, mla_dtype part_dtype,
                          float* part_lse, int32_t* split_indptr, void* out_latent, mla_dtype out_dtype,
                          float* lse, void* stream);

/* Merge of split partial states, per (b,t,h) over rows k in
 * [split_indptr[b], split_indptr[b+1]):  M = max_k lse_k, w_k = exp(lse_k - M),
 * lse = M + log(sum_k w_k), out = sum_k w_k * part_out[k] / sum_k w_k.  Rows with
 * lse_k = -inf carry no weight.  Natural-log units only: an LSE in log2 units
 * merges into a plausible but wrong average (mlxcel Stage 2).
 *   part_out [*,T,H,r] f32 or bf16 (part_dtype), part_lse [*,T,H] f32,
 *   split_indptr [B+1] int32
 *   out_latent [B,T,H,r] bf16 or f32 (out_dtype), lse [B,T,H] f32 (nullable)
 * Source: M5.8 0x0C (exact merge of (m_r, l_r, o_r); averaging is wrong). */
int mla_merge_splits(const void* part_out, mla_dtype part_dtype, const float* part_lse,
                     const int32_t* split_indptr, int B, int T, int H, int r, void* out_latent,
                     mla_dtype out_dtype, float* lse, void* stream);

/* Un-absorb: out[b,t,h,v] = sum_{c<r} latent[b,t,h,c] * W_UV[h,v,c]; latent is
 * rounded to bf16 for the matrix cores when given as f32; fp32 accumulation.
 *   latent [B,T,H,r] bf16 or f32 (latent_dtype)   w_uv [H,d_V,r] bf16
 *   out    [B,T,H,d_V] f32
 * Source: "MLA in full detail", Step 4 (bmm (N,B,L) x (N,L,V)); M5.8 0x04
 * (einsum bhqc,hvc->bhqv; W_UV [H,d_V,d_c]). */
int mla_unabsorb_out(const void* latent, mla_dtype latent_dtype, const uint16_t* w_uv, float* out,
                     int B, int T, int H, int r, int d_V, void* stream);

/* Merge of split partials and un-absorb in one launch: the merge of
 * mla_merge_splits with a bf16 out_latent, followed by mla_unabsorb_out of that
 * latent.  The merged rows are rounded to bf16 in on-chip memory and multiplied
 * by W_UV there; only out and lse are written.
 *   part_out [*,T,H,r] f32 or bf16 (part_dtype), part_lse [*,T,H] f32,
 *   split_indptr [B+1] int32 (rows of each (b) as written by mla_decode_latent
 *   or mla_decode_sparse with merge left to the caller), w_uv [H,d_V,r] bf16
 *   out [B,T,H,d_V] f32, lse [B,T,H] f32 (nullable; the merged lse)
 * Errors (nothing is launched): MLA_ERR_SHAPE for B < 0, T < 1, H < 1 or
 * B*T > 2^24; MLA_ERR_UNSUPPORTED for r != 512, d_V != 128, T > 1024, H > 128
 * or another part_dtype; MLA_ERR_NULL / MLA_ERR_ALIGN for pointers.  B == 0
 * is a no-op.  Rows with no split (split_indptr[b] == split_indptr[b+1]) give
 * out = 0 and lse = -inf.  Results equal the two separate calls' (lse bit for
 * bit, out up to the order of the fp32 sums).  Faster than those calls when
 * every row has at most four splits and the partials are bf16 (a 32-row
 * block's loads all go out before any arithmetic); with more splits a row is
 * merged by one wave at a time and the separate calls are faster.
 * Sources: M5.8 0x0C (exact merge of split states) and "MLA in full detail",
 * Step 4 (W_UV folded into the output). */
int mla_merge_unabsorb(const void* part_out, mla_dtype part_dtype, const float* part_lse,
                       const int32_t* split_indptr, const uint16_t* w_uv, int B, int T, int H, int r, int d_V,
                       float* out, float* lse, void* stream);

/* Cache append: writes the T new rows [c (r) || k_pe (d_R)] of every sequence
 * into the paged cache, new row t of sequence b at logical position
 * j = seqlens[b] - T + t, i.e. at physical row
 *     block_table[b, j / page_size] * page_size + j % page_size
 * -- the convention mla_decode_latent reads with (seqlens counts the T new
 * rows).  Bytes are copied unchanged.  Rows whose position or block-table
 * entry is out of range are skipped (mla_validate_inputs checks the table).
 *   c_new [B,T,r] bf16, kpe_new [B,T,d_R] bf16 (already rotated),
 *   kv_cache [num_blocks,page_size,r+d_R] bf16 (written), block_table
 *   [B,max_blocks_per_seq] int32, seqlens [B] int32 (lengths after the append)
 * All pointers are device memory owned by the caller; c_new, kpe_new and
 * kv_cache 16-byte aligned, the int32 arrays 4-byte aligned.  Errors (nothing
 * is launched): MLA_ERR_SHAPE for B, num_blocks or max_blocks_per_seq < 0,
 * T < 1, or (B > 0) num_blocks or max_blocks_per_seq == 0;
 * MLA_ERR_UNSUPPORTED for r != 512, d_R != 64, T > 1024, page_size not a
 * multiple of 16 in [16, 1024], or B*T > 2^24; MLA_ERR_NULL / MLA_ERR_ALIGN
 * for pointers.  B == 0 is a no-op.
 * Source: M5.8 0x05, "Prefill publication contract" and "Exact phase
 * algorithms and commit state" (the decode step takes the new row once, at the
 * position the page table assigns it) and "Paged and ragged address
 * translation".  Synchronisation: stream order; the decode that reads the rows
 * must be launched after this call on the same stream (or after an event). */
int mla_append_cache(const uint16_t* c_new, const uint16_t* kpe_new, uint16_t* kv_cache, int num_blocks,
                     int page_size, const int32_t* block_table, int max_blocks_per_seq,
                     const int32_t* seqlens, int B, int T, int r, int d_R, void* stream);

/* Synchronous check of the device-resident index data of mla_decode_latent:
 * every needed block-table entry is in [0, num_blocks) and every seqlen is in
 * [T, max_seqlen] with ceil(seqlen/page_size) <= max_blocks_per_seq.  Copies
 * seqlens and the needed table entries to the host (blocking on `stream`).
 * Returns MLA_OK or MLA_ERR_INVALID_INDEX.  For debugging and tests. */
int mla_validate_inputs(const int32_t* block_table, int max_blocks_per_seq,
                        const int32_t* seqlens, int B, int T, int max_seqlen, int page_size,
                        int num_blocks, void* stream);

/* Static string for a status code. */
const char* mla_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MLA_LATENT_H */
