/*
 * mla_normal.h -- C ABI of libmla_normal.so, the Normal-path comparison library
 * of the matrix-absorbed MLA decode path (MI355X, gfx950).
 *
 * It computes the same attention as mla_absorb_q + mla_decode_latent +
 * mla_unabsorb_out (mla_latent.h) in the other association order: every
 * cached latent is up-projected per head into a 128-wide key part and a
 * 128-wide value, and each head runs ordinary attention with the 192-wide key
 * [k_nope || k_pe].  It exists to measure where the two orders cross over
 * ("MLA in full detail", cost analysis of the Normal and Absorb paths; M5.8
 * 0x06 "Crossover"), and is kept out of libmla_latent.so because its two
 * up-projection GEMMs are rocBLAS calls and rocBLAS keeps a handle, with its
 * own device workspace, per device.
 *
 * Status codes and conventions are those of mla_latent.h (device pointers,
 * caller-owned row-major buffers, a hipStream_t passed as void*, negative
 * mla_status on error with nothing enqueued), except that this library
 * allocates: the first call on a device creates that device's rocBLAS handle,
 * held until the process ends, and calls on one device are serialised by a
 * mutex while they enqueue.
 */
#ifndef MLA_NORMAL_H
#define MLA_NORMAL_H

#include <stddef.h>
#include <stdint.h>

#include "mla_latent.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Workspace of mla_decode_normal: the chunk's gathered latent and rope rows,
 * its up-projected keys and values ([B*chunk,H,128] bf16 each) and, with more
 * than one chunk (ceil(max_seqlen/chunk) > 1), the running state carried
 * between chunks.  B*chunk is at most 2^24 (MLA_ERR_UNSUPPORTED beyond).
 * Pure function of its arguments. */
int mla_normal_workspace_size(int B, int T, int H, int max_seqlen, int chunk, size_t* workspace_bytes);

/* The Normal (non-absorbed) path on the GPU: k_nope = W_UK[h] c_j and
 * v_j = W_UV[h] c_j for every cached latent c_j, then per head softmax of
 * (q_nope . k_nope + q_pe . k_pe) * scale over the visible keys and the
 * weighted sum of the v_j ("MLA in full detail", Steps 2-3 before the weights
 * are folded; M5.8 0x05 naive path).  The cache is processed `chunk` tokens
 * per sequence at a time: rows gathered through the block table, two rocBLAS
 * GEMMs for the up-projection, an MFMA attention kernel that carries the
 * running max, sum and unnormalised output from chunk to chunk (the exact
 * log-sum-exp combination of M5.8 0x0C).
 *   q_nope [B,T,H,128], q_pe [B,T,H,64], w_uk, w_uv [H,128,512] bf16; kv_cache,
 *   block_table, seqlens, max_seqlen, softmax_scale as for mla_decode_latent
 *   (causal over the T current rows).
 *   workspace  device memory of mla_normal_workspace_size bytes (16-byte aligned)
 *   out [B,T,H,128] f32, lse [B,T,H] f32 natural-log (nullable).
 * Returns MLA_ERR_WORKSPACE when the workspace is missing or smaller than
 * mla_normal_workspace_size reports, MLA_ERR_DEVICE when the current device
 * cannot be queried, MLA_ERR_LAUNCH when a kernel or GEMM fails to launch. */
int mla_decode_normal(const uint16_t* q_nope, const uint16_t* q_pe, const uint16_t* w_uk,
                      const uint16_t* w_uv, const uint16_t* kv_cache, int num_blocks, int page_size,
                      const int32_t* block_table, int max_blocks_per_seq, const int32_t* seqlens, int B,
                      int T, int H, int d_nope, int d_R, int d_V, int r, int max_seqlen,
                      float softmax_scale, int chunk, void* workspace, size_t workspace_bytes, float* out,
                      float* lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_NORMAL_H */
