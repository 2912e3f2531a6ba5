// Internal launch interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

struct DecodeParams {
  const uint16_t* q_lat;       // [B,T,H,512] bf16
  const uint16_t* q_pe;        // [B,T,H,64] bf16
  const void* cache;           // [num_blocks,P,576] bf16 rows, or [num_blocks,P,656] FP8 rows
  const int32_t* block_table;  // [B,max_blocks]
  const int32_t* seqlens;      // [B]
  const int32_t* work;         // automatic split: [n][4] = (b, j0, j1, slot); NULL = uniform
  const int32_t* n_items;      // automatic split: number of work items (device)
  int num_splits;              // uniform split count (work == NULL)
  int32_t* split_indptr;       // uniform split: written by the decode kernel
  int B, T, H, page_size, max_blocks;
  int n_rg;                    // workgroups per work item (ceil(T*H/128))
  int n_units;                 // work items x n_rg (unused with the automatic work list)
  float scale_log2;            // softmax_scale * log2(e)
  void* part_out;              // split mode: [*,T,H,512] f32 or bf16
  float* part_lse;             // split mode: [*,T,H] f32
  void* out;                   // unsplit: [B,T,H,512] bf16 or f32
  float* lse;                  // unsplit: [B,T,H] f32, nullable
  // sparse (top-k) mode: the kernel's "sequences" are the B*T query tokens
  // (T = 1 above); each reads the rows listed in its index row
  const int32_t* indices;      // [B*T, topk] physical row ids
  const int32_t* topk_length;  // [B] valid prefix per sequence, nullable
  int topk, sp_T;              // entries per index row; query tokens per sequence
  uint32_t num_rows;           // rows in the cache pool (index clamp)
};

struct PlanParams {
  const int32_t* seqlens;
  int B, num_splits, page_size;
  int target_units, min_chunk, cap;  // automatic split policy
  int32_t* work;
  int32_t* n_items;
  int32_t* split_indptr;
};

struct MergeParams {
  const void* part_out;        // [*,TH,512] f32 or bf16
  const float* part_lse;
  const int32_t* split_indptr;
  int B, TH;
  void* out;
  float* lse;
};

struct AbsorbParams {
  const uint16_t* q_nope;  // [M,H,128] (M = B*T)
  const uint16_t* w_uk;    // [H,128,512]
  uint16_t* q_lat;         // [M,H,512]
  int M, H;
};

struct UnabsorbParams {
  const void* latent;      // [M,H,512] bf16 or f32
  const uint16_t* w_uv;    // [H,128,512]
  float* out;              // [M,H,128]
  int M, H;
};

// Query rows per block of the merge + un-absorb kernel (one workgroup takes
// blocks j, j + groups, ... of one head).
constexpr int kMergeUnabsorbRows = 32;

struct MergeUnabsorbParams {
  const void* part_out;        // [*,T,H,512] f32 or bf16 (split rows of split_indptr)
  const float* part_lse;       // [*,T,H]
  const int32_t* split_indptr; // [B+1]
  const uint16_t* w_uv;        // [H,128,512]
  float* out;                  // [B,T,H,128]
  float* lse;                  // [B,T,H], nullable
  int M, T, H;                 // M = B*T query rows
  int groups;                  // workgroups per head, 1 .. ceil(M / kMergeUnabsorbRows)
};

struct AppendParams {
  const uint16_t* c_new;       // [B,T,512] bf16
  const uint16_t* kpe_new;     // [B,T,64] bf16
  uint16_t* cache;             // [num_blocks,P,576] bf16
  const int32_t* block_table;  // [B,max_blocks]
  const int32_t* seqlens;      // [B], counting the T new rows
  int B, T, page_size, max_blocks, num_blocks;
};

struct NormalParams {
  const uint16_t* q_nope;      // [B,T,H,128]
  const uint16_t* q_pe;        // [B,T,H,64]
  const uint16_t* cache;       // [num_blocks,P,576]
  const int32_t* block_table;  // [B,max_blocks]
  const int32_t* seqlens;      // [B]
  uint16_t* lat;               // [B*chunk,512] gathered latent rows of the chunk
  uint16_t* rope;              // [B*chunk,64]  their rope parts
  const uint16_t* kbuf;        // [B*chunk,H,128] up-projected keys
  const uint16_t* vbuf;        // [B*chunk,H,128] up-projected values
  float* o_state;              // [B,T,H,128] unnormalised output carried between chunks
  float* m_state;              // [B,T,H] running max (log2 units)
  float* l_state;              // [B,T,H] running sum
  float* out;                  // [B,T,H,128]
  float* lse;                  // [B,T,H], nullable
  int B, T, H, page_size, max_blocks, chunk, c, first, last;
  float scale_log2;
};

// max_units: upper bound of work items x n_rg (the grid is derived from it)
hipError_t launch_decode(const DecodeParams& p, int max_units, bool split, bool out_f32, hipStream_t st,
                         bool sparse = false, bool fp8 = false);
hipError_t launch_plan(const PlanParams& p, hipStream_t st);
hipError_t launch_merge(const MergeParams& p, bool part_f32, bool out_f32, hipStream_t st);
hipError_t launch_absorb(const AbsorbParams& p, hipStream_t st);
hipError_t launch_unabsorb(const UnabsorbParams& p, bool latent_f32, hipStream_t st);
hipError_t launch_merge_unabsorb(const MergeUnabsorbParams& p, bool part_f32, hipStream_t st);
hipError_t launch_append(const AppendParams& p, hipStream_t st);
hipError_t launch_gather(const NormalParams& p, hipStream_t st);
hipError_t launch_mha(const NormalParams& p, hipStream_t st);

}  // namespace mla
