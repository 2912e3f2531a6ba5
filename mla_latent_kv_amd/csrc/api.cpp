// C ABI of the absorbed MLA decode path: argument validation, workspace
// sizing and kernel launches.  No entry point allocates, synchronises (except
// mla_validate_inputs) or keeps state, and everything is enqueued on the
// caller's stream.  (The Normal-path comparison, whose rocBLAS GEMMs keep a
// handle per device, is a separate library: normal_api.cpp.)
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <vector>

#include "../../include/mla_latent.h"
#include "abi_check.hpp"
#include "launch.hpp"

namespace {

using namespace mla_abi;

constexpr int kMinChunk = 256;   // automatic split: smallest chunk in tokens
constexpr int kAutoCap = 128;    // automatic split: most chunks per sequence

int n_row_groups(int T, int H) { return (T * H + 127) / 128; }

int launch_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH; }

int device_cus(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_DEVICE;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return MLA_ERR_DEVICE;
  *cus = n;
  return MLA_OK;
}

// Workspace layout for split mode: [n_items (int32, padded to 256 B)] [work list int4 x max]
size_t plan_bytes(long long max_items) { return 256 + (size_t)max_items * 16; }

}  // namespace

extern "C" {

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL: return "required pointer is NULL";
    case MLA_ERR_ALIGN: return "pointer not 16-byte aligned (4-byte for int32 arrays)";
    case MLA_ERR_SHAPE: return "size out of range or inconsistent";
    case MLA_ERR_UNSUPPORTED: return "geometry not supported by this library";
    case MLA_ERR_WORKSPACE: return "workspace or partial-state buffers missing or too small";
    case MLA_ERR_LAUNCH: return "kernel launch failed";
    case MLA_ERR_INVALID_INDEX: return "block table entry or sequence length out of range";
    case MLA_ERR_DEVICE: return "HIP device query failed";
    default: return "unknown status";
  }
}

int mla_absorb_q(const uint16_t* q_nope, const uint16_t* w_uk, uint16_t* q_lat, int B, int T,
                 int H, int d_nope, int r, void* stream) {
  if (B < 0) return MLA_ERR_SHAPE;
  int st = check_heads(T, H);
  if (st) return st;
  if (d_nope != kDN || r != kR) return MLA_ERR_UNSUPPORTED;
  if (B == 0) return MLA_OK;
  if ((st = check_ptr16(q_nope)) || (st = check_ptr16(w_uk)) || (st = check_ptr16(q_lat))) return st;
  if ((long long)B * T > (1LL << 24)) return MLA_ERR_SHAPE;
  mla::AbsorbParams p{q_nope, w_uk, q_lat, B * T, H};
  return launch_status(mla::launch_absorb(p, (hipStream_t)stream));
}

int mla_unabsorb_out(const void* latent, mla_dtype latent_dtype, const uint16_t* w_uv, float* out,
                     int B, int T, int H, int r, int d_V, void* stream) {
  if (B < 0) return MLA_ERR_SHAPE;
  int st = check_heads(T, H);
  if (st) return st;
  if (r != kR || d_V != kDV) return MLA_ERR_UNSUPPORTED;
  if (latent_dtype != MLA_BF16 && latent_dtype != MLA_F32) return MLA_ERR_UNSUPPORTED;
  if (B == 0) return MLA_OK;
  if ((st = check_ptr16(latent)) || (st = check_ptr16(w_uv)) || (st = check_ptr16(out))) return st;
  if ((long long)B * T > (1LL << 24)) return MLA_ERR_SHAPE;
  mla::UnabsorbParams p{latent, w_uv, out, B * T, H};
  return launch_status(mla::launch_unabsorb(p, latent_dtype == MLA_F32, (hipStream_t)stream));
}

int mla_decode_workspace_size(int B, int T, int H, int r, int max_seqlen, int page_size,
                              int num_splits, size_t* workspace_bytes, int* max_total_splits) {
  if (!workspace_bytes || !max_total_splits) return MLA_ERR_NULL;
  if (B < 0 || max_seqlen < 0 || num_splits < 0) return MLA_ERR_SHAPE;
  int st = check_heads(T, H);
  if (st) return st;
  if (r != kR) return MLA_ERR_UNSUPPORTED;
  if (!page_size_ok(page_size)) return MLA_ERR_UNSUPPORTED;
  if (num_splits == 1 || B == 0) {
    *workspace_bytes = 0;
    *max_total_splits = 0;
    return MLA_OK;
  }
  long long max_items;
  if (num_splits > 1) {
    max_items = (long long)B * num_splits;
  } else {
    int cus = 0;
    if ((st = device_cus(&cus))) return st;
    max_items = std::min<long long>((long long)B * kAutoCap, (long long)B + cus);
  }
  if (max_items > (1LL << 30)) return MLA_ERR_SHAPE;
  // only the automatic mode keeps a device work list; uniform splits need none
  *workspace_bytes = num_splits == 0 ? plan_bytes(max_items) : 0;
  *max_total_splits = (int)max_items;
  return MLA_OK;
}

// dense decode over bf16 rows (fp8 false) or FP8 rows (fp8 true)
static int decode_impl(const uint16_t* q_lat, const uint16_t* q_pe, const void* kv_cache, bool fp8,
                       int num_blocks, int page_size, const int32_t* block_table,
                       int max_blocks_per_seq, const int32_t* seqlens, int B, int T, int H, int r,
                       int d_R, int max_seqlen, float softmax_scale, int num_splits,
                       void* workspace, size_t workspace_bytes, void* part_out,
                       mla_dtype part_dtype, float* part_lse, int32_t* split_indptr,
                       void* out_latent, mla_dtype out_dtype, float* lse, void* stream) {
  if (B < 0 || num_blocks < 1 || max_blocks_per_seq < 1 || max_seqlen < 0 || num_splits < 0)
    return MLA_ERR_SHAPE;
  int st = check_heads(T, H);
  if (st) return st;
  if (r != kR || d_R != kDR) return MLA_ERR_UNSUPPORTED;
  if (!page_size_ok(page_size)) return MLA_ERR_UNSUPPORTED;
  if (out_dtype != MLA_BF16 && out_dtype != MLA_F32) return MLA_ERR_UNSUPPORTED;
  if (part_dtype != MLA_BF16 && part_dtype != MLA_F32) return MLA_ERR_UNSUPPORTED;
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale)) return MLA_ERR_SHAPE;
  if (B == 0) return MLA_OK;
  if (max_seqlen < T) return MLA_ERR_SHAPE;
  if ((long long)(max_seqlen + page_size - 1) / page_size > max_blocks_per_seq) return MLA_ERR_SHAPE;
  if ((st = check_ptr16(q_lat)) || (st = check_ptr16(q_pe)) || (st = check_ptr16(kv_cache)))
    return st;
  if ((st = check_ptr4(block_table)) || (st = check_ptr4(seqlens))) return st;
  if (lse && !aligned4(lse)) return MLA_ERR_ALIGN;

  const int n_rg = n_row_groups(T, H);
  mla::DecodeParams p{};
  p.q_lat = q_lat;
  p.q_pe = q_pe;
  p.cache = kv_cache;
  p.block_table = block_table;
  p.seqlens = seqlens;
  p.B = B;
  p.T = T;
  p.H = H;
  p.page_size = page_size;
  p.max_blocks = max_blocks_per_seq;
  p.n_rg = n_rg;
  p.scale_log2 = softmax_scale * 1.4426950408889634f;
  hipStream_t s = (hipStream_t)stream;

  if (num_splits == 0 && out_latent) {
    // automatic mode with the merged result wanted: when one work unit per
    // sequence already fills every CU, the rule gives each sequence a single
    // chunk, so run unsplit (no partials, no merge)
    int cus = 0;
    if ((st = device_cus(&cus))) return st;
    if ((long long)B * n_rg >= cus) num_splits = 1;
  }
  if (num_splits == 1) {
    if ((st = check_ptr16(out_latent))) return st;
    p.out = out_latent;
    p.lse = lse;
    if ((long long)B * n_rg > (1LL << 31) - 8) return MLA_ERR_SHAPE;
    p.n_units = B * n_rg;
    return launch_status(mla::launch_decode(p, B * n_rg, false, out_dtype == MLA_F32, s, false, fp8));
  }

  // split mode
  size_t need = 0;
  int max_items = 0;
  if ((st = mla_decode_workspace_size(B, T, H, r, max_seqlen, page_size, num_splits, &need,
                                      &max_items)))
    return st;
  if (!part_out || !part_lse || !split_indptr) return MLA_ERR_WORKSPACE;
  if (need > 0 && (!workspace || workspace_bytes < need)) return MLA_ERR_WORKSPACE;
  if ((workspace && !aligned16(workspace)) || !aligned16(part_out) || !aligned4(part_lse) ||
      !aligned4(split_indptr))
    return MLA_ERR_ALIGN;
  if (out_latent && !aligned16(out_latent)) return MLA_ERR_ALIGN;
  if ((long long)max_items * n_rg > (1LL << 31) - 8) return MLA_ERR_SHAPE;

  p.part_out = part_out;
  p.part_lse = part_lse;
  p.split_indptr = split_indptr;
  p.num_splits = num_splits;
  p.n_units = max_items * n_rg;
  if (num_splits == 0) {
    // automatic split counts need the lengths: a one-workgroup plan kernel builds
    // the work list on the device (no host synchronisation)
    int32_t* n_items = (int32_t*)workspace;
    int32_t* work = (int32_t*)((char*)workspace + 256);
    mla::PlanParams pp{};
    pp.seqlens = seqlens;
    pp.B = B;
    pp.num_splits = 0;
    pp.page_size = page_size;
    pp.min_chunk = kMinChunk;
    pp.cap = kAutoCap;
    int cus = 0;
    if ((st = device_cus(&cus))) return st;
    pp.target_units = std::max(1, cus / n_rg);
    pp.work = work;
    pp.n_items = n_items;
    pp.split_indptr = split_indptr;
    if ((st = launch_status(mla::launch_plan(pp, s)))) return st;
    p.work = work;
    p.n_items = n_items;
  }
  const bool part_f32 = part_dtype == MLA_F32;
  if ((st = launch_status(mla::launch_decode(p, max_items * n_rg, true, part_f32, s, false, fp8)))) return st;
  if (out_latent) {
    mla::MergeParams mp{part_out, part_lse, split_indptr, B, T * H, out_latent, lse};
    return launch_status(mla::launch_merge(mp, part_f32, out_dtype == MLA_F32, s));
  }
  return MLA_OK;
}

int mla_decode_latent(const uint16_t* q_lat, const uint16_t* q_pe, const uint16_t* kv_cache,
                      int num_blocks, int page_size, const int32_t* block_table,
                      int max_blocks_per_seq, const int32_t* seqlens, int B, int T, int H, int r,
                      int d_R, int max_seqlen, float softmax_scale, int num_splits,
                      void* workspace, size_t workspace_bytes, void* part_out,
                      mla_dtype part_dtype, float* part_lse, int32_t* split_indptr,
                      void* out_latent, mla_dtype out_dtype, float* lse, void* stream) {
  return decode_impl(q_lat, q_pe, kv_cache, false, num_blocks, page_size, block_table, max_blocks_per_seq,
                     seqlens, B, T, H, r, d_R, max_seqlen, softmax_scale, num_splits, workspace,
                     workspace_bytes, part_out, part_dtype, part_lse, split_indptr, out_latent, out_dtype, lse,
                     stream);
}

int mla_decode_latent_fp8(const uint16_t* q_lat, const uint16_t* q_pe, const uint8_t* kv_cache,
                          int num_blocks, int page_size, const int32_t* block_table,
                          int max_blocks_per_seq, const int32_t* seqlens, int B, int T, int H, int r,
                          int d_R, int max_seqlen, float softmax_scale, int num_splits,
                          void* workspace, size_t workspace_bytes, void* part_out,
                          mla_dtype part_dtype, float* part_lse, int32_t* split_indptr,
                          void* out_latent, mla_dtype out_dtype, float* lse, void* stream) {
  return decode_impl(q_lat, q_pe, kv_cache, true, num_blocks, page_size, block_table, max_blocks_per_seq,
                     seqlens, B, T, H, r, d_R, max_seqlen, softmax_scale, num_splits, workspace,
                     workspace_bytes, part_out, part_dtype, part_lse, split_indptr, out_latent, out_dtype, lse,
                     stream);
}

int mla_sparse_split_count(int B, int T, int H, int topk, int num_splits, int* splits) {
  if (!splits) return MLA_ERR_NULL;
  if (B < 0 || topk < 1 || num_splits < 0) return MLA_ERR_SHAPE;
  int st = check_heads(T, H);
  if (st) return st;
  if (num_splits > 0) {
    *splits = num_splits;
    return MLA_OK;
  }
  if (B == 0) {
    *splits = 1;
    return MLA_OK;
  }
  // every index row has the same capacity topk: one uniform split count that
  // brings the work units up to the CU count, with chunks of at least
  // kMinChunk entries
  int cus = 0;
  if ((st = device_cus(&cus))) return st;
  const long long units = (long long)B * T * ((H + 127) / 128);
  long long sc = cus / units;
  sc = std::min<long long>(sc, (topk + kMinChunk - 1) / kMinChunk);
  sc = std::min<long long>(std::max<long long>(sc, 1), kAutoCap);
  *splits = (int)sc;
  return MLA_OK;
}

// sparse decode over bf16 rows (fp8 false) or FP8 rows (fp8 true)
static int sparse_impl(const uint16_t* q_lat, const uint16_t* q_pe, const void* kv_cache, bool fp8,
                       int num_blocks, int page_size, const int32_t* indices, int topk,
                       const int32_t* topk_length, int B, int T, int H, int r, int d_R,
                       float softmax_scale, int num_splits, void* part_out, mla_dtype part_dtype,
                       float* part_lse, int32_t* split_indptr, void* out_latent, mla_dtype out_dtype,
                       float* lse, void* stream) {
  if (B < 0 || num_blocks < 1 || topk < 1 || num_splits < 0) return MLA_ERR_SHAPE;
  int st = check_heads(T, H);
  if (st) return st;
  if (r != kR || d_R != kDR) return MLA_ERR_UNSUPPORTED;
  if (!page_size_ok(page_size)) return MLA_ERR_UNSUPPORTED;
  if (out_dtype != MLA_BF16 && out_dtype != MLA_F32) return MLA_ERR_UNSUPPORTED;
  if (part_dtype != MLA_BF16 && part_dtype != MLA_F32) return MLA_ERR_UNSUPPORTED;
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale)) return MLA_ERR_SHAPE;
  if (B == 0) return MLA_OK;
  const long long rows = (long long)num_blocks * page_size;
  if (rows > 0xFFFFFFFFLL) return MLA_ERR_UNSUPPORTED;
  if ((st = check_ptr16(q_lat)) || (st = check_ptr16(q_pe)) || (st = check_ptr16(kv_cache))) return st;
  if ((st = check_ptr4(indices))) return st;
  if ((topk_length && !aligned4(topk_length)) || (lse && !aligned4(lse))) return MLA_ERR_ALIGN;
  int S = 0;
  if ((st = mla_sparse_split_count(B, T, H, topk, num_splits, &S))) return st;

  // the kernel's work sequences are the B*T query tokens, one query row group
  // per token (its H heads), each over its own index row
  const long long BT = (long long)B * T;
  const int n_rg = (H + 127) / 128;
  if (BT * S * n_rg > (1LL << 31) - 8) return MLA_ERR_SHAPE;
  mla::DecodeParams p{};
  p.q_lat = q_lat;
  p.q_pe = q_pe;
  p.cache = kv_cache;
  p.indices = indices;
  p.topk_length = topk_length;
  p.topk = topk;
  p.sp_T = T;
  p.num_rows = (uint32_t)rows;
  p.B = (int)BT;
  p.T = 1;
  p.H = H;
  p.page_size = 32;  // chunk rounding of the uniform split: whole 32-entry steps
  p.n_rg = n_rg;
  p.scale_log2 = softmax_scale * 1.4426950408889634f;
  hipStream_t s = (hipStream_t)stream;
  if (S == 1) {
    if ((st = check_ptr16(out_latent))) return st;
    p.out = out_latent;
    p.lse = lse;
    p.n_units = (int)(BT * n_rg);
    return launch_status(mla::launch_decode(p, p.n_units, false, out_dtype == MLA_F32, s, true, fp8));
  }
  if (!part_out || !part_lse || !split_indptr) return MLA_ERR_WORKSPACE;
  if (!aligned16(part_out) || !aligned4(part_lse) || !aligned4(split_indptr)) return MLA_ERR_ALIGN;
  if (out_latent && !aligned16(out_latent)) return MLA_ERR_ALIGN;
  p.part_out = part_out;
  p.part_lse = part_lse;
  p.split_indptr = split_indptr;
  p.num_splits = S;
  p.n_units = (int)(BT * S * n_rg);
  const bool part_f32 = part_dtype == MLA_F32;
  if ((st = launch_status(mla::launch_decode(p, p.n_units, true, part_f32, s, true, fp8)))) return st;
  if (out_latent) {
    mla::MergeParams mp{part_out, part_lse, split_indptr, (int)BT, H, out_latent, lse};
    return launch_status(mla::launch_merge(mp, part_f32, out_dtype == MLA_F32, s));
  }
  return MLA_OK;
}

int mla_decode_sparse(const uint16_t* q_lat, const uint16_t* q_pe, const uint16_t* kv_cache,
                      int num_blocks, int page_size, const int32_t* indices, int topk,
                      const int32_t* topk_length, int B, int T, int H, int r, int d_R,
                      float softmax_scale, int num_splits, void* part_out, mla_dtype part_dtype,
                      float* part_lse, int32_t* split_indptr, void* out_latent, mla_dtype out_dtype,
                      float* lse, void* stream) {
  return sparse_impl(q_lat, q_pe, kv_cache, false, num_blocks, page_size, indices, topk, topk_length, B, T, H, r,
                     d_R, softmax_scale, num_splits, part_out, part_dtype, part_lse, split_indptr, out_latent,
                     out_dtype, lse, stream);
}

int mla_decode_sparse_fp8(const uint16_t* q_lat, const uint16_t* q_pe, const uint8_t* kv_cache,
                          int num_blocks, int page_size, const int32_t* indices, int topk,
                          const int32_t* topk_length, int B, int T, int H, int r, int d_R,
                          float softmax_scale, int num_splits, void* part_out, mla_dtype part_dtype,
                          float* part_lse, int32_t* split_indptr, void* out_latent, mla_dtype out_dtype,
                          float* lse, void* stream) {
  return sparse_impl(q_lat, q_pe, kv_cache, true, num_blocks, page_size, indices, topk, topk_length, B, T, H, r,
                     d_R, softmax_scale, num_splits, part_out, part_dtype, part_lse, split_indptr, out_latent,
                     out_dtype, lse, stream);
}

int mla_append_cache(const uint16_t* c_new, const uint16_t* kpe_new, uint16_t* kv_cache, int num_blocks,
                     int page_size, const int32_t* block_table, int max_blocks_per_seq,
                     const int32_t* seqlens, int B, int T, int r, int d_R, void* stream) {
  if (B < 0 || num_blocks < 0 || max_blocks_per_seq < 0) return MLA_ERR_SHAPE;
  if (T < 1) return MLA_ERR_SHAPE;
  if (T > kMaxT) return MLA_ERR_UNSUPPORTED;
  if (r != kR || d_R != kDR) return MLA_ERR_UNSUPPORTED;
  if (!page_size_ok(page_size)) return MLA_ERR_UNSUPPORTED;
  if (B == 0) return MLA_OK;
  if (num_blocks < 1 || max_blocks_per_seq < 1) return MLA_ERR_SHAPE;
  int st;
  if ((st = check_ptr16(c_new)) || (st = check_ptr16(kpe_new)) || (st = check_ptr16(kv_cache)) ||
      (st = check_ptr4(block_table)) || (st = check_ptr4(seqlens)))
    return st;
  if ((long long)B * T > (1LL << 24)) return MLA_ERR_UNSUPPORTED;  // grid of B*T/4 workgroups
  mla::AppendParams p{c_new, kpe_new, kv_cache, block_table, seqlens, B, T, page_size, max_blocks_per_seq,
                      num_blocks};
  return launch_status(mla::launch_append(p, (hipStream_t)stream));
}

int mla_merge_splits(const void* part_out, mla_dtype part_dtype, const float* part_lse,
                     const int32_t* split_indptr, int B, int T, int H, int r, void* out_latent,
                     mla_dtype out_dtype, float* lse, void* stream) {
  if (B < 0) return MLA_ERR_SHAPE;
  int st = check_heads(T, H);
  if (st) return st;
  if (r != kR) return MLA_ERR_UNSUPPORTED;
  if (out_dtype != MLA_BF16 && out_dtype != MLA_F32) return MLA_ERR_UNSUPPORTED;
  if (part_dtype != MLA_BF16 && part_dtype != MLA_F32) return MLA_ERR_UNSUPPORTED;
  if (B == 0) return MLA_OK;
  if ((st = check_ptr16(part_out)) || (st = check_ptr4(part_lse)) || (st = check_ptr4(split_indptr)) ||
      (st = check_ptr16(out_latent)))
    return st;
  if (lse && !aligned4(lse)) return MLA_ERR_ALIGN;
  if ((long long)B * T * H > (1LL << 31) - 1) return MLA_ERR_SHAPE;
  mla::MergeParams mp{part_out, part_lse, split_indptr, B, T * H, out_latent, lse};
  return launch_status(
      mla::launch_merge(mp, part_dtype == MLA_F32, out_dtype == MLA_F32, (hipStream_t)stream));
}

// Workgroups per head of the merge + un-absorb kernel: enough row blocks per
// head to give each of the 256 CUs one workgroup, never more than there are
// blocks (a workgroup holds one head's W_UV in LDS for all the blocks it takes).
static int merge_unabsorb_groups(int M, int H) {
  const int blocks = (M + mla::kMergeUnabsorbRows - 1) / mla::kMergeUnabsorbRows;
  const int want = (256 + H - 1) / H;
  return blocks < want ? blocks : want;
}

int mla_merge_unabsorb(const void* part_out, mla_dtype part_dtype, const float* part_lse,
                       const int32_t* split_indptr, const uint16_t* w_uv, int B, int T, int H, int r, int d_V,
                       float* out, float* lse, void* stream) {
  if (B < 0) return MLA_ERR_SHAPE;
  int st = check_heads(T, H);
  if (st) return st;
  if (r != kR || d_V != kDV) return MLA_ERR_UNSUPPORTED;
  if (part_dtype != MLA_BF16 && part_dtype != MLA_F32) return MLA_ERR_UNSUPPORTED;
  if (B == 0) return MLA_OK;
  if ((st = check_ptr16(part_out)) || (st = check_ptr4(part_lse)) || (st = check_ptr4(split_indptr)) ||
      (st = check_ptr16(w_uv)) || (st = check_ptr16(out)))
    return st;
  if (lse && !aligned4(lse)) return MLA_ERR_ALIGN;
  if ((long long)B * T > (1LL << 24)) return MLA_ERR_SHAPE;
  const int M = B * T;
  mla::MergeUnabsorbParams p{part_out, part_lse, split_indptr, w_uv, out, lse, M, T, H,
                             merge_unabsorb_groups(M, H)};
  return launch_status(mla::launch_merge_unabsorb(p, part_dtype == MLA_F32, (hipStream_t)stream));
}

int mla_validate_inputs(const int32_t* block_table, int max_blocks_per_seq,
                        const int32_t* seqlens, int B, int T, int max_seqlen, int page_size,
                        int num_blocks, void* stream) {
  if (B < 0 || T < 1 || max_blocks_per_seq < 1 || page_size < 1 || num_blocks < 1)
    return MLA_ERR_SHAPE;
  if (B == 0) return MLA_OK;
  int st;
  if ((st = check_ptr4(block_table)) || (st = check_ptr4(seqlens))) return st;
  hipStream_t s = (hipStream_t)stream;
  std::vector<int32_t> sl(B), bt((size_t)B * max_blocks_per_seq);
  if (hipMemcpyAsync(sl.data(), seqlens, sizeof(int32_t) * B, hipMemcpyDeviceToHost, s) !=
          hipSuccess ||
      hipMemcpyAsync(bt.data(), block_table, sizeof(int32_t) * bt.size(), hipMemcpyDeviceToHost,
                     s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return MLA_ERR_DEVICE;
  for (int b = 0; b < B; ++b) {
    const int L = sl[b];
    if (L < T || L > max_seqlen) return MLA_ERR_INVALID_INDEX;
    const long long pages = ((long long)L + page_size - 1) / page_size;
    if (pages > max_blocks_per_seq) return MLA_ERR_INVALID_INDEX;
    for (long long pg = 0; pg < pages; ++pg) {
      const int32_t e = bt[(size_t)b * max_blocks_per_seq + pg];
      if (e < 0 || e >= num_blocks) return MLA_ERR_INVALID_INDEX;
    }
  }
  return MLA_OK;
}

}  // extern "C"
