// mla_decode_latent_noalloc: the split-KV decode with its scratch (automatic
// split plan, split table, bf16 partial states) in a file-scope device array
// instead of caller buffers, for callers that cannot allocate device memory.
//
// The array is a `__device__` global of kScratchBytes: every GPU this library
// runs on holds its own copy from the moment the code object is loaded until
// the process ends.  Host code never uses the array's name as an address (on
// the host it is only a stand-in symbol); the device address is resolved once
// per device with hipGetSymbolAddress, with that device current, and kept in
// g_noalloc_ptr[device].  That table and its mutex are the only mutable host state
// of libmla_latent.so, and they belong to this entry point alone.
//
// Every call on one GPU shares that GPU's array, which keeps the last call's
// contents: calls that overlap on one GPU (other streams, other host threads)
// race on it.  Nothing in it needs clearing between calls: the plan kernel
// writes the work list and split table, the decode kernel writes every partial
// row the merge reads (empty chunks write a zero row and lse -inf).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "../../include/mla_latent.h"
#include "abi_check.hpp"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;   // 64 MiB per device
constexpr int kMaxDevices = 64;

__device__ __attribute__((aligned(256))) uint8_t noalloc_scratch[kScratchBytes];

std::mutex g_noalloc_mu;
void* g_noalloc_ptr[kMaxDevices] = {};

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Device address of this device's scratch array (resolved on first use).
int scratch_ptr(void** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  if (!g_noalloc_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(noalloc_scratch)) != hipSuccess || !p) return MLA_ERR_DEVICE;
    g_noalloc_ptr[dev] = p;
  }
  *ptr = g_noalloc_ptr[dev];
  return MLA_OK;
}

// Scratch bytes a call needs: the automatic plan's work list, the split table,
// the partials' lse and the bf16 partial outputs, each 256-byte aligned.
int scratch_bytes(int B, int T, int H, int max_seqlen, int page_size, int num_splits, size_t* bytes) {
  size_t ws = 0;
  int rows = 0;
  int st = mla_decode_workspace_size(B, T, H, mla_abi::kR, max_seqlen, page_size, num_splits, &ws, &rows);
  if (st) return st;
  if (num_splits == 1 || B == 0) {
    *bytes = 0;
    return MLA_OK;
  }
  const size_t th = (size_t)T * (size_t)H;
  *bytes = round256(ws) + round256(4 * ((size_t)B + 1)) + round256(4 * (size_t)rows * th) +
           round256(2 * (size_t)rows * th * mla_abi::kR);
  return MLA_OK;
}

}  // namespace

extern "C" {

int mla_decode_latent_noalloc(const uint16_t* q_lat, const uint16_t* q_pe, const uint16_t* kv_cache,
                              int num_blocks, int page_size, const int32_t* block_table, int max_blocks_per_seq,
                              const int32_t* seqlens, int B, int T, int H, int r, int d_R, int max_seqlen,
                              float softmax_scale, int num_splits, void* out_latent, mla_dtype out_dtype,
                              float* lse, void* stream) {
  if (!out_latent && B > 0) return MLA_ERR_NULL;
  if (num_splits == 1 || B <= 0)
    return mla_decode_latent(q_lat, q_pe, kv_cache, num_blocks, page_size, block_table, max_blocks_per_seq,
                             seqlens, B, T, H, r, d_R, max_seqlen, softmax_scale, 1, nullptr, 0, nullptr, MLA_BF16,
                             nullptr, nullptr, out_latent, out_dtype, lse, stream);
  if (r != mla_abi::kR) return MLA_ERR_UNSUPPORTED;
  size_t need = 0;
  int st = scratch_bytes(B, T, H, max_seqlen, page_size, num_splits, &need);
  if (st) return st;
  if (need > kScratchBytes) return MLA_ERR_WORKSPACE;
  size_t ws = 0;
  int rows = 0;
  if ((st = mla_decode_workspace_size(B, T, H, r, max_seqlen, page_size, num_splits, &ws, &rows))) return st;
  void* base = nullptr;
  if ((st = scratch_ptr(&base))) return st;
  // layout: [work list][split_indptr][part_lse][part_out], each 256-byte aligned
  const size_t th = (size_t)T * (size_t)H;
  uint8_t* p = (uint8_t*)base;
  void* work = ws ? p : nullptr;
  p += round256(ws);
  int32_t* indptr = (int32_t*)p;
  p += round256(4 * ((size_t)B + 1));
  float* part_lse = (float*)p;
  p += round256(4 * (size_t)rows * th);
  void* part_out = p;
  return mla_decode_latent(q_lat, q_pe, kv_cache, num_blocks, page_size, block_table, max_blocks_per_seq, seqlens,
                           B, T, H, r, d_R, max_seqlen, softmax_scale, num_splits, work, ws, part_out, MLA_BF16,
                           part_lse, indptr, out_latent, out_dtype, lse, stream);
}

}  // extern "C"
