// Cache append: the T new rows of every sequence written into the paged latent
// cache before the decode that reads them (gfx950).
//
// The decode step projects the new token's cache row [c (512) || k_pe (64)] and
// attends over it once, at the position the page table gives it ("M5.8 -
// Multi-Head Latent Attention", 0x05: prefill publication contract, exact phase
// algorithms and commit state); rows live at
//     physical(j) = block_table[b, j / P] * P + j % P
// (0x05, paged and ragged address translation).
// With the decode's convention -- seqlens counts the T new rows, which are the
// last T positions -- new row t of sequence b goes to position
// j = seqlens[b] - T + t.
//
// One wave per row: 64 lanes copy the 1024-byte latent part and eight of them
// the 128-byte positional part, 16 bytes each.  Bytes are copied unchanged
// (bit-exact); a row whose position or block-table entry is out of range is
// skipped.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
  const int l = lane_id();
  const long long m = (long long)blockIdx.x * 4 + wave_id();  // new row (b, t)
  if (m >= (long long)p.B * p.T) return;
  const int b = (int)(m / p.T), t = (int)(m - (long long)b * p.T);
  const int j = p.seqlens[b] - p.T + t;
  if (j < 0) return;
  const int page = j / p.page_size;
  if (page >= p.max_blocks) return;
  const int blk = p.block_table[(size_t)b * p.max_blocks + page];
  if (blk < 0 || blk >= p.num_blocks) return;
  uint16_t* dst = p.cache + ((size_t)blk * p.page_size + (j - page * p.page_size)) * kRow;
  const uint16_t* c = p.c_new + (size_t)m * kR;
  const uint16_t* kpe = p.kpe_new + (size_t)m * kDR;
  *(u32x4*)(dst + 8 * l) = *(const u32x4*)(c + 8 * l);
  if (l < kDR / 8) *(u32x4*)(dst + kR + 8 * l) = *(const u32x4*)(kpe + 8 * l);
}

hipError_t launch_append(const AppendParams& prm, hipStream_t st) {
  const long long rows = (long long)prm.B * prm.T;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, prm);
  return hipGetLastError();
}

}  // namespace mla
