// C ABI of the Normal-path comparison library (libmla_normal.so): the same
// attention as the absorbed path, computed with per-head up-projected keys and
// values.  It is kept out of libmla_latent.so because its two up-projection
// GEMMs are rocBLAS calls, and rocBLAS keeps a handle (and its own workspace)
// per device: the one piece of state and allocation in this project, confined
// to this library.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/mla_normal.h"
#include "abi_check.hpp"
#include "launch.hpp"

namespace {

using namespace mla_abi;

int launch_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH; }

// rocBLAS handle of each device, created on first use and kept until the
// process ends
std::mutex g_blas_mu;
rocblas_handle g_blas[64] = {};

// (the caller holds g_blas_mu: a handle's stream is set per call, so host
// threads that share the device's handle take turns enqueueing)
int blas_handle(rocblas_handle* h) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MLA_ERR_DEVICE;
  if (!g_blas[dev] && rocblas_create_handle(&g_blas[dev]) != rocblas_status_success) return MLA_ERR_LAUNCH;
  *h = g_blas[dev];
  return MLA_OK;
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

struct NormalLayout {
  size_t lat, rope, k, v, o, m, l, total;
};
NormalLayout normal_layout(long long B, long long T, long long H, long long chunk, bool state) {
  NormalLayout w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += round256(bytes);
    return at;
  };
  w.lat = take((size_t)(B * chunk * kR * 2));
  w.rope = take((size_t)(B * chunk * kDR * 2));
  w.k = take((size_t)(B * chunk * H * kDN * 2));
  w.v = take((size_t)(B * chunk * H * kDV * 2));
  if (state) {
    w.o = take((size_t)(B * T * H * kDV * 4));
    w.m = take((size_t)(B * T * H * 4));
    w.l = take((size_t)(B * T * H * 4));
  }
  w.total = off;
  return w;
}

}  // namespace

extern "C" {

int mla_normal_workspace_size(int B, int T, int H, int max_seqlen, int chunk, size_t* workspace_bytes) {
  if (!workspace_bytes) return MLA_ERR_NULL;
  if (B < 0 || max_seqlen < 0 || chunk < 1) return MLA_ERR_SHAPE;
  int st = check_heads(T, H);
  if (st) return st;
  if ((long long)B * chunk > (1LL << 24)) return MLA_ERR_UNSUPPORTED;
  const bool state = ((long long)max_seqlen + chunk - 1) / chunk > 1;
  *workspace_bytes = B == 0 ? 0 : normal_layout(B, T, H, chunk, state).total;
  return MLA_OK;
}

int mla_decode_normal(const uint16_t* q_nope, const uint16_t* q_pe, const uint16_t* w_uk,
                      const uint16_t* w_uv, const uint16_t* kv_cache, int num_blocks, int page_size,
                      const int32_t* block_table, int max_blocks_per_seq, const int32_t* seqlens, int B,
                      int T, int H, int d_nope, int d_R, int d_V, int r, int max_seqlen,
                      float softmax_scale, int chunk, void* workspace, size_t workspace_bytes, float* out,
                      float* lse, void* stream) {
  if (B < 0 || num_blocks < 1 || max_blocks_per_seq < 1 || max_seqlen < 0 || chunk < 1)
    return MLA_ERR_SHAPE;
  int st = check_heads(T, H);
  if (st) return st;
  if (d_nope != kDN || d_R != kDR || d_V != kDV || r != kR) return MLA_ERR_UNSUPPORTED;
  if (!page_size_ok(page_size)) return MLA_ERR_UNSUPPORTED;
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale)) return MLA_ERR_SHAPE;
  if (B == 0) return MLA_OK;
  if (max_seqlen < T) return MLA_ERR_SHAPE;
  if (((long long)max_seqlen + page_size - 1) / page_size > max_blocks_per_seq) return MLA_ERR_SHAPE;
  size_t need = 0;
  if ((st = mla_normal_workspace_size(B, T, H, max_seqlen, chunk, &need))) return st;
  if (!workspace || workspace_bytes < need) return MLA_ERR_WORKSPACE;
  if ((st = check_ptr16(q_nope)) || (st = check_ptr16(q_pe)) || (st = check_ptr16(w_uk)) ||
      (st = check_ptr16(w_uv)) || (st = check_ptr16(kv_cache)) || (st = check_ptr16(out)) ||
      (st = check_ptr16(workspace)))
    return st;
  if ((st = check_ptr4(block_table)) || (st = check_ptr4(seqlens))) return st;
  if (lse && !aligned4(lse)) return MLA_ERR_ALIGN;
  const long long units = (long long)B * H * ((T + 127) / 128);
  if (units > (1LL << 31) - 1) return MLA_ERR_SHAPE;

  const int n_chunks = std::max(1, (int)(((long long)max_seqlen + chunk - 1) / chunk));
  const NormalLayout wl = normal_layout(B, T, H, chunk, n_chunks > 1);
  char* ws = (char*)workspace;
  hipStream_t s = (hipStream_t)stream;
  std::lock_guard<std::mutex> lock(g_blas_mu);
  rocblas_handle bh = nullptr;
  if ((st = blas_handle(&bh))) return st;
  if (rocblas_set_stream(bh, s) != rocblas_status_success) return MLA_ERR_LAUNCH;

  mla::NormalParams p{};
  p.q_nope = q_nope;
  p.q_pe = q_pe;
  p.cache = kv_cache;
  p.block_table = block_table;
  p.seqlens = seqlens;
  p.lat = (uint16_t*)(ws + wl.lat);
  p.rope = (uint16_t*)(ws + wl.rope);
  p.kbuf = (const uint16_t*)(ws + wl.k);
  p.vbuf = (const uint16_t*)(ws + wl.v);
  if (n_chunks > 1) {
    p.o_state = (float*)(ws + wl.o);
    p.m_state = (float*)(ws + wl.m);
    p.l_state = (float*)(ws + wl.l);
  }
  p.out = out;
  p.lse = lse;
  p.B = B;
  p.T = T;
  p.H = H;
  p.page_size = page_size;
  p.max_blocks = max_blocks_per_seq;
  p.chunk = chunk;
  p.scale_log2 = softmax_scale * 1.4426950408889634f;
  // up-projection of the chunk's latents, all heads at once:
  //   K[m, h*128 + n] = sum_c lat[m, c] W_UK[h, n, c]   (V likewise with W_UV)
  // column-major view: K^T (N x M) = W^T(op T of the 512 x N view) x lat^T (512 x M)
  const int M = B * chunk, N = H * kDN;
  const float alpha = 1.f, beta = 0.f;
  for (int c = 0; c < n_chunks; ++c) {
    p.c = c;
    p.first = c == 0;
    p.last = c == n_chunks - 1;
    if ((st = launch_status(mla::launch_gather(p, s)))) return st;
    const uint16_t* wts[2] = {w_uk, w_uv};
    void* dst[2] = {ws + wl.k, ws + wl.v};
    for (int g = 0; g < 2; ++g) {
      if (rocblas_gemm_ex(bh, rocblas_operation_transpose, rocblas_operation_none, N, M, kR, &alpha, wts[g],
                          rocblas_datatype_bf16_r, kR, p.lat, rocblas_datatype_bf16_r, kR, &beta, dst[g],
                          rocblas_datatype_bf16_r, N, dst[g], rocblas_datatype_bf16_r, N, rocblas_datatype_f32_r,
                          rocblas_gemm_algo_standard, 0, 0) != rocblas_status_success)
        return MLA_ERR_LAUNCH;
    }
    if ((st = launch_status(mla::launch_mha(p, s)))) return st;
  }
  return MLA_OK;
}

}  // extern "C"
