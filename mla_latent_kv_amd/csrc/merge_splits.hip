// Exact log-sum-exp merge of split-KV partial states (gfx950).
//
// Each partial k of a query row carries o_k (its output already divided by its
// own softmax denominator) and lse_k (natural log).  The merged row is
//     M = max_k lse_k,  w_k = exp(lse_k - M),
//     out = sum_k w_k o_k / sum_k w_k,   lse = M + log(sum_k w_k),
// which equals attention over the union of the chunks (M5.8 0x0C: the exact
// merge of (m_r, l_r, o_r); mlxcel Stage 2 merge contract with normalised
// partials).  Chunks with lse = -inf (no visible key) carry no weight.
//
// One workgroup per query row: wave w folds the partials k0 + w, k0 + w + 4, ...
// into its own running (max, weight sum, 512-wide sum) -- 8 columns per lane --
// and the four wave states are combined through LDS.  HBM-bound: every partial
// byte is read once.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

template <bool F32>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  __shared__ float m_s[4], w_s[4];
  __shared__ __attribute__((aligned(16))) float o_s[4][kR];
  const int w = wave_id(), l = lane_id();
  const long long row = blockIdx.x;  // (b, gr)
  const int b = (int)(row / p.TH);
  const int gr = (int)(row - (long long)b * p.TH);
  const int TH = p.TH;
  const int k0 = p.split_indptr[b], k1 = p.split_indptr[b + 1];
  constexpr float kLog2e = 1.4426950408889634f;

  float M = -INFINITY;
  for (int k = k0 + w; k < k1; k += 4) M = fmaxf(M, p.part_lse[(size_t)k * TH + gr]);
  float wsum = 0.f;
  f32x4 a0 = {}, a1 = {};
  if (M != -INFINITY) {
#pragma unroll 4
    for (int k = k0 + w; k < k1; k += 4) {
      const float x = p.part_lse[(size_t)k * TH + gr];
      const float wk = (x == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((x - M) * kLog2e);
      const float* src = p.part_out + ((size_t)k * TH + gr) * kR + 8 * l;
      const f32x4 v0 = *(const f32x4*)src;
      const f32x4 v1 = *(const f32x4*)(src + 4);
      wsum += wk;
      a0 += wk * v0;
      a1 += wk * v1;
    }
  }
  if (l == 0) {
    m_s[w] = M;
    w_s[w] = wsum;
  }
  *(f32x4*)&o_s[w][8 * l] = a0;
  *(f32x4*)&o_s[w][8 * l + 4] = a1;
  __syncthreads();
  // combine the four wave states; every thread finishes 2 of the 512 columns
  float Mg = fmaxf(fmaxf(m_s[0], m_s[1]), fmaxf(m_s[2], m_s[3]));
  float sc[4], tot = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sc[i] = (m_s[i] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m_s[i] - Mg) * kLog2e);
    tot += sc[i] * w_s[i];
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  const int c = 2 * threadIdx.x;
  float o[2];
#pragma unroll
  for (int e = 0; e < 2; ++e)
    o[e] = (sc[0] * o_s[0][c + e] + sc[1] * o_s[1][c + e] + sc[2] * o_s[2][c + e] +
            sc[3] * o_s[3][c + e]) * inv;
  const size_t orow = (size_t)b * TH + gr;
  if constexpr (F32) {
    float* dst = (float*)p.out + orow * kR + c;
    dst[0] = o[0];
    dst[1] = o[1];
  } else {
    *(uint32_t*)((uint16_t*)p.out + orow * kR + c) = pack_bf16x2(o[0], o[1]);
  }
  if (threadIdx.x == 0 && p.lse) {
    p.lse[orow] = tot > 0.f ? Mg + __builtin_amdgcn_logf(tot) * 0.69314718055994530942f
                            : -INFINITY;
  }
}

hipError_t launch_merge(const MergeParams& prm, bool out_f32, hipStream_t st) {
  const long long rows = (long long)prm.B * prm.TH;
  if (rows == 0) return hipSuccess;
  if (out_f32)
    hipLaunchKernelGGL(merge_kernel<true>, dim3((unsigned)rows), dim3(256), 0, st, prm);
  else
    hipLaunchKernelGGL(merge_kernel<false>, dim3((unsigned)rows), dim3(256), 0, st, prm);
  return hipGetLastError();
}

}  // namespace mla
