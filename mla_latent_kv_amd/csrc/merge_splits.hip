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
// One wave per query row, 8 of the 512 columns per lane.  The row's lse values
// are loaded one per lane (64 splits at a time), their maximum and weights are
// formed with cross-lane reductions, and each split's weight is broadcast from
// its lane while the partial rows stream in, eight in flight per wave (indices
// past the row's last split are clamped and carry weight 0).  Partials are fp32
// or bf16, accumulation is fp32.  HBM-bound: every partial byte is read once.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

template <bool PART_F32>
__device__ __forceinline__ void load8(const void* base, size_t elem, f32x4& lo, f32x4& hi) {
  if constexpr (PART_F32) {
    const float* src = (const float*)base + elem;
    lo = *(const f32x4*)src;
    hi = *(const f32x4*)(src + 4);
  } else {
    const u32x4 u = *(const u32x4*)((const uint16_t*)base + elem);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      lo[2 * i] = __builtin_bit_cast(float, u[i] << 16);
      lo[2 * i + 1] = __builtin_bit_cast(float, u[i] & 0xFFFF0000u);
      hi[2 * i] = __builtin_bit_cast(float, u[2 + i] << 16);
      hi[2 * i + 1] = __builtin_bit_cast(float, u[2 + i] & 0xFFFF0000u);
    }
  }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <bool PART_F32, bool OUT_F32>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  const int w = wave_id(), l = lane_id();
  const long long row = (long long)blockIdx.x * 4 + w;  // (b, gr)
  const int TH = p.TH;
  if (row >= (long long)p.B * TH) return;
  const int b = (int)(row / TH);
  const int gr = (int)(row - (long long)b * TH);
  const int k0 = p.split_indptr[b], k1 = p.split_indptr[b + 1];
  constexpr float kLog2e = 1.4426950408889634f;
  const float* lse_col = p.part_lse + gr;

  float M = -INFINITY;
  for (int k = k0 + l; k < k1; k += 64) M = fmaxf(M, lse_col[(size_t)k * TH]);
  M = wave_max(M);
  float wsum = 0.f;
  f32x4 a0 = {}, a1 = {};
  if (M != -INFINITY) {
    for (int kc = k0; kc < k1; kc += 64) {
      // weight of split kc + l in lane l
      const int kl = kc + l;
      const float x = kl < k1 ? lse_col[(size_t)kl * TH] : -INFINITY;
      const float wl = (x == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((x - M) * kLog2e);
      wsum += wave_sum(wl);
      const int n = min(64, k1 - kc);
      for (int u0 = 0; u0 < n; u0 += 8) {
        f32x4 v[8][2];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int k = kc + min(u0 + u, n - 1);
          load8<PART_F32>(p.part_out, ((size_t)k * TH + gr) * kR + 8 * l, v[u][0], v[u][1]);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float wk = (u0 + u < n) ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                                   __builtin_bit_cast(int, wl), u0 + u))
                                        : 0.f;
          a0 += wk * v[u][0];
          a1 += wk * v[u][1];
        }
      }
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  a0 *= inv;
  a1 *= inv;
  const size_t orow = (size_t)row;
  if constexpr (OUT_F32) {
    float* dst = (float*)p.out + orow * kR + 8 * l;
    *(f32x4*)dst = a0;
    *(f32x4*)(dst + 4) = a1;
  } else {
    const u32x2 lo = cvt_bf16x4(a0), hi = cvt_bf16x4(a1);
    *(u32x4*)((uint16_t*)p.out + orow * kR + 8 * l) = u32x4{lo[0], lo[1], hi[0], hi[1]};
  }
  if (l == 0 && p.lse) {
    p.lse[orow] = wsum > 0.f ? M + __builtin_amdgcn_logf(wsum) * 0.69314718055994530942f : -INFINITY;
  }
}

template <bool PF, bool OF>
static void launch_merge_t(const MergeParams& prm, unsigned grid, hipStream_t st) {
  hipLaunchKernelGGL((merge_kernel<PF, OF>), dim3(grid), dim3(256), 0, st, prm);
}

hipError_t launch_merge(const MergeParams& prm, bool part_f32, bool out_f32, hipStream_t st) {
  const long long rows = (long long)prm.B * prm.TH;
  if (rows == 0) return hipSuccess;
  const unsigned grid = (unsigned)((rows + 3) / 4);
  if (part_f32) {
    if (out_f32) launch_merge_t<true, true>(prm, grid, st);
    else launch_merge_t<true, false>(prm, grid, st);
  } else {
    if (out_f32) launch_merge_t<false, true>(prm, grid, st);
    else launch_merge_t<false, false>(prm, grid, st);
  }
  return hipGetLastError();
}

}  // namespace mla
