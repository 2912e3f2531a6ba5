// Per-head absorb / un-absorb batched GEMMs on the matrix cores (gfx950).
//
// Absorb ("MLA in full detail", Step 2; M5.8 0x04 einsum bhqn,hnc->bhqc):
//     q_lat[m,h,c] = sum_{n<128} q_nope[m,h,n] * W_UK[h,n,c]        (m = b*T + t)
// Un-absorb ("MLA in full detail", Step 4; M5.8 0x04 einsum bhqc,hvc->bhqv):
//     out[m,h,v]   = sum_{c<512} latent[m,h,c] * W_UV[h,v,c]
//
// Both are weight-bandwidth bound at decode batch sizes (each head's 128 KB
// weight is used by only B*T query rows), so each workgroup streams a disjoint
// slice of one head's weight exactly once and every query row is a cheap L2 hit.
// Products are computed transposed (D^T = W^T q^T and W_UV lat^T) so that the
// MFMA accumulator layout gives each lane four consecutive output columns of
// one row, stored as one 8- or 16-byte write.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace mla {

// ---------------- absorb ----------------
// Workgroup = (head h, 128-column block of c).  W_UK[h, :, cblk] (128 x 128 bf16)
// is staged in LDS with a padded row stride and read transposed
// (ds_read_b64_tr_b16) as the A operand W^T[32 c x 16 n]; wave w owns columns
// [32w, 32w+32) of the block.  B operand q^T[16 n x 32 m] comes from global.
// Every load of a chunk of 64 query rows is issued before the first wait (the
// kernel is a few memory round trips long, so latency is what it costs): the
// weight slice, then the query rows, whose indices are clamped to M-1 so the
// loads need no branch; columns of D^T past M are computed and never stored.
constexpr int kAbsStride = 144;  // bf16 elements per staged W row (128 + 16 pad)

__global__ __launch_bounds__(256) void absorb_kernel(AbsorbParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t wt[kDN * kAbsStride];
  const int w = wave_id(), l = lane_id();
  const int h = blockIdx.x >> 2;
  const int cblk = blockIdx.x & 3;
  const int H = p.H, M = p.M;
  // W_UK[h][n][cblk*128 .. +128]: 2048 chunks of 8 elements, 8 per thread
  const uint16_t* wsrc = p.w_uk + (size_t)h * kDN * kR + cblk * 128;
  u32x4 wv[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int id = threadIdx.x + 256 * k;
    wv[k] = *(const u32x4*)(wsrc + (size_t)(id >> 4) * kR + 8 * (id & 15));
  }
  // query rows of the first chunk: q^T operand of k-step ks for row m = lane & 31
  bf16x8 bq[2][8];
  auto load_q = [&](int m0) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int m = min(m0 + 32 * mb + (l & 31), M - 1);
      const uint16_t* qsrc = p.q_nope + ((size_t)m * H + h) * kDN + 8 * (l >> 5);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) bq[mb][ks] = *(const bf16x8*)(qsrc + 16 * ks);
    }
  };
  load_q(0);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int id = threadIdx.x + 256 * k;
    *(u32x4*)&wt[(id >> 4) * kAbsStride + 8 * (id & 15)] = wv[k];
  }
  __syncthreads();
  // A operands for the 8 k-steps: lane gets column c = 32w + (l & 31), rows
  // n = 16ks + 8(l>>5) + 4r + e (two transposing reads per k-step)
  bf16x8 A[8];
  {
    const int g = l >> 4, j = l & 15;
    const uint32_t base = lds_addr_of(wt);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      s16x4 x[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int n = 16 * ks + 8 * (g >> 1) + 4 * r + (j >> 2);
        const int c = 32 * w + 16 * (g & 1) + 4 * (j & 3);
        x[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(uintptr_t)(base + (n * kAbsStride + c) * 2));
      }
      A[ks] = join8(x[0], x[1]);
    }
  }
  for (int m0 = 0; m0 < M; m0 += 64) {
    f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[ks], bq[mb][ks], acc[mb], 0, 0, 0);
    if (m0 + 64 < M) load_q(m0 + 64);
    // D^T lane layout: row m = m0 + 32mb + (l & 31), columns 32w + 8q4 + 4(l>>5) + e
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int m = m0 + 32 * mb + (l & 31);
      if (m < M) {
        uint16_t* dst = p.q_lat + ((size_t)m * H + h) * kR + cblk * 128 + 32 * w + 4 * (l >> 5);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 v = {acc[mb][4 * q4], acc[mb][4 * q4 + 1], acc[mb][4 * q4 + 2], acc[mb][4 * q4 + 3]};
          *(u32x2*)(dst + 8 * q4) = cvt_bf16x4(v);
        }
      }
    }
  }
}

hipError_t launch_absorb(const AbsorbParams& prm, hipStream_t st) {
  if (prm.M == 0) return hipSuccess;
  hipLaunchKernelGGL(absorb_kernel, dim3(prm.H * 4), dim3(256), 0, st, prm);
  return hipGetLastError();
}

// ---------------- un-absorb ----------------
// Workgroup = (head h, 32-row block of v).  Wave w contracts c in
// [128w, 128w+128): A = W_UV[h][32 v x 16 c] and B = lat^T[16 c x 32 m] both
// come straight from global memory (16 contiguous bytes per lane); the four
// partial sums are added through LDS.  As in the absorb kernel, all loads of a
// 64-row chunk are issued before the first wait, with row indices clamped.
template <bool LAT_F32>
__global__ __launch_bounds__(256) void unabsorb_kernel(UnabsorbParams p) {
  __shared__ __attribute__((aligned(16))) float red[4][64 * 32];
  const int w = wave_id(), l = lane_id();
  const int h = blockIdx.x >> 2;
  const int vblk = blockIdx.x & 3;
  const int H = p.H, M = p.M;
  const int v = 32 * vblk + (l & 31);
  bf16x8 A[8];
  {
    const uint16_t* wsrc = p.w_uv + ((size_t)h * kDV + v) * kR + 128 * w + 8 * (l >> 5);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) A[ks] = *(const bf16x8*)(wsrc + 16 * ks);
  }
  // latent^T operands of a 64-row chunk (fp32 latent: two 16-byte loads per operand)
  typedef typename std::conditional<LAT_F32, f32x4, bf16x8>::type raw_t;
  raw_t raw[2][8][LAT_F32 ? 2 : 1];
  auto load_lat = [&](int m0) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int m = min(m0 + 32 * mb + (l & 31), M - 1);
      const size_t row = ((size_t)m * H + h) * kR + 128 * w + 8 * (l >> 5);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        if constexpr (LAT_F32) {
          const float* src = (const float*)p.latent + row + 16 * ks;
          raw[mb][ks][0] = *(const f32x4*)src;
          raw[mb][ks][LAT_F32 ? 1 : 0] = *(const f32x4*)(src + 4);
        } else {
          raw[mb][ks][0] = *(const bf16x8*)((const uint16_t*)p.latent + row + 16 * ks);
        }
      }
    }
  };
  load_lat(0);
  for (int m0 = 0; m0 < M; m0 += 64) {
    f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        bf16x8 bl;
        if constexpr (LAT_F32) bl = pack8(raw[mb][ks][0], raw[mb][ks][LAT_F32 ? 1 : 0]);
        else bl = raw[mb][ks][0];
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[ks], bl, acc[mb], 0, 0, 0);
      }
    }
    if (m0 + 64 < M) load_lat(m0 + 64);
    // D^T lane layout: row m = 32mb + (l & 31), column v = 8(r>>2) + 4(l>>5) + (r&3)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 s = {acc[mb][4 * q4], acc[mb][4 * q4 + 1], acc[mb][4 * q4 + 2], acc[mb][4 * q4 + 3]};
        *(f32x4*)&red[w][(32 * mb + (l & 31)) * 32 + 8 * q4 + 4 * (l >> 5)] = s;
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int id = threadIdx.x + 256 * k;  // (mloc, 4-column group)
      const int mloc = id >> 3, vq = id & 7;
      const int m = m0 + mloc;
      if (m < M) {
        const f32x4 s = *(const f32x4*)&red[0][mloc * 32 + 4 * vq] + *(const f32x4*)&red[1][mloc * 32 + 4 * vq] +
                        *(const f32x4*)&red[2][mloc * 32 + 4 * vq] + *(const f32x4*)&red[3][mloc * 32 + 4 * vq];
        *(f32x4*)(p.out + ((size_t)m * H + h) * kDV + 32 * vblk + 4 * vq) = s;
      }
    }
    __syncthreads();
  }
}

hipError_t launch_unabsorb(const UnabsorbParams& prm, bool latent_f32, hipStream_t st) {
  if (prm.M == 0) return hipSuccess;
  if (latent_f32)
    hipLaunchKernelGGL(unabsorb_kernel<true>, dim3(prm.H * 4), dim3(256), 0, st, prm);
  else
    hipLaunchKernelGGL(unabsorb_kernel<false>, dim3(prm.H * 4), dim3(256), 0, st, prm);
  return hipGetLastError();
}

}  // namespace mla
