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
// [32w, 32w+32) of the block.  The B operand q^T[16 n x 32 m] and the output
// both go through an LDS block of 64 rows x 256 B, so that every global access
// is a whole 256-byte row segment: in the MFMA operand layout a load or store
// instruction touches 32 rows with 16-32 bytes each, and at this kernel's size
// the L2 request rate of those scattered pieces, not the weight stream, set the
// time.  Query row indices are clamped to M-1 (rows past M are computed and
// never stored), so no load needs a branch.
//
// Row-block layout in LDS (64 rows, 16 chunks of 16 B each): chunk c of row r
// sits at chunk c ^ (r & 15), so the operand reads (16 rows, one chunk) and the
// row-segment accesses (one row, 16 chunks) are both conflict-free.  The
// output uses the same layout with the two 8-byte halves of a chunk swapped
// when bit 4 of r is set (conflict-free 8-byte writes from the accumulator).
constexpr int kAbsStride = 144;  // bf16 elements per staged W row (128 + 16 pad)

__device__ __forceinline__ int rb_off(int r, int c) { return r * 128 + 8 * (c ^ (r & 15)); }

// (head, quarter) of workgroup g.  Workgroup g runs on XCD g % 8; with H a
// multiple of 8 the four quarters of a head go to one XCD, so the head's query
// or latent rows are fetched into that XCD's L2 once and shared.
__device__ __forceinline__ void head_quarter(int g, int H, int& h, int& q) {
  if ((H & 7) == 0) {
    const int k = g >> 3;
    h = (g & 7) + 8 * (k >> 2);
    q = k & 3;
  } else {
    h = g >> 2;
    q = g & 3;
  }
}

__global__ __launch_bounds__(256) void absorb_kernel(AbsorbParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t wt[kDN * kAbsStride];
  __shared__ __attribute__((aligned(16))) uint16_t blk[64 * 128];
  const int w = wave_id(), l = lane_id();
  const int H = p.H, M = p.M;
  int h, cblk;
  head_quarter(blockIdx.x, H, h, cblk);
  // W_UK[h][n][cblk*128 .. +128]: 2048 chunks of 8 elements, 8 per thread
  const uint16_t* wsrc = p.w_uk + (size_t)h * kDN * kR + cblk * 128;
  u32x4 wv[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int id = threadIdx.x + 256 * k;
    wv[k] = *(const u32x4*)(wsrc + (size_t)(id >> 4) * kR + 8 * (id & 15));
  }
  // query rows m0 .. m0+63 as whole 256-byte rows: 4 chunks per thread
  u32x4 qv[4];
  auto load_q = [&](int m0) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int id = threadIdx.x + 256 * k;
      const int m = min(m0 + (id >> 4), M - 1);
      qv[k] = *(const u32x4*)(p.q_nope + ((size_t)m * H + h) * kDN + 8 * (id & 15));
    }
  };
  auto stage_q = [&]() {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int id = threadIdx.x + 256 * k;
      *(u32x4*)&blk[rb_off(id >> 4, id & 15)] = qv[k];
    }
  };
  load_q(0);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int id = threadIdx.x + 256 * k;
    *(u32x4*)&wt[(id >> 4) * kAbsStride + 8 * (id & 15)] = wv[k];
  }
  stage_q();
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
    for (int mb = 0; mb < 2; ++mb) {
      const int r = 32 * mb + (l & 31);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 bq = *(const bf16x8*)&blk[rb_off(r, 2 * ks + (l >> 5))];
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[ks], bq, acc[mb], 0, 0, 0);
      }
    }
    if (m0 + 64 < M) load_q(m0 + 64);
    __syncthreads();  // every wave has read the query block
    // D^T lane layout: row 32mb + (l & 31), columns 32w + 8q4 + 4(l>>5) + e
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int r = 32 * mb + (l & 31);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 v = {acc[mb][4 * q4], acc[mb][4 * q4 + 1], acc[mb][4 * q4 + 2], acc[mb][4 * q4 + 3]};
        const int hh = (l >> 5) ^ ((r >> 4) & 1);
        *(u32x2*)&blk[rb_off(r, 4 * w + q4) + 4 * hh] = cvt_bf16x4(v);
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int id = threadIdx.x + 256 * k;  // (row, 16-byte chunk)
      const int r = id >> 4, c = id & 15;
      u32x4 v = *(const u32x4*)&blk[rb_off(r, c)];
      if ((r >> 4) & 1) v = u32x4{v[2], v[3], v[0], v[1]};
      if (m0 + r < M) *(u32x4*)(p.q_lat + ((size_t)(m0 + r) * H + h) * kR + cblk * 128 + 8 * c) = v;
    }
    if (m0 + 64 < M) {
      __syncthreads();  // the output block has been read
      stage_q();
      __syncthreads();
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
// [128w, 128w+128): A = W_UV[h][32 v x 16 c] and B = lat^T[16 c x 32 m]; the
// four partial sums are added through LDS.  As in the absorb kernel, the rows
// are fetched as whole 256-byte segments (each wave's slice of 32 weight rows,
// then of 64 latent rows) and rearranged into operand layout through the
// wave's own LDS block, which needs no barrier.  An fp32 latent (twice the
// bytes) is read directly in operand layout.  Row indices are clamped to M-1.
template <bool LAT_F32>
__global__ __launch_bounds__(256) void unabsorb_kernel(UnabsorbParams p) {
  // per wave: 64 rows x 256 B (row-block layout); reused for the cross-wave sum
  __shared__ __attribute__((aligned(16))) uint16_t blk[4][64 * 128];
  float* const red = (float*)&blk[0][0];  // [4][64 * 32] floats, after the MFMAs
  const int w = wave_id(), l = lane_id();
  const int H = p.H, M = p.M;
  int h, vblk;
  head_quarter(blockIdx.x, H, h, vblk);
  uint16_t* const mine = blk[w];
  // this wave's weight slice: rows v = 32 vblk + r (r < 32), columns 128w .. +128
  u32x4 wv[8];
  {
    const uint16_t* wsrc = p.w_uv + ((size_t)h * kDV + 32 * vblk) * kR + 128 * w;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int id = l + 64 * k;  // (row, chunk): 4 rows per instruction
      wv[k] = *(const u32x4*)(wsrc + (size_t)(id >> 4) * kR + 8 * (id & 15));
    }
  }
  // latent rows m0 .. m0+63, columns 128w .. +128 (bf16 path)
  u32x4 lv[16];
  auto load_lat = [&](int m0) {
    if constexpr (!LAT_F32) {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int id = l + 64 * k;
        const int m = min(m0 + (id >> 4), M - 1);
        lv[k] = *(const u32x4*)((const uint16_t*)p.latent + ((size_t)m * H + h) * kR + 128 * w + 8 * (id & 15));
      }
    }
  };
  load_lat(0);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int id = l + 64 * k;
    *(u32x4*)&mine[rb_off(id >> 4, id & 15)] = wv[k];
  }
  bf16x8 A[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) A[ks] = *(const bf16x8*)&mine[rb_off(l & 31, 2 * ks + (l >> 5))];
  for (int m0 = 0; m0 < M; m0 += 64) {
    if constexpr (!LAT_F32) {
      // (LDS operations of one wave complete in order: the weight reads above
      // finish before these writes land)
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int id = l + 64 * k;
        *(u32x4*)&mine[rb_off(id >> 4, id & 15)] = lv[k];
      }
    }
    f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int r = 32 * mb + (l & 31);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        bf16x8 bl;
        if constexpr (LAT_F32) {
          const int m = min(m0 + r, M - 1);
          const float* src = (const float*)p.latent + ((size_t)m * H + h) * kR + 128 * w + 16 * ks + 8 * (l >> 5);
          bl = pack8(*(const f32x4*)src, *(const f32x4*)(src + 4));
        } else {
          bl = *(const bf16x8*)&mine[rb_off(r, 2 * ks + (l >> 5))];
        }
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[ks], bl, acc[mb], 0, 0, 0);
      }
    }
    if (m0 + 64 < M) load_lat(m0 + 64);
    __syncthreads();  // every wave is done with its latent block (red aliases it)
    // D^T lane layout: row m = 32mb + (l & 31), column v = 8(r>>2) + 4(l>>5) + (r&3)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 sv = {acc[mb][4 * q4], acc[mb][4 * q4 + 1], acc[mb][4 * q4 + 2], acc[mb][4 * q4 + 3]};
        *(f32x4*)&red[w * 2048 + (32 * mb + (l & 31)) * 32 + 8 * q4 + 4 * (l >> 5)] = sv;
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int id = threadIdx.x + 256 * k;  // (mloc, 4-column group)
      const int mloc = id >> 3, vq = id & 7;
      const int m = m0 + mloc;
      if (m < M) {
        const int o = mloc * 32 + 4 * vq;
        const f32x4 sv = *(const f32x4*)&red[o] + *(const f32x4*)&red[2048 + o] +
                         *(const f32x4*)&red[4096 + o] + *(const f32x4*)&red[6144 + o];
        *(f32x4*)(p.out + ((size_t)m * H + h) * kDV + 32 * vblk + 4 * vq) = sv;
      }
    }
    __syncthreads();  // the sums have been read before the next block is staged
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
