// Merge of split-KV partials and the un-absorb in one launch (gfx950).
//
// For every query row m (= b*T + t) and head h:
//     lat[m,h,:] = sum_k w_k o_k / sum_k w_k,   w_k = exp(lse_k - max_k lse_k)
//                        (M5.8 0x0C, the exact merge; mlxcel Stage 2 merge contract)
//     out[m,h,v] = sum_c bf16(lat[m,h,c]) * W_UV[h,v,c]
//                        ("MLA in full detail", Step 4: W_UV folded into the output)
// The arithmetic of the merge kernel with a bf16 latent followed by the
// un-absorb, without the merged latent's round trip through memory and without
// the launch between the two.
//
// Workgroup = (head h, 32-row blocks j, j + G, j + 2G, ... of the M query
// rows).  W_UV[h] (128 rows v of 1 KB) goes to LDS once per workgroup through
// direct-to-LDS loads, one row per instruction, and stays there for every block
// the workgroup takes.  For each block, wave w merges rows w, w + 4, ..., w + 28:
// the 64 lanes hold one row's 512 columns, 8 each; the row's lse values (one
// split per lane) and, for up to four splits, the partial rows are requested
// together before any arithmetic, so every load of the block is in flight at
// once.  The merged rows, rounded to bf16, go to a 32 KB LDS block; then wave w
// computes the 32 x 32 tile out^T[v = 32w .. 32w+31][32 rows] with 32 MFMAs
// (K = 512), A = W_UV rows and B = merged rows, both read from LDS.
//
// LDS (160 KB, one workgroup per CU): both blocks are row-major with 1 KB rows
// and 16-byte chunk c of row r stored at chunk c ^ (r & 15), so the operand
// reads (32 rows, one chunk each) are free of bank conflicts.  With H a
// multiple of 8, the G workgroups of a head run on one XCD (workgroup g runs
// on XCD g % 8) and W_UV[h] is fetched from HBM once for them.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

namespace {

constexpr int kMuRows = kMergeUnabsorbRows;   // query rows per block
constexpr int kMuFast = 4;    // splits per row loaded before the arithmetic

__device__ __forceinline__ uint32_t mu_off(int r, int c) { return r * 1024 + 16 * (c ^ (r & 15)); }

__device__ __forceinline__ void bf16x8_to_f32(u32x4 u, f32x4& lo, f32x4& hi) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    lo[2 * i] = __builtin_bit_cast(float, u[i] << 16);
    lo[2 * i + 1] = __builtin_bit_cast(float, u[i] & 0xFFFF0000u);
    hi[2 * i] = __builtin_bit_cast(float, u[2 + i] << 16);
    hi[2 * i + 1] = __builtin_bit_cast(float, u[2 + i] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ float mu_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float mu_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
// Value of lane l ^ 1 / l ^ 2 within each quad of lanes (DPP quad permutes:
// no LDS round trip).
__device__ __forceinline__ float quad_xor1(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_xor2(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_value(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

}  // namespace

template <bool PART_F32>
__global__ __launch_bounds__(256, 1) void merge_unabsorb_kernel(MergeUnabsorbParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t wlds[kDV * 1024];       // W_UV[h]
  __shared__ __attribute__((aligned(16))) uint8_t mlds[kMuRows * 1024];   // merged rows, bf16
  constexpr float kLog2e = 1.4426950408889634f;
  const int w = wave_id(), l = lane_id();
  const int H = p.H, T = p.T, TH = T * H, M = p.M, G = p.groups;
  const int nmb = (M + kMuRows - 1) / kMuRows;
  int h, j;
  {
    const int g = blockIdx.x;
    if ((H & 7) == 0) {
      const int k = g >> 3;
      h = (g & 7) + 8 * (k / G);
      j = k - (k / G) * G;
    } else {
      h = g / G;
      j = g - h * G;
    }
  }
  const uint32_t w_lds = lds_addr_of(wlds), m_lds = lds_addr_of(mlds);

  // Rows r = w + 4k (k < 8) of block mb, merged by this wave: their split
  // ranges, then their lse values (lane 4k + u: split u of row k) and up to
  // four partial rows each, all in flight together.  Rows past M (the last
  // block's tail) take no split and merge to zero.  The loads are straight-line
  // code: a row without splits reads W_UV[h] in place of partials (every
  // address stays valid; with all its lse values -inf the row never uses what
  // it read), so the compiler's waits in the merge below count these loads
  // exactly instead of draining everything at a branch join.
  int gr[8], k0[8], ns[8];
  u32x4 raw[8][kMuFast];
  float xq;   // lse of split (l & 3) of row (l >> 2) & 7 (valid where that split exists)
  int nsq;    // splits of row (l >> 2) & 7
  int nsmax;  // the most splits of any of the 8 rows
  auto issue_block = [&](int mb) __attribute__((always_inline)) {
    // split ranges by scalar loads (the table is read-only here; through the
    // constant address space the loads are scalar and wait on their own counter)
    typedef const __attribute__((address_space(4))) int32_t cint;
    const cint* ind = (const cint*)(uintptr_t)p.split_indptr;
    // (all sixteen loads are issued before any of them is used)
    int bk[8], k1[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int mc = min(mb * kMuRows + w + 4 * k, M - 1);
      bk[k] = mc / T;
      gr[k] = (mc - bk[k] * T) * H + h;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      k0[k] = ind[bk[k]];
      k1[k] = ind[bk[k] + 1];
    }
    int e = 0;   // lane 2k: first split row of row k, lane 2k + 1: one past its last
                 // (of the clamped row for rows past M)
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      ns[k] = mb * kMuRows + w + 4 * k < M ? k1[k] - k0[k] : 0;
      e = l == 2 * k ? k0[k] : e;
      e = l == 2 * k + 1 ? k1[k] : e;
    }
    nsmax = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) nsmax = max(nsmax, ns[k]);
    if (nsmax > kMuFast) return;   // the rows are merged by the general loop below
    // the lse values first: the merge needs them before any partial row
    {
      // this lane's row kq: its split range from lanes 2kq and 2kq + 1 of e
      const int kq = (l >> 2) & 7, uq = l & 3;
      const int k0q = __builtin_amdgcn_ds_bpermute(8 * kq, e);
      const int e1q = __builtin_amdgcn_ds_bpermute(8 * kq + 4, e);
      const int mq = mb * kMuRows + w + 4 * kq;
      const int mcq = min(mq, M - 1);
      const int grq = (mcq - (mcq / T) * T) * H + h;
      nsq = mq < M ? e1q - k0q : 0;
      const float* qsrc = nsq > 0 ? p.part_lse + (size_t)(k0q + min(uq, nsq - 1)) * TH + grq
                                  : (const float*)(p.w_uv + (size_t)h * kDV * kR) + l;
      xq = *qsrc;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const bool has = ns[k] > 0;
      const int n = has ? min(ns[k], kMuFast) : 1;
#pragma unroll
      for (int u = 0; u < kMuFast; ++u) {
        // splits past the row's last one re-read that one (weight 0 below)
        const size_t s = (size_t)(k0[k] + min(u, n - 1));
        const size_t e8 = (s * TH + gr[k]) * kR + 8 * l;
        const u32x4* src = has ? (PART_F32 ? (const u32x4*)((const float*)p.part_out + e8)
                                           : (const u32x4*)((const uint16_t*)p.part_out + e8))
                               : (const u32x4*)(p.w_uv + (size_t)h * kDV * kR) + l;
        raw[k][u] = *src;
      }
    }
  };

  // W_UV[h] -> LDS: wave w brings rows v = w + 4i; lane l fetches logical chunk
  // l ^ (v & 15) of the row, which lands in physical chunk l
  {
    const uint8_t* wsrc = (const uint8_t*)(p.w_uv + (size_t)h * kDV * kR);
#pragma unroll 8
    for (int i = 0; i < kDV / 4; ++i) {
      const int v = w + 4 * i;
      dma16s((uint32_t)(v * 1024 + 16 * (l ^ (v & 15))), wsrc, w_lds + v * 1024);
    }
  }

  // Merge of block mb (its loads issued by issue_block) into the LDS block.
  auto merge_block = [&](int mb) __attribute__((always_inline)) {
    if (nsmax <= kMuFast) {
      // Every row has at most four splits: lane 4k + u (k < 8) holds split u of
      // row k, and one quad reduction serves all eight rows.  (The sum takes
      // lane pairs at distance 2, then 1: the order of the last two steps of
      // the merge kernel's 64-lane butterfly, whose other steps add zeros, so
      // weights and lse match it bit for bit.)
      const int kq = (l >> 2) & 7, uq = l & 3;
      const float x = uq < nsq ? xq : -INFINITY;
      float mq = fmaxf(x, quad_xor2(x));
      mq = fmaxf(mq, quad_xor1(mq));
      const float wq = (x == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((x - mq) * kLog2e);
      float sq = wq + quad_xor2(wq);
      sq = sq + quad_xor1(sq);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int r = w + 4 * k;
        const float Mx = lane_value(mq, 4 * k);
        const float wsum = lane_value(sq, 4 * k);
        f32x4 a0 = {}, a1 = {};
        if (Mx != -INFINITY) {
#pragma unroll
          for (int u = 0; u < kMuFast; ++u) {
            const float wk = u < ns[k] ? lane_value(wq, 4 * k + u) : 0.f;
            f32x4 lo, hi;
            if constexpr (PART_F32) {
              // (the high halves were not loaded with the block: fp32 partials
              // would need twice the registers)
              const size_t s = (size_t)(k0[k] + min(u, ns[k] - 1));
              lo = __builtin_bit_cast(f32x4, raw[k][u]);
              hi = *(const f32x4*)((const float*)p.part_out + (s * TH + gr[k]) * kR + 8 * l + 4);
            } else {
              bf16x8_to_f32(raw[k][u], lo, hi);
            }
            a0 += wk * lo;
            a1 += wk * hi;
          }
        }
        const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
        const u32x2 lo = cvt_bf16x4(a0 * inv), hi = cvt_bf16x4(a1 * inv);
        *(__attribute__((address_space(3))) u32x4*)(uintptr_t)(m_lds + mu_off(r, l)) =
            u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
      // lse of row k from lane 4k (lanes 32..63 repeat lanes 0..31)
      const int mq_row = mb * kMuRows + w + 4 * kq;
      if (p.lse && l < 32 && uq == 0 && mq_row < M)
        p.lse[(size_t)mq_row * H + h] = sq > 0.f ? mq + __builtin_amdgcn_logf(sq) * 0.69314718055994530942f
                                                 : -INFINITY;
    } else {
      // Some row has more than four splits: row by row, the lse values 64 at a
      // time (each split's weight in its lane), partial rows eight in flight
      // (indices past the last split are clamped and carry weight 0).
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int r = w + 4 * k;
        const int m = mb * kMuRows + r;
        float Mx = -INFINITY;
        for (int s = l; s < ns[k]; s += 64) Mx = fmaxf(Mx, p.part_lse[(size_t)(k0[k] + s) * TH + gr[k]]);
        Mx = mu_max(Mx);
        float wsum = 0.f;
        f32x4 a0 = {}, a1 = {};
        if (Mx != -INFINITY) {
          for (int sc = 0; sc < ns[k]; sc += 64) {
            const float x = sc + l < ns[k] ? p.part_lse[(size_t)(k0[k] + sc + l) * TH + gr[k]] : -INFINITY;
            const float wl = (x == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((x - Mx) * kLog2e);
            wsum += mu_sum(wl);
            const int n = min(64, ns[k] - sc);
            for (int u0 = 0; u0 < n; u0 += 8) {
              f32x4 lo[8], hi[8];
#pragma unroll
              for (int u = 0; u < 8; ++u) {
                const size_t s = (size_t)(k0[k] + sc + min(u0 + u, n - 1));
                if constexpr (PART_F32) {
                  const float* src = (const float*)p.part_out + (s * TH + gr[k]) * kR + 8 * l;
                  lo[u] = *(const f32x4*)src;
                  hi[u] = *(const f32x4*)(src + 4);
                } else {
                  bf16x8_to_f32(*(const u32x4*)((const uint16_t*)p.part_out + (s * TH + gr[k]) * kR + 8 * l),
                                lo[u], hi[u]);
                }
              }
#pragma unroll
              for (int u = 0; u < 8; ++u) {
                const float wk = u0 + u < n ? lane_value(wl, u0 + u) : 0.f;
                a0 += wk * lo[u];
                a1 += wk * hi[u];
              }
            }
          }
        }
        const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
        const u32x2 lo = cvt_bf16x4(a0 * inv), hi = cvt_bf16x4(a1 * inv);
        *(__attribute__((address_space(3))) u32x4*)(uintptr_t)(m_lds + mu_off(r, l)) =
            u32x4{lo[0], lo[1], hi[0], hi[1]};
        if (l == 0 && p.lse && m < M)
          p.lse[(size_t)m * H + h] = wsum > 0.f ? Mx + __builtin_amdgcn_logf(wsum) * 0.69314718055994530942f
                                                : -INFINITY;
      }
    }

  };
  // Un-absorb of block mb from the LDS blocks.
  auto unabsorb_block = [&](int mb) __attribute__((always_inline)) {
    // ---- un-absorb of the block: wave w computes out^T[32w .. 32w+31][32 rows]
    wait_vm0();        // this wave's W_UV rows have landed (and every partial it read)
    __syncthreads();   // every wave's W_UV rows and merged rows are in LDS
    f32x16 acc = {};
    {
      // operands read four MFMAs ahead of their use
      const int v = 32 * w + (l & 31), row = l & 31;
      auto opnd = [&](uint32_t base, int r, int ks) {
        return *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)(base + mu_off(r, 2 * ks + (l >> 5)));
      };
      constexpr int kAhead = 4;
      bf16x8 a[kAhead], bm[kAhead];
#pragma unroll
      for (int i = 0; i < kAhead; ++i) {
        a[i] = opnd(w_lds, v, i);
        bm[i] = opnd(m_lds, row, i);
      }
#pragma unroll
      for (int ks = 0; ks < kR / 16; ++ks) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks % kAhead], bm[ks % kAhead], acc, 0, 0, 0);
        if (ks + kAhead < kR / 16) {
          a[ks % kAhead] = opnd(w_lds, v, ks + kAhead);
          bm[ks % kAhead] = opnd(m_lds, row, ks + kAhead);
        }
      }
    }
    // D^T lane layout: query row l & 31 of the block, v = 32w + 8q + 4(l >> 5) + e
    const int m = mb * kMuRows + (l & 31);
    if (m < M) {
      float* dst = p.out + ((size_t)m * H + h) * kDV + 32 * w + 4 * (l >> 5);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *(f32x4*)(dst + 8 * q) = f32x4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
    }
    __syncthreads();   // every wave has read the merged block before the next one is written
  };

  // The W_UV rows are requested first, at the start of the kernel.  The direct-
  // to-LDS loads are inline assembly the compiler does not count; a wait it
  // places for one of its own later loads also waits for them (the counter
  // drains in issue order), which the merge of the first block can afford:
  // W_UV[h] was requested before its partial rows.  The first block is taken
  // apart from the loop over the others so that its merge is straight-line
  // code whose waits count the block's loads exactly (at the loop's head they
  // would be merged with the other path's and drain everything).
  if (j < nmb) {
    issue_block(j);
    merge_block(j);
    unabsorb_block(j);
  }
  for (int mb = j + G; mb < nmb; mb += G) {
    issue_block(mb);
    merge_block(mb);
    unabsorb_block(mb);
  }
  wait_vm0();          // a workgroup without a block still drains its W_UV loads
}

hipError_t launch_merge_unabsorb(const MergeUnabsorbParams& prm, bool part_f32, hipStream_t st) {
  const long long n = (long long)prm.H * prm.groups;
  if (prm.M == 0 || n == 0) return hipSuccess;
  if (part_f32)
    hipLaunchKernelGGL(merge_unabsorb_kernel<true>, dim3((unsigned)n), dim3(256), 0, st, prm);
  else
    hipLaunchKernelGGL(merge_unabsorb_kernel<false>, dim3((unsigned)n), dim3(256), 0, st, prm);
  return hipGetLastError();
}

}  // namespace mla
