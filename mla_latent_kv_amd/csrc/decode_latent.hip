// Absorbed MLA decode attention over a paged latent cache (gfx950).
//
// What is computed ("MLA in full detail", Step 3; M5.8 0x04 batched absorption
// trace): for every query row (t, h) of sequence b and every visible cached
// token j,
//     s = (q~[t,h,:] . c_j + q_pe[t,h,:] . kpe_j) * scale
//     out[t,h,:] = sum_j softmax_j(s) c_j            (512 wide, per head)
// where row j of the cache is [c_j (512) || kpe_j (64)], found through the
// block table (M5.8 0x05).  All heads share the one latent KV head, so every
// 1152-byte row is read from HBM once per workgroup and reused by all 128
// query rows: the score GEMM is [128 x 576] x [576 x tile] and the value GEMM
// is [128 x tile] x [tile x 512], both on the matrix cores in bf16 with fp32
// accumulation.  The softmax is accumulated over KV tiles against one
// reference maximum per row and normalised once at the end (M5.8 0x0A: tiles
// are never normalised independently).
//
// Workgroup layout (256 threads = 4 waves of 64, one workgroup per CU):
//  * KV tiles of 16 tokens (18 KB) stream HBM -> LDS with direct-to-LDS loads
//    into a ring of NB buffers, NB-1 tiles ahead of use.  Every wave issues a
//    quarter of each tile's 18 load instructions.
//  * Score phase: wave w owns query rows [32w, 32w+32) and computes
//    S^T[16 tok x 32 rows] with 16x16x32 MFMAs; the K operand is read from LDS
//    with ds_read_b128, the query lives in registers for the whole kernel.
//  * Softmax: log2 domain against a per-row reference m_ref (the max of the
//    row's first tile with a visible key), so exponentials are bounded by
//    2^kLazy; the fp32 accumulator is never rescaled.  If a later tile's max
//    exceeds m_ref by more than kLazy, m_ref is raised and the work unit is
//    replayed from its first tile (exact for any finite scores; not taken for
//    scores of ordinary magnitude).
//  * Probabilities (bf16) of all 128 rows are exchanged through LDS.
//  * Value phase: wave w owns latent columns [128w, 128w+128) of all 128 rows
//    (O^T accumulator 128 x 128 fp32 = 256 registers) and multiplies
//    V^T[32 cols x 16 tok] (transposing LDS reads) by P^T[16 tok x 32 rows]
//    with 32x32x16 MFMAs.  Splitting the value GEMM by columns rather than by
//    rows means each V element is read from LDS once per workgroup instead of
//    once per wave.
//
// Tile LDS layout (chunk-major): the 16-byte chunk c (c < 72) of tile row t is
// stored at chunk position 16c + (t ^ 4(c & 1)).  A K read (16 rows of one
// chunk) is then 256 contiguous bytes, a transposing V read (4 rows x 2
// adjacent chunks per 16 lanes) touches 32 distinct banks, and every address
// is one per-lane base plus an immediate offset.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

constexpr float kLazy = 64.0f;  // log2-domain growth of the max tolerated before a replay


template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Cross-lane pair exchange.  v_permlane16_swap exchanges the odd 16-lane rows of
// its first operand with the even rows of its second; with both operands
// holding v, lane l ends up with v of lanes l and l^16 (permlane32: l and l^32).
// Written as inline assembly: the builtin has been seen to compile to code that
// reads only one of the two results.  The swap reads its operands two wait
// states after a VALU write at the earliest, hence the s_nop.
__device__ __forceinline__ void xpair16(float v, float& a, float& b) {
  a = v;
  b = v;
  asm volatile("s_nop 2\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void xpair32(float v, float& a, float& b) {
  a = v;
  b = v;
  asm volatile("s_nop 2\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
// max / sum over the four lanes l, l^16, l^32, l^48
__device__ __forceinline__ float max4lanes(float v) {
  float a, b;
  xpair16(v, a, b);
  xpair32(fmaxf(a, b), a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float sum4lanes(float v) {
  float a, b;
  xpair16(v, a, b);
  xpair32(a + b, a, b);
  return a + b;
}

__device__ __forceinline__ bf16x8 lds_b128(uint32_t addr) {
  return *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)addr;
}
// Transposing LDS read: within each 16-lane group, lane i receives element i%4
// of the 8-byte rows read by lanes i/4, i/4+4, i/4+8, i/4+12 (in that order).
__device__ __forceinline__ s16x4 lds_tr16(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(uintptr_t)addr);
}

template <int NB, bool SPLIT, bool OUT_F32>
__global__ __launch_bounds__(256, 1) void decode_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t tiles[NB * kTileBytes];
  __shared__ __attribute__((aligned(16))) uint16_t pbuf[kRowsPerWG * kTile];
  __shared__ __attribute__((aligned(16))) float inv_s[kRowsPerWG];
  __shared__ __attribute__((aligned(16))) unsigned flag_s[4];

  const int w = wave_id();
  const int l = lane_id();
  const int wg = blockIdx.x;
  const int item = wg / p.n_rg;
  const int rg = wg - item * p.n_rg;

  int b, j0, j1, slot;
  if constexpr (SPLIT) {
    if (p.work) {  // automatic split counts: work list from the plan kernel
      if (item >= *p.n_items) return;
      const int32_t* wi = p.work + 4 * item;
      b = wi[0];
      j0 = wi[1];
      j1 = wi[2];
      slot = wi[3];
    } else {  // S uniform chunks of ceil(ceil(L/S)/P)*P tokens per sequence
      const int S = p.num_splits;
      b = item / S;
      const int s = item - b * S;
      const int Lb = p.seqlens[b];
      const int chunk = (((Lb + S - 1) / S + p.page_size - 1) / p.page_size) * p.page_size;
      j0 = min(s * chunk, Lb);
      j1 = min(j0 + chunk, Lb);
      slot = item;
      if (s == 0 && rg == 0 && threadIdx.x == 0) {
        p.split_indptr[b + 1] = (b + 1) * S;
        if (b == 0) p.split_indptr[0] = 0;
      }
    }
  } else {
    b = item;
    j0 = 0;
    j1 = p.seqlens[b];
    slot = b;
  }
  const int L = p.seqlens[b];
  const int T = p.T, H = p.H, TH = T * H;
  const int P = p.page_size;
  const int row0 = rg * kRowsPerWG;

  // ---- query rows of this wave (score phase) and their visible limits ----
  bf16x8 q[2][18];
  int lim[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int gr = row0 + 32 * w + 16 * nb + (l & 15);
    if (gr < TH) {
      const int t = gr / H;
      const int h = gr - t * H;
      lim[nb] = min(L - T + t + 1, j1);
      const uint16_t* ql = p.q_lat + ((size_t)(b * T + t) * H + h) * kR + 8 * (l >> 4);
      const uint16_t* qp = p.q_pe + ((size_t)(b * T + t) * H + h) * kDR + 8 * (l >> 4);
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) q[nb][ks] = *(const bf16x8*)(ql + 32 * ks);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) q[nb][16 + ks] = *(const bf16x8*)(qp + 32 * ks);
    } else {
      lim[nb] = j0;  // padded row: nothing visible
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) q[nb][ks] = bf16x8{};
    }
  }

  const int ntiles = (j1 - j0 + kTile - 1) / kTile;
  const uint32_t tiles_lds = lds_addr_of(tiles);
  const uint8_t* cache = (const uint8_t*)p.cache;
  const int32_t* bt_row = p.block_table + (size_t)b * p.max_blocks;

  // physical pages of logical pages [pg_base, pg_base + 64), one per lane
  int pg_base = j0 / P;
  int pg_vec = 0;
  {
    const int pg = pg_base + l;
    if (pg < p.max_blocks && pg * P < j1) pg_vec = bt_row[pg];
  }
  // q and the first page ids must be complete before any tile load is in flight:
  // this wait is visible to the compiler, so it does not later wait for them
  // against the (compiler-invisible) tile loads.
  __builtin_amdgcn_s_waitcnt(0);

  // Load tile `it` into ring buffer it % NB: this wave issues instructions
  // k = w, w+4, ... of the tile's 18; instruction k fills chunk positions
  // [64k, 64k+64), i.e. chunks 4k .. 4k+3 of all 16 rows.  Lane l brings chunk
  // 4k + (l>>4) of row (l & 15) ^ 4((l>>4) & 1).
  const uint32_t dma_lane = (((l & 15) ^ (4 * ((l >> 4) & 1))) * kRowChunks + (l >> 4)) * 16;
  auto issue = [&](int it) {
    const int jt = j0 + it * kTile;
    const int page = jt / P;
    if (page >= pg_base + 64) {
      pg_base += 64;
      const int pg = pg_base + l;
      pg_vec = (pg < p.max_blocks && pg * P < j1) ? bt_row[pg] : 0;
    }
    const int phys = __builtin_amdgcn_readlane(pg_vec, page - pg_base);
    const uint8_t* tb = cache + ((size_t)phys * P + (jt - page * P)) * kRowBytes + dma_lane;
    const uint32_t lb = tiles_lds + (it % NB) * kTileBytes;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const int k = w + 4 * i;
      if (k < 18) dma16(tb + 64 * k, lb + k * 1024);
    }
  };

  // score-phase K reads: lane reads chunk 4ks + (l>>4) of tile row (l & 15)
  const uint32_t k_lane = (((l >> 4) * 16) + ((l & 15) ^ (4 * ((l >> 4) & 1)))) * 16;
  // value-phase transposing reads: group g = l>>4, lane j = l&15; read r covers rows
  // 8(g>>1) + 4r + (j>>2) and columns 32fb + 16(g&1) + 4(j&3) .. +3, i.e. chunk
  // 4fb + 2(g&1) + ((j>>1)&1), byte 8(j&1) of the chunk
  uint32_t v_lane[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int g = l >> 4, j = l & 15;
    const int tok = 8 * (g >> 1) + 4 * r + (j >> 2);
    const int cl = 2 * (g & 1) + ((j >> 1) & 1);
    v_lane[r] = (cl * 16 + (tok ^ (4 * (cl & 1)))) * 16 + 8 * (j & 1);
  }
  const uint32_t pbuf_lds = lds_addr_of(pbuf);
  const uint32_t flag_lds = lds_addr_of(flag_s);
  const float sl2 = p.scale_log2;

  // Softmax reference per row: the max of the row's first tile with a visible key.
  // Probabilities are exp2(s - m_ref).  A tile whose max exceeds m_ref by more
  // than kLazy raises m_ref; the pass is then finished and replayed from the
  // first tile (exact for any finite scores; never taken for scores of O(1)).
  float m_ref[2] = {-INFINITY, -INFINITY};
  float l_part[2];
  f32x16 acc[4][4];
  for (;;) {
    if (pg_base != j0 / P) {  // a replay after the page window moved: rewind it
      pg_base = j0 / P;
      const int pg = pg_base + l;
      pg_vec = (pg < p.max_blocks && pg * P < j1) ? bt_row[pg] : 0;
    }
    l_part[0] = l_part[1] = 0.f;
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) acc[x][y] = f32x16{};
    for (int it = 0; it < NB - 1 && it < ntiles; ++it) issue(it);
    bool replay = false;
    for (int i = 0; i < ntiles; ++i) {
      // tile i has landed once at most NB-2 later tiles of this wave's loads are in flight
      if (i + NB - 2 < ntiles) {
        if (w < 2) wait_vm<5 * (NB - 2)>();
        else wait_vm<4 * (NB - 2)>();
      } else {
        wait_vm<0>();
      }
      barrier();
      if (i + NB - 1 < ntiles) issue(i + NB - 1);
      const uint32_t buf = tiles_lds + (i % NB) * kTileBytes;
      const int nvalid = j1 - (j0 + i * kTile);
      if (nvalid < kTile) {
        // Rows past the end of the range were loaded from the rest of the page,
        // which may hold anything: clear them so that 0-probability x row stays 0.
        for (int x = threadIdx.x; x < kRowChunks * kTile; x += 256) {
          const int c = x >> 4, t = x & 15;
          if (t >= nvalid)
            *(__attribute__((address_space(3))) u32x4*)(uintptr_t)(buf + (c * 16 + (t ^ (4 * (c & 1)))) * 16) =
                u32x4{0u, 0u, 0u, 0u};
        }
        wait_lgkm0();
        barrier();
      }

      // ---- scores: S^T[16 tok x 32 rows], K operand reads 4 steps ahead ----
      f32x4 s0 = {}, s1 = {};
      {
        constexpr int PF = 4;
        bf16x8 kb[PF];
#pragma unroll
        for (int ks = 0; ks < PF; ++ks) kb[ks] = lds_b128(buf + k_lane + 1024 * ks);
#pragma unroll
        for (int ks = 0; ks < 18; ++ks) {
          const bf16x8 kop = kb[ks % PF];
          if (ks + PF < 18)
            kb[ks % PF] = lds_b128(buf + k_lane + 1024 * (ks + PF));
          s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, q[0][ks], s0, 0, 0, 0);
          s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, q[1][ks], s1, 0, 0, 0);
          // keep the read of step ks+PF ahead of these MFMAs (no code motion across)
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      // ---- mask, scale (log2 domain), probabilities ----
      const int jl = j0 + i * kTile + 4 * (l >> 4);
      float sv[2][4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sv[0][r] = (jl + r < lim[0]) ? s0[r] * sl2 : -INFINITY;
        sv[1][r] = (jl + r < lim[1]) ? s1[r] * sl2 : -INFINITY;
      }
      bool grow = false;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        float mx = fmaxf(fmaxf(sv[nb][0], sv[nb][1]), fmaxf(sv[nb][2], sv[nb][3]));
        mx = max4lanes(mx);
        if (m_ref[nb] == -INFINITY) {
          m_ref[nb] = mx;
        } else if (mx > m_ref[nb] + kLazy) {
          m_ref[nb] = mx;
          grow = true;
        }
        const float mb = (m_ref[nb] == -INFINITY) ? 0.f : m_ref[nb];
        float pr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) pr[r] = __builtin_amdgcn_exp2f(sv[nb][r] - mb);
        l_part[nb] += (pr[0] + pr[1]) + (pr[2] + pr[3]);
        u32x2 pk;
        pk[0] = pack_bf16x2(pr[0], pr[1]);
        pk[1] = pack_bf16x2(pr[2], pr[3]);
        const int row = 32 * w + 16 * nb + (l & 15);
        *(__attribute__((address_space(3))) u32x2*)(uintptr_t)(pbuf_lds + row * 32 + (l >> 4) * 8) = pk;
      }
      const bool any = __builtin_amdgcn_ballot_w64(grow) != 0;
      if (l == 0) flag_s[w] = any ? 1u : 0u;
      wait_lgkm0();
      barrier();
      const u32x4 fl = *(const __attribute__((address_space(3))) u32x4*)(uintptr_t)flag_lds;
      // a flagged pass is finished (its result is discarded) and then replayed
      replay |= (fl[0] | fl[1] | fl[2] | fl[3]) != 0u;

      // ---- values: O^T[128 cols x 128 rows] += V^T P^T, next V operand read ahead ----
      bf16x8 pb[4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
        pb[rb] = lds_b128(pbuf_lds + (32 * rb + (l & 31)) * 32 + (l >> 5) * 16);
      bf16x8 vop[2];
#pragma unroll
      for (int fbl = 0; fbl < 4; ++fbl) {
        const int fb = 4 * w + fbl;
        if (fbl == 0)
          vop[0] = join8(lds_tr16(buf + v_lane[0] + 1024 * fb), lds_tr16(buf + v_lane[1] + 1024 * fb));
        __builtin_amdgcn_sched_barrier(0);
        if (fbl < 3)
          vop[(fbl + 1) & 1] = join8(lds_tr16(buf + v_lane[0] + 1024 * (fb + 1)),
                                     lds_tr16(buf + v_lane[1] + 1024 * (fb + 1)));
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
          acc[fbl][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[fbl & 1], pb[rb], acc[fbl][rb], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (!replay) break;
    wait_vm<0>();
    barrier();
  }

  // ---- finalize: row sums, lse, normalisation ----
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const float ls = sum4lanes(l_part[nb]);
    const int rl = 32 * w + 16 * nb + (l & 15);
    const int gr = row0 + rl;
    const float inv = ls > 0.f ? 1.f / ls : 0.f;
    if ((l >> 4) == 0) {
      inv_s[rl] = inv;
      if (gr < TH) {
        // lse in natural log: (m + log2(sum)) * ln 2
        const float lse2 = (ls > 0.f) ? m_ref[nb] + __builtin_amdgcn_logf(ls) : -INFINITY;
        const float lse_nat = lse2 * 0.69314718055994530942f;
        if constexpr (SPLIT) {
          p.part_lse[(size_t)slot * TH + gr] = lse_nat;
        } else {
          if (p.lse) p.lse[(size_t)b * TH + gr] = lse_nat;
        }
      }
    }
  }
  wait_lgkm0();
  barrier();
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int rl = 32 * rb + (l & 31);
    const int gr = row0 + rl;
    if (gr >= TH) continue;
    const float inv = inv_s[rl];
    const size_t orow = (size_t)(SPLIT ? slot : b) * TH + gr;
#pragma unroll
    for (int fbl = 0; fbl < 4; ++fbl) {
      const int colb = 128 * w + 32 * fbl + 4 * (l >> 5);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int col = colb + 8 * q4;
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[fbl][rb][4 * q4 + e] * inv;
        if constexpr (SPLIT || OUT_F32) {
          float* dst = (SPLIT ? p.part_out : (float*)p.out) + orow * kR + col;
          *(f32x4*)dst = v;
        } else {
          u32x2 pk;
          pk[0] = pack_bf16x2(v[0], v[1]);
          pk[1] = pack_bf16x2(v[2], v[3]);
          *(u32x2*)((uint16_t*)p.out + orow * kR + col) = pk;
        }
      }
    }
  }
}

// ---- split plan: work list (b, j0, j1, slot) and split_indptr ----
// S > 0: every sequence cut into S chunks of ceil(ceil(L/S)/P)*P tokens.
// S == 0: chunk = max(min_chunk, ceil(sum(L)/target_units) rounded up to P);
//         S_b = clamp(ceil(L_b/chunk), 1, cap); chunk_b = ceil(ceil(L_b/S_b)/P)*P.
__global__ __launch_bounds__(1024) void plan_kernel(PlanParams p) {
  __shared__ int red[1024];
  __shared__ long long total_s;
  const int tid = threadIdx.x;
  const int B = p.B, P = p.page_size;
  const int per = (B + 1023) / 1024;
  const int b0 = min(B, tid * per), b1 = min(B, b0 + per);
  int chunk_auto = 0;
  if (p.num_splits == 0) {
    long long sum = 0;
    for (int b = b0; b < b1; ++b) sum += p.seqlens[b];
    // block reduction of the total length
    __shared__ long long sred[1024];
    sred[tid] = sum;
    __syncthreads();
    for (int s = 512; s > 0; s >>= 1) {
      if (tid < s) sred[tid] += sred[tid + s];
      __syncthreads();
    }
    if (tid == 0) total_s = sred[0];
    __syncthreads();
    const long long tot = total_s;
    long long c = (tot + p.target_units - 1) / p.target_units;
    c = ((c + P - 1) / P) * P;
    if (c < p.min_chunk) c = p.min_chunk;
    chunk_auto = (int)c;
  }
  // split count per sequence and local prefix
  int local = 0;
  for (int b = b0; b < b1; ++b) {
    int s;
    if (p.num_splits > 0) s = p.num_splits;
    else {
      const int L = p.seqlens[b];
      s = (L + chunk_auto - 1) / chunk_auto;
      s = max(1, min(p.cap, s));
    }
    local += s;
  }
  red[tid] = local;
  __syncthreads();
  // inclusive scan (Hillis-Steele) over 1024 partial sums
  for (int off = 1; off < 1024; off <<= 1) {
    int v = tid >= off ? red[tid - off] : 0;
    __syncthreads();
    red[tid] += v;
    __syncthreads();
  }
  int base = red[tid] - local;
  if (tid == 1023) *p.n_items = red[1023];
  if (tid == 0) p.split_indptr[0] = 0;
  for (int b = b0; b < b1; ++b) {
    const int L = p.seqlens[b];
    int s;
    if (p.num_splits > 0) s = p.num_splits;
    else {
      s = (L + chunk_auto - 1) / chunk_auto;
      s = max(1, min(p.cap, s));
    }
    const int per_s = (L + s - 1) / s;
    const int chunk = ((per_s + P - 1) / P) * P;
    for (int k = 0; k < s; ++k) {
      long long a0 = (long long)k * chunk, a1 = a0 + chunk;
      if (a0 > L) a0 = L;
      if (a1 > L) a1 = L;
      int* wi = p.work + 4 * (size_t)(base + k);
      wi[0] = b;
      wi[1] = (int)a0;
      wi[2] = (int)a1;
      wi[3] = base + k;
    }
    base += s;
    p.split_indptr[b + 1] = base;
  }
}

template <int NB, bool SPLIT, bool F32>
static hipError_t launch_decode_t(const DecodeParams& prm, int grid, hipStream_t st) {
  hipLaunchKernelGGL((decode_kernel<NB, SPLIT, F32>), dim3(grid), dim3(256), 0, st, prm);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams& prm, int grid, bool split, bool out_f32,
                         hipStream_t st) {
  constexpr int NB = 6;
  if (split) return launch_decode_t<NB, true, true>(prm, grid, st);
  if (out_f32) return launch_decode_t<NB, false, true>(prm, grid, st);
  return launch_decode_t<NB, false, false>(prm, grid, st);
}

hipError_t launch_plan(const PlanParams& prm, hipStream_t st) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, st, prm);
  return hipGetLastError();
}

}  // namespace mla
