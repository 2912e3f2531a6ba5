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
//    into a ring of NB buffers.  Every wave issues a quarter of each tile's 18
//    load instructions.
//  * Score phase: wave w owns query rows [32w, 32w+32) and computes
//    S^T[16 tok x 32 rows] with 16x16x32 MFMAs; the K operand is read from LDS
//    with ds_read_b128, the query lives in registers for the whole kernel.
//  * Softmax: log2 domain against a per-row reference m_ref (the max of the
//    row's first tile with a visible key), so exponentials are bounded by
//    2^kLazy and the fp32 accumulator is never rescaled.  Each lane checks its
//    own scores against m_ref + kLazy; only when one exceeds it is the row max
//    reduced across lanes, m_ref raised and the work unit replayed from its
//    first tile (exact for any finite scores; never taken for scores of
//    ordinary magnitude).
//  * Probabilities (bf16) of all 128 rows are exchanged through LDS (two
//    buffers, alternating tiles).
//  * Value phase: wave w owns latent columns [128w, 128w+128) of all 128 rows
//    (O^T accumulator 128 x 128 fp32 = 256 registers) and multiplies
//    V^T[32 cols x 16 tok] (transposing LDS reads) by P^T[16 tok x 32 rows]
//    with 32x32x16 MFMAs.  Splitting the value GEMM by columns rather than by
//    rows means each V element is read from LDS once per workgroup instead of
//    once per wave.
//  * Software pipeline, one barrier per tile: after the barrier of step i the
//    wave computes the scores of tile i+1, then issues the value MFMAs of tile
//    i with the softmax of tile i+1 placed between them, so the vector ALU
//    work runs while the matrix core is busy.
//
// Tile LDS layout (chunk-major): the 16-byte chunk c (c < 72) of tile row t is
// stored at chunk position 16c + (t ^ g(c & 3)) with g = (0, 12, 8, 4).  A K
// read (16 rows of 4 chunks) and a transposing V read are then both free of
// bank conflicts on gfx950 (measured with SQ_LDS_BANK_CONFLICT; g = (0, 4, 8,
// 12), the obvious choice, makes the 16-byte K reads conflict 2-way); the
// direct-to-LDS loads write 1 KB contiguous.
//
// Probability buffer: row R (of 128) holds 16 bf16 = two 16-byte chunks, chunk c
// (tokens 8c..8c+7) at byte 32R + 16(c ^ s(R)), s(R) = ((R >> 2) ^ (R >> 4)) & 1;
// 16-byte writes and reads of it are conflict-free.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace mla {

constexpr float kLazy = 64.0f;  // log2-domain growth of the max tolerated before a replay

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_lgkm() {
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until at most `tiles` of this wave's most recent tile loads are in
// flight (PER = load instructions per tile issued by this wave).
template <int PER, int MAXT>
__device__ __forceinline__ void wait_tiles(int tiles) {
  static_assert(MAXT <= 6, "extend the switch");
  switch (tiles < MAXT ? tiles : MAXT) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<PER>(); break;
    case 2: wait_vm<2 * PER>(); break;
    case 3: if constexpr (MAXT >= 3) wait_vm<3 * PER>(); break;
    case 4: if constexpr (MAXT >= 4) wait_vm<4 * PER>(); break;
    case 5: if constexpr (MAXT >= 5) wait_vm<5 * PER>(); break;
    default: if constexpr (MAXT >= 6) wait_vm<6 * PER>(); break;
  }
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

// max of four floats in two VALU ops (v_max3 does not canonicalise its inputs;
// the scores here are never signalling NaNs)
__device__ __forceinline__ float max4(float a, float b, float c, float d) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  asm("v_max3_f32 %0, %1, %2, %2" : "=v"(r) : "v"(r), "v"(d));
  return r;
}

__device__ __forceinline__ bf16x8 lds_b128(uint32_t addr) {
  return *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)addr;
}
// Transposing LDS read: within each 16-lane group, lane i receives element i%4
// of the 8-byte rows read by lanes i/4, i/4+4, i/4+8, i/4+12 (in that order).
__device__ __forceinline__ s16x4 lds_tr16(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(uintptr_t)addr);
}
__device__ __forceinline__ void lds_st64(uint32_t addr, u32x2 v) {
  *(__attribute__((address_space(3))) u32x2*)(uintptr_t)addr = v;
}

// Value-phase MFMA with its accumulator pinned to AGPRs (the 128x128 fp32 O^T
// block of a wave fills all 256 of them); written as inline assembly so that
// the score accumulators, which the softmax reads, stay in VGPRs.  The operands
// come straight from LDS reads (the compiler's wait counts cover them); the
// accumulator is next touched by VALU code only after mfma_drain().
__device__ __forceinline__ void mfma_pv(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// Wait states between the last value MFMA and any VALU access to its
// accumulator (a 16-pass XDL result needs at most 18).
__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// Row swizzle of the tile layout and the position (in 16-byte units) of chunk c
// of tile row t.
__device__ __forceinline__ int tile_swz(int c) { return (-4 * c) & 12; }
__device__ __forceinline__ int tile_pos(int c, int t) { return 16 * c + (t ^ tile_swz(c & 3)); }
// probability-buffer chunk swap of row r
__device__ __forceinline__ int pbuf_swz(int r) { return ((r >> 2) ^ (r >> 4)) & 1; }
// v_permlane16_swap of two different registers: afterwards a = [a.r0, b.r0,
// a.r2, b.r2] and b = [a.r1, b.r1, a.r3, b.r3] (r = 16-lane row)
__device__ __forceinline__ void swap16(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 2\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}

template <int NB, bool SPLIT, bool OUT_F32>
__global__ __launch_bounds__(256, 1) void decode_kernel(DecodeParams p) {
  // tile ring; after the last tile it is reused to stage the 128 KB output block
  constexpr int kRingBytes = NB * kTileBytes > 128 * 1024 ? NB * kTileBytes : 128 * 1024;
  __shared__ __attribute__((aligned(16))) uint8_t tiles[kRingBytes];
  __shared__ __attribute__((aligned(16))) uint16_t pbuf[2 * kRowsPerWG * kTile];
  __shared__ __attribute__((aligned(16))) float inv_s[kRowsPerWG];
  __shared__ unsigned flag_s;

  const int w = wave_id();
  const int l = lane_id();

  // ---- work unit.  Units u = item * n_rg + rg are dealt to the XCDs in
  // contiguous ranges (workgroup i runs on XCD i % 8), so the splits of one
  // sequence share an L2 and re-read its query rows from there.
  const int n_units = (SPLIT && p.work) ? *p.n_items * p.n_rg : p.n_units;
  const int per_xcd = (n_units + 7) >> 3;
  const int kx = blockIdx.x >> 3;
  if (kx >= per_xcd) return;
  const int u = (blockIdx.x & 7) * per_xcd + kx;
  if (u >= n_units) return;
  const int item = u / p.n_rg;
  const int rg = u - item * p.n_rg;

  int b, j0, j1, slot;
  if constexpr (SPLIT) {
    if (p.work) {  // automatic split counts: work list from the plan kernel
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
  // work-unit scalars are wave-uniform: keep them in scalar registers
  b = __builtin_amdgcn_readfirstlane(b);
  j0 = __builtin_amdgcn_readfirstlane(j0);
  j1 = __builtin_amdgcn_readfirstlane(j1);
  slot = __builtin_amdgcn_readfirstlane(slot);
  const int L = __builtin_amdgcn_readfirstlane(p.seqlens[b]);
  const int T = p.T, H = p.H, TH = T * H;
  const int P = p.page_size;
  const int row0 = rg * kRowsPerWG;

  // ---- query rows of this wave (score phase) and their visible limits ----
  // dd[nb] = (first invisible key of the row) - j0 - 4(l>>4): key r of the lane's
  // 4-key group in tile i is visible iff r < dd[nb] - 16 i.  Padding rows past
  // T*H get a zero query and see every key (their scores are 0, never stored).
  bf16x8 q[2][18];
  int dd[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int gr = row0 + 32 * w + 16 * nb + (l & 15);
    int lim = j1;
    if (gr < TH) {
      const int t = gr / H;
      const int h = gr - t * H;
      lim = min(L - T + t + 1, j1);
      const uint16_t* ql = p.q_lat + ((size_t)(b * T + t) * H + h) * kR + 8 * (l >> 4);
      const uint16_t* qp = p.q_pe + ((size_t)(b * T + t) * H + h) * kDR + 8 * (l >> 4);
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) q[nb][ks] = *(const bf16x8*)(ql + 32 * ks);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) q[nb][16 + ks] = *(const bf16x8*)(qp + 32 * ks);
    } else {
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) q[nb][ks] = bf16x8{};
    }
    dd[nb] = lim - j0 - 4 * (l >> 4);
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
  if (threadIdx.x == 0) flag_s = 0u;
  // q and the first page ids must be complete before any tile load is in flight:
  // this wait is visible to the compiler, so it does not later wait for them
  // against the (compiler-invisible) tile loads.
  __builtin_amdgcn_s_waitcnt(0);

  // Load tile `it` into ring buffer it % NB: this wave issues instructions
  // k = w, w+4, ... of the tile's 18; instruction k fills chunk positions
  // [64k, 64k+64), i.e. chunks 4k .. 4k+3 of all 16 rows.  Lane l writes
  // position 64k + l: chunk 4k + (l>>4) of row (l & 15) ^ g(l>>4).
  const uint32_t dma_lane = ((l & 15) ^ tile_swz(l >> 4)) * kRowBytes + 16 * (l >> 4);
  // Tile loads are issued a few instructions at a time between the MFMAs:
  // issue_prep(it) selects tile `it` (its page and ring buffer), issue_part(n)
  // issues this wave's n-th load instruction of it (k = w + 4n < 18).  The
  // tile's global base is wave-uniform (scalar registers); lane offsets are
  // dma_lane + 64w + 256n.
  const uint32_t dma_voff = dma_lane + 64 * w;
  const uint8_t* dma_base = cache;
  uint32_t dma_dst = 0;
  auto issue_prep = [&](int it) {
    const int jt = j0 + it * kTile;
    const int page = jt / P;
    if (page >= pg_base + 64) {
      pg_base += 64;
      const int pg = pg_base + l;
      pg_vec = (pg < p.max_blocks && pg * P < j1) ? bt_row[pg] : 0;
      // complete the reload here, visibly to the compiler, so that the common
      // path carries no wait for it (a vector-memory wait would also drain the
      // in-flight tile loads)
      __builtin_amdgcn_s_waitcnt(0);
    }
    const int phys = __builtin_amdgcn_readlane(pg_vec, page - pg_base);
    dma_base = cache + ((size_t)phys * P + (jt - page * P)) * kRowBytes;
    dma_dst = tiles_lds + (it % NB) * kTileBytes + 1024 * w;
  };
  auto issue_part = [&](auto n_const) {
    constexpr int n = decltype(n_const)::value;
    if (w + 4 * n < 18) dma16s(dma_voff + 256 * n, dma_base, dma_dst + 4096 * n);
  };
  auto issue = [&](int it) {
    issue_prep(it);
    issue_part(std::integral_constant<int, 0>{});
    issue_part(std::integral_constant<int, 1>{});
    issue_part(std::integral_constant<int, 2>{});
    issue_part(std::integral_constant<int, 3>{});
    issue_part(std::integral_constant<int, 4>{});
  };
  // Rows past the end of the range were loaded from the rest of the page, which
  // may hold anything: clear their value chunks so that 0-probability x row is 0.
  auto clear_tail = [&](int it) {
    const int nvalid = j1 - (j0 + it * kTile);
    if (nvalid >= kTile) return;
    const uint32_t buf = tiles_lds + (it % NB) * kTileBytes;
    for (int x = threadIdx.x; x < 64 * kTile; x += 256) {
      const int c = x >> 4, t = x & 15;
      if (t >= nvalid)
        *(__attribute__((address_space(3))) u32x4*)(uintptr_t)(buf + tile_pos(c, t) * 16) = u32x4{0u, 0u, 0u, 0u};
    }
  };

  // score-phase K reads: lane reads chunk 4ks + (l>>4) of tile row (l & 15)
  const uint32_t k_lane = ((l >> 4) * 16 + ((l & 15) ^ tile_swz(l >> 4))) * 16;
  // value-phase transposing reads: group g = l>>4, lane j = l&15; read r covers
  // rows 8(g>>1) + 4r + (j>>2) and columns 32fb + 16(g&1) + 4(j&3) .. +3, i.e.
  // chunk 4fb + cl with cl = 2(g&1) + ((j>>1)&1), byte 8(j&1) of the chunk
  uint32_t v_lane[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int g = l >> 4, j = l & 15;
    const int tok = 8 * (g >> 1) + 4 * r + (j >> 2);
    const int cl = 2 * (g & 1) + ((j >> 1) & 1);
    v_lane[r] = (16 * cl + (tok ^ tile_swz(cl))) * 16 + 8 * (j & 1);
  }
  // probability buffer: after the row exchange in sm_store lane l holds tokens
  // 8(l>>5) .. +7 of row 32w + (l & 31); the value phase reads row 32rb + (l & 31),
  // chunk l>>5 (the P^T operand layout)
  const uint32_t pbuf_lds = lds_addr_of(pbuf);
  const uint32_t p_rd = (l & 31) * 32 + 16 * ((l >> 5) ^ pbuf_swz(l & 31));
  const uint32_t p_wr = 32 * 32 * w + p_rd;
  const float sl2 = p.scale_log2;
  const float lazy_raw = kLazy / sl2;

  // Per-row softmax reference (log2 domain) and the raw-score threshold above
  // which a replay is needed; nmb = -m_ref (0 while the row has no visible key).
  float m_ref[2] = {-INFINITY, -INFINITY};
  float nmb[2] = {0.f, 0.f};
  float thr[2] = {INFINITY, INFINITY};
  bool ref_pending = true;
  float l_part[2];
  f32x16 acc[4][4];

  // ---- softmax pieces of one tile (scores s0, s1 of tile `it`) ----
  float x[2][4], mxl[2];
  float (&pr)[2][4] = x;  // probabilities overwrite the masked scores
  bool grow = false;
  auto sm_mask = [&](int nb, const f32x4& s, int it) {
    const int rel = dd[nb] - kTile * it;
#pragma unroll
    for (int r = 0; r < 4; ++r) x[nb][r] = (r < rel) ? s[r] : -INFINITY;
  };
  auto sm_check = [&]() {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) mxl[nb] = max4(x[nb][0], x[nb][1], x[nb][2], x[nb][3]);
    grow = __builtin_amdgcn_ballot_w64((mxl[0] > thr[0]) | (mxl[1] > thr[1])) != 0;
  };
  auto sm_reference = [&]() {  // first visible tile of a row: fix m_ref
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const float mx = max4lanes(max4(x[nb][0], x[nb][1], x[nb][2], x[nb][3]));
      if (m_ref[nb] == -INFINITY && mx != -INFINITY) {
        m_ref[nb] = mx * sl2;
        nmb[nb] = -m_ref[nb];
        thr[nb] = mx + lazy_raw;
      }
    }
    ref_pending = __builtin_amdgcn_ballot_w64((m_ref[0] == -INFINITY) | (m_ref[1] == -INFINITY)) != 0;
  };
  auto sm_fma = [&](int nb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) pr[nb][r] = __builtin_fmaf(x[nb][r], sl2, nmb[nb]);
  };
  auto sm_exp = [&](int nb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) pr[nb][r] = __builtin_amdgcn_exp2f(pr[nb][r]);
  };
  auto sm_sum = [&]() {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) l_part[nb] += (pr[nb][0] + pr[nb][1]) + (pr[nb][2] + pr[nb][3]);
  };
  // Probabilities to bf16, then one row exchange turns the score layout (lane:
  // row (l&15) + 16nb, tokens 4(l>>4)..+3) into 8 consecutive tokens of one row
  // per lane (row l & 31, tokens 8(l>>5)..+7), stored with one 16-byte write.
  auto sm_store = [&](int it) {
    const uint32_t base = pbuf_lds + (it & 1) * (kRowsPerWG * kTile * 2);
    u32x2 a = cvt_bf16x4(f32x4{pr[0][0], pr[0][1], pr[0][2], pr[0][3]});
    u32x2 c = cvt_bf16x4(f32x4{pr[1][0], pr[1][1], pr[1][2], pr[1][3]});
    uint32_t a0 = a[0], a1 = a[1], c0 = c[0], c1 = c[1];
    swap16(a0, c0);
    swap16(a1, c1);
    *(__attribute__((address_space(3))) u32x4*)(uintptr_t)(base + p_wr) = u32x4{a0, a1, c0, c1};
  };
  // a row's max grew by more than kLazy: raise its reference, flag a replay
  auto sm_grow = [&]() {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const float mx = max4lanes(mxl[nb]);
      if (mx > thr[nb]) {
        m_ref[nb] = mx * sl2;
        nmb[nb] = -m_ref[nb];
        thr[nb] = mx + lazy_raw;
      }
    }
    if (l == 0) flag_s = 1u;
  };
  // whole softmax of one tile, not interleaved (first tile, rows still without
  // a reference)
  auto softmax_tile = [&](const f32x4& s0, const f32x4& s1, int it) {
    sm_mask(0, s0, it);
    sm_mask(1, s1, it);
    if (ref_pending) sm_reference();
    sm_check();
    sm_fma(0);
    sm_fma(1);
    sm_exp(0);
    sm_exp(1);
    sm_sum();
    sm_store(it);
    if (grow) sm_grow();
  };

  // scores S^T of tile `it` (not interleaved: prologue)
  auto scores_plain = [&](int it, f32x4& s0, f32x4& s1) {
    const uint32_t kbase = tiles_lds + (it % NB) * kTileBytes + k_lane;
    s0 = f32x4{};
    s1 = f32x4{};
    constexpr int PF = 4;
    bf16x8 kb[PF];
#pragma unroll
    for (int ks = 0; ks < PF; ++ks) kb[ks] = lds_b128(kbase + 1024 * ks);
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      const bf16x8 kop = kb[ks % PF];
      if (ks + PF < 18) kb[ks % PF] = lds_b128(kbase + 1024 * (ks + PF));
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, q[0][ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, q[1][ks], s1, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Smallest key limit over this wave's rows: a tile ending at or before it
  // needs no mask for any of them.
  int lim_lo = j1;
  {
    const int g0 = row0 + 32 * w;
    if (g0 < TH) lim_lo = min(L - T + g0 / H + 1, j1);
  }

  // At most one replay: after a flagged pass every row's reference is within
  // kLazy of its true maximum, so the replay cannot flag again.
  for (int pass = 0;; ++pass) {
    if (pg_base != j0 / P) {  // a replay after the page window moved: rewind it
      pg_base = j0 / P;
      const int pg = pg_base + l;
      pg_vec = (pg < p.max_blocks && pg * P < j1) ? bt_row[pg] : 0;
      __builtin_amdgcn_s_waitcnt(0);
    }
    l_part[0] = l_part[1] = 0.f;
#pragma unroll
    for (int xx = 0; xx < 4; ++xx)
#pragma unroll
      for (int y = 0; y < 4; ++y) acc[xx][y] = f32x16{};
    for (int it = 0; it < NB - 1 && it < ntiles; ++it) issue(it);

    // Two-stage pipeline.  Step i (after its barrier): value MFMAs of tile i
    // (probabilities P(i) written during step i-1), score MFMAs of tile i+2,
    // and the softmax of tile i+1 (scores from step i-1) producing P(i+1).
    // The first K operands of tile i+3 are read at the end of step i, so every
    // step starts with MFMAs; tile i+3 has therefore landed before barrier i.
    // Resident ring buffers: tiles i .. i+3; up to NB-5 more in flight.
    constexpr int PF = 4;  // K operand reads in flight
    bf16x8 kb[PF];
    auto k_first = [&](int it) {
      const uint32_t kbase = tiles_lds + (it % NB) * kTileBytes + k_lane;
#pragma unroll
      for (int ks = 0; ks < PF; ++ks) kb[ks] = lds_b128(kbase + 1024 * ks);
    };
    f32x4 s0 = {-INFINITY, -INFINITY, -INFINITY, -INFINITY}, s1 = s0;  // scores of tile i+1
    if (ntiles > 0) {
      // prologue: tiles 0, 1 and 2 landed; P(0), the scores of tile 1 and the
      // first K operands of tile 2
      const int ahead = max(0, min(NB - 1, ntiles) - 3);
      if (w < 2) wait_tiles<5, NB - 4>(ahead);
      else wait_tiles<4, NB - 4>(ahead);
      barrier();
      clear_tail(0);
      if (ntiles > 1) clear_tail(1);
      if (ntiles > 2) clear_tail(2);
      f32x4 t0, t1;
      scores_plain(0, t0, t1);
      softmax_tile(t0, t1, 0);
      if (ntiles > 1) scores_plain(1, s0, s1);
      k_first(2);
    }
    for (int i = 0; i < ntiles; ++i) {
      const bool do_qk = i + 2 < ntiles;
      const bool do_sm = i + 1 < ntiles;
      const bool do_issue = i + NB - 1 < ntiles;
      // tile i+3 must have landed; up to NB-5 later tiles may stay in flight
      if (i + 3 < ntiles) {
        if (w < 2) wait_tiles<5, NB - 5>(min(NB - 5, ntiles - i - 4));
        else wait_tiles<4, NB - 5>(min(NB - 5, ntiles - i - 4));
      }
      // this wave's probability writes and tail clears must be complete; LDS
      // operations complete in order, so allowing only the PF K reads issued
      // last (by k_first) to remain in flight is enough
      wait_lgkm<PF>();
      barrier();
      if (i + 3 < ntiles) clear_tail(i + 3);
      if (do_issue) issue_prep(i + NB - 1);

      // softmax of tile i+1 done up front when some row still needs its
      // reference; the interleaved copy below then runs on -inf scores, which
      // makes every one of its steps a no-op (its probabilities are not stored)
      bool sm_here = do_sm;
      if (do_sm && ref_pending) {
        softmax_tile(s0, s1, i + 1);
        sm_here = false;
        s0 = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        s1 = s0;
      }
      const bool full = j0 + kTile * (i + 2) <= lim_lo;  // tile i+1 needs no mask

      const uint32_t kbase = tiles_lds + ((i + 2) % NB) * kTileBytes + k_lane;
      const uint32_t pbase = pbuf_lds + (i & 1) * (kRowsPerWG * kTile * 2) + p_rd;
      const uint32_t vbuf = tiles_lds + (i % NB) * kTileBytes + 4096 * w;
      const uint32_t vb0 = vbuf + v_lane[0], vb1 = vbuf + v_lane[1];
      bf16x8 pb[4], vop[2];
#pragma unroll
      for (int m = 0; m < 4; ++m) pb[m] = lds_b128(pbase + 1024 * m);
      vop[0] = join8(lds_tr16(vb0), lds_tr16(vb1));
      // (the score MFMAs also run in the last two steps, on a stale buffer; their
      // results are discarded)
      f32x4 n0 = {}, n1 = {};  // scores of tile i+2
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) {
        {
          const bf16x8 kop = kb[ks % PF];
          if (ks + PF < 18) kb[ks % PF] = lds_b128(kbase + 1024 * (ks + PF));
          n0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, q[0][ks], n0, 0, 0, 0);
          n1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, q[1][ks], n1, 0, 0, 0);
        }
        // value MFMAs: none in steps 0-3 (their operands, read after the
        // barrier, are still arriving), one per step in 4-13, two in 14-16
        constexpr int kPvBegin[18] = {0, 0, 0, 0, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 12, 14, 16};
        constexpr int kPvEnd[18] = {0, 0, 0, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 12, 14, 16, 16};
#pragma unroll
        for (int v = kPvBegin[ks]; v < kPvEnd[ks]; ++v) {
          const int f = v >> 2, rb = v & 3;
          mfma_pv(acc[f][rb], vop[f & 1], pb[rb]);
        }
        // V operand of column block f read a block ahead (two alternating slots)
        if (ks == 2 || ks == 8 || ks == 12) {
          const int f = ks == 2 ? 1 : ks == 8 ? 2 : 3;
          vop[f & 1] = join8(lds_tr16(vb0 + 1024 * f), lds_tr16(vb1 + 1024 * f));
        }
        {
          if (ks == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) x[0][r] = s0[r];
            if (!full) sm_mask(0, s0, i + 1);
          }
          if (ks == 1) {
#pragma unroll
            for (int r = 0; r < 4; ++r) x[1][r] = s1[r];
            if (!full) sm_mask(1, s1, i + 1);
          }
          if (ks == 2) sm_check();
          if (ks == 3) sm_fma(0);
          if (ks == 4) { pr[0][0] = __builtin_amdgcn_exp2f(pr[0][0]); pr[0][1] = __builtin_amdgcn_exp2f(pr[0][1]); }
          if (ks == 5) { pr[0][2] = __builtin_amdgcn_exp2f(pr[0][2]); pr[0][3] = __builtin_amdgcn_exp2f(pr[0][3]); }
          if (ks == 6) sm_fma(1);
          if (ks == 7) { pr[1][0] = __builtin_amdgcn_exp2f(pr[1][0]); pr[1][1] = __builtin_amdgcn_exp2f(pr[1][1]); }
          if (ks == 8) { pr[1][2] = __builtin_amdgcn_exp2f(pr[1][2]); pr[1][3] = __builtin_amdgcn_exp2f(pr[1][3]); }
          if (ks == 9) sm_sum();
          if (ks == 10 && sm_here) sm_store(i + 1);
        }
        if (do_issue) {
          if (ks == 2) issue_part(std::integral_constant<int, 0>{});
          if (ks == 6) issue_part(std::integral_constant<int, 1>{});
          if (ks == 10) issue_part(std::integral_constant<int, 2>{});
          if (ks == 14) issue_part(std::integral_constant<int, 3>{});
          if (ks == 17) issue_part(std::integral_constant<int, 4>{});
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (grow) sm_grow();
      k_first(i + 3);  // (a stale buffer near the end; never used then)
      const f32x4 ninf = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      s0 = do_qk ? n0 : ninf;
      s1 = do_qk ? n1 : ninf;
    }
    mfma_drain();
    wait_lgkm0();
    barrier();
    const bool replay = flag_s != 0u && pass == 0;
    if (!replay) break;
    // a flagged pass is discarded and replayed with the raised references
    wait_vm0();
    barrier();
    if (threadIdx.x == 0) flag_s = 0u;
    wait_lgkm0();
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

  // ---- store: the workgroup's rows [row0, row0 + 128) of its output are one
  // contiguous block (1 KB per row in bf16, 2 KB in fp32).  The normalised
  // accumulators are staged through the (now idle) tile ring in row-major
  // order, then written with 16-byte-per-lane contiguous stores.  Staging
  // swizzle: 16-byte chunk c of staged row r sits at chunk c ^ (r & 15); in the
  // bf16 layout the two 8-byte halves of a chunk are also swapped when bit 4 of
  // r is set (both make the staging writes and the reads conflict-free).
  const int n_rows = min(kRowsPerWG, TH - row0);
  char* const dst_base = (char*)(SPLIT ? p.part_out : p.out) + ((size_t)slot * TH + row0) * kR * (OUT_F32 ? 4 : 2);
  constexpr int kRowOut = kR * (OUT_F32 ? 4 : 2);      // bytes per output row
  constexpr int kStageRows = OUT_F32 ? 64 : 128;       // rows per staging round (128 KB)
  static_assert(kStageRows * kRowOut <= kRingBytes, "staging block exceeds the tile ring");
#pragma unroll
  for (int half = 0; half < 128 / kStageRows; ++half) {
#pragma unroll
    for (int rbl = 0; rbl < kStageRows / 32; ++rbl) {
      const int rb = half * (kStageRows / 32) + rbl;
      const int r = 32 * rbl + (l & 31);  // staged row
      const float inv = inv_s[32 * rb + (l & 31)];
#pragma unroll
      for (int fbl = 0; fbl < 4; ++fbl) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[fbl][rb][4 * q4 + e] * inv;
          // columns 128w + 32fbl + 8q4 + 4(l>>5) + [0,4)
          if constexpr (OUT_F32) {
            const int c = 32 * w + 8 * fbl + 2 * q4 + (l >> 5);
            *(__attribute__((address_space(3))) f32x4*)(uintptr_t)(tiles_lds + r * kRowOut + ((c ^ (r & 15)) * 16)) = v;
          } else {
            const int c = 16 * w + 4 * fbl + q4;
            const int hh = (l >> 5) ^ ((r >> 4) & 1);
            lds_st64(tiles_lds + r * kRowOut + ((c ^ (r & 15)) * 16) + 8 * hh, cvt_bf16x4(v));
          }
        }
      }
    }
    wait_lgkm0();
    barrier();
    const int rows_here = min(kStageRows, n_rows - half * kStageRows);
    char* const dst = dst_base + (size_t)half * kStageRows * kRowOut;
    constexpr int kChunksPerRow = kRowOut / 16;
    for (int x = threadIdx.x; x < rows_here * kChunksPerRow; x += 256) {
      const int r = x / kChunksPerRow, c = x - r * kChunksPerRow;
      u32x4 v = *(const __attribute__((address_space(3))) u32x4*)(uintptr_t)(tiles_lds + r * kRowOut + ((c ^ (r & 15)) * 16));
      if (!OUT_F32 && ((r >> 4) & 1)) v = u32x4{v[2], v[3], v[0], v[1]};
      *(u32x4*)(dst + (size_t)r * kRowOut + 16 * c) = v;
    }
    if (half + 1 < 128 / kStageRows) barrier();
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

hipError_t launch_decode(const DecodeParams& prm, int max_units, bool split, bool out_f32,
                         hipStream_t st) {
  constexpr int NB = 8;
  const int grid = ((max_units + 7) / 8) * 8;  // whole XCD rounds; extra workgroups exit
  if (split) {
    if (out_f32) return launch_decode_t<NB, true, true>(prm, grid, st);
    return launch_decode_t<NB, true, false>(prm, grid, st);
  }
  if (out_f32) return launch_decode_t<NB, false, true>(prm, grid, st);
  return launch_decode_t<NB, false, false>(prm, grid, st);
}

hipError_t launch_plan(const PlanParams& prm, hipStream_t st) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, st, prm);
  return hipGetLastError();
}

}  // namespace mla
