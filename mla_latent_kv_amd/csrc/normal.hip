// Normal (non-absorbed) MLA decode on the GPU, chunked over the cache (gfx950).
//
// The reference form of the attention ("MLA in full detail", Step 3 before the
// weight folding; M5.8 0x05 naive path): every cached latent c_j is
// up-projected per head to k_nope = W_UK[h] c_j (128) and v = W_UV[h] c_j (128),
// and each head runs ordinary attention with the 192-wide key [k_nope || k_pe]
// and the 128-wide value:
//     s = (q_nope . k_nope + q_pe . k_pe) * scale,  out = sum_j softmax_j(s) v_j.
// The cache is processed in chunks of `chunk` tokens per sequence (the
// chunked-KV form that bounds the up-projected working set):
//   1. gather_kernel: the chunk's rows of every sequence, through the block
//      table, into a dense latent matrix [B*chunk, 512] and a rope matrix
//      [B*chunk, 64] (rows past a sequence's end are zero);
//   2. two library GEMMs (rocBLAS, bf16 in and out, fp32 accumulation): the
//      up-projected keys K [B*chunk, H, 128] and values V [B*chunk, H, 128];
//   3. mha_kernel: per (sequence, head, 128 query rows) attention over the
//      chunk's keys, continuing a running state (max, sum, unnormalised
//      output) carried from the previous chunk -- the exact log-sum-exp
//      combination of chunk results (M5.8 0x0C) done online -- and writing the
//      normalised output and lse after the last chunk.
//
// mha_kernel layout: 4 waves x 32 query rows; scores S^T[32 keys x 32 rows]
// take 12 32x32x16 MFMAs over the 192-wide key, values O^T[128 x 32 rows] 8
// MFMAs per 32 keys.  Keys stream HBM -> LDS with direct-to-LDS loads in steps
// of 32 (two 16-row halves of 40 16-byte chunks: key 0-15, rope 16-23, value
// 24-39), in the chunk-major swizzled layout of the absorbed kernel (conflict-
// free K reads and transposing V reads), four steps in flight.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

namespace {

constexpr int kNChunks = 40;                      // 16-byte chunks per staged key row
constexpr int kNHalf = 16 * kNChunks * 16;        // 10240 bytes per 16-row half
constexpr int kNStep = 2 * kNHalf;                // 32 keys
constexpr int kNB = 4;                            // steps in the ring
constexpr int kQks = 12;                          // 192 / 16 score MFMAs

__device__ __forceinline__ int swz(int c) { return (-4 * c) & 12; }

// 16 bytes per lane from a 64-bit per-lane address into LDS at lds + 16 * lane;
// the immediate offset moves the global address and the LDS slot together
template <int OFF>
__device__ __forceinline__ void dma_v(const void* addr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off offset:%2" ::"v"(addr),
               "s"(lds - OFF), "n"(OFF)
               : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vm_n() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace

// ---- 1. gather: one wave per (sequence, chunk row) ----
__global__ __launch_bounds__(256) void gather_kernel(NormalParams p) {
  const int l = lane_id();
  const long long m = (long long)blockIdx.x * 4 + wave_id();
  if (m >= (long long)p.B * p.chunk) return;
  const int b = (int)(m / p.chunk);
  const int jj = (int)(m - (long long)b * p.chunk);
  const int j = p.c * p.chunk + jj;
  u32x4 lat = {0u, 0u, 0u, 0u}, rope = {0u, 0u, 0u, 0u};
  if (j < p.seqlens[b]) {
    const int page = j / p.page_size;
    const int blk = p.block_table[(size_t)b * p.max_blocks + page];
    const uint16_t* row = p.cache + ((size_t)blk * p.page_size + (j - page * p.page_size)) * kRow;
    lat = *(const u32x4*)(row + 8 * l);
    if (l < kDR / 8) rope = *(const u32x4*)(row + kR + 8 * l);
  }
  *(u32x4*)(p.lat + (size_t)m * kR + 8 * l) = lat;
  if (l < kDR / 8) *(u32x4*)(p.rope + (size_t)m * kDR + 8 * l) = rope;
}

// ---- 3. attention over one chunk ----
__global__ __launch_bounds__(256, 2) void mha_kernel(NormalParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[kNB * kNStep];
  const int w = wave_id(), l = lane_id(), hl = l >> 5;
  const int T = p.T, H = p.H;
  const int n_tq = (T + 127) / 128;
  int u = blockIdx.x;
  const int tile = u % n_tq;
  u /= n_tq;
  const int h = u % H;
  const int b = u / H;
  const int L = p.seqlens[b];
  const int j0 = p.c * p.chunk;
  const int j1 = min(j0 + p.chunk, L);
  const int nk = max(j1 - j0, 0);                  // keys of this chunk
  const int t = tile * 128 + 32 * w + (l & 31);    // query row of this lane (lanes l, l ^ 32)
  const bool row_ok = t < T;
  const int tq = min(t, T - 1);
  const int lim = row_ok ? min(L - T + t + 1, j1) : j1;  // keys j < lim are visible
  const size_t qrow = ((size_t)b * T + tq) * H + h;
  const float sl2 = p.scale_log2;

  // query: q[ks] = elements 16ks + 8hl .. +7 of [q_nope || q_pe]
  bf16x8 q[kQks];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) q[ks] = *(const bf16x8*)(p.q_nope + qrow * kDN + 16 * ks + 8 * hl);
#pragma unroll
  for (int ks = 8; ks < kQks; ++ks) q[ks] = *(const bf16x8*)(p.q_pe + qrow * kDR + 16 * (ks - 8) + 8 * hl);

  // running state (log2 units): m, this lane's half of the sum, O^T accumulators
  // (acc[cb] register 4 q4 + e = column 32 cb + 8 q4 + 4 hl + e of the row)
  float m = -INFINITY, lsum = 0.f;
  f32x16 acc[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) acc[cb] = f32x16{};
  if (!p.first) {
    m = p.m_state[qrow];
    lsum = hl == 0 ? p.l_state[qrow] : 0.f;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 v = *(const f32x4*)(p.o_state + qrow * kDV + 32 * cb + 8 * q4 + 4 * hl);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[cb][4 * q4 + e] = v[e];
      }
  }
  // every compiler-visible load completes here, before the direct-to-LDS loads
  // start (a later wait for one of them would also drain those)
#pragma unroll
  for (int ks = 0; ks < kQks; ++ks) asm volatile("" ::"v"(q[ks]));
  asm volatile("" ::"v"(m), "v"(lsum));
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) asm volatile("" ::"v"(acc[cb][0]));
  __builtin_amdgcn_s_waitcnt(0);

  // loads: wave w fills half hw = w >> 1 of a step, instructions k = (w & 1) + 2n
  // (n < 5); lane l brings chunk 4k + (l >> 4) of half row rsw
  const int hw = w >> 1;
  const int rsw = (l & 15) ^ swz(l >> 4);
  const uint32_t ring_lds = (uint32_t)(uintptr_t)(const lds_void*)ring;
  const size_t kv_stride = (size_t)H * kDV * 2;              // bytes between consecutive keys
  const uint8_t* kb0 = (const uint8_t*)p.kbuf + ((size_t)b * p.chunk * H + h) * kDV * 2 + 16 * (l >> 4);
  const uint8_t* vb0 = (const uint8_t*)p.vbuf + ((size_t)b * p.chunk * H + h) * kDV * 2 + 16 * (l >> 4);
  const uint8_t* rb0 = (const uint8_t*)p.rope + (size_t)b * p.chunk * kDR * 2 + 16 * (l >> 4);
  auto issue = [&](int it) {
    int jj = 32 * it + 16 * hw + rsw;
    jj = jj < nk ? jj : 0;   // rows past the chunk's end repeat its first key (masked)
    const uint8_t* ka = kb0 + (size_t)jj * kv_stride;
    const uint8_t* va = vb0 + (size_t)jj * kv_stride;
    const uint8_t* ra = rb0 + (size_t)jj * kDR * 2;
    const uint32_t dst = ring_lds + (it % kNB) * kNStep + hw * kNHalf;
    if (w & 1) {
      dma_v<64>(ka, dst + 1024 * 1);
      dma_v<192>(ka, dst + 1024 * 3);
      dma_v<64>(ra, dst + 1024 * 5);
      dma_v<64>(va, dst + 1024 * 7);
      dma_v<192>(va, dst + 1024 * 9);
    } else {
      dma_v<0>(ka, dst + 1024 * 0);
      dma_v<128>(ka, dst + 1024 * 2);
      dma_v<0>(ra, dst + 1024 * 4);
      dma_v<0>(va, dst + 1024 * 6);
      dma_v<128>(va, dst + 1024 * 8);
    }
  };

  // operand addresses: K rows (A operand of the scores) -- lane reads key l & 31
  // (half (l >> 4) & 1), chunk 2ks + hl; V^T (A operand of the values) through
  // transposing reads, token order inside a 16-key block matching the score
  // registers (see the absorbed kernel)
  uint32_t k_lane[2], v_lane[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) k_lane[e] = kNHalf * ((l >> 4) & 1) + 256 * hl + 16 * ((l & 15) ^ swz(2 * e + hl));
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int g = l >> 4, jl = l & 15;
    const int tok = 4 * (g >> 1) + 8 * r + (jl >> 2);
    const int cl = 2 * (g & 1) + ((jl >> 1) & 1);
    v_lane[r] = (16 * cl + (tok ^ swz(cl))) * 16 + 8 * (jl & 1);
  }

  const int nsteps = (nk + 31) / 32;
#pragma unroll
  for (int it = 0; it < kNB - 1; ++it)
    if (it < nsteps) issue(it);
  for (int i = 0; i < nsteps; ++i) {
    // step i landed: at most the later issued steps (5 loads each) in flight
    const int later = min(nsteps - 1 - i, kNB - 2);
    if (later >= 2) wait_vm_n<10>();
    else if (later == 1) wait_vm_n<5>();
    else wait_vm_n<0>();
    // (a barrier without the memory fence of __syncthreads, which would also
    // wait for the loads still in flight)
    __builtin_amdgcn_s_barrier();
    if (i + kNB - 1 < nsteps) issue(i + kNB - 1);
    const uint32_t buf = ring_lds + (i % kNB) * kNStep;
    // scores
    f32x16 S = {};
#pragma unroll
    for (int ks = 0; ks < kQks; ++ks) {
      const bf16x8 kop = *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)(buf + k_lane[ks & 1] + 512 * ks);
      S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, q[ks], S, 0, 0, 0);
    }
    // mask (key j0 + 32i + tok(r) visible iff below lim), running max
    const int rel = lim - j0 - 32 * i - 4 * hl;
    float x[16];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      x[r] = (8 * (r >> 2) + (r & 3) < rel) ? S[r] * sl2 : -INFINITY;
      mx = fmaxf(mx, x[r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);
    if (__builtin_amdgcn_ballot_w64(m_new > m) != 0) {
      const float alpha = (m_new > m) ? __builtin_amdgcn_exp2f(m - m_new) : 1.f;  // exp2(-inf) = 0
      lsum *= alpha;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) acc[cb] *= alpha;
      m = m_new;
    }
    const float mb = m == -INFINITY ? 0.f : m;
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      x[r] = __builtin_amdgcn_exp2f(x[r] - mb);
      s += x[r];
    }
    lsum += s;
    bf16x8 pv[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const u32x2 lo = cvt_bf16x4(f32x4{x[8 * kb], x[8 * kb + 1], x[8 * kb + 2], x[8 * kb + 3]});
      const u32x2 hi = cvt_bf16x4(f32x4{x[8 * kb + 4], x[8 * kb + 5], x[8 * kb + 6], x[8 * kb + 7]});
      pv[kb] = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
    }
    // values: O^T[cb] += V^T[cb, kb] P^T[kb]
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const uint32_t off = buf + kb * kNHalf + 1024 * (6 + cb);
        const bf16x8 vop = join8(
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(uintptr_t)(off + v_lane[0])),
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(uintptr_t)(off + v_lane[1])));
        acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pv[kb], acc[cb], 0, 0, 0);
      }
  }

  const float ltot = lsum + __shfl_xor(lsum, 32);
  if (!row_ok) return;
  if (p.last) {
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[cb][4 * q4 + e] * inv;
        *(f32x4*)(p.out + qrow * kDV + 32 * cb + 8 * q4 + 4 * hl) = v;
      }
    if (hl == 0 && p.lse)
      p.lse[qrow] = ltot > 0.f ? (m + __builtin_amdgcn_logf(ltot)) * 0.69314718055994530942f : -INFINITY;
  } else {
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[cb][4 * q4 + e];
        *(f32x4*)(p.o_state + qrow * kDV + 32 * cb + 8 * q4 + 4 * hl) = v;
      }
    if (hl == 0) {
      p.m_state[qrow] = m;
      p.l_state[qrow] = ltot;
    }
  }
}

hipError_t launch_gather(const NormalParams& prm, hipStream_t st) {
  const long long rows = (long long)prm.B * prm.chunk;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, prm);
  return hipGetLastError();
}

hipError_t launch_mha(const NormalParams& prm, hipStream_t st) {
  const long long units = (long long)prm.B * prm.H * ((prm.T + 127) / 128);
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL(mha_kernel, dim3((unsigned)units), dim3(256), 0, st, prm);
  return hipGetLastError();
}

}  // namespace mla
