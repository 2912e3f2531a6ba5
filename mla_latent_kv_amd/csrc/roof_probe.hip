// Practical roofs of the part under its power limit, for the benchmark's
// context lines (not part of the decode path; built into libmla_probe.so).
//
// One workgroup of four waves per CU (160 KB of LDS each, as the decode
// kernel).  Each wave runs `iters` groups of four independent bf16 MFMAs
// 32x32x16 and, depending on the mode:
//   mode 0  the MFMAs only;
//   mode 1  1 KB direct-to-LDS loads from HBM only (`iters` of them);
//   mode 2  the MFMAs plus one 1 KB load after every `ratio` MFMAs
//           (floor(4 iters / ratio) loads: 32768 * ratio / 1024 FLOP per byte);
//   mode 3  as mode 2, plus one 16-byte-per-lane LDS read (1 KB per wave)
//           feeding each MFMA's B operand, read one group ahead (about the
//           decode kernel's LDS operand traffic per MFMA);
//   mode 4  the MFMAs with their LDS operand reads, no HBM stream.
// In modes 3 and 4 each wave first fills its 32 KB LDS window from `src`, so
// with random data in `src` the MFMA operands change from one instruction to
// the next as they do in the decode kernel (the matrix cores draw more power
// on toggling operands than on constant ones, modes 0 and 2).
// Workgroup g streams its own slice [g * slice, (g + 1) * slice) of `src`
// (at most 24 loads in flight per wave).  The work per launch is known
// exactly, so rate = work / duration; a long run of launches, sampled for
// clock and power, gives the MFMA rate and the HBM rate the part sustains at
// its power limit for a given FLOP/byte mix.
//
// A second kernel, pipe_kernel, is the decode kernel's data flow with its
// arithmetic taken out, to split the decode's time into parts: per work unit
// (one workgroup of four waves, one per CU), 32-token tiles of 36 KB read from
// pages of 64 rows of 1152 bytes placed anywhere in the pool (a page list per
// unit), direct-to-LDS through a ring of four tiles issued three steps ahead,
// each wave waiting for its own loads of the step and one barrier per step,
// as the decode kernel does.  Flags add, one at a time:
//   1  68 bf16 MFMAs 32x32x16 per wave and step, B operands (1 KB per MFMA)
//      read from the current tile one group of four ahead;
//   2  at the end, the unit's 128 KB output block written from LDS to `out`
//      (the decode's split partials), 32 stores of 16 bytes per thread;
//   4  with 2: those stores with the streaming hint.
//
// extern "C" int mla_probe_launch(const void* src, size_t slice, int grid, int iters,
//                                 int mode, int ratio, float* sink, void* stream)
//   src: device buffer of at least grid * slice bytes, slice a multiple of 4 KB
//   and at least 32 KB; mode 0..4; iters even; ratio 1..64; sink: 256 floats (never
//   written for these inputs; keeps the results live).  Returns a hipError_t.
// extern "C" int mla_pipe_probe_launch(const void* pool, size_t pool_pages, const int* pages,
//                                      int units, int pages_per_unit, int flags, void* out,
//                                      float* sink, void* stream)
//   pool: pool_pages pages of 73,728 bytes; pages: units x pages_per_unit page
//   ids, each below pool_pages (not checked on the device); 2 * pages_per_unit
//   steps per unit; out: units x 128 KB (written only with flag 2); flags 0..7.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void dma16s(uint32_t voff, const void* base, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base),
               "s"(lds_addr)
               : "memory");
}

constexpr int kLds = 160 * 1024;

__global__ __launch_bounds__(256, 1) void roof_kernel(const uint8_t* src, size_t slice, int iters, int mode,
                                                      int ratio, float* sink) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds;
  const uint32_t win = lds_base + (uint32_t)(w * 32768);   // this wave's 32 KB of the first 128 KB
  f32x16 a0 = {}, a1 = {}, a2 = {}, a3 = {};
  bf16x8 x, y;
  for (int e = 0; e < 8; ++e) {
    x[e] = (__bf16)(0.001f * (l + e));
    y[e] = (__bf16)(0.002f * (l - e));
  }
  const uint8_t* base = src + (size_t)blockIdx.x * slice;
  const uint32_t nblk = (uint32_t)(slice / 1024);   // >= 4
  uint32_t blk = (uint32_t)w;
  uint32_t slot = 0;
  auto load = [&]() {
    dma16s(blk * 1024u + 16u * (uint32_t)l, base, __builtin_amdgcn_readfirstlane(win + slot * 1024u));
    slot = (slot + 1) & 31u;
    blk += 4;
    if (blk >= nblk) blk = (uint32_t)w;
    asm volatile("s_waitcnt vmcnt(24)" ::: "memory");
  };
  int credit = 0;
  auto loads_due = [&]() {
    credit += 4;
    while (credit >= ratio) {
      credit -= ratio;
      load();
    }
  };
  auto group = [&](const bf16x8& b0, const bf16x8& b1, const bf16x8& b2, const bf16x8& b3) {
    a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, b0, a0, 0, 0, 0);
    a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, b1, a1, 0, 0, 0);
    a2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, b2, a2, 0, 0, 0);
    a3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, b3, a3, 0, 0, 0);
  };
  auto rd16 = [&](uint32_t off) {
    return *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)(win + (off & 32767u) + 16u * (uint32_t)l);
  };
  if (mode >= 3) {   // fill this wave's window with 32 KB of `src`
    for (int k = 0; k < 32; ++k) load();
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  if (mode == 0) {
    for (int i = 0; i < iters; ++i) group(y, y, y, y);
  } else if (mode == 1) {
    for (int i = 0; i < iters; ++i) load();
  } else if (mode == 2) {
    for (int i = 0; i < iters; ++i) {
      group(y, y, y, y);
      loads_due();
    }
  } else {
    // two groups per iteration: group A uses ya (while yb is read), group B yb;
    // mode 4 issues no loads (ratio is ignored)
    if (mode == 4) ratio = 1 << 30;
    uint32_t off = 0;
    bf16x8 ya0 = rd16(off), ya1 = rd16(off + 1024), ya2 = rd16(off + 2048), ya3 = rd16(off + 3072);
    off += 4096;
    for (int i = 0; i < iters; i += 2) {
      const bf16x8 yb0 = rd16(off), yb1 = rd16(off + 1024), yb2 = rd16(off + 2048), yb3 = rd16(off + 3072);
      group(ya0, ya1, ya2, ya3);
      loads_due();
      ya0 = rd16(off + 4096);
      ya1 = rd16(off + 5120);
      ya2 = rd16(off + 6144);
      ya3 = rd16(off + 7168);
      group(yb0, yb1, yb2, yb3);
      loads_due();
      off += 8192;
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  float s = 0.f;
  for (int e = 0; e < 16; ++e) s += a0[e] + a1[e] + a2[e] + a3[e];
  if (s == 1.2345e30f) sink[threadIdx.x] = s;   // never true for these inputs: keeps the MFMAs live
}

constexpr int kRowB = 1152, kTileB = 32 * kRowB, kHalfB = kTileB / 2, kPageB = 2 * kTileB;
constexpr int kRing = 4;   // tiles in the LDS ring (147,456 bytes)

__global__ __launch_bounds__(256, 1) void pipe_kernel(const uint8_t* pool, const int* pages, int ppu, int flags,
                                                      uint8_t* out, float* sink) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63;
  const int hw = w >> 1, pw = w & 1;   // wave w loads 9 of the 18 1 KB chunks of half hw of a tile
  const uint32_t ring = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds;
  // page ids through the constant address space: scalar loads, which the
  // compiler waits for on their own counter (a vector load's wait would also
  // wait for the tile loads in flight)
  typedef const __attribute__((address_space(4))) int cint;
  const cint* pg = (const cint*)(uintptr_t)(pages + (size_t)blockIdx.x * ppu);
  const int steps = 2 * ppu;
  auto issue = [&](int it) {
    const int page = pg[min(it >> 1, ppu - 1)];   // past the last step: the last page again
    const uint8_t* base = pool + (size_t)page * kPageB;
    const uint32_t dst = ring + (uint32_t)((it % kRing) * kTileB + hw * kHalfB);
#pragma unroll
    for (int n = 0; n < 9; ++n) {
      const int c = pw + 2 * n;
      dma16s((uint32_t)((it & 1) * kTileB + hw * kHalfB + c * 1024 + 16 * l), base,
             __builtin_amdgcn_readfirstlane(dst + c * 1024));
    }
  };
  f32x16 a0 = {}, a1 = {};
  bf16x8 x;
  for (int e = 0; e < 8; ++e) x[e] = (__bf16)(0.001f * (l + e));
  for (int it = 0; it < kRing - 1; ++it) issue(it);
  for (int it = 0; it < steps; ++it) {
    asm volatile("s_waitcnt vmcnt(18)" ::: "memory");   // this wave's 9 loads of step it (18 later ones in flight)
    __syncthreads();                                      // every wave's share of tile it is in LDS
    issue(it + kRing - 1);                                // into the buffer of step it - 1, read by all
    if (flags & 1) {
      // reads and waits in inline assembly: plain reads are sunk to their MFMAs
      // by the compiler, one LDS latency each
      const uint32_t t = ring + (uint32_t)((it % kRing) * kTileB) + 16u * l;
      bf16x8 y[2][4];
      auto rd4 = [&](int g, int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          asm volatile("ds_read_b128 %0, %1" : "=v"(y[buf][e]) : "v"(t + (uint32_t)(((4 * g + e) * 1024) % kTileB)));
      };
      rd4(0, 0);
#pragma unroll
      for (int g = 0; g < 17; ++g) {
        const int cur = g & 1;
        if (g + 1 < 17) {
          rd4(g + 1, cur ^ 1);
          asm volatile("s_waitcnt lgkmcnt(4)" : "+v"(y[cur][0]), "+v"(y[cur][1]), "+v"(y[cur][2]), "+v"(y[cur][3]));
        } else {
          asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(y[cur][0]), "+v"(y[cur][1]), "+v"(y[cur][2]), "+v"(y[cur][3]));
        }
        a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y[cur][0], a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y[cur][1], a1, 0, 0, 0);
        a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y[cur][2], a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y[cur][3], a1, 0, 0, 0);
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (flags & 2) {
    __syncthreads();
    uint8_t* dst = out + (size_t)blockIdx.x * 131072;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      u32x4 v[16];
#pragma unroll
      for (int k = 0; k < 16; ++k)
        v[k] = *(const __attribute__((address_space(3))) u32x4*)(uintptr_t)(ring + (uint32_t)(16 * (threadIdx.x + 256 * (16 * g + k))));
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        u32x4* d = (u32x4*)(dst + 16 * (threadIdx.x + 256 * (16 * g + k)));
        // (the data of a store wider than 8 bytes is read after issue: the
        // s_nop keeps the next vector instruction from overwriting it first)
        if (flags & 4) asm volatile("global_store_dwordx4 %0, %1, off nt\n\ts_nop 1" ::"v"(d), "v"(v[k]) : "memory");
        else *d = v[k];
      }
    }
  }
  float s = 0.f;
  for (int e = 0; e < 16; ++e) s += a0[e] + a1[e];
  if (s == 1.2345e30f) sink[threadIdx.x] = s;   // never true for these inputs: keeps the MFMAs live
}

}  // namespace

extern "C" int mla_pipe_probe_launch(const void* pool, size_t pool_pages, const int* pages, int units,
                                     int pages_per_unit, int flags, void* out, float* sink, void* stream) {
  if (!pool || !pages || !sink || pool_pages < 1 || units < 1 || pages_per_unit < 1 || flags < 0 || flags > 7 ||
      ((flags & 2) && !out))
    return (int)hipErrorInvalidValue;
  const int lds = kRing * kTileB;
  hipError_t e = hipFuncSetAttribute((const void*)pipe_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return (int)e;
  hipLaunchKernelGGL(pipe_kernel, dim3(units), dim3(256), lds, (hipStream_t)stream, (const uint8_t*)pool, pages,
                     pages_per_unit, flags, (uint8_t*)out, sink);
  return (int)hipGetLastError();
}

extern "C" int mla_probe_launch(const void* src, size_t slice, int grid, int iters, int mode, int ratio,
                                float* sink, void* stream) {
  if (!src || !sink || grid < 1 || iters < 2 || iters % 2 || mode < 0 || mode > 4 || ratio < 1 || ratio > 64 ||
      slice < 32768 || slice % 4096)
    return (int)hipErrorInvalidValue;
  hipError_t e = hipFuncSetAttribute((const void*)roof_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
  if (e != hipSuccess) return (int)e;
  hipLaunchKernelGGL(roof_kernel, dim3(grid), dim3(256), kLds, (hipStream_t)stream, (const uint8_t*)src, slice,
                     iters, mode, ratio, sink);
  return (int)hipGetLastError();
}
