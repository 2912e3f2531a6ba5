// Device helpers shared by the gfx950 kernels of the absorbed MLA decode path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// Geometry fixed by this library ("MLA in full detail", shapes table: kv_lora_rank 512,
// rope 64, nope 128, v_head 128).
constexpr int kR = 512;                 // latent width
constexpr int kDR = 64;                 // rope width
constexpr int kRow = kR + kDR;          // 576 values per cached row
constexpr int kRowBytes = kRow * 2;     // 1152 bytes
constexpr int kRowChunks = kRowBytes / 16;  // 72 chunks of 16 bytes
constexpr int kDN = 128;
constexpr int kDV = 128;
constexpr int kTile = 16;               // tokens per KV tile
constexpr int kTileBytes = kTile * kRowBytes;  // 18432
constexpr int kRowsPerWG = 128;         // query rows (t, h) handled by one workgroup

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// float -> bf16 bits, round to nearest even (inputs here are finite or +-inf/NaN-free).
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf2f(uint16_t h) {
  return __builtin_bit_cast(float, ((uint32_t)h) << 16);
}
// two floats -> packed bf16x2 (low = a), nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
}

// four floats -> four bf16 with the hardware conversion (v_cvt_pk_bf16_f32,
// round to nearest even), packed two per dword, element 0 in the low half.
__device__ __forceinline__ u32x2 cvt_bf16x4(f32x4 v) {
  return __builtin_bit_cast(u32x2, __builtin_convertvector(v, bf16x4));
}

// Operands are assembled from whole vectors (bit casts and shuffles), never by
// inserting bf16 elements one at a time: the element-wise form has been seen to
// compile to code that drops half of the values.
__device__ __forceinline__ bf16x8 join8(s16x4 lo, s16x4 hi) {
  return __builtin_shufflevector(__builtin_bit_cast(bf16x4, lo), __builtin_bit_cast(bf16x4, hi), 0, 1,
                                 2, 3, 4, 5, 6, 7);
}
// eight floats -> eight bf16 (nearest even), element i of the result = input i
__device__ __forceinline__ bf16x8 pack8(f32x4 lo, f32x4 hi) {
  u32x4 u;
  u[0] = pack_bf16x2(lo[0], lo[1]);
  u[1] = pack_bf16x2(lo[2], lo[3]);
  u[2] = pack_bf16x2(hi[0], hi[1]);
  u[3] = pack_bf16x2(hi[2], hi[3]);
  return __builtin_bit_cast(bf16x8, u);
}

// 16-byte global -> LDS copy for every lane of the wave: lane i of the wave
// writes LDS bytes [lds_addr + 16 i, lds_addr + 16 i + 16).  Issued as inline
// assembly so that the compiler's wait-count pass does not serialise later
// LDS reads behind it; the caller orders it with explicit vmcnt waits.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(lds_addr)
               : "memory");
}

// Same copy with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane
// offset (the instruction's scalar-base form): lane i reads base + voff_i.  The
// instruction's immediate offset is left at 0: for these loads it displaces
// the LDS destination as well as the global address.
__device__ __forceinline__ void dma16s(uint32_t voff, const void* base, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base),
               "s"(lds_addr)
               : "memory");
}

// 16 bytes per lane from a 64-bit per-lane address into LDS at lds_addr + 16 * lane.
// The immediate offset OFF moves the global address and the LDS destination
// alike, so M0 is set to lds_addr - OFF (one address register serves all the
// 128-byte column steps of a row).
template <int OFF>
__device__ __forceinline__ void dma16v(const void* addr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off offset:%2" ::"v"(addr),
               "s"(lds_addr - OFF), "n"(OFF)
               : "memory");
}

// 4 bytes per lane (scalar base + vector offset) into LDS at lds_addr + 4 * lane.
__device__ __forceinline__ void dma4s(uint32_t voff, const void* base, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(base),
               "s"(lds_addr)
               : "memory");
}

// 4 bytes per lane from a 64-bit per-lane address into LDS at lds_addr + 4 * lane.
__device__ __forceinline__ void dma4v(const void* addr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(addr), "s"(lds_addr)
               : "memory");
}

__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 16-byte global store with the non-temporal (streaming) hint, for output
// written once at the end of a launch and read only by a later one.  The
// compiler has no equivalent form on this target (its nontemporal store keeps
// the default policy).  The store counts on the vector-memory counter like any
// other, so the compiler's own waits stay conservative around it.  The data
// of a store wider than 8 bytes is read from its VGPRs after the instruction
// issues: a vector instruction that writes them next needs wait states between
// the two, which the compiler provides for its own stores (by its schedule or an
// s_nop) but cannot for one inside inline assembly -- hence the s_nop in the
// statement.
__device__ __forceinline__ void store16_nt(void* dst, u32x4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off nt\n\ts_nop 1" ::"v"(dst), "v"(v) : "memory");
}

__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// Workgroup barrier without the memory fence that __syncthreads() adds (the
// fence would also wait for the in-flight tile prefetches).
__device__ __forceinline__ void barrier() { __builtin_amdgcn_s_barrier(); }

}  // namespace mla
