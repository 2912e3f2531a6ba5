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
// query rows; both GEMMs run on the matrix cores in bf16 with fp32
// accumulation.  The softmax is accumulated over KV tiles against one
// reference maximum per row and normalised once at the end (M5.8 0x0A: tiles
// are never normalised independently).
//
// Workgroup layout (256 threads = 4 waves of 64, one workgroup per CU).  Wave w
// owns query rows [32w, 32w + 32) for the scores and the softmax, and latent
// columns [128w, 128w + 128) of all 128 rows for the value GEMM:
//  * KV rows stream HBM -> LDS with direct-to-LDS loads in steps of 32 tokens
//    (two 16-row halves, 36 KB) into a ring of NB step buffers; waves 0-1 load
//    the first half of every step, waves 2-3 the second.
//  * Scores: S^T[32 tok x 32 rows] = K[32 x 576] q~^T with 36 32x32x16 MFMAs;
//    K comes from LDS (ds_read_b128), the query rows live in registers.  A lane
//    then holds 16 scores of one query row.
//  * Softmax: log2 domain against a per-row reference m_ref (the max of the
//    row's first step with a visible key), so exponentials are bounded by
//    2^kLazy and the fp32 accumulator is never rescaled.  Each lane checks its
//    own scores against m_ref + kLazy; only when one exceeds it is m_ref
//    raised and the work unit replayed from its first step (exact for any
//    finite scores; never taken for scores of ordinary magnitude).
//  * Values: O^T[128 cols x 128 rows] += V^T P^T with 32 32x32x16 MFMAs per
//    step (4 column blocks x 4 row blocks x 2 token blocks; 256 accumulator
//    registers).  The score accumulator layout is exactly the P^T operand
//    layout (with the token order inside each 16-token block taken as the
//    MFMA's k order and V read in the same order): a wave uses its own rows'
//    probabilities straight from registers and writes them to a 16 KB LDS
//    double buffer for the other waves.  V comes from LDS through transposing
//    reads (ds_read_b64_tr_b16), each operand read once and used for four row
//    blocks.
//  * Software pipeline, one barrier per 32-token step: the value MFMAs of step
//    i and the score MFMAs of step i+1 form one MFMA stream (a compile-time
//    slot table); the softmax of step i+1 runs on the vector ALU under the
//    last value MFMAs; LDS operand reads and this wave's load instructions
//    for step i+NB-1 sit in between.  With one wave per SIMD every non-MFMA
//    instruction competes for the same issue slots, so the loop keeps them
//    few (68 MFMAs, about 60 LDS, 160 vector and 60 scalar instructions per
//    32 tokens).
//
// Variants (template flags): split partials or the final result, fp32 or bf16
// output, sparse index rows in place of the block table (M5.8 0x0B), and FP8
// rows (656 bytes, M5.8 0x0B) whose latent codes each wave dequantizes into
// the bf16 tile layout below, so that everything downstream is shared.
//
// LDS layout of a 16-row half (chunk-major): the 16-byte chunk c (c < 72) of
// row t is stored at chunk position 16c + (t ^ g(c & 3)), g = (0, 12, 8, 4).
// The K reads (32 rows x 2 chunks) and the transposing V reads are then both
// free of bank conflicts on gfx950 (measured with SQ_LDS_BANK_CONFLICT); the
// direct-to-LDS loads write 1 KB contiguous.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace mla {

constexpr float kLazy = 64.0f;               // log2-domain growth of the max tolerated before a replay
constexpr int kStepTok = 32;                 // tokens per pipeline step
constexpr int kStepBytes = 2 * kTileBytes;   // two 16-row halves
constexpr int kQk = kRow / 16;               // 36 score MFMAs per step (k = 16 each)
constexpr int kPv = 2 * (kR / 32);  // value MFMAs per wave and step (2 token blocks x 4 row blocks x 4 column blocks)

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_lgkm() {
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N) : "memory");
}

// Hide a value's known bits from the compiler, so that address arithmetic on it
// stays base + constant (folded into the LDS instruction's offset field).
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Compile-time loop: f(integral_constant<int, S>) for S = B .. E-1.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// v of lane l and of lane l ^ 32.  v_permlane32_swap exchanges the upper half
// of its first operand with the lower half of its second; it reads its
// operands two wait states after a VALU write at the earliest, hence the s_nop.
// (Inline assembly: the builtin has been seen to compile to code that reads
// only one of the two results.)
__device__ __forceinline__ void xpair32(float v, float& a, float& b) {
  a = v;
  b = v;
  asm volatile("s_nop 2\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
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

// Value-phase MFMA with its accumulator pinned to AGPRs (the 512x32 fp32 O^T
// block of a wave fills all 256 of them); written as inline assembly so that
// the score accumulator, which the softmax reads, stays in VGPRs.  The operands
// come straight from LDS reads and register conversions (the compiler's wait
// counts cover the reads); the accumulator is next touched by VALU code only
// after mfma_drain().
__device__ __forceinline__ void mfma_pv(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// Wait states between the last value MFMA and any VALU access to its
// accumulator (a 16-pass XDL result needs at most 18).
__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// Row swizzle of the tile layout and the position (in 16-byte units) of chunk c
// of half-tile row t.
__device__ __forceinline__ int tile_swz(int c) { return (-4 * c) & 12; }
__device__ __forceinline__ int tile_pos(int c, int t) { return 16 * c + (t ^ tile_swz(c & 3)); }

// ---- stream schedule of one step: 68 MFMA slots ----
// slots 0-3: value MFMAs v = 0..3; slots 4-43: the 36 score MFMAs ks = 0..35
// with value MFMAs v = 4..7 after every ninth; slots 44-67: value MFMAs
// v = 8..31.  The softmax of the next step (about 70 vector instructions, 16
// of them quarter-rate exponentials) is spread over slots 45-64, so that it
// fits in the vector-ALU time the matrix core leaves free.
struct Slot {
  int qk;  // score MFMA k-step or -1
  int pv;  // value MFMA index or -1
};
constexpr int kSlots = kQk + kPv;
constexpr Slot slot_of(int s) {
  if (s < 4) return Slot{-1, s};
  if (s < 44) {
    const int x = s - 4;  // 40 slots: nine score MFMAs, then one value MFMA (x4)
    return (x % 10 == 9) ? Slot{-1, 4 + x / 10} : Slot{x / 10 * 9 + x % 10, -1};
  }
  return Slot{-1, 8 + (s - 44)};
}
// softmax stages of the next step, by slot
constexpr int kSmLoad = 45, kSmCheck = 46, kSmRef = 47, kSmExp0 = 48, kSmSum = 64, kSmPack = 65;
// sparse mode: slot at which the row ids of a later step are read back (after
// the last load instruction of the step)
constexpr int kSpIds = 57;
// value MFMA v: token block kb = v >> 4 (16 tokens), row block ri = (v >> 2) & 3
// (the rows of wave w + ri), this wave's column block cb = v & 3

// slots at which this wave issues its 9 load instructions of a step
constexpr int kDmaSlot0 = 0, kDmaStride = 7;
constexpr int dma_part_at(int s) {
  return (s >= kDmaSlot0 && (s - kDmaSlot0) % kDmaStride == 0 && (s - kDmaSlot0) / kDmaStride < 9)
             ? (s - kDmaSlot0) / kDmaStride
             : -1;
}
static_assert(kDmaSlot0 + 8 * kDmaStride < kSpIds && kSpIds < kSmPack,
              "sparse ids are read after the step's last load and before the probability writes");

// ---- FP8 cache rows (M5.8 0x0B, "Exact 656-byte FP8 row"): 512 E4M3 codes
// (byte c = latent column c), four fp32 scales (scale g covers columns
// [128g, 128g + 128)), 64 bf16 rope values.  The latent is dequantized to bf16
// (code x scale, rounded to nearest even) into the same tile layout as a bf16
// row, so the attention itself is unchanged.
constexpr int kF8Row = 656;
constexpr int kF8Scales = 512;   // byte offset of the scales in a row
constexpr int kF8Rope = 528;     // byte offset of the rope values
// Staging buffer of one step's codes and scales: codes [half][wave parity]
// [4 load instructions] x 1 KB, then one 256-byte copy of its half's scales
// per wave.
constexpr int kStgCodes = 2 * 2 * 4 * 1024;
constexpr int kStgBytes = kStgCodes + 4 * 256;
// slots of the six FP8 load instructions of a step (rope of the tile two
// ahead, then codes and scales of the tile three ahead), the wait for the
// previous step's loads, and the conversion of the tile two ahead: unit n
// (one 1 KB code block) is read at kF8Cvt0 + kF8CvtStride n and written out in
// two halves, 3 and 5 slots later
constexpr int kF8Wait = 11, kF8Cvt0 = 12, kF8CvtStride = 6;
constexpr int f8_part_at(int s) { return (s <= 10 && s % 2 == 0) ? s / 2 : -1; }
// conversion work at slot s: 4 n + phase (0 read unit n, 1 and 2 its two output chunks), or -1
constexpr int f8_cvt_at(int s) {
  if (s < kF8Cvt0) return -1;
  const int x = s - kF8Cvt0, n = x / kF8CvtStride, r = x % kF8CvtStride;
  if (n >= 4) return -1;
  return r == 0 ? 4 * n : r == 3 ? 4 * n + 1 : r == 5 ? 4 * n + 2 : -1;
}
static_assert(kF8Cvt0 + 3 * kF8CvtStride + 5 < 4 + 40, "conversion stays among the score MFMAs");

// dma16s with the instruction's immediate offset OFF, which moves the global
// address and the LDS destination alike (so M0 = lds_addr - OFF): one offset
// register serves several 1 KB blocks of a row group.
template <int OFF>
__device__ __forceinline__ void dma16s_imm(uint32_t voff, const void* base, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 offset:%3" ::"v"(voff), "s"(base),
               "s"(lds_addr - OFF), "n"(OFF)
               : "memory");
}

// four E4M3 codes (one dword, code i in byte i) times scale -> four bf16 (two dwords)
__device__ __forceinline__ u32x2 f8x4_to_bf16(uint32_t codes, float scale) {
  const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes, false);
  const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes, true);
  return cvt_bf16x4(f32x4{a[0] * scale, a[1] * scale, b[0] * scale, b[1] * scale});
}

// Key count of work sequence bb: its length, or in sparse mode the valid
// prefix of its index row (sequence bb / sp_T's topk_length, at most topk).
template <bool SPARSE>
__device__ __forceinline__ int unit_keys(const DecodeParams& p, int bb) {
  if constexpr (SPARSE) {
    if (!p.topk_length) return p.topk;
    return min(max(p.topk_length[bb / p.sp_T], 0), p.topk);
  } else {
    return p.seqlens[bb];
  }
}

// Timeline build (MLA_DECODE_TIMELINE, a separate library): every wave of the
// first 2048 workgroups stamps the 100 MHz real-time counter at eight points
// of its unit into g_timeline[workgroup][wave][point] -- 0 unit start, 1 query
// and first loads issued, 2 first tile landed, 3 last step done, 4 partial
// state final, 5 output block staged, 6 output stores issued, 7 stores done;
// mla_timeline_read copies the array (the last launch's stamps) to the host.
// In the ordinary build the points compile to nothing.
#ifdef MLA_DECODE_TIMELINE
__device__ unsigned long long g_timeline[2048 * 4 * 8];
#define MLA_TS(k)                                                                                  \
  do {                                                                                             \
    if (blockIdx.x < 2048) g_timeline[((size_t)blockIdx.x * 4 + w) * 8 + (k)] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#define MLA_TS_DRAIN() asm volatile("s_waitcnt vmcnt(0)" ::: "memory")
#else
#define MLA_TS(k) \
  do {            \
  } while (0)
#define MLA_TS_DRAIN() \
  do {                 \
  } while (0)
#endif

template <int NB, bool SPLIT, bool OUT_F32, bool SPARSE, bool FP8>
__global__ __launch_bounds__(256, 1) void decode_kernel(DecodeParams p) {
  static_assert(!FP8 || NB == 3, "FP8 ring: the tiles of steps i, i+1 and the one being converted");
  constexpr int kRB = FP8 ? kF8Row : kRowBytes;  // bytes per cached row
  // step ring (FP8: followed by two code staging buffers); after the last step
  // it is reused to stage the 128 KB output block
  constexpr int kRingUse = NB * kStepBytes + (FP8 ? 2 * kStgBytes : 0);
  constexpr int kRingBytes = kRingUse > 128 * 1024 ? kRingUse : 128 * 1024;
  __shared__ __attribute__((aligned(16))) uint8_t tiles[kRingBytes];
  // probabilities of all 128 rows, two steps: [step & 1][kb][row block][lane] x 16 B
  __shared__ __attribute__((aligned(16))) uint8_t pbuf[2 * 2 * 4 * 64 * 16];
  // FP8 rows selected by index: the row ids of this wave's half for four
  // steps, [wave][step & 3][16] int32 (1 KB of the 2 KB the FP8 ring leaves)
  __shared__ __attribute__((aligned(16))) int f8_idbuf[SPARSE && FP8 ? 4 * 4 * 16 : 1];

  const int w = wave_id();
  const int l = lane_id();
  const int hl = l >> 5;  // lane half: token sub-block 4*hl of each 8-token group

  // ---- work unit.  Units u = item * n_rg + rg are dealt to the XCDs in
  // contiguous ranges (workgroup i runs on XCD i % 8), so the splits of one
  // sequence share an L2 and re-read its query rows from there.
  const int n_units = (SPLIT && p.work) ? *p.n_items * p.n_rg : p.n_units;
  const int per_xcd = (n_units + 7) >> 3;
  const int kx = blockIdx.x >> 3;
  if (kx >= per_xcd) return;
  const int u = (blockIdx.x & 7) * per_xcd + kx;
  if (u >= n_units) return;
  MLA_TS(0);
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
      const int Lb = unit_keys<SPARSE>(p, b);
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
    j1 = unit_keys<SPARSE>(p, b);
    slot = b;
  }
  // work-unit scalars are wave-uniform: keep them in scalar registers
  b = __builtin_amdgcn_readfirstlane(b);
  j0 = __builtin_amdgcn_readfirstlane(j0);
  j1 = __builtin_amdgcn_readfirstlane(j1);
  slot = __builtin_amdgcn_readfirstlane(slot);
  const int L = __builtin_amdgcn_readfirstlane(unit_keys<SPARSE>(p, b));
  const int T = p.T, H = p.H, TH = T * H;
  const int P = p.page_size;
  const int row0 = rg * kRowsPerWG;

  // ---- this lane's query row (lanes l and l ^ 32 share it) ----
  // q[ks] holds elements 16ks + 8hl .. +7 of [q~ || q_pe] (the B operand of the
  // score MFMA).  Key j of the row is visible iff j < lim.  Padding rows past
  // T*H load the query of the last real row (so every load is unconditional),
  // see every key of the range and are never stored.
  const int rloc = 32 * w + (l & 31);
  const int grow_ = row0 + rloc;
  bf16x8 q[kQk];
  int lim = j1;
  const int qrow = min(grow_, TH - 1);
  {
    const int t = qrow / H;
    if (grow_ < TH) lim = min(L - T + t + 1, j1);
  }
  const uint16_t* ql = p.q_lat + ((size_t)b * TH + qrow) * kR + 8 * hl;
  const uint16_t* qp = p.q_pe + ((size_t)b * TH + qrow) * kDR + 8 * hl;
  // score register r of step it is token j0 + 32 it + tok(r) + 4 hl with
  // tok(r) = 8 (r >> 2) + (r & 3): visible iff tok(r) < dd - 32 it
  const int dd = lim - j0 - 4 * hl;

  const int nsteps = (j1 - j0 + kStepTok - 1) / kStepTok;
  const uint32_t tiles_lds = lds_addr_of(tiles);
  const uint8_t* cache = (const uint8_t*)p.cache;
  const int32_t* bt_row = p.block_table + (size_t)b * p.max_blocks;

  // ---- loads.  Wave w loads half hw = w >> 1 of every step (16 rows, 18 load
  // instructions shared by waves 2hw and 2hw+1: instruction kk = (w & 1) + 2n,
  // n < 9).  Instruction kk fills chunk positions [64kk, 64kk + 64) of the
  // half: lane l brings chunk 4kk + (l >> 4) of row (l & 15) ^ g(l >> 4).
  // Physical pages come from a window of 64 block-table entries held one per
  // lane; the page of the next half-tile is tracked incrementally.
  const int hw = w >> 1;
  const uint32_t dma_voff = ((l & 15) ^ tile_swz(l >> 4)) * kRowBytes + 16 * (l >> 4) + 64 * (w & 1);
  const int rsw = (l & 15) ^ tile_swz(l >> 4);  // sparse: row of the half this lane loads
  const uint32_t dma_coff = 16 * (l >> 4) + 64 * (w & 1);
  // FP8 rows selected by index: the rows of the half whose codes, scales and
  // rope values this lane loads (the lane layout of the FP8 loads below)
  const int f8_rc = l & 15, f8_rs = l >> 2, f8_rr = (l & 15) ^ tile_swz(l >> 4);
  // FP8 rows, per wave and step: the rope values of its half's 16 rows straight
  // into the tile (lane l: rope chunk 4 pw + (l >> 4) of row (l & 15) ^ g(l >> 4),
  // i.e. tile chunk 64 + 4 pw + (l >> 4)); four 1 KB code blocks into the
  // staging buffer (instruction n, lane l: codes 16 cp .. 16 cp + 15 of row
  // l & 15, cp = 16 pw + 4 n + (l >> 4)); the half's 64 scales (lane l: scale
  // l & 3 of row l >> 2).
  const int pw = w & 1;
  const uint32_t f8_rope_voff = ((l & 15) ^ tile_swz(l >> 4)) * kF8Row + kF8Rope + 64 * pw + 16 * (l >> 4);
  const uint32_t f8_code_voff = (l & 15) * kF8Row + 256 * pw + 16 * (l >> 4);
  const uint32_t f8_scale_voff = (l >> 2) * kF8Row + kF8Scales + 4 * (l & 3);
  int pg_base = 0, pg_vec = 0;
  auto load_window = [&](int base) {
    pg_base = base;
    const int pg = base + l;
    pg_vec = (pg < p.max_blocks && pg * P < j1) ? bt_row[pg] : 0;
  };
  // This wave's half of the next step to issue: page index, row in the page and
  // the address of those rows, advanced step by step (a block-table lookup only
  // when the half crosses into another page; page_size is a multiple of 16).
  int dma_page = 0, dma_off = 0;
  const uint8_t* dma_row = cache;
  const uint32_t page_bytes = (uint32_t)P * kRB;
  auto page_ptr = [&](int page) -> const uint8_t* {
    if (page < pg_base || page >= pg_base + 64) {
      load_window(page);
      // complete the reload here, visibly to the compiler, so that the common
      // path carries no wait for it (a vector-memory wait would also drain the
      // in-flight tile loads)
      __builtin_amdgcn_s_waitcnt(0);
    }
    const uint32_t phys = (uint32_t)__builtin_amdgcn_readlane(pg_vec, page - pg_base);
    return cache + (uint64_t)phys * page_bytes;
  };
  auto half_live = [&](int it) { return j0 + kStepTok * it + 16 * hw < j1; };
  auto dma_reset = [&]() {
    const int jt = j0 + 16 * hw;
    dma_page = jt / P;
    dma_off = jt - dma_page * P;
  };
  // Sparse mode: no pages.  The row of every lane comes from the unit's index
  // row (entry j0 + 32 it + 16 hw + rsw for step it, clamped into the list and
  // the row id into the pool).  The first NB steps' ids are loaded here; each
  // later step's 32 ids arrive by a direct-to-LDS load issued NB steps ahead
  // into this wave's quarter of the idle probability buffer (see the step body).
  const int32_t* const idx_row = SPARSE ? p.indices + (size_t)b * p.topk : nullptr;
  auto idx_at = [&](int it, int r) { return min(j0 + kStepTok * it + 16 * hw + r, p.topk - 1); };
  auto idx_of = [&](int it) { return idx_at(it, rsw); };
  // Steps whose row ids are loaded before the loop; during step i the ids of
  // step i + kIdsAhead arrive (FP8: one step more, the codes are loaded three
  // steps ahead).  FP8 keeps three ids per lane and step: the rows of its code,
  // scale and rope loads.
  constexpr int kIdsAhead = FP8 ? NB + 1 : NB;
  int sidx_pro[NB];
  int sidx = 0;  // row id of this lane for the next step to issue
  // FP8 sparse: the ids of step k sit in slot k & 3 of this wave's part of
  // f8_idbuf (16 ids of its half); the first steps' ids are written by the
  // lanes below, later ones by a direct-to-LDS load four steps ahead.
  // f8c / f8s / f8r: the code, scale and rope row ids of this lane, read back
  // from the slots for the step about to be issued (f8r: its rope step)
  const uint32_t f8_ids_lds = lds_addr_of(f8_idbuf) + w * 256;
  int f8c = 0, f8s = 0, f8r = 0;
  auto f8_id_at = [&](int k, int r) {
    return *(const __attribute__((address_space(3))) int*)(uintptr_t)(f8_ids_lds + 64 * (k & 3) + 4 * r);
  };
  auto f8_load_ids = [&]() {
    // lanes 0-15 write the ids of the first kIdsAhead steps (visible to this
    // wave's own reads after its next LDS wait)
    if (l < 16) {
#pragma unroll
      for (int it = 0; it < kIdsAhead; ++it)
        *(__attribute__((address_space(3))) int*)(uintptr_t)(f8_ids_lds + 64 * (it & 3) + 4 * l) =
            idx_row[idx_at(it, l)];
    }
  };
  if constexpr (SPARSE && FP8) {
    f8_load_ids();
  } else if constexpr (SPARSE) {
#pragma unroll
    for (int it = 0; it < NB; ++it) sidx_pro[it] = idx_row[idx_of(it)];
  } else {
    dma_reset();
    load_window(dma_page);
  }
  // The query rows are loaded after the page ids, so the compiler's wait for the
  // page ids (at their first use) leaves the query loads in flight, overlapped
  // with the first tile loads.  The score MFMAs of the first step consume all of
  // q, so the compiler's waits for q all fall before the main loop (where a
  // vector-memory wait would also drain the in-flight tile loads).
#pragma unroll
  for (int ks = 0; ks < kR / 16; ++ks) q[ks] = *(const bf16x8*)(ql + 16 * ks);
#pragma unroll
  for (int ks = 0; ks < kDR / 16; ++ks) q[kR / 16 + ks] = *(const bf16x8*)(qp + 16 * ks);
  // consume the page ids here: the compiler's wait for them then counts the
  // query loads behind them exactly
  if constexpr (SPARSE && FP8) {
    wait_lgkm0();   // the first steps' ids are in LDS
  } else if constexpr (SPARSE) {
#pragma unroll
    for (int it = 0; it < NB; ++it) asm volatile("" ::"v"(sidx_pro[it]));
  } else {
    asm volatile("" ::"v"(pg_vec));
  }
  auto dma_start = [&]() {
    if (half_live(0)) dma_row = page_ptr(dma_page) + (uint32_t)dma_off * kRB;
  };

  const uint8_t* dma_base = cache;
  const uint8_t* dma_vaddr = cache;  // sparse: this lane's row + dma_coff
  const uint8_t* f8_code_va = cache;   // FP8 sparse: this lane's code row + its column offset
  bool f8_live_c = false, f8_live_r = false;   // FP8 sparse: the half of the code / rope step is in range
  // FP8 sparse: row of this lane's load (rows past the range read rows 0-15 of
  // the pool, like the dense path)
  auto f8_row = [&](bool live, int id, int dead) {
    return live ? min((uint32_t)id, p.num_rows - 1u) : (uint32_t)dead;
  };
  uint32_t dma_dst = 0;
  const uint32_t stg_lds = tiles_lds + NB * kStepBytes;  // FP8 code staging (two steps)
  uint32_t f8_scale_dst = 0;
  const uint8_t* f8_rope_base = cache;  // FP8: rows whose rope values the step loads
  uint32_t f8_rope_dst = 0;
  // A half past the end of the range (the second half of a short last step,
  // and every load issued past the last step: the pipeline issues NB-1 steps
  // ahead unconditionally) reads rows 0-15 of the cache, which are valid memory
  // the L2 keeps; its rows are cleared or masked before any use, and no wave
  // reads a buffer filled past the last step.  This keeps the issue path and
  // the wait counts free of branches.
  auto issue_prep = [&](int it) {
    if constexpr (FP8) {
      dma_dst = stg_lds + (it & 1) * kStgBytes + hw * 8192 + pw * 4096;
      f8_scale_dst = stg_lds + (it & 1) * kStgBytes + kStgCodes + w * 256;
    } else {
      dma_dst = tiles_lds + (it % NB) * kStepBytes + hw * kTileBytes + 1024 * (w & 1);
    }
    if constexpr (SPARSE && FP8) {
      f8_live_c = half_live(it);   // (the addresses are formed at each load: short live ranges)
      return;
    } else if constexpr (SPARSE) {
      const uint32_t row = half_live(it) ? min((uint32_t)sidx, p.num_rows - 1u) : (uint32_t)rsw;
      dma_vaddr = cache + (uint64_t)row * kRowBytes + dma_coff;
      return;
    }
    dma_base = half_live(it) ? dma_row : cache;
    // advance to the same half of the next step
    dma_off += kStepTok;
    if (dma_off >= P) {
      dma_off -= P;
      ++dma_page;
      if (dma_off >= P) {
        dma_off -= P;
        ++dma_page;
      }
      if (half_live(it + 1)) dma_row = page_ptr(dma_page) + (uint32_t)dma_off * kRB;
    } else {
      dma_row += kStepTok * kRB;
    }
  };
  auto issue_part = [&](auto n_const) {
    constexpr int n = decltype(n_const)::value;
    if constexpr (SPARSE) dma16v<128 * n>(dma_vaddr, dma_dst + 2048 * n);
    else dma16s(dma_voff + 128 * n, dma_base, dma_dst + 2048 * n);
  };
  // FP8 load instruction n of a step: 0 the rope values (rows f8_rope_base into
  // the ring), 1-4 the codes and 5 the scales (rows dma_base into staging)
  auto f8_issue_part = [&](auto n_const) {
    constexpr int n = decltype(n_const)::value;
    if constexpr (SPARSE) {
      if constexpr (n == 0) {
        dma16v<0>(cache + (uint64_t)f8_row(f8_live_r, f8r, f8_rr) * kF8Row + (kF8Rope + 64 * pw + 16 * (l >> 4)),
                  f8_rope_dst);
      } else if constexpr (n <= 4) {
        if constexpr (n == 1)
          f8_code_va = cache + (uint64_t)f8_row(f8_live_c, f8c, f8_rc) * kF8Row + (256 * pw + 16 * (l >> 4));
        dma16v<64 * (n - 1)>(f8_code_va, dma_dst + 1024 * (n - 1));
      } else {
        dma4v(cache + (uint64_t)f8_row(f8_live_c, f8s, f8_rs) * kF8Row + (kF8Scales + 4 * (l & 3)), f8_scale_dst);
      }
    } else {
      if constexpr (n == 0) dma16s(f8_rope_voff, f8_rope_base, f8_rope_dst);
      else if constexpr (n <= 4) dma16s_imm<64 * (n - 1)>(f8_code_voff, dma_base, dma_dst + 1024 * (n - 1));
      else dma4s(f8_scale_voff, dma_base, f8_scale_dst);
    }
  };
  // tile k's rope values come from the rows of the codes prepared last (sparse:
  // from rope row id rid of tile k)
  auto f8_rope_prep = [&](int k) {
    if constexpr (SPARSE) f8_live_r = half_live(k);
    f8_rope_base = dma_base;
    f8_rope_dst = tiles_lds + (k % NB) * kStepBytes + hw * kTileBytes + (kTileBytes - 2048) + 1024 * pw;
  };
  // FP8 conversion of tile k by this wave: unit n turns the 16 codes per lane of
  // its load instruction n into chunks 2 cp and 2 cp + 1 of row l & 15 (bf16,
  // times scale 2 pw + (n >> 1) of the row).  Chunk c = 2 cp + e of row t sits
  // at tile_pos(c, t), with c & 3 = 2 ((l >> 4) & 1) + e.
  u32x4 f8_raw;
  float f8_sc;
  // Lane terms: f8_rl = 16 l for the code reads (16 (l & 15) for the scales);
  // f8_wl for output chunk 2 cp, and f8_wl ^ 192 for chunk 2 cp + 1 (the row
  // swizzles of c & 3 = 2a and 2a + 1 differ by 12 for either a).
  const uint32_t f8_rl = 16 * l;
  const uint32_t f8_wl = 512 * (l >> 4) + 16 * ((l & 15) ^ tile_swz(2 * ((l >> 4) & 1)));
  // Per-tile LDS bases of the conversion (staging reads, scale reads and the
  // two lane patterns of the tile writes), recomputed for each tile and hidden
  // behind opaque() so that every access is base + immediate: precomputed per
  // (buffer, unit, half) the addresses outnumber the free registers and were
  // spilled, and each reload then waited for every tile load in flight.
  uint32_t f8_rb = 0, f8_sb = 0, f8_wb0 = 0, f8_wb1 = 0;
  auto f8_bases = [&](int k) {
    const uint32_t sb = stg_lds + (k & 1) * kStgBytes;
    f8_rb = opaque(sb + hw * 8192 + pw * 4096 + f8_rl);
    f8_sb = opaque(sb + kStgCodes + w * 256 + 8 * pw + (f8_rl & 0xF0u));
    const uint32_t tb = tiles_lds + (k % NB) * kStepBytes + hw * kTileBytes + 8192 * pw;
    f8_wb0 = opaque(tb + f8_wl);
    f8_wb1 = opaque(tb + (f8_wl ^ 192u));
  };
  auto f8_read = [&](auto n_const) {
    constexpr int n = decltype(n_const)::value;
    f8_raw = *(const __attribute__((address_space(3))) u32x4*)(uintptr_t)(f8_rb + 1024 * n);
    f8_sc = *(const __attribute__((address_space(3))) float*)(uintptr_t)(f8_sb + 4 * (n >> 1));
  };
  auto f8_write = [&](auto n_const, auto e_const) {
    constexpr int n = decltype(n_const)::value, e = decltype(e_const)::value;
    const u32x2 v0 = f8x4_to_bf16(f8_raw[2 * e], f8_sc), v1 = f8x4_to_bf16(f8_raw[2 * e + 1], f8_sc);
    const uint32_t dst = (e ? f8_wb1 : f8_wb0) + 2048 * n + 256 * e;
    *(__attribute__((address_space(3))) u32x4*)(uintptr_t)dst = u32x4{v0[0], v0[1], v1[0], v1[1]};
  };
  auto f8_convert = [&](int k) {  // the whole tile, not interleaved (prologue)
    f8_bases(k);
    static_for<0, 4>([&](auto n) {
      f8_read(n);
      f8_write(n, std::integral_constant<int, 0>{});
      f8_write(n, std::integral_constant<int, 1>{});
    });
  };
  auto f8_issue_codes = [&]() {
    static_for<1, 6>([&](auto n) { f8_issue_part(n); });
  };

  // sparse: during step i, the ids of step i + NB (entries j0 + 32 (i + NB) +
  // (l & 31)) go to this wave's quarter of probability buffer (i + 1) & 1,
  // which no wave touches between the barrier of step i and this wave's own
  // probability writes for step i + 1 (slot kSmPack); the ids are read back at
  // slot kSpIds, after a wait for the load
  // probability buffer: [step parity][token block][row block][lane] x 16 B
  constexpr uint32_t kPbufRowBlock = 64 * 16, kPbufParity = 2 * 4 * kPbufRowBlock;
  static_assert(2 * kPbufParity == sizeof(pbuf), "probability buffer layout");
  const uint32_t ids_lds0 = lds_addr_of(pbuf) + w * kPbufRowBlock;  // token block 0, row block w
  auto ids_lds = [&](int i) { return ids_lds0 + ((i + 1) & 1) * kPbufParity; };
  auto idx_dma = [&](int i) {
    if constexpr (FP8) {
      // the ids of this wave's half of step i + 4, lanes 0-15 only (64 bytes)
      if (l < 16) {
        const uint32_t voff = 4u * (uint32_t)min(j0 + kStepTok * (i + kIdsAhead) + 16 * hw + l, p.topk - 1);
        dma4s(voff, idx_row, f8_ids_lds + 64 * ((i + kIdsAhead) & 3));
      }
    } else {
      const uint32_t voff = 4u * (uint32_t)min(j0 + kStepTok * (i + kIdsAhead) + (l & 31), p.topk - 1);
      dma4s(voff, idx_row, ids_lds(i));
    }
  };
  auto issue = [&](int it) {
    issue_prep(it);
    issue_part(std::integral_constant<int, 0>{});
    issue_part(std::integral_constant<int, 1>{});
    issue_part(std::integral_constant<int, 2>{});
    issue_part(std::integral_constant<int, 3>{});
    issue_part(std::integral_constant<int, 4>{});
    issue_part(std::integral_constant<int, 5>{});
    issue_part(std::integral_constant<int, 6>{});
    issue_part(std::integral_constant<int, 7>{});
    issue_part(std::integral_constant<int, 8>{});
  };
  // Rows of the last step past the end of the range hold other tokens (or are
  // loaded twice): clear their value chunks so that 0-probability x row is 0.
  auto clear_tail = [&](int it) {
    const int nvalid = j1 - (j0 + kStepTok * it);
    if (nvalid >= kStepTok) return;
    const uint32_t buf = tiles_lds + (it % NB) * kStepBytes;
    for (int x = threadIdx.x; x < 2 * 64 * 16; x += 256) {
      const int hf = x >> 10, c = (x >> 4) & 63, t = x & 15;
      if (16 * hf + t >= nvalid)
        *(__attribute__((address_space(3))) u32x4*)(uintptr_t)(buf + hf * kTileBytes + tile_pos(c, t) * 16) =
            u32x4{0u, 0u, 0u, 0u};
    }
  };

  // score-phase K reads (A operand): lane reads row l & 31 of the step (half
  // (l >> 4) & 1), chunk 2ks + hl; address buf + k_lane[ks & 1] + 512 ks
  uint32_t k_lane[2];
#pragma unroll
  for (int e = 0; e < 2; ++e)
    k_lane[e] = kTileBytes * ((l >> 4) & 1) + 256 * hl + 16 * ((l & 15) ^ tile_swz(2 * e + hl));
  // value-phase transposing reads (A operand V^T of column block cb, token block
  // kb): group g = l >> 4, lane j = l & 15; read r covers tokens
  // 16kb + 4(g>>1) + 8r + (j>>2) and columns 32cb + 16(g&1) + 4(j&3) .. +3, i.e.
  // chunk 4cb + cl with cl = 2(g&1) + ((j>>1)&1), byte 8(j&1) of the chunk;
  // address buf + kb * kTileBytes + 1024 cb + v_lane[r]
  uint32_t v_lane[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int g = l >> 4, j = l & 15;
    const int tok = 4 * (g >> 1) + 8 * r + (j >> 2);
    const int cl = 2 * (g & 1) + ((j >> 1) & 1);
    v_lane[r] = (16 * cl + (tok ^ tile_swz(cl))) * 16 + 8 * (j & 1);
  }
  const float sl2 = p.scale_log2;
  const float lazy_raw = kLazy / sl2;

  // Per-row softmax reference (log2 domain) and the raw-score threshold above
  // which a replay is needed; nmb = -m_ref (0 while the row has no visible key).
  float m_ref = -INFINITY, nmb = 0.f, thr = INFINITY;
  bool ref_pending = true;
  bool grew = false;  // this wave raised a reference in the current pass
  float l_part;
  f32x16 acc[kR / 32];

  // ---- softmax of one step (scores S of step it) -> value operands pv[2] ----
  float x[16];
  float mxl = -INFINITY;
  bool grow = false;
  auto sm_load = [&](const f32x16& S) {
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = S[r];
  };
  auto sm_mask = [&](int it) {
    const int rel = dd - kStepTok * it;
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = (8 * (r >> 2) + (r & 3) < rel) ? x[r] : -INFINITY;
  };
  auto sm_check = [&]() {
    const float m0 = max4(x[0], x[1], x[2], x[3]), m1 = max4(x[4], x[5], x[6], x[7]);
    const float m2 = max4(x[8], x[9], x[10], x[11]), m3 = max4(x[12], x[13], x[14], x[15]);
    mxl = max4(m0, m1, m2, m3);
    grow = __builtin_amdgcn_ballot_w64(mxl > thr) != 0;
  };
  auto sm_reference = [&]() {  // first visible step of a row: fix m_ref
    float a, c;
    xpair32(mxl, a, c);
    const float mx = fmaxf(a, c);
    if (m_ref == -INFINITY && mx != -INFINITY) {
      m_ref = mx * sl2;
      nmb = -m_ref;
      thr = mx + lazy_raw;
    }
    ref_pending = __builtin_amdgcn_ballot_w64(m_ref == -INFINITY) != 0;
  };
  auto sm_exp = [&](int r0, int r1) {
#pragma unroll
    for (int r = r0; r < r1; ++r) x[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[r], sl2, nmb));
  };
  auto sm_sum = [&]() {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; r += 4) s += (x[r] + x[r + 1]) + (x[r + 2] + x[r + 3]);
    l_part += s;
  };
  auto sm_pack = [&](bf16x8 (&pv)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const u32x2 lo = cvt_bf16x4(f32x4{x[8 * kb], x[8 * kb + 1], x[8 * kb + 2], x[8 * kb + 3]});
      const u32x2 hi = cvt_bf16x4(f32x4{x[8 * kb + 4], x[8 * kb + 5], x[8 * kb + 6], x[8 * kb + 7]});
      pv[kb] = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
    }
  };
  // a row's max grew by more than kLazy: raise its reference, flag a replay
  auto sm_grow = [&]() {
    float a, c;
    xpair32(mxl, a, c);
    const float mx = fmaxf(a, c);
    if (mx > thr) {
      m_ref = mx * sl2;
      nmb = -m_ref;
      thr = mx + lazy_raw;
    }
    grew = true;
  };
  // whole softmax of one step, not interleaved (prologue)
  auto softmax_step = [&](const f32x16& S, int it, bf16x8 (&pv)[2]) {
    sm_load(S);
    sm_mask(it);
    sm_check();
    if (ref_pending) sm_reference();
    sm_exp(0, 16);
    sm_sum();
    sm_pack(pv);
    if (grow) sm_grow();
  };

  // scores of step it, not interleaved (prologue)
  auto scores_plain = [&](int it, f32x16& S) {
    const uint32_t kbuf = tiles_lds + (it % NB) * kStepBytes;
    const uint32_t kbase[2] = {opaque(kbuf + k_lane[0]), opaque(kbuf + k_lane[1])};
    S = f32x16{};
    constexpr int PF = 4;
    bf16x8 kb[PF];
#pragma unroll
    for (int ks = 0; ks < PF; ++ks) kb[ks] = lds_b128(kbase[ks & 1] + 512 * ks);
#pragma unroll
    for (int ks = 0; ks < kQk; ++ks) {
      const bf16x8 kop = kb[ks % PF];
      if (ks + PF < kQk) kb[ks % PF] = lds_b128(kbase[(ks + PF) & 1] + 512 * (ks + PF));
      S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, q[ks], S, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // V operand of value MFMA v from the step whose buffer bases are vb
  // (buffer + v_lane[0], buffer + v_lane[1])
  // (this wave's value columns are [128w, 128w + 128): column blocks 4w .. 4w+3)
  auto v_bases = [&](int it, uint32_t (&vb)[2]) {
    const uint32_t buf = tiles_lds + (it % NB) * kStepBytes + 4096 * w;
    vb[0] = opaque(buf + v_lane[0]);
    vb[1] = opaque(buf + v_lane[1]);
  };
  auto v_read = [&](const uint32_t (&vb)[2], int kb, int cb) -> bf16x8 {
    const uint32_t off = kb * kTileBytes + 1024 * cb;
    return join8(lds_tr16(vb[0] + off), lds_tr16(vb[1] + off));
  };
  // probability operands: this wave's rows go to LDS after each softmax; row
  // block rb of token block kb of a step is read back by every wave
  const uint32_t pbuf_lds = lds_addr_of(pbuf);
  auto p_write = [&](int it, const bf16x8 (&pv)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      *(__attribute__((address_space(3))) bf16x8*)(uintptr_t)(pbuf_lds + ((((it & 1) * 2 + kb) * 4 + w) * 64 + l) * 16) = pv[kb];
  };
  auto p_read = [&](int it, int kb, int ri) -> bf16x8 {
    const int rb = (w + ri) & 3;
    return lds_b128(pbuf_lds + ((((it & 1) * 2 + kb) * 4 + rb) * 64 + l) * 16);
  };

  // Smallest key limit over this wave's rows: a step ending at or before it
  // needs no mask for any of them.
  int lim_lo = j1;
  {
    const int g0 = row0 + 32 * w;
    if (g0 < TH) lim_lo = min(L - T + g0 / H + 1, j1);
  }

  constexpr int PF = FP8 ? 2 : 4;   // K operand reads in flight (FP8: registers for the conversion)

  // At most one replay: after a flagged pass every row's reference is within
  // kLazy of its true maximum, so the replay cannot flag again.
  // An empty range (no key of the sequence in this unit) skips the pipeline:
  // zero output and lse -inf.  Every path into the pipeline then passes through
  // the first step's score MFMAs, which consume all of q, so the compiler's
  // waits for the query loads never fall inside the main loop.
  l_part = 0.f;
#pragma unroll
  for (int cb = 0; cb < kR / 32; ++cb) acc[cb] = f32x16{};
  MLA_TS(1);
  if (nsteps > 0) for (int pass = 0;; ++pass) {
    if (pass > 0) {
      if constexpr (SPARSE && FP8) {
        f8_load_ids();
      } else if constexpr (SPARSE) {
#pragma unroll
        for (int it = 0; it < NB; ++it) sidx_pro[it] = idx_row[idx_of(it)];
      } else {
        dma_reset();
        load_window(dma_page);
      }
      __builtin_amdgcn_s_waitcnt(0);
    }
    if constexpr (!SPARSE) dma_start();
    if (pass > 0) {
      l_part = 0.f;
#pragma unroll
      for (int cb = 0; cb < kR / 32; ++cb) acc[cb] = f32x16{};
    }
    if constexpr (SPARSE && !FP8) {
#pragma unroll
      for (int it = 0; it < NB - 1; ++it) {
        sidx = sidx_pro[it];
        issue(it);
      }
      sidx = sidx_pro[NB - 1];
    } else if constexpr (FP8) {
      // tiles 0 and 1: codes, scales and rope values
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        if constexpr (SPARSE) {
          f8c = f8_id_at(it, f8_rc);
          f8s = f8_id_at(it, f8_rs);
          f8r = f8_id_at(it, f8_rr);
        }
        issue_prep(it);
        f8_rope_prep(it);
        f8_issue_part(std::integral_constant<int, 0>{});
        f8_issue_codes();
      }
    } else {
      for (int it = 0; it < NB - 1; ++it) issue(it);
    }

    // One-stage pipeline.  Step i (after its barrier): value MFMAs of step i
    // (probabilities pv from the softmax at the end of step i-1) interleaved
    // with the score MFMAs of step i+1, then the softmax of step i+1 under the
    // last value MFMAs.  Resident ring buffers: steps i and i+1; step i+2 in
    // flight, step i+3 issued during the step (into the buffer of step i-1).
    f32x16 S;
    bf16x8 pv[2];
    bf16x8 vc[4];  // V operands of the current token block, column blocks 0..3
    bf16x8 pp[3];  // probability operands of row blocks w+1 .. w+3
    {
      // prologue: step 0 landed; its scores and probabilities, first V operands
      if constexpr (FP8) {
        // tiles 0 and 1 converted; tile 2's codes requested once the staging
        // reads of tile 0 are done
        wait_vm0();
        f8_convert(0);
        f8_convert(1);
        wait_lgkm0();
        if constexpr (SPARSE) {
          f8c = f8_id_at(2, f8_rc);
          f8s = f8_id_at(2, f8_rs);
        }
        issue_prep(2);
        f8_issue_codes();
      } else {
        wait_vm<9 * (NB - 2)>();
      }
      barrier();
      MLA_TS(2);
      if (nsteps == 1 && j1 - j0 < kStepTok) {
        clear_tail(0);
        wait_lgkm0();
        barrier();
      }
      scores_plain(0, S);
      softmax_step(S, 0, pv);
      p_write(0, pv);
      uint32_t vb[2];
      v_bases(0, vb);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) vc[cb] = v_read(vb, 0, cb);
    }

    // body of step i (this wave's loads of step i+NB-1 are issued in it; FP8:
    // the rope values of tile i+2 and the codes of tile i+3, and tile i+2 is
    // converted)
    auto step = [&](int i) {
      if constexpr (FP8) {
        f8_rope_prep(i + 2);
        issue_prep(i + 3);
      } else {
        issue_prep(i + NB - 1);
      }
      if constexpr (SPARSE) idx_dma(i);
      const bool full = j0 + kStepTok * (i + 2) <= lim_lo;  // step i+1 needs no mask
      // K of step i+1 (after the last step: a resident stale buffer, whose
      // scores the mask discards)
      const uint32_t kbuf = tiles_lds + ((i + 1) % NB) * kStepBytes;
      const uint32_t kbase[2] = {opaque(kbuf + k_lane[0]), opaque(kbuf + k_lane[1])};
      uint32_t vb_cur[2], vb_next[2];
      v_bases(i, vb_cur);
      v_bases(i + 1, vb_next);
      bf16x8 kb[PF];
#pragma unroll
      for (int ks = 0; ks < PF; ++ks) kb[ks] = lds_b128(kbase[ks & 1] + 512 * ks);
      f32x16 Sn = {};
      static_for<0, kSlots>([&](auto s_c) {
        constexpr int s = decltype(s_c)::value;
        constexpr Slot sl = slot_of(s);
        if constexpr (sl.qk >= 0) {
          constexpr int ks = sl.qk;
          const bf16x8 kop = kb[ks % PF];
          if constexpr (ks + PF < kQk) kb[ks % PF] = lds_b128(kbase[(ks + PF) & 1] + 512 * (ks + PF));
          Sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, q[ks], Sn, 0, 0, 0);
        }
        if constexpr (sl.pv >= 0) {
          // value MFMA v: token block kb, row block ri (rows of wave w + ri), column
          // block cb; the own row block's probabilities come from registers
          constexpr int v = sl.pv;
          constexpr int kb = v >> 4, ri = (v >> 2) & 3, cb = v & 3;
          if constexpr (ri == 0) mfma_pv(acc[4 * cb], vc[cb], pv[kb]);
          else mfma_pv(acc[4 * cb + ri], vc[cb], pp[ri - 1]);
          // next row block's probabilities, four MFMAs ahead
          if constexpr (cb == 0 && ri < 3) pp[ri] = p_read(i, kb, ri + 1);
          // after its last use, the V operand of the next token block (the next
          // step's first block at the end)
          if constexpr (ri == 3) {
            if constexpr (kb == 0) vc[cb] = v_read(vb_cur, 1, cb);
            else vc[cb] = v_read(vb_next, 0, cb);
          }
        }
        if constexpr (FP8) {
          if constexpr (f8_part_at(s) >= 0) f8_issue_part(std::integral_constant<int, f8_part_at(s)>{});
          // the previous step's loads (codes of tile i+2) have landed once at most
          // this step's six are in flight
          if constexpr (s == kF8Wait) {
            wait_vm<SPARSE ? 7 : 6>();
            f8_bases(i + 2);   // (here, not at the step start: short live ranges)
          }
          constexpr int cv = f8_cvt_at(s);
          if constexpr (cv >= 0) {
            constexpr int n = cv >> 2, ph = cv & 3;
            if constexpr (ph == 0) f8_read(std::integral_constant<int, n>{});
            else f8_write(std::integral_constant<int, n>{}, std::integral_constant<int, ph - 1>{});
          }
        } else if constexpr (dma_part_at(s) >= 0) {
          issue_part(std::integral_constant<int, dma_part_at(s)>{});
        }
        if constexpr (SPARSE && !FP8 && s == kSpIds) {
          // the ids of step i + NB have landed once at most the nine tile loads
          // issued after them are in flight
          wait_vm<9>();
          sidx = *(const __attribute__((address_space(3))) int*)(uintptr_t)(ids_lds(i) + 4 * (16 * hw + rsw));
        }

        // softmax of step i+1 (past the last step every score is masked)
        if constexpr (s == kSmLoad) {
          sm_load(Sn);
          if (!full) sm_mask(i + 1);
        }
        if constexpr (s == kSmCheck) sm_check();
        if constexpr (s == kSmRef) {
          if (ref_pending) sm_reference();
        }
        if constexpr (s >= kSmExp0 && s < kSmExp0 + 16) sm_exp(s - kSmExp0, s - kSmExp0 + 1);
        if constexpr (s == kSmSum) sm_sum();
        if constexpr (s == kSmPack) {
          // probabilities of step i+1 (the value MFMAs of step i are past pv)
          sm_pack(pv);
          p_write(i + 1, pv);
        }
        __builtin_amdgcn_sched_barrier(0);
      });
      if (grow) sm_grow();
    };

    for (int i = 0; i < nsteps; ++i) {
      // step i+1 must have landed; the NB-3 later steps may stay in flight
      // (FP8: the rope values of tile i+1 have landed, the five code and scale
      // loads issued after them may stay in flight)
      wait_vm<FP8 ? 5 : 9 * (NB - 3)>();
      // this wave's probability writes are done; the last two V operand reads
      // (two LDS reads each) may stay in flight
      wait_lgkm<4>();
      if constexpr (SPARSE && FP8) {
        // row ids of this step's loads (codes and scales of step i + 3, rope of
        // step i + 2), in LDS since the wait above (their load preceded the
        // rope values of step i + 1); read under the barrier
        f8c = f8_id_at(i + 3, f8_rc);
        f8s = f8_id_at(i + 3, f8_rs);
        f8r = f8_id_at(i + 2, f8_rr);
      }
      barrier();
      if (i + 2 == nsteps && j1 - (j0 + kStepTok * (i + 1)) < kStepTok) {
        // the last step is partial: clear its rows past the end before any
        // wave reads it (once per work unit)
        clear_tail(i + 1);
        wait_lgkm0();
        barrier();
      }
      step(i);
    }
    MLA_TS(3);
    wait_vm0();  // the loads issued past the last step
    mfma_drain();
    wait_lgkm0();
    barrier();
    // replay decision: the waves' flags meet in the (now idle) ring
    if (l == 0) *(__attribute__((address_space(3))) unsigned*)(uintptr_t)(tiles_lds + 4 * w) = grew ? 1u : 0u;
    wait_lgkm0();
    barrier();
    const u32x4 fl = *(const __attribute__((address_space(3))) u32x4*)(uintptr_t)tiles_lds;
    wait_lgkm0();
    barrier();  // every wave has read the flags before the ring is reused
    if (!((fl[0] | fl[1] | fl[2] | fl[3]) != 0u && pass == 0)) break;
    // a flagged pass is discarded and replayed with the raised references
    grew = false;
  }

  MLA_TS(4);
  // ---- finalize: row sums (lanes l and l ^ 32 hold halves of each row), lse ----
  float ls;
  {
    float a, c;
    xpair32(l_part, a, c);
    ls = a + c;
  }
  // every wave stores all 128 rows (its 128 columns): the inverse row sums meet
  // in the (now idle) probability buffer
  if (hl == 0) *(__attribute__((address_space(3))) float*)(uintptr_t)(pbuf_lds + 4 * rloc) = ls > 0.f ? 1.f / ls : 0.f;
  if (hl == 0 && grow_ < TH) {
    // lse in natural log: (m + log2(sum)) * ln 2
    const float lse2 = (ls > 0.f) ? m_ref + __builtin_amdgcn_logf(ls) : -INFINITY;
    const float lse_nat = lse2 * 0.69314718055994530942f;
    if constexpr (SPLIT) {
      p.part_lse[(size_t)slot * TH + grow_] = lse_nat;
    } else {
      if (p.lse) p.lse[(size_t)b * TH + grow_] = lse_nat;
    }
  }

  // ---- store: the workgroup's rows [row0, row0 + 128) of its output are one
  // contiguous block (1 KB per row in bf16, 2 KB in fp32).  The normalised
  // accumulators are staged through the (now idle) step ring in row-major
  // order, then written with 16-byte-per-lane contiguous stores that carry the
  // streaming hint (every unit writes its block at the same moment, at the end
  // of the launch; the hint lets the writes drain faster).  Staging
  // swizzle: 16-byte chunk c of staged row r sits at chunk c ^ (r & 15); in the
  // bf16 layout the two 8-byte halves of a chunk are also swapped when bit 4 of
  // r is set (both make the staging writes and the reads conflict-free).
  // Accumulator acc[4cb + ri] register 4 q4 + e holds column
  // 128w + 32cb + 8q4 + 4hl + e of row 32 rb + (l & 31), rb = (w + ri) & 3.
  wait_lgkm0();
  barrier();
  MLA_TS(5);
  float inv[4];
#pragma unroll
  for (int ri = 0; ri < 4; ++ri)
    inv[ri] = *(const __attribute__((address_space(3))) float*)(uintptr_t)(pbuf_lds + 4 * (32 * ((w + ri) & 3) + (l & 31)));
  const int n_rows = min(kRowsPerWG, TH - row0);
  char* const dst_base = (char*)(SPLIT ? p.part_out : p.out) + ((size_t)slot * TH + row0) * kR * (OUT_F32 ? 4 : 2);
  constexpr int kRowOut = kR * (OUT_F32 ? 4 : 2);      // bytes per output row
  constexpr int kStageRows = OUT_F32 ? 64 : 128;       // rows per staging round (128 KB)
  static_assert(kStageRows * kRowOut <= kRingBytes, "staging block exceeds the ring");
#pragma unroll
  for (int round = 0; round < 128 / kStageRows; ++round) {
#pragma unroll
    for (int ri = 0; ri < 4; ++ri) {
      const int rb = (w + ri) & 3;
      if ((32 * rb) / kStageRows != round) continue;
      const int r = 32 * rb - round * kStageRows + (l & 31);  // staged row
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[4 * cb + ri][4 * q4 + e] * inv[ri];
          if constexpr (OUT_F32) {
            const int c = 32 * w + 8 * cb + 2 * q4 + hl;
            *(__attribute__((address_space(3))) f32x4*)(uintptr_t)(tiles_lds + r * kRowOut + ((c ^ (r & 15)) * 16)) = v;
          } else {
            const int c = 16 * w + 4 * cb + q4;
            const int hh = hl ^ ((r >> 4) & 1);
            lds_st64(tiles_lds + r * kRowOut + ((c ^ (r & 15)) * 16) + 8 * hh, cvt_bf16x4(v));
          }
        }
      }
    }
    wait_lgkm0();
    barrier();
    const int rows_here = min(kStageRows, n_rows - round * kStageRows);
    char* const dst = dst_base + (size_t)round * kStageRows * kRowOut;
    constexpr int kChunksPerRow = kRowOut / 16;
    auto out_chunk = [&](int xx, u32x4& v) {   // staged chunk xx -> v (bf16: halves back in order)
      const int r = xx / kChunksPerRow, c = xx - r * kChunksPerRow;
      v = *(const __attribute__((address_space(3))) u32x4*)(uintptr_t)(tiles_lds + r * kRowOut + ((c ^ (r & 15)) * 16));
      return r;
    };
    if (rows_here == kStageRows) {
      // a whole block (every unit of a 128-row group): 32 chunks per thread, 16
      // LDS reads in flight before their stores (one at a time, each read's wait
      // would stand between consecutive stores)
      constexpr int kPer = kStageRows * kChunksPerRow / 256, kBatch = 16;
      static_assert(kPer % kBatch == 0, "whole batches");
#pragma unroll
      for (int g = 0; g < kPer / kBatch; ++g) {
        u32x4 v[kBatch];
        int rr[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) rr[k] = out_chunk(threadIdx.x + 256 * (kBatch * g + k), v[k]);
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          const int xx = threadIdx.x + 256 * (kBatch * g + k);
          const int r = rr[k], c = xx - r * kChunksPerRow;
          u32x4 o = v[k];
          if (!OUT_F32 && ((r >> 4) & 1)) o = u32x4{o[2], o[3], o[0], o[1]};
          store16_nt(dst + (size_t)r * kRowOut + 16 * c, o);
        }
      }
    } else {
      for (int xx = threadIdx.x; xx < rows_here * kChunksPerRow; xx += 256) {
        u32x4 v;
        const int r = out_chunk(xx, v), c = xx - r * kChunksPerRow;
        if (!OUT_F32 && ((r >> 4) & 1)) v = u32x4{v[2], v[3], v[0], v[1]};
        store16_nt(dst + (size_t)r * kRowOut + 16 * c, v);
      }
    }
    if (round + 1 < 128 / kStageRows) barrier();
  }
  MLA_TS(6);
  MLA_TS_DRAIN();
  MLA_TS(7);
}

#ifdef MLA_DECODE_TIMELINE
extern "C" int mla_timeline_read(void* host, size_t bytes) {
  if (!host || bytes > sizeof(g_timeline)) return (int)hipErrorInvalidValue;
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(g_timeline), bytes, 0, hipMemcpyDeviceToHost);
}
#endif

// ---- automatic split plan: work list (b, j0, j1, slot) and split_indptr ----
// One workgroup.  The decode launch runs one work unit per CU at a time, so its
// time is set by the longest unit: the chunk length is the smallest multiple of
// the page size (at least min_chunk) for which the units
//     units(c) = sum_b clamp(ceil(L_b / c), 1, cap)
// fit in target_units (the CU count).  With B < target_units the answer is at
// most c = sum/(target - B) (each sequence rounding up by a whole unit, which
// always fits) and at least min_chunk; a search over that range, 32 candidates
// a round (32 threads per candidate, each counting every 32nd sequence, so each
// thread divides only B/32 times a round: the kernel is one CU's work), narrows
// it 32-fold a round until it is exact.  If one unit per sequence
// already exceeds the target, every sequence is one unit.  A sequence's S_b
// chunks are equal up to the page rounding: chunk_b = ceil(ceil(L_b/S_b)/P)*P.
__global__ __launch_bounds__(1024) void plan_kernel(PlanParams p) {
  constexpr int kLens = 4096;  // lengths cached in LDS (more are read from memory)
  __shared__ int lens[kLens];
  __shared__ int red_max, red_best;
  __shared__ unsigned long long red_sum;
  __shared__ int wave_tot[16];
  __shared__ int cand_units[256];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int B = p.B, P = p.page_size;
  if (tid == 0) {
    red_max = 0;
    red_best = 0x7fffffff;
    red_sum = 0ull;
  }
  __syncthreads();
  int mx = 0;
  unsigned long long sm = 0;
  for (int b = tid; b < B; b += 1024) {
    const int L = max(0, p.seqlens[b]);
    if (b < kLens) lens[b] = L;
    mx = max(mx, L);
    sm += (unsigned)L;
  }
  // wave reductions first: same-address LDS atomics from every lane serialise
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mx = max(mx, __shfl_xor(mx, o));
    sm += __shfl_xor(sm, o);
  }
  if (lane == 0) {
    atomicMax(&red_max, mx);
    atomicAdd(&red_sum, sm);
  }
  __syncthreads();
  auto len = [&](int b) { return b < kLens ? lens[b] : max(0, p.seqlens[b]); };
  auto splits = [&](int L, unsigned chunk) {
    const unsigned s = ((unsigned)L + chunk - 1u) / chunk;
    return (int)max(1u, min((unsigned)p.cap, s));
  };
  const int kmax = max(1, (red_max + P - 1) / P);  // one unit per sequence
  int kbest = kmax;
  if (B < p.target_units) {
    const unsigned long long tot = red_sum;
    const int kmin = max(1, (p.min_chunk + P - 1) / P);
    const unsigned long long per_hi = (tot + (unsigned long long)(p.target_units - B) * P - 1) /
                                      ((unsigned long long)(p.target_units - B) * P);
    int hi = (int)min((unsigned long long)kmax, max(per_hi, (unsigned long long)kmin));
    int lo = min(kmin, hi);
    // Each round: candidates k_c = min(hi, lo + c * step), c < 32, step =
    // ceil((hi - lo + 1) / 32), so the last is within step of hi.  The answer
    // lies in (best - step, best] for the smallest feasible candidate best (hi
    // when none is: hi is always feasible), which is the next range.  lo and hi
    // come from shared values, so every thread runs the same rounds.
    while (lo < hi) {
      const int step = (hi - lo + 32) / 32;  // ceil((hi - lo + 1) / 32)
      // thread (candidate c, group g) counts the units of sequences b = g mod 32
      const int c = tid & 31, g = tid >> 5;
      const int k = min(hi, lo + c * step);
      if (tid < 32) cand_units[tid] = 0;
      __syncthreads();
      int units = 0;
      for (int b = g; b < B; b += 32) units += splits(len(b), (unsigned)k * (unsigned)P);
      units += __shfl_xor(units, 32);  // lanes l and l + 32 count for the same candidate
      if (lane < 32) atomicAdd(&cand_units[c], units);
      __syncthreads();
      // smallest feasible candidate (wave 0)
      if (tid < 64) {
        int kb = (lane < 32 && cand_units[lane] <= p.target_units) ? k : 0x7fffffff;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) kb = min(kb, __shfl_xor(kb, o));
        if (lane == 0) red_best = kb;
      }
      __syncthreads();
      const int best = min(red_best, hi);
      hi = best;
      lo = max(lo, best - step + 1);
      __syncthreads();  // every thread has read red_best and cand_units before the next round
    }
    kbest = hi;
  }
  const unsigned chunk = (unsigned)kbest * (unsigned)P;
  // split counts of this thread's contiguous range of sequences, and their prefix
  const int per = (B + 1023) / 1024;
  const int b0 = min(B, tid * per), b1 = min(B, b0 + per);
  int local = 0;
  for (int b = b0; b < b1; ++b) local += splits(len(b), chunk);
  // exclusive scan over the 1024 threads: within each wave, then across waves
  int incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wave_tot[wv] = incl;
  __syncthreads();
  int before = 0;
  for (int k = 0; k < wv; ++k) before += wave_tot[k];
  int base = before + incl - local;
  if (tid == 1023) *p.n_items = before + incl;
  if (tid == 0) p.split_indptr[0] = 0;
  for (int b = b0; b < b1; ++b) {
    const int L = len(b);
    const int sb = splits(L, chunk);
    const int cb = ((L + sb - 1) / sb + P - 1) / P * P;
    for (int k = 0; k < sb; ++k) {
      const long long a0 = min((long long)L, (long long)k * cb);
      const long long a1 = min((long long)L, a0 + cb);
      int* wi = p.work + 4 * (size_t)(base + k);
      wi[0] = b;
      wi[1] = (int)a0;
      wi[2] = (int)a1;
      wi[3] = base + k;
    }
    base += sb;
    p.split_indptr[b + 1] = base;
  }
}

template <int NB, bool SPLIT, bool F32, bool SPARSE, bool FP8 = false>
static hipError_t launch_decode_t(const DecodeParams& prm, int grid, hipStream_t st) {
  hipLaunchKernelGGL((decode_kernel<NB, SPLIT, F32, SPARSE, FP8>), dim3(grid), dim3(256), 0, st, prm);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams& prm, int max_units, bool split, bool out_f32,
                         hipStream_t st, bool sparse, bool fp8) {
  constexpr int NB = 4;
  const int grid = ((max_units + 7) / 8) * 8;  // whole XCD rounds; extra workgroups exit
  if (fp8 && sparse) {
    if (split) {
      if (out_f32) return launch_decode_t<3, true, true, true, true>(prm, grid, st);
      return launch_decode_t<3, true, false, true, true>(prm, grid, st);
    }
    if (out_f32) return launch_decode_t<3, false, true, true, true>(prm, grid, st);
    return launch_decode_t<3, false, false, true, true>(prm, grid, st);
  }
  if (fp8) {
    if (split) {
      if (out_f32) return launch_decode_t<3, true, true, false, true>(prm, grid, st);
      return launch_decode_t<3, true, false, false, true>(prm, grid, st);
    }
    if (out_f32) return launch_decode_t<3, false, true, false, true>(prm, grid, st);
    return launch_decode_t<3, false, false, false, true>(prm, grid, st);
  }
  if (sparse) {
    if (split) {
      if (out_f32) return launch_decode_t<NB, true, true, true>(prm, grid, st);
      return launch_decode_t<NB, true, false, true>(prm, grid, st);
    }
    if (out_f32) return launch_decode_t<NB, false, true, true>(prm, grid, st);
    return launch_decode_t<NB, false, false, true>(prm, grid, st);
  }
  if (split) {
    if (out_f32) return launch_decode_t<NB, true, true, false>(prm, grid, st);
    return launch_decode_t<NB, true, false, false>(prm, grid, st);
  }
  if (out_f32) return launch_decode_t<NB, false, true, false>(prm, grid, st);
  return launch_decode_t<NB, false, false, false>(prm, grid, st);
}

hipError_t launch_plan(const PlanParams& prm, hipStream_t st) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, st, prm);
  return hipGetLastError();
}

}  // namespace mla
