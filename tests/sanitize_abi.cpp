// Host side of the C ABI under AddressSanitizer + UndefinedBehaviorSanitizer
// (test infrastructure: tests/test_sanitize_abi.py builds it with g++ together
// with csrc/api.cpp and csrc/normal_api.cpp and runs it, no GPU).
//
// The kernel launchers (mla::launch_*), the few HIP runtime calls the ABI
// makes and the three rocBLAS calls of the Normal path are replaced by stubs
// that record what they were given, so every validation branch, workspace
// size and launch decision of the entry points runs for real on the host.
// Buffers the host code reads (mla_validate_inputs copies the lengths and the
// block table) are allocated at their exact sizes, so an access past them is
// reported.  Prints "ok" at the end; any failed expectation exits with 1.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../include/mla_latent.h"
#include "../include/mla_normal.h"
#include "../mla_latent_kv_amd/csrc/launch.hpp"

namespace {
struct Rec {
  int decode = 0, plan = 0, merge = 0, absorb = 0, unabsorb = 0, append = 0, gather = 0, mha = 0, gemm = 0,
      merge_unabsorb = 0;
  mla::DecodeParams dp{};
  int max_units = 0;
  bool split = false, out_f32 = false, sparse = false, fp8 = false;
  mla::PlanParams pp{};
  mla::MergeParams mp{};
  mla::MergeUnabsorbParams mup{};
  bool mu_f32 = false;
  int absorb_M = 0, unabsorb_M = 0;
} rec;
int failures = 0;

void expect(bool ok, const char* what, int line) {
  if (!ok) {
    std::fprintf(stderr, "FAILED line %d: %s\n", line, what);
    ++failures;
  }
}
#define EXPECT(c) expect((c), #c, __LINE__)
#define EXPECT_EQ(a, b) expect((a) == (b), #a " == " #b, __LINE__)
}  // namespace

// ---- stubs of the kernel launchers ----
namespace mla {
hipError_t launch_decode(const DecodeParams& p, int max_units, bool split, bool out_f32, hipStream_t, bool sparse,
                         bool fp8) {
  ++rec.decode;
  rec.dp = p;
  rec.max_units = max_units;
  rec.split = split;
  rec.out_f32 = out_f32;
  rec.sparse = sparse;
  rec.fp8 = fp8;
  return hipSuccess;
}
hipError_t launch_plan(const PlanParams& p, hipStream_t) {
  ++rec.plan;
  rec.pp = p;
  return hipSuccess;
}
hipError_t launch_merge(const MergeParams& p, bool, bool, hipStream_t) {
  ++rec.merge;
  rec.mp = p;
  return hipSuccess;
}
hipError_t launch_absorb(const AbsorbParams& p, hipStream_t) {
  ++rec.absorb;
  rec.absorb_M = p.M;
  return hipSuccess;
}
hipError_t launch_unabsorb(const UnabsorbParams& p, bool, hipStream_t) {
  ++rec.unabsorb;
  rec.unabsorb_M = p.M;
  return hipSuccess;
}
hipError_t launch_merge_unabsorb(const MergeUnabsorbParams& p, bool part_f32, hipStream_t) {
  ++rec.merge_unabsorb;
  rec.mup = p;
  rec.mu_f32 = part_f32;
  return hipSuccess;
}
hipError_t launch_append(const AppendParams&, hipStream_t) {
  ++rec.append;
  return hipSuccess;
}
hipError_t launch_gather(const NormalParams&, hipStream_t) {
  ++rec.gather;
  return hipSuccess;
}
hipError_t launch_mha(const NormalParams&, hipStream_t) {
  ++rec.mha;
  return hipSuccess;
}
}  // namespace mla

// ---- stubs of the HIP runtime calls the ABI makes (a 256-CU device 0) ----
extern "C" {
hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int) {
  *v = 256;
  return hipSuccess;
}
hipError_t hipGetLastError(void) { return hipSuccess; }
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind, hipStream_t) {
  std::memcpy(dst, src, n);   // "device" buffers here are host arrays of exact size
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }

// ---- stubs of the rocBLAS calls of the Normal path ----
static int g_handle_storage;
rocblas_status rocblas_create_handle(rocblas_handle* h) {
  *h = (rocblas_handle)&g_handle_storage;
  return rocblas_status_success;
}
rocblas_status rocblas_set_stream(rocblas_handle, hipStream_t) { return rocblas_status_success; }
rocblas_status rocblas_gemm_ex(rocblas_handle, rocblas_operation, rocblas_operation, rocblas_int m, rocblas_int n,
                               rocblas_int k, const void*, const void* a, rocblas_datatype, rocblas_int, const void* b,
                               rocblas_datatype, rocblas_int, const void*, const void* c, rocblas_datatype,
                               rocblas_int, void* d, rocblas_datatype, rocblas_int, rocblas_datatype,
                               rocblas_gemm_algo, int32_t, uint32_t) {
  ++rec.gemm;
  return (m > 0 && n > 0 && k > 0 && a && b && c && d) ? rocblas_status_success : rocblas_status_invalid_size;
}
}  // extern "C"

namespace {
// fake device addresses: 16-byte aligned, never dereferenced by host code
void* const D = (void*)(uintptr_t)(1u << 20);
void* const Dmis = (void*)(uintptr_t)((1u << 20) + 2);
const uint16_t* const Q = (const uint16_t*)D;

int decode(bool fp8, int B, int T, int H, int maxL, int S, void* ws, size_t wsb, void* po, float* pl, int32_t* si,
           void* out, int P = 64, int nb = 4096, int r = 512, int dr = 64, float scale = 0.07f, int mb = -1) {
  if (mb < 0) mb = (maxL + P - 1) / P;
  if (fp8)
    return mla_decode_latent_fp8(Q, Q, (const uint8_t*)D, nb, P, (const int32_t*)D, mb, (const int32_t*)D, B, T, H,
                                 r, dr, maxL, scale, S, ws, wsb, po, MLA_BF16, pl, si, out, MLA_BF16, nullptr,
                                 nullptr);
  return mla_decode_latent(Q, Q, Q, nb, P, (const int32_t*)D, mb, (const int32_t*)D, B, T, H, r, dr, maxL, scale, S,
                           ws, wsb, po, MLA_F32, pl, si, out, MLA_BF16, nullptr, nullptr);
}

void test_absorb_unabsorb() {
  EXPECT_EQ(mla_absorb_q(Q, Q, (uint16_t*)D, 64, 1, 128, 128, 512, nullptr), MLA_OK);
  EXPECT_EQ(rec.absorb_M, 64);
  EXPECT_EQ(mla_absorb_q(Q, Q, (uint16_t*)D, 32, 4, 32, 128, 512, nullptr), MLA_OK);
  EXPECT_EQ(rec.absorb_M, 128);
  EXPECT_EQ(mla_absorb_q(Q, Q, (uint16_t*)Dmis, 2, 1, 128, 128, 512, nullptr), MLA_ERR_ALIGN);
  EXPECT_EQ(mla_absorb_q(Q, Q, (uint16_t*)D, 1 << 14, 1024, 128, 128, 512, nullptr), MLA_OK);   // B*T = 2^24
  EXPECT_EQ(mla_absorb_q(Q, Q, (uint16_t*)D, (1 << 14) + 1, 1024, 128, 128, 512, nullptr), MLA_ERR_SHAPE);
  EXPECT_EQ(mla_absorb_q(Q, Q, (uint16_t*)D, 2, 1, 128, 64, 512, nullptr), MLA_ERR_UNSUPPORTED);
  EXPECT_EQ(mla_unabsorb_out(D, MLA_F32, Q, (float*)D, 64, 1, 128, 512, 128, nullptr), MLA_OK);
  EXPECT_EQ(rec.unabsorb_M, 64);
  EXPECT_EQ(mla_unabsorb_out(D, (mla_dtype)5, Q, (float*)D, 64, 1, 128, 512, 128, nullptr), MLA_ERR_UNSUPPORTED);
  EXPECT_EQ(mla_unabsorb_out(nullptr, MLA_BF16, Q, (float*)D, 64, 1, 128, 512, 128, nullptr), MLA_ERR_NULL);
  EXPECT_EQ(mla_unabsorb_out(nullptr, MLA_BF16, nullptr, nullptr, 0, 1, 128, 512, 128, nullptr), MLA_OK);
}

void test_workspace_and_decode() {
  size_t wsb = 0;
  int rows = 0;
  EXPECT_EQ(mla_decode_workspace_size(64, 1, 128, 512, 4096, 64, 1, &wsb, &rows), MLA_OK);
  EXPECT(wsb == 0 && rows == 0);
  EXPECT_EQ(mla_decode_workspace_size(64, 1, 128, 512, 4096, 64, 4, &wsb, &rows), MLA_OK);
  EXPECT(wsb == 0 && rows == 256);
  EXPECT_EQ(mla_decode_workspace_size(64, 1, 128, 512, 4096, 64, 0, &wsb, &rows), MLA_OK);
  EXPECT(rows == 64 + 256 && wsb == 256 + 16 * (size_t)rows);   // B + CUs work items
  EXPECT_EQ(mla_decode_workspace_size(4, 1, 128, 512, 131072, 64, 0, &wsb, &rows), MLA_OK);
  EXPECT_EQ(rows, 4 + 256);                                       // min(128 B, B + CUs)
  EXPECT_EQ(mla_decode_workspace_size(1, 1, 128, 512, 131072, 64, 0, &wsb, &rows), MLA_OK);
  EXPECT_EQ(rows, 128);                                           // at most 128 chunks per sequence
  EXPECT_EQ(mla_decode_workspace_size(64, 1, 128, 512, 4096, 64, 0, nullptr, &rows), MLA_ERR_NULL);
  EXPECT_EQ(mla_decode_workspace_size(64, 1, 128, 512, 4096, 24, 0, &wsb, &rows), MLA_ERR_UNSUPPORTED);
  EXPECT_EQ(mla_decode_workspace_size(1 << 30, 1, 128, 512, 4096, 64, 64, &wsb, &rows), MLA_ERR_SHAPE);

  for (bool fp8 : {false, true}) {
    // unsplit: one launch, B * ceil(T*H/128) units
    rec = Rec{};
    EXPECT_EQ(decode(fp8, 64, 1, 128, 4096, 1, nullptr, 0, nullptr, nullptr, nullptr, D), MLA_OK);
    EXPECT(rec.decode == 1 && !rec.split && rec.max_units == 64 && rec.dp.n_units == 64 && rec.fp8 == fp8);
    EXPECT_EQ(decode(fp8, 8, 4, 128, 300, 1, nullptr, 0, nullptr, nullptr, nullptr, D), MLA_OK);
    EXPECT_EQ(rec.dp.n_rg, 4);
    // uniform split with merge
    rec = Rec{};
    EXPECT_EQ(decode(fp8, 64, 1, 128, 4096, 4, nullptr, 0, D, (float*)D, (int32_t*)D, D), MLA_OK);
    EXPECT(rec.decode == 1 && rec.split && rec.max_units == 256 && rec.merge == 1 && rec.plan == 0);
    // uniform split without merge (out_latent NULL)
    rec = Rec{};
    EXPECT_EQ(decode(fp8, 64, 1, 128, 4096, 4, nullptr, 0, D, (float*)D, (int32_t*)D, nullptr), MLA_OK);
    EXPECT(rec.decode == 1 && rec.merge == 0);
    // automatic: plan + decode + merge, target units = CUs / row groups
    std::vector<uint8_t> ws(256 + 16 * 320);
    rec = Rec{};
    EXPECT_EQ(decode(fp8, 64, 1, 128, 4096, 0, D, ws.size(), D, (float*)D, (int32_t*)D, nullptr), MLA_OK);
    EXPECT(rec.plan == 1 && rec.pp.target_units == 256 && rec.decode == 1 && rec.split && rec.max_units == 320);
    // automatic with B * row groups >= CUs: runs unsplit when the merged result is wanted
    rec = Rec{};
    EXPECT_EQ(decode(fp8, 256, 1, 128, 4096, 0, D, 1 << 20, D, (float*)D, (int32_t*)D, D), MLA_OK);
    EXPECT(rec.plan == 0 && rec.decode == 1 && !rec.split);
    // errors
    EXPECT_EQ(decode(fp8, 64, 1, 128, 4096, 0, D, 100, D, (float*)D, (int32_t*)D, nullptr), MLA_ERR_WORKSPACE);
    EXPECT_EQ(decode(fp8, 64, 1, 128, 4096, 4, nullptr, 0, nullptr, (float*)D, (int32_t*)D, D), MLA_ERR_WORKSPACE);
    EXPECT_EQ(decode(fp8, 64, 1, 128, 4096, 4, nullptr, 0, Dmis, (float*)D, (int32_t*)D, D), MLA_ERR_ALIGN);
    EXPECT_EQ(decode(fp8, 64, 1, 128, 4096, 1, nullptr, 0, nullptr, nullptr, nullptr, nullptr), MLA_ERR_NULL);
    EXPECT_EQ(decode(fp8, 64, 1, 128, 4096, 1, nullptr, 0, nullptr, nullptr, nullptr, D, 64, 4096, 512, 64,
                     0.0f), MLA_ERR_SHAPE);
    EXPECT_EQ(decode(fp8, 64, 1, 128, 4096, 1, nullptr, 0, nullptr, nullptr, nullptr, D, 64, 4096, 512, 64,
                     std::nanf("")), MLA_ERR_SHAPE);
    EXPECT_EQ(decode(fp8, 64, 1, 128, 4096, 1, nullptr, 0, nullptr, nullptr, nullptr, D, 64, 4096, 512, 64,
                     0.07f, 63), MLA_ERR_SHAPE);   // table too narrow for max_seqlen
    EXPECT_EQ(decode(fp8, 64, 1, 128, 4096, 1, nullptr, 0, nullptr, nullptr, nullptr, D, 48), MLA_OK);
    EXPECT_EQ(decode(fp8, 64, 1, 128, 4096, 1, nullptr, 0, nullptr, nullptr, nullptr, D, 24), MLA_ERR_UNSUPPORTED);
    EXPECT_EQ(decode(fp8, 64, 1, 129, 4096, 1, nullptr, 0, nullptr, nullptr, nullptr, D), MLA_ERR_UNSUPPORTED);
    EXPECT_EQ(decode(fp8, 64, 1025, 1, 4096, 1, nullptr, 0, nullptr, nullptr, nullptr, D), MLA_ERR_UNSUPPORTED);
    EXPECT_EQ(decode(fp8, 64, 2, 1, 1, 1, nullptr, 0, nullptr, nullptr, nullptr, D), MLA_ERR_SHAPE);  // maxL < T
    EXPECT_EQ(decode(fp8, 0, 1, 128, 4096, 4, nullptr, 0, nullptr, nullptr, nullptr, nullptr), MLA_OK);
  }
}

void test_merge_append_sparse() {
  EXPECT_EQ(mla_merge_splits(D, MLA_BF16, (float*)D, (int32_t*)D, 64, 1, 128, 512, D, MLA_BF16, nullptr, nullptr),
            MLA_OK);
  EXPECT(rec.mp.B == 64 && rec.mp.TH == 128);
  EXPECT_EQ(mla_merge_splits(D, MLA_BF16, (float*)D, (int32_t*)D, 64, 1, 128, 256, D, MLA_BF16, nullptr, nullptr),
            MLA_ERR_UNSUPPORTED);
  EXPECT_EQ(mla_merge_splits(D, MLA_BF16, (float*)Dmis, (int32_t*)D, 64, 1, 128, 512, D, MLA_BF16, nullptr,
                             nullptr), MLA_ERR_ALIGN);
  // merge + un-absorb: the grid (heads x groups) and its validation
  EXPECT_EQ(mla_merge_unabsorb(D, MLA_BF16, (float*)D, (int32_t*)D, Q, 64, 1, 128, 512, 128, (float*)D, nullptr,
                               nullptr), MLA_OK);
  EXPECT(rec.mup.M == 64 && rec.mup.T == 1 && rec.mup.H == 128 && rec.mup.groups == 2 && !rec.mu_f32);
  EXPECT_EQ(mla_merge_unabsorb(D, MLA_F32, (float*)D, (int32_t*)D, Q, 32, 4, 32, 512, 128, (float*)D, (float*)D,
                               nullptr), MLA_OK);
  EXPECT(rec.mup.M == 128 && rec.mup.groups == 4 && rec.mu_f32);   // 4 blocks, up to 8 wanted
  EXPECT_EQ(mla_merge_unabsorb(D, MLA_BF16, (float*)D, (int32_t*)D, Q, 1, 1, 1, 512, 128, (float*)D, nullptr,
                               nullptr), MLA_OK);
  EXPECT(rec.mup.groups == 1);
  EXPECT_EQ(mla_merge_unabsorb(D, MLA_BF16, (float*)D, (int32_t*)D, Q, 1, 1024, 1, 512, 128, (float*)D, nullptr,
                               nullptr), MLA_OK);
  EXPECT(rec.mup.groups == 32);                                   // 32 blocks of one head
  const int mu_calls = rec.merge_unabsorb;
  EXPECT_EQ(mla_merge_unabsorb(D, MLA_BF16, (float*)D, (int32_t*)D, Q, 64, 1, 128, 256, 128, (float*)D, nullptr,
                               nullptr), MLA_ERR_UNSUPPORTED);
  EXPECT_EQ(mla_merge_unabsorb(D, MLA_BF16, (float*)D, (int32_t*)D, Q, 64, 1, 129, 512, 128, (float*)D, nullptr,
                               nullptr), MLA_ERR_UNSUPPORTED);
  EXPECT_EQ(mla_merge_unabsorb(D, (mla_dtype)7, (float*)D, (int32_t*)D, Q, 64, 1, 128, 512, 128, (float*)D,
                               nullptr, nullptr), MLA_ERR_UNSUPPORTED);
  EXPECT_EQ(mla_merge_unabsorb(D, MLA_BF16, (float*)Dmis, (int32_t*)D, Q, 64, 1, 128, 512, 128, (float*)D, nullptr,
                               nullptr), MLA_ERR_ALIGN);
  EXPECT_EQ(mla_merge_unabsorb(D, MLA_BF16, (float*)D, (int32_t*)D, Q, 64, 1, 128, 512, 128, (float*)D,
                               (float*)Dmis, nullptr), MLA_ERR_ALIGN);
  EXPECT_EQ(mla_merge_unabsorb(nullptr, MLA_BF16, (float*)D, (int32_t*)D, Q, 64, 1, 128, 512, 128, (float*)D,
                               nullptr, nullptr), MLA_ERR_NULL);
  EXPECT_EQ(mla_merge_unabsorb(D, MLA_BF16, (float*)D, (int32_t*)D, Q, -1, 1, 128, 512, 128, (float*)D, nullptr,
                               nullptr), MLA_ERR_SHAPE);
  EXPECT_EQ(mla_merge_unabsorb(D, MLA_BF16, (float*)D, (int32_t*)D, Q, 1 << 24, 2, 1, 512, 128, (float*)D, nullptr,
                               nullptr), MLA_ERR_SHAPE);
  EXPECT_EQ(rec.merge_unabsorb, mu_calls);                        // nothing launched on an error
  EXPECT_EQ(mla_merge_unabsorb(nullptr, MLA_BF16, nullptr, nullptr, nullptr, 0, 1, 128, 512, 128, nullptr, nullptr,
                               nullptr), MLA_OK);
  EXPECT_EQ(rec.merge_unabsorb, mu_calls);
  EXPECT_EQ(mla_append_cache(Q, Q, (uint16_t*)D, 4096, 64, (int32_t*)D, 64, (int32_t*)D, 64, 1, 512, 64, nullptr),
            MLA_OK);
  EXPECT_EQ(mla_append_cache(Q, Q, (uint16_t*)D, 4096, 64, (int32_t*)D, 64, (int32_t*)D, 64, 0, 512, 64, nullptr),
            MLA_ERR_SHAPE);
  EXPECT_EQ(mla_append_cache(Q, Q, (uint16_t*)D, 0, 64, (int32_t*)D, 64, (int32_t*)D, 64, 1, 512, 64, nullptr),
            MLA_ERR_SHAPE);
  int S = 0;
  EXPECT_EQ(mla_sparse_split_count(64, 1, 128, 2048, 0, &S), MLA_OK);
  EXPECT_EQ(S, 4);
  EXPECT_EQ(mla_sparse_split_count(1, 1, 128, 100000, 0, &S), MLA_OK);
  EXPECT_EQ(S, 128);
  EXPECT_EQ(mla_sparse_split_count(1, 1, 128, 2048, 0, nullptr), MLA_ERR_NULL);
  rec = Rec{};
  EXPECT_EQ(mla_decode_sparse(Q, Q, Q, 512, 64, (int32_t*)D, 2048, nullptr, 64, 1, 128, 512, 64, 0.07f, 0, D,
                              MLA_BF16, (float*)D, (int32_t*)D, D, MLA_BF16, nullptr, nullptr), MLA_OK);
  EXPECT(rec.decode == 1 && rec.sparse && rec.split && rec.dp.n_units == 256 && rec.merge == 1);
  rec = Rec{};
  EXPECT_EQ(mla_decode_sparse(Q, Q, Q, 512, 64, (int32_t*)D, 2048, nullptr, 64, 1, 128, 512, 64, 0.07f, 1, nullptr,
                              MLA_BF16, nullptr, nullptr, D, MLA_BF16, nullptr, nullptr), MLA_OK);
  EXPECT(rec.decode == 1 && !rec.split && rec.dp.n_units == 64);
  rec = Rec{};
  EXPECT_EQ(mla_decode_sparse_fp8(Q, Q, (const uint8_t*)D, 512, 64, (int32_t*)D, 2048, nullptr, 64, 1, 128, 512, 64,
                                  0.07f, 0, D, MLA_BF16, (float*)D, (int32_t*)D, D, MLA_BF16, nullptr, nullptr),
            MLA_OK);
  EXPECT(rec.decode == 1 && rec.sparse && rec.fp8 && rec.split && rec.merge == 1);
  EXPECT_EQ(mla_decode_sparse(Q, Q, Q, 1 << 27, 64, (int32_t*)D, 2048, nullptr, 64, 1, 128, 512, 64, 0.07f, 1,
                              nullptr, MLA_BF16, nullptr, nullptr, D, MLA_BF16, nullptr, nullptr),
            MLA_ERR_UNSUPPORTED);   // more than 2^32 - 1 rows
  EXPECT_EQ(mla_decode_sparse(Q, Q, Q, 512, 64, (int32_t*)D, 2048, nullptr, 64, 1, 128, 512, 64, 0.07f, 4, nullptr,
                              MLA_BF16, (float*)D, (int32_t*)D, D, MLA_BF16, nullptr, nullptr), MLA_ERR_WORKSPACE);
}

void test_validate_inputs() {
  // exact-size host arrays stand in for device memory (the stub copy reads them)
  const int B = 3, mb = 5, P = 16, nb = 40;
  std::vector<int32_t> sl = {1, 80, 33};
  std::vector<int32_t> bt(B * mb, -1);
  for (int b = 0; b < B; ++b)
    for (int pg = 0; pg < (sl[b] + P - 1) / P; ++pg) bt[b * mb + pg] = (7 * b + 3 * pg) % nb;
  EXPECT_EQ(mla_validate_inputs(bt.data(), mb, sl.data(), B, 1, 80, P, nb, nullptr), MLA_OK);
  bt[1 * mb + 4] = nb;   // a needed entry past the pool
  EXPECT_EQ(mla_validate_inputs(bt.data(), mb, sl.data(), B, 1, 80, P, nb, nullptr), MLA_ERR_INVALID_INDEX);
  bt[1 * mb + 4] = 0;
  bt[2 * mb + 3] = 12345;   // not needed (sequence 2 has 3 pages): ignored
  EXPECT_EQ(mla_validate_inputs(bt.data(), mb, sl.data(), B, 1, 80, P, nb, nullptr), MLA_OK);
  sl[0] = 81;   // longer than max_seqlen
  EXPECT_EQ(mla_validate_inputs(bt.data(), mb, sl.data(), B, 1, 80, P, nb, nullptr), MLA_ERR_INVALID_INDEX);
  sl[0] = 1;
  EXPECT_EQ(mla_validate_inputs(bt.data(), mb, sl.data(), B, 2, 80, P, nb, nullptr), MLA_ERR_INVALID_INDEX);  // T > L
  EXPECT_EQ(mla_validate_inputs(bt.data(), 0, sl.data(), B, 1, 80, P, nb, nullptr), MLA_ERR_SHAPE);
}

void test_normal() {
  size_t wsb = 0;
  EXPECT_EQ(mla_normal_workspace_size(4, 1, 128, 4096, 1024, &wsb), MLA_OK);
  rec = Rec{};
  EXPECT_EQ(mla_decode_normal(Q, Q, Q, Q, Q, 256, 64, (int32_t*)D, 64, (int32_t*)D, 4, 1, 128, 128, 64, 128, 512,
                              4096, 0.07f, 1024, D, wsb, (float*)D, nullptr, nullptr), MLA_OK);
  EXPECT(rec.gather == 4 && rec.mha == 4 && rec.gemm == 8);   // 4 chunks, two GEMMs each
  EXPECT_EQ(mla_decode_normal(Q, Q, Q, Q, Q, 256, 64, (int32_t*)D, 64, (int32_t*)D, 4, 1, 128, 128, 64, 128, 512,
                              4096, 0.07f, 1024, D, wsb - 1, (float*)D, nullptr, nullptr), MLA_ERR_WORKSPACE);
  EXPECT_EQ(mla_normal_workspace_size(1 << 16, 1, 128, 4096, 512, &wsb), MLA_ERR_UNSUPPORTED);
}

void test_status_strings() {
  for (int s = 1; s >= -9; --s) EXPECT(mla_status_string(s) != nullptr && std::strlen(mla_status_string(s)) > 0);
}
}  // namespace

int main() {
  test_absorb_unabsorb();
  test_workspace_and_decode();
  test_merge_append_sparse();
  test_validate_inputs();
  test_normal();
  test_status_strings();
  if (failures) {
    std::fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
