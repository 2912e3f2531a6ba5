// Host-side argument checks shared by the C ABI files (pure functions of their
// arguments: no state, no device calls).
#pragma once

#include <cstdint>

#include "../../include/mla_latent.h"

namespace mla_abi {

constexpr int kR = 512, kDR = 64, kDN = 128, kDV = 128;
constexpr int kMaxH = 128, kMaxT = 1024;

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

inline int check_ptr16(const void* p) {
  if (!p) return MLA_ERR_NULL;
  if (!aligned16(p)) return MLA_ERR_ALIGN;
  return MLA_OK;
}
inline int check_ptr4(const void* p) {
  if (!p) return MLA_ERR_NULL;
  if (!aligned4(p)) return MLA_ERR_ALIGN;
  return MLA_OK;
}

inline int check_heads(int T, int H) {
  if (T < 1 || H < 1) return MLA_ERR_SHAPE;
  if (T > kMaxT || H > kMaxH) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

inline bool page_size_ok(int P) { return P >= 16 && P <= 1024 && P % 16 == 0; }

}  // namespace mla_abi
