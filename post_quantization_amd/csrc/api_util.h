// Host-side helpers shared by the ABI translation units.
#pragma once

#include <algorithm>
#include <stdint.h>
#include <stddef.h>

#include "common.h"
#include "kernels.h"

namespace omq {

inline hipStream_t S(void* stream) { return reinterpret_cast<hipStream_t>(stream); }
inline bool dt_ok(int dt) { return dt == OMQ_F32 || dt == OMQ_BF16; }
inline bool bits_ok(int b) { return (b >= 2 && b <= 8) || b == 16; }
inline bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool al4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Carves 256-byte-aligned regions out of a caller-provided workspace; with a NULL
// base it only measures.
struct Bump {
  char* base;
  size_t off = 0;
  explicit Bump(void* b) : base(reinterpret_cast<char*>(b)) {}
  template <typename T>
  T* take(int64_t n) {
    off = (off + 255) & ~size_t(255);
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += (size_t)std::max<int64_t>(n, 0) * sizeof(T);
    return p;
  }
};

}  // namespace omq
