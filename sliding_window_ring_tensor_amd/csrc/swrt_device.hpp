// swrt_device.hpp -- shared device/host helpers of libswrt (gfx950).
//
// Payload is moved as raw bits in 1/2/4/8/16-byte words; no element is ever
// interpreted, so every type (bf16, fp8 encodings, NaN payloads, -0, int4
// pairs, complex) round-trips bit-exactly.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <initializer_list>

#include "swrt.h"

namespace swrt {

constexpr int kBlock = 256;  // threads per workgroup of the small kernels (4 wave64s)

// ---------------------------------------------------------------------------
// raw-bit words
// ---------------------------------------------------------------------------
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int VEC> struct Word;
template <> struct Word<1> { using T = uint8_t; };
template <> struct Word<2> { using T = uint16_t; };
template <> struct Word<4> { using T = uint32_t; };
template <> struct Word<8> { using T = u32x2; };
template <> struct Word<16> { using T = u32x4; };

// Streaming access: every byte of the path is read once and written once, so
// the non-temporal hint keeps the copies from displacing other data in the
// caches. Plain loads and stores otherwise.
#ifndef SWRT_NONTEMPORAL
#define SWRT_NONTEMPORAL 1
#endif
#ifndef SWRT_NT_LOADS
#define SWRT_NT_LOADS SWRT_NONTEMPORAL
#endif
#ifndef SWRT_NT_STORES
#define SWRT_NT_STORES SWRT_NONTEMPORAL
#endif

template <typename T>
__device__ __forceinline__ T ld(const T *p) {
#if SWRT_NT_LOADS
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}

template <typename T>
__device__ __forceinline__ void st(T *p, T v) {
#if SWRT_NT_STORES
  __builtin_nontemporal_store(v, p);
#else
  *p = v;
#endif
}

// a 64-bit value that is equal on every lane of the wave, from its first lane
// (it then lives in scalar registers)
__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
  const uint32_t lo = uint32_t(__builtin_amdgcn_readfirstlane(int32_t(uint32_t(v))));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readfirstlane(int32_t(uint32_t(v >> 32))));
  return (uint64_t(hi) << 32) | lo;
}

// ---------------------------------------------------------------------------
// n / d for 0 <= n < 2^31 with a precomputed multiplier (round-up method:
// l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1, q = (mulhi(n, m) + n) >> l).
// ---------------------------------------------------------------------------
struct FastDiv {
  uint32_t d = 1, m = 1, l = 0;

  FastDiv() = default;
  __host__ explicit FastDiv(uint32_t divisor) : d(divisor) {
    l = 0;
    while ((uint64_t(1) << l) < divisor) ++l;
    m = uint32_t(((uint64_t(1) << 32) * ((uint64_t(1) << l) - divisor)) / divisor + 1);
  }
  __host__ __device__ __forceinline__ uint32_t div(uint32_t n) const {
#if defined(__HIP_DEVICE_COMPILE__)
    const uint32_t t = __umulhi(n, m);
#else
    const uint32_t t = uint32_t((uint64_t(n) * m) >> 32);
#endif
    return (t + n) >> l;
  }
};

// ---------------------------------------------------------------------------
// host-side helpers
// ---------------------------------------------------------------------------
inline bool valid_elem_bits(int bits) {
  return bits == 4 || bits == 8 || bits == 16 || bits == 32 || bits == 64 || bits == 128;
}

// Largest word (16, 8, 4, 2, 1 bytes) dividing `bytes` and every address /
// stride in `vals`.
inline int pick_vec(uint64_t bytes, std::initializer_list<uint64_t> vals) {
  int v = 16;
  while (v > 1) {
    bool ok = (bytes % v) == 0;
    for (uint64_t x : vals) ok = ok && (x % v) == 0;
    if (ok) break;
    v >>= 1;
  }
  return v;
}

// [a, a+na) and [b, b+nb) overlap (empty ranges never do)
inline bool overlaps(const void *a, uint64_t na, const void *b, uint64_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// A byte range a call touches; `written` ranges may overlap nothing else,
// read-only ranges may overlap each other.
struct Range {
  uintptr_t lo, hi;  // [lo, hi)
  bool written;
};

// true when some written range overlaps any other range. Sort by start, then
// sweep: an earlier range p overlaps the current one c iff p.hi > c.lo.
inline bool written_overlap(Range *r, int n) {
  std::sort(r, r + n, [](const Range &x, const Range &y) { return x.lo < y.lo; });
  uintptr_t max_hi_any = 0, max_hi_written = 0;
  bool seen = false;
  for (int i = 0; i < n; ++i) {
    if (r[i].hi == r[i].lo) continue;  // empty
    if (seen && (r[i].lo < max_hi_written || (r[i].written && r[i].lo < max_hi_any))) return true;
    seen = true;
    max_hi_any = std::max(max_hi_any, r[i].hi);
    if (r[i].written) max_hi_written = std::max(max_hi_written, r[i].hi);
  }
  return false;
}

inline Range range(const void *p, uint64_t n, bool written) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, p ? a + n : a, written};
}

// a * b into *out; false on overflow of int64
inline bool mul_ok(int64_t a, int64_t b, int64_t *out) {
  return !__builtin_mul_overflow(a, b, out);
}

inline int launch_status() {
  return hipGetLastError() == hipSuccess ? SWRT_OK : SWRT_E_LAUNCH;
}

}  // namespace swrt
