// Device-side bounds checks of the debug build (compiled with -DFKL_DEBUG).
//
// Each kernel carries a DebugCheck: a pointer to a 32-bit violation word in
// the call's workspace and the byte extents (spans) the host planned for the
// buffers the kernel touches. In the debug build every checked global access
// is compared with its span first; an access outside it is skipped (a load
// returns zero) and sets the access class's bit in the word, so nothing ever
// reads or writes out of bounds and no kernel traps. The entry point clears
// the word before its first launch, synchronises after its last, and returns
// FKL_EDEVICE naming the classes that fired. In the release build DebugCheck
// is empty and dload / dstore are plain accesses.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <cstdlib>
#include <initializer_list>

#include "fkl_internal.h"

namespace fkl {

constexpr int kDebugSpans = 6;

struct DebugSpan {
  const char* lo;
  uint64_t bytes;
};

#ifdef FKL_DEBUG
struct DebugCheck {
  uint32_t* word;
  DebugSpan s[kDebugSpans];
};

__device__ __forceinline__ bool dbg_in(const DebugCheck& d, int span, uint32_t bit, const void* p, uint64_t n) {
  const char* c = static_cast<const char*>(p);
  const DebugSpan& s = d.s[span];
  if (s.lo != nullptr && c >= s.lo && n <= s.bytes && static_cast<uint64_t>(c - s.lo) <= s.bytes - n) return true;
  atomicOr(d.word, bit);
  return false;
}
#else
struct DebugCheck {};
#endif

// *p, or T{} (and the class's bit set) when p lies outside span `span`.
template <class T>
__device__ __forceinline__ T dload(const DebugCheck& d, int span, uint32_t bit, const T* p) {
#ifdef FKL_DEBUG
  if (!dbg_in(d, span, bit, p, sizeof(T))) return T{};
#else
  (void)d, (void)span, (void)bit;
#endif
  return *p;
}

// *p = v, skipped (and the class's bit set) when p lies outside span `span`.
template <class T>
__device__ __forceinline__ void dstore(const DebugCheck& d, int span, uint32_t bit, T* p, const T& v) {
#ifdef FKL_DEBUG
  if (!dbg_in(d, span, bit, p, sizeof(T))) return;
#else
  (void)d, (void)span, (void)bit;
#endif
  *p = v;
}

// Checks that the byte range [p, p + n) lies in span `span` (debug build);
// true in the release build.
__device__ __forceinline__ bool dcheck_range(const DebugCheck& d, int span, uint32_t bit, const void* p,
                                             uint64_t n) {
#ifdef FKL_DEBUG
  return n == 0 || dbg_in(d, span, bit, p, n);
#else
  (void)d, (void)span, (void)bit, (void)p, (void)n;
  return true;
#endif
}

// Host side: a DebugCheck from the word and up to kDebugSpans (pointer, bytes)
// pairs, in span order (the release build ignores them).
struct HostSpan {
  const void* p;
  uint64_t bytes;
};

inline DebugCheck make_debug_check(uint32_t* word, std::initializer_list<HostSpan> spans) {
  DebugCheck d{};
#ifdef FKL_DEBUG
  d.word = word;
  int i = 0;
  for (const HostSpan& s : spans) {
    if (i == kDebugSpans) break;
    d.s[i++] = DebugSpan{static_cast<const char*>(s.p), s.bytes};
  }
#else
  (void)word, (void)spans;
#endif
  return d;
}

// Debug build: FKL_DEBUG_SHRINK_G=1 narrows the gradient block's span by its
// last 4 KiB, so a call that writes the block's last row makes the check fire
// and skip those stores, which stay inside the real block: a test of the
// reporting path. The release build ignores it.
inline uint64_t debug_g_bytes(uint64_t bytes) {
#ifdef FKL_DEBUG
  const char* v = std::getenv("FKL_DEBUG_SHRINK_G");
  if (v && v[0] == '1' && bytes > 4096) return bytes - 4096;
#endif
  return bytes;
}

}  // namespace fkl
