// Internal helpers shared by the HIP sources of libengram.so (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/engram.h"

namespace engram {

// Record a one-line failure description for engram_last_error() and return `status`.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// ENGRAM_EHIP with the runtime's message if the last launch failed, else ENGRAM_OK.
int check_launch(const char* what);

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// 16-byte vector of 32-bit words: the unit of every wide global access.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

}  // namespace engram
