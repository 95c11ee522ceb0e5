// Internal helpers shared by the host and device translation units of libpagedattn.so.
#pragma once

#include <cstdarg>
#include <cstdint>

#include "pagedattn.h"

namespace pa {

// Records a message as the calling thread's last error and returns `code`.
int set_error(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clears the calling thread's last error and returns PA_OK.
int clear_error();

inline bool is_pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }

inline bool block_size_ok(int32_t bs) { return bs >= 16 && bs <= 256 && is_pow2(bs); }

inline bool head_dim_ok(int32_t d) { return d == 64 || d == 128; }

// Largest query-head group one decode task covers (the MFMA column tile is 16 wide).
constexpr int32_t kMaxGroup = 16;
// Largest prefill query tile (rows per workgroup of the MFMA tile kernel).
constexpr int32_t kMaxQTile = 128;
// Key granularity of split boundaries (decode chunks and prefill key tiles both divide it).
constexpr int32_t kSplitQuantum = 64;
// Most workgroups one launch may have along its grid's x dimension: HIP keeps a dimension's
// work-items (workgroups x threads) below 2^32, and the widest workgroup here has 512 threads.
constexpr int32_t kMaxWorkgroups = (1 << 23) - 1;

}  // namespace pa
