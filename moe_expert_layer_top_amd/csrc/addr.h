// Address arithmetic shared by the host launch code and the GPU kernels, kept free of
// any HIP dependency so that a plain C++ build can check it on the CPU.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define MOE_HD __host__ __device__
#else
#define MOE_HD
#endif

namespace moe {

// A 64-bit address rebuilt from its two 32-bit halves.  On the GPU each half comes out
// of a readfirstlane (a 32-bit lane value made wave-uniform), whose builtin yields a
// signed int: both halves are converted to uint32_t before widening, so a low half with
// bit 31 set can never sign-extend into (and corrupt) the high half.
template <typename Lo, typename Hi>
MOE_HD inline uint64_t join_u32_halves(Lo lo, Hi hi) {
  return (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) |
         static_cast<uint64_t>(static_cast<uint32_t>(lo));
}

// The DMA kernels address a row of a gathered operand with a 32-bit per-lane byte offset
// (row * pitch + column bytes) from a wave-uniform 64-bit base.  Every such offset stays
// below rows * cols * elem_bytes, so the operand is addressable when that product is at
// most 2^32 - 1 bytes.
MOE_HD inline bool lane_offsets_fit_u32(long long elem_bytes, long long rows, long long cols) {
  if (elem_bytes <= 0 || rows < 0 || cols < 0) return false;
  if (rows == 0 || cols == 0) return true;
  // rows * cols * elem_bytes <= 2^32 - 1, without overflowing 64 bits
  const unsigned long long lim = 0xffffffffULL;
  const unsigned long long rc = static_cast<unsigned long long>(rows) * static_cast<unsigned long long>(cols);
  if (rows > static_cast<long long>(lim) || cols > static_cast<long long>(lim)) return false;
  return rc <= lim / static_cast<unsigned long long>(elem_bytes);
}

}  // namespace moe
