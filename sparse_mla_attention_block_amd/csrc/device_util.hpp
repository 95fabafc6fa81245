// Device helpers shared by the kernel files (decode and writer).  Kept out
// of internal.hpp so that the host-side sources compile with any C++ host
// compiler.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsv4 {

// Two bf16 with any NaN or infinite half replaced by +0.  A half is not
// finite when its magnitude bits are >= 0x7F80 (all exponent bits set);
// adding 0x80 to the magnitude then sets bit 15 of that half, with no carry
// into the other half, and an arithmetic shift by 15 spreads bit 15 into a
// half-wide mask.
__device__ __forceinline__ uint32_t scrub_pair(uint32_t w) {
    typedef int16_t i16x2 __attribute__((ext_vector_type(2)));
    const uint32_t t = (w & 0x7FFF7FFFu) + 0x00800080u;
    const uint32_t bad = __builtin_bit_cast(uint32_t, __builtin_bit_cast(i16x2, t) >> (int16_t)15);
    return w & ~bad;
}

}  // namespace dsv4
