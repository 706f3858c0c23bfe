// kda_bounds.h -- the one rule every kernel applies to sequence offsets read
// from cu_seqlens.  Plain C++ with no HIP dependency: constexpr functions are
// callable from device code under hipcc, and the host tests compile this
// header with g++ to check the rule on malformed offsets.
#pragma once

#include <stdint.h>

namespace kda {

struct SeqRange {
    int64_t a, b;  // tokens [a, b)
};

// Token range of a sequence whose offsets read x = cu[n], y = cu[n + 1], in a
// tensor of T tokens: both bounds are clamped to [0, T] and b to at least a.
// Well-formed offsets (0 <= x <= y <= T) pass unchanged; malformed ones can
// change which tokens a sequence covers, never make it reach outside the
// tensor.
constexpr SeqRange clamp_seq(int64_t x, int64_t y, int64_t T) {
    const int64_t a = x < 0 ? 0 : (x > T ? T : x);
    const int64_t b = y < a ? a : (y > T ? T : y);
    return SeqRange{a, b};
}

}  // namespace kda
