// Balanced contiguous ranges over a flat list of work units (the Stream-K decomposition of the
// spark-kernels post, "stream-k proper"): range w of `grid` is [floor(w U / grid),
// floor((w + 1) U / grid)). Whenever grid is a multiple of the units' natural groups (strips),
// the range boundaries fall on group boundaries, so no range spans two groups.
//
// Every step is 32-bit integer or float arithmetic (U < 2^31, grid <= 2^15): a 64-bit division
// is a long emulated sequence on the GPU's scalar unit, and these run before a kernel's first
// load. Plain C++ with no GPU dependency, so host code and tests use the same functions.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define GLK_HD __host__ __device__
#else
#define GLK_HD
#endif

namespace glk {

struct UnitSplit {
    int32_t grid;  // number of ranges, 1 <= grid <= min(U, 2^15)
    int32_t q, r;  // U = q grid + r, 0 <= r < grid
    float inv;     // grid / U, rounded: only the starting guess of range_of
};

GLK_HD inline UnitSplit make_unit_split(int32_t units, int32_t grid) {
    UnitSplit s;
    s.grid = grid;
    s.q = units / grid;
    s.r = units % grid;
    s.inv = (float)grid / (float)units;
    return s;
}

// first unit of range w, 0 <= w <= grid: floor(w U / grid) = w q + floor(w r / grid), and
// w r < grid^2 <= 2^30
GLK_HD inline int32_t range_begin(const UnitSplit& s, int32_t w) {
    return w * s.q + (int32_t)((uint32_t)(w * s.r) / (uint32_t)s.grid);
}

// the range holding unit u, 0 <= u < U: the largest w with range_begin(w) <= u, which is
// ceil((u + 1) grid / U) - 1. The float estimate is within 0.01 of that quotient (three
// roundings of 2^-24 relative on a value <= 2^15), so its ceiling is off by at most one either
// way, and one exact comparison step fixes it.
GLK_HD inline int32_t range_of(const UnitSplit& s, int32_t u) {
    const float y = (float)(u + 1) * s.inv;
    int32_t w = (int32_t)__builtin_ceilf(y) - 1;
    w = w < 0 ? 0 : (w > s.grid - 1 ? s.grid - 1 : w);
    if (range_begin(s, w) > u) {
        --w;
    } else if (range_begin(s, w + 1) <= u) {
        ++w;
    }
    return w;
}

}  // namespace glk
