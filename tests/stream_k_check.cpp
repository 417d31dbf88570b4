// Checks range_begin / range_of of the skinny kernel's unit split against the exact 64-bit
// definitions: range w = [floor(w U / grid), floor((w + 1) U / grid)), and the range holding
// unit u is floor(((u + 1) grid - 1) / U). Exhaustive on small sizes; range boundaries and
// pseudo-random units on sizes up to U = 2^31 - 1, grid = 2^15. Prints "ok" and exits 0, or
// prints the first mismatch and exits 1.
#include <stdint.h>
#include <stdio.h>

#include "stream_k.h"

static int64_t begin_exact(int64_t U, int64_t g, int64_t w) { return w * U / g; }
static int64_t range_exact(int64_t U, int64_t g, int64_t u) { return ((u + 1) * g - 1) / U; }

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint64_t next() {  // xorshift64*
    rng ^= rng >> 12; rng ^= rng << 25; rng ^= rng >> 27;
    return rng * 0x2545F4914F6CDD1Dull;
}

static bool check_unit(const glk::UnitSplit& s, int64_t U, int64_t u) {
    if (u < 0 || u >= U) return true;
    const int64_t want = range_exact(U, s.grid, u);
    const int32_t got = glk::range_of(s, (int32_t)u);
    if (got != want) {
        printf("range_of mismatch U=%lld grid=%d u=%lld: got %d want %lld\n", (long long)U, s.grid,
               (long long)u, got, (long long)want);
        return false;
    }
    return true;
}

static bool check(int64_t U, int32_t g, bool exhaustive) {
    const glk::UnitSplit s = glk::make_unit_split((int32_t)U, g);
    for (int32_t w = 0; w <= g; ++w) {
        const int64_t b = begin_exact(U, g, w);
        if (glk::range_begin(s, w) != b) {
            printf("range_begin mismatch U=%lld grid=%d w=%d: got %d want %lld\n", (long long)U, g, w,
                   glk::range_begin(s, w), (long long)b);
            return false;
        }
        if (!exhaustive)
            for (int64_t d = -2; d <= 2; ++d)
                if (!check_unit(s, U, b + d)) return false;
    }
    if (exhaustive) {
        for (int64_t u = 0; u < U; ++u)
            if (!check_unit(s, U, u)) return false;
    } else {
        for (int i = 0; i < 20000; ++i)
            if (!check_unit(s, U, (int64_t)(next() % (uint64_t)U))) return false;
    }
    return true;
}

int main() {
    long cases = 0;
    for (int64_t U = 1; U <= 700; ++U)
        for (int32_t g = 1; g <= U && g <= 80; ++g, ++cases)
            if (!check(U, g, true)) return 1;
    const int64_t Us[] = {5504, 5505, 6016, 88064, 1000003, 16777215, 16777216, 16777217, 123456789,
                          1073741824, 1073741827, 2147483646, 2147483647};
    const int32_t gs[] = {1, 2, 3, 7, 8, 31, 32, 86, 255, 256, 257, 304, 1000, 1024, 4096, 32767, 32768};
    for (int64_t U : Us)
        for (int32_t g : gs)
            if (g <= U) {
                ++cases;
                if (!check(U, g, false)) return 1;
            }
    for (int i = 0; i < 3000; ++i, ++cases) {
        const int64_t U = 1 + (int64_t)(next() % 2147483647ull);
        int32_t g = 1 + (int32_t)(next() % 32768);
        if (g > U) g = (int32_t)U;
        if (!check(U, g, false)) return 1;
    }
    printf("ok %ld cases\n", cases);
    return 0;
}
