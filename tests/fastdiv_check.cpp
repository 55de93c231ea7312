// Host check of the launch-constant division (FastDiv in skinny_internal.h)
// against plain unsigned division: every divisor below 2^17 with the
// quotient boundaries around several multiples and the extremes of x, then
// random 32-bit divisors and numerators.  Prints "ok <checks>" or the first
// mismatch and exits non-zero.
#include <stdint.h>
#include <stdio.h>

#include "../skinny_bf16_decode_amd/csrc/skinny_internal.h"

using skinny::FastDiv;
using skinny::fastdiv_eval;
using skinny::make_fastdiv;

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32()
{
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return (uint32_t)(state >> 16);
}

static long checks = 0;
static bool check(uint32_t x, uint32_t d, const FastDiv &f)
{
    ++checks;
    if (fastdiv_eval(x, f) != x / d) {
        printf("mismatch: x=%u d=%u got %u want %u\n", x, d, fastdiv_eval(x, f), x / d);
        return false;
    }
    return true;
}

static bool check_divisor(uint32_t d)
{
    const FastDiv f = make_fastdiv(d);
    const uint32_t edges[] = {0u, 1u, d - 1u, d, d + 1u, 0xFFFFFFFFu, 0xFFFFFFFEu, 0x80000000u, 0x7FFFFFFFu};
    for (uint32_t x : edges)
        if (!check(x, d, f))
            return false;
    const uint64_t ks[] = {2, 3, 7, 255, 256, 65535, 65536, 1000003};
    for (uint64_t k : ks) {
        const uint64_t m = k * d;
        for (int64_t dx = -1; dx <= 1; ++dx) {
            const uint64_t x = m + dx;
            if (x <= 0xFFFFFFFFull && !check((uint32_t)x, d, f))
                return false;
        }
    }
    for (int i = 0; i < 8; ++i)
        if (!check(next_u32(), d, f))
            return false;
    return true;
}

int main()
{
    for (uint32_t d = 1; d < (1u << 17); ++d)
        if (!check_divisor(d))
            return 1;
    for (int i = 0; i < 200000; ++i) {
        uint32_t d = next_u32() >> (next_u32() % 32);
        if (d == 0)
            d = 1;
        if (!check_divisor(d))
            return 1;
    }
    printf("ok %ld\n", checks);
    return 0;
}
