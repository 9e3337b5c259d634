// Host check of the vector-body heads (line_head16, line_head32 in
// zr_internal.hpp) over every address phase in two 128-byte lines and lengths
// around the head sizes: the head never exceeds 63 elements or the length; the
// leading array starts a 128-byte line there (so the fp32 array keeps the
// 16-byte phase its vector body needs); the 2-byte array starts a line there
// too whenever one element index puts both on lines.  Prints "ok: <count>".
#include <cstdint>
#include <cstdio>

#include "zr_internal.hpp"

using zr::line_head16;
using zr::line_head32;

static int fails = 0;

static void check(bool c, const char *what, uintptr_t f, uintptr_t b, int64_t n, int64_t h)
{
    if (!c && fails++ < 20)
        std::printf("FAIL %s: f32 at %#lx, b16 at %#lx, n %lld -> head %lld\n", what, (unsigned long)f,
                    (unsigned long)b, (long long)n, (long long)h);
}

int main()
{
    const int64_t lengths[] = {0, 1, 3, 31, 62, 63, 64, 65, 1000, int64_t(1) << 40};
    const uintptr_t bases[] = {0x100000, 0x7f0000001000ull};
    long count = 0;
    for (uintptr_t base : bases)
        for (int64_t n : lengths) {
            for (uintptr_t b = 0; b < 256; b += 2) {
                const uintptr_t bb = base + b;
                const int64_t h = line_head16(reinterpret_cast<const void *>(bb), n);
                check(h >= 0 && h <= 63 && h <= n, "16: range", 0, bb, n, h);
                if (n >= 64)
                    check((bb + 2 * (uintptr_t)h) % 128 == 0, "16: on a line", 0, bb, n, h);
                ++count;
            }
            for (uintptr_t f = 0; f < 256; f += 4)
                for (uintptr_t b = 0; b < 256; b += 2) {
                    const uintptr_t ff = base + f, bb = base + 0x40000 + b;
                    const int64_t h = line_head32(reinterpret_cast<const float *>(ff), reinterpret_cast<const void *>(bb), n);
                    check(h >= 0 && h <= 63 && h <= n, "32: range", ff, bb, n, h);
                    if (n >= 64) {
                        check((ff + 4 * (uintptr_t)h) % 128 == 0, "32: f32 on a line", ff, bb, n, h);
                        bool both = false;
                        for (int64_t j = 0; j < 64; ++j)
                            both = both || ((ff + 4 * j) % 128 == 0 && (bb + 2 * j) % 128 == 0);
                        if (both)
                            check((bb + 2 * (uintptr_t)h) % 128 == 0, "32: b16 on a line when possible", ff, bb, n, h);
                        else
                            check(h < 32, "32: f32's own head otherwise", ff, bb, n, h);
                    }
                    ++count;
                }
        }
    if (fails) {
        std::printf("%d failures\n", fails);
        return 1;
    }
    std::printf("ok: %ld cases\n", count);
    return 0;
}
