// Host check of qkvx::FastDiv (the multiply-shift divider of the transport
// kernels' index arithmetic) against the hardware division, over the range the
// header states: every divisor d >= 1 and dividend 0 <= n < 2^31.  Divisors:
// 1..4096, powers of two and their neighbours up to 2^31, and seeded random
// ones; dividends: the edges around multiples of d, the top of the range, and
// seeded random ones.  Prints "ok <count>" or the first failure.
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

#include "qkvx_internal.h"

int main() {
    std::mt19937_64 rng(20261202);
    const uint32_t top = 0x7FFFFFFFu;            // largest dividend in range
    std::vector<uint32_t> divisors;
    for (uint32_t d = 1; d <= 4096; ++d) divisors.push_back(d);
    for (int s = 12; s <= 31; ++s)
        for (int e = -2; e <= 2; ++e) {
            const int64_t d = (int64_t(1) << s) + e;
            if (d >= 1 && d <= int64_t(top)) divisors.push_back(uint32_t(d));
        }
    for (int i = 0; i < 4000; ++i) divisors.push_back(uint32_t(1 + rng() % top));
    uint64_t checked = 0;
    for (const uint32_t d : divisors) {
        const qkvx::FastDiv f(d);
        std::vector<uint32_t> ns = {0u, 1u, top, top - 1u};
        const uint32_t last = (top / d) * d;     // largest multiple of d in range
        for (uint32_t base : {d, 2u * d <= top ? 2u * d : d, last}) {
            ns.push_back(base);
            ns.push_back(base - 1u);
            if (base < top) ns.push_back(base + 1u);
        }
        for (int i = 0; i < 64; ++i) ns.push_back(uint32_t(rng() % (uint64_t(top) + 1)));
        for (const uint32_t n : ns) {
            uint32_t q = 0, r = 0;
            f.divmod(n, q, r);
            if (q != n / d || r != n % d || f.div(n) != n / d) {
                std::printf("FAIL d=%u n=%u: got q=%u r=%u, want q=%u r=%u\n", d, n, q, r, n / d,
                            n % d);
                return 1;
            }
            ++checked;
        }
    }
    std::printf("ok %llu\n", (unsigned long long)checked);
    return 0;
}
