// Host check of the fused kernel's tile order (qkvx::TileOrder, the same code
// the kernel runs) and of its tile-claim protocol.
//  1. For every order (XCD-lockstep bands, with one or more column ranges per
//     row run, or grouped rows, over the whole grid or destination by
//     destination), queue count and a range of grid shapes:
//     the queue positions name every logical tile exactly once, and coords()
//     maps the logical tiles one to one onto the tile grid.
//  2. The claim protocol, simulated with seeded random interleavings of the
//     workgroups: a workgroup takes positions qfirst and qfirst + stride of its
//     queue, then claims positions from 2 * stride on through the queue's
//     counter; once that queue is used up it reads every counter and claims
//     from the queue with the most positions left, until none is left.  Every
//     tile is run exactly once and every workgroup stops.
//  3. lockstep_bands() and lockstep_csplit() on the benchmark shapes and
//     their exclusions.
//  4. small_div's correction step: from a quotient estimate off by the
//     relative error of the device's approximate reciprocal (a few units of
//     2^-24, bounded here by 2^-22), it returns the exact quotient.
// Prints "ok <count>" or the first failure.
#include <cstdint>
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <random>
#include <vector>

#include "qkvx_internal.h"

using qkvx::TileOrder;

static int fails = 0;
#define CHECK(c, ...)                         \
    do {                                      \
        if (!(c)) {                           \
            if (fails++ < 5) {                \
                printf("FAIL: " __VA_ARGS__); \
                printf("\n");                 \
            }                                 \
        }                                     \
    } while (0)

static bool covers(const TileOrder& o) {
    const int total = o.tiles_m * o.tiles_n;
    // a workgroup's copy with its own queue kept (own()) maps every position of
    // every queue as the plain order does
    for (int w : {0, o.nq / 2, o.nq - 1}) {
        TileOrder k = o;
        k.own(w);
        for (int x = 0; x < o.nq; ++x) {
            if (k.len(x) != o.len(x)) return false;
            for (int i = 0; i < o.len(x); ++i)
                if (k.logical(x, i) != o.logical(x, i)) return false;
        }
    }
    std::vector<int> seen(total, 0), grid(total, 0);
    for (int x = 0; x < o.nq; ++x)
        for (int i = 0; i < o.len(x); ++i) {
            const int l = o.logical(x, i);
            if (l < 0 || l >= total) return false;
            seen[l] += 1;
        }
    for (int l = 0; l < total; ++l) {
        int tm, tn;
        o.coords(l, tm, tn);
        if (tm < 0 || tm >= o.tiles_m || tn < 0 || tn >= o.tiles_n) return false;
        grid[tm * o.tiles_n + tn] += 1;
    }
    for (int l = 0; l < total; ++l)
        if (seen[l] != 1 || grid[l] != 1) return false;
    return true;
}

// The claim protocol of a launch of G workgroups (nq queues), one random
// interleaving: returns true if every tile ran exactly once.
static bool claims_cover(const TileOrder& o, int G, std::mt19937_64& rng) {
    const int nq = o.nq, stride = G / nq;
    const int total = o.tiles_m * o.tiles_n;
    std::vector<unsigned> counter(nq, 0);
    std::vector<int> ran(total, 0);
    struct Wg { int xcd, cur, nxt, cvict; bool done; };
    std::vector<Wg> wgs;
    for (int b = 0; b < G; ++b) {
        Wg w{nq == 1 ? 0 : b % nq, -1, -1, 0, false};
        const int qfirst = nq == 1 ? b : b / nq;
        w.cvict = w.xcd;
        if (qfirst >= o.len(w.xcd)) {
            w.done = true;
        } else {
            w.cur = o.logical(w.xcd, qfirst);
            w.nxt = qfirst + stride < o.len(w.xcd) ? o.logical(w.xcd, qfirst + stride) : -1;
        }
        wgs.push_back(w);
    }
    int live = 0;
    for (auto& w : wgs) live += !w.done;
    long guard = 0;
    while (live > 0) {
        if (++guard > 100L * total + 100000) return false;   // a workgroup that never stops
        Wg& w = wgs[rng() % wgs.size()];
        if (w.done) continue;
        ran[w.cur] += 1;                                    // the current tile runs
        if (w.nxt < 0) {
            w.done = true;
            --live;
            continue;
        }
        int t = -1;
        int reply = int(counter[w.cvict]++);               // claim the tile after nxt
        for (;;) {
            const int idx = 2 * stride + reply;
            if (idx < o.len(w.cvict)) {
                t = o.logical(w.cvict, idx);
                break;
            }
            int best = -1, most = 0;                        // the fullest queue left
            for (int q = 0; q < nq; ++q) {
                const int left = o.len(q) - (2 * stride + int(counter[q]));
                if (left > most) {
                    most = left;
                    best = q;
                }
            }
            if (best < 0) break;
            w.cvict = best;
            reply = int(counter[w.cvict]++);
        }
        w.cur = w.nxt;
        w.nxt = t;
    }
    for (int l = 0; l < total; ++l)
        if (ran[l] != 1) return false;
    return true;
}

int main() {
    std::mt19937_64 rng(20261203);
    long checked = 0;
    // 1 + 2: orders over grid shapes, queue counts and band counts
    for (int tm = 1; tm <= 80; ++tm)
        for (int tn : {1, 2, 3, 5, 12, 48, 72, 84}) {
            for (int nq : {1, 8}) {
                std::vector<int> band_counts = {0};
                // bands of fewer than 8 rows leave some queues without rows in a band
                if (nq == 8 && tm >= 8)
                    for (int b = 1; b <= 4 && b <= tm; ++b) band_counts.push_back(b);
                for (int bands : band_counts)
                    for (int cs : {1, 2, 4, 8}) {
                        // column ranges apply to banded orders of 8 queues
                        if (cs > 1 && (bands == 0 || cs > tn)) continue;
                        const TileOrder o(tm, tn, 8, nq, bands, 0, 0, cs);
                        CHECK(covers(o), "order tm %d tn %d nq %d bands %d csplit %d", tm, tn, nq,
                              bands, cs);
                        ++checked;
                        const int total = tm * tn;
                        for (int G : {8, 64, 248, 256}) {
                            int g = total < G ? total : G;
                            if (nq == 8 && g % 8 != 0) continue;
                            if (nq == 1 && g % 8 == 0 && g > 1) g -= 1;
                            if (g < 1) continue;
                            for (int rep = 0; rep < 3; ++rep) {
                                CHECK(claims_cover(o, g, rng),
                                      "claims tm %d tn %d nq %d bands %d csplit %d G %d", tm, tn,
                                      nq, bands, cs, g);
                                ++checked;
                            }
                        }
                    }
            }
        }
    // destination by destination (readiness words): dest_cols tile columns per
    // destination and part, grouped or in lockstep bands
    for (int tm = 1; tm <= 40; ++tm)
        for (int dc : {1, 2, 3, 7})
            for (int world : {1, 2, 4, 8})
                for (int nq : {1, 8})
                    for (int bands = 0; bands <= 2; ++bands)
                        for (int cs : {1, 2, 4}) {
                            if (bands > 0 && (nq != 8 || tm < 8)) continue;
                            if (cs > 1 && (bands == 0 || cs > 3 * dc)) continue;
                            const int part_cols = dc * world;
                            const TileOrder o(tm, 3 * part_cols, 8, nq, bands, dc, part_cols, cs);
                            CHECK(covers(o), "dest-major tm %d dc %d world %d nq %d bands %d cs %d",
                                  tm, dc, world, nq, bands, cs);
                            const int total = tm * 3 * part_cols;
                            int g = total < 248 ? total : 248;
                            if (nq == 8) g -= g % 8;
                            if (g >= 1) {
                                CHECK(claims_cover(o, g, rng),
                                      "dest-major claims tm %d dc %d world %d bands %d cs %d", tm,
                                      dc, world, bands, cs);
                                ++checked;
                            }
                            ++checked;
                        }
    // 3: band counts of the benchmark shapes (256 x 256 tiles, 256 workgroups)
    CHECK(qkvx::lockstep_bands(37, 7168, 256, 256, 8) == 1, "56-head U4 bands");
    CHECK(qkvx::lockstep_bands(74, 7168, 256, 256, 8) == 2, "56-head U2 bands");
    CHECK(qkvx::lockstep_bands(64, 6144, 256, 256, 8) == 1, "48-head U8 bands");
    CHECK(qkvx::lockstep_bands(16, 4096, 256, 256, 8) == 1, "32-head bands");
    CHECK(qkvx::lockstep_bands(37, 7168, 256, 248, 8) == 1, "readiness grid of 248");
    CHECK(qkvx::lockstep_bands(7, 7168, 256, 256, 8) == 0, "fewer rows than XCDs");
    CHECK(qkvx::lockstep_bands(37, 7168, 256, 250, 8) == 0, "grid not a multiple of 8");
    CHECK(qkvx::lockstep_bands(400, 8192, 256, 256, 8) == 8, "bands of at most 50 rows");
    CHECK(qkvx::lockstep_bands(9, 65536, 256, 256, 8) == 2, "bands of up to 8 rows when a row exceeds the budget");
    // column ranges: the 32-head shape's 16 rows in one band run as 4 x 8
    // tiles per XCD (two ranges); the others keep one range
    CHECK(qkvx::lockstep_csplit(16, 48, 1, 256, 8) == 2, "32-head column ranges");
    CHECK(qkvx::lockstep_csplit(37, 84, 1, 256, 8) == 1, "56-head U4 column ranges");
    CHECK(qkvx::lockstep_csplit(74, 84, 2, 256, 8) == 1, "56-head U2 column ranges");
    CHECK(qkvx::lockstep_csplit(64, 72, 1, 256, 8) == 1, "48-head U8 column ranges");
    CHECK(qkvx::lockstep_csplit(37, 84, 1, 248, 8) == 1, "readiness grid of 248");
    CHECK(qkvx::lockstep_csplit(8, 84, 1, 256, 8) == 4, "one row per XCD");
    CHECK(qkvx::lockstep_csplit(8, 3, 1, 256, 8) == 2, "ranges of at least one column");
    CHECK(qkvx::lockstep_csplit(37, 84, 0, 256, 8) == 1, "no bands");
    checked += 17;
    // 4: the division's correction step from perturbed estimates
    {
        std::uniform_int_distribution<int> da(0, (1 << 22) - 1), db(1, (1 << 22) - 1);
        auto one = [&](int a, int b) {
            const double t = double(a) / double(b);
            for (double e : {-1.0, 0.0, 1.0}) {
                const int est = int(float(t * (1.0 + e * std::ldexp(1.0, -22))));
                const int q = qkvx::div_fix(a, b, est);
                CHECK(q == a / b, "div_fix a %d b %d est %d -> %d", a, b, est, q);
            }
            CHECK(qkvx::small_div(a, b) == a / b, "small_div a %d b %d", a, b);
            ++checked;
        };
        for (int b = 1; b <= 600; ++b)
            for (int k : {0, 1, 2, 7, 100, 1000, 6000})
                for (int d : {-1, 0, 1}) {
                    const long a = long(k) * b + d;
                    if (a >= 0 && a < (1 << 22)) one(int(a), b);
                }
        for (int i = 0; i < 200000; ++i) one(da(rng), std::max(1, db(rng) >> (i % 20)));
    }
    if (fails) {
        printf("%d failures\n", fails);
        return 1;
    }
    printf("ok %ld\n", checked);
    return 0;
}
