// Host check of the prefill kernels' workgroup -> tile mapping, built and run by
// tests/test_tile_map.py.  It calls the mapping's own inline functions
// (attn_fwd_tile_map.h: make_fastdiv, fdiv, plan_tile_map, map_tile) on the host.
//
// Checked:
//   * fdiv(n, make_fastdiv(d)) == n / d for every divisor up to 4096 and a set of
//     larger ones, on the edge numerators of each divisor and on random ones below 2^31;
//   * for each launch shape given on the command line (B Hq Hkv nq), map_tile sends
//     the B * Hq * nq workgroups onto the (batch, query head, query tile) triples
//     one to one, with kvh = hq / (Hq / Hkv);
//   * inside a bundle the query tiles come heaviest first (non-increasing qt in the
//     order the workgroups of one XCD are dispatched);
//   * when the plan remaps bundles to XCDs, every workgroup of one key/value-head
//     group lands on the same XCD (w % 8).
// Prints "ok" and exits 0, or prints the first failure and exits 1.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "attn_fwd_internal.h"
#include "attn_fwd_tile_map.h"

using namespace attn_impl;

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static uint32_t rnd() {             // xorshift64*
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (uint32_t)((rng_state * 0x2545f4914f6cdd1dull) >> 32);
}

static int check_div(uint32_t d) {
    const FastDiv f = make_fastdiv(d);
    const uint32_t top = 0x7fffffffu;
    uint32_t ns[] = {0u, 1u, d - 1, d, d + 1, 2 * d - 1, 2 * d, top, top - 1, top - d,
                     (top / d) * d, (top / d) * d - 1};
    for (uint32_t n : ns) {
        if (n > top) continue;
        if (fdiv(n, f) != n / d) {
            printf("fdiv(%u, %u) = %u, want %u\n", n, d, fdiv(n, f), n / d);
            return 1;
        }
    }
    for (int i = 0; i < 2000; ++i) {
        const uint32_t n = rnd() & top;
        if (fdiv(n, f) != n / d) {
            printf("fdiv(%u, %u) = %u, want %u\n", n, d, fdiv(n, f), n / d);
            return 1;
        }
    }
    return 0;
}

static int check_map(int B, int Hq, int Hkv, int nq) {
    AttnParams p = {};
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.nq = nq;
    const int R = Hq / Hkv;
    const int64_t groups = (int64_t)B * Hkv, per_group = (int64_t)R * nq;
    plan_tile_map(p, groups, per_group, R);
    const int64_t nwg = groups * per_group;
    std::vector<int> seen((size_t)nwg, 0);
    std::vector<int> xcd_of_group((size_t)groups, -1);
    std::vector<int> last_qt(8, 1 << 30), last_bundle(8, -1);
    const int64_t bu = (int64_t)p.gbundle * per_group;
    for (int64_t w = 0; w < nwg; ++w) {
        const TileCoord t = map_tile(p, (int)w);
        if (t.b < 0 || t.b >= B || t.hq < 0 || t.hq >= Hq || t.qt < 0 || t.qt >= nq ||
            t.kvh != t.hq / R) {
            printf("B%d Hq%d Hkv%d nq%d: workgroup %lld -> (b %d, hq %d, kvh %d, qt %d) out of range\n",
                   B, Hq, Hkv, nq, (long long)w, t.b, t.hq, t.kvh, t.qt);
            return 1;
        }
        const int64_t idx = ((int64_t)t.b * Hq + t.hq) * nq + t.qt;
        if (seen[(size_t)idx]++) {
            printf("B%d Hq%d Hkv%d nq%d: tile (b %d, hq %d, qt %d) mapped twice\n", B, Hq, Hkv, nq,
                   t.b, t.hq, t.qt);
            return 1;
        }
        // dispatch order within the stream of one XCD (or of the whole launch)
        const int lane = p.xcd_remap ? (int)(w & 7) : 0;
        const int64_t slot = p.xcd_remap ? (w >> 3) : w;
        const int bundle = (int)(slot / bu);
        if (bundle != last_bundle[lane]) {
            last_bundle[lane] = bundle;
            last_qt[lane] = 1 << 30;
        }
        if (t.qt > last_qt[lane]) {
            printf("B%d Hq%d Hkv%d nq%d: query tile %d after %d inside a bundle\n", B, Hq, Hkv, nq,
                   t.qt, last_qt[lane]);
            return 1;
        }
        last_qt[lane] = t.qt;
        if (p.xcd_remap) {
            const int64_t g = (int64_t)t.b * Hkv + t.kvh;
            int& x = xcd_of_group[(size_t)g];
            if (x < 0) x = (int)(w & 7);
            if (x != (int)(w & 7)) {
                printf("B%d Hq%d Hkv%d nq%d: group %lld on XCDs %d and %d\n", B, Hq, Hkv, nq,
                       (long long)g, x, (int)(w & 7));
                return 1;
            }
        }
    }
    for (int64_t i = 0; i < nwg; ++i)
        if (!seen[(size_t)i]) {
            printf("B%d Hq%d Hkv%d nq%d: tile %lld never mapped\n", B, Hq, Hkv, nq, (long long)i);
            return 1;
        }
    return 0;
}

int main(int argc, char** argv) {
    for (uint32_t d = 1; d <= 4096; ++d)
        if (check_div(d)) return 1;
    const uint32_t big[] = {4097u, 65535u, 65536u, 65537u, 1000003u, (1u << 20) + 7,
                            (1u << 30) - 1, 1u << 30, (1u << 30) + 1, 0x7fffffffu};
    for (uint32_t d : big)
        if (check_div(d)) return 1;
    if ((argc - 1) % 4 != 0) {
        printf("usage: %s [B Hq Hkv nq]...\n", argv[0]);
        return 2;
    }
    for (int a = 1; a + 3 < argc; a += 4) {
        const int B = atoi(argv[a]), Hq = atoi(argv[a + 1]), Hkv = atoi(argv[a + 2]), nq = atoi(argv[a + 3]);
        if (check_map(B, Hq, Hkv, nq)) return 1;
    }
    printf("ok\n");
    return 0;
}
