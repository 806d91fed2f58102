// attn_fwd_tile_map.h -- the prefill kernels' workgroup -> tile mapping (16-bit and
// fp32 kernels): the host plans it (plan_tile_map), every workgroup decodes its own
// tile (map_tile).  Both sides are plain inline code, so the host test of the mapping
// runs the same functions the kernels do.
#ifndef ATTN_FWD_TILE_MAP_H
#define ATTN_FWD_TILE_MAP_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_fwd_internal.h"

namespace attn_impl {

// Workgroup -> (batch, query head, query tile).  Workgroups are taken in "bundles"
// of p.gbundle consecutive key/value-head groups; inside a bundle the order is
// query tile first (heaviest causal tiles of every head in the bundle before any
// lighter one), then group, then query head.  A bundle is sized (on the host) to
// fill the workgroup slots of an XCD, which keeps the causal tail balanced while
// the K/V heads in flight stay few enough for one XCD's L2.  When the groups split
// evenly over the 8 XCDs (workgroup w is dispatched to XCD w % 8), each XCD gets
// whole bundles, so every query tile and query head that reads one K/V head runs
// on the XCD that caches it.
struct TileCoord { int b, hq, kvh, qt; };
__host__ __device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) {
    return (uint32_t)(((uint64_t)n * f.m) >> f.s);
}
__host__ __device__ __forceinline__ TileCoord map_tile(const AttnParams& p, int w) {
    const uint32_t R = p.R;              // query heads per key/value head
    const uint32_t G = p.gbundle;        // key/value-head groups per bundle
    const uint32_t BU = G * R * p.nq;    // workgroups per bundle
    uint32_t bundle, u;
    if (p.xcd_remap) {
        const uint32_t xcd = w & 7, slot = (uint32_t)w >> 3;
        const uint32_t k = fdiv(slot, p.div_bu);
        bundle = xcd + 8 * k;
        u = slot - k * BU;
    } else {
        bundle = fdiv(w, p.div_bu);
        u = w - bundle * BU;
    }
    TileCoord t;
    t.qt = p.nq - 1 - (int)fdiv(u, p.div_gr);
    const uint32_t ur = fdiv(u, p.div_r);
    const uint32_t g = bundle * G + (ur & (G - 1));
    const uint32_t r = u - ur * R;
    const uint32_t b = fdiv(g, p.div_hkv);
    t.b = b;
    t.kvh = g - b * p.Hkv;
    t.hq = t.kvh * R + r;
    return t;
}

// The multiplier and shift of FastDiv for a divisor d >= 1 (host).
inline FastDiv make_fastdiv(uint32_t d) {
    uint32_t l = 0;
    while (l < 31 && (1u << l) < d) ++l;                 // l = ceil(log2 d)
    const uint32_t s = 31 + l;
    const uint64_t m = (((uint64_t)1 << s) + d - 1) / d;  // ceil(2^s / d) < 2^32
    return FastDiv{(uint32_t)m, s};
}

// Host side of the mapping for `groups` key/value-head groups (B * Hkv) of `per_group`
// workgroups each (R * nq): bundle groups until a bundle holds at least 64 workgroups
// (two rounds of an XCD's 32 CUs), heaviest query tiles of the whole bundle first; the
// bundle count must divide the groups, and whole bundles go to each XCD when the
// bundles split evenly over the 8 XCDs.  Needs p.Hkv, p.nq and R = Hq / Hkv.
inline void plan_tile_map(AttnParams& p, int64_t groups, int64_t per_group, int R) {
    int gb = 1;
    while (gb * per_group < 64 && groups % (2 * gb) == 0) gb *= 2;
    p.gbundle = gb;
    p.xcd_remap = ((groups / gb) % 8 == 0) ? 1 : 0;
    p.R = R;
    p.div_bu = make_fastdiv((uint32_t)((int64_t)gb * per_group));
    p.div_gr = make_fastdiv((uint32_t)(gb * R));
    p.div_r = make_fastdiv((uint32_t)R);
    p.div_hkv = make_fastdiv((uint32_t)p.Hkv);
}

}  // namespace attn_impl

#endif
