// attn_fwd_tile_map.h -- the prefill kernels' workgroup -> tile mapping (16-bit and
// fp32 kernels).  Included by the .hip sources only.
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
__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) {
    return (uint32_t)(((uint64_t)n * f.m) >> f.s);
}
__device__ __forceinline__ TileCoord map_tile(const AttnParams& p, int w) {
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

}  // namespace attn_impl

#endif
