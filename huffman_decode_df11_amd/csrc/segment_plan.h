// Address arithmetic of one segment's output, shared by the decode kernels
// and a host program that checks it (df11_bounds_check): every global write
// and every staging access a segment makes is derived here from its two
// segment records alone, never from the exponent stream, so a corrupt
// stream can change decoded values but not where they are written.
//
// [P3] "DFloat11重新定义LLM无损压缩的技术边界" 2.2: the reconstruct phase
// writes each decoded element at the position the prefix sum gives it; here
// a segment's positions are the element range [g0, g1) its records name.
//
// The includer defines DF11_HD (host and device qualifiers for the kernels,
// nothing for a host-only build).
#pragma once

#include <stdint.h>

#ifndef DF11_HD
#define DF11_HD inline
#endif

namespace df11plan {

// Elements [g0, g1) of a segment, staged at stg + (g - gbase) and merged in
// 8-element units from gbase.  valid: the records are consistent (g0 <= g1
// <= n) and the segment fits the staging (head offset, elements and a
// 32-byte tail).  An invalid segment has no units and is skipped whole.
struct SegPlan {
    uint64_t g0, g1, gbase;
    uint32_t head, nunits;
    bool valid;
};

DF11_HD SegPlan plan_segment(uint64_t g0, uint64_t g1, uint64_t n, uint32_t stg_bytes)
{
    SegPlan p;
    p.g0 = g0;
    p.g1 = g1;
    p.gbase = g0 & ~7ull;
    p.head = (uint32_t)(g0 & 7);
    p.valid = g1 <= n && g1 >= g0 && (uint64_t)p.head + (g1 - g0) + 32 <= stg_bytes;
    p.nunits = p.valid ? (uint32_t)((((g1 + 7) & ~7ull) - p.gbase) >> 3) : 0u;
    return p;
}

// Unit ui of a plan covers elements [gbase + 8 ui, + 8); it is written with
// one 16-byte store when it lies inside [lo, hi).
DF11_HD bool unit_inside(const SegPlan &p, uint64_t lo, uint64_t hi, uint32_t ui)
{
    const uint64_t gs = p.gbase + 8ull * ui;
    return ui < p.nunits && gs >= lo && gs + 8 <= hi;
}

// The ragged ends of [lo, hi): the elements before the first and after the
// last whole 8-element unit, one per lane (lanes 0..7 the head, lanes
// 8..15 the tail).
struct RaggedLane {
    uint64_t g;
    bool act;
};

DF11_HD RaggedLane ragged_lane(uint64_t lo, uint64_t hi, uint32_t lane)
{
    const uint64_t hend = ((lo + 7) & ~7ull) < hi ? ((lo + 7) & ~7ull) : hi;
    const uint64_t t = hi & ~7ull;
    const uint64_t tstart = t > hend ? t : hend;
    RaggedLane r;
    r.g = lane < 8 ? lo + lane : tstart + (lane - 8);
    r.act = lane < 8 ? r.g < hend : (lane < 16 && r.g < hi);
    return r;
}

// A segment inside one 32-row tile of the fused kernel's order (8-column
// groups: element e of a tile is row (e % 256) / 8, column 8 (e / 256) +
// e % 8), written to row-major BF16.  Offsets are relative to the output
// and to the sign+mantissa array.
struct TileSeg {
    uint64_t sm_off;       // sign+mantissa byte of the tile's first element
    uint64_t out_off;      // output element of the tile's first element
    uint32_t lo, hi;       // the segment's elements within the tile
    uint32_t grp_a, grp_b; // first and last column group touched
    uint32_t stg_t;        // staging byte of tile element 0 (modulo 2^32)
};

// tcs: log2 of the tile width; the tile holds 32 << tcs elements.
DF11_HD TileSeg tile_seg(const SegPlan &p, uint32_t tcs, uint32_t tiles_per_row, uint64_t cols, uint32_t stg)
{
    const uint32_t ts = 5 + tcs;
    const uint64_t tile = p.g0 >> ts, tile_start = tile << ts;
    TileSeg q;
    q.lo = (uint32_t)(p.g0 - tile_start);
    q.hi = (uint32_t)(p.g1 - tile_start);
    q.grp_a = q.lo >> 8;
    q.grp_b = (q.hi - 1) >> 8;
    const uint32_t t32 = (uint32_t)tile, rb = t32 / tiles_per_row, cb = t32 - rb * tiles_per_row;
    q.out_off = ((uint64_t)rb << 5) * cols + ((uint64_t)cb << tcs);
    q.sm_off = tile_start;
    q.stg_t = stg + (uint32_t)(tile_start - p.gbase);
    return q;
}

// element offset (in the tile) of a lane's unit in pass k of group batch gb:
// lane l takes row 8k + l / 8 of column group gb + l % 8
DF11_HD uint32_t tile_unit(uint32_t gb, uint32_t k, uint32_t lane)
{
    return ((gb + (lane & 7u)) << 8) + ((8u * k + (lane >> 3)) << 3);
}

DF11_HD bool tile_unit_in(const TileSeg &q, uint32_t gb, uint32_t e0, uint32_t lane)
{
    return gb + (lane & 7u) <= q.grp_b && e0 >= q.lo && e0 + 8 <= q.hi;
}

// output element (relative to the tile's first) of the unit at e0 for lane
DF11_HD uint64_t tile_unit_out(uint32_t gb, uint32_t k, uint32_t lane, uint64_t cols)
{
    const uint32_t r = 8u * k + (lane >> 3), grp = gb + (lane & 7u);
    return (uint64_t)r * cols + (grp << 3);
}

}  // namespace df11plan
