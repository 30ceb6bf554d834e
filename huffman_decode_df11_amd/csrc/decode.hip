// df11_decode: restore BF16 weights from the DFloat11 stream on the GPU,
// right before the matmul that consumes them.
//
// [P1] "DFloat11无损压缩技术：基于哈夫曼编码的BFloat16大模型显存优化方案" 2.2
//      item 3: compressed weights stay in GPU memory; a kernel reads, decodes
//      and restores BF16 just before use, with no CPU work.
// [P3] "DFloat11重新定义LLM无损压缩的技术边界" 2.2: lookup tables in on-chip
//      memory, a locate phase, a prefix sum for positions and a reconstruct
//      phase; 5.2: occupancy is the tuning lever.
//
// Mapping to gfx950: one 64-lane wavefront per segment, so the prefix sum is
// a wavefront scan and no workgroup barrier sits on the decode path.  A
// workgroup of WAVES waves stages the tables in LDS once; each wave then
// walks its segments with the next segment's stream words, gaps and code
// counts and this segment's sign+mantissa bytes already in flight, so
// global-memory latency overlaps the decode.  A lane's stream words stay in
// registers; segment records come through scalar loads.  Exponents are
// staged in LDS and merged with the sign+mantissa bytes in 8-element units,
// lane l of a round taking unit l, so each wave-wide store writes one
// contiguous kilobyte of BF16; the at most 14 elements of a segment's two
// ragged units are written one per lane.  The whole layer decode is bound by
// HBM traffic (the decode itself hides behind it), so the loop is ordered
// for the memory system: loads that the next step needs are issued before
// stores that it need not wait for (loads and stores share one completion
// counter), and launches whose output overflows the last-level cache
// stream it.
#include <hip/hip_runtime.h>

#include <atomic>

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "df11_device.h"
#include "df11_internal.h"

using namespace df11dev;

namespace {

constexpr uint32_t kChunkBytes = 16;
constexpr uint32_t kChunkBits = 8 * kChunkBytes;
constexpr uint32_t kSegWords = 64 * kChunkBytes / 4;
constexpr int kPrefetchRounds = 5;   // 8-element units per lane prefetched before the decode

struct ViewArgs {
    const uint32_t *words;
    const uint8_t *sm;
    const uint8_t *gaps;
    const uint8_t *counts;
    const df11_segment *segs;
    uint16_t *out;
    uint64_t n;
    uint64_t n_segments;
    // tile order (tr == 0: row-major); kc > 0: column groups inside a tile
    uint32_t tr, tc, tiles_per_row, kc;
    uint64_t cols;
    // bit 31 set: tr, tc and kc (when > 0) are powers of two with these
    // shifts in bits 0-4, 5-9 and 10-14 (the fused kernel's layout is), so
    // the placement takes shifts and one 32-bit division
    uint32_t pow2;
    uint32_t reserved;
};

// Up to kMaxBatch views per launch, passed by value; segments of all views
// form one flat index space (view i owns [seg_begin[i], seg_begin[i + 1])).
constexpr uint32_t kMaxBatch = 16;
struct BatchArgs {
    ViewArgs v[kMaxBatch];
    uint64_t seg_begin[kMaxBatch + 1];
    uint32_t count;
    uint32_t stream;          // nonzero: streaming (nontemporal) sign+mantissa loads and BF16 stores
};

// A launch whose BF16 output is larger than the last-level cache (the
// 256 MB Infinity Cache) cannot leave it there for the matmul that follows,
// so it streams: sign+mantissa bytes are read and BF16 written with
// nontemporal accesses, which keeps the write-allocate and eviction of data
// used once out of the cache.  Smaller outputs are written normally and are
// still cache-resident when the consumer reads them.
constexpr uint64_t kStreamOutBytes = 256ull << 20;

typedef unsigned int v2u32 __attribute__((ext_vector_type(2)));
typedef unsigned int v4u32g __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint2 load_sm8(const uint8_t *p, bool stream)
{
    if (stream) {
        const v2u32 t = __builtin_nontemporal_load(reinterpret_cast<const v2u32 *>(p));
        return make_uint2(t.x, t.y);
    }
    return *reinterpret_cast<const uint2 *>(p);
}

__device__ __forceinline__ void store_bf16x8(uint16_t *p, uint4 v, bool stream)
{
    if (stream) {
        const v4u32g t = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(t, reinterpret_cast<v4u32g *>(p));
    } else {
        *reinterpret_cast<uint4 *>(p) = v;
    }
}

__device__ __forceinline__ uint32_t view_of(const BatchArgs &b, uint64_t s, uint32_t i = 0)
{
    while (i + 1 < b.count && b.seg_begin[i + 1] <= s) i++;
    return i;
}

struct TableArgs {
    const uint16_t *chain;
    const uint32_t *fast;
    uint32_t n_chain;         // uint16 entries
    uint32_t stg_bytes;       // per-wave exponent staging bytes
};

__device__ __forceinline__ uint64_t out_index(const ViewArgs &v, uint64_t g)
{
    if (!v.tr) return g;
    if (v.pow2) {
        const uint32_t trs = v.pow2 & 31u, tcs = (v.pow2 >> 5) & 31u, kcs = (v.pow2 >> 10) & 31u;
        const uint32_t ts = trs + tcs;
        const uint32_t t = (uint32_t)(g >> ts), w = (uint32_t)g & ((1u << ts) - 1u);
        uint32_t r, c;
        if (v.kc) {
            const uint32_t gs = trs + kcs, in = w & ((1u << gs) - 1u);
            r = in >> kcs;
            c = ((w >> gs) << kcs) | (in & ((1u << kcs) - 1u));
        } else {
            r = w >> tcs;
            c = w & ((1u << tcs) - 1u);
        }
        const uint32_t rb = t / v.tiles_per_row, cb = t - rb * v.tiles_per_row;
        return (uint64_t)((rb << trs) + r) * v.cols + (cb << tcs) + c;
    }
    const uint64_t tile = (uint64_t)v.tr * v.tc;
    const uint64_t t = g / tile;
    const uint32_t w = (uint32_t)(g - t * tile);
    uint32_t r, c;
    if (v.kc) {
        const uint32_t grp = w / (v.tr * v.kc), in = w - grp * (v.tr * v.kc);
        r = in / v.kc;
        c = grp * v.kc + (in - r * v.kc);
    } else {
        r = w / v.tc;
        c = w - r * v.tc;
    }
    const uint64_t rb = t / v.tiles_per_row, cb = t - rb * v.tiles_per_row;
    return (rb * v.tr + r) * v.cols + cb * v.tc + c;
}

// Segment records are read-only for the whole launch: reading them through
// the constant address space lets the wave fetch them with scalar loads,
// which are tracked apart from the vector loads and stores.
template <class T>
__device__ __forceinline__ const __attribute__((address_space(4))) T *as_const(const T *p)
{
    return (const __attribute__((address_space(4))) T *)p;
}

// Everything a wave needs from global memory to start a segment.  The
// vector part (stream words, gap, stored count) is always loaded from valid
// addresses, so the loads carry no condition and are first waited for where
// the decode uses them.
struct SegLoad {
    uint4 own;          // this lane's 4 stream words
    uint32_t next;      // the following word (look-ahead)
    uint32_t gap;
    uint32_t count;     // codes that start in this lane's chunk (meaningful when the view stores counts)
    uint32_t nbits;
    uint64_t g0, g1;
};

__device__ __forceinline__ SegLoad load_segment(const ViewArgs &v, uint64_t s, uint32_t lane)
{
    SegLoad L;
    const uint32_t *w = v.words + s * kSegWords + lane * 4;
    L.own = *reinterpret_cast<const uint4 *>(w);
    L.next = w[4];
    L.gap = v.gaps[s * 64 + lane];
    const uint8_t *cp = v.counts ? v.counts : v.gaps;
    L.count = cp[s * 64 + lane];
    const auto *rec = as_const(v.segs + s);
    L.g0 = rec[0].elem_off;
    L.g1 = rec[1].elem_off;
    L.nbits = rec[0].nbits;
    return L;
}

// ------------------------------------------------------------ one segment
struct SegPlan {
    uint64_t g0, g1, gbase;   // elements [g0, g1); 8-element units from gbase
    uint32_t head, nunits;
    bool valid;               // records consistent and the segment fits the staging
};

__device__ __forceinline__ SegPlan plan_segment(const SegLoad &cur, uint64_t n, uint32_t stg_bytes)
{
    SegPlan p;
    p.g0 = cur.g0;
    p.g1 = cur.g1;
    p.gbase = p.g0 & ~7ull;
    p.head = (uint32_t)(p.g0 & 7);
    p.valid = p.g1 <= n && p.g1 >= p.g0 && (uint64_t)p.head + (p.g1 - p.g0) + 32 <= stg_bytes;
    p.nunits = p.valid ? (uint32_t)((((p.g1 + 7) & ~7ull) - p.gbase) >> 3) : 0u;
    return p;
}

// the segment's sign+mantissa bytes for the first kPrefetchRounds rounds of
// units.  Lanes past the last unit load the last unit again (an address
// that is always inside the array), so no value has to be selected and the
// loads stay in flight during the decode.
__device__ __forceinline__ void prefetch_sm(const SegPlan &p, const uint8_t *sm, uint32_t lane, bool stream,
                                            uint2 (&smp)[kPrefetchRounds])
{
    const uint32_t last = p.nunits ? p.nunits - 1 : 0u;
    const uint64_t base = p.nunits ? p.gbase : 0ull;
#pragma unroll
    for (int r = 0; r < kPrefetchRounds; r++)
        smp[r] = load_sm8(sm + base + 8ull * min(lane + 64u * r, last), stream);
}

// Locate, scan and emit one segment into the wave's staging (exponent of
// element g at stg + g - gbase).  The lane's code count is the stored one
// when the view carries counts, else the locate pass walks the chunk.
// False when the counts disagree with the segment's records (then nothing
// is staged).
template <int K>
__device__ __forceinline__ bool stage_segment(const SegLoad &cur, const SegPlan &p, bool stored, uint32_t stg,
                                              uint32_t fast, uint32_t chain, uint32_t lane)
{
    const Window win = make_window(cur.own, cur.next, cur.gap);
    uint32_t cnt = cur.count;
    if (!stored) {
        const uint32_t c0 = lane * kChunkBits;
        const uint32_t end = cur.nbits > c0 ? min(kChunkBits, cur.nbits - c0) : 0u;
        cnt = cur.gap < end ? count_codes<K>(win, fast, chain, cur.gap, end) : 0u;
    }
    uint32_t total;
    const uint32_t excl = wave_exclusive_scan(cnt, &total);
    if (total != (uint32_t)(p.g1 - p.g0)) return false;
    emit_codes<K>(win, fast, chain, stg + p.head + excl, cnt);
    wave_lds_sync();
    return true;
}

// Output placement of decoded element g of a view (row-major, tile order or
// column-group tiles).
struct ViewOut {
    const ViewArgs &v;
    __device__ __forceinline__ uint16_t *at(uint64_t g) const { return v.out + out_index(v, g); }
};

// Output placement of element g of row r into row i of a gather: out_row + (g - r * cols).
struct RowOut {
    uint16_t *out_row;
    uint64_t row_start;
    __device__ __forceinline__ uint16_t *at(uint64_t g) const { return out_row + (g - row_start); }
};

// One 8-element unit ui of the segment: staged exponents + sign+mantissa
// bytes smv -> BF16, one 16-byte store when the unit lies inside [lo, hi).
// Lane l of a round takes unit 64r + l, so every store instruction of the
// wave writes one contiguous kilobyte (an 8-element unit never crosses a
// row of any output order: tile and column-group widths are multiples of 8).
template <class Out>
__device__ __forceinline__ void merge_unit(const SegPlan &p, uint64_t lo, uint64_t hi, uint32_t ui, uint2 smv,
                                           const Out &out, uint32_t stg, bool stream)
{
    const uint64_t gs = p.gbase + 8ull * ui;
    if (ui < p.nunits && gs >= lo && gs + 8 <= hi) {
        const uint2 rx = ld64(stg + 8 * ui);
        const uint2 a = assemble4(smv.x, rx.x), b = assemble4(smv.y, rx.y);
        store_bf16x8(out.at(gs), make_uint4(a.x, a.y, b.x, b.y), stream);
    }
}

// The ragged ends of [lo, hi): the elements before the first and after the
// last whole 8-element unit, one per lane (lanes 0..7 the head, lanes
// 8..15 the tail).
struct RaggedLane {
    uint64_t g;
    bool act;
};

__device__ __forceinline__ RaggedLane ragged_lane(uint64_t lo, uint64_t hi, uint32_t lane)
{
    const uint64_t hend = min((lo + 7) & ~7ull, hi);
    const uint64_t tstart = max(hi & ~7ull, hend);
    RaggedLane r;
    r.g = lane < 8 ? lo + lane : tstart + (lane - 8);
    r.act = lane < 8 ? r.g < hend : (lane < 16 && r.g < hi);
    return r;
}

// Merge the staged exponents of elements [lo, hi) (inside the segment) with
// their sign+mantissa bytes and store BF16: whole 8-element units with
// 16-byte stores (the first rounds from the prefetched bytes), the ragged
// ends one element per lane from rag_sm, the lane's ragged element's
// sign+mantissa byte (loaded by the caller).
template <class Out>
__device__ __forceinline__ void merge_range(const SegPlan &p, uint64_t lo, uint64_t hi, const uint2 (&smp)[kPrefetchRounds],
                                            uint32_t rag_sm, const uint8_t *sm, const Out &out, uint32_t stg, uint32_t lane,
                                            bool stream)
{
    // the ragged ends first: their store then waits only for loads issued
    // before the decode, not for the unit stores below
    const RaggedLane rg = ragged_lane(lo, hi, lane);
    if (rg.act) {
        const uint32_t rx = *(const lds_u8 *)(size_t)(stg + (uint32_t)(rg.g - p.gbase));
        *out.at(rg.g) = assemble1(rag_sm, rx);
    }
#pragma unroll
    for (int r = 0; r < kPrefetchRounds; r++) merge_unit(p, lo, hi, lane + 64u * r, smp[r], out, stg, stream);
    for (uint32_t r = kPrefetchRounds; 64u * r < p.nunits; r++) {
        const uint32_t ui = lane + 64u * r;
        const uint2 smv = ui < p.nunits ? load_sm8(sm + p.gbase + 8ull * ui, stream) : make_uint2(0, 0);
        merge_unit(p, lo, hi, ui, smv, out, stg, stream);
    }
}

// A segment inside one tile of the fused kernel's order (32-row tiles,
// 8-column groups: unit u of a tile is row u % 32, columns 8 * (u / 32) ..
// + 7), written to row-major BF16.  Taking the units in stream order would
// give every lane of a wave-wide store a different row; here lane l takes
// row 8k + l / 8 of group g + l % 8, so each store instruction writes 8 rows
// x 128 contiguous bytes and each sign+mantissa load reads 8 runs of 64
// contiguous bytes.  The loads of the first two 8-group batches (the whole
// segment at up to ~4K elements) go out before the decode, like the
// row-major prefetch; later batches load after it.  Ragged ends as in
// merge_range.
struct TileSeg {
    const uint8_t *smt;        // sign+mantissa bytes of the tile
    uint16_t *obase;           // output of the tile's first element
    uint32_t lo, hi;           // the segment's elements within the tile
    uint32_t grp_a, grp_b;     // first and last column group touched
    uint32_t stg_t;            // staging byte of tile element 0 (modulo 2^32)
};

__device__ __forceinline__ TileSeg tile_seg(const SegPlan &p, const ViewArgs &v, uint32_t stg)
{
    const uint32_t tcs = (v.pow2 >> 5) & 31u, ts = 5 + tcs;
    const uint64_t tile = p.g0 >> ts, tile_start = tile << ts;
    TileSeg q;
    q.lo = (uint32_t)(p.g0 - tile_start);
    q.hi = (uint32_t)(p.g1 - tile_start);
    q.grp_a = q.lo >> 8;
    q.grp_b = (q.hi - 1) >> 8;
    const uint32_t t32 = (uint32_t)tile, rb = t32 / v.tiles_per_row, cb = t32 - rb * v.tiles_per_row;
    q.obase = v.out + ((uint64_t)rb << 5) * v.cols + ((uint64_t)cb << tcs);
    q.smt = v.sm + tile_start;
    q.stg_t = stg + (uint32_t)(tile_start - p.gbase);
    return q;
}

// element offset (in the tile) of lane's unit in pass k of group batch gb
__device__ __forceinline__ uint32_t tile_unit(uint32_t gb, uint32_t k, uint32_t lane)
{
    return ((gb + (lane & 7u)) << 8) + ((8u * k + (lane >> 3)) << 3);
}

__device__ __forceinline__ bool tile_unit_in(const TileSeg &q, uint32_t gb, uint32_t e0, uint32_t lane)
{
    return gb + (lane & 7u) <= q.grp_b && e0 >= q.lo && e0 + 8 <= q.hi;
}

// sign+mantissa bytes of the lane's units in the first two group batches,
// loaded before the decode (units outside the segment reload its first unit)
__device__ __forceinline__ void prefetch_tile8(const TileSeg &q, uint32_t lane, bool stream, uint2 (&tsv)[8])
{
#pragma unroll
    for (int bb = 0; bb < 2; bb++)
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const uint32_t gb = q.grp_a + 8u * bb;
            const uint32_t e0 = tile_unit(gb, k, lane);
            tsv[4 * bb + k] = load_sm8(q.smt + (tile_unit_in(q, gb, e0, lane) ? e0 : (q.lo & ~7u)), stream);
        }
}

__device__ __forceinline__ void merge_tile_groups8(const SegPlan &p, const ViewArgs &v, const TileSeg &q,
                                                   const uint2 (&tsv)[8], uint32_t rag_sm, uint32_t stg,
                                                   uint32_t lane, bool stream)
{
    const RaggedLane rg = ragged_lane(p.g0, p.g1, lane);
    if (rg.act) {
        const uint32_t rx = *(const lds_u8 *)(size_t)(stg + (uint32_t)(rg.g - p.gbase));
        *(v.out + out_index(v, rg.g)) = assemble1(rag_sm, rx);
    }
    auto unit = [&](uint32_t gb, uint32_t k, uint2 sv) {
        const uint32_t e0 = tile_unit(gb, k, lane);
        if (tile_unit_in(q, gb, e0, lane)) {
            const uint2 rx = ld64(q.stg_t + e0);
            const uint2 a = assemble4(sv.x, rx.x), b = assemble4(sv.y, rx.y);
            const uint32_t r = 8u * k + (lane >> 3), grp = gb + (lane & 7u);
            store_bf16x8(q.obase + (uint64_t)r * v.cols + (grp << 3), make_uint4(a.x, a.y, b.x, b.y), stream);
        }
    };
#pragma unroll
    for (int k = 0; k < 4; k++) unit(q.grp_a, k, tsv[k]);
    if (q.grp_a + 8 <= q.grp_b)
#pragma unroll
        for (int k = 0; k < 4; k++) unit(q.grp_a + 8, k, tsv[4 + k]);
    for (uint32_t gb = q.grp_a + 16; gb <= q.grp_b; gb += 8) {
        uint2 sv[4];
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const uint32_t e0 = tile_unit(gb, k, lane);
            sv[k] = load_sm8(q.smt + (tile_unit_in(q, gb, e0, lane) ? e0 : (q.lo & ~7u)), stream);
        }
#pragma unroll
        for (int k = 0; k < 4; k++) unit(gb, k, sv[k]);
    }
}

// ------------------------------------------------------------ kernels
template <int K, int WAVES, bool TILE8>
__device__ __forceinline__ void decode_body(const BatchArgs &b, const TableArgs &t)
{
    extern __shared__ __align__(16) uint8_t lds_raw[];
    const uint32_t lds0 = (uint32_t)(size_t)(lds_u8 *)lds_raw;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lane0 = lane_id();
    const uint32_t stg = lds0 + 16 + wave * t.stg_bytes;
    const uint32_t fast = lds0 + 16 + WAVES * t.stg_bytes;
    const uint32_t chain = fast + (8u << K);

    // the first segment's words in flight while the tables go into LDS
    const uint64_t n_total = b.seg_begin[b.count];
    uint64_t s = (uint64_t)blockIdx.x * WAVES + wave;
    const uint64_t stride = (uint64_t)gridDim.x * WAVES;
    const bool stream = b.stream != 0;
    uint32_t vi = 0;
    SegLoad nx{};
    if (s < n_total) {
        vi = view_of(b, s);
        nx = load_segment(b.v[vi], s - b.seg_begin[vi], lane0);
    }
    stage_tables<K, WAVES * 64>(fast, chain, t.fast, t.chain, t.n_chain);
    __syncthreads();
    if (s >= n_total) return;
    for (;;) {
        // In the tile-order kernel the lane index passes through an empty
        // asm statement, so that its lane-derived offsets are formed per
        // segment: held across the loop they spill (27 VGPRs with the
        // prefetch below).  The row-major kernel is faster as it is.
        uint32_t lane = lane0;
        if constexpr (TILE8) asm volatile("" : "+v"(lane));
        const SegLoad cur = nx;
        const ViewArgs &v = b.v[vi];
        const SegPlan p = plan_segment(cur, v.n, t.stg_bytes);
        // The next segment's words and records first (the last segment
        // loads itself again), then this segment's sign+mantissa bytes:
        // the merge waits for the latter, which leaves the former complete
        // before the next decode, without waiting on this merge's stores.
        const uint64_t s_next = s + stride;
        const bool more = s_next < n_total;
        const uint32_t vi_next = more ? view_of(b, s_next, vi) : vi;
        nx = load_segment(b.v[vi_next], (more ? s_next : s) - b.seg_begin[vi_next], lane);
        uint2 smp[kPrefetchRounds];
        uint2 tsv[TILE8 ? 8 : 1];
        TileSeg q{};
        bool tiled = false;
        if constexpr (TILE8) {   // launches holding a view in the fused kernel's tile order
            const uint32_t ts = 5 + ((v.pow2 >> 5) & 31u);
            tiled = p.valid && v.kc == 8 && v.pow2 && v.tr == 32 && p.g1 > p.g0 && (p.g0 >> ts) == ((p.g1 - 1) >> ts);
            if (tiled) {
                q = tile_seg(p, v, stg);
                prefetch_tile8(q, lane, stream, tsv);
            }
        }
        if (!tiled) prefetch_sm(p, v.sm, lane, stream, smp);
        const RaggedLane rg = ragged_lane(p.g0, p.g1, lane);
        const uint32_t rag_sm = v.sm[p.valid && rg.act ? rg.g : 0];

        if (p.valid && stage_segment<K>(cur, p, v.counts != nullptr, stg, fast, chain, lane)) {
            bool merged = false;
            if constexpr (TILE8)
                if (tiled) {
                    merge_tile_groups8(p, v, q, tsv, rag_sm, stg, lane, stream);
                    merged = true;
                }
            if (!merged) merge_range(p, p.g0, p.g1, smp, rag_sm, v.sm, ViewOut{v}, stg, lane, stream);
        }
        wave_lds_sync();   // the staging is reused by the next segment
        if (!more) break;
        s = s_next;
        vi = vi_next;
    }
}

// Two kernels from one body, both at 8 waves per SIMD (64 VGPRs): the
// row-major one, and one with the tile-order merge for launches that hold
// such a view (its prefetch and bookkeeping spill a few registers, which
// costs less than fewer waves: 55 us against 61 us at 7 waves per SIMD on
// up_proj), so that the row-major kernel stays free of spills.
template <int K, int WAVES>
__global__ void __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(8, 8)))
decode_kernel(BatchArgs b, TableArgs t)
{
    decode_body<K, WAVES, false>(b, t);
}

template <int K, int WAVES>
__global__ void __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(8, 8)))
decode_kernel_t8(BatchArgs b, TableArgs t)
{
    decode_body<K, WAVES, true>(b, t);
}

// Row gather: up to four waves per requested row (about as many as the
// segments a row overlaps); the row's first segment is found by segment_of,
// wave j of the row decodes the overlapping
// segments j, j + split, ... whole into its staging, and only the row's
// elements are written.
struct RowArgs {
    ViewArgs v;               // row-major view (out unused)
    const int64_t *rows;      // requested row ids
    uint16_t *out;            // [n_rows, cols]
    uint64_t n_rows, n_view_rows;
    uint32_t split;           // waves per row: wave j of a row takes its overlapping segments j, j + split, ...
};

// The last segment whose first element is <= e (segment records sorted by
// element offset): one probe of the 64 records around the interpolated
// position, then, if the answer lies outside them, a 64-way search, every
// lane probing one of 64 evenly
// spaced records of the open range per step, so a range of n segments
// takes about log_65(n) dependent loads (3 for 170K segments) instead of
// log_2(n).  Lane l probes p_l = s0 + (l + 1) * span / 65, non-decreasing
// in l and inside [s0, s1); "record p <= e" holds for a prefix of the
// lanes, whose length k gives the new range [p_(k-1), p_k).
__device__ __forceinline__ uint64_t segment_of(const ViewArgs &v, uint64_t e, uint32_t lane)
{
    uint64_t s0 = 0, s1 = v.n_segments;   // invariant: elem_off[s0] <= e, and s1 = end or elem_off[s1] > e
    if (s1 > 64) {
        // Segments hold nearly equal numbers of elements, so e / n * segments
        // lands within a few records of the answer: the 64 records around it
        // usually bracket it, and one load settles the search.
        const uint64_t g = (uint64_t)((float)e * ((float)s1 / (float)v.n));
        const uint64_t base = min(g > 32 ? g - 32 : 0, s1 - 64);
        const bool le = v.segs[base + lane].elem_off <= e;
        const uint32_t k = (uint32_t)__popcll(__ballot(le));
        if (k > 0 && k < 64) return base + k - 1;
        if (k == 0) s1 = base;
        else s0 = base + 63;
    }
    while (s1 - s0 > 1) {
        const uint64_t span = s1 - s0;
        const uint64_t p = s0 + ((uint64_t)(lane + 1) * span) / 65u;
        const bool le = (p <= s0) | (v.segs[p].elem_off <= e);
        const uint32_t k = (uint32_t)__popcll(__ballot(le));
        const uint64_t lo_p = s0 + ((uint64_t)k * span) / 65u;
        if (k < 64) s1 = s0 + ((uint64_t)(k + 1) * span) / 65u;
        s0 = lo_p;
    }
    return s0;
}

// (6 waves per SIMD by registers: the staging in LDS allows no more for
// the usual tables, and at 8 the segment search spills)
template <int K, int WAVES>
__global__ void __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(6, 8)))
decode_rows_kernel(RowArgs a, TableArgs t)
{
    extern __shared__ __align__(16) uint8_t lds_raw[];
    const uint32_t lds0 = (uint32_t)(size_t)(lds_u8 *)lds_raw;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lane = lane_id();
    const uint32_t stg = lds0 + 16 + wave * t.stg_bytes;
    const uint32_t fast = lds0 + 16 + WAVES * t.stg_bytes;
    const uint32_t chain = fast + (8u << K);
    stage_tables<K, WAVES * 64>(fast, chain, t.fast, t.chain, t.n_chain);
    __syncthreads();

    const ViewArgs &v = a.v;
    const uint64_t items = a.n_rows * a.split;
    for (uint64_t w = (uint64_t)blockIdx.x * WAVES + wave; w < items; w += (uint64_t)gridDim.x * WAVES) {
        const uint64_t i = w / a.split;
        const uint32_t j = (uint32_t)(w - i * a.split);
        const int64_t r = a.rows[i];
        if (r < 0 || (uint64_t)r >= a.n_view_rows) continue;   // out-of-range id: row left as it is
        const uint64_t lo = (uint64_t)r * v.cols, hi = lo + v.cols;
        const uint64_t s0 = segment_of(v, lo, lane);
        const RowOut out{a.out + i * v.cols, lo};
        for (uint64_t s = s0 + j; s < v.n_segments; s += a.split) {
            const SegLoad cur = load_segment(v, s, lane);
            if (cur.g0 >= hi) break;
            const SegPlan p = plan_segment(cur, v.n, t.stg_bytes);
            uint2 smp[kPrefetchRounds];
            prefetch_sm(p, v.sm, lane, false, smp);
            const uint64_t mlo = max(lo, p.g0), mhi = min(hi, p.g1);
            const RaggedLane rg = ragged_lane(mlo, mhi, lane);
            const uint32_t rag_sm = v.sm[p.valid && mlo < mhi && rg.act ? rg.g : 0];
            if (p.valid && cur.g1 > lo && stage_segment<K>(cur, p, v.counts != nullptr, stg, fast, chain, lane))
                merge_range(p, mlo, mhi, smp, rag_sm, v.sm, out, stg, lane, false);
            wave_lds_sync();
        }
    }
}

int check_view(const df11_view *v)
{
    if (!v) return df11::fail(DF11_E_ARG, "null view");
    if (v->seg_lanes != 64 || v->chunk_bytes != kChunkBytes)
        return df11::fail(DF11_E_UNSUPPORTED, "decode kernels are built for 16-byte chunks and 64-lane segments (got %u, %u)",
                          v->chunk_bytes, v->seg_lanes);
    if (v->fast_bits < DF11_FAST_BITS_MIN || v->fast_bits > DF11_FAST_BITS_MAX)
        return df11::fail(DF11_E_ARG, "fast_bits %u out of range", v->fast_bits);
    if (v->n_tables < 1 || v->n_tables > DF11_MAX_TABLES || v->n_chain != (uint64_t)v->n_tables * 256 ||
        v->n_fast != (2ull << v->fast_bits))
        return df11::fail(DF11_E_ARG, "table sizes inconsistent");
    if (v->n_segs != v->n_segments + 1 || v->n_gaps != v->n_segments * 64 ||
        (v->n_counts && (v->n_counts != v->n_segments * 64 || !v->counts)) ||
        v->n_exp_words < v->n_segments * kSegWords + 2 || v->n_sm < (v->n + 15) / 16 * 16)
        return df11::fail(DF11_E_ARG, "view array sizes inconsistent with n / n_segments");
    if (v->n && (!v->exp_words || !v->sm || !v->gaps || !v->segs || !v->chain || !v->fast))
        return df11::fail(DF11_E_ARG, "null array in view");
    if (((uintptr_t)v->sm & 15) || ((uintptr_t)v->exp_words & 15) || ((uintptr_t)v->fast & 15) ||
        ((uintptr_t)v->chain & 15) || ((uintptr_t)v->segs & 7))
        return df11::fail(DF11_E_ARG, "view arrays must be 16-byte aligned (sm, exp_words, fast, chain)");
    if (v->tile_rows) {
        if (!v->tile_cols || v->tile_cols % 16 || !v->cols || v->cols % v->tile_cols ||
            (uint64_t)v->tile_rows * v->tile_cols > 0xFFFFFFFFull ||
            (v->tile_kchunk && (v->tile_kchunk % 8 || v->tile_cols % v->tile_kchunk || v->tile_rows % 2)))
            return df11::fail(DF11_E_ARG, "bad tile order in view");
    }
    return DF11_OK;
}

// Exponent staging per wave: room for the most codes any segment of this
// tensor holds (recorded by the encoder, at most segment bits / shortest
// code), an 8-element head offset and a tail unit.
uint32_t staging_bytes(const df11_view *v)
{
    const uint32_t seg_bits = 64u * kChunkBits;
    const uint32_t minlen = std::max(1u, v->min_len);
    const uint32_t tmax = std::min(seg_bits / minlen + 1, std::max(1u, v->max_seg_elems));
    return (16 + tmax + 32 + 15) & ~15u;
}

int device_cu_count() { return df11::cu_count(); }

ViewArgs make_args(const df11_view *v, uint16_t *out)
{
    ViewArgs a{};
    a.words = v->exp_words;
    a.sm = v->sm;
    a.gaps = v->gaps;
    a.counts = v->n_counts ? v->counts : nullptr;   // no counts: the decode runs the locate pass
    a.segs = v->segs;
    a.out = out;
    a.n = v->n;
    a.n_segments = v->n_segments;
    a.tr = v->tile_rows;
    a.tc = v->tile_cols;
    a.tiles_per_row = v->tile_rows ? (uint32_t)(v->cols / v->tile_cols) : 0;
    a.kc = v->tile_rows ? v->tile_kchunk : 0;
    a.cols = v->cols;
    auto log2_exact = [](uint64_t x) -> int {
        if (!x || (x & (x - 1))) return -1;
        int k = 0;
        while ((1ull << k) != x) k++;
        return k;
    };
    if (a.tr) {
        const int trs = log2_exact(a.tr), tcs = log2_exact(a.tc), kcs = a.kc ? log2_exact(a.kc) : 0;
        if (trs >= 0 && tcs >= 0 && kcs >= 0 && trs + tcs < 31 && (v->n >> (trs + tcs)) < (1ull << 32) &&
            ((uint64_t)v->rows >> trs) < (1ull << 32))
            a.pow2 = (1u << 31) | (uint32_t)trs | ((uint32_t)tcs << 5) | ((uint32_t)kcs << 10);
    }
    return a;
}

// LDS bytes of a workgroup of `waves` waves: exponent staging and tables.
uint32_t lds_bytes(int waves, uint32_t stg, uint32_t fast_bits, uint32_t n_tables)
{
    return 16 + (uint32_t)waves * stg + (8u << fast_bits) + n_tables * 512u;
}

template <int K, int W, bool T8>
int try_launch(int waves, const BatchArgs &a, const TableArgs &t, uint32_t lds, uint64_t nseg,
               hipStream_t st, int *resident)
{
    if (waves != W) return 1;
    // *resident > 0: the resident waves per CU are already known
    int per_cu = *resident > 0 ? *resident / W : 0;
    if (per_cu < 1 &&
        (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, T8 ? decode_kernel_t8<K, W> : decode_kernel<K, W>, W * 64, lds) !=
             hipSuccess || per_cu < 1))
        per_cu = 1;
    *resident = per_cu * W;
    if (!nseg) return 0;   // query only
    // every resident slot busy: the decode is latency-bound per wave, so
    // more waves in flight beat an evenly split last round
    const uint64_t groups = std::min<uint64_t>((nseg + W - 1) / W, (uint64_t)device_cu_count() * per_cu);
    if (groups) {
        if constexpr (T8)
            hipLaunchKernelGGL((decode_kernel_t8<K, W>), dim3((uint32_t)groups), dim3(W * 64), lds, st, a, t);
        else
            hipLaunchKernelGGL((decode_kernel<K, W>), dim3((uint32_t)groups), dim3(W * 64), lds, st, a, t);
    }
    return 0;
}

constexpr int kWaveChoices[] = {4, 6, 8, 10, 12, 14, 16};

template <int K, bool T8>
int run_shape(int waves, const BatchArgs &a, const TableArgs &t, uint32_t lds, uint64_t nseg,
              hipStream_t st, int *resident)
{
    return try_launch<K, 4, T8>(waves, a, t, lds, nseg, st, resident) &&
           try_launch<K, 6, T8>(waves, a, t, lds, nseg, st, resident) &&
           try_launch<K, 8, T8>(waves, a, t, lds, nseg, st, resident) &&
           try_launch<K, 10, T8>(waves, a, t, lds, nseg, st, resident) &&
           try_launch<K, 12, T8>(waves, a, t, lds, nseg, st, resident) &&
           try_launch<K, 14, T8>(waves, a, t, lds, nseg, st, resident) &&
           try_launch<K, 16, T8>(waves, a, t, lds, nseg, st, resident);
}

// Waves per workgroup.  Occupancy (LDS and registers) gives, for every
// choice whose exponent staging stays in the first 64 KB of LDS (the emit
// loop keeps byte addresses in 16 bits), the waves that can be resident per
// CU.  A tensor with more segments than all CUs can hold at once takes the
// choice whose resident waves per CU are closest above 24 (or the most, if
// none reaches 24); a smaller one takes the choice that
// puts the fewest waves on the busiest CU (ties: larger workgroups, fewer
// table copies), since each wave's segment is then latency-bound.
// DF11_DECODE_WAVES overrides the choice for tuning.  Occupancy answers
// depend only on (device, K, staging bytes, table count) and the last few
// are kept so that a sequence of launches does not repeat the queries.
constexpr int kNumChoices = sizeof(kWaveChoices) / sizeof(kWaveChoices[0]);
constexpr int kSaturatedWaves = 24;
struct ShapeKey {
    int dev, k;
    uint32_t stg, n_tables;
    bool t8;
    bool operator==(const ShapeKey &o) const
    {
        return dev == o.dev && k == o.k && stg == o.stg && n_tables == o.n_tables && t8 == o.t8;
    }
};
std::mutex g_shape_mu;
ShapeKey g_shape_key[8];
int g_shape_res[8][kNumChoices];
uint32_t g_shape_n = 0;

// res[i]: resident waves per CU with kWaveChoices[i] waves per workgroup (0: does not fit)
template <int K, bool T8>
void resident_waves(const TableArgs &t, const df11_view *v, hipStream_t st, int res[kNumChoices])
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = -1;
    const ShapeKey key{dev, K, t.stg_bytes, v->n_tables, T8};
    {
        std::lock_guard<std::mutex> g(g_shape_mu);
        for (uint32_t i = 0; i < std::min(g_shape_n, 8u); i++)
            if (g_shape_key[i] == key) {
                std::memcpy(res, g_shape_res[i], sizeof(int) * kNumChoices);
                return;
            }
    }
    BatchArgs probe{};
    for (int i = 0; i < kNumChoices; i++) {
        const int w = kWaveChoices[i];
        const uint32_t lds = lds_bytes(w, t.stg_bytes, v->fast_bits, v->n_tables);
        res[i] = 0;
        if (16 + (uint32_t)w * t.stg_bytes > 65520 || lds > 160u * 1024u) continue;
        run_shape<K, T8>(w, probe, t, lds, 0, st, &res[i]);
    }
    std::lock_guard<std::mutex> g(g_shape_mu);
    g_shape_key[g_shape_n % 8] = key;
    std::memcpy(g_shape_res[g_shape_n % 8], res, sizeof(int) * kNumChoices);
    g_shape_n++;
}

// The choice index for nseg segments, or -1 when nothing fits.
int pick_waves(const int res[kNumChoices], uint64_t nseg, uint64_t cus)
{
    const char *env = getenv("DF11_DECODE_WAVES");
    const int forced = env ? atoi(env) : 0;
    int best = -1;
    for (int i = 0; i < kNumChoices; i++) {
        if (!res[i]) continue;
        if (forced) {
            if (kWaveChoices[i] == forced) return i;
            continue;
        }
        if (best < 0 || res[i] > res[best]) best = i;
    }
    if (forced || best < 0) return best;
    if (nseg >= cus * (uint64_t)res[best]) {
        // several rounds: 24 resident waves per CU already keep HBM busy
        // (more waves measured slower on a whole layer in one launch, with
        // more requests contending); take the shape closest above that,
        // smaller workgroups on ties (a whole layer: 6- and 8-wave groups
        // 141 us, 12-wave groups 150 us, all at 24 waves per CU)
        int pick = -1;
        for (int i = 0; i < kNumChoices; i++)
            if (res[i] >= kSaturatedWaves && (pick < 0 || res[i] < res[pick])) pick = i;
        return pick >= 0 ? pick : best;
    }
    uint64_t best_load = ~0ull;
    for (int i = 0; i < kNumChoices; i++) {
        if (!res[i]) continue;
        const uint64_t w = kWaveChoices[i], groups = (nseg + w - 1) / w;
        if (groups > cus * (uint64_t)(res[i] / w)) continue;   // would not be resident at once
        const uint64_t load = (groups + cus - 1) / cus * w;    // waves on the busiest CU
        if (load <= best_load) { best_load = load; best = i; }
    }
    return best;
}

template <int K, bool T8>
int launch_decode_t(const BatchArgs &a, const TableArgs &t, const df11_view *v, hipStream_t st)
{
    int res[kNumChoices];
    resident_waves<K, T8>(t, v, st, res);
    const int i = pick_waves(res, a.seg_begin[a.count], (uint64_t)device_cu_count());
    if (i < 0) return df11::fail(DF11_E_UNSUPPORTED, "tables and staging do not fit in LDS");
    int r = res[i];
    run_shape<K, T8>(kWaveChoices[i], a, t, lds_bytes(kWaveChoices[i], t.stg_bytes, v->fast_bits, v->n_tables),
                     a.seg_begin[a.count], st, &r);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return df11::fail(DF11_E_DEVICE, "decode launch: %s", hipGetErrorString(e));
    return DF11_OK;
}


// Views in 8-column-group tile order take a kernel with the row-wise merge
// for them (merge_tile_groups8); all other launches a kernel without it.
template <int K>
int launch_decode(const BatchArgs &a, const TableArgs &t, const df11_view *v, hipStream_t st)
{
    bool t8 = false;
    for (uint32_t i = 0; i < a.count; i++)
        t8 = t8 || (a.v[i].kc == 8 && a.v[i].pow2 && a.v[i].tr == 32);
    return t8 ? launch_decode_t<K, true>(a, t, v, st) : launch_decode_t<K, false>(a, t, v, st);
}

}  // namespace

namespace {

// One launch over up to kMaxBatch views that share their tables.
int decode_views(const df11_view *views, uint16_t *const *outs, uint32_t count, hipStream_t st)
{
    BatchArgs b{};
    uint32_t stg = 0;
    uint64_t out_bytes = 0;
    const df11_view *v0 = nullptr;
    for (uint32_t i = 0; i < count; i++) {
        const df11_view *v = &views[i];
        if (!v->n) continue;
        if (!outs[i] || ((uintptr_t)outs[i] & 15))
            return df11::fail(DF11_E_ARG, "output %u must be a 16-byte aligned device pointer", i);
        if (v0 && (v->fast != v0->fast || v->chain != v0->chain || v->fast_bits != v0->fast_bits ||
                   v->n_tables != v0->n_tables))
            return df11::fail(DF11_E_ARG, "views of one batch must share their device tables (view %u differs)", i);
        if (!v0) v0 = v;
        b.v[b.count] = make_args(v, outs[i]);
        b.seg_begin[b.count + 1] = b.seg_begin[b.count] + v->n_segments;
        b.count++;
        out_bytes += 2 * v->n;
        stg = std::max(stg, staging_bytes(v));
    }
    if (!b.count || !b.seg_begin[b.count]) return DF11_OK;
    b.stream = out_bytes > kStreamOutBytes;
    TableArgs t{v0->chain, v0->fast, (uint32_t)v0->n_chain, stg};
    switch (v0->fast_bits) {
    case 8: return launch_decode<8>(b, t, v0, st);
    case 9: return launch_decode<9>(b, t, v0, st);
    case 10: return launch_decode<10>(b, t, v0, st);
    case 11: return launch_decode<11>(b, t, v0, st);
    default: return launch_decode<12>(b, t, v0, st);
    }
}

template <int K, int W>
int launch_rows_w(const RowArgs &a, const TableArgs &t, uint32_t lds, int resident, hipStream_t st)
{
    const uint64_t per_cu = std::max(1, resident / W);
    const uint64_t groups = std::min<uint64_t>((a.n_rows * a.split + W - 1) / W, (uint64_t)device_cu_count() * per_cu);
    hipLaunchKernelGGL((decode_rows_kernel<K, W>), dim3((uint32_t)groups), dim3(W * 64), lds, st, a, t);
    return DF11_OK;
}

template <int K>
int launch_rows(const RowArgs &a, const TableArgs &t, const df11_view *v, hipStream_t st)
{
    int res[kNumChoices];
    resident_waves<K, false>(t, v, st, res);
    const int i = pick_waves(res, a.n_rows * a.split, (uint64_t)device_cu_count());
    if (i < 0) return df11::fail(DF11_E_UNSUPPORTED, "tables and staging do not fit in LDS");
    const uint32_t lds = lds_bytes(kWaveChoices[i], t.stg_bytes, v->fast_bits, v->n_tables);
    switch (kWaveChoices[i]) {
    case 4: launch_rows_w<K, 4>(a, t, lds, res[i], st); break;
    case 6: launch_rows_w<K, 6>(a, t, lds, res[i], st); break;
    case 8: launch_rows_w<K, 8>(a, t, lds, res[i], st); break;
    case 10: launch_rows_w<K, 10>(a, t, lds, res[i], st); break;
    case 12: launch_rows_w<K, 12>(a, t, lds, res[i], st); break;
    case 14: launch_rows_w<K, 14>(a, t, lds, res[i], st); break;
    default: launch_rows_w<K, 16>(a, t, lds, res[i], st); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return df11::fail(DF11_E_DEVICE, "decode_rows launch: %s", hipGetErrorString(e));
    return DF11_OK;
}

}  // namespace

extern "C" int df11_decode_rows(const df11_view *v, const int64_t *rows, uint64_t n_rows, uint16_t *out,
                                void *stream)
{
    int rc = check_view(v);
    if (rc) return rc;
    if (!n_rows) return DF11_OK;
    if (!rows || !out || ((uintptr_t)out & 15) || ((uintptr_t)rows & 7))
        return df11::fail(DF11_E_ARG, "df11_decode_rows: rows (8-byte aligned) and out (16-byte aligned) are device pointers");
    if (v->tile_rows || !v->cols || !v->rows || v->rows * v->cols != v->n || v->cols % 8)
        return df11::fail(DF11_E_ARG, "df11_decode_rows needs a row-major [rows, cols] view with cols a multiple of 8");
    RowArgs a{};
    a.v = make_args(v, nullptr);
    a.rows = rows;
    a.out = out;
    a.n_rows = n_rows;
    a.n_view_rows = v->rows;
    // a row spans about cols / (elements per segment) + 1 segments: that
    // many waves per row (at most 4) decode them side by side
    a.split = 1;
    if (v->n_segments) {
        const uint64_t per_seg = std::max<uint64_t>(1, v->n / v->n_segments);
        a.split = (uint32_t)std::min<uint64_t>(4, v->cols / per_seg + 1);
    }
    if (n_rows > (UINT64_MAX >> 3)) return df11::fail(DF11_E_ARG, "df11_decode_rows: too many rows");
    TableArgs t{v->chain, v->fast, (uint32_t)v->n_chain, staging_bytes(v)};
    hipStream_t st = (hipStream_t)stream;
    switch (v->fast_bits) {
    case 8: return launch_rows<8>(a, t, v, st);
    case 9: return launch_rows<9>(a, t, v, st);
    case 10: return launch_rows<10>(a, t, v, st);
    case 11: return launch_rows<11>(a, t, v, st);
    default: return launch_rows<12>(a, t, v, st);
    }
}

extern "C" int df11_decode(const df11_view *v, uint16_t *out, void *stream)
{
    int rc = check_view(v);
    if (rc) return rc;
    if (!v->n) return DF11_OK;
    if (!out || ((uintptr_t)out & 15)) return df11::fail(DF11_E_ARG, "out must be a 16-byte aligned device pointer");
    uint16_t *outs[1] = {out};
    return decode_views(v, outs, 1, (hipStream_t)stream);
}

extern "C" int df11_decode_batch(const df11_view *views, uint16_t *const *outs, uint32_t count, void *stream)
{
    if (count && (!views || !outs)) return df11::fail(DF11_E_ARG, "df11_decode_batch: null pointer");
    for (uint32_t i = 0; i < count; i++) {
        int rc = check_view(&views[i]);
        if (rc) return rc;
    }
    for (uint32_t i = 0; i < count; i += kMaxBatch) {
        int rc = decode_views(views + i, outs + i, std::min(kMaxBatch, count - i), (hipStream_t)stream);
        if (rc) return rc;
    }
    return DF11_OK;
}

namespace df11 {

int cu_count()
{
    constexpr int kDevices = 64;
    static std::atomic<int> cached[kDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev >= 0 && dev < kDevices) {
        const int c = cached[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) return 256;
    if (dev >= 0 && dev < kDevices) cached[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

}  // namespace df11
