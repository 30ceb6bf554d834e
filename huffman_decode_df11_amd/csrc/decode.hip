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
#define DF11_HD __host__ __device__ __forceinline__
#include "segment_plan.h"

using namespace df11dev;
using df11plan::RaggedLane;
using df11plan::SegPlan;
using df11plan::TileSeg;

namespace {

// A lane's chunk of the stream: CB = 16 or 8 bytes, loaded as CB / 4 words
// (the window adds the next chunk's first word).
template <int CB> struct Chunk;
template <> struct Chunk<16> { typedef uint4 words_t; };
template <> struct Chunk<8> { typedef uint2 words_t; };
template <int CB> constexpr uint32_t chunk_bits() { return 8u * CB; }
template <int CB> constexpr uint32_t seg_words() { return 64u * CB / 4u; }
// Rounds of 8-element units per lane whose sign+mantissa bytes are loaded
// before the decode.  A 16-byte-chunk segment of Gaussian-like weights holds
// ~2,800-3,200 elements, 6-7 rounds: the rounds after the prefetched ones
// are loaded after the decode, one exposed round trip, which costs most
// where each wave takes a single segment (a 16M-element tensor: 17.2 us
// with 5, 15.6 with 6; 7 spills registers at 8 waves per SIMD, 16.9).  The
// sixth round costs one spilled register, which a launch that streams more
// output than the Infinity Cache holds pays for (the 8B model pass: 5.52 ms
// with 5 rounds, 5.80 with 6), so those launches keep 5.  An 8-byte-chunk
// segment holds ~1,400 elements, 3 rounds (5 kept: 3 measured no faster).
template <int CB, bool STREAM = false>
constexpr int prefetch_rounds()
{
    return CB == 16 && !STREAM ? 6 : 5;
}

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
    uint32_t stream;          // nonzero: streaming (nontemporal) BF16 stores
};

// A launch whose BF16 output is larger than the last-level cache (the
// 256 MB Infinity Cache) cannot leave it there for the matmul that follows,
// so it streams: BF16 is written with nontemporal stores, which keeps the
// write-allocate and eviction of data used once out of the cache.  Smaller
// outputs are written normally and are still cache-resident when the
// consumer reads them.  Sign+mantissa bytes are always read with normal
// loads: the 128-byte line at each segment boundary is read by two waves,
// usually of one workgroup, and a cached line serves the second (the 8B
// model pass: 5.53 ms with nontemporal loads, 5.49 with normal ones; its
// reads were 7.3% above the algorithmic bytes).
constexpr uint64_t kStreamOutBytes = 256ull << 20;

typedef unsigned int v2u32 __attribute__((ext_vector_type(2)));
typedef unsigned int v4u32g __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint2 load_sm8(const uint8_t *p)
{
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
template <int CB>
struct SegLoad {
    typename Chunk<CB>::words_t own;   // this lane's stream words
    uint32_t next;      // the following word (look-ahead)
    uint32_t gap;
    uint32_t count;     // codes that start in this lane's chunk (meaningful when the view stores counts)
    uint32_t nbits;
    uint64_t g0, g1;
};

template <int CB>
__device__ __forceinline__ SegLoad<CB> load_segment(const ViewArgs &v, uint64_t s, uint32_t lane)
{
    typedef typename Chunk<CB>::words_t words_t;
    SegLoad<CB> L;
    const uint32_t *w = v.words + s * seg_words<CB>() + lane * (CB / 4);
    L.own = *reinterpret_cast<const words_t *>(w);
    L.next = w[CB / 4];
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
// (plan_segment, ragged_lane and the tile placement: segment_plan.h)
template <int CB>
__device__ __forceinline__ SegPlan plan_segment(const SegLoad<CB> &cur, uint64_t n, uint32_t stg_bytes)
{
    return df11plan::plan_segment(cur.g0, cur.g1, n, stg_bytes);
}

// the segment's sign+mantissa bytes for the first PR rounds of
// units.  Lanes past the last unit load the last unit again (an address
// that is always inside the array), so no value has to be selected and the
// loads stay in flight during the decode.
template <int PR>
__device__ __forceinline__ void prefetch_sm(const SegPlan &p, const uint8_t *sm, uint32_t lane,
                                            uint2 (&smp)[PR])
{
    const uint32_t last = p.nunits ? p.nunits - 1 : 0u;
    const uint64_t base = p.nunits ? p.gbase : 0ull;
#pragma unroll
    for (int r = 0; r < PR; r++)
        smp[r] = load_sm8(sm + base + 8ull * min(lane + 64u * r, last));
}

// Locate, scan and emit one segment into the wave's staging (exponent of
// element g at stg + g - gbase).  The lane's code count is the stored one
// when the view carries counts, else the locate pass walks the chunk.
// False when the counts disagree with the segment's records (then nothing
// is staged).
template <int K, int CB>
__device__ __forceinline__ bool stage_segment(const SegLoad<CB> &cur, const SegPlan &p, bool stored, uint32_t stg,
                                              uint32_t fast, uint32_t chain, uint32_t lane)
{
    const auto win = make_window(cur.own, cur.next, cur.gap);
    uint32_t cnt = cur.count;
    if (!stored) {
        const uint32_t c0 = lane * chunk_bits<CB>();
        const uint32_t end = cur.nbits > c0 ? min(chunk_bits<CB>(), cur.nbits - c0) : 0u;
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
    if (df11plan::unit_inside(p, lo, hi, ui)) {
        const uint64_t gs = p.gbase + 8ull * ui;
        const uint2 rx = ld64(stg + 8 * ui);
        const uint2 a = assemble4(smv.x, rx.x), b = assemble4(smv.y, rx.y);
        store_bf16x8(out.at(gs), make_uint4(a.x, a.y, b.x, b.y), stream);
    }
}

__device__ __forceinline__ RaggedLane ragged_lane(uint64_t lo, uint64_t hi, uint32_t lane)
{
    return df11plan::ragged_lane(lo, hi, lane);
}

// Merge the staged exponents of elements [lo, hi) (inside the segment) with
// their sign+mantissa bytes and store BF16: whole 8-element units with
// 16-byte stores (the first rounds from the prefetched bytes), the ragged
// ends one element per lane from rag_sm, the lane's ragged element's
// sign+mantissa byte (loaded by the caller).
template <class Out, int PR>
__device__ __forceinline__ void merge_range(const SegPlan &p, uint64_t lo, uint64_t hi, const uint2 (&smp)[PR],
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
    for (int r = 0; r < PR; r++) merge_unit(p, lo, hi, lane + 64u * r, smp[r], out, stg, stream);
    for (uint32_t r = PR; 64u * r < p.nunits; r++) {
        const uint32_t ui = lane + 64u * r;
        const uint2 smv = ui < p.nunits ? load_sm8(sm + p.gbase + 8ull * ui) : make_uint2(0, 0);
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
__device__ __forceinline__ TileSeg tile_seg(const SegPlan &p, const ViewArgs &v, uint32_t stg)
{
    return df11plan::tile_seg(p, (v.pow2 >> 5) & 31u, v.tiles_per_row, v.cols, stg);
}

using df11plan::tile_unit;
using df11plan::tile_unit_in;

// sign+mantissa bytes of the lane's units in the first two group batches,
// loaded before the decode (units outside the segment reload its first unit)
__device__ __forceinline__ void prefetch_tile8(const TileSeg &q, const ViewArgs &v, uint32_t lane,
                                               uint2 (&tsv)[8])
{
#pragma unroll
    for (int bb = 0; bb < 2; bb++)
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const uint32_t gb = q.grp_a + 8u * bb;
            const uint32_t e0 = tile_unit(gb, k, lane);
            tsv[4 * bb + k] = load_sm8(v.sm + q.sm_off + (tile_unit_in(q, gb, e0, lane) ? e0 : (q.lo & ~7u)));
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
            store_bf16x8(v.out + q.out_off + df11plan::tile_unit_out(gb, k, lane, v.cols), make_uint4(a.x, a.y, b.x, b.y),
                         stream);
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
            sv[k] = load_sm8(v.sm + q.sm_off + (tile_unit_in(q, gb, e0, lane) ? e0 : (q.lo & ~7u)));
        }
#pragma unroll
        for (int k = 0; k < 4; k++) unit(gb, k, sv[k]);
    }
}

// ------------------------------------------------------------ kernels
template <int K, int WAVES, bool TILE8, int CB, int PR>
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
    SegLoad<CB> nx{};
    if (s < n_total) {
        vi = view_of(b, s);
        nx = load_segment<CB>(b.v[vi], s - b.seg_begin[vi], lane0);
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
        const SegLoad<CB> cur = nx;
        const ViewArgs &v = b.v[vi];
        const SegPlan p = plan_segment(cur, v.n, t.stg_bytes);
        // The next segment's words and records first (the last segment
        // loads itself again), then this segment's sign+mantissa bytes:
        // the merge waits for the latter, which leaves the former complete
        // before the next decode, without waiting on this merge's stores.
        const uint64_t s_next = s + stride;
        const bool more = s_next < n_total;
        const uint32_t vi_next = more ? view_of(b, s_next, vi) : vi;
        nx = load_segment<CB>(b.v[vi_next], (more ? s_next : s) - b.seg_begin[vi_next], lane);
        uint2 smp[PR];
        uint2 tsv[TILE8 ? 8 : 1];
        TileSeg q{};
        bool tiled = false;
        if constexpr (TILE8) {   // launches holding a view in the fused kernel's tile order
            const uint32_t ts = 5 + ((v.pow2 >> 5) & 31u);
            tiled = p.valid && v.kc == 8 && v.pow2 && v.tr == 32 && p.g1 > p.g0 && (p.g0 >> ts) == ((p.g1 - 1) >> ts);
            if (tiled) {
                q = tile_seg(p, v, stg);
                prefetch_tile8(q, v, lane, tsv);
            }
        }
        if (!tiled) prefetch_sm(p, v.sm, lane, smp);
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

// Kernels from one body, all at 8 waves per SIMD (64 VGPRs): the row-major
// one (PR prefetched rounds: 6 for 16-byte chunks, 5 in the form for
// streaming launches and for 8-byte chunks), and one with the tile-order
// merge for launches that hold such a view (its prefetch and bookkeeping
// spill a few registers, which costs less than fewer waves: 55 us against
// 61 us at 7 waves per SIMD on up_proj).
template <int K, int WAVES, int CB, int PR>
__global__ void __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(8, 8)))
decode_kernel(BatchArgs b, TableArgs t)
{
    decode_body<K, WAVES, false, CB, PR>(b, t);
}

// (the fused kernel's layout always has 16-byte chunks)
template <int K, int WAVES, int CB>
__global__ void __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(8, 8)))
decode_kernel_t8(BatchArgs b, TableArgs t)
{
    static_assert(CB == 16, "tile-order views are encoded with 16-byte chunks");
    decode_body<K, WAVES, true, CB, prefetch_rounds<CB, true>()>(b, t);
}

// Row gather: up to eight waves per requested row (as many as the segments
// a row can overlap); the row's first segment is found by segment_of, wave
// j of the row decodes the overlapping segments j, j + split, ... whole
// into its staging, and only the row's elements are written.  The window
// kernel below (win > 0, the view's row window) gives wave j of a row
// segment g(r) + win_lo + j of the window, which holds every segment the
// row overlaps, with no search before its loads.
struct RowArgs {
    ViewArgs v;               // row-major view (out unused)
    const int64_t *rows;      // requested row ids
    uint16_t *out;            // [n_rows, cols]
    uint64_t n_rows, n_view_rows;
    uint32_t split;           // waves per row: wave j of a row takes its overlapping segments j, j + split, ...
    uint32_t win;             // window kernel: the window's segments
    int32_t win_lo;
    double seg_per_elem;      // n_segments / n, as the encoder computed it
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
template <int K, int WAVES, int CB>
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
    const ViewArgs &v = a.v;
    const uint64_t items = a.n_rows * a.split;
    // A work item w is piece j of requested row i.  The first item's
    // segment search and first segment load go out before the tables are
    // staged, so that their latency overlaps the staging.
    struct Item {
        uint64_t i, lo, hi, s;   // s: the item's first segment (n_segments: nothing to do)
        uint32_t j;
    };
    auto item = [&](uint64_t w) {
        Item it;
        it.i = w / a.split;
        it.j = (uint32_t)(w - it.i * a.split);
        const int64_t r = a.rows[it.i];
        it.s = v.n_segments;
        it.lo = it.hi = 0;
        if (r >= 0 && (uint64_t)r < a.n_view_rows) {   // an out-of-range id leaves its row as it is
            it.lo = (uint64_t)r * v.cols;
            it.hi = it.lo + v.cols;
            it.s = min(segment_of(v, it.lo, lane) + it.j, v.n_segments);
        }
        return it;
    };
    uint64_t w = (uint64_t)blockIdx.x * WAVES + wave;
    Item it{};
    SegLoad<CB> first{};
    if (w < items) {
        it = item(w);
        if (it.s < v.n_segments) first = load_segment<CB>(v, it.s, lane);
    }
    stage_tables<K, WAVES * 64>(fast, chain, t.fast, t.chain, t.n_chain);
    __syncthreads();

    for (bool head = true; w < items; w += (uint64_t)gridDim.x * WAVES, head = false) {
        if (!head) it = item(w);
        const uint64_t lo = it.lo, hi = it.hi;
        const RowOut out{a.out + it.i * v.cols, lo};
        for (uint64_t s = it.s; s < v.n_segments; s += a.split) {
            const SegLoad<CB> cur = head && s == it.s ? first : load_segment<CB>(v, s, lane);
            if (cur.g0 >= hi) break;
            const SegPlan p = plan_segment(cur, v.n, t.stg_bytes);
            uint2 smp[prefetch_rounds<CB>()];
            prefetch_sm(p, v.sm, lane, smp);
            const uint64_t mlo = max(lo, p.g0), mhi = min(hi, p.g1);
            const RaggedLane rg = ragged_lane(mlo, mhi, lane);
            const uint32_t rag_sm = v.sm[p.valid && mlo < mhi && rg.act ? rg.g : 0];
            if (p.valid && cur.g1 > lo && stage_segment<K>(cur, p, v.counts != nullptr, stg, fast, chain, lane))
                merge_range(p, mlo, mhi, smp, rag_sm, v.sm, out, stg, lane, false);
            wave_lds_sync();
        }
    }
}

// Row gather in window mode, one workgroup per requested row (WAVES >= the
// view's row window): wave j loads segment g(r) + win_lo + j of the window
// right after the row id, while the whole workgroup copies the row's
// sign+mantissa bytes into LDS next to the tables, so the merge waits on
// no global load after the decode.  LDS: [guard][WAVES x staging][the row's
// sign+mantissa bytes][tables].
template <int K, int WAVES, int CB>
__global__ void __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(4, 8)))
decode_row_window_kernel(RowArgs a, TableArgs t, uint32_t row_sm_bytes)
{
    constexpr uint32_t kThreads = WAVES * 64;
    constexpr uint32_t kPieces = 4;   // 8-byte pieces of the row's bytes per thread (cols <= 32 * kThreads)
    extern __shared__ __align__(16) uint8_t lds_raw[];
    const uint32_t lds0 = (uint32_t)(size_t)(lds_u8 *)lds_raw;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lane = lane_id();
    const uint32_t stg = lds0 + 16 + wave * t.stg_bytes;
    const uint32_t row_sm = lds0 + 16 + WAVES * t.stg_bytes;
    const uint32_t fast = row_sm + row_sm_bytes;
    const uint32_t chain = fast + (8u << K);
    const ViewArgs &v = a.v;
    const uint64_t i = blockIdx.x;
    const int64_t r = a.rows[i];
    const bool in_range = r >= 0 && (uint64_t)r < a.n_view_rows;   // an out-of-range id leaves its row as it is
    const uint64_t lo = in_range ? (uint64_t)r * v.cols : 0, hi = in_range ? lo + v.cols : 0;
    uint64_t s = v.n_segments;
    if (in_range && wave < a.win) {
        const int64_t sg = (int64_t)floor((double)lo * a.seg_per_elem) + a.win_lo + (int64_t)wave;
        if (sg >= 0 && (uint64_t)sg < v.n_segments) s = (uint64_t)sg;
    }
    SegLoad<CB> cur{};
    if (s < v.n_segments) cur = load_segment<CB>(v, s, lane);
    // the row's sign+mantissa bytes (8-byte pieces; cols is a multiple of 8)
    const uint32_t n8 = in_range ? (uint32_t)(v.cols / 8) : 0u;
    uint2 piece[kPieces];
#pragma unroll
    for (uint32_t k = 0; k < kPieces; k++) {
        const uint32_t idx = threadIdx.x + k * kThreads;
        piece[k] = idx < n8 ? *reinterpret_cast<const uint2 *>(v.sm + lo + 8ull * idx) : make_uint2(0, 0);
    }
    stage_tables<K, kThreads>(fast, chain, t.fast, t.chain, t.n_chain);
#pragma unroll
    for (uint32_t k = 0; k < kPieces; k++) {
        const uint32_t idx = threadIdx.x + k * kThreads;
        if (idx < n8) *(lds_u2 *)(size_t)(row_sm + 8 * idx) = v2u32{piece[k].x, piece[k].y};
    }
    __syncthreads();
    if (s >= v.n_segments || cur.g0 >= hi || cur.g1 <= lo) return;
    const SegPlan p = plan_segment(cur, v.n, t.stg_bytes);
    if (!p.valid || !stage_segment<K>(cur, p, v.counts != nullptr, stg, fast, chain, lane)) return;
    const uint64_t mlo = max(lo, p.g0), mhi = min(hi, p.g1);
    uint16_t *out = a.out + i * v.cols;
    const RaggedLane rg = ragged_lane(mlo, mhi, lane);
    if (rg.act) {
        const uint32_t rx = *(const lds_u8 *)(size_t)(stg + (uint32_t)(rg.g - p.gbase));
        const uint32_t sm = *(const lds_u8 *)(size_t)(row_sm + (uint32_t)(rg.g - lo));
        out[rg.g - lo] = assemble1(sm, rx);
    }
    for (uint32_t ui = lane; ui < p.nunits; ui += 64) {
        if (!df11plan::unit_inside(p, mlo, mhi, ui)) continue;
        const uint64_t gs = p.gbase + 8ull * ui;
        const uint2 rx = ld64(stg + 8 * ui);
        const uint2 sv = ld64(row_sm + (uint32_t)(gs - lo));
        const uint2 x = assemble4(sv.x, rx.x), y = assemble4(sv.y, rx.y);
        *reinterpret_cast<uint4 *>(out + (gs - lo)) = make_uint4(x.x, x.y, y.x, y.y);
    }
}

template <int K, int CB>
int launch_row_window(const RowArgs &a, const TableArgs &t, const df11_view *v, hipStream_t st)
{
    const uint32_t w = a.win <= 8 ? 8u : a.win <= 12 ? 12u : 16u;
    const uint32_t row_bytes = (uint32_t)((v->cols + 15) & ~15ull);
    const uint32_t lds = 16 + w * t.stg_bytes + row_bytes + (8u << K) + v->n_tables * 512u;
    const dim3 grid((uint32_t)a.n_rows), block(w * 64);
    if (w == 8) hipLaunchKernelGGL((decode_row_window_kernel<K, 8, CB>), grid, block, lds, st, a, t, row_bytes);
    else if (w == 12) hipLaunchKernelGGL((decode_row_window_kernel<K, 12, CB>), grid, block, lds, st, a, t, row_bytes);
    else hipLaunchKernelGGL((decode_row_window_kernel<K, 16, CB>), grid, block, lds, st, a, t, row_bytes);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return df11::fail(DF11_E_DEVICE, "row gather launch: %s", hipGetErrorString(e));
    return DF11_OK;
}

// The window kernel's LDS for this view and window (0 when it does not fit:
// the staging within the first 64 KB, the row's bytes at most 32 pieces of
// 8 bytes per thread, everything within a CU's 160 KB).
uint32_t row_window_lds(const df11_view *v, uint32_t win, uint32_t stg)
{
    const uint32_t w = win <= 8 ? 8u : win <= 12 ? 12u : 16u;
    if (v->cols > 32ull * w * 64 || 16 + w * stg > 65520) return 0;
    const uint64_t lds = 16 + (uint64_t)w * stg + ((v->cols + 15) & ~15ull) + (8u << v->fast_bits) + v->n_tables * 512u;
    return lds <= 160u * 1024u ? (uint32_t)lds : 0u;
}

int check_view(const df11_view *v)
{
    if (!v) return df11::fail(DF11_E_ARG, "null view");
    if (v->seg_lanes != 64 || (v->chunk_bytes != 16 && v->chunk_bytes != 8))
        return df11::fail(DF11_E_ARG, "view: chunk_bytes %u and seg_lanes %u (need 8 or 16, and 64)",
                          v->chunk_bytes, v->seg_lanes);
    if (v->fast_bits < DF11_FAST_BITS_MIN || v->fast_bits > DF11_FAST_BITS_MAX)
        return df11::fail(DF11_E_ARG, "fast_bits %u out of range", v->fast_bits);
    if (v->n_tables < 1 || v->n_tables > DF11_MAX_TABLES || v->n_chain != (uint64_t)v->n_tables * 256 ||
        v->n_fast != (2ull << v->fast_bits))
        return df11::fail(DF11_E_ARG, "table sizes inconsistent");
    const uint64_t seg_words = 64ull * v->chunk_bytes / 4;
    if (v->n_segs != v->n_segments + 1 || v->n_gaps != v->n_segments * 64 ||
        (v->n_counts && (v->n_counts != v->n_segments * 64 || !v->counts)) ||
        v->n_exp_words < v->n_segments * seg_words + 2 || v->n_sm < (v->n + 15) / 16 * 16)
        return df11::fail(DF11_E_ARG, "view array sizes inconsistent with n / n_segments");
    if (v->n) {
        if (!v->exp_words || !v->sm || !v->gaps || !v->segs || !v->chain || !v->fast)
            return df11::fail(DF11_E_ARG, "null array in view");
        // the staging is sized from max_seg_elems: it must be set, and no
        // segment can hold more codes than its bits at the shortest length
        const uint64_t seg_bits = 8ull * seg_words * 4;
        if (v->min_len < 1 || v->min_len > v->max_len || v->max_len > DF11_MAX_LEN || !v->max_seg_elems ||
            v->max_seg_elems > (seg_bits + v->min_len - 1) / v->min_len)
            return df11::fail(DF11_E_ARG, "view: code lengths %u..%u or max_seg_elems %u out of range", v->min_len,
                              v->max_len, v->max_seg_elems);
    }
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
    const uint32_t seg_bits = 64u * 8u * v->chunk_bytes;
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

// The kernel of a launch: KIND 0 row-major decode, 1 its tile-order form,
// 2 the row gather, 3 the row-major decode of a streaming launch.
template <int K, int W, int CB, int KIND>
constexpr auto kernel_of()
{
    if constexpr (KIND == 0) return decode_kernel<K, W, CB, prefetch_rounds<CB>()>;
    else if constexpr (KIND == 1) return decode_kernel_t8<K, W, CB>;
    else if constexpr (KIND == 2) return decode_rows_kernel<K, W, CB>;
    else return decode_kernel<K, W, CB, prefetch_rounds<CB, true>()>;
}

constexpr int kWaveChoices[] = {4, 6, 8, 10, 12, 14, 16};
constexpr int kNumChoices = sizeof(kWaveChoices) / sizeof(kWaveChoices[0]);

// Resident workgroups per CU of kernel_of<K, W, CB, KIND> with `lds` bytes
// of LDS, or 0 when the query fails.
template <int K, int CB, int KIND>
int occupancy(int waves, uint32_t lds)
{
    int per_cu = 0;
    auto q = [&](auto kern, int w) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, w * 64, lds) != hipSuccess) per_cu = 0;
    };
    switch (waves) {
    case 4: q(kernel_of<K, 4, CB, KIND>(), 4); break;
    case 6: q(kernel_of<K, 6, CB, KIND>(), 6); break;
    case 8: q(kernel_of<K, 8, CB, KIND>(), 8); break;
    case 10: q(kernel_of<K, 10, CB, KIND>(), 10); break;
    case 12: q(kernel_of<K, 12, CB, KIND>(), 12); break;
    case 14: q(kernel_of<K, 14, CB, KIND>(), 14); break;
    default: q(kernel_of<K, 16, CB, KIND>(), 16); break;
    }
    return per_cu;
}

// Waves per workgroup.  Occupancy (LDS and registers) gives, for every
// choice whose exponent staging stays in the first 64 KB of LDS (the emit
// loop keeps byte addresses in 16 bits), the waves that can be resident per
// CU.  A tensor with more segments than all CUs can hold at once takes the
// choice whose resident waves per CU are closest above 24 (or the most, if
// none reaches 24); a smaller one takes the choice that
// puts the fewest waves on the busiest CU (ties: larger workgroups, fewer
// table copies), since each wave's segment is then latency-bound.
// Occupancy answers depend only on (device, kernel, staging bytes, table
// count) and the last few are kept so that a sequence of launches does not
// repeat the queries.
constexpr int kSaturatedWaves = 24;
struct ShapeKey {
    int dev, k, cb, kind;
    uint32_t stg, n_tables;
    bool operator==(const ShapeKey &o) const
    {
        return dev == o.dev && k == o.k && cb == o.cb && kind == o.kind && stg == o.stg && n_tables == o.n_tables;
    }
};
std::mutex g_shape_mu;
ShapeKey g_shape_key[8];
int g_shape_res[8][kNumChoices];
uint32_t g_shape_n = 0;

// res[i]: resident waves per CU with kWaveChoices[i] waves per workgroup (0: does not fit)
template <int K, int CB, int KIND>
void resident_waves(uint32_t stg_bytes, uint32_t fast_bits, uint32_t n_tables, int res[kNumChoices])
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = -1;
    const ShapeKey key{dev, K, CB, KIND, stg_bytes, n_tables};
    {
        std::lock_guard<std::mutex> g(g_shape_mu);
        for (uint32_t i = 0; i < std::min(g_shape_n, 8u); i++)
            if (g_shape_key[i] == key) {
                std::memcpy(res, g_shape_res[i], sizeof(int) * kNumChoices);
                return;
            }
    }
    for (int i = 0; i < kNumChoices; i++) {
        const int w = kWaveChoices[i];
        const uint32_t lds = lds_bytes(w, stg_bytes, fast_bits, n_tables);
        res[i] = 0;
        if (16 + (uint32_t)w * stg_bytes > 65520 || lds > 160u * 1024u) continue;
        res[i] = std::max(1, occupancy<K, CB, KIND>(w, lds)) * w;
    }
    std::lock_guard<std::mutex> g(g_shape_mu);
    g_shape_key[g_shape_n % 8] = key;
    std::memcpy(g_shape_res[g_shape_n % 8], res, sizeof(int) * kNumChoices);
    g_shape_n++;
}

// The choice index for `items` wave tasks (segments or row pieces), or -1
// when nothing fits; `forced` (nonzero) takes that many waves per workgroup.
int pick_waves(const int res[kNumChoices], uint64_t items, uint64_t cus, uint32_t forced)
{
    int best = -1;
    for (int i = 0; i < kNumChoices; i++) {
        if (!res[i]) continue;
        if (forced) {
            if ((uint32_t)kWaveChoices[i] == forced) return i;
            continue;
        }
        if (best < 0 || res[i] > res[best]) best = i;
    }
    if (forced || best < 0) return best;
    // fewer than two rounds at the most resident waves: take them all (a
    // 16M-element tensor in 8-byte chunks, 10.6K segments: 15.4 us at 32
    // resident waves per CU against 17.1 us at 24)
    if (items >= cus * (uint64_t)res[best] && items < 2 * cus * (uint64_t)res[best]) return best;
    if (items >= cus * (uint64_t)res[best]) {
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
        const uint64_t w = kWaveChoices[i], groups = (items + w - 1) / w;
        if (groups > cus * (uint64_t)(res[i] / w)) continue;   // would not be resident at once
        const uint64_t load = (groups + cus - 1) / cus * w;    // waves on the busiest CU
        if (load <= best_load) { best_load = load; best = i; }
    }
    return best;
}

// One launch of kernel_of<K, W, CB, KIND> with every resident slot busy:
// the decode is latency-bound per wave, so more waves in flight beat an
// evenly split last round.
template <int K, int CB, int KIND, class Args>
int launch_waves(int choice, int resident, const Args &a, const TableArgs &t, uint32_t lds, uint64_t items,
                 uint32_t forced_groups, hipStream_t st)
{
    const int w = kWaveChoices[choice];
    const uint64_t per_cu = std::max(1, resident / w);
    const uint64_t groups = std::min<uint64_t>((items + w - 1) / w,
                                               forced_groups ? forced_groups : (uint64_t)device_cu_count() * per_cu);
    if (!groups) return DF11_OK;
    const dim3 grid((uint32_t)groups), block(w * 64);
    switch (w) {
    case 4: hipLaunchKernelGGL((kernel_of<K, 4, CB, KIND>()), grid, block, lds, st, a, t); break;
    case 6: hipLaunchKernelGGL((kernel_of<K, 6, CB, KIND>()), grid, block, lds, st, a, t); break;
    case 8: hipLaunchKernelGGL((kernel_of<K, 8, CB, KIND>()), grid, block, lds, st, a, t); break;
    case 10: hipLaunchKernelGGL((kernel_of<K, 10, CB, KIND>()), grid, block, lds, st, a, t); break;
    case 12: hipLaunchKernelGGL((kernel_of<K, 12, CB, KIND>()), grid, block, lds, st, a, t); break;
    case 14: hipLaunchKernelGGL((kernel_of<K, 14, CB, KIND>()), grid, block, lds, st, a, t); break;
    default: hipLaunchKernelGGL((kernel_of<K, 16, CB, KIND>()), grid, block, lds, st, a, t); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return df11::fail(DF11_E_DEVICE, "decode launch: %s", hipGetErrorString(e));
    return DF11_OK;
}

template <int K, int CB, int KIND, class Args>
int launch_kind(const Args &a, const TableArgs &t, const df11_view *v, uint64_t items, uint32_t forced_waves,
                uint32_t forced_groups, hipStream_t st)
{
    int res[kNumChoices];
    resident_waves<K, CB, KIND>(t.stg_bytes, v->fast_bits, v->n_tables, res);
    const int i = pick_waves(res, items, (uint64_t)device_cu_count(), forced_waves);
    if (i < 0)
        return df11::fail(forced_waves ? DF11_E_ARG : DF11_E_UNSUPPORTED,
                          forced_waves ? "%u waves per workgroup do not fit this tensor's staging and tables"
                                       : "tables and staging do not fit in LDS",
                          forced_waves);
    return launch_waves<K, CB, KIND>(i, res[i], a, t, lds_bytes(kWaveChoices[i], t.stg_bytes, v->fast_bits, v->n_tables),
                                     items, forced_groups, st);
}

// Views in 8-column-group tile order (16-byte chunks) take a kernel with the
// row-wise merge for them (merge_tile_groups8); all other launches a kernel
// without it.
template <int K, int CB>
int launch_decode(const BatchArgs &a, const TableArgs &t, const df11_view *v, const df11_decode_tuning &tune,
                  hipStream_t st)
{
    bool t8 = false;
    for (uint32_t i = 0; i < a.count; i++)
        t8 = t8 || (a.v[i].kc == 8 && a.v[i].pow2 && a.v[i].tr == 32);
    const uint64_t nseg = a.seg_begin[a.count];
    if constexpr (CB == 16)
        if (t8) return launch_kind<K, CB, 1>(a, t, v, nseg, tune.waves, tune.groups, st);
    if constexpr (CB == 16)
        if (a.stream) return launch_kind<K, CB, 3>(a, t, v, nseg, tune.waves, tune.groups, st);
    return launch_kind<K, CB, 0>(a, t, v, nseg, tune.waves, tune.groups, st);
}

}  // namespace

namespace {

// One launch over up to kMaxBatch views that share their tables and chunk size.
int decode_views(const df11_view *views, uint16_t *const *outs, uint32_t count, const df11_decode_tuning &tune,
                 hipStream_t st)
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
        if (v0 && v->chunk_bytes != v0->chunk_bytes)
            return df11::fail(DF11_E_ARG, "views of one batch must share their chunk size (view %u differs)", i);
        if (!v0) v0 = v;
        b.v[b.count] = make_args(v, outs[i]);
        b.seg_begin[b.count + 1] = b.seg_begin[b.count] + v->n_segments;
        b.count++;
        out_bytes += 2 * v->n;
        stg = std::max(stg, staging_bytes(v));
    }
    if (!b.count || !b.seg_begin[b.count]) return DF11_OK;
    b.stream = tune.stores == DF11_STORES_AUTO ? out_bytes > kStreamOutBytes : tune.stores == DF11_STORES_STREAMING;
    TableArgs t{v0->chain, v0->fast, (uint32_t)v0->n_chain, stg};
    if (v0->chunk_bytes == 8) {
        switch (v0->fast_bits) {
        case 8: return launch_decode<8, 8>(b, t, v0, tune, st);
        case 9: return launch_decode<9, 8>(b, t, v0, tune, st);
        case 10: return launch_decode<10, 8>(b, t, v0, tune, st);
        case 11: return launch_decode<11, 8>(b, t, v0, tune, st);
        default: return launch_decode<12, 8>(b, t, v0, tune, st);
        }
    }
    switch (v0->fast_bits) {
    case 8: return launch_decode<8, 16>(b, t, v0, tune, st);
    case 9: return launch_decode<9, 16>(b, t, v0, tune, st);
    case 10: return launch_decode<10, 16>(b, t, v0, tune, st);
    case 11: return launch_decode<11, 16>(b, t, v0, tune, st);
    default: return launch_decode<12, 16>(b, t, v0, tune, st);
    }
}

template <int CB>
int launch_rows(const RowArgs &a, const TableArgs &t, const df11_view *v, hipStream_t st)
{
    const uint64_t items = a.n_rows * a.split;
    switch (v->fast_bits) {
    case 8: return launch_kind<8, CB, 2>(a, t, v, items, 0, 0, st);
    case 9: return launch_kind<9, CB, 2>(a, t, v, items, 0, 0, st);
    case 10: return launch_kind<10, CB, 2>(a, t, v, items, 0, 0, st);
    case 11: return launch_kind<11, CB, 2>(a, t, v, items, 0, 0, st);
    default: return launch_kind<12, CB, 2>(a, t, v, items, 0, 0, st);
    }
}

int check_tuning(const df11_decode_tuning &t)
{
    if (t.waves && std::find(std::begin(kWaveChoices), std::end(kWaveChoices), (int)t.waves) == std::end(kWaveChoices))
        return df11::fail(DF11_E_ARG, "tuning: %u waves per workgroup (need 0 or one of 4, 6, ..., 16)", t.waves);
    if (t.stores > DF11_STORES_STREAMING) return df11::fail(DF11_E_ARG, "tuning: stores = %u", t.stores);
    if (t.groups > 0x7FFFFFFFu) return df11::fail(DF11_E_ARG, "tuning: groups = %u", t.groups);
    return DF11_OK;
}

}  // namespace

// Widest row window the row gather takes in window mode (waves per row).
constexpr uint32_t kRowWindowMax = 16;

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
    // A row overlaps at most cols / (elements per segment) + 2 segments.  A
    // few rows take that many waves each (at most 8), so that no wave
    // decodes two of a row's segments in turn; many rows take one wave
    // fewer, since every wave decodes a whole segment of which the row uses
    // a part (128256 x 4096 table, 8-byte chunks: 4.9 / 5.4 us for 1 / 32
    // ids at four waves per row; 2048 ids: 17.7 us at four, 12.7 at three).
    a.split = 1;
    const uint64_t slots = 16ull * (uint64_t)device_cu_count();
    const TableArgs t{v->chain, v->fast, (uint32_t)v->n_chain, staging_bytes(v)};
    if (v->n_segments && v->row_win_span && v->row_win_span <= kRowWindowMax && n_rows * v->row_win_span <= slots &&
        row_window_lds(v, v->row_win_span, t.stg_bytes)) {
        // window kernel: a workgroup per row, one wave per segment of the
        // row's window, no search before the segment loads, the row's bytes
        // in LDS (128256 x 4096 table, 8-byte chunks, an 11-segment window:
        // 1 / 32 ids in 4.4 / 4.8 us against 4.9 / 5.4 us with the search;
        // 16-byte chunks, 7 segments: 5.4 / 5.8 against 6.0 / 6.7)
        a.win = v->row_win_span;
        a.win_lo = v->row_win_lo;
        a.seg_per_elem = (double)v->n_segments / (double)v->n;
    } else if (v->n_segments) {
        const uint64_t per_seg = std::max<uint64_t>(1, v->n / v->n_segments);
        const uint64_t wide = std::min<uint64_t>(8, v->cols / per_seg + 2);
        a.split = (uint32_t)(n_rows * wide <= slots ? wide : std::max<uint64_t>(1, wide - 1));
    }
    if (n_rows > (UINT64_MAX >> 3)) return df11::fail(DF11_E_ARG, "df11_decode_rows: too many rows");
    hipStream_t st = (hipStream_t)stream;
    if (a.win) {
        // one workgroup per row, the row's sign+mantissa bytes in LDS
        const bool c8 = v->chunk_bytes == 8;
        switch (v->fast_bits) {
        case 8: return c8 ? launch_row_window<8, 8>(a, t, v, st) : launch_row_window<8, 16>(a, t, v, st);
        case 9: return c8 ? launch_row_window<9, 8>(a, t, v, st) : launch_row_window<9, 16>(a, t, v, st);
        case 10: return c8 ? launch_row_window<10, 8>(a, t, v, st) : launch_row_window<10, 16>(a, t, v, st);
        case 11: return c8 ? launch_row_window<11, 8>(a, t, v, st) : launch_row_window<11, 16>(a, t, v, st);
        default: return c8 ? launch_row_window<12, 8>(a, t, v, st) : launch_row_window<12, 16>(a, t, v, st);
        }
    }
    return v->chunk_bytes == 8 ? launch_rows<8>(a, t, v, st) : launch_rows<16>(a, t, v, st);
}

extern "C" int df11_decode(const df11_view *v, uint16_t *out, void *stream)
{
    int rc = check_view(v);
    if (rc) return rc;
    if (!v->n) return DF11_OK;
    if (!out || ((uintptr_t)out & 15)) return df11::fail(DF11_E_ARG, "out must be a 16-byte aligned device pointer");
    uint16_t *outs[1] = {out};
    return decode_views(v, outs, 1, df11_decode_tuning{}, (hipStream_t)stream);
}

extern "C" int df11_decode_batch_tuned(const df11_view *views, uint16_t *const *outs, uint32_t count,
                                       const df11_decode_tuning *tuning, void *stream)
{
    if (count && (!views || !outs)) return df11::fail(DF11_E_ARG, "df11_decode_batch: null pointer");
    const df11_decode_tuning tune = tuning ? *tuning : df11_decode_tuning{};
    int rc = check_tuning(tune);
    if (rc) return rc;
    for (uint32_t i = 0; i < count; i++) {
        rc = check_view(&views[i]);
        if (rc) return rc;
    }
    for (uint32_t i = 0; i < count; i += kMaxBatch) {
        rc = decode_views(views + i, outs + i, std::min(kMaxBatch, count - i), tune, (hipStream_t)stream);
        if (rc) return rc;
    }
    return DF11_OK;
}

extern "C" int df11_decode_batch(const df11_view *views, uint16_t *const *outs, uint32_t count, void *stream)
{
    return df11_decode_batch_tuned(views, outs, count, nullptr, stream);
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
