// df11_decode_gemm: y = x * W^T with the DFloat11 weight W decoded tile by
// tile into LDS and fed straight to bf16 matrix cores; the BF16 weight never
// exists in HBM.
//
// [P1] "DFloat11无损压缩技术：基于哈夫曼编码的BFloat16大模型显存优化方案" 2.2
//      item 3: weights are restored on the GPU right before the matmul and
//      dropped after it; the restore cost per forward does not depend on the
//      batch, so larger batches amortise it.
// [P3] "DFloat11重新定义LLM无损压缩的技术边界" 2.2 (locate, prefix sum,
//      reconstruct), 5.2 (a batch of 32 or more hides the decode cost).
//
// Layout (df11_gemm_layout): W [N, K] in 32 x 512 tiles, tiles row block by
// row block, each tile starting a new segment (block_seg[t] is its first
// segment), and inside a tile 8-column groups: group c holds rows 0..31, 8
// columns each.  That is the order of the B operand of
// v_mfma_f32_32x32x16_bf16: lane l reads row l % 32, columns 8 * (2 * step +
// l / 32) .. + 7, i.e. 8 consecutive stream elements, so operand reads are
// contiguous across lanes.
//
// Four kernels, chosen by the rows of x (B):
//   decode_gemm_vec_kernel   (B <= 2): the segment-parallel walk below with
//       the products formed as dot products on the vector ALU, one float32
//       partial sum per row of x and lane, at 6 waves per SIMD.
//   decode_gemm_seg_kernel   (B <= 40, the product path for small batches):
//       every wave walks its own segments of a 32-row block, decodes each
//       into its staging and feeds the matrix cores in rounds of 512
//       elements, with no barrier until the row block's partial sums are
//       reduced; one or two 32-row batch tiles.
//   decode_gemm_wide_kernel  (B > 40, and w_debug calls above 32 rows): a
//       workgroup decodes the next weight tile of one or two row blocks
//       into exponent planes while its matrix cores run on the current
//       tile, which was merged once into a BF16 plane in LDS shared by all
//       batch tiles.
//   decode_gemm_kernel       (w_debug calls up to 32 rows; DF11_GEMM_NARROW):
//       tile-synchronous, two exponent planes, every wave assembling its
//       own B operands from a plane and sign+mantissa bytes read from HBM.
// B operands are assembled with two bit-selects and two byte permutes per
// four weights; A operands (x, the batch) come from L2.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <type_traits>

#include "df11_device.h"
#include "df11_internal.h"

using namespace df11dev;

namespace {

constexpr uint32_t kTR = 32, kTC = 512, kKC = 8, kTile = kTR * kTC;
constexpr uint32_t kChunkBits = 128;
constexpr uint32_t kSegWords = 256;

typedef __attribute__((address_space(3))) float lds_f32;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

struct GemmArgs {
    const uint32_t *words;
    const uint8_t *sm;
    const uint8_t *gaps;
    const uint8_t *counts;
    const df11_segment *segs;
    const uint64_t *block_seg;
    const uint16_t *chain;
    const uint32_t *fast;
    const uint16_t *x;       // [B, K] bf16
    void *y;                 // [B, N] float32, or BF16 when y_bf16
    uint32_t y_bf16;
    uint16_t *w_debug;       // [N, K] or null
    uint32_t n_chain;
    uint32_t N, K, B;
    uint32_t tiles_per_row;  // K / 512
    uint32_t n_rowblocks;    // N / 32
    uint32_t split;          // K ranges per row block; > 1: y accumulated atomically
    uint32_t tiles_per_split;
    uint32_t parts;          // segment-parallel form: segment ranges per row block (> 1: y accumulated atomically)
    uint32_t stg_bytes;      // segment-parallel form: exponent staging per wave
    uint64_t n_segments;
    const uint4 *xo;         // x packed in operand order (x_pack_kernel), or null: x read in place
    uint32_t xo_tiles;       // batch tiles of the packing
};

struct SegLoad {
    uint4 own;
    uint32_t next, gap, count, nbits;
    uint64_t g0, g1;
};

// Segment records and tile starts are read-only for the launch: read through
// the constant address space they become scalar loads, tracked apart from
// the vector loads.
template <class T>
__device__ __forceinline__ const __attribute__((address_space(4))) T *as_const(const T *p)
{
    return (const __attribute__((address_space(4))) T *)p;
}

// The vector part is loaded unconditionally (the count from the gaps array
// when the view stores no counts), so no load carries a condition and each
// is first waited for where the decode uses it.
__device__ __forceinline__ SegLoad load_segment(const GemmArgs &g, uint64_t s, uint32_t lane)
{
    SegLoad L;
    const uint32_t *w = g.words + s * kSegWords + lane * 4;
    L.own = *reinterpret_cast<const uint4 *>(w);
    L.next = w[4];
    L.gap = g.gaps[s * 64 + lane];
    const uint8_t *cp = g.counts ? g.counts : g.gaps;
    L.count = cp[s * 64 + lane];
    const auto *rec = as_const(g.segs + s);
    L.g0 = rec[0].elem_off;
    L.g1 = rec[1].elem_off;
    L.nbits = rec[0].nbits;
    return L;
}

// float32 -> BF16, round to nearest, ties to even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t bf16_rne(float f)
{
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// y[i] = v for i = b * N + n: stored as float32 (added atomically when
// partial sums from several workgroups meet) or rounded once to BF16 (one
// writer per element).
__device__ __forceinline__ void store_y_at(const GemmArgs &g, uint64_t i, float v, bool add)
{
    if (g.y_bf16)
        reinterpret_cast<uint16_t *>(g.y)[i] = bf16_rne(v);
    else if (add)
        unsafeAtomicAdd(reinterpret_cast<float *>(g.y) + i, v);
    else
        reinterpret_cast<float *>(g.y)[i] = v;
}

__device__ __forceinline__ void store_y(const GemmArgs &g, uint32_t b, uint32_t n, float v, bool add)
{
    store_y_at(g, (uint64_t)b * g.N + n, v, add);
}

// Decode one tile-aligned segment into the exponent plane of its tile.
template <int K>
__device__ __forceinline__ void decode_into_plane(const SegLoad &L, uint64_t tile_start, uint32_t plane, bool stored,
                                                  uint32_t fast, uint32_t chain, uint32_t lane)
{
    if (L.g0 >= tile_start && L.g1 >= L.g0 && L.g1 <= tile_start + kTile) {
        const auto win = make_window(L.own, L.next, L.gap);
        uint32_t cnt = L.count;
        if (!stored) {   // no stored counts: the locate pass walks the chunk
            const uint32_t c0 = lane * kChunkBits;
            const uint32_t end = L.nbits > c0 ? min(kChunkBits, L.nbits - c0) : 0u;
            cnt = L.gap < end ? count_codes<K>(win, fast, chain, L.gap, end) : 0u;
        }
        uint32_t total;
        const uint32_t excl = wave_exclusive_scan(cnt, &total);
        if (total == (uint32_t)(L.g1 - L.g0))
            emit_codes<K>(win, fast, chain, plane + (uint32_t)(L.g0 - tile_start) + excl, cnt);
    }
}

// One workgroup of WAVES wavefronts takes a unit = (32-row block, range of
// K tiles).  MT: 32-row tiles of the batch (B <= 32 * MT).  Wave w works on
// batch tiles m = w % MT (and + WAVES, ... when MT > WAVES) and on the
// k-steps ks = w / MT (mod WAVES / MT) of every weight tile.
template <int K, int MT, int WAVES>
__global__ void __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(4, 8)))
decode_gemm_kernel(GemmArgs g)
{
    constexpr int kMPerWave = MT > WAVES ? MT / WAVES : 1;
    constexpr int kKSlices = MT >= WAVES ? 1 : WAVES / MT;
    constexpr uint32_t kThreads = WAVES * 64;
    extern __shared__ __align__(16) uint8_t lds_raw[];
    const uint32_t lds0 = (uint32_t)(size_t)(lds_u8 *)lds_raw;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lane = lane_id();
    // [guard][exponent plane 0][exponent plane 1][tables]
    const uint32_t eplane0 = lds0 + 16;
    const uint32_t fast = eplane0 + 2 * kTile;
    const uint32_t chain = fast + (8u << K);

    stage_tables<K, kThreads>(fast, chain, g.fast, g.chain, g.n_chain);
    __syncthreads();

    const uint32_t kslice = kKSlices > 1 ? wave / MT : 0;
    const uint32_t m_first = kKSlices > 1 ? wave % MT : wave;
    const uint32_t n_l = lane & 31, khalf = lane >> 5;
    const bool writes_w = g.w_debug && m_first == 0;
    const uint32_t n_units = g.n_rowblocks * g.split;

    for (uint32_t unit = blockIdx.x; unit < n_units; unit += gridDim.x) {
        const uint32_t rb = unit / g.split, sp = unit - rb * g.split;
        const uint32_t kt0 = sp * g.tiles_per_split;
        const uint32_t kt1 = min(kt0 + g.tiles_per_split, g.tiles_per_row);
        f32x16 acc[kMPerWave];
#pragma unroll
        for (int m = 0; m < kMPerWave; m++)
#pragma unroll
            for (int j = 0; j < 16; j++) acc[m][j] = 0.0f;

        {   // first tile of the range
            const uint64_t t0 = (uint64_t)rb * g.tiles_per_row + kt0;
            const uint64_t s1 = min(g.block_seg[t0 + 1], g.n_segments);
            for (uint64_t s = g.block_seg[t0] + wave; s < s1; s += WAVES)
                decode_into_plane<K>(load_segment(g, s, lane), t0 * kTile, eplane0, g.counts != nullptr, fast, chain, lane);
            __syncthreads();
        }

        for (uint32_t kt = kt0; kt < kt1; kt++) {
            const uint32_t cur = (kt - kt0) & 1;
            const bool has_next = kt + 1 < kt1;
            const uint64_t t = (uint64_t)rb * g.tiles_per_row + kt;
            // next tile's first segment in flight during the matrix work
            SegLoad nseg{};
            uint64_t ns0 = 0, ns1 = 0;
            if (has_next) {
                ns0 = g.block_seg[t + 1] + wave;
                ns1 = min(g.block_seg[t + 2], g.n_segments);
                if (ns0 < ns1) nseg = load_segment(g, ns0, lane);
            }

            const uint32_t ep = eplane0 + cur * kTile;
            const uint8_t *smt = g.sm + t * kTile;
            if constexpr (MT == 1) {
                // one batch tile: this tile's sign+mantissa bytes and x loads
                // go out first and land while the next tile decodes
                constexpr uint32_t kS = kTC / 16 / kKSlices;
                uint2 svs[kS];
#pragma unroll
                for (uint32_t i = 0; i < kS; i++) {
                    const uint32_t ks = kslice + i * kKSlices;
                    const uint32_t off = (2 * ks + khalf) * (kTR * kKC) + n_l * kKC;
                    svs[i] = *reinterpret_cast<const uint2 *>(smt + off);
                }
                if (has_next) {
                    const uint32_t np = eplane0 + (cur ^ 1) * kTile;
                    for (uint64_t s = ns0; s < ns1; s += WAVES)
                        decode_into_plane<K>(s == ns0 ? nseg : load_segment(g, s, lane), (t + 1) * kTile, np,
                                             g.counts != nullptr, fast, chain, lane);
                }
#pragma unroll
                for (uint32_t i = 0; i < kS; i++) {
                    const uint32_t ks = kslice + i * kKSlices;
                    const uint32_t c = 2 * ks + khalf;
                    const uint32_t off = c * (kTR * kKC) + n_l * kKC;
                    const uint2 rx = ld64(ep + off);
                    const uint2 lo = assemble4(svs[i].x, rx.x), hi = assemble4(svs[i].y, rx.y);
                    if (writes_w)
                        *reinterpret_cast<uint4 *>(g.w_debug + (uint64_t)(rb * kTR + n_l) * g.K + kt * kTC + c * kKC) =
                            make_uint4(lo.x, lo.y, hi.x, hi.y);
                    uint4 xa = make_uint4(0, 0, 0, 0);
                    if (n_l < g.B)
                        xa = *reinterpret_cast<const uint4 *>(g.x + (uint64_t)n_l * g.K + kt * kTC + ks * 16 + khalf * 8);
                    acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, xa), __builtin_bit_cast(bf16x8, v4u32{lo.x, lo.y, hi.x, hi.y}),
                        acc[0], 0, 0, 0);
                }
            } else {
                // matrix cores on tile t: B operand = 8 weights of row n_l, group c
    #pragma unroll 4
                for (uint32_t i = 0; i < kTC / 16 / kKSlices; i++) {
                    const uint32_t ks = kslice + i * kKSlices;
                    const uint32_t c = 2 * ks + khalf;
                    const uint32_t off = c * (kTR * kKC) + n_l * kKC;
                    const uint2 sv = *reinterpret_cast<const uint2 *>(smt + off);
                    const uint2 rx = ld64(ep + off);
                    const uint2 lo = assemble4(sv.x, rx.x), hi = assemble4(sv.y, rx.y);
                    const v4u32 wb{lo.x, lo.y, hi.x, hi.y};
                    if (writes_w)
                        *reinterpret_cast<uint4 *>(g.w_debug + (uint64_t)(rb * kTR + n_l) * g.K + kt * kTC + c * kKC) =
                            make_uint4(lo.x, lo.y, hi.x, hi.y);
                    const bf16x8 bop = __builtin_bit_cast(bf16x8, wb);
#pragma unroll
                    for (int m = 0; m < kMPerWave; m++) {
                        const uint32_t brow = (m_first + m * WAVES) * 32 + n_l;
                        uint4 xa = make_uint4(0, 0, 0, 0);
                        if (brow < g.B)
                            xa = *reinterpret_cast<const uint4 *>(g.x + (uint64_t)brow * g.K + kt * kTC + ks * 16 + khalf * 8);
                        acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, xa), bop, acc[m], 0, 0, 0);
                    }
                }

                // next tile into the other plane
                if (has_next) {
                    const uint32_t np = eplane0 + (cur ^ 1) * kTile;
                    for (uint64_t s = ns0; s < ns1; s += WAVES)
                        decode_into_plane<K>(s == ns0 ? nseg : load_segment(g, s, lane), (t + 1) * kTile, np,
                                             g.counts != nullptr, fast, chain, lane);
                }
            }
            __syncthreads();
        }

        // reduce the k-slices through LDS (the planes are free after the last barrier)
        if (kKSlices > 1) {
            lds_f32 *red = (lds_f32 *)(size_t)eplane0;
            if (kslice > 0)
#pragma unroll
                for (int j = 0; j < 16; j++) red[((kslice - 1) * MT + m_first) * 1024 + j * 64 + lane] = acc[0][j];
            __syncthreads();
            if (kslice == 0) {
#pragma unroll 1
                for (uint32_t ksl = 1; ksl < (uint32_t)kKSlices; ksl++)
#pragma unroll
                    for (int j = 0; j < 16; j++) acc[0][j] += red[((ksl - 1) * MT + m_first) * 1024 + j * 64 + lane];
            }
        }
        // y[b, n]: lane holds n = rb*32 + lane%32, b = m*32 + 8*blk + 4*(lane/32) + e
        if (kslice == 0) {
#pragma unroll
            for (int m = 0; m < kMPerWave; m++) {
                const uint32_t mt = m_first + m * WAVES;
#pragma unroll
                for (int blk = 0; blk < 4; blk++)
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const uint32_t b = mt * 32 + 8 * blk + 4 * khalf + e;
                        if (b < g.B) store_y(g, b, rb * kTR + n_l, acc[m][4 * blk + e], g.split > 1);
                    }
            }
        }
        __syncthreads();   // the reduction buffer and planes are reused by the next unit
    }
}


// ---------------------------------------------------------------- B <= 40
// Segment-parallel form for one or two batch tiles.  The tile-synchronous kernel
// above decodes a weight tile (~6 segments) per step with a barrier between
// steps, so a workgroup waits for one segment's decode latency per 16K
// weights.  Here every wave walks its own run of segments of one row block,
// like the plain decode: the next segment's words and this segment's
// sign+mantissa bytes and x operands are in flight during the decode, and
// nothing waits on a barrier until the row block's partial sums are
// reduced.  A segment's elements are taken in rounds of 64 units of 8
// (aligned to 512 elements of the tile, i.e. to one 16-column k-step): in
// the 8-column-group tile order, unit u of a tile is row u % 32, columns
// 8 * (u / 32) .. + 7, so a round is exactly the B operand of one
// v_mfma_f32_32x32x16_bf16 (lanes 0..31 the even column group, 32..63 the
// odd one), issued once per batch tile.  Elements of the round outside the
// segment are masked to zero,
// so the neighbouring segments that share a round add their own parts.
constexpr int kSegRounds = 4;   // rounds whose operands are loaded before the decode

// byte mask of elements [first, last) of an 8-element unit
__device__ __forceinline__ uint2 unit_mask(int first, int last)
{
    first = max(first, 0);
    last = min(last, 8);
    if (first >= last) return make_uint2(0u, 0u);
    const uint64_t m = (~0ull << (8 * first)) & (~0ull >> (64 - 8 * last));
    return make_uint2((uint32_t)m, (uint32_t)(m >> 32));
}

template <int K>
__device__ __forceinline__ bool stage_seg(const SegLoad &L, bool stored, uint32_t dst, uint32_t fast,
                                          uint32_t chain, uint32_t lane)
{
    const auto win = make_window(L.own, L.next, L.gap);
    uint32_t cnt = L.count;
    if (!stored) {
        const uint32_t c0 = lane * kChunkBits;
        const uint32_t end = L.nbits > c0 ? min(kChunkBits, L.nbits - c0) : 0u;
        cnt = L.gap < end ? count_codes<K>(win, fast, chain, L.gap, end) : 0u;
    }
    uint32_t total;
    const uint32_t excl = wave_exclusive_scan(cnt, &total);
    if (total != (uint32_t)(L.g1 - L.g0)) return false;
    emit_codes<K>(win, fast, chain, dst + excl, cnt);
    wave_lds_sync();
    return true;
}

template <int K, int WAVES, int MT>
__global__ void __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(4, 8)))
decode_gemm_seg_kernel(GemmArgs g)
{
    // MT batch tiles of 32 rows share each round's B operand.  With one tile
    // its x operands are loaded with the sign+mantissa bytes before the
    // decode; with two, the registers go to the second accumulator and x
    // is loaded in the round (from L2).
    static_assert(MT == 1 || MT == 2, "one or two batch tiles");
    extern __shared__ __align__(16) uint8_t lds_raw[];
    const uint32_t lds0 = (uint32_t)(size_t)(lds_u8 *)lds_raw;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lane = lane_id();
    // [guard][staging: WAVES x stg_bytes, also the reduction buffer][tables]
    const uint32_t area = lds0 + 16;
    const uint32_t stg = area + wave * g.stg_bytes;
    const uint32_t fast = area + WAVES * g.stg_bytes;
    const uint32_t chain = fast + (8u << K);
    stage_tables<K, WAVES * 64>(fast, chain, g.fast, g.chain, g.n_chain);
    __syncthreads();

    const uint32_t n_l = lane & 31, khalf = lane >> 5;
    const bool stored = g.counts != nullptr;
    const uint64_t n_elems = (uint64_t)g.N * g.K;
    const uint32_t n_units = g.n_rowblocks * g.parts;
    for (uint32_t unit = blockIdx.x; unit < n_units; unit += gridDim.x) {
        const uint32_t rb = unit / g.parts, part = unit - rb * g.parts;
        const auto *bs = as_const(g.block_seg);
        const uint64_t S0 = min(bs[(uint64_t)rb * g.tiles_per_row], g.n_segments);
        const uint64_t S1 = min(bs[(uint64_t)(rb + 1) * g.tiles_per_row], g.n_segments);
        const uint64_t len = S1 > S0 ? (S1 - S0 + g.parts - 1) / g.parts : 0;
        const uint64_t s_begin = S0 + part * len, s_end = min(S1, s_begin + len);

        f32x16 acc[MT];
#pragma unroll
        for (int m = 0; m < MT; m++)
#pragma unroll
            for (int j = 0; j < 16; j++) acc[m][j] = 0.0f;

        uint64_t s = s_begin + wave;
        SegLoad nx{};
        if (s < s_end) nx = load_segment(g, s, lane);
        while (s < s_end) {
            const SegLoad cur = nx;
            const uint64_t s_next = s + WAVES;
            const bool more = s_next < s_end;
            nx = load_segment(g, more ? s_next : s, lane);

            // the segment inside its tile: elements [lo, hi), rounds from unit u0
            const uint64_t t = cur.g0 >> 14;
            bool valid = cur.g0 < n_elems && cur.g1 >= cur.g0 && cur.g1 <= min((t + 1) << 14, n_elems) &&
                         t / g.tiles_per_row == rb;
            const uint64_t tile_start = valid ? t << 14 : 0ull;
            const uint32_t lo = valid ? (uint32_t)(cur.g0 - tile_start) : 0u;
            const uint32_t hi = valid ? (uint32_t)(cur.g1 - tile_start) : 0u;
            const uint32_t u0 = (lo >> 9) << 6, head = lo & 511u;
            valid = valid && head + (hi - lo) + 512 <= g.stg_bytes;
            const uint32_t nrounds = valid ? (hi - u0 * 8 + 511) >> 9 : 0u;
            const uint32_t kt = valid ? (uint32_t)(t - (uint64_t)rb * g.tiles_per_row) : 0u;
            const uint8_t *smt = g.sm + tile_start;
            const uint16_t *xr = g.x + (uint64_t)n_l * g.K + kt * kTC + khalf * 8;
            // x operand of batch tile m in round r (rows past B are zero)
            auto x_op = [&](int m, uint32_t r) {
                if (g.xo) return g.xo[((uint64_t)(kt * 32u + u0 / 64 + r) * g.xo_tiles + m) * 64 + lane];
                return n_l + 32u * m < g.B
                           ? *reinterpret_cast<const uint4 *>(xr + (uint64_t)(32u * m) * g.K + (u0 / 64 + r) * 16)
                           : make_uint4(0, 0, 0, 0);
            };

            // operands of the first rounds (rounds past the segment reload its last round)
            uint2 smp[kSegRounds];
            uint4 xp[MT == 1 ? kSegRounds : 1];
            const uint32_t last_round = nrounds ? nrounds - 1 : 0u;
#pragma unroll
            for (int r = 0; r < kSegRounds; r++) {
                const uint32_t rr = min((uint32_t)r, last_round);
                smp[r] = *reinterpret_cast<const uint2 *>(smt + 8 * (u0 + 64 * rr + lane));
                if constexpr (MT == 1) xp[r] = x_op(0, rr);
            }

            if (valid && stage_seg<K>(cur, stored, stg + head, fast, chain, lane)) {
                auto round = [&](uint32_t r, uint2 sv, const uint4 *xa) {
                    uint4 xl[MT];
                    if constexpr (MT > 1)
#pragma unroll
                        for (int m = 0; m < MT; m++) xl[m] = x_op(m, r);
                    const uint32_t u = u0 + 64 * r + lane;
                    const uint2 mk = unit_mask((int)lo - (int)(8 * u), (int)hi - (int)(8 * u));
                    const uint2 rx = ld64(stg + 8 * (64 * r + lane));
                    const uint2 a = assemble4(sv.x & mk.x, rx.x & mk.x), b = assemble4(sv.y & mk.y, rx.y & mk.y);
                    const bf16x8 bop = __builtin_bit_cast(bf16x8, v4u32{a.x, a.y, b.x, b.y});
#pragma unroll
                    for (int m = 0; m < MT; m++)
                        acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            __builtin_bit_cast(bf16x8, MT == 1 ? *xa : xl[m]), bop, acc[m], 0, 0, 0);
                };
#pragma unroll
                for (int r = 0; r < kSegRounds; r++)
                    if ((uint32_t)r < nrounds) round(r, smp[r], &xp[MT == 1 ? r : 0]);
                for (uint32_t r = kSegRounds; r < nrounds; r++) {
                    const uint2 sv = *reinterpret_cast<const uint2 *>(smt + 8 * (u0 + 64 * r + lane));
                    uint4 xa[1];
                    if constexpr (MT == 1) xa[0] = x_op(0, r);
                    round(r, sv, xa);
                }
            }
            wave_lds_sync();   // the staging is reused by the next segment
            s = s_next;
        }

        // reduce the waves' partial sums through LDS, one batch tile at a
        // time (the staging is free after the barrier and holds WAVES - 1
        // tiles of 32 x 32 floats)
        lds_f32 *red = (lds_f32 *)(size_t)area;
#pragma unroll
        for (int m = 0; m < MT; m++) {
            __syncthreads();
            if (wave > 0)
#pragma unroll
                for (int j = 0; j < 16; j++) red[(wave - 1) * 1024 + j * 64 + lane] = acc[m][j];
            __syncthreads();
            if (wave == 0) {
#pragma unroll 1
                for (uint32_t w = 1; w < (uint32_t)WAVES; w++)
#pragma unroll
                    for (int j = 0; j < 16; j++) acc[m][j] += red[(w - 1) * 1024 + j * 64 + lane];
                // y[b, n]: lane holds n = rb*32 + lane%32, b = 32*m + 8*blk + 4*(lane/32) + e.
                // B and N pass through an empty asm so that the sixteen
                // addresses and masks are formed here, not kept in registers
                // across the unit loop.
                uint32_t nB = g.B, nN = g.N;
                asm volatile("" : "+s"(nB), "+s"(nN));
#pragma unroll
                for (int blk = 0; blk < 4; blk++)
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const uint32_t b = 32 * m + 8 * blk + 4 * khalf + e;
                        if (b < nB) store_y_at(g, (uint64_t)b * nN + rb * kTR + n_l, acc[m][4 * blk + e], g.parts > 1);
                    }
            }
        }
        __syncthreads();   // the staging is reused by the next unit
    }
}

// ---------------------------------------------------------------- B <= 2
// Vector form for one or two rows of x.  A matrix-core product spends its
// 16-register accumulator and 16-byte operands on 32 batch rows of which
// one or two are used; here the products are dot products on the vector
// ALU (v_dot2c_f32_bf16, two BF16 products and a float32 add per
// instruction), so a wave holds one float32 partial sum per row of x and
// the kernel fits 6 waves per SIMD (80 VGPRs) against the segment-parallel
// kernel's 4, which is what the latency-bound decode chain needs.  The walk
// over a row block's segments, the staging and the 512-element rounds are
// those of the segment-parallel kernel: unit u0 + 64 r + lane of a round is
// row lane % 32 of the row block and columns 16 (u0 / 64 + r) + 8 (lane /
// 32) .. + 7 of the tile, so a lane's row is fixed for the whole row block
// and it needs the 16 bytes of x at those columns.  At the end of a row
// block lanes l and l + 32 (the two column halves) are added, then the
// waves through LDS, and one wave writes the 32 sums per row of x.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t w, uint32_t x, float acc)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, x), acc, false);
}

template <int K, int WAVES, int NB>
__global__ void __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(6, 8)))
decode_gemm_vec_kernel(GemmArgs g)
{
    constexpr int kXAhead = 4 / NB;   // rounds whose x slices are loaded before the decode
    extern __shared__ __align__(16) uint8_t lds_raw[];
    const uint32_t lds0 = (uint32_t)(size_t)(lds_u8 *)lds_raw;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lane = lane_id();
    // [guard][staging: WAVES x stg_bytes, also the reduction buffer][tables]
    const uint32_t area = lds0 + 16;
    const uint32_t stg = area + wave * g.stg_bytes;
    const uint32_t fast = area + WAVES * g.stg_bytes;
    const uint32_t chain = fast + (8u << K);
    stage_tables<K, WAVES * 64>(fast, chain, g.fast, g.chain, g.n_chain);
    __syncthreads();

    const uint32_t khalf = lane >> 5;
    const bool stored = g.counts != nullptr;
    const uint64_t n_elems = (uint64_t)g.N * g.K;
    const uint32_t n_units = g.n_rowblocks * g.parts;
    for (uint32_t unit = blockIdx.x; unit < n_units; unit += gridDim.x) {
        const uint32_t rb = unit / g.parts, part = unit - rb * g.parts;
        const auto *bs = as_const(g.block_seg);
        const uint64_t S0 = min(bs[(uint64_t)rb * g.tiles_per_row], g.n_segments);
        const uint64_t S1 = min(bs[(uint64_t)(rb + 1) * g.tiles_per_row], g.n_segments);
        const uint64_t len = S1 > S0 ? (S1 - S0 + g.parts - 1) / g.parts : 0;
        const uint64_t s_begin = S0 + part * len, s_end = min(S1, s_begin + len);
        float acc[NB];
#pragma unroll
        for (int b = 0; b < NB; b++) acc[b] = 0.0f;

        uint64_t s = s_begin + wave;
        SegLoad nx{};
        if (s < s_end) nx = load_segment(g, s, lane);
        while (s < s_end) {
            const SegLoad cur = nx;
            const uint64_t s_next = s + WAVES;
            const bool more = s_next < s_end;
            nx = load_segment(g, more ? s_next : s, lane);

            // the segment inside its tile: elements [lo, hi), rounds from unit u0
            const uint64_t t = cur.g0 >> 14;
            bool valid = cur.g0 < n_elems && cur.g1 >= cur.g0 && cur.g1 <= min((t + 1) << 14, n_elems) &&
                         t / g.tiles_per_row == rb;
            const uint64_t tile_start = valid ? t << 14 : 0ull;
            const uint32_t lo = valid ? (uint32_t)(cur.g0 - tile_start) : 0u;
            const uint32_t hi = valid ? (uint32_t)(cur.g1 - tile_start) : 0u;
            const uint32_t u0 = (lo >> 9) << 6, head = lo & 511u;
            valid = valid && head + (hi - lo) + 512 <= g.stg_bytes;
            const uint32_t nrounds = valid ? (hi - u0 * 8 + 511) >> 9 : 0u;
            const uint32_t kt = valid ? (uint32_t)(t - (uint64_t)rb * g.tiles_per_row) : 0u;
            const uint8_t *smt = g.sm + tile_start;
            const uint16_t *xr = g.x + kt * kTC + (u0 / 64) * 16 + khalf * 8;
            // the 8 x values of round r for row b of x (b < B)
            auto x_at = [&](int b, uint32_t r) {
                return *reinterpret_cast<const uint4 *>(xr + (uint64_t)min((uint32_t)b, g.B - 1) * g.K + r * 16);
            };

            // operands of the first rounds (rounds past the segment reload its last round)
            uint2 smp[kSegRounds];
            uint4 xp[kXAhead][NB];
            const uint32_t last_round = nrounds ? nrounds - 1 : 0u;
#pragma unroll
            for (int r = 0; r < kSegRounds; r++) {
                const uint32_t rr = min((uint32_t)r, last_round);
                smp[r] = *reinterpret_cast<const uint2 *>(smt + 8 * (u0 + 64 * rr + lane));
                if (r < kXAhead)
#pragma unroll
                    for (int b = 0; b < NB; b++) xp[r < kXAhead ? r : 0][b] = x_at(b, rr);
            }

            if (valid && stage_seg<K>(cur, stored, stg + head, fast, chain, lane)) {
                auto round = [&](uint32_t r, uint2 sv, const uint4 *xv) {
                    const uint32_t u = u0 + 64 * r + lane;
                    const uint2 mk = unit_mask((int)lo - (int)(8 * u), (int)hi - (int)(8 * u));
                    const uint2 rx = ld64(stg + 8 * (64 * r + lane));
                    const uint2 a = assemble4(sv.x & mk.x, rx.x & mk.x), c = assemble4(sv.y & mk.y, rx.y & mk.y);
#pragma unroll
                    for (int b = 0; b < NB; b++) {
                        float v = dot2_bf16(a.x, xv[b].x, acc[b]);
                        v = dot2_bf16(a.y, xv[b].y, v);
                        v = dot2_bf16(c.x, xv[b].z, v);
                        acc[b] = dot2_bf16(c.y, xv[b].w, v);
                    }
                };
#pragma unroll
                for (int r = 0; r < kSegRounds; r++)
                    if ((uint32_t)r < nrounds) {
                        if (r < kXAhead) {
                            round(r, smp[r], xp[r < kXAhead ? r : 0]);
                        } else {
                            uint4 xv[NB];
#pragma unroll
                            for (int b = 0; b < NB; b++) xv[b] = x_at(b, r);
                            round(r, smp[r], xv);
                        }
                    }
                for (uint32_t r = kSegRounds; r < nrounds; r++) {
                    const uint2 sv = *reinterpret_cast<const uint2 *>(smt + 8 * (u0 + 64 * r + lane));
                    uint4 xv[NB];
#pragma unroll
                    for (int b = 0; b < NB; b++) xv[b] = x_at(b, r);
                    round(r, sv, xv);
                }
            }
            wave_lds_sync();   // the staging is reused by the next segment
            s = s_next;
        }

        // the two column halves, then the waves through LDS (the staging is
        // free after the barrier); wave 0 sums them in wave order
        lds_f32 *red = (lds_f32 *)(size_t)area;
#pragma unroll
        for (int b = 0; b < NB; b++) acc[b] += __shfl_xor(acc[b], 32);
        __syncthreads();
        if (lane < 32)
#pragma unroll
            for (int b = 0; b < NB; b++) red[(wave * NB + b) * 32 + lane] = acc[b];
        __syncthreads();
        if (wave == 0 && lane < 32) {
#pragma unroll
            for (int b = 0; b < NB; b++) {
                float v = 0.0f;
#pragma unroll 1
                for (uint32_t w = 0; w < (uint32_t)WAVES; w++) v += red[(w * NB + b) * 32 + lane];
                if ((uint32_t)b < g.B) store_y_at(g, (uint64_t)b * g.N + rb * kTR + lane, v, g.parts > 1);
            }
        }
        __syncthreads();   // the staging is reused by the next unit
    }
}

// ---------------------------------------------------------------- B > 40
// Wide batches.  In the tile-synchronous kernel every wave builds the B
// operand of every k-step (exponent plane + sign+mantissa bytes, two
// bit-selects and two byte permutes per four weights) for its own batch
// tile, so a weight is assembled and its byte loaded once per batch tile.
// Here the decoded tile is merged once per workgroup into a BF16 plane in
// LDS, laid out in the tile order, which is the operand order of
// v_mfma_f32_32x32x16_bf16: the B operand of k-step s for lane l is the 16
// bytes of unit (2s + l/32) * 32 + l%32, a conflict-free 16-byte LDS read
// shared by all batch tiles.  Per weight tile:
//   1. the next tile's sign+mantissa bytes (4 units per thread) and this
//      wave's first x operands are loaded, and the next tile's segments are
//      decoded into the exponent plane (one wave per segment);
//   2. matrix cores on the current tile from the BF16 plane;
//   3. barrier; the next tile is merged into the BF16 plane; barrier.
// LDS: one 16 KB exponent plane, one 32 KB BF16 plane and the tables.
constexpr int kWideXAhead = 8;   // k-steps whose x operands are loaded before the decode

// RB row blocks per unit (8 * RB waves): each x operand feeds RB matrix
// core products, so x is read from L2 once per RB row blocks.
template <int K, int MT, int RB>
__global__ void __launch_bounds__(8 * RB * 64) __attribute__((amdgpu_waves_per_eu(4, 8)))
decode_gemm_wide_kernel(GemmArgs g)
{
    constexpr int WAVES = 8 * RB;
    constexpr int kKSlices = WAVES / MT;
    constexpr int kSteps = (int)(kTC / 16) / kKSlices;             // k-steps per wave and tile
    constexpr int kAhead = kSteps < kWideXAhead ? kSteps : kWideXAhead;
    constexpr uint32_t kThreads = WAVES * 64;
    constexpr uint32_t kTileUnits = kTile / 8;
    constexpr uint32_t kPerThread = RB * kTileUnits / kThreads;     // merge units per thread
    static_assert(WAVES % MT == 0 && kPerThread * kThreads == RB * kTileUnits, "shape");
    extern __shared__ __align__(16) uint8_t lds_raw[];
    const uint32_t lds0 = (uint32_t)(size_t)(lds_u8 *)lds_raw;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lane = lane_id();
    // [guard][RB exponent planes][RB BF16 planes][tables]
    const uint32_t eplane = lds0 + 16;
    const uint32_t wplane = eplane + RB * kTile;
    const uint32_t fast = wplane + RB * 2 * kTile;
    const uint32_t chain = fast + (8u << K);

    stage_tables<K, kThreads>(fast, chain, g.fast, g.chain, g.n_chain);
    __syncthreads();

    const uint32_t kslice = wave / MT;
    const uint32_t m = wave % MT;   // this wave's batch tile
    const bool stored = g.counts != nullptr;
    const uint32_t n_groups = (g.n_rowblocks + RB - 1) / RB;
    const uint32_t n_units = n_groups * g.split;

    // (tid: the thread index, passed through an empty asm statement per tile
    // step so that the thread-derived addresses are formed where they are
    // used instead of being kept in registers across the loops)
    auto load_sm = [&](uint32_t tid, uint32_t rb0, uint32_t nrb, uint32_t kt, uint2 (&sv)[kPerThread]) {
#pragma unroll
        for (uint32_t j = 0; j < kPerThread; j++) {
            const uint32_t u = tid + j * kThreads, r = u / kTileUnits, uu = u % kTileUnits;
            const uint64_t t = (uint64_t)(rb0 + (r < nrb ? r : 0)) * g.tiles_per_row + kt;
            sv[j] = *reinterpret_cast<const uint2 *>(g.sm + t * kTile + 8u * uu);
        }
    };
    auto decode_tiles = [&](uint32_t rb0, uint32_t nrb, uint32_t kt) {
        const auto *bs = as_const(g.block_seg);
        uint64_t first[RB], count[RB], total = 0;
#pragma unroll
        for (int r = 0; r < RB; r++) {
            const uint64_t t = (uint64_t)(rb0 + r) * g.tiles_per_row + kt;
            first[r] = (uint32_t)r < nrb ? min(bs[t], g.n_segments) : 0;
            const uint64_t end = (uint32_t)r < nrb ? min(bs[t + 1], g.n_segments) : 0;
            count[r] = end > first[r] ? end - first[r] : 0;
            total += count[r];
        }
        for (uint64_t j = wave; j < total; j += WAVES) {
            uint64_t jj = j;
            int r = 0;
#pragma unroll
            for (int q = 0; q + 1 < RB; q++)
                if (r == q && jj >= count[q]) { jj -= count[q]; r = q + 1; }
            const uint64_t t = (uint64_t)(rb0 + r) * g.tiles_per_row + kt;
            decode_into_plane<K>(load_segment(g, first[r] + jj, lane), t * kTile, eplane + r * kTile, stored, fast,
                                 chain, lane);
        }
    };
    // exponent planes + bytes -> BF16 planes (and w_debug), units u = tid + j * threads
    auto merge = [&](uint32_t tid, const uint2 (&sv)[kPerThread], uint32_t rb0, uint32_t nrb, uint32_t kt) {
#pragma unroll
        for (uint32_t j = 0; j < kPerThread; j++) {
            const uint32_t u = tid + j * kThreads, r = u / kTileUnits, uu = u % kTileUnits;
            if (r < nrb) {
                const uint2 rx = ld64(eplane + r * kTile + 8u * uu);
                const uint2 a = assemble4(sv[j].x, rx.x), b = assemble4(sv[j].y, rx.y);
                *(lds_u4 *)(size_t)(wplane + r * 2 * kTile + 16u * uu) = v4u32{a.x, a.y, b.x, b.y};
                if (g.w_debug)
                    *reinterpret_cast<uint4 *>(g.w_debug + (uint64_t)((rb0 + r) * kTR + (uu & 31u)) * g.K + kt * kTC +
                                               (uu >> 5) * kKC) = make_uint4(a.x, a.y, b.x, b.y);
            }
        }
    };
    auto x_op = [&](uint32_t tid, uint32_t kt, uint32_t ks) {
        if (g.xo) return g.xo[((uint64_t)(kt * 32u + ks) * MT + m) * 64 + (tid & 63u)];
        const uint32_t brow = m * 32 + (tid & 31u), khalf = (tid >> 5) & 1u;
        return brow < g.B ? *reinterpret_cast<const uint4 *>(g.x + (uint64_t)brow * g.K + kt * kTC + ks * 16 + khalf * 8)
                          : make_uint4(0, 0, 0, 0);
    };

    for (uint32_t unit = blockIdx.x; unit < n_units; unit += gridDim.x) {
        const uint32_t grp = unit / g.split, sp = unit - grp * g.split;
        const uint32_t rb0 = grp * RB, nrb = min((uint32_t)RB, g.n_rowblocks - rb0);
        const uint32_t kt0 = sp * g.tiles_per_split;
        const uint32_t kt1 = min(kt0 + g.tiles_per_split, g.tiles_per_row);
        f32x16 acc[RB];
#pragma unroll
        for (int r = 0; r < RB; r++)
#pragma unroll
            for (int j = 0; j < 16; j++) acc[r][j] = 0.0f;

        {   // the first tiles of the range
            uint32_t tid = threadIdx.x;
            asm volatile("" : "+v"(tid));
            uint2 sv[kPerThread];
            load_sm(tid, rb0, nrb, kt0, sv);
            decode_tiles(rb0, nrb, kt0);
            __syncthreads();
            merge(tid, sv, rb0, nrb, kt0);
            __syncthreads();
        }
        for (uint32_t kt = kt0; kt < kt1; kt++) {
            uint32_t tid = threadIdx.x;
            asm volatile("" : "+v"(tid));
            const uint32_t n_l = tid & 31u, khalf = (tid >> 5) & 1u;
            const bool has_next = kt + 1 < kt1;
            uint2 sv[kPerThread];
            uint4 xa[kAhead];
#pragma unroll
            for (int i = 0; i < kAhead; i++) xa[i] = x_op(tid, kt, kslice + i * kKSlices);
            if (has_next) {
                load_sm(tid, rb0, nrb, kt + 1, sv);
                decode_tiles(rb0, nrb, kt + 1);
            }
            // matrix cores on tile kt of every row block from the BF16 planes
            auto mma = [&](uint32_t ks, uint4 xv) {
#pragma unroll
                for (int r = 0; r < RB; r++)
                    if (RB == 1 || (uint32_t)r < nrb) {
                        const v4u32 wb =
                            *(const lds_u4 *)(size_t)(wplane + r * 2 * kTile + 16u * ((2 * ks + khalf) * kTR + n_l));
                        acc[r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, xv),
                                                                        __builtin_bit_cast(bf16x8, wb), acc[r], 0, 0, 0);
                    }
            };
#pragma unroll
            for (int i = 0; i < kAhead; i++) mma(kslice + i * kKSlices, xa[i]);
#pragma unroll 4
            for (int i = kAhead; i < kSteps; i++) {
                const uint32_t ks = kslice + i * kKSlices;
                mma(ks, x_op(tid, kt, ks));
            }
            __syncthreads();   // the BF16 planes are read, the next tiles' exponents are staged
            if (has_next) {
                merge(tid, sv, rb0, nrb, kt + 1);
                __syncthreads();
            }
        }

        // per row block: reduce the k-slices through LDS (the planes are free
        // after the last barrier) and store y[b, n]: lane holds
        // n = rb*32 + lane%32, b = 32*m + 8*blk + 4*(lane/32) + e
        lds_f32 *red = (lds_f32 *)(size_t)eplane;
#pragma unroll
        for (int r = 0; r < RB; r++) {
            if (kKSlices > 1) {
                if (r > 0) __syncthreads();
                if (kslice > 0)
#pragma unroll
                    for (int j = 0; j < 16; j++) red[((kslice - 1) * MT + m) * 1024 + j * 64 + lane] = acc[r][j];
                __syncthreads();
                if (kslice == 0) {
#pragma unroll 1
                    for (uint32_t ksl = 1; ksl < (uint32_t)kKSlices; ksl++)
#pragma unroll
                        for (int j = 0; j < 16; j++) acc[r][j] += red[((ksl - 1) * MT + m) * 1024 + j * 64 + lane];
                }
            }
            if (kslice == 0 && (uint32_t)r < nrb) {
                const uint32_t n_l = lane & 31u, khalf = lane >> 5;
                uint32_t nB = g.B, nN = g.N;
                asm volatile("" : "+s"(nB), "+s"(nN));   // addresses formed here, not kept across the unit loop
#pragma unroll
                for (int blk = 0; blk < 4; blk++)
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const uint32_t b = m * 32 + 8 * blk + 4 * khalf + e;
                        if (b < nB)
                            store_y_at(g, (uint64_t)b * nN + (rb0 + r) * kTR + n_l, acc[r][4 * blk + e], g.split > 1);
                    }
            }
        }
        __syncthreads();   // the planes are reused by the next unit
    }
}

// ---------------------------------------------------------------------------
// Pipelined kernel: decoder waves and matrix-core waves of one workgroup work
// on different tiles at once, handing tiles over through a ring of BF16 tile
// planes in LDS and two counters per ring slot, with no workgroup barrier
// after the table staging.
//
//   decoder waves (all but the first nm): take the segments of the
//     workgroup's tile sequence in turn (running segment index = wave
//     number mod the decoder count), wait until the tile's slot has been
//     released by every matrix-core wave, write each code's rotated
//     exponent into the high byte of its BF16 slot, merge the segment's
//     sign+mantissa bytes in place (whole 8-element units with one 16-byte
//     store, the units shared with a neighbouring segment element by
//     element), then add one to the slot's ready counter.  The next
//     segment's stream words and sign+mantissa bytes are loaded before the
//     current one is decoded.
//   matrix-core waves (waves 0 .. nm - 1, nm = ceil(ceil(B / 32) / TPW)):
//     wave m owns the TPW 32-row batch tiles m TPW .. m TPW + TPW - 1 and a
//     32 x 32 float32 accumulator for each; per tile it waits for the slot's
//     ready counter to reach the segments decoded into that slot so far,
//     runs the tile's 32 k-steps of v_mfma_f32_32x32x16_bf16 from the plane
//     (each B operand read once from LDS and used by TPW products), and
//     adds one to the slot's release counter.  Each y element has one writer
//     (unless K is split).  The decode bounds the kernel, so every wave the
//     products do not need decodes: two batch tiles per matrix-core wave
//     leave more decoder waves at large B.
//
// Waits are bounded spins on LDS (s_sleep between reads); a wait that runs
// out (not reachable with well-formed arguments: every counter is advanced
// by a wave that only waits on earlier tiles) lets the wave continue and
// makes the matrix-core wave store NaN.
constexpr uint32_t kPipePlane = 2 * kTile;         // bytes of one BF16 tile plane
constexpr uint32_t kPipeGuard = 16;                // LDS bytes before the first plane
constexpr uint32_t kPipeMaxSlots = 3;
// The emit cursor's high half holds plane / 2 + element index and must stay
// within 16 bits up to one past a tile's last element (the emit loops'
// end); the guard keeps the lowest position above 3 (its 4-code bound).
static_assert((kPipeGuard + kPipeMaxSlots * kPipePlane) / 2 <= 65535, "pipelined planes beyond the emit cursor");
static_assert(kPipeGuard / 2 >= 3, "pipelined emit bound");
constexpr uint32_t kPipePieces = 8;                // 8-element units per lane loaded ahead
constexpr uint32_t kPipeSpin = 1u << 22;

__device__ __forceinline__ bool lds_wait_geq(uint32_t addr, uint32_t target)
{
    bool ok = false;
    for (uint32_t i = 0; i < kPipeSpin; i++) {
        const uint32_t v = __builtin_amdgcn_readfirstlane(
            __hip_atomic_load((lds_u32 *)(size_t)addr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
        if ((int32_t)(v - target) >= 0) {
            ok = true;
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    return ok;
}

// all LDS accesses of this wave done, then one lane adds 1 to the counter
__device__ __forceinline__ void lds_signal(uint32_t addr, uint32_t lane)
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    if (lane == 0) __hip_atomic_fetch_add((lds_u32 *)(size_t)addr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// emit_codes with each rotated exponent written to the high byte of a
// 16-bit slot: the cursor's high half holds (plane byte address / 2 +
// element index) and, its low half never dropping below 32768, st >> 15 is
// the byte address of that high byte.  wpos >= 3 and wpos + cnt <= 65535.
template <int K, int NW>
__device__ __forceinline__ void emit_codes_hi(Window<NW> w, uint32_t fast, uint32_t chain, uint32_t wpos, uint32_t cnt)
{
    uint32_t st = (wpos << 16) | kM0;
    const uint32_t bound = (wpos + cnt - 3u) << 16;   // st < bound <=> at least 4 codes left
    while (st < bound) {
        const uint2 f = ld64(lshl_add_s<3>(w.w[0] >> (32 - K), fast));
        uint32_t syms = f.x, meta = f.y;
        if (meta == 0) {
            const uint32_t e = chain_decode(chain, w.w[0]);
            syms = rot_exp(e & 0xFFu);
            meta = (1u << 16) - ((e >> 8) & 0x3Fu);
        }
        const uint32_t a = st >> 15;
        uint32_t t = syms >> 8;
        asm("" : "+v"(t));
        st8(a, syms);
        st8(a + 2, t);
        st8(a + 4, syms >> 16);
        st8(a + 6, t >> 16);
        w.consume(meta);
        st += meta;
    }
    const uint32_t lend = wpos + cnt;
    while ((st >> 16) < lend) {
        const uint32_t e = chain_decode(chain, w.w[0]);
        const uint32_t step = (1u << 16) - ((e >> 8) & 0x3Fu);
        st8(st >> 15, rot_exp(e & 0xFFu));
        w.consume(step);
        st += step;
    }
}

// 8 BF16 slots holding rotated exponents in their high bytes + 8
// sign+mantissa bytes -> 8 BF16 words
__device__ __forceinline__ uint4 merge_hi(uint4 v, uint2 sm)
{
    const uint32_t rlo = __builtin_amdgcn_perm(v.y, v.x, 0x07050301u);
    const uint32_t rhi = __builtin_amdgcn_perm(v.w, v.z, 0x07050301u);
    const uint2 a = assemble4(sm.x, rlo), b = assemble4(sm.y, rhi);
    return make_uint4(a.x, a.y, b.x, b.y);
}

// 16 bytes from a pointer known to be global memory (a global, not a flat,
// load: it does not count against the LDS wait counter)
__device__ __forceinline__ uint4 ld_global128(const __attribute__((address_space(1))) uint8_t *p)
{
    const v4u32 v = *(const __attribute__((address_space(1))) v4u32 *)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint2 ld_global64(const __attribute__((address_space(1))) uint8_t *p)
{
    const v2u32 v = *(const __attribute__((address_space(1))) v2u32 *)p;
    return make_uint2(v.x, v.y);
}

// One segment job of a decoder wave, loaded ahead of its decode.
struct PipeJob {
    SegLoad L;
    uint2 sv[kPipePieces];
    uint64_t ts;          // first element of the segment's tile
    uint32_t a, b;        // the segment's elements inside its tile, [a, b); a = b when out of range
    uint32_t q;           // ring slot of the tile | its earlier uses of that slot << 2
};

// Walks the workgroup's tile sequence: units blockIdx.x, + gridDim.x, ...;
// unit = (row block, K range); tiles kt0 .. kt1 - 1 of the row block.
struct PipeSeq {
    uint32_t unit, kt, kt1, q;
    uint32_t t, first, nseg;   // tile, its first segment and segment count (n_segments < 2^32)
};

// block_seg[i] clamped to n_segments in 32-bit scalar arithmetic (64-bit
// ordered compares would run on the vector ALU)
__device__ __forceinline__ uint32_t pipe_seg(const GemmArgs &g, uint32_t i)
{
    const uint64_t v = as_const(g.block_seg)[i];
    const uint32_t n = (uint32_t)g.n_segments;
    return (uint32_t)(v >> 32) ? n : min((uint32_t)v, n);
}

__device__ __forceinline__ void pipe_tile(const GemmArgs &g, PipeSeq &p)
{
    p.first = pipe_seg(g, p.t);
    const uint32_t end = pipe_seg(g, p.t + 1);
    p.nseg = end > p.first ? end - p.first : 0;
}

__device__ __forceinline__ bool pipe_unit(const GemmArgs &g, PipeSeq &p, uint32_t n_units)
{
    if (p.unit >= n_units) return false;
    const uint32_t rb = p.unit / g.split, sp = p.unit - rb * g.split;
    p.kt = sp * g.tiles_per_split;
    p.kt1 = min(p.kt + g.tiles_per_split, g.tiles_per_row);
    p.t = rb * g.tiles_per_row + p.kt;
    pipe_tile(g, p);
    return true;
}

// next tile of the sequence; false past the last
__device__ __forceinline__ bool pipe_next(const GemmArgs &g, PipeSeq &p, uint32_t n_units)
{
    p.q++;
    if (p.kt + 1 < p.kt1) {
        p.kt++;
        p.t++;
        pipe_tile(g, p);
        return true;
    }
    p.unit += gridDim.x;
    return pipe_unit(g, p, n_units);
}

template <int K, int MT, int W, int TPW>
__global__ void __launch_bounds__(W * 64) decode_gemm_pipe_kernel(GemmArgs g, uint32_t nslot)
{
    static_assert((TPW == 1 || TPW == 2) && TPW <= MT, "batch tiles per matrix-core wave");
    extern __shared__ __align__(16) uint8_t lds_raw[];
    const uint32_t lds0 = (uint32_t)(size_t)(lds_u8 *)lds_raw;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lane = lane_id();
    // [guard][nslot BF16 planes][ready[4], release[4]][tables]
    const uint32_t planes = lds0 + kPipeGuard;
    const uint32_t ctr = planes + nslot * kPipePlane;
    const uint32_t fast = ctr + 64;
    const uint32_t chain = fast + (8u << K);
    if (threadIdx.x < 8) st32(ctr + 4 * threadIdx.x, 0u);
    stage_tables<K, W * 64>(fast, chain, g.fast, g.chain, g.n_chain);
    __syncthreads();

    // matrix-core waves, TPW batch tiles each (with two, a tile past the
    // rows of x reads zero rows of the packed x, or row B - 1 in place, and
    // its sums are not stored)
    const uint32_t nm = ((g.B + 31) / 32 + TPW - 1) / TPW;
    const uint32_t n_units = g.n_rowblocks * g.split;
    const bool stored = g.counts != nullptr;

    if (wave < nm) {
        // ---- matrix-core wave: batch tiles m0 .. m0 + TPW - 1
        const uint32_t m0 = wave * TPW;
        const bool writes_w = g.w_debug && m0 == 0;
        uint32_t cum[kPipeMaxSlots] = {};
        bool ok = true;
        f32x16 acc[TPW];
#pragma unroll
        for (int t = 0; t < TPW; t++)
#pragma unroll
            for (int j = 0; j < 16; j++) acc[t][j] = 0.0f;
        // one tile from ring slot `sl`: x operands of k-step ks and batch
        // tile m0 + t at xb[t] + ks * xs bytes (packed: the operand kilobyte
        // of that tile; in place: row (m0 + t) * 32 + n_l, clamped to row
        // B - 1, whose products only reach rows of y that are not stored),
        // issued before the wait; no branch inside the k-loop (w_debug calls
        // run their own copy of it)
        auto run_tile = [&](auto wd_tag, const PipeSeq &p, uint32_t sl, uint32_t target) {
            constexpr bool kWD = decltype(wd_tag)::value;
            uint32_t ln = lane;
            asm volatile("" : "+v"(ln));
            constexpr int kAhead = 8 / TPW;   // k-steps of x operands in flight per batch tile
            // global address space named explicitly: a generic (flat) load
            // would also count against the LDS wait counter, and every wait
            // for a plane read would then wait for the x loads in flight
            const __attribute__((address_space(1))) uint8_t *xb[TPW];
#pragma unroll
            for (int t = 0; t < TPW; t++) {
                const uint32_t brow = min((m0 + t) * 32 + (ln & 31u), g.B - 1);
                const uint8_t *gp = g.xo ? reinterpret_cast<const uint8_t *>(g.xo + ((uint64_t)p.kt * 32u * MT + m0 + t) * 64 + ln)
                                         : reinterpret_cast<const uint8_t *>(g.x + (uint64_t)brow * g.K + p.kt * kTC + (ln >> 5) * 8);
                xb[t] = (const __attribute__((address_space(1))) uint8_t *)gp;
            }
            const uint32_t xs = g.xo ? MT * 64u * 16u : 32u;
            uint4 xa[kAhead][TPW];
#pragma unroll
            for (int i = 0; i < kAhead; i++)
#pragma unroll
                for (int t = 0; t < TPW; t++) {
                    xa[i][t] = ld_global128(xb[t]);
                    xb[t] += xs;
                }
            ok &= lds_wait_geq(ctr + 4 * sl, target);
            const uint32_t rb = p.unit / g.split;
            const uint32_t pl = planes + sl * kPipePlane + 16u * ((ln >> 5) * kTR + (ln & 31u));
            uint16_t *wd = nullptr;
            if constexpr (kWD) wd = g.w_debug + (uint64_t)(rb * kTR + (ln & 31u)) * g.K + p.kt * kTC + (ln >> 5) * kKC;
            // k-step i: groups c = 2 i + lane / 32, row n_l; the plane's
            // operands are read kWAhead k-steps before their products
            constexpr int kWAhead = 4 / TPW;
            v4u32 wq[kWAhead];
#pragma unroll
            for (int i = 0; i < kWAhead; i++) wq[i] = *(const lds_u4 *)(size_t)(pl + 16u * (2 * i * kTR));
#pragma unroll
            for (int i = 0; i < 32; i++) {
                const v4u32 wb = wq[i % kWAhead];
                if (i + kWAhead < 32) wq[i % kWAhead] = *(const lds_u4 *)(size_t)(pl + 16u * (2 * (i + kWAhead) * kTR));
                if constexpr (kWD) *reinterpret_cast<uint4 *>(wd + 2 * i * kKC) = make_uint4(wb.x, wb.y, wb.z, wb.w);
#pragma unroll
                for (int t = 0; t < TPW; t++) {
                    acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, xa[i % kAhead][t]),
                                                                     __builtin_bit_cast(bf16x8, wb), acc[t], 0, 0, 0);
                    if (i + kAhead < 32) {
                        xa[i % kAhead][t] = ld_global128(xb[t]);
                        xb[t] += xs;
                    }
                }
                __builtin_amdgcn_sched_barrier(0);   // keeps the loads ahead of their products as written
            }
        };
        PipeSeq p{blockIdx.x, 0, 0, 0, 0, 0, 0};
        uint32_t slot = 0;
        for (bool more = pipe_unit(g, p, n_units); more;) {
#pragma unroll
            for (uint32_t i = 0; i < kPipeMaxSlots; i++)
                if (i == slot) cum[i] += p.nseg;
            uint32_t target = cum[0];
#pragma unroll
            for (uint32_t i = 1; i < kPipeMaxSlots; i++)
                if (i == slot) target = cum[i];
            if (writes_w) run_tile(std::true_type{}, p, slot, target);
            else run_tile(std::false_type{}, p, slot, target);
            const uint32_t rb = p.unit / g.split;
            lds_signal(ctr + 16 + 4 * slot, lane);
            slot = slot + 1 == nslot ? 0 : slot + 1;
            const bool last = p.kt + 1 == p.kt1;
            if (last) {
                // lane holds n = rb*32 + lane%32, b = 32*(m0+t) + 8*blk + 4*(lane/32) + e
                // (addresses formed here, not kept across the tile loop)
                uint32_t ln = lane, nB = g.B, nN = g.N;
                asm volatile("" : "+v"(ln), "+s"(nB), "+s"(nN));
#pragma unroll
                for (int t = 0; t < TPW; t++)
#pragma unroll
                    for (int blk = 0; blk < 4; blk++)
#pragma unroll
                        for (int e = 0; e < 4; e++) {
                            const uint32_t b = (m0 + t) * 32 + 8 * blk + 4 * (ln >> 5) + e;
                            if (b < nB)
                                store_y_at(g, (uint64_t)b * nN + rb * kTR + (ln & 31u),
                                           ok ? acc[t][4 * blk + e] : __builtin_nanf(""), g.split > 1);
                        }
#pragma unroll
                for (int t = 0; t < TPW; t++)
#pragma unroll
                    for (int j = 0; j < 16; j++) acc[t][j] = 0.0f;
            }
            more = pipe_next(g, p, n_units);
        }
        return;
    }

    // ---- decoder wave d of nd
    const uint32_t nd = W - nm, d = wave - nm;
    PipeSeq p{blockIdx.x, 0, 0, 0, 0, 0, 0};
    bool more = pipe_unit(g, p, n_units);
    uint32_t c = 0;        // segments of the sequence before tile p.q
    uint32_t r = d;        // running index of this wave's next segment
    uint32_t slot = 0, use = 0;   // ring slot of tile p.q and its earlier uses
    // Load the next job; false past the sequence.  The loads are issued on
    // every path (a job past the end loads segment 0 and is not decoded) and
    // at clamped addresses, so the number of loads in flight is the same on
    // every path and the decode of the current job waits only for its own.
    auto next_job = [&](PipeJob &j) {
        while (more && r >= c + p.nseg) {
            c += p.nseg;
            more = pipe_next(g, p, n_units);
            if (++slot == nslot) {
                slot = 0;
                use++;
            }
        }
        const bool has = more;
        const uint32_t s = has ? p.first + (r - c) : 0;
        if (has) r += nd;
        j.L = load_segment(g, s, lane);
        j.ts = has ? (uint64_t)p.t * kTile : 0;
        j.q = slot | use << 2;
        const bool valid = has && j.L.g0 >= j.ts && j.L.g1 >= j.L.g0 && j.L.g1 <= j.ts + kTile;
        j.a = valid ? (uint32_t)(j.L.g0 - j.ts) : 0u;
        j.b = valid ? (uint32_t)(j.L.g1 - j.ts) : 0u;
        const uint8_t *smt = g.sm + j.ts;
#pragma unroll
        for (uint32_t k = 0; k < kPipePieces; k++) {
            const uint32_t u = min((j.a >> 3) + lane + 64 * k, kTile / 8 - 1);
            j.sv[k] = *reinterpret_cast<const uint2 *>(smt + 8 * u);
        }
        return has;
    };
    // one merge unit: the high bytes of slots 8u .. 8u + 7 with their
    // sign+mantissa bytes; units shared with a neighbouring segment are
    // written element by element
    auto merge_unit_hi = [&](uint32_t plane, uint32_t u, uint2 sv, uint32_t a, uint32_t b) {
        const uint4 v = merge_hi(ld128(plane + 16 * u), sv);
        if (8 * u >= a && 8 * u + 8 <= b) {
            *(lds_u4 *)(size_t)(plane + 16 * u) = v4u32{v.x, v.y, v.z, v.w};
        } else {
            const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (uint32_t e = 0; e < 8; e++) {
                const uint32_t idx = 8 * u + e;
                if (idx >= a && idx < b) *(lds_u16 *)(size_t)(plane + 2 * idx) = (uint16_t)(wv[e / 2] >> (16 * (e & 1)));
            }
        }
    };
    auto process = [&](const PipeJob &j) {
        // every load of this job is waited for here, so that refilling its
        // buffer afterwards waits for none of the other buffer's loads
#pragma unroll
        for (uint32_t k = 0; k < kPipePieces; k++) asm volatile("" ::"v"(j.sv[k].x), "v"(j.sv[k].y));
        asm volatile("" ::"v"(j.L.own.x), "v"(j.L.own.y), "v"(j.L.own.z), "v"(j.L.own.w), "v"(j.L.next), "v"(j.L.gap),
                     "v"(j.L.count));
        const uint32_t jslot = j.q & 3u, juse = j.q >> 2;
        lds_wait_geq(ctr + 16 + 4 * jslot, juse * nm);
        const uint32_t plane = planes + jslot * kPipePlane;
        // decode: counts, positions, exponents into the high bytes
        const auto win = make_window(j.L.own, j.L.next, j.L.gap);
        uint32_t cnt = j.L.count;
        if (!stored) {
            const uint32_t c0 = lane * kChunkBits;
            const uint32_t end = j.L.nbits > c0 ? min(kChunkBits, j.L.nbits - c0) : 0u;
            cnt = j.L.gap < end ? count_codes<K>(win, fast, chain, j.L.gap, end) : 0u;
        }
        uint32_t total;
        const uint32_t excl = wave_exclusive_scan(cnt, &total);
        if (j.b > j.a && total == j.b - j.a) emit_codes_hi<K>(win, fast, chain, plane / 2 + j.a + excl, cnt);
        wave_lds_sync();
        // merge the segment's units in place: the first 64 * kPipePieces
        // from the bytes loaded ahead, any further ones (segments of more
        // than 4088 elements) loaded here
        const uint32_t u0 = j.a >> 3, u_end = (j.b + 7) >> 3;
#pragma unroll
        for (uint32_t k = 0; k < kPipePieces; k++) {
            const uint32_t u = u0 + lane + 64 * k;
            if (u < u_end) merge_unit_hi(plane, u, j.sv[k], j.a, j.b);
        }
        const uint8_t *smt = g.sm + j.ts;
        for (uint32_t u = u0 + 64 * kPipePieces + lane; u < u_end; u += 64)
            merge_unit_hi(plane, u, *reinterpret_cast<const uint2 *>(smt + 8 * u), j.a, j.b);
        lds_signal(ctr + 4 * jslot, lane);
    };
    // two job buffers in turn: one decoded while the other's loads land
    PipeJob ja, jb;
    bool ha = next_job(ja);
    while (ha) {
        const bool hb = next_job(jb);
        process(ja);
        if (!hb) break;
        ha = next_job(ja);
        process(jb);
    }
}

// Exponent-ring kernel: the pipelined kernel's hand-over with planes that
// hold only the rotated exponents (16 KB per tile instead of a 32 KB BF16
// plane), so that three ring slots and the tables fit in 80 KB and two
// 12-wave workgroups share a CU: 22 decoder waves per CU at one batch tile
// instead of 15.
//   decoder waves: decode each segment of the tile sequence into its slot's
//     exponent plane (count, scan, emit; no sign+mantissa bytes and no
//     merge), then add one to the slot's ready counter.
//   matrix-core waves: KS per batch tile, wave (m, ks) taking k-steps
//     ks * 32 / KS .. (ks + 1) * 32 / KS - 1 of every tile for batch tile m;
//     per k-step, 8 exponent bytes from the plane and the same 8
//     sign+mantissa bytes, loaded from global memory kAhead k-steps ahead
//     with x, give the B operand of v_mfma_f32_32x32x16_bf16 (two
//     bit-selects and two byte permutes per 4 weights).  A wave's loads of
//     a tile form a chain of 32 / KS / kAhead round trips to memory (the
//     sign+mantissa bytes come from HBM), which is what bounds one wave per
//     batch tile; with KS = 2 the second wave of a batch tile hands its
//     partial sums to the first through LDS at the end of each row block
//     (two more counters per batch tile: sums written, sums read), and the
//     first adds them in a fixed order and writes y.
// Waits and counters as in the pipelined kernel above.
constexpr uint32_t kRingSlots = 3;
constexpr uint32_t kRingGuard = 16;   // emit_codes writes from position >= 3

constexpr uint32_t kRingRed = 32 * 32 * 4;   // one batch tile's partial sums (KS = 2)

uint32_t ring_lds_bytes(uint32_t fast_bits, uint32_t n_tables, uint32_t ks)
{
    return kRingGuard + kRingSlots * kTile + 64 + (ks == 2 ? 2 * kRingRed : 0) + (8u << fast_bits) + n_tables * 512u;
}
static_assert(kRingGuard + kRingSlots * kTile < 65536, "ring planes beyond the emit cursor");

template <int K, int MT, int W, int KS>
__global__ void __launch_bounds__(W * 64, 6) decode_gemm_ring_kernel(GemmArgs g)
{
    static_assert(KS == 1 || (KS == 2 && MT <= 2), "k-slices per batch tile");
    extern __shared__ __align__(16) uint8_t lds_raw[];
    const uint32_t lds0 = (uint32_t)(size_t)(lds_u8 *)lds_raw;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lane = lane_id();
    // [guard][3 exponent planes][ready[4], release[4], sums written[2], sums
    // read[2], unused[4]][KS = 2: two batch tiles' partial sums][tables]
    const uint32_t planes = lds0 + kRingGuard;
    const uint32_t ctr = planes + kRingSlots * kTile;
    const uint32_t red = ctr + 64;
    const uint32_t fast = red + (KS == 2 ? 2 * kRingRed : 0);
    const uint32_t chain = fast + (8u << K);
    if (threadIdx.x < 16) st32(ctr + 4 * threadIdx.x, 0u);
    stage_tables<K, W * 64>(fast, chain, g.fast, g.chain, g.n_chain);
    __syncthreads();

    const uint32_t nm = (g.B + 31) / 32 * KS;
    const uint32_t n_units = g.n_rowblocks * g.split;
    const bool stored = g.counts != nullptr;

    if (wave < nm) {
        // ---- matrix-core wave: batch tile m, k-slice ks
        const uint32_t m = wave / KS, ks = wave % KS;
        constexpr int kSteps = 32 / KS;   // k-steps of a tile per wave
        const bool writes_w = g.w_debug && m == 0;
        uint32_t cum[kRingSlots] = {};
        uint32_t nred = 0;   // row blocks whose partial sums were handed over
        bool ok = true;
        f32x16 acc;
#pragma unroll
        for (int j = 0; j < 16; j++) acc[j] = 0.0f;
        // k-step i of a tile: column group c = 2 i + lane / 32, row n_l; its
        // 8 weights sit at tile-order bytes c * 256 + n_l * 8 of the
        // exponent plane and of the tile's sign+mantissa bytes
        auto run_tile = [&](auto wd_tag, const PipeSeq &p, uint32_t sl, uint32_t target) {
            constexpr bool kWD = decltype(wd_tag)::value;
            uint32_t ln = lane;
            asm volatile("" : "+v"(ln));
            constexpr int kAhead = 4;
            const uint32_t kb = ks * kSteps;   // first k-step of this wave in the tile
            const uint32_t brow = min(m * 32 + (ln & 31u), g.B - 1);
            const uint8_t *gx = g.xo ? reinterpret_cast<const uint8_t *>(g.xo + ((uint64_t)(p.kt * 32u + kb) * MT + m) * 64 + ln)
                                     : reinterpret_cast<const uint8_t *>(g.x + (uint64_t)brow * g.K + p.kt * kTC + kb * 16 + (ln >> 5) * 8);
            const __attribute__((address_space(1))) uint8_t *xb = (const __attribute__((address_space(1))) uint8_t *)gx;
            const uint32_t xs = g.xo ? MT * 64u * 16u : 32u;
            const uint32_t lo_off = (ln >> 5) * (kTR * kKC) + (ln & 31u) * kKC + kb * 2 * kTR * kKC;
            const __attribute__((address_space(1))) uint8_t *sb =
                (const __attribute__((address_space(1))) uint8_t *)(g.sm + (uint64_t)p.t * kTile + lo_off);
            uint4 xa[kAhead];
            uint2 sv[kAhead];
#pragma unroll
            for (int i = 0; i < kAhead; i++) {
                xa[i] = ld_global128(xb);
                xb += xs;
                sv[i] = ld_global64(sb);
                sb += 2 * kTR * kKC;
            }
            ok &= lds_wait_geq(ctr + 4 * sl, target);
            const uint32_t rb = p.unit / g.split;
            const uint32_t ep = planes + sl * kTile + lo_off;
            uint16_t *wd = nullptr;
            if constexpr (kWD)
                wd = g.w_debug + (uint64_t)(rb * kTR + (ln & 31u)) * g.K + p.kt * kTC + kb * 16 + (ln >> 5) * kKC;
            constexpr int kEAhead = 2;
            uint2 rq[kEAhead];
#pragma unroll
            for (int i = 0; i < kEAhead; i++) rq[i] = ld64(ep + i * 2 * kTR * kKC);
#pragma unroll
            for (int i = 0; i < kSteps; i++) {
                const uint2 rx = rq[i % kEAhead];
                if (i + kEAhead < kSteps) rq[i % kEAhead] = ld64(ep + (i + kEAhead) * 2 * kTR * kKC);
                const uint2 svi = sv[i % kAhead];
                const uint2 lo = assemble4(svi.x, rx.x), hi = assemble4(svi.y, rx.y);
                if constexpr (kWD) *reinterpret_cast<uint4 *>(wd + 2 * i * kKC) = make_uint4(lo.x, lo.y, hi.x, hi.y);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, xa[i % kAhead]),
                                                              __builtin_bit_cast(bf16x8, v4u32{lo.x, lo.y, hi.x, hi.y}),
                                                              acc, 0, 0, 0);
                if (i + kAhead < kSteps) {
                    xa[i % kAhead] = ld_global128(xb);
                    xb += xs;
                    sv[i % kAhead] = ld_global64(sb);
                    sb += 2 * kTR * kKC;
                }
                __builtin_amdgcn_sched_barrier(0);   // keeps the loads ahead of their products as written
            }
        };
        PipeSeq p{blockIdx.x, 0, 0, 0, 0, 0, 0};
        uint32_t slot = 0;
        for (bool more = pipe_unit(g, p, n_units); more;) {
#pragma unroll
            for (uint32_t i = 0; i < kRingSlots; i++)
                if (i == slot) cum[i] += p.nseg;
            uint32_t target = cum[0];
#pragma unroll
            for (uint32_t i = 1; i < kRingSlots; i++)
                if (i == slot) target = cum[i];
            if (writes_w) run_tile(std::true_type{}, p, slot, target);
            else run_tile(std::false_type{}, p, slot, target);
            const uint32_t rb = p.unit / g.split;
            lds_signal(ctr + 16 + 4 * slot, lane);
            slot = slot + 1 == kRingSlots ? 0 : slot + 1;
            bool store = p.kt + 1 == p.kt1;
            if constexpr (KS == 2) {
                if (store) {
                    // k-slice 1 hands its sums to k-slice 0 (element j of
                    // lane l at float j * 64 + l of the batch tile's area)
                    const uint32_t area = red + m * kRingRed;
                    if (ks == 1) {
                        ok &= lds_wait_geq(ctr + 40 + 4 * m, nred);   // the previous sums were read
#pragma unroll
                        for (int j = 0; j < 16; j++)
                            *(lds_f32 *)(size_t)(area + 4 * (j * 64 + lane)) = ok ? acc[j] : __builtin_nanf("");
                        lds_signal(ctr + 32 + 4 * m, lane);
#pragma unroll
                        for (int j = 0; j < 16; j++) acc[j] = 0.0f;
                        store = false;
                    } else {
                        ok &= lds_wait_geq(ctr + 32 + 4 * m, nred + 1);
#pragma unroll
                        for (int j = 0; j < 16; j++) acc[j] += *(const lds_f32 *)(size_t)(area + 4 * (j * 64 + lane));
                        lds_signal(ctr + 40 + 4 * m, lane);
                    }
                    nred++;
                }
            }
            if (store) {
                // lane holds n = rb*32 + lane%32, b = 32*m + 8*blk + 4*(lane/32) + e
                uint32_t ln = lane, nB = g.B, nN = g.N;
                asm volatile("" : "+v"(ln), "+s"(nB), "+s"(nN));
#pragma unroll
                for (int blk = 0; blk < 4; blk++)
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const uint32_t b = m * 32 + 8 * blk + 4 * (ln >> 5) + e;
                        if (b < nB)
                            store_y_at(g, (uint64_t)b * nN + rb * kTR + (ln & 31u),
                                       ok ? acc[4 * blk + e] : __builtin_nanf(""), g.split > 1);
                    }
#pragma unroll
                for (int j = 0; j < 16; j++) acc[j] = 0.0f;
            }
            more = pipe_next(g, p, n_units);
        }
        return;
    }

    // ---- decoder wave d of nd: segments d, d + nd, ... of the sequence
    const uint32_t nd = W - nm, d = wave - nm;
    PipeSeq p{blockIdx.x, 0, 0, 0, 0, 0, 0};
    bool more = pipe_unit(g, p, n_units);
    uint32_t c = 0;               // segments of the sequence before tile p
    uint32_t r = d;               // running index of this wave's next segment
    uint32_t slot = 0, use = 0;   // ring slot of tile p and its earlier uses
    struct RingJob {
        SegLoad L;
        uint64_t ts;
        uint32_t q;
    };
    // the next job's records and words are loaded before the current job
    // is decoded; a job past the sequence loads segment 0 and is not decoded
    auto next_job = [&](RingJob &j) {
        while (more && r >= c + p.nseg) {
            c += p.nseg;
            more = pipe_next(g, p, n_units);
            if (++slot == kRingSlots) {
                slot = 0;
                use++;
            }
        }
        const bool has = more;
        const uint32_t s = has ? p.first + (r - c) : 0;
        if (has) r += nd;
        j.L = load_segment(g, s, lane);
        j.ts = has ? (uint64_t)p.t * kTile : 0;
        j.q = slot | use << 2;
        return has;
    };
    auto process = [&](const RingJob &j) {
        asm volatile("" ::"v"(j.L.own.x), "v"(j.L.own.y), "v"(j.L.own.z), "v"(j.L.own.w), "v"(j.L.next), "v"(j.L.gap),
                     "v"(j.L.count));
        const uint32_t jslot = j.q & 3u, juse = j.q >> 2;
        lds_wait_geq(ctr + 16 + 4 * jslot, juse * nm);
        decode_into_plane<K>(j.L, j.ts, planes + jslot * kTile, stored, fast, chain, lane);
        lds_signal(ctr + 4 * jslot, lane);
    };
    RingJob ja, jb;
    bool ha = next_job(ja);
    while (ha) {
        const bool hb = next_job(jb);
        process(ja);
        if (!hb) break;
        ha = next_job(ja);
        process(jb);
    }
}

// x [B, K] in the matrix cores' A-operand order: piece (s, m, l) holds the 8
// BF16 of row 32 m + l % 32, columns 16 s + 8 (l / 32) .. + 7 (zero past row
// B), at index (s * tiles + m) * 64 + l, so that the operand of k-step s and
// batch tile m is one contiguous kilobyte.  A workgroup of 256 threads takes
// batch tile m = blockIdx.y and the kXPackSteps k-steps from blockIdx.x *
// kXPackSteps: it reads the 32 rows' pieces of those columns whole (256
// contiguous bytes per row) into LDS, then writes the kXPackSteps packed
// kilobytes.  K is a multiple of 16 * kXPackSteps (the fused layout's
// 512-column tiles).
constexpr uint32_t kXPackSteps = 8;
__global__ void __launch_bounds__(256) x_pack_kernel(const uint16_t *x, uint32_t B, uint32_t K, uint32_t tiles, uint4 *xo)
{
    constexpr uint32_t kPieces = 2 * kXPackSteps;   // 16-byte pieces per row in the block's columns
    __shared__ uint4 buf[32][kPieces + 1];
    const uint32_t m = blockIdx.y, s0 = blockIdx.x * kXPackSteps;
    const uint32_t c0 = s0 * 16;
#pragma unroll
    for (uint32_t j = 0; j < 32 * kPieces / 256; j++) {
        const uint32_t p = threadIdx.x + 256 * j;
        const uint32_t r = p / kPieces, q = p % kPieces;
        const uint32_t row = m * 32 + r;
        buf[r][q] = row < B ? *reinterpret_cast<const uint4 *>(x + (uint64_t)row * K + c0 + q * 8) : make_uint4(0, 0, 0, 0);
    }
    __syncthreads();
#pragma unroll
    for (uint32_t j = 0; j < kXPackSteps * 64 / 256; j++) {
        const uint32_t o = threadIdx.x + 256 * j;
        const uint32_t sl = o / 64, l = o % 64;
        xo[((uint64_t)(s0 + sl) * tiles + m) * 64 + l] = buf[l & 31][2 * sl + (l >> 5)];
    }
}

// batch tiles of the packed x for B rows: the wide kernel's 2, 4 or 8
uint32_t packed_tiles(uint32_t B) { return B <= 64 ? 2 : B <= 128 ? 4 : 8; }

uint64_t packed_bytes(uint32_t K, uint32_t B) { return B <= 32 ? 0 : (uint64_t)(K / 16) * packed_tiles(B) * 64 * 16; }

__global__ void zero_kernel(float4 *p, uint64_t n4)
{
    for (uint64_t i = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x; i < n4; i += (uint64_t)gridDim.x * blockDim.x)
        p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

__global__ void zero_tail_kernel(float *p, uint64_t n)
{
    const uint64_t i = threadIdx.x;
    if (i < n) p[i] = 0.f;
}

// y = 0 (float32) before partial sums are added into it; a fill kernel, not a
// memset, so that the call can be captured in a graph.
void clear_y(const GemmArgs &a, hipStream_t st)
{
    float *y = reinterpret_cast<float *>(a.y);
    const uint64_t n = (uint64_t)a.B * a.N, n4 = n / 4;
    if (n4) hipLaunchKernelGGL(zero_kernel, dim3((uint32_t)std::min<uint64_t>((n4 + 255) / 256, 4096)), dim3(256), 0, st,
                               reinterpret_cast<float4 *>(y), n4);
    if (n & 3) hipLaunchKernelGGL(zero_tail_kernel, dim3(1), dim3(64), 0, st, y + n4 * 4, n & 3);
}

uint32_t gemm_lds_bytes(uint32_t fast_bits, uint32_t n_tables)
{
    return 16 + 2 * kTile + (8u << fast_bits) + n_tables * 512u;
}

int cu_count() { return df11::cu_count(); }

// Row blocks per unit of work: RB (the wide kernel's row-block group) > 1
// divides the unit count.
template <int K, int MT, int W, bool WIDE, int RB = 1>
int launch(GemmArgs a, uint32_t lds, uint32_t forced_split, hipStream_t st)
{
    void (*kern)(GemmArgs) = nullptr;
    if constexpr (WIDE) kern = decode_gemm_wide_kernel<K, MT, RB>;
    else kern = decode_gemm_kernel<K, MT, W>;
    const uint32_t n_groups = (a.n_rowblocks + RB - 1) / RB;
    // resident workgroups per CU, queried once per (device, LDS size)
    static std::mutex mu;
    static int q_dev = -1, q_per_cu = 0;
    static uint32_t q_lds = 0;
    int dev = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = -1;
    {
        std::lock_guard<std::mutex> lk(mu);
        if (q_dev == dev && q_lds == lds) per_cu = q_per_cu;
    }
    if (!per_cu) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, W * 64, lds) != hipSuccess ||
            per_cu < 1)
            per_cu = 1;
        std::lock_guard<std::mutex> lk(mu);
        q_dev = dev;
        q_lds = lds;
        q_per_cu = per_cu;
    }
    const uint32_t slots = (uint32_t)(cu_count() * per_cu);
    // split K when there are too few row blocks to fill every slot
    uint32_t split = 1;
    if (forced_split) split = forced_split;
    else if (2 * n_groups <= slots) split = (slots + n_groups - 1) / n_groups;
    split = std::max(1u, std::min(split, a.tiles_per_row));
    if (a.y_bf16) split = 1;   // one writer per BF16 element (a request for more is refused before)
    a.tiles_per_split = (a.tiles_per_row + split - 1) / split;
    a.split = (a.tiles_per_row + a.tiles_per_split - 1) / a.tiles_per_split;
    if (a.split > 1) clear_y(a, st);
    const uint32_t units = n_groups * a.split;
    const uint32_t groups = std::min<uint32_t>(units, slots);
    hipLaunchKernelGGL(kern, dim3(groups), dim3(W * 64), lds, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return df11::fail(DF11_E_DEVICE, "decode_gemm launch: %s", hipGetErrorString(e));
    return DF11_OK;
}

// Segment-parallel launch (B <= 32 * MT): row blocks split into `parts`
// segment ranges so that every resident workgroup slot has work.
// Per-wave staging of the segment-parallel kernel: a segment's elements, its
// offset inside its first 512-element round and a round of slack.
uint32_t seg_staging_bytes(uint32_t max_seg_elems)
{
    return std::max(4096u, (max_seg_elems + 1024u + 16u + 15u) & ~15u);
}

// The segment-parallel kernel's 8 waves keep their staging in the first
// 64 KB of LDS (the emit loop holds byte addresses in 16 bits) and the
// tables after it within the 160 KB of a CU.
bool seg_kernel_fits(uint32_t fast_bits, uint32_t n_tables, uint32_t max_seg_elems)
{
    const uint32_t stg = seg_staging_bytes(max_seg_elems);
    return 16 + 8 * stg <= 65520 && 16 + 8 * stg + (8u << fast_bits) + n_tables * 512u <= 160u * 1024u;
}

template <int K, int W, int MT>
int launch_seg(GemmArgs a, uint32_t n_tables, uint32_t max_seg_elems, uint32_t forced_parts, hipStream_t st)
{
    static_assert(W == 8, "staging limit computed for 8 waves");
    a.stg_bytes = seg_staging_bytes(max_seg_elems);
    const uint32_t lds = 16 + W * a.stg_bytes + (8u << K) + n_tables * 512u;
    if (!seg_kernel_fits(K, n_tables, max_seg_elems))
        return df11::fail(DF11_E_UNSUPPORTED, "decode_gemm: segment staging and tables do not fit in LDS");
    static std::mutex mu;
    static int q_dev = -1, q_per_cu = 0;
    static uint32_t q_lds = 0;
    int dev = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = -1;
    {
        std::lock_guard<std::mutex> lk(mu);
        if (q_dev == dev && q_lds == lds) per_cu = q_per_cu;
    }
    if (!per_cu) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_gemm_seg_kernel<K, W, MT>, W * 64, lds) != hipSuccess ||
            per_cu < 1)
            per_cu = 1;
        std::lock_guard<std::mutex> lk(mu);
        q_dev = dev;
        q_lds = lds;
        q_per_cu = per_cu;
    }
    const uint32_t slots = (uint32_t)(cu_count() * per_cu);
    const uint64_t segs_per_rb = (a.n_segments + a.n_rowblocks - 1) / a.n_rowblocks;
    // as many parts as fit whole into the resident slots (a second partial
    // wave of workgroups costs more than idle slots: up_proj, 448 row blocks
    // on 512 slots, 44 us in one part, 47 us in two)
    uint32_t parts = 1;
    if (forced_parts) {
        parts = forced_parts;
    } else {
        parts = std::max(1u, slots / a.n_rowblocks);
        // at least one segment per wave
        parts = (uint32_t)std::max<uint64_t>(1, std::min<uint64_t>(parts, segs_per_rb / W));
    }
    if (a.y_bf16) parts = 1;   // one writer per BF16 element
    a.parts = parts;
    if (parts > 1) clear_y(a, st);
    const uint64_t units = (uint64_t)a.n_rowblocks * parts;
    const uint32_t groups = (uint32_t)std::min<uint64_t>(units, 1u << 20);
    hipLaunchKernelGGL((decode_gemm_seg_kernel<K, W, MT>), dim3(groups), dim3(W * 64), lds, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return df11::fail(DF11_E_DEVICE, "decode_gemm launch: %s", hipGetErrorString(e));
    return DF11_OK;
}

// Resident workgroups per CU of `kern` with `lds` bytes of LDS; the last
// answers per (kernel, device, LDS size) are kept so that a sequence of
// calls does not repeat the query.
int resident_groups(const void *kern, uint32_t threads, uint32_t lds)
{
    struct Answer {
        const void *kern;
        int dev;
        uint32_t lds;
        int per_cu;
    };
    static std::mutex mu;
    static Answer kept[16];
    static uint32_t n_kept = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = -1;
    {
        std::lock_guard<std::mutex> lk(mu);
        for (uint32_t i = 0; i < std::min(n_kept, 16u); i++)
            if (kept[i].kern == kern && kept[i].dev == dev && kept[i].lds == lds) return kept[i].per_cu;
    }
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, (int)threads, lds) != hipSuccess || per_cu < 1)
        per_cu = 1;
    std::lock_guard<std::mutex> lk(mu);
    kept[n_kept % 16] = Answer{kern, dev, lds, per_cu};
    n_kept++;
    return per_cu;
}

// Waves per workgroup of the vector kernel for this weight: 12 when their
// staging stays in the first 64 KB of LDS (the emit loop keeps byte
// addresses in 16 bits), else 8; 0 when neither fits (up_proj at 1 row of
// x: 38.3 us with 12-wave groups, two per CU, 43.0 with 8-wave groups,
// three per CU).
uint32_t vec_kernel_waves(uint32_t fast_bits, uint32_t n_tables, uint32_t max_seg_elems)
{
    const uint32_t stg = seg_staging_bytes(max_seg_elems);
    for (uint32_t w : {12u, 8u})
        if (16 + w * stg <= 65520 && 16 + w * stg + (8u << fast_bits) + n_tables * 512u <= 160u * 1024u) return w;
    return 0;
}

template <int K, int W, int NB>
int launch_vec(GemmArgs a, uint32_t n_tables, uint32_t max_seg_elems, uint32_t forced_parts, hipStream_t st)
{
    a.stg_bytes = seg_staging_bytes(max_seg_elems);
    const uint32_t lds = 16 + W * a.stg_bytes + (8u << K) + n_tables * 512u;
    const uint32_t slots =
        (uint32_t)(cu_count() * resident_groups((const void *)decode_gemm_vec_kernel<K, W, NB>, W * 64, lds));
    const uint64_t segs_per_rb = (a.n_segments + a.n_rowblocks - 1) / a.n_rowblocks;
    // as many runs per row block as fit whole into the resident slots, at
    // least one segment per wave (as for the segment-parallel kernel)
    uint32_t parts = forced_parts;
    if (!parts) {
        parts = std::max(1u, slots / a.n_rowblocks);
        parts = (uint32_t)std::max<uint64_t>(1, std::min<uint64_t>(parts, segs_per_rb / W));
    }
    if (a.y_bf16) parts = 1;   // one writer per BF16 element
    a.parts = parts;
    if (parts > 1) clear_y(a, st);
    const uint64_t units = (uint64_t)a.n_rowblocks * parts;
    const uint32_t groups = (uint32_t)std::min<uint64_t>(units, 1u << 20);
    hipLaunchKernelGGL((decode_gemm_vec_kernel<K, W, NB>), dim3(groups), dim3(W * 64), lds, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return df11::fail(DF11_E_DEVICE, "decode_gemm launch: %s", hipGetErrorString(e));
    return DF11_OK;
}

// LDS of the pipelined kernel with nslot tile planes
uint32_t pipe_lds_bytes(uint32_t nslot, uint32_t fast_bits, uint32_t n_tables)
{
    return kPipeGuard + nslot * kPipePlane + 64 + (8u << fast_bits) + n_tables * 512u;
}

// Pipelined launch: as many ring slots (up to 3) as fit beside the tables;
// K split when there are too few row blocks to fill every resident slot.
template <int K, int MT, int TPW>
int launch_pipe(GemmArgs a, uint32_t n_tables, uint32_t forced_split, hipStream_t st)
{
    constexpr int W = 16;   // 1024 threads: the most a workgroup holds
    uint32_t nslot = kPipeMaxSlots;
    while (nslot >= 2 && pipe_lds_bytes(nslot, K, n_tables) > 160u * 1024u) nslot--;
    if (nslot < 2) return df11::fail(DF11_E_UNSUPPORTED, "decode_gemm: pipelined kernel planes and tables do not fit in LDS");
    if (a.xo && a.xo_tiles != (uint32_t)MT) return df11::fail(DF11_E_ARG, "decode_gemm: packed x tiles");
    if (a.n_segments >= (1ull << 32) || (uint64_t)a.n_rowblocks * a.tiles_per_row >= (1ull << 32))
        return df11::fail(DF11_E_UNSUPPORTED, "decode_gemm: the pipelined kernel takes fewer than 2^32 segments and tiles");
    const uint32_t lds = pipe_lds_bytes(nslot, K, n_tables);
    const void *kern = (const void *)decode_gemm_pipe_kernel<K, MT, W, TPW>;
    const uint32_t slots = (uint32_t)(cu_count() * resident_groups(kern, W * 64, lds));
    uint32_t split = 1;
    if (forced_split) split = forced_split;
    else if (2 * a.n_rowblocks <= slots) split = (slots + a.n_rowblocks - 1) / a.n_rowblocks;
    split = std::max(1u, std::min(split, a.tiles_per_row));
    if (a.y_bf16) split = 1;
    a.tiles_per_split = (a.tiles_per_row + split - 1) / split;
    a.split = (a.tiles_per_row + a.tiles_per_split - 1) / a.tiles_per_split;
    if (a.split > 1) clear_y(a, st);
    const uint32_t units = a.n_rowblocks * a.split;
    const uint32_t groups = std::min<uint32_t>(units, slots);
    hipLaunchKernelGGL((decode_gemm_pipe_kernel<K, MT, W, TPW>), dim3(groups), dim3(W * 64), lds, st, a, nslot);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return df11::fail(DF11_E_DEVICE, "decode_gemm launch: %s", hipGetErrorString(e));
    return DF11_OK;
}

// matrix-core waves per batch tile of the exponent-ring kernel: the
// tuning's choice, else by the batch tiles of x
uint32_t ring_k_slices(uint32_t B, uint32_t forced)
{
    // up_proj: 36.5 / 40.9 / 44.8 us at 8 / 32 / 64 rows with two, 56.9 /
    // 59.6 / 50.3 with one (one wave's chain of sign+mantissa and x loads
    // per tile bounds it)
    if (forced) return forced;
    return B <= 64 ? 2u : 1u;
}

// batch tiles per matrix-core wave of the pipelined kernel: the tuning's
// choice, else by the batch tiles of x
uint32_t pipe_tiles_per_wave(uint32_t B, uint32_t forced)
{
    // up_proj, x packed: one tile per wave 63.1 / 69.3 / 75.0 / 95.2 us at
    // 128 / 160 / 192 / 256 rows, two 65.7 / 69.0 / 70.0 / 77.6
    if (forced) return forced;
    return B <= 128 ? 1u : 2u;
}

template <int K, int MT>
int launch_pipe_mt(GemmArgs a, uint32_t n_tables, uint32_t forced_split, uint32_t tpw, hipStream_t st)
{
    if constexpr (MT >= 2)
        if (tpw == 2) return launch_pipe<K, MT, 2>(a, n_tables, forced_split, st);
    return launch_pipe<K, MT, 1>(a, n_tables, forced_split, st);
}

// Exponent-ring launch: 12-wave workgroups, two per CU where the planes
// and tables fit in 80 KB; K split as for the pipelined kernel.
template <int K, int MT, int KS>
int launch_ring(GemmArgs a, uint32_t n_tables, uint32_t forced_split, hipStream_t st)
{
    constexpr int W = 12;
    const uint32_t lds = ring_lds_bytes(K, n_tables, KS);
    if (lds > 160u * 1024u) return df11::fail(DF11_E_UNSUPPORTED, "decode_gemm: exponent-ring planes and tables do not fit in LDS");
    if (a.xo && a.xo_tiles != (uint32_t)MT) return df11::fail(DF11_E_ARG, "decode_gemm: packed x tiles");
    if (a.n_segments >= (1ull << 32) || (uint64_t)a.n_rowblocks * a.tiles_per_row >= (1ull << 32))
        return df11::fail(DF11_E_UNSUPPORTED, "decode_gemm: the exponent-ring kernel takes fewer than 2^32 segments and tiles");
    const void *kern = (const void *)decode_gemm_ring_kernel<K, MT, W, KS>;
    const uint32_t slots = (uint32_t)(cu_count() * resident_groups(kern, W * 64, lds));
    uint32_t split = 1;
    if (forced_split) split = forced_split;
    else if (2 * a.n_rowblocks <= slots) split = (slots + a.n_rowblocks - 1) / a.n_rowblocks;
    split = std::max(1u, std::min(split, a.tiles_per_row));
    if (a.y_bf16) split = 1;
    a.tiles_per_split = (a.tiles_per_row + split - 1) / split;
    a.split = (a.tiles_per_row + a.tiles_per_split - 1) / a.tiles_per_split;
    if (a.split > 1) clear_y(a, st);
    const uint32_t units = a.n_rowblocks * a.split;
    const uint32_t groups = std::min<uint32_t>(units, slots);
    hipLaunchKernelGGL((decode_gemm_ring_kernel<K, MT, W, KS>), dim3(groups), dim3(W * 64), lds, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return df11::fail(DF11_E_DEVICE, "decode_gemm launch: %s", hipGetErrorString(e));
    return DF11_OK;
}

template <int K>
int launch_mt(GemmArgs a, uint32_t n_tables, uint32_t max_seg_elems, const df11_gemm_tuning &tune_in, void *ws,
              hipStream_t st)
{
    // one writer per element of y: no segment runs and no K ranges
    df11_gemm_tuning tune = tune_in;
    if (tune.one_writer) tune.parts = tune.split = 1;
    // Automatic choice: up to 128 rows of x the exponent-ring kernel (two
    // matrix-core waves per batch tile up to 64 rows, one above), above
    // that the pipelined kernel (below).  w_debug calls take the
    // tile-synchronous kernel up to 32 rows, the wide one above.
    const uint32_t mt = (a.B + 31) / 32;
    const uint32_t vec_waves = vec_kernel_waves(K, n_tables, max_seg_elems);
    uint32_t kernel = tune.kernel;
    if (kernel == DF11_GEMM_AUTO) {
        // 1 to 128 rows: the exponent-ring kernel (up_proj, 8 weight copies
        // cycled, two k-slices: 36.0 / 36.4 / 36.5 / 40.9 / 44.5 / 44.8 us
        // at 1 / 2 / 8 / 32 / 33 / 64 rows against 36.3 / 39.3 on the vector
        // kernel at 1 / 2, 42.4 / 48.5 on the segment-parallel one at 8 /
        // 32, 55.8 / 55.6 on the wide one at 33 / 64; one k-slice: 53.1 /
        // 60.3 us at 96 / 128 against 68.6 / 69.4 on the wide kernel), x
        // packed above 32 rows, or read in place up to 64
        if (!a.w_debug && (ws || mt <= 2) && mt <= 4 && ring_lds_bytes(K, n_tables, 2) <= 160u * 1024u)
            kernel = DF11_GEMM_RING;
        // above 128 rows with x packed, the pipelined kernel with two batch
        // tiles per matrix-core wave (69.0 / 70.0 / 77.6 us at 160 / 192 /
        // 256 rows against 94.5 / 95.7 / 96.6 on the wide kernel); with x
        // read in place it is slower than the wide kernel (145 against 97
        // us at 256 rows)
        else if (ws && mt >= 2 && !a.w_debug && pipe_lds_bytes(2, K, n_tables) <= 160u * 1024u)
            kernel = DF11_GEMM_PIPE;
        // where the ring's planes and tables would not fit in LDS: the
        // vector kernel at one or two rows, the segment-parallel one up to
        // 32, the wide one above
        else if (a.B <= 2 && !a.w_debug && vec_waves) kernel = DF11_GEMM_VECTOR;
        else if (a.B <= 32u && !a.w_debug && seg_kernel_fits(K, n_tables, max_seg_elems))
            kernel = DF11_GEMM_SEGMENT;
        else kernel = mt <= 1 ? DF11_GEMM_TILED : DF11_GEMM_WIDE;
    }
    if (kernel == DF11_GEMM_VECTOR) {
        if (a.w_debug || a.B > 2)
            return df11::fail(DF11_E_ARG, "tuning: the vector kernel takes one or two rows of x and no w_debug");
        if (!vec_waves)
            return df11::fail(DF11_E_UNSUPPORTED, "decode_gemm: vector kernel staging and tables do not fit in LDS");
        if (vec_waves == 12)
            return a.B == 1 ? launch_vec<K, 12, 1>(a, n_tables, max_seg_elems, tune.parts, st)
                            : launch_vec<K, 12, 2>(a, n_tables, max_seg_elems, tune.parts, st);
        return a.B == 1 ? launch_vec<K, 8, 1>(a, n_tables, max_seg_elems, tune.parts, st)
                        : launch_vec<K, 8, 2>(a, n_tables, max_seg_elems, tune.parts, st);
    }
    // every kernel but the tile-synchronous one reads x from the packed copy
    // when there is one
    if (ws && mt >= 2 && kernel != DF11_GEMM_TILED) {
        const uint32_t tiles = packed_tiles(a.B);
        if (a.K % (16 * kXPackSteps)) return df11::fail(DF11_E_ARG, "decode_gemm: K %u not a multiple of %u", a.K, 16 * kXPackSteps);
        hipLaunchKernelGGL(x_pack_kernel, dim3(a.K / (16 * kXPackSteps), tiles), dim3(256), 0, st,
                           a.x, a.B, a.K, tiles, reinterpret_cast<uint4 *>(ws));
        a.xo = reinterpret_cast<const uint4 *>(ws);
        a.xo_tiles = tiles;
    }
    if (kernel == DF11_GEMM_RING) {
        const uint32_t kslices = ring_k_slices(a.B, tune.k_slices);
        if (mt <= 1) return kslices == 2 ? launch_ring<K, 1, 2>(a, n_tables, tune.split, st)
                                         : launch_ring<K, 1, 1>(a, n_tables, tune.split, st);
        if (mt <= 2) return kslices == 2 ? launch_ring<K, 2, 2>(a, n_tables, tune.split, st)
                                         : launch_ring<K, 2, 1>(a, n_tables, tune.split, st);
        if (kslices == 2) return df11::fail(DF11_E_ARG, "tuning: two k-slices per batch tile take up to 64 rows of x");
        if (mt <= 4) return launch_ring<K, 4, 1>(a, n_tables, tune.split, st);
        return df11::fail(DF11_E_ARG, "tuning: the exponent-ring kernel takes up to 128 rows of x");
    }
    if (kernel == DF11_GEMM_PIPE) {
        const uint32_t tpw = pipe_tiles_per_wave(a.B, tune.tiles_per_wave);
        if (mt <= 1) return launch_pipe_mt<K, 1>(a, n_tables, tune.split, tpw, st);
        if (mt <= 2) return launch_pipe_mt<K, 2>(a, n_tables, tune.split, tpw, st);
        if (mt <= 4) return launch_pipe_mt<K, 4>(a, n_tables, tune.split, tpw, st);
        return launch_pipe_mt<K, 8>(a, n_tables, tune.split, tpw, st);
    }
    if (kernel == DF11_GEMM_SEGMENT) {
        if (a.w_debug || mt > 2)
            return df11::fail(DF11_E_ARG, "tuning: the segment-parallel kernel takes up to 64 rows of x and no w_debug");
        if (mt <= 1) return launch_seg<K, 8, 1>(a, n_tables, max_seg_elems, tune.parts, st);
        return launch_seg<K, 8, 2>(a, n_tables, max_seg_elems, tune.parts, st);
    }
    constexpr int W = 8;
    const uint32_t lds = gemm_lds_bytes(K, n_tables);
    if (lds > 160u * 1024u) return df11::fail(DF11_E_UNSUPPORTED, "decode_gemm tables do not fit in LDS");
    if (kernel == DF11_GEMM_TILED) {
        if (mt <= 1) return launch<K, 1, W, false>(a, lds, tune.split, st);
        if (mt <= 2) return launch<K, 2, W, false>(a, lds, tune.split, st);
        if (mt <= 4) return launch<K, 4, W, false>(a, lds, tune.split, st);
        return launch<K, 8, W, false>(a, lds, tune.split, st);
    }
    // the wide kernel: a BF16 plane takes the place of the second exponent
    // plane and 16 KB more; above 112 rows of x two row blocks share each x
    // operand (a second exponent plane and BF16 plane; up_proj at 128 / 192
    // / 256 rows: 88.1 / 95.5 / 104.5 us against 92.6 / 113.7 / 141.0 with
    // one, even at 96); with x packed, above 128 rows (packed: 70.6 / 105.8 /
    // 107.3 us with one row block against 69.8 / 95.1 / 95.9 with two)
    if (mt < 2) return df11::fail(DF11_E_ARG, "tuning: the wide kernel takes more than 32 rows of x");
    const uint32_t lds_wide = lds + kTile, lds_wide2 = lds_wide + 3 * kTile;
    if (lds_wide > 160u * 1024u) {
        if (tune.kernel == DF11_GEMM_WIDE) return df11::fail(DF11_E_UNSUPPORTED, "decode_gemm: wide kernel planes do not fit in LDS");
        if (mt <= 2) return launch<K, 2, W, false>(a, lds, tune.split, st);
        if (mt <= 4) return launch<K, 4, W, false>(a, lds, tune.split, st);
        return launch<K, 8, W, false>(a, lds, tune.split, st);
    }
    const bool fits2 = lds_wide2 <= 160u * 1024u;
    if (tune.row_blocks == 2 && !fits2)
        return df11::fail(DF11_E_UNSUPPORTED, "decode_gemm: two row blocks' planes do not fit in LDS");
    const bool two = tune.row_blocks ? tune.row_blocks == 2 : fits2 && a.B > (a.xo ? 128u : 112u);
    if (mt <= 2) return two ? launch<K, 2, 16, true, 2>(a, lds_wide2, tune.split, st)
                            : launch<K, 2, W, true>(a, lds_wide, tune.split, st);
    if (mt <= 4) return two ? launch<K, 4, 16, true, 2>(a, lds_wide2, tune.split, st)
                            : launch<K, 4, W, true>(a, lds_wide, tune.split, st);
    return two ? launch<K, 8, 16, true, 2>(a, lds_wide2, tune.split, st)
               : launch<K, 8, W, true>(a, lds_wide, tune.split, st);
}

int check_gemm_tuning(const df11_gemm_tuning &t, bool bf16_y)
{
    if (t.kernel > DF11_GEMM_RING) return df11::fail(DF11_E_ARG, "tuning: kernel %u", t.kernel);
    if (t.row_blocks > 2 || (t.row_blocks && t.kernel != DF11_GEMM_WIDE))
        return df11::fail(DF11_E_ARG, "tuning: row_blocks %u (0, or 1 or 2 with the wide kernel)", t.row_blocks);
    if (t.parts && t.kernel != DF11_GEMM_SEGMENT && t.kernel != DF11_GEMM_VECTOR)
        return df11::fail(DF11_E_ARG, "tuning: parts applies to the segment-parallel and vector kernels");
    if (t.split && t.kernel != DF11_GEMM_WIDE && t.kernel != DF11_GEMM_TILED && t.kernel != DF11_GEMM_PIPE &&
        t.kernel != DF11_GEMM_RING)
        return df11::fail(DF11_E_ARG, "tuning: split applies to the wide, tile-synchronous and pipelined kernels");
    if (bf16_y && (t.parts > 1 || t.split > 1))
        return df11::fail(DF11_E_ARG, "tuning: a BF16 y has one writer per element (parts and split 1)");
    if (t.one_writer && (t.parts > 1 || t.split > 1))
        return df11::fail(DF11_E_ARG, "tuning: one_writer takes parts and split 1");
    if (t.parts > (1u << 16) || t.split > (1u << 16)) return df11::fail(DF11_E_ARG, "tuning: parts or split too large");
    if (t.k_slices && (t.kernel != DF11_GEMM_RING || t.k_slices > 2))
        return df11::fail(DF11_E_ARG, "tuning: k_slices %u (0, or 1 or 2 with the exponent-ring kernel)", t.k_slices);
    if (t.tiles_per_wave && (t.kernel != DF11_GEMM_PIPE || t.tiles_per_wave > 2))
        return df11::fail(DF11_E_ARG, "tuning: tiles_per_wave %u (0, or 1 or 2 with the pipelined kernel)", t.tiles_per_wave);
    return DF11_OK;
}

// Scratch of df11_decode_gemm_noalloc: the packed x of callers that cannot
// allocate, one copy per device (each device that loads the library holds it
// until the process ends), shared by every such call on that device.
constexpr uint64_t kScratchBytes = 16ull << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// Device address of this device's copy of `scratch`, looked up once per
// device with the device current.  The array's name in host code is only a
// stand-in for the symbol; kernels get this address.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

int scratch_address(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return df11::fail(DF11_E_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return df11::fail(DF11_E_UNSUPPORTED, "device %d: scratch kept for %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return df11::fail(DF11_E_DEVICE, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return DF11_OK;
}

}  // namespace

extern "C" int df11_decode_gemm(const df11_view *w, const uint16_t *x, uint32_t B, float *y,
                                uint16_t *w_debug, void *stream)
{
    return df11_decode_gemm_out(w, x, B, y, DF11_Y_F32, w_debug, stream);
}

extern "C" int df11_decode_gemm_out(const df11_view *w, const uint16_t *x, uint32_t B, void *y, int y_dtype,
                                    uint16_t *w_debug, void *stream)
{
    return df11_decode_gemm_ex(w, x, B, y, y_dtype, w_debug, nullptr, nullptr, 0, stream);
}

extern "C" uint64_t df11_decode_gemm_workspace_bytes(const df11_view *w, uint32_t B)
{
    if (!w || w->tile_rows != kTR || w->tile_cols != kTC || w->tile_kchunk != kKC || !w->cols || w->cols % kTC ||
        w->cols > 0xFFFFFFFFull || B > 256)
        return 0;
    return packed_bytes((uint32_t)w->cols, B);
}

extern "C" int df11_decode_gemm_ex(const df11_view *w, const uint16_t *x, uint32_t B, void *y, int y_dtype,
                                   uint16_t *w_debug, const df11_gemm_tuning *tuning, void *workspace,
                                   uint64_t workspace_bytes, void *stream)
{
    if (y_dtype != DF11_Y_F32 && y_dtype != DF11_Y_BF16)
        return df11::fail(DF11_E_ARG, "df11_decode_gemm_out: unknown y_dtype %d", y_dtype);
    const df11_gemm_tuning tune = tuning ? *tuning : df11_gemm_tuning{};
    int rc = check_gemm_tuning(tune, y_dtype == DF11_Y_BF16);
    if (rc) return rc;
    if (!w || !x || !y) return df11::fail(DF11_E_ARG, "df11_decode_gemm: null pointer");
    if (B < 1 || B > 256) return df11::fail(DF11_E_ARG, "B = %u outside 1..256", B);
    if (tune.kernel == DF11_GEMM_RING && B > 128)
        return df11::fail(DF11_E_ARG, "tuning: the exponent-ring kernel takes up to 128 rows of x");
    if (tune.kernel == DF11_GEMM_RING && tune.k_slices == 2 && B > 64)
        return df11::fail(DF11_E_ARG, "tuning: two k-slices per batch tile take up to 64 rows of x");
    if (w->tile_rows != kTR || w->tile_cols != kTC || w->tile_kchunk != kKC || w->align_elems != kTile ||
        w->chunk_bytes != 16 || w->seg_lanes != 64 || !w->rows || !w->cols || w->rows % kTR ||
        w->cols % kTC || w->rows * w->cols != w->n)
        return df11::fail(DF11_E_ARG, "weight was not encoded with df11_gemm_layout");
    if (w->rows > 0xFFFFFFFFull || w->cols > 0xFFFFFFFFull)
        return df11::fail(DF11_E_ARG, "weight too large");
    const uint64_t nb = w->n / kTile;
    if (w->n_block_seg != nb + 1 || !w->block_seg || w->n_segs != w->n_segments + 1 ||
        w->n_gaps != w->n_segments * 64 || (w->n_counts && (w->n_counts != w->n_segments * 64 || !w->counts)) || w->n_exp_words < w->n_segments * kSegWords + 2 || w->n_sm < w->n)
        return df11::fail(DF11_E_ARG, "view array sizes inconsistent");
    if (w->fast_bits < DF11_FAST_BITS_MIN || w->fast_bits > DF11_FAST_BITS_MAX || w->n_tables < 1 ||
        w->n_tables > DF11_MAX_TABLES || w->n_chain != (uint64_t)w->n_tables * 256 || w->n_fast != (2ull << w->fast_bits))
        return df11::fail(DF11_E_ARG, "table sizes inconsistent");
    // staging is sized from max_seg_elems; a segment of 64 16-byte chunks
    // holds at most 8192 / min_len codes
    if (w->min_len < 1 || w->min_len > w->max_len || w->max_len > DF11_MAX_LEN || !w->max_seg_elems ||
        w->max_seg_elems > (8192u + w->min_len - 1) / w->min_len)
        return df11::fail(DF11_E_ARG, "view: code lengths %u..%u or max_seg_elems %u out of range", w->min_len, w->max_len,
                          w->max_seg_elems);
    if (!w->exp_words || !w->sm || !w->gaps || !w->segs || !w->chain || !w->fast)
        return df11::fail(DF11_E_ARG, "null array in view");
    if (((uintptr_t)x & 15) || ((uintptr_t)y & 15) || ((uintptr_t)w_debug & 15) || ((uintptr_t)w->sm & 15) ||
        ((uintptr_t)w->exp_words & 15) || ((uintptr_t)w->fast & 15) || ((uintptr_t)w->chain & 15))
        return df11::fail(DF11_E_ARG, "x, y, w_debug and the view arrays must be 16-byte aligned");
    if (workspace && (((uintptr_t)workspace & 255) || workspace_bytes < packed_bytes((uint32_t)w->cols, B)))
        return df11::fail(DF11_E_ARG, "workspace: %llu bytes at %p; need %llu, 256-byte aligned",
                          (unsigned long long)workspace_bytes, workspace,
                          (unsigned long long)packed_bytes((uint32_t)w->cols, B));
    GemmArgs a{};
    a.words = w->exp_words;
    a.sm = w->sm;
    a.gaps = w->gaps;
    a.counts = w->n_counts ? w->counts : nullptr;   // no counts: the decode runs the locate pass
    a.segs = w->segs;
    a.block_seg = w->block_seg;
    a.chain = w->chain;
    a.fast = w->fast;
    a.x = x;
    a.y = y;
    a.y_bf16 = y_dtype == DF11_Y_BF16;
    a.w_debug = w_debug;
    a.n_chain = (uint32_t)w->n_chain;
    a.N = (uint32_t)w->rows;
    a.K = (uint32_t)w->cols;
    a.B = B;
    a.tiles_per_row = a.K / kTC;
    a.n_rowblocks = a.N / kTR;
    a.n_segments = w->n_segments;
    hipStream_t st = (hipStream_t)stream;
    switch (w->fast_bits) {
    case 8: return launch_mt<8>(a, w->n_tables, w->max_seg_elems, tune, workspace, st);
    case 9: return launch_mt<9>(a, w->n_tables, w->max_seg_elems, tune, workspace, st);
    case 10: return launch_mt<10>(a, w->n_tables, w->max_seg_elems, tune, workspace, st);
    case 11: return launch_mt<11>(a, w->n_tables, w->max_seg_elems, tune, workspace, st);
    default: return launch_mt<12>(a, w->n_tables, w->max_seg_elems, tune, workspace, st);
    }
}

extern "C" int df11_decode_gemm_noalloc(const df11_view *w, const uint16_t *x, uint32_t B, void *y, int y_dtype,
                                        uint16_t *w_debug, const df11_gemm_tuning *tuning, void *stream)
{
    const uint64_t need = df11_decode_gemm_workspace_bytes(w, B);
    if (need > kScratchBytes)
        return df11::fail(DF11_E_UNSUPPORTED,
                          "df11_decode_gemm_noalloc: %llu bytes of packed x for B = %u and K = %llu; the library's "
                          "scratch holds %llu",
                          (unsigned long long)need, B, (unsigned long long)w->cols, (unsigned long long)kScratchBytes);
    void *ws = nullptr;
    if (need) {
        int rc = scratch_address(&ws);
        if (rc) return rc;
    }
    return df11_decode_gemm_ex(w, x, B, y, y_dtype, w_debug, tuning, ws, ws ? kScratchBytes : 0, stream);
}
