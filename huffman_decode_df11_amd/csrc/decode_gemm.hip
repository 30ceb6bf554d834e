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
// Three kernels, chosen by the rows of x (B):
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
        const Window win = make_window(L.own, L.next, L.gap);
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
    const Window win = make_window(L.own, L.next, L.gap);
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
int launch(GemmArgs a, uint32_t lds, hipStream_t st)
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
    if (const char *e = getenv("DF11_GEMM_SPLIT")) split = (uint32_t)atoi(e);
    else if (2 * n_groups <= slots) split = (slots + n_groups - 1) / n_groups;
    split = std::max(1u, std::min(split, a.tiles_per_row));
    if (a.y_bf16) split = 1;   // one writer per BF16 element
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
template <int K, int W, int MT>
int launch_seg(GemmArgs a, uint32_t n_tables, uint32_t max_seg_elems, hipStream_t st)
{
    a.stg_bytes = std::max(4096u, (max_seg_elems + 1024u + 16u + 15u) & ~15u);
    const uint32_t lds = 16 + W * a.stg_bytes + (8u << K) + n_tables * 512u;
    if (lds > 160u * 1024u) return df11::fail(DF11_E_UNSUPPORTED, "decode_gemm staging and tables do not fit in LDS");
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
    if (const char *e = getenv("DF11_GEMM_PARTS")) parts = (uint32_t)atoi(e);
    else parts = std::max(1u, slots / a.n_rowblocks);
    // at least one segment per wave
    parts = (uint32_t)std::max<uint64_t>(1, std::min<uint64_t>(parts, segs_per_rb / W));
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

template <int K>
int launch_mt(const GemmArgs &a, uint32_t n_tables, uint32_t max_seg_elems, hipStream_t st)
{
    // the tile-synchronous kernel also serves the w_debug output
    // segment-parallel up to 40 rows of x (one batch tile to 32, two above);
    // from 41 rows the wide kernel is faster (up_proj: 58.5 against 60.7 us
    // at 33 rows, 66.8 against 64.9 at 48, 76.4 against 67.7 at 64)
    if (a.B <= 40 && !a.w_debug && !getenv("DF11_GEMM_TILED")) {
        if (a.B <= 32) return launch_seg<K, 8, 1>(a, n_tables, max_seg_elems, st);
        return launch_seg<K, 8, 2>(a, n_tables, max_seg_elems, st);
    }
    constexpr int W = 8;
    const uint32_t lds = gemm_lds_bytes(K, n_tables);
    if (lds > 160u * 1024u) return df11::fail(DF11_E_UNSUPPORTED, "decode_gemm tables do not fit in LDS");
    const uint32_t mt = (a.B + 31) / 32;
    if (mt <= 1) return launch<K, 1, W, false>(a, lds, st);
    // two or more batch tiles: the kernel with the shared BF16 plane (which
    // takes the place of the second exponent plane and 16 KB more);
    // DF11_GEMM_NARROW selects the tile-synchronous kernel instead
    const uint32_t lds_wide = lds + kTile;
    const bool wide = lds_wide <= 160u * 1024u && !getenv("DF11_GEMM_NARROW");
    // above 112 rows of x two row blocks share each x operand (a second
    // exponent plane and BF16 plane; up_proj at 128 / 192 / 256 rows: 88.1 /
    // 95.5 / 104.5 us against 92.6 / 113.7 / 141.0 with one, even at 96);
    // DF11_GEMM_RB = 1 or 2 overrides
    const uint32_t lds_wide2 = lds_wide + 3 * kTile;
    const char *rbe = getenv("DF11_GEMM_RB");
    const bool two = wide && lds_wide2 <= 160u * 1024u && (rbe ? atoi(rbe) == 2 : a.B > 112);
    if (mt <= 2) return two ? launch<K, 2, 16, true, 2>(a, lds_wide2, st)
                            : wide ? launch<K, 2, W, true>(a, lds_wide, st) : launch<K, 2, W, false>(a, lds, st);
    if (mt <= 4) return two ? launch<K, 4, 16, true, 2>(a, lds_wide2, st)
                            : wide ? launch<K, 4, W, true>(a, lds_wide, st) : launch<K, 4, W, false>(a, lds, st);
    return two ? launch<K, 8, 16, true, 2>(a, lds_wide2, st)
               : wide ? launch<K, 8, W, true>(a, lds_wide, st) : launch<K, 8, W, false>(a, lds, st);
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
    if (y_dtype != DF11_Y_F32 && y_dtype != DF11_Y_BF16)
        return df11::fail(DF11_E_ARG, "df11_decode_gemm_out: unknown y_dtype %d", y_dtype);
    if (!w || !x || !y) return df11::fail(DF11_E_ARG, "df11_decode_gemm: null pointer");
    if (B < 1 || B > 256) return df11::fail(DF11_E_ARG, "B = %u outside 1..256", B);
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
    if (((uintptr_t)x & 15) || ((uintptr_t)y & 15) || ((uintptr_t)w_debug & 15) || ((uintptr_t)w->sm & 15) ||
        ((uintptr_t)w->exp_words & 15) || ((uintptr_t)w->fast & 15) || ((uintptr_t)w->chain & 15))
        return df11::fail(DF11_E_ARG, "x, y, w_debug and the view arrays must be 16-byte aligned");
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
    case 8: return launch_mt<8>(a, w->n_tables, w->max_seg_elems, st);
    case 9: return launch_mt<9>(a, w->n_tables, w->max_seg_elems, st);
    case 10: return launch_mt<10>(a, w->n_tables, w->max_seg_elems, st);
    case 11: return launch_mt<11>(a, w->n_tables, w->max_seg_elems, st);
    default: return launch_mt<12>(a, w->n_tables, w->max_seg_elems, st);
    }
}
