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
// Layout: W [N, K] is encoded in tile order with 32 x 512 tiles, each tile
// starting a new segment (df11_gemm_layout), so the segments of one tile are
// block_seg[t] .. block_seg[t+1].  A workgroup owns a block of 32 weight rows
// (32 output features) and walks its K / 512 tiles:
//   decode  the waves take the tile's segments, each decoded by one wavefront
//           exactly as in df11_decode, writing rotated exponents into a
//           16 KiB LDS plane at the element's offset in the tile;
//   merge   all threads join exponents with the sign+mantissa bytes into a
//           32 KiB BF16 tile in LDS, 16-byte chunks XOR-swizzled by row so
//           that the matrix-core operand reads are bank-conflict free;
//   mfma    v_mfma_f32_32x32x16_bf16 with A = x rows (the batch, from
//           global memory / L2) and B = the decoded tile, float32 accumulate.
// The next tile's decode overlaps other waves' matrix work; the barrier after
// each decode also separates one tile's matrix reads from the next merge.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>

#include "df11_device.h"
#include "df11_internal.h"

using namespace df11dev;

namespace {

constexpr uint32_t kTR = 32, kTC = 512, kTile = kTR * kTC;
constexpr uint32_t kChunkBits = 128;
constexpr uint32_t kSegWords = 256;
constexpr uint32_t kPlaneBytes = kTile + 16;       // exponent plane (+ spare)
constexpr uint32_t kBfBytes = kTile * 2;           // BF16 tile

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

struct GemmArgs {
    const uint32_t *words;
    const uint8_t *sm;
    const uint8_t *gaps;
    const df11_segment *segs;
    const uint64_t *block_seg;
    const uint16_t *chain;
    const uint32_t *fast;
    const uint16_t *x;       // [B, K] bf16
    float *y;                // [B, N]
    uint16_t *w_debug;       // [N, K] or null
    uint32_t n_chain;
    uint32_t N, K, B;
    uint32_t tiles_per_row;  // K / 512
    uint32_t n_rowblocks;    // N / 32
    uint64_t n_segments;
};

// Decode one segment of tile-aligned stream into the exponent plane.
template <int K>
__device__ __forceinline__ void decode_segment_to_plane(const GemmArgs &g, uint64_t s, uint64_t tile_start,
                                                        uint32_t plane, uint32_t fast, uint32_t chain,
                                                        uint32_t lane)
{
    const uint32_t *w = g.words + s * kSegWords + lane * 4;
    const uint4 own = *reinterpret_cast<const uint4 *>(w);
    const uint32_t next = w[4];
    const uint32_t gap = g.gaps[s * 64 + lane];
    const uint64_t g0 = g.segs[s].elem_off, g1 = g.segs[s + 1].elem_off;
    const uint32_t nbits = g.segs[s].nbits;
    if (g0 >= tile_start && g1 >= g0 && g1 <= tile_start + kTile) {
        const uint32_t c0 = lane * kChunkBits;
        const uint32_t end = nbits > c0 ? min(kChunkBits, nbits - c0) : 0u;
        const Window win = make_window(own, next, gap);
        const uint32_t cnt = gap < end ? count_codes<K>(win, fast, chain, gap, end) : 0u;
        uint32_t total;
        const uint32_t excl = wave_exclusive_scan(cnt, &total);
        if (total == (uint32_t)(g1 - g0))
            emit_codes<K>(win, fast, chain, plane + (uint32_t)(g0 - tile_start) + excl, cnt);
    }
}

// BF16 tile address of the 16-byte chunk `c` (8 columns) of tile row r.
__device__ __forceinline__ uint32_t bf_chunk(uint32_t bf, uint32_t r, uint32_t c)
{
    return bf + r * (kTC * 2) + ((c ^ r) << 4);
}

// MT: 32-row tiles of the batch (B <= 32 * MT).  WAVES: waves per workgroup.
// Wave w works on batch tiles m = w % MT (+ WAVES, ... when MT > WAVES) and on
// k-steps ks = w / MT (mod WAVES / MT) of every tile.
template <int K, int MT, int WAVES>
__global__ void __launch_bounds__(WAVES * 64)
decode_gemm_kernel(GemmArgs g)
{
    constexpr int kMPerWave = MT > WAVES ? MT / WAVES : 1;
    constexpr int kKSlices = MT >= WAVES ? 1 : WAVES / MT;
    extern __shared__ __align__(16) uint8_t lds_raw[];
    const uint32_t lds0 = (uint32_t)(size_t)(lds_u8 *)lds_raw;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lane = lane_id();
    const uint32_t plane = lds0 + 16;
    const uint32_t bf = lds0 + 16 + kPlaneBytes;
    const uint32_t fast = bf + kBfBytes;
    const uint32_t chain = fast + (8u << K);

    for (uint32_t i = threadIdx.x; i < (2u << K); i += blockDim.x) st32(fast + 4 * i, g.fast[i]);
    for (uint32_t i = threadIdx.x; i < g.n_chain; i += blockDim.x)
        *(lds_u16 *)(size_t)(chain + 2 * i) = g.chain[i];
    __syncthreads();

    const uint32_t kslice = kKSlices > 1 ? wave / MT : 0;
    const uint32_t m_first = kKSlices > 1 ? wave % MT : wave;

    for (uint32_t rb = blockIdx.x; rb < g.n_rowblocks; rb += gridDim.x) {
        f32x16 acc[kMPerWave];
#pragma unroll
        for (int m = 0; m < kMPerWave; m++)
            for (int j = 0; j < 16; j++) acc[m][j] = 0.0f;

        for (uint32_t kt = 0; kt < g.tiles_per_row; kt++) {
            const uint64_t t = (uint64_t)rb * g.tiles_per_row + kt;
            const uint64_t tile_start = t * kTile;
            // decode the tile's segments (one wave per segment)
            const uint64_t s0 = g.block_seg[t], s1 = min(g.block_seg[t + 1], g.n_segments);
            for (uint64_t s = s0 + wave; s < s1; s += WAVES)
                decode_segment_to_plane<K>(g, s, tile_start, plane, fast, chain, lane);
            __syncthreads();

            // merge exponents and sign+mantissa bytes into the swizzled BF16 tile
            for (uint32_t q = threadIdx.x; q < kTile / 16; q += WAVES * 64) {
                const uint32_t r = q >> 5, c = (q & 31) * 2;
                const uint4 smv = *reinterpret_cast<const uint4 *>(g.sm + tile_start + 16ull * q);
                const uint4 rx = ld128(plane + 16 * q);
                const uint2 a = assemble4(smv.x, rx.x), b = assemble4(smv.y, rx.y);
                const uint2 cc = assemble4(smv.z, rx.z), d = assemble4(smv.w, rx.w);
                *(lds_u4 *)(size_t)bf_chunk(bf, r, c) = v4u32{a.x, a.y, b.x, b.y};
                *(lds_u4 *)(size_t)bf_chunk(bf, r, c + 1) = v4u32{cc.x, cc.y, d.x, d.y};
                if (g.w_debug) {
                    uint4 *dst = reinterpret_cast<uint4 *>(g.w_debug + (uint64_t)(rb * kTR + r) * g.K + kt * kTC + c * 8);
                    dst[0] = make_uint4(a.x, a.y, b.x, b.y);
                    dst[1] = make_uint4(cc.x, cc.y, d.x, d.y);
                }
            }
            __syncthreads();

            // matrix cores: acc[m] += x[m-tile, k-step] * tile^T
            const uint32_t n_l = lane & 31, khalf = lane >> 5;
            for (uint32_t ks = kslice; ks < kTC / 16; ks += kKSlices) {
                const v4u32 wb = *(const lds_u4 *)(size_t)bf_chunk(bf, n_l, 2 * ks + khalf);
                const bf16x8 bop = __builtin_bit_cast(bf16x8, wb);
#pragma unroll
                for (int m = 0; m < kMPerWave; m++) {
                    const uint32_t brow = (m_first + m * WAVES) * 32 + n_l;
                    uint4 xa = make_uint4(0, 0, 0, 0);
                    if (brow < g.B)
                        xa = *reinterpret_cast<const uint4 *>(g.x + (uint64_t)brow * g.K + kt * kTC + ks * 16 + khalf * 8);
                    const bf16x8 aop = __builtin_bit_cast(bf16x8, xa);
                    acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, bop, acc[m], 0, 0, 0);
                }
            }
        }
        // reduce the k-slices through LDS (the BF16 tile is free after this barrier)
        if (kKSlices > 1) {
            __syncthreads();
            float *red = (float *)lds_raw + (bf - lds0) / 4;
            if (kslice > 0)
                for (int j = 0; j < 16; j++) red[((kslice - 1) * MT + m_first) * 1024 + j * 64 + lane] = acc[0][j];
            __syncthreads();
            if (kslice == 0)
                for (uint32_t ksl = 1; ksl < (uint32_t)kKSlices; ksl++)
                    for (int j = 0; j < 16; j++) acc[0][j] += red[((ksl - 1) * MT + m_first) * 1024 + j * 64 + lane];
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
                        const uint32_t b = mt * 32 + 8 * blk + 4 * (lane >> 5) + e;
                        if (b < g.B) g.y[(uint64_t)b * g.N + rb * kTR + (lane & 31)] = acc[m][4 * blk + e];
                    }
            }
        }
        __syncthreads();   // the reduction buffer and planes are reused by the next row block
    }
}

uint32_t gemm_lds_bytes(uint32_t fast_bits, uint32_t n_tables)
{
    return 16 + kPlaneBytes + kBfBytes + (8u << fast_bits) + n_tables * 512u;
}

int cu_count()
{
    static int cus = 0;
    if (!cus) {
        int dev = 0;
        hipDeviceProp_t p;
        if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&p, dev) != hipSuccess) return 256;
        cus = p.multiProcessorCount;
    }
    return cus;
}

template <int K, int MT, int W>
int launch(const GemmArgs &a, uint32_t lds, hipStream_t st)
{
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_gemm_kernel<K, MT, W>, W * 64, lds) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    const uint32_t groups = std::min<uint32_t>(a.n_rowblocks, (uint32_t)(cu_count() * per_cu));
    hipLaunchKernelGGL((decode_gemm_kernel<K, MT, W>), dim3(groups), dim3(W * 64), lds, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return df11::fail(DF11_E_DEVICE, "decode_gemm launch: %s", hipGetErrorString(e));
    return DF11_OK;
}

template <int K>
int launch_mt(const GemmArgs &a, uint32_t n_tables, hipStream_t st)
{
    constexpr int W = 8;
    const uint32_t lds = gemm_lds_bytes(K, n_tables);
    if (lds > 160u * 1024u) return df11::fail(DF11_E_UNSUPPORTED, "decode_gemm tables do not fit in LDS");
    const uint32_t mt = (a.B + 31) / 32;
    if (mt <= 1) return launch<K, 1, W>(a, lds, st);
    if (mt <= 2) return launch<K, 2, W>(a, lds, st);
    if (mt <= 4) return launch<K, 4, W>(a, lds, st);
    return launch<K, 8, W>(a, lds, st);
}

}  // namespace

extern "C" int df11_decode_gemm(const df11_view *w, const uint16_t *x, uint32_t B, float *y,
                                uint16_t *w_debug, void *stream)
{
    if (!w || !x || !y) return df11::fail(DF11_E_ARG, "df11_decode_gemm: null pointer");
    if (B < 1 || B > 256) return df11::fail(DF11_E_ARG, "B = %u outside 1..256", B);
    if (w->tile_rows != kTR || w->tile_cols != kTC || w->align_elems != kTile || w->chunk_bytes != 16 ||
        w->seg_lanes != 64 || !w->rows || !w->cols || w->rows % kTR || w->cols % kTC ||
        w->rows * w->cols != w->n)
        return df11::fail(DF11_E_ARG, "weight was not encoded with df11_gemm_layout");
    if (w->rows > 0xFFFFFFFFull || w->cols > 0xFFFFFFFFull)
        return df11::fail(DF11_E_ARG, "weight too large");
    const uint64_t nb = w->n / kTile;
    if (w->n_block_seg != nb + 1 || !w->block_seg || w->n_segs != w->n_segments + 1 ||
        w->n_gaps != w->n_segments * 64 || w->n_exp_words < w->n_segments * kSegWords + 2 || w->n_sm < w->n)
        return df11::fail(DF11_E_ARG, "view array sizes inconsistent");
    if (w->fast_bits < DF11_FAST_BITS_MIN || w->fast_bits > DF11_FAST_BITS_MAX || w->n_tables < 1 ||
        w->n_tables > DF11_MAX_TABLES || w->n_chain != (uint64_t)w->n_tables * 256 || w->n_fast != (2ull << w->fast_bits))
        return df11::fail(DF11_E_ARG, "table sizes inconsistent");
    if (((uintptr_t)x & 15) || ((uintptr_t)y & 3) || ((uintptr_t)w_debug & 15) || ((uintptr_t)w->sm & 15) ||
        ((uintptr_t)w->exp_words & 15))
        return df11::fail(DF11_E_ARG, "x, w_debug and the view arrays must be 16-byte aligned");
    GemmArgs a{};
    a.words = w->exp_words;
    a.sm = w->sm;
    a.gaps = w->gaps;
    a.segs = w->segs;
    a.block_seg = w->block_seg;
    a.chain = w->chain;
    a.fast = w->fast;
    a.x = x;
    a.y = y;
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
    case 8: return launch_mt<8>(a, w->n_tables, st);
    case 9: return launch_mt<9>(a, w->n_tables, st);
    case 10: return launch_mt<10>(a, w->n_tables, st);
    case 11: return launch_mt<11>(a, w->n_tables, st);
    default: return launch_mt<12>(a, w->n_tables, st);
    }
}
