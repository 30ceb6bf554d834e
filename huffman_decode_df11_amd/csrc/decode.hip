// df11_decode / df11_decode_batch: restore BF16 weights from the DFloat11
// stream on the GPU, right before the matmul that consumes them.
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
// workgroup of WAVES waves stages the tables in LDS once and then loops over
// segments.  Exponents are staged in LDS and merged with the sign+mantissa
// bytes in 16-element groups: 16-byte loads of sm, 32-byte BF16 stores.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>

#include "df11_device.h"
#include "df11_internal.h"

using namespace df11dev;

namespace {

struct ViewArgs {
    const uint32_t *words;
    const uint8_t *sm;
    const uint8_t *gaps;
    const df11_segment *segs;
    uint16_t *out;
    uint64_t n;
    uint64_t n_segments;
    uint64_t seg_begin;       // first global segment id of this view (batch launches)
    // tile order (tr == 0: row-major)
    uint32_t tr, tc, tiles_per_row, pad;
    uint64_t cols;
};

struct TableArgs {
    const uint16_t *chain;
    const uint32_t *fast;
    uint32_t n_chain;         // uint16 entries
    uint32_t stg_bytes;       // per-wave exponent staging bytes
};

__device__ __forceinline__ uint64_t out_index(const ViewArgs &v, uint64_t g)
{
    if (!v.tr) return g;
    const uint64_t tile = (uint64_t)v.tr * v.tc;
    const uint64_t t = g / tile, w = g - t * tile;
    const uint32_t r = (uint32_t)(w / v.tc), c = (uint32_t)(w - (uint64_t)r * v.tc);
    const uint64_t rb = t / v.tiles_per_row, cb = t - rb * v.tiles_per_row;
    return (rb * v.tr + r) * v.cols + cb * v.tc + c;
}

// Decode segment `s` of view v with one wavefront.  stg: LDS byte offset of
// this wave's exponent staging; ereg: LDS byte offset of its word region.
template <int CB, int K>
__device__ __forceinline__ void decode_segment(const ViewArgs &v, uint64_t s, uint8_t *lds,
                                               uint32_t stg, uint32_t ereg, uint32_t stg_bytes,
                                               const uint2 *fast, const uint16_t *chain)
{
    constexpr uint32_t kChunkBits = 8 * CB;
    const uint32_t lane = lane_id();
    const uint64_t g0 = v.segs[s].elem_off;
    const uint64_t g1 = v.segs[s + 1].elem_off;
    const uint32_t nbits = v.segs[s].nbits;
    if (g1 > v.n || g1 < g0) return;                                   // corrupt records
    const uint32_t head = (uint32_t)(g0 & 15);
    if ((uint64_t)head + (g1 - g0) + 32 > stg_bytes) return;           // cannot be a valid segment

    const uint32_t rbase = stage_segment<CB>(lds, ereg, v.words, s);
    const uint32_t gap = v.gaps[s * 64 + lane];
    wave_lds_sync();

    const SegWindow win{lds, rbase};
    const uint32_t c0 = lane * kChunkBits;
    const uint32_t p0 = c0 + gap;
    const uint32_t end = min(c0 + kChunkBits, nbits);
    const uint32_t cnt = p0 < end ? count_codes<K>(win, fast, chain, p0, end) : 0u;
    uint32_t total;
    const uint32_t excl = wave_exclusive_scan(cnt, &total);
    if (total != (uint32_t)(g1 - g0)) return;                          // stream and records disagree

    emit_codes<K>(win, fast, chain, lds, p0, stg + head + excl, cnt);
    wave_lds_sync();

    // merge: 16-element groups aligned to the stream index
    const uint64_t gbase = g0 & ~15ull;
    const uint32_t ngroups = (uint32_t)((((g1 + 15) & ~15ull) - gbase) >> 4);
    const uint8_t *sm = v.sm;
    for (uint32_t gi = lane; gi < ngroups; gi += 64) {
        const uint64_t gs = gbase + 16ull * gi;
        const uint4 smv = *reinterpret_cast<const uint4 *>(sm + gs);
        const uint4 rx = *reinterpret_cast<const uint4 *>(lds + stg + 16 * gi);
        const uint64_t o = out_index(v, gs);
        if (gs >= g0 && gs + 16 <= g1) {
            const uint2 a = assemble4(smv.x, rx.x), b = assemble4(smv.y, rx.y);
            const uint2 c = assemble4(smv.z, rx.z), d = assemble4(smv.w, rx.w);
            uint4 *dst = reinterpret_cast<uint4 *>(v.out + o);
            dst[0] = make_uint4(a.x, a.y, b.x, b.y);
            dst[1] = make_uint4(c.x, c.y, d.x, d.y);
        } else {
            const uint32_t smw[4] = {smv.x, smv.y, smv.z, smv.w};
            const uint32_t rxw[4] = {rx.x, rx.y, rx.z, rx.w};
#pragma unroll
            for (uint32_t j = 0; j < 16; j++) {
                const uint64_t g = gs + j;
                if (g >= g0 && g < g1)
                    v.out[o + j] = assemble1(smw[j >> 2] >> (8 * (j & 3)), rxw[j >> 2] >> (8 * (j & 3)));
            }
        }
    }
    wave_lds_sync();   // staging is reused by this wave's next segment
}

template <int CB>
constexpr uint32_t ereg_bytes() { return (64 * (CB / 4) + 8) * 4; }

// Stage both tables into LDS once per workgroup.
template <int K>
__device__ __forceinline__ void stage_tables(uint8_t *lds, uint32_t fast_off, uint32_t chain_off,
                                             const TableArgs &t)
{
    uint32_t *fl = reinterpret_cast<uint32_t *>(lds + fast_off);
    for (uint32_t i = threadIdx.x; i < (2u << K); i += blockDim.x) fl[i] = t.fast[i];
    uint16_t *cl = reinterpret_cast<uint16_t *>(lds + chain_off);
    for (uint32_t i = threadIdx.x; i < t.n_chain; i += blockDim.x) cl[i] = t.chain[i];
    __syncthreads();
}

template <int CB, int K, int WAVES>
__global__ void __launch_bounds__(WAVES * 64)
decode_kernel(ViewArgs v, TableArgs t)
{
    extern __shared__ __align__(16) uint8_t lds[];
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t stg = 16 + wave * t.stg_bytes;
    const uint32_t ereg_off = 16 + WAVES * t.stg_bytes;
    const uint32_t ereg = ereg_off + wave * ereg_bytes<CB>();
    const uint32_t fast_off = ereg_off + WAVES * ereg_bytes<CB>();
    const uint32_t chain_off = fast_off + (8u << K);
    stage_tables<K>(lds, fast_off, chain_off, t);
    const uint2 *fast = reinterpret_cast<const uint2 *>(lds + fast_off);
    const uint16_t *chain = reinterpret_cast<const uint16_t *>(lds + chain_off);
    for (uint64_t s = (uint64_t)blockIdx.x * WAVES + wave; s < v.n_segments; s += (uint64_t)gridDim.x * WAVES)
        decode_segment<CB, K>(v, s, lds, stg, ereg, t.stg_bytes, fast, chain);
}

int check_view(const df11_view *v, uint64_t out_elems)
{
    if (!v) return df11::fail(DF11_E_ARG, "null view");
    if (v->seg_lanes != 64 || v->chunk_bytes != 16)
        return df11::fail(DF11_E_UNSUPPORTED, "decode kernels are built for 16-byte chunks and 64-lane segments (got %u, %u)",
                          v->chunk_bytes, v->seg_lanes);
    if (v->fast_bits < DF11_FAST_BITS_MIN || v->fast_bits > DF11_FAST_BITS_MAX)
        return df11::fail(DF11_E_ARG, "fast_bits %u out of range", v->fast_bits);
    if (v->n_tables < 1 || v->n_tables > DF11_MAX_TABLES || v->n_chain != (uint64_t)v->n_tables * 256 ||
        v->n_fast != (2ull << v->fast_bits))
        return df11::fail(DF11_E_ARG, "table sizes inconsistent");
    const uint64_t seg_words = 64ull * v->chunk_bytes / 4;
    if (v->n_segs != v->n_segments + 1 || v->n_gaps != v->n_segments * 64 ||
        v->n_exp_words < v->n_segments * seg_words + 2 || v->n_sm < (v->n + 15) / 16 * 16)
        return df11::fail(DF11_E_ARG, "view array sizes inconsistent with n / n_segments");
    if (v->n && (!v->exp_words || !v->sm || !v->gaps || !v->segs || !v->chain || !v->fast))
        return df11::fail(DF11_E_ARG, "null array in view");
    if (((uintptr_t)v->sm & 15) || ((uintptr_t)v->exp_words & 15) || ((uintptr_t)v->fast & 7) ||
        ((uintptr_t)v->segs & 7))
        return df11::fail(DF11_E_ARG, "view arrays must be 16-byte aligned (sm, exp_words)");
    if (v->tile_rows) {
        if (!v->tile_cols || v->tile_cols % 16 || !v->cols || v->cols % v->tile_cols ||
            (uint64_t)v->tile_rows * v->tile_cols > 0xFFFFFFFFull)
            return df11::fail(DF11_E_ARG, "bad tile order in view");
    }
    (void)out_elems;
    return DF11_OK;
}

uint32_t staging_bytes(const df11_view *v)
{
    const uint32_t seg_bits = 64u * 8u * v->chunk_bytes;
    const uint32_t minlen = std::max(1u, v->min_len);
    const uint32_t tmax = seg_bits / minlen + 1;
    return (16 + tmax + 32 + 15) & ~15u;
}

struct LaunchShape {
    int waves;
    uint32_t lds;
};

// Pick waves per workgroup so that exponent staging stays under 64 KB (the
// emit loop keeps LDS addresses in 16 bits) and the total fits 160 KB.
int pick_shape(uint32_t stg, uint32_t fast_bits, uint32_t n_tables, LaunchShape *sh)
{
    const uint32_t tables = (8u << fast_bits) + ((n_tables * 512u + 15) & ~15u);
    for (int w : {8, 4, 2, 1}) {
        const uint32_t total = 16 + w * stg + w * ereg_bytes<16>() + tables;
        if (16 + (uint32_t)w * stg <= 65520 && total <= 160 * 1024) {
            sh->waves = w;
            sh->lds = total;
            return DF11_OK;
        }
    }
    return df11::fail(DF11_E_UNSUPPORTED, "tables and staging do not fit in LDS");
}

int device_cu_count()
{
    static int cus = 0;
    if (!cus) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) return 256;
        hipDeviceProp_t p;
        if (hipGetDeviceProperties(&p, dev) != hipSuccess) return 256;
        cus = p.multiProcessorCount;
    }
    return cus;
}

ViewArgs make_args(const df11_view *v, uint16_t *out, uint64_t seg_begin)
{
    ViewArgs a{};
    a.words = v->exp_words;
    a.sm = v->sm;
    a.gaps = v->gaps;
    a.segs = v->segs;
    a.out = out;
    a.n = v->n;
    a.n_segments = v->n_segments;
    a.seg_begin = seg_begin;
    a.tr = v->tile_rows;
    a.tc = v->tile_cols;
    a.tiles_per_row = v->tile_rows ? (uint32_t)(v->cols / v->tile_cols) : 0;
    a.cols = v->cols;
    return a;
}

template <int K>
int launch_one(const ViewArgs &a, const TableArgs &t, const LaunchShape &sh, uint64_t nseg, hipStream_t st)
{
    const uint64_t groups_needed = (nseg + sh.waves - 1) / sh.waves;
    const uint64_t per_cu = std::max<uint64_t>(1, std::min<uint64_t>((160u * 1024u) / sh.lds, 32 / sh.waves));
    const uint64_t groups = std::min<uint64_t>(groups_needed, (uint64_t)device_cu_count() * per_cu);
    if (!groups) return DF11_OK;
    switch (sh.waves) {
    case 8: hipLaunchKernelGGL((decode_kernel<16, K, 8>), dim3((uint32_t)groups), dim3(512), sh.lds, st, a, t); break;
    case 4: hipLaunchKernelGGL((decode_kernel<16, K, 4>), dim3((uint32_t)groups), dim3(256), sh.lds, st, a, t); break;
    case 2: hipLaunchKernelGGL((decode_kernel<16, K, 2>), dim3((uint32_t)groups), dim3(128), sh.lds, st, a, t); break;
    default: hipLaunchKernelGGL((decode_kernel<16, K, 1>), dim3((uint32_t)groups), dim3(64), sh.lds, st, a, t); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return df11::fail(DF11_E_DEVICE, "decode launch: %s", hipGetErrorString(e));
    return DF11_OK;
}

}  // namespace

extern "C" int df11_decode(const df11_view *v, uint16_t *out, void *stream)
{
    int rc = check_view(v, v ? v->n : 0);
    if (rc) return rc;
    if (!v->n) return DF11_OK;
    if (!out || ((uintptr_t)out & 15)) return df11::fail(DF11_E_ARG, "out must be a 16-byte aligned device pointer");
    const uint32_t stg = staging_bytes(v);
    LaunchShape sh;
    if ((rc = pick_shape(stg, v->fast_bits, v->n_tables, &sh))) return rc;
    TableArgs t{v->chain, v->fast, (uint32_t)v->n_chain, stg};
    const ViewArgs a = make_args(v, out, 0);
    hipStream_t st = (hipStream_t)stream;
    switch (v->fast_bits) {
    case 8: return launch_one<8>(a, t, sh, v->n_segments, st);
    case 9: return launch_one<9>(a, t, sh, v->n_segments, st);
    case 10: return launch_one<10>(a, t, sh, v->n_segments, st);
    case 11: return launch_one<11>(a, t, sh, v->n_segments, st);
    default: return launch_one<12>(a, t, sh, v->n_segments, st);
    }
}
