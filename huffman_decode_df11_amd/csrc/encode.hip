// The DFloat11 encoder on the GPU: exponent histogram, code placement and
// segment metadata for a BF16 tensor already in device memory.  It writes
// the same bytes as df11_encode on the host for the same codebook and
// layout.
//
// [P1] "DFloat11无损压缩技术：基于哈夫曼编码的BFloat16大模型显存优化方案" 2.2
//      items 1-2: count exponent frequencies, build the Huffman code, store
//      the coded exponents and the verbatim sign+mantissa bytes.
// [P3] "DFloat11重新定义LLM无损压缩的技术边界" 4.1: the offline compression of
//      a large model takes hours on the CPU; here every step but the
//      256-symbol code construction runs on the device.
//
// Steps: (1) hist_kernel counts exponents (LDS sub-histograms per wave);
// the host builds the codebook from the counts.  (2) bits_kernel sums the
// code lengths of fixed blocks of E elements in stream order.  (3) The host
// turns the block sums into block start bits (adding the padding that
// starts an aligned block on a segment boundary), which fixes the stream
// length, the segment count and every output size.  (4) emit_kernel: per
// block, a workgroup scan of the code lengths gives each element's first
// bit; the code is OR-ed into the zeroed stream words with 32-bit atomics
// (a code touches at most two words, shared with neighbours), the
// sign+mantissa byte is stored, and the elements at segment and chunk
// boundaries write the gaps and segment records.  (5) seg_max_kernel finds
// the largest segment.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <new>
#include <numeric>
#include <vector>

#include "df11_internal.h"

struct df11_device_encoded {
    uint64_t n = 0, total_bits = 0, n_segments = 0;
    df11_layout layout{};
    uint32_t min_len = 0, max_len = 0, n_tables = 0, fast_bits = 0, max_seg_elems = 0;
    int32_t row_win_lo = 0;
    uint32_t row_win_span = 0;
    uint32_t *exp_words = nullptr;
    uint8_t *sm = nullptr;
    uint8_t *gaps = nullptr;
    df11_segment *segs = nullptr;
    uint16_t *chain = nullptr;
    uint32_t *fast = nullptr;
    uint64_t *block_seg = nullptr;
    uint8_t *counts = nullptr;
    uint64_t n_exp_words = 0, n_sm = 0, n_gaps = 0, n_segs = 0, n_chain = 0, n_fast = 0, n_block_seg = 0, n_counts = 0;
    void *blob = nullptr;   // one device allocation holding every array above
};

namespace {

constexpr uint32_t kThreads = 256;
constexpr uint32_t kMaxBlock = 4096;   // elements per scan block

// Stream position g -> index of the source element (row-major, tile order,
// column groups inside tiles), as the layout defines it.
struct DevOrder {
    uint64_t cols, tr, tc, kc, tile, tiles_per_row;
    uint32_t pow2, trs, tcs, kcs;   // pow2: tr, tc (and kc when set) are powers of two with these shifts
    __device__ __forceinline__ uint64_t operator()(uint64_t g) const
    {
        if (!tr) return g;
        if (pow2) {
            const uint64_t t = g >> (trs + tcs), w = g & ((1ull << (trs + tcs)) - 1);
            uint64_t r, c;
            if (kc) {
                const uint64_t in = w & ((1ull << (trs + kcs)) - 1);
                r = in >> kcs;
                c = ((w >> (trs + kcs)) << kcs) | (in & ((1ull << kcs) - 1));
            } else {
                r = w >> tcs;
                c = w & ((1ull << tcs) - 1);
            }
            const uint64_t rb = t / tiles_per_row, cb = t - rb * tiles_per_row;
            return ((rb << trs) + r) * cols + (cb << tcs) + c;
        }
        const uint64_t t = g / tile, w = g - t * tile;
        uint64_t r, c;
        if (kc) {
            const uint64_t grp = w / (tr * kc), in = w - grp * (tr * kc);
            r = in / kc;
            c = grp * kc + (in - r * kc);
        } else {
            r = w / tc;
            c = w - r * tc;
        }
        const uint64_t rb = t / tiles_per_row, cb = t - rb * tiles_per_row;
        return (rb * tr + r) * cols + cb * tc + c;
    }
};

DevOrder make_order(const df11_layout &L)
{
    DevOrder o{};
    if (L.tile_rows) {
        o.cols = L.cols;
        o.tr = L.tile_rows;
        o.tc = L.tile_cols;
        o.kc = L.tile_kchunk;
        o.tile = o.tr * o.tc;
        o.tiles_per_row = L.cols / L.tile_cols;
        auto lg = [](uint64_t x) -> int {
            if (!x || (x & (x - 1))) return -1;
            int k = 0;
            while ((1ull << k) != x) k++;
            return k;
        };
        const int a = lg(o.tr), b = lg(o.tc), c = o.kc ? lg(o.kc) : 0;
        if (a >= 0 && b >= 0 && c >= 0) {
            o.pow2 = 1;
            o.trs = (uint32_t)a;
            o.tcs = (uint32_t)b;
            o.kcs = (uint32_t)c;
        }
    }
    return o;
}

struct CodeTable {
    uint8_t len[256];
    uint32_t code[256];
};

// Exponent histogram.  Gaussian-like weights put most exponents in a handful
// of bins, so 64 lanes adding into one histogram collide on the same LDS
// words; each wave keeps kSub copies (lane l adds into copy l % kSub), which
// are summed per bin at the end.  Eight elements per lane per load.
constexpr uint32_t kSub = 16;

__global__ void __launch_bounds__(kThreads) hist_kernel(const uint16_t *bits, uint64_t n, unsigned long long *hist)
{
    __shared__ uint32_t h[kThreads / 64 * kSub][256];
    uint32_t *hf = &h[0][0];
    for (uint32_t i = threadIdx.x; i < kThreads / 64 * kSub * 256; i += kThreads) hf[i] = 0;
    __syncthreads();
    uint32_t *mine = h[(threadIdx.x >> 6) * kSub + (threadIdx.x & (kSub - 1))];
    const uint64_t n8 = n / 8;
    const uint4 *b8 = reinterpret_cast<const uint4 *>(bits);
    const bool aligned = ((uintptr_t)bits & 15) == 0;
    if (aligned) {
        for (uint64_t i = blockIdx.x * (uint64_t)kThreads + threadIdx.x; i < n8; i += (uint64_t)gridDim.x * kThreads) {
            const uint4 v = b8[i];
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int k = 0; k < 4; k++) {
                atomicAdd(&mine[(w[k] >> 7) & 0xFFu], 1u);
                atomicAdd(&mine[(w[k] >> 23) & 0xFFu], 1u);
            }
        }
    }
    for (uint64_t i = (aligned ? n8 * 8 : 0) + blockIdx.x * (uint64_t)kThreads + threadIdx.x; i < n;
         i += (uint64_t)gridDim.x * kThreads)
        atomicAdd(&mine[(bits[i] >> 7) & 0xFF], 1u);
    __syncthreads();
    for (uint32_t e = threadIdx.x; e < 256; e += kThreads) {
        uint64_t c = 0;
        for (uint32_t k = 0; k < kThreads / 64 * kSub; k++) c += h[k][e];
        if (c) atomicAdd(&hist[e], (unsigned long long)c);
    }
}

// Sum of the code lengths of each block of E elements (stream order); an
// exponent without a code sets *uncoded.
__global__ void __launch_bounds__(kThreads) bits_kernel(const uint16_t *bits, uint64_t n, uint32_t E, DevOrder order,
                                                        CodeTable ct, uint32_t *block_bits, uint32_t *uncoded)
{
    __shared__ uint8_t len[256];
    __shared__ uint32_t part[kThreads / 64];
    for (uint32_t i = threadIdx.x; i < 256; i += kThreads) len[i] = ct.len[i];
    __syncthreads();
    const uint64_t g0 = (uint64_t)blockIdx.x * E;
    uint32_t sum = 0, bad = 0;
    for (uint32_t i = threadIdx.x; i < E && g0 + i < n; i += kThreads) {
        const uint32_t L = len[(bits[order(g0 + i)] >> 7) & 0xFF];
        bad |= L == 0;
        sum += L;
    }
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = sum;
    if (bad) atomicOr(uncoded, 1u);
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
        for (uint32_t w = 0; w < kThreads / 64; w++) t += part[w];
        block_bits[blockIdx.x] = t;
    }
}

struct EmitArgs {
    const uint16_t *bits;
    uint64_t n, nseg, seg_bits, chunk_bits;
    uint32_t sb_shift, cb_shift;   // seg_bits = 1 << sb_shift, chunk_bits = 1 << cb_shift
    uint32_t E;
    DevOrder order;
    const uint64_t *base;   // [nblocks + 1]: first bit of each block; base[nblocks] = ~0
    const uint64_t *end;    // [nblocks]: bit after each block's last code
    uint32_t *words;
    uint8_t *sm;
    uint8_t *gaps;
    df11_segment *segs;
    uint32_t *counts32;     // codes starting in each chunk (accumulated)
};

// One block of E elements per workgroup: each thread takes consecutive
// elements (their codes' bit positions from a workgroup scan of the lengths),
// ORs its codes into the block's stream words and counts code starts per
// chunk in LDS, and stages the sign+mantissa bytes there; the words, bytes
// and counts then go out with plain coalesced stores, except the block's
// first and last word and chunk, which it may share with its neighbours
// (atomic OR / add into memory cleared beforehand).
constexpr uint32_t kPer = kMaxBlock / kThreads;   // elements per thread at most
constexpr uint32_t kMaxWords = kMaxBlock + 2;       // stream words of a block of codes of at most 32 bits
constexpr uint32_t kMaxChunks = kMaxBlock * 32 / 64 + 2;   // chunks of at least 8 bytes

__global__ void __launch_bounds__(kThreads) emit_kernel(EmitArgs a, CodeTable ct)
{
    __shared__ uint8_t len[256];
    __shared__ uint32_t code[256];
    __shared__ uint32_t scan[kThreads];
    __shared__ uint32_t words[kMaxWords];
    __shared__ uint32_t ccount[kMaxChunks];
    __shared__ __align__(16) uint8_t smb[kMaxBlock];
    const uint64_t b = blockIdx.x;
    const uint64_t g0 = b * a.E;
    const uint32_t cnt = (uint32_t)min<uint64_t>(a.E, a.n - g0);
    const uint64_t bbase = a.base[b], bend = a.end[b];
    const uint32_t cbs = a.cb_shift, sbs = a.sb_shift;
    const uint64_t wlo = bbase >> 5, clo = bbase >> cbs;
    const uint32_t nw = (uint32_t)(((bend - 1) >> 5) - wlo + 1);
    const uint32_t nc = (uint32_t)(((bend - 1) >> cbs) - clo + 1);
    for (uint32_t i = threadIdx.x; i < 256; i += kThreads) {
        len[i] = ct.len[i];
        code[i] = ct.code[i];
    }
    for (uint32_t i = threadIdx.x; i < nw; i += kThreads) words[i] = 0;
    for (uint32_t i = threadIdx.x; i < nc; i += kThreads) ccount[i] = 0;
    const uint32_t per = (cnt + kThreads - 1) / kThreads;       // consecutive elements per thread
    const uint32_t i0 = min(cnt, threadIdx.x * per), i1 = min(cnt, i0 + per);
    __syncthreads();
    uint16_t uu[kPer];
    uint32_t mine = 0;
#pragma unroll
    for (uint32_t k = 0; k < kPer; k++) {
        uu[k] = i0 + k < i1 ? a.bits[a.order(g0 + i0 + k)] : 0;
        if (i0 + k < i1) mine += len[(uu[k] >> 7) & 0xFF];
    }
    scan[threadIdx.x] = mine;
    __syncthreads();
    for (uint32_t off = 1; off < kThreads; off <<= 1) {   // inclusive Hillis-Steele scan
        const uint32_t v = threadIdx.x >= off ? scan[threadIdx.x - off] : 0u;
        __syncthreads();
        scan[threadIdx.x] += v;
        __syncthreads();
    }
    uint64_t pos = bbase + (scan[threadIdx.x] - mine);
    // start of the element before i0
    uint64_t prev;
    bool has_prev = g0 + i0 > 0;
    if (!has_prev) {
        prev = 0;
    } else {
        const uint32_t lp = len[(a.bits[a.order(g0 + i0 - 1)] >> 7) & 0xFF];
        prev = (i0 == 0 ? a.end[b - 1] : pos) - lp;
    }
    const uint64_t SB = a.seg_bits, CB = a.chunk_bits;
    uint64_t run_chunk = ~0ull;   // chunk of the codes counted in run_n, not yet added
    uint32_t run_n = 0;
#pragma unroll
    for (uint32_t k = 0; k < kPer; k++) {
        if (i0 + k >= i1) break;
        const uint32_t i = i0 + k;
        const uint64_t g = g0 + i;
        const uint16_t u = uu[k];
        const uint32_t e = (u >> 7) & 0xFF;
        const uint32_t L = len[e];
        // the code, first bit at bit (31 - pos % 32) of word pos / 32
        const uint32_t w = (uint32_t)((pos >> 5) - wlo), off = (uint32_t)(pos & 31);
        const uint64_t wide = (uint64_t)code[e] << (64 - off - L);
        const uint32_t hi = (uint32_t)(wide >> 32), lo = (uint32_t)wide;
        if (hi) atomicOr(&words[w], hi);
        if (lo) atomicOr(&words[w + 1], lo);
        smb[i] = (uint8_t)(((u >> 8) & 0x80) | (u & 0x7F));
        if ((pos >> cbs) != run_chunk) {
            if (run_n) atomicAdd(&ccount[run_chunk - clo], run_n);
            run_chunk = pos >> cbs;
            run_n = 0;
        }
        run_n++;
        const uint64_t s = pos >> sbs;
        // gap of the chunk holding this code's first bit, when no earlier code starts in it
        const uint64_t c0 = pos & ~(CB - 1);
        if (!has_prev || prev < c0) a.gaps[c0 >> cbs] = (uint8_t)(pos - c0);
        // this element opens segments (previous segment, s]
        const uint64_t sp = has_prev ? prev >> sbs : ~0ull;
        for (uint64_t t = sp + 1; t <= s; t++) a.segs[t].elem_off = g;
        // last code of its segment: segment length in bits and the gap of a chunk it runs into
        const uint64_t vend = pos + L;
        const uint64_t next = i + 1 < cnt ? vend : a.base[b + 1];
        if (next == ~0ull || (next >> sbs) > s) {
            a.segs[s].nbits = (uint32_t)min<uint64_t>(SB, vend - (s << sbs));
            const uint64_t c1 = c0 + CB;
            if (c1 < vend && c1 < ((s + 1) << sbs)) a.gaps[c1 >> cbs] = (uint8_t)(vend - c1);
        }
        if (g + 1 == a.n)   // trailing segments without a code start, and the closing record
            for (uint64_t t = s + 1; t <= a.nseg; t++) a.segs[t].elem_off = a.n;
        prev = pos;
        has_prev = true;
        pos = vend;
    }
    if (run_n) atomicAdd(&ccount[run_chunk - clo], run_n);
    __syncthreads();
    // words and chunks strictly inside the block's bits belong to it alone
    for (uint32_t i = threadIdx.x; i < nw; i += kThreads) {
        const uint32_t v = words[i];
        if (i == 0 || i + 1 == nw) {
            if (v) atomicOr(&a.words[wlo + i], v);
        } else {
            a.words[wlo + i] = v;
        }
    }
    for (uint32_t i = threadIdx.x; i < nc; i += kThreads) {
        const uint32_t v = ccount[i];
        if (i == 0 || i + 1 == nc) {
            if (v) atomicAdd(&a.counts32[clo + i], v);
        } else {
            a.counts32[clo + i] = v;
        }
    }
    // sign+mantissa bytes [g0, g0 + cnt): 16-byte stores where they align
    uint8_t *smo = a.sm + g0;
    const uint32_t head = (uint32_t)((16 - ((uintptr_t)smo & 15)) & 15);
    const uint32_t h = min(head, cnt);
    for (uint32_t i = threadIdx.x; i < h; i += kThreads) smo[i] = smb[i];
    const uint32_t body = (cnt - h) / 16;
    for (uint32_t q = threadIdx.x; q < body; q += kThreads) {
        uint4 v;
        uint8_t *vb = reinterpret_cast<uint8_t *>(&v);
#pragma unroll
        for (int k = 0; k < 16; k++) vb[k] = smb[h + 16 * q + k];
        *reinterpret_cast<uint4 *>(smo + h + 16 * q) = v;
    }
    for (uint32_t i = h + 16 * body + threadIdx.x; i < cnt; i += kThreads) smo[i] = smb[i];
}

__global__ void narrow_counts_kernel(const uint32_t *c32, uint8_t *c8, uint64_t n)
{
    for (uint64_t i = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x; i < n; i += (uint64_t)gridDim.x * blockDim.x)
        c8[i] = (uint8_t)c32[i];
}

__global__ void seg_max_kernel(const df11_segment *segs, uint64_t nseg, uint32_t *out)
{
    uint32_t m = 0;
    for (uint64_t s = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x; s < nseg; s += (uint64_t)gridDim.x * blockDim.x)
        m = max(m, (uint32_t)(segs[s + 1].elem_off - segs[s].elem_off));
    for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor(m, off));
    if ((threadIdx.x & 63) == 0 && m) atomicMax(out, m);
}

int hip_fail(hipError_t e, const char *what)
{
    return df11::fail(e == hipErrorOutOfMemory ? DF11_E_ALLOC : DF11_E_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

#define HIP_TRY(call, what)                          \
    do {                                             \
        hipError_t e_ = (call);                      \
        if (e_ != hipSuccess) return hip_fail(e_, what); \
    } while (0)

uint32_t grid_for(uint64_t items, uint32_t per_group)
{
    return (uint32_t)std::max<uint64_t>(1, std::min<uint64_t>((items + per_group - 1) / per_group, 65535ull * 16));
}

void free_device(df11_device_encoded *d)
{
    if (!d) return;
    if (d->blob) (void)hipFree(d->blob);
    delete d;
}

// Byte offsets of consecutive 256-byte aligned parts of one allocation.
struct Carve {
    uint64_t total = 0;
    uint64_t take(uint64_t bytes)
    {
        const uint64_t off = total;
        total += (std::max<uint64_t>(bytes, 16) + 255) / 256 * 256;
        return off;
    }
};

// Device scratch freed on every return path.
struct Scratch {
    std::vector<void *> ptrs;
    ~Scratch()
    {
        for (void *p : ptrs) (void)hipFree(p);
    }
    template <class T>
    hipError_t alloc(T **p, uint64_t count)
    {
        *p = nullptr;
        hipError_t e = hipMalloc((void **)p, std::max<uint64_t>(count, 1) * sizeof(T));
        if (e == hipSuccess) ptrs.push_back(*p);
        return e;
    }
};

}  // namespace

extern "C" int df11_hist_device(const uint16_t *bits, uint64_t n, uint64_t hist[256], void *stream)
{
    if (!hist || (n && !bits)) return df11::fail(DF11_E_ARG, "df11_hist_device: null pointer");
    if (!n) return DF11_OK;
    hipStream_t st = (hipStream_t)stream;
    Scratch s;
    unsigned long long *dh;
    HIP_TRY(s.alloc(&dh, 256), "hist buffer");
    HIP_TRY(hipMemsetAsync(dh, 0, 256 * sizeof(unsigned long long), st), "hist clear");
    hipLaunchKernelGGL(hist_kernel, dim3(std::min<uint32_t>(grid_for(n, kThreads * 64), 2048)), dim3(kThreads), 0, st,
                       bits, n, dh);
    HIP_TRY(hipGetLastError(), "hist launch");
    unsigned long long h[256];
    HIP_TRY(hipMemcpyAsync(h, dh, sizeof h, hipMemcpyDeviceToHost, st), "hist copy");
    HIP_TRY(hipStreamSynchronize(st), "hist sync");
    for (int i = 0; i < 256; i++) hist[i] += h[i];
    return DF11_OK;
}

extern "C" int df11_encode_device(const uint16_t *bits, uint64_t n, const df11_codebook *cb,
                                  const df11_layout *layout_in, void *stream, df11_device_encoded **out)
{
    if (!out || !cb || (n && !bits)) return df11::fail(DF11_E_ARG, "df11_encode_device: null pointer");
    *out = nullptr;
    const df11_layout L = df11::complete_layout(layout_in);
    int rc = df11::check_layout(L, n);
    if (rc) return rc;
    if (cb->fast_bits < DF11_FAST_BITS_MIN || cb->fast_bits > DF11_FAST_BITS_MAX || cb->n_tables < 1 ||
        cb->n_tables > DF11_MAX_TABLES || cb->max_len > DF11_MAX_LEN)
        return df11::fail(DF11_E_ARG, "codebook not built by df11_codebook_build");
    rc = df11::check_counts_fit(L, cb);
    if (rc) return rc;
    hipStream_t st = (hipStream_t)stream;
    const uint64_t chunk_bits = 8ull * L.chunk_bytes, seg_bits = chunk_bits * L.seg_lanes, seg_words = seg_bits / 32;
    // scan blocks nest in aligned blocks, so padding only falls between scan blocks
    const uint32_t E = L.align_elems ? (uint32_t)std::gcd<uint64_t>(L.align_elems, kMaxBlock) : kMaxBlock;
    const uint64_t nb = (n + E - 1) / E;
    const DevOrder order = make_order(L);
    CodeTable ct;
    for (int i = 0; i < 256; i++) {
        ct.len[i] = (uint8_t)cb->len[i];
        ct.code[i] = cb->code[i];
    }

    Scratch s;
    std::vector<uint64_t> base(nb + 1), end(nb);
    uint64_t total = 0;
    if (n) {
        uint32_t *dbits, *dflag;
        HIP_TRY(s.alloc(&dbits, nb + 1), "block sums");
        dflag = dbits + nb;
        HIP_TRY(hipMemsetAsync(dflag, 0, sizeof(uint32_t), st), "flag clear");
        hipLaunchKernelGGL(bits_kernel, dim3((uint32_t)nb), dim3(kThreads), 0, st, bits, n, E, order, ct, dbits, dflag);
        HIP_TRY(hipGetLastError(), "block sum launch");
        std::vector<uint32_t> bb(nb);
        uint32_t flag = 0;
        HIP_TRY(hipMemcpyAsync(bb.data(), dbits, nb * sizeof(uint32_t), hipMemcpyDeviceToHost, st), "block sum copy");
        HIP_TRY(hipMemcpyAsync(&flag, dflag, sizeof flag, hipMemcpyDeviceToHost, st), "flag copy");
        HIP_TRY(hipStreamSynchronize(st), "block sum sync");
        if (flag) return df11::fail(DF11_E_UNCODED, "an exponent of the tensor has no code");
        for (uint64_t b = 0; b < nb; b++) {
            const uint64_t g = b * E;
            if (L.align_elems && g && g % L.align_elems == 0) total = (total + seg_bits - 1) / seg_bits * seg_bits;
            base[b] = total;
            total += bb[b];
            end[b] = total;
        }
    }
    base[nb] = ~0ull;
    const uint64_t nseg = (total + seg_bits - 1) / seg_bits;

    df11_device_encoded *d = new (std::nothrow) df11_device_encoded();
    if (!d) return df11::fail(DF11_E_ALLOC, "out of host memory");
    struct Guard {
        df11_device_encoded *&d;
        ~Guard() { free_device(d); }
    } guard{d};
    d->n = n;
    d->total_bits = total;
    d->n_segments = nseg;
    d->layout = L;
    d->min_len = cb->min_len;
    d->max_len = cb->max_len;
    d->n_tables = cb->n_tables;
    d->fast_bits = cb->fast_bits;
    d->n_exp_words = nseg * seg_words + 2;
    d->n_sm = (n + 15) / 16 * 16;
    d->n_gaps = nseg * L.seg_lanes;
    d->n_counts = d->n_gaps;
    d->n_segs = nseg + 1;
    d->n_chain = (uint64_t)cb->n_tables * 256;
    d->n_fast = 2ull << cb->fast_bits;
    d->n_block_seg = L.align_elems ? (n + L.align_elems - 1) / L.align_elems + 1 : 0;
    // every array in one allocation (one hipMalloc and one hipFree per
    // encoding); the parts the emit kernel fills only in part are cleared
    // in one fill: stream words, sign+mantissa bytes, gaps, counts, records
    Carve cv;
    const uint64_t o_words = cv.take(d->n_exp_words * 4), o_sm = cv.take(d->n_sm), o_gaps = cv.take(d->n_gaps),
                   o_counts = cv.take(d->n_counts), o_segs = cv.take(d->n_segs * sizeof(df11_segment));
    const uint64_t cleared = cv.total;
    const uint64_t o_chain = cv.take(d->n_chain * 2), o_fast = cv.take(d->n_fast * 4),
                   o_bseg = cv.take(d->n_block_seg * 8);
    HIP_TRY(hipMalloc(&d->blob, cv.total), "encoded arrays");
    uint8_t *blob = static_cast<uint8_t *>(d->blob);
    d->exp_words = reinterpret_cast<uint32_t *>(blob + o_words);
    d->sm = blob + o_sm;
    d->gaps = blob + o_gaps;
    d->counts = blob + o_counts;
    d->segs = reinterpret_cast<df11_segment *>(blob + o_segs);
    d->chain = reinterpret_cast<uint16_t *>(blob + o_chain);
    d->fast = reinterpret_cast<uint32_t *>(blob + o_fast);
    d->block_seg = d->n_block_seg ? reinterpret_cast<uint64_t *>(blob + o_bseg) : nullptr;
    HIP_TRY(hipMemsetAsync(blob, 0, cleared, st), "clear");
    HIP_TRY(hipMemcpyAsync(d->chain, cb->chain, d->n_chain * 2, hipMemcpyHostToDevice, st), "tables");
    HIP_TRY(hipMemcpyAsync(d->fast, cb->fast, d->n_fast * 4, hipMemcpyHostToDevice, st), "tables");
    std::vector<uint64_t> bseg(d->n_block_seg);
    for (uint64_t a = 0; a + 1 < d->n_block_seg; a++) bseg[a] = base[a * L.align_elems / E] / seg_bits;
    if (d->n_block_seg) {
        bseg[d->n_block_seg - 1] = nseg;
        HIP_TRY(hipMemcpyAsync(d->block_seg, bseg.data(), d->n_block_seg * 8, hipMemcpyHostToDevice, st), "block index");
    }
    if (n) {
        // block starts and ends, then the segment maximum and the 32-bit
        // chunk counts (cleared), in one scratch allocation
        uint64_t *dbase, *dend;
        uint32_t *dmax, *dcnt;
        HIP_TRY(s.alloc(&dbase, (nb + 1) + nb + 1 + (d->n_counts + 2) / 2), "encode scratch");
        dend = dbase + nb + 1;
        dmax = reinterpret_cast<uint32_t *>(dend + nb);
        dcnt = dmax + 2;
        HIP_TRY(hipMemcpyAsync(dbase, base.data(), (nb + 1) * 8, hipMemcpyHostToDevice, st), "block starts");
        HIP_TRY(hipMemcpyAsync(dend, end.data(), nb * 8, hipMemcpyHostToDevice, st), "block ends");
        HIP_TRY(hipMemsetAsync(dmax, 0, 8 + std::max<uint64_t>(d->n_counts, 1) * 4, st), "clear");
        // chunk and segment sizes are powers of two (8 or 16 bytes, 64 lanes)
        const uint32_t cbs = L.chunk_bytes == 8 ? 6u : 7u, sbs = cbs + 6u;
        EmitArgs a{bits, n, nseg, seg_bits, chunk_bits, sbs, cbs, E, order, dbase, dend, d->exp_words, d->sm,
                   d->gaps, d->segs, dcnt};
        hipLaunchKernelGGL(emit_kernel, dim3((uint32_t)nb), dim3(kThreads), 0, st, a, ct);
        HIP_TRY(hipGetLastError(), "emit launch");
        if (d->n_counts)
            hipLaunchKernelGGL(narrow_counts_kernel, dim3(grid_for(d->n_counts, 1024)), dim3(256), 0, st, dcnt, d->counts,
                               d->n_counts);
        HIP_TRY(hipGetLastError(), "counts launch");
        hipLaunchKernelGGL(seg_max_kernel, dim3(grid_for(nseg, 256)), dim3(256), 0, st, d->segs, nseg, dmax);
        HIP_TRY(hipGetLastError(), "segment max launch");
        HIP_TRY(hipMemcpyAsync(&d->max_seg_elems, dmax, 4, hipMemcpyDeviceToHost, st), "max copy");
        HIP_TRY(hipStreamSynchronize(st), "encode sync");
        if (L.rows && L.cols && !L.tile_rows) {
            // the row window from the records, computed as the host encoder does
            std::vector<df11_segment> hs;
            try {
                hs.resize(d->n_segs);
            } catch (...) {
                return df11::fail(DF11_E_ALLOC, "out of host memory");
            }
            HIP_TRY(hipMemcpyAsync(hs.data(), d->segs, d->n_segs * sizeof(df11_segment), hipMemcpyDeviceToHost, st),
                    "segment records");
            HIP_TRY(hipStreamSynchronize(st), "encode sync");
            df11::row_window(hs.data(), nseg, n, L, &d->row_win_lo, &d->row_win_span);
        }
    } else {
        HIP_TRY(hipStreamSynchronize(st), "encode sync");
    }
    *out = d;
    d = nullptr;   // ownership passes to the caller
    return DF11_OK;
}

extern "C" void df11_device_encoded_free(df11_device_encoded *enc) { free_device(enc); }

extern "C" int df11_device_encoded_view(const df11_device_encoded *d, df11_view *v)
{
    if (!d || !v) return df11::fail(DF11_E_ARG, "df11_device_encoded_view: null pointer");
    std::memset(v, 0, sizeof(*v));
    v->n = d->n;
    v->total_bits = d->total_bits;
    v->n_segments = d->n_segments;
    v->chunk_bytes = d->layout.chunk_bytes;
    v->seg_lanes = d->layout.seg_lanes;
    v->rows = d->layout.rows;
    v->cols = d->layout.cols;
    v->tile_rows = d->layout.tile_rows;
    v->tile_cols = d->layout.tile_cols;
    v->tile_kchunk = d->layout.tile_kchunk;
    v->align_elems = d->layout.align_elems;
    v->min_len = d->min_len;
    v->max_len = d->max_len;
    v->n_tables = d->n_tables;
    v->fast_bits = d->fast_bits;
    v->max_seg_elems = d->max_seg_elems;
    v->row_win_lo = d->row_win_lo;
    v->row_win_span = d->row_win_span;
    v->exp_words = d->exp_words;  v->n_exp_words = d->n_exp_words;
    v->sm = d->sm;                v->n_sm = d->n_sm;
    v->gaps = d->gaps;            v->n_gaps = d->n_gaps;
    v->segs = d->segs;            v->n_segs = d->n_segs;
    v->chain = d->chain;          v->n_chain = d->n_chain;
    v->fast = d->fast;            v->n_fast = d->n_fast;
    v->block_seg = d->block_seg;  v->n_block_seg = d->n_block_seg;
    v->counts = d->counts;        v->n_counts = d->n_counts;
    return DF11_OK;
}

extern "C" int df11_device_encoded_to_host(const df11_device_encoded *d, df11_encoded **out)
{
    if (!d || !out) return df11::fail(DF11_E_ARG, "df11_device_encoded_to_host: null pointer");
    *out = nullptr;
    df11_encoded *h = new (std::nothrow) df11_encoded();
    if (!h) return df11::fail(DF11_E_ALLOC, "out of host memory");
    try {
        h->exp_words.resize(d->n_exp_words);
        h->sm.resize(d->n_sm);
        h->gaps.resize(d->n_gaps);
        h->segs.resize(d->n_segs);
        h->chain.resize(d->n_chain);
        h->fast.resize(d->n_fast);
        h->block_seg.resize(d->n_block_seg);
        h->counts.resize(d->n_counts);
    } catch (...) {
        delete h;
        return df11::fail(DF11_E_ALLOC, "out of host memory");
    }
    h->n = d->n;
    h->total_bits = d->total_bits;
    h->n_segments = d->n_segments;
    h->layout = d->layout;
    h->min_len = d->min_len;
    h->max_len = d->max_len;
    h->n_tables = d->n_tables;
    h->fast_bits = d->fast_bits;
    h->max_seg_elems = d->max_seg_elems;
    h->row_win_lo = d->row_win_lo;
    h->row_win_span = d->row_win_span;
    struct { void *dst; const void *src; uint64_t bytes; } parts[] = {
        {h->exp_words.data(), d->exp_words, d->n_exp_words * 4}, {h->sm.data(), d->sm, d->n_sm},
        {h->gaps.data(), d->gaps, d->n_gaps}, {h->segs.data(), d->segs, d->n_segs * sizeof(df11_segment)},
        {h->chain.data(), d->chain, d->n_chain * 2}, {h->fast.data(), d->fast, d->n_fast * 4},
        {h->block_seg.data(), d->block_seg, d->n_block_seg * 8}, {h->counts.data(), d->counts, d->n_counts}};
    for (auto &p : parts) {
        if (!p.bytes) continue;
        hipError_t e = hipMemcpy(p.dst, p.src, p.bytes, hipMemcpyDeviceToHost);
        if (e != hipSuccess) {
            delete h;
            return hip_fail(e, "device to host copy");
        }
    }
    *out = h;
    return DF11_OK;
}

