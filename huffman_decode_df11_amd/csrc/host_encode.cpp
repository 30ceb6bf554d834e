// Host encoder, view, validator and error reporting of libdf11.
//
// [P1] "DFloat11无损压缩技术：基于哈夫曼编码的BFloat16大模型显存优化方案" 2.2
//      item 2: a weight becomes its variable-length exponent code plus the
//      unchanged sign and 7 mantissa bits, packed into aligned blocks.
// [P3] "DFloat11重新定义LLM无损压缩的技术边界" 4.2: every GPU thread takes a
//      fixed run of encoded bytes; 5.2: data aligned to 256 bytes.
#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <string>

#include "df11_internal.h"

namespace df11 {

static thread_local std::string g_error;

int fail(int code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_error = buf;
    return code;
}

void clear_error() { g_error.clear(); }

}  // namespace df11

using namespace df11;

// Gemm tiles: 32 weight rows by 512 columns, one tile per segment run.
static const uint32_t kGemmTileRows = 32;
static const uint32_t kGemmTileCols = 512;
static const uint32_t kGemmKChunk = 8;

extern "C" uint32_t df11_gemm_tile_rows(void) { return kGemmTileRows; }
extern "C" uint32_t df11_gemm_tile_cols(void) { return kGemmTileCols; }

extern "C" int df11_gemm_layout(uint64_t rows, uint64_t cols, df11_layout *layout)
{
    if (!layout) return fail(DF11_E_ARG, "df11_gemm_layout: null layout");
    if (!rows || !cols || rows % kGemmTileRows || cols % kGemmTileCols)
        return fail(DF11_E_ARG, "weight [%llu, %llu] is not a multiple of the %ux%u gemm tile",
                    (unsigned long long)rows, (unsigned long long)cols, kGemmTileRows, kGemmTileCols);
    std::memset(layout, 0, sizeof(*layout));
    layout->chunk_bytes = 16;
    layout->seg_lanes = DF11_SEG_LANES;
    layout->rows = rows;
    layout->cols = cols;
    layout->tile_rows = kGemmTileRows;
    layout->tile_cols = kGemmTileCols;
    layout->tile_kchunk = kGemmKChunk;
    layout->align_elems = (uint64_t)kGemmTileRows * kGemmTileCols;
    return DF11_OK;
}

namespace df11 {

int check_layout(const df11_layout &L, uint64_t n)
{
    // the decode kernels read 16- and 8-byte chunks: no other layout is written
    if (L.chunk_bytes != 16 && L.chunk_bytes != 8)
        return fail(DF11_E_ARG, "chunk_bytes %u: the decoders read 8- or 16-byte chunks", L.chunk_bytes);
    if (L.seg_lanes != DF11_SEG_LANES)
        return fail(DF11_E_ARG, "seg_lanes %u: this build decodes one segment per 64-lane wavefront", L.seg_lanes);
    if (L.align_elems % 16)
        return fail(DF11_E_ARG, "align_elems %llu: need a multiple of 16", (unsigned long long)L.align_elems);
    if (L.tile_rows || L.tile_cols) {
        if (!L.tile_rows || !L.tile_cols || !L.rows || !L.cols)
            return fail(DF11_E_ARG, "tile order needs rows, cols, tile_rows and tile_cols");
        if (L.rows * L.cols != n)
            return fail(DF11_E_ARG, "rows*cols = %llu but n = %llu",
                        (unsigned long long)(L.rows * L.cols), (unsigned long long)n);
        if (L.rows % L.tile_rows || L.cols % L.tile_cols || L.tile_cols % 16)
            return fail(DF11_E_ARG, "tile %ux%u does not divide [%llu, %llu] or tile_cols %% 16 != 0",
                        L.tile_rows, L.tile_cols, (unsigned long long)L.rows, (unsigned long long)L.cols);
        if (L.tile_kchunk && (L.tile_kchunk % 8 || L.tile_cols % L.tile_kchunk || L.tile_rows % 2))
            return fail(DF11_E_ARG, "tile_kchunk %u: need a multiple of 8 dividing tile_cols, even tile_rows",
                        L.tile_kchunk);
    } else if (L.cols && L.rows * L.cols != n) {
        return fail(DF11_E_ARG, "rows*cols != n");
    }
    if (L.tile_kchunk && !L.tile_rows) return fail(DF11_E_ARG, "tile_kchunk needs tile order");
    return DF11_OK;
}

int check_counts_fit(const df11_layout &L, const df11_codebook *cb)
{
    if (8ull * L.chunk_bytes / std::max(1u, cb->min_len) > 255)
        return fail(DF11_E_ARG, "chunk_bytes %u with %u-bit codes: a chunk's code count would not fit a byte",
                    L.chunk_bytes, cb->min_len);
    return DF11_OK;
}

df11_layout complete_layout(const df11_layout *in)
{
    df11_layout L{};
    if (in) L = *in;
    if (!L.chunk_bytes) L.chunk_bytes = 16;
    if (!L.seg_lanes) L.seg_lanes = DF11_SEG_LANES;
    return L;
}

}  // namespace df11

namespace {

// Row-major index of stream element g.
struct Order {
    bool tiled = false;
    uint64_t cols = 0, tr = 0, tc = 0, kc = 0, tile = 0, tiles_per_row = 0;
    explicit Order(const df11_layout &L)
    {
        if (L.tile_rows) {
            tiled = true;
            cols = L.cols; tr = L.tile_rows; tc = L.tile_cols; kc = L.tile_kchunk;
            tile = tr * tc;
            tiles_per_row = cols / tc;
        }
    }
    inline uint64_t operator()(uint64_t g) const
    {
        if (!tiled) return g;
        uint64_t t = g / tile, w = g - t * tile;
        uint64_t r, c;
        if (kc) {
            const uint64_t grp = w / (tr * kc), in = w - grp * (tr * kc);
            r = in / kc;
            c = grp * kc + (in - r * kc);
        } else {
            r = w / tc;
            c = w - r * tc;
        }
        uint64_t rb = t / tiles_per_row, cb = t - rb * tiles_per_row;
        return (rb * tr + r) * cols + cb * tc + c;
    }
};

}  // namespace

extern "C" int df11_encode(const uint16_t *bits, uint64_t n, const df11_codebook *cb,
                           const df11_layout *layout_in, df11_encoded **out)
{
    if (!out || !cb || (n && !bits)) return fail(DF11_E_ARG, "df11_encode: null pointer");
    *out = nullptr;
    const df11_layout L = complete_layout(layout_in);
    int rc = check_layout(L, n);
    if (rc) return rc;
    if (cb->fast_bits < DF11_FAST_BITS_MIN || cb->fast_bits > DF11_FAST_BITS_MAX || cb->n_tables < 1 ||
        cb->n_tables > DF11_MAX_TABLES || cb->max_len > DF11_MAX_LEN)
        return fail(DF11_E_ARG, "codebook not built by df11_codebook_build");
    rc = check_counts_fit(L, cb);
    if (rc) return rc;

    const Order order(L);
    const uint64_t chunk_bits = 8ull * L.chunk_bytes;
    const uint64_t lanes = L.seg_lanes;
    const uint64_t seg_bits = chunk_bits * lanes;
    const uint64_t seg_words = seg_bits / 32;

    // pass 1: stream length with block padding, and the uncoded check
    uint64_t pos = 0;
    for (uint64_t g = 0; g < n; g++) {
        if (L.align_elems && g && g % L.align_elems == 0) pos = (pos + seg_bits - 1) / seg_bits * seg_bits;
        uint32_t e = (bits[order(g)] >> 7) & 0xFF;
        if (!cb->len[e]) return fail(DF11_E_UNCODED, "exponent %u of element %llu has no code", e, (unsigned long long)order(g));
        pos += cb->len[e];
    }
    const uint64_t total_bits = pos;
    const uint64_t nseg = (total_bits + seg_bits - 1) / seg_bits;

    df11_encoded *enc = new (std::nothrow) df11_encoded();
    if (!enc) return fail(DF11_E_ALLOC, "out of host memory");
    try {
        enc->exp_words.assign(nseg * seg_words + 2, 0u);
        enc->sm.assign((n + 15) / 16 * 16, 0);
        enc->gaps.assign(nseg * lanes, 0);
        enc->counts.assign(nseg * lanes, 0);
        enc->segs.assign(nseg + 1, df11_segment{0, 0, 0});
        enc->chain.assign(cb->chain, cb->chain + (size_t)cb->n_tables * 256);
        enc->fast.assign(cb->fast, cb->fast + (2u << cb->fast_bits));
        if (L.align_elems) enc->block_seg.assign((n + L.align_elems - 1) / L.align_elems + 1, nseg);
    } catch (...) {
        delete enc;
        return fail(DF11_E_ALLOC, "out of host memory for %llu elements", (unsigned long long)n);
    }
    enc->n = n;
    enc->total_bits = total_bits;
    enc->n_segments = nseg;
    enc->layout = L;
    enc->min_len = cb->min_len;
    enc->max_len = cb->max_len;
    enc->n_tables = cb->n_tables;
    enc->fast_bits = cb->fast_bits;

    uint32_t *W = enc->exp_words.data();
    uint8_t *gaps = enc->gaps.data();
    df11_segment *segs = enc->segs.data();

    // pass 2: codes, sign+mantissa bytes and the per-lane / per-segment records
    uint64_t cs = 0;                 // segment whose codes are being written
    uint64_t next_chunk = 0;         // first chunk of cs without a gap yet
    uint64_t vend = 0;               // end of the last code that starts in cs
    auto close_segment = [&](uint64_t s) {
        const uint64_t s0 = s * seg_bits;
        for (; next_chunk < (s + 1) * lanes; next_chunk++) {
            uint64_t c0 = next_chunk * chunk_bits;
            gaps[next_chunk] = (uint8_t)(c0 < vend ? vend - c0 : 0);
        }
        uint64_t nb = vend > s0 ? vend - s0 : 0;
        segs[s].nbits = (uint32_t)(nb < seg_bits ? nb : seg_bits);
    };
    pos = 0;
    for (uint64_t g = 0; g < n; g++) {
        if (L.align_elems && g && g % L.align_elems == 0) pos = (pos + seg_bits - 1) / seg_bits * seg_bits;
        if (L.align_elems && g % L.align_elems == 0) enc->block_seg[g / L.align_elems] = pos / seg_bits;
        const uint64_t s = pos / seg_bits;
        while (cs < s) {
            close_segment(cs);
            cs++;
            segs[cs].elem_off = g;
            next_chunk = cs * lanes;
            vend = cs * seg_bits;
        }
        while (next_chunk < (cs + 1) * lanes && next_chunk * chunk_bits <= pos) {
            gaps[next_chunk] = (uint8_t)(pos - next_chunk * chunk_bits);
            next_chunk++;
        }
        const uint16_t u = bits[order(g)];
        const uint32_t e = (u >> 7) & 0xFF;
        const uint32_t len = cb->len[e];
        const uint64_t code = cb->code[e];
        const uint64_t w = pos >> 5, off = pos & 31;
        // place the code so that its first bit is bit (31 - off) of word w
        const uint64_t wide = code << (64 - off - len);
        W[w] |= (uint32_t)(wide >> 32);
        W[w + 1] |= (uint32_t)wide;
        enc->sm[g] = (uint8_t)(((u >> 8) & 0x80) | (u & 0x7F));
        enc->counts[pos / chunk_bits]++;
        vend = pos + len;
        pos += len;
    }
    if (nseg) {
        close_segment(cs);
        for (uint64_t s = cs + 1; s < nseg; s++) {
            segs[s].elem_off = n;
            next_chunk = s * lanes;
            vend = s * seg_bits;
            close_segment(s);
        }
    }
    segs[nseg].elem_off = n;
    for (uint64_t s = 0; s < nseg; s++) {
        const uint64_t c = segs[s + 1].elem_off - segs[s].elem_off;
        if (c > enc->max_seg_elems) enc->max_seg_elems = (uint32_t)c;
    }
    df11::row_window(segs, nseg, n, enc->layout, &enc->row_win_lo, &enc->row_win_span);
    *out = enc;
    return DF11_OK;
}

void df11::row_window(const df11_segment *segs, uint64_t n_segments, uint64_t n, const df11_layout &L, int32_t *lo,
                      uint32_t *span)
{
    *lo = 0;
    *span = 0;
    if (!n || !n_segments || !L.rows || !L.cols || L.tile_rows || L.rows * L.cols != n) return;
    const double ratio = (double)n_segments / (double)n;
    int64_t lo_min = INT64_MAX, hi_max = INT64_MIN;
    uint64_t s0 = 0, s1 = 0;   // last segment starting at or before the row's first / last element
    for (uint64_t r = 0; r < L.rows; r++) {
        const uint64_t e0 = r * L.cols, e1 = e0 + L.cols - 1;
        while (s0 + 1 < n_segments && segs[s0 + 1].elem_off <= e0) s0++;
        if (s1 < s0) s1 = s0;
        while (s1 + 1 < n_segments && segs[s1 + 1].elem_off <= e1) s1++;
        const int64_t g = (int64_t)std::floor((double)e0 * ratio);
        lo_min = std::min(lo_min, (int64_t)s0 - g);
        hi_max = std::max(hi_max, (int64_t)s1 - g);
    }
    const int64_t w = hi_max - lo_min + 1;
    if (lo_min < INT32_MIN || lo_min > INT32_MAX || w < 1 || w > (int64_t)UINT32_MAX) return;
    *lo = (int32_t)lo_min;
    *span = (uint32_t)w;
}

extern "C" void df11_encoded_free(df11_encoded *enc) { delete enc; }

extern "C" int df11_encoded_view(const df11_encoded *enc, df11_view *v)
{
    if (!enc || !v) return fail(DF11_E_ARG, "df11_encoded_view: null pointer");
    std::memset(v, 0, sizeof(*v));
    v->n = enc->n;
    v->total_bits = enc->total_bits;
    v->n_segments = enc->n_segments;
    v->chunk_bytes = enc->layout.chunk_bytes;
    v->seg_lanes = enc->layout.seg_lanes;
    v->rows = enc->layout.rows;
    v->cols = enc->layout.cols;
    v->tile_rows = enc->layout.tile_rows;
    v->tile_cols = enc->layout.tile_cols;
    v->tile_kchunk = enc->layout.tile_kchunk;
    v->align_elems = enc->layout.align_elems;
    v->min_len = enc->min_len;
    v->max_len = enc->max_len;
    v->n_tables = enc->n_tables;
    v->fast_bits = enc->fast_bits;
    v->max_seg_elems = enc->max_seg_elems;
    v->row_win_lo = enc->row_win_lo;
    v->row_win_span = enc->row_win_span;
    v->exp_words = enc->exp_words.data();  v->n_exp_words = enc->exp_words.size();
    v->sm = enc->sm.data();                v->n_sm = enc->sm.size();
    v->gaps = enc->gaps.data();            v->n_gaps = enc->gaps.size();
    v->segs = enc->segs.data();            v->n_segs = enc->segs.size();
    v->chain = enc->chain.data();          v->n_chain = enc->chain.size();
    v->fast = enc->fast.data();            v->n_fast = enc->fast.size();
    v->block_seg = enc->block_seg.data();  v->n_block_seg = enc->block_seg.size();
    v->counts = enc->counts.data();        v->n_counts = enc->counts.size();
    return DF11_OK;
}

extern "C" const char *df11_status_string(int status)
{
    switch (status) {
    case DF11_OK: return "ok";
    case DF11_E_ARG: return "invalid argument";
    case DF11_E_UNCODED: return "exponent without a code";
    case DF11_E_CODE_LEN: return "code length limit";
    case DF11_E_FORMAT: return "inconsistent stream or codebook";
    case DF11_E_DEVICE: return "device error";
    case DF11_E_ALLOC: return "allocation failed";
    case DF11_E_UNSUPPORTED: return "unsupported";
    default: return "unknown status";
    }
}

extern "C" const char *df11_last_error(void) { return g_error.c_str(); }

extern "C" const char *df11_version(void) { return "df11-mi355x 0.1"; }
