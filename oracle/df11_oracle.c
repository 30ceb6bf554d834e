/*
 * DF11 CPU ORACLE -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, serial, deliberately slow implementation of what the DFloat11
 * (Dynamic-length Float) codec computes, used only by the tests, the smoke
 * check and the CPU-baseline leg of the benchmark, to check the HIP library.
 * It shares no source with the library (no headers, tables or helpers) and
 * the library never calls it.
 *
 * Sources (the method's description, cited by page title and section):
 *   [P1] "DFloat11无损压缩技术：基于哈夫曼编码的BFloat16大模型显存优化方案"
 *        (jsqmd.com), section 2.1 (BF16 fields) and 2.2 (frequency count,
 *        Huffman code of the exponent, sign and mantissa kept verbatim,
 *        decode on the GPU before the matmul).
 *   [P2] "DFloat11：用于高效 GPU 推理的 LLM 和扩散模型无损压缩"
 *        (gittoolsai.com), section "工作原理" (Huffman-coded BF16 exponent,
 *        bit-for-bit identical outputs).
 *   [P3] "DFloat11重新定义LLM无损压缩的技术边界" (ocdem.com), sections 2.2 and
 *        4.2 (per-thread bit chunks, locate/reconstruct, prefix sum).
 * Where the pages leave a step open, the reading taken is stated at the step.
 *
 * Every function here is pinned by tests against closed forms, brute force,
 * a published worked example (RFC 1951 section 3.2.2) or invariants; none is
 * "parity unpinned".
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- BF16 fields ([P1] 2.1: 1 sign bit, 8 exponent bits, 7 mantissa bits) */
static unsigned bf16_sign(uint16_t u) { return (u >> 15) & 1u; }
static unsigned bf16_exponent(uint16_t u) { return (u >> 7) & 0xFFu; }
static unsigned bf16_mantissa(uint16_t u) { return u & 0x7Fu; }

/* ---- exponent histogram ([P1] 2.2 item 1: count how often every exponent
 * value occurs over all weights; exact, every element counted). */
void orc_histogram(const uint16_t *u, uint64_t n, uint64_t *hist)
{
    for (int s = 0; s < 256; s++) hist[s] = 0;
    for (uint64_t i = 0; i < n; i++) hist[bf16_exponent(u[i])] += 1;
}

/* ---- Huffman code lengths ([P1] 2.2 item 1, [P2] "工作原理").
 * Textbook construction: start with one node per exponent that occurs,
 * repeatedly join the two nodes of lowest weight (ties: lower node id, where
 * a leaf's id is its exponent value and the k-th joined node gets 256 + k),
 * and read each leaf's depth.  One occurring symbol gets length 1.
 * Returns the longest length, 0 when nothing occurs. */
int orc_huffman_lengths(const uint64_t *hist, uint8_t *len)
{
    uint64_t weight[511];
    int parent[511], alive[511];
    int nodes = 256, nsym = 0, last = -1;
    for (int s = 0; s < 256; s++) {
        len[s] = 0;
        weight[s] = hist[s];
        parent[s] = -1;
        alive[s] = hist[s] > 0;
        if (alive[s]) { nsym++; last = s; }
    }
    if (nsym == 0) return 0;
    if (nsym == 1) { len[last] = 1; return 1; }
    for (int step = 0; step < nsym - 1; step++) {
        int a = -1, b = -1;
        for (int i = 0; i < nodes; i++) {
            if (!alive[i]) continue;
            if (a < 0 || weight[i] < weight[a]) { b = a; a = i; }
            else if (b < 0 || weight[i] < weight[b]) { b = i; }
        }
        int m = nodes++;
        weight[m] = weight[a] + weight[b];
        parent[m] = -1;
        alive[m] = 1;
        alive[a] = alive[b] = 0;
        parent[a] = parent[b] = m;
    }
    int maxlen = 0;
    for (int s = 0; s < 256; s++) {
        if (!hist[s]) continue;
        int d = 0;
        for (int v = s; parent[v] >= 0; v = parent[v]) d++;
        len[s] = (uint8_t)d;
        if (d > maxlen) maxlen = d;
    }
    return maxlen;
}

/* ---- length-limited optimal code: package-merge (Larmore and Hirschberg,
 * 1990), in its coin-collector form.  The pages do not say how codes are
 * kept within a maximum length; this reading takes the optimal limited code.
 * Items carry a per-symbol multiplicity; a symbol's length is how many of the
 * first 2(n-1) items of the final list contain it.  Returns the longest
 * length, or -1 when 2^lmax < number of occurring symbols. */
typedef struct { uint64_t w; uint8_t cnt[256]; } orc_item;

int orc_package_merge(const uint64_t *hist, int lmax, uint8_t *len)
{
    int nsym = 0;
    for (int s = 0; s < 256; s++) { len[s] = 0; if (hist[s]) nsym++; }
    if (nsym == 0) return 0;
    if (nsym == 1) { for (int s = 0; s < 256; s++) if (hist[s]) len[s] = 1; return 1; }
    if (lmax < 31 && (1 << lmax) < nsym) return -1;
    /* leaves sorted by weight (stable on symbol value) */
    orc_item *leaves = (orc_item *)calloc((size_t)nsym, sizeof(orc_item));
    orc_item *list = (orc_item *)calloc((size_t)2 * nsym, sizeof(orc_item));
    orc_item *next = (orc_item *)calloc((size_t)2 * nsym, sizeof(orc_item));
    int k = 0;
    for (int s = 0; s < 256; s++)
        if (hist[s]) { leaves[k].w = hist[s]; leaves[k].cnt[s] = 1; k++; }
    /* insertion sort keeps equal weights in symbol order */
    for (int i = 1; i < nsym; i++) {
        orc_item t = leaves[i];
        int j = i - 1;
        while (j >= 0 && leaves[j].w > t.w) { leaves[j + 1] = leaves[j]; j--; }
        leaves[j + 1] = t;
    }
    int nl = nsym;
    memcpy(list, leaves, sizeof(orc_item) * (size_t)nsym);
    for (int level = 1; level < lmax; level++) {
        /* package adjacent pairs of the current list */
        int np = nl / 2, nn = 0, i = 0, j = 0;
        orc_item *pk = (orc_item *)calloc((size_t)(np ? np : 1), sizeof(orc_item));
        for (int p = 0; p < np; p++) {
            pk[p].w = list[2 * p].w + list[2 * p + 1].w;
            for (int s = 0; s < 256; s++)
                pk[p].cnt[s] = (uint8_t)(list[2 * p].cnt[s] + list[2 * p + 1].cnt[s]);
        }
        /* merge the leaves with the packages (leaves first on ties) */
        while (i < nsym || j < np) {
            if (j >= np || (i < nsym && leaves[i].w <= pk[j].w)) next[nn++] = leaves[i++];
            else next[nn++] = pk[j++];
        }
        free(pk);
        orc_item *t = list; list = next; next = t;
        nl = nn;
    }
    int take = 2 * (nsym - 1), maxlen = 0;
    for (int i = 0; i < take && i < nl; i++)
        for (int s = 0; s < 256; s++) len[s] = (uint8_t)(len[s] + list[i].cnt[s]);
    for (int s = 0; s < 256; s++) if (len[s] > maxlen) maxlen = len[s];
    free(leaves); free(list); free(next);
    return maxlen;
}

/* Huffman lengths, replaced by the optimal limited code only when the
 * Huffman code is longer than lmax. */
int orc_code_lengths(const uint64_t *hist, int lmax, uint8_t *len)
{
    int m = orc_huffman_lengths(hist, len);
    if (m <= lmax) return m;
    return orc_package_merge(hist, lmax, len);
}

/* ---- canonical codes.  The pages say only that frequent exponents get short
 * codes.  Reading: canonical code in (length, symbol) order, as in
 * RFC 1951 section 3.2.2: the first code is all zeros, and each next code is
 * the previous one plus one, shifted left by the growth in length. */
void orc_canonical_codes(const uint8_t *len, uint32_t *code)
{
    int order[256], k = 0;
    for (int l = 1; l <= 32; l++)
        for (int s = 0; s < 256; s++)
            if (len[s] == l) order[k++] = s;
    for (int s = 0; s < 256; s++) code[s] = 0;
    uint64_t c = 0;
    for (int i = 0; i < k; i++) {
        if (i > 0) c = (c + 1) << (len[order[i]] - len[order[i - 1]]);
        code[order[i]] = (uint32_t)c;
    }
}

/* ---- sign+mantissa byte ([P1] 2.2 item 2: sign and 7 mantissa bits stored
 * unchanged).  Reading: the sign in bit 7 and the mantissa in bits 6..0. */
void orc_sign_mantissa(const uint16_t *u, uint64_t n, uint8_t *sm)
{
    for (uint64_t i = 0; i < n; i++)
        sm[i] = (uint8_t)((bf16_sign(u[i]) << 7) | bf16_mantissa(u[i]));
}

/* ---- code start positions in the exponent bitstream.  Codes are laid end
 * to end in element order.  When align_elems > 0 the codes of element
 * align_elems*b start on the next multiple of seg_bits (zero bits pad the
 * gap), so every block of align_elems elements begins a segment.
 * Returns the total number of bits (end of the last code). */
uint64_t orc_code_starts(const uint16_t *u, uint64_t n, const uint8_t *len,
                         uint64_t seg_bits, uint64_t align_elems, uint64_t *start)
{
    uint64_t pos = 0;
    for (uint64_t i = 0; i < n; i++) {
        if (align_elems && i > 0 && i % align_elems == 0)
            pos = (pos + seg_bits - 1) / seg_bits * seg_bits;
        start[i] = pos;
        pos += len[bf16_exponent(u[i])];
    }
    return pos;
}

/* ---- exponent bitstream: every code written most significant bit first at
 * its start position, bytes filled from bit 7 down.  E must hold
 * ceil(total_bits / 8) zeroed bytes. */
void orc_write_stream(const uint16_t *u, uint64_t n, const uint8_t *len,
                      const uint32_t *code, const uint64_t *start, uint8_t *E)
{
    for (uint64_t i = 0; i < n; i++) {
        unsigned e = bf16_exponent(u[i]);
        for (int b = 0; b < len[e]; b++) {
            unsigned bit = (code[e] >> (len[e] - 1 - b)) & 1u;
            uint64_t p = start[i] + (uint64_t)b;
            if (bit) E[p >> 3] |= (uint8_t)(0x80u >> (p & 7));
        }
    }
}

/* ---- decode: walk the bitstream one bit at a time with the canonical
 * first-code-per-length rule (a different algorithm from table lookup), then
 * rebuild each BF16 word from its sign+mantissa byte and decoded exponent.
 * Returns 0, or -1 on a bit pattern that is no code. */
int orc_decode(const uint8_t *E, uint64_t nbits, const uint8_t *sm, uint64_t n,
               const uint8_t *len, uint64_t seg_bits, uint64_t align_elems,
               uint16_t *out)
{
    int count[33] = {0}, order[256], k = 0;
    uint32_t first[33];
    for (int s = 0; s < 256; s++) if (len[s]) count[len[s]]++;
    for (int l = 1; l <= 32; l++)
        for (int s = 0; s < 256; s++) if (len[s] == l) order[k++] = s;
    /* first canonical code of each length, and index of its symbol in order[] */
    int offset[33];
    uint64_t c = 0;
    int idx = 0;
    for (int l = 1; l <= 32; l++) {
        first[l] = (uint32_t)c;
        offset[l] = idx;
        idx += count[l];
        c = (c + (uint64_t)count[l]) << 1;
    }
    uint64_t pos = 0;
    for (uint64_t i = 0; i < n; i++) {
        if (align_elems && i > 0 && i % align_elems == 0)
            pos = (pos + seg_bits - 1) / seg_bits * seg_bits;
        uint64_t v = 0;
        int sym = -1;
        for (int l = 1; l <= 32; l++) {
            if (pos >= nbits) return -1;
            v = (v << 1) | ((E[pos >> 3] >> (7 - (pos & 7))) & 1u);
            pos++;
            if (count[l] && v >= first[l] && v - first[l] < (uint64_t)count[l]) {
                sym = order[offset[l] + (int)(v - first[l])];
                break;
            }
        }
        if (sym < 0) return -1;
        out[i] = (uint16_t)(((unsigned)(sm[i] & 0x80) << 8) | ((unsigned)sym << 7) | (sm[i] & 0x7Fu));
    }
    return 0;
}

/* ---- per-lane gaps and per-segment element offsets.  The stream is cut
 * into segments of seg_bits bits, each cut into lanes of chunk_bits bits.
 * valid_end[s] is where the codes that start in segment s stop (the end of
 * the last code of segment s's element block).  A lane owns the codes that
 * start in [chunk start + gap, min(chunk end, valid end)).  gap is the
 * distance from the chunk start to the first code start at or after it,
 * capped at the valid end, and 0 for chunks that begin at or past it.
 * seg_elem[s] counts the codes that start before segment s's first bit;
 * seg_elem[nseg] = n.  seg_nbits[s] = valid end - segment start, at most
 * seg_bits. */
void orc_metadata(const uint64_t *start, const uint16_t *u, uint64_t n,
                  const uint8_t *len, uint64_t chunk_bits, uint64_t seg_bits,
                  uint64_t nseg, uint8_t *gaps, uint64_t *seg_elem,
                  uint32_t *seg_nbits)
{
    uint64_t lanes = seg_bits / chunk_bits;
    uint64_t i = 0;
    for (uint64_t s = 0; s < nseg; s++) {
        uint64_t s0 = s * seg_bits;
        while (i < n && start[i] < s0) i++;
        seg_elem[s] = i;
        /* valid end: the end of the last code that starts in this segment */
        uint64_t j = i, vend = s0;
        while (j < n && start[j] < s0 + seg_bits) {
            vend = start[j] + len[bf16_exponent(u[j])];
            j++;
        }
        uint64_t nb = vend > s0 ? vend - s0 : 0;
        seg_nbits[s] = (uint32_t)(nb < seg_bits ? nb : seg_bits);
        uint64_t q = i;
        for (uint64_t l = 0; l < lanes; l++) {
            uint64_t c0 = s0 + l * chunk_bits;
            uint64_t g = 0;
            if (c0 < vend) {
                while (q < j && start[q] < c0) q++;
                uint64_t firststart = (q < j) ? start[q] : vend;
                g = firststart - c0;
            }
            gaps[s * lanes + l] = (uint8_t)g;
        }
    }
    seg_elem[nseg] = n;
}

/* ---- per-lane code counts: counts[c] = the number of codes whose first bit
 * lies in chunk c, i.e. in [c * chunk_bits, (c + 1) * chunk_bits), for the
 * nchunks chunks of the stream.  (The lane that owns chunk c decodes exactly
 * these codes; storing the count spares the decoder a counting pass.)  A
 * count is stored in one byte: if any chunk holds more than 255 codes the
 * layout cannot carry its counts, and the function returns -1 (counts then
 * hold nothing meaningful) instead of storing a wrapped value; else 0. */
int orc_chunk_counts(const uint64_t *start, uint64_t n, uint64_t chunk_bits, uint64_t nchunks,
                     uint8_t *counts)
{
    for (uint64_t c = 0; c < nchunks; c++) counts[c] = 0;
    for (uint64_t i = 0; i < n; i++) {
        uint64_t c = start[i] / chunk_bits;
        if (c >= nchunks) continue;
        if (counts[c] == 255) return -1;
        counts[c] = (uint8_t)(counts[c] + 1);
    }
    return 0;
}

/* ---- matrix product that consumes the decoded weights ([P1] 2.2 item 3:
 * decoded BF16 weights feed the matmul).  Y[b][j] = sum_k X[b][k] * W[j][k]
 * with W in nn.Linear layout [N, K].  BF16 operands widen exactly to float;
 * the sum runs over k in order, in float (orc_gemm_f32) or double
 * (orc_gemm_f64). */
static float bf16_to_f32(uint16_t h)
{
    uint32_t w = (uint32_t)h << 16;
    float f;
    memcpy(&f, &w, 4);
    return f;
}

void orc_gemm_f32(const uint16_t *X, const uint16_t *W, uint64_t B, uint64_t N,
                  uint64_t K, float *Y)
{
    for (uint64_t b = 0; b < B; b++)
        for (uint64_t j = 0; j < N; j++) {
            float acc = 0.0f;
            for (uint64_t k = 0; k < K; k++)
                acc += bf16_to_f32(X[b * K + k]) * bf16_to_f32(W[j * K + k]);
            Y[b * N + j] = acc;
        }
}

void orc_gemm_f64(const uint16_t *X, const uint16_t *W, uint64_t B, uint64_t N,
                  uint64_t K, double *Y)
{
    for (uint64_t b = 0; b < B; b++)
        for (uint64_t j = 0; j < N; j++) {
            double acc = 0.0;
            for (uint64_t k = 0; k < K; k++)
                acc += (double)bf16_to_f32(X[b * K + k]) * (double)bf16_to_f32(W[j * K + k]);
            Y[b * N + j] = acc;
        }
}

/* ---- element order for tiled streams: a [rows, cols] matrix cut into
 * tile_rows x tile_cols tiles, tiles taken row-block by row-block.  Inside a
 * tile the elements go row-major (kc = 0), or, with kc > 0, in column groups
 * of kc: group by group, each group row by row, kc elements per row. */
void orc_tile_order(const uint16_t *u, uint64_t rows, uint64_t cols,
                    uint64_t tr, uint64_t tc, uint64_t kc, uint16_t *out)
{
    uint64_t k = 0;
    for (uint64_t rb = 0; rb < rows / tr; rb++)
        for (uint64_t cb = 0; cb < cols / tc; cb++) {
            if (!kc) {
                for (uint64_t r = 0; r < tr; r++)
                    for (uint64_t c = 0; c < tc; c++)
                        out[k++] = u[(rb * tr + r) * cols + cb * tc + c];
            } else {
                for (uint64_t g = 0; g < tc / kc; g++)
                    for (uint64_t r = 0; r < tr; r++)
                        for (uint64_t c = 0; c < kc; c++)
                            out[k++] = u[(rb * tr + r) * cols + cb * tc + g * kc + c];
            }
        }
}
