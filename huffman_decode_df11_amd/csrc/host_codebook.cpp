// Host half of the codec: exponent histogram, length-limited Huffman code,
// canonical codes and the lookup tables the GPU kernels read.
//
// [P1] "DFloat11无损压缩技术：基于哈夫曼编码的BFloat16大模型显存优化方案" 2.2
//      item 1: count every exponent value, give frequent ones short codes.
// [P3] "DFloat11重新定义LLM无损压缩的技术边界" 2.2: decoding goes through a
//      few small hierarchical lookup tables.
#include <algorithm>
#include <cstring>
#include <queue>
#include <vector>

#include "df11_internal.h"

using namespace df11;

extern "C" int df11_hist_accumulate(const uint16_t *bits, uint64_t n, uint64_t hist[256])
{
    if (!hist || (n && !bits)) return fail(DF11_E_ARG, "df11_hist_accumulate: null pointer");
    // four partial histograms break the store-to-load dependence on repeats
    std::vector<uint64_t> part(4 * 256, 0);
    uint64_t i = 0;
    for (; i + 4 <= n; i += 4) {
        part[0 * 256 + ((bits[i + 0] >> 7) & 0xFF)]++;
        part[1 * 256 + ((bits[i + 1] >> 7) & 0xFF)]++;
        part[2 * 256 + ((bits[i + 2] >> 7) & 0xFF)]++;
        part[3 * 256 + ((bits[i + 3] >> 7) & 0xFF)]++;
    }
    for (; i < n; i++) part[(bits[i] >> 7) & 0xFF]++;
    for (int s = 0; s < 256; s++) hist[s] += part[s] + part[256 + s] + part[512 + s] + part[768 + s];
    return DF11_OK;
}

namespace {

// Huffman code lengths with a binary heap keyed on (weight, node order).
int huffman_lengths(const uint64_t *hist, uint8_t *len)
{
    struct Node { uint64_t w; int order; int parent; };
    std::vector<Node> nodes;
    nodes.reserve(512);
    typedef std::pair<uint64_t, int> Key;   // (weight, node index)
    std::priority_queue<Key, std::vector<Key>, std::greater<Key>> heap;
    std::vector<int> leaf_of(256, -1);
    for (int s = 0; s < 256; s++) {
        len[s] = 0;
        if (hist[s]) {
            leaf_of[s] = (int)nodes.size();
            nodes.push_back({hist[s], (int)nodes.size(), -1});
            heap.push({hist[s], leaf_of[s]});
        }
    }
    if (nodes.empty()) return 0;
    if (nodes.size() == 1) {
        for (int s = 0; s < 256; s++) if (hist[s]) len[s] = 1;
        return 1;
    }
    while (heap.size() > 1) {
        Key a = heap.top(); heap.pop();
        Key b = heap.top(); heap.pop();
        int m = (int)nodes.size();
        nodes.push_back({a.first + b.first, m, -1});
        nodes[a.second].parent = m;
        nodes[b.second].parent = m;
        heap.push({a.first + b.first, m});
    }
    int maxlen = 0;
    for (int s = 0; s < 256; s++) {
        if (leaf_of[s] < 0) continue;
        int d = 0;
        for (int v = leaf_of[s]; nodes[v].parent >= 0; v = nodes[v].parent) d++;
        len[s] = (uint8_t)d;
        maxlen = std::max(maxlen, d);
    }
    return maxlen;
}

// Optimal code with lengths <= lmax: package-merge over `lmax` levels.  Each
// list entry remembers whether it is a leaf or a package of two entries of
// the previous level's list; lengths are counted by expanding the first
// 2(n-1) entries of the final list.
int limited_lengths(const uint64_t *hist, int lmax, uint8_t *len)
{
    std::vector<int> sym;
    for (int s = 0; s < 256; s++) { len[s] = 0; if (hist[s]) sym.push_back(s); }
    const int n = (int)sym.size();
    if (n <= 1) { for (int s : sym) len[s] = 1; return n; }
    if (lmax < 31 && (1 << lmax) < n) return -1;
    std::stable_sort(sym.begin(), sym.end(), [&](int a, int b) { return hist[a] < hist[b]; });
    struct Entry { uint64_t w; int leaf; int left; };   // leaf >= 0, or a package of prev[left], prev[left+1]
    std::vector<std::vector<Entry>> level(lmax);
    // level 0 is the deepest (length lmax); each next level packages the previous
    level[0].resize(n);
    for (int i = 0; i < n; i++) level[0][i] = {hist[sym[i]], sym[i], -1};
    for (int d = 1; d < lmax; d++) {
        const std::vector<Entry> &prev = level[d - 1];
        std::vector<Entry> &cur = level[d];
        int np = (int)prev.size() / 2, i = 0, j = 0;
        cur.reserve(n + np);
        while (i < n || j < np) {
            uint64_t pw = j < np ? prev[2 * j].w + prev[2 * j + 1].w : 0;
            if (j >= np || (i < n && hist[sym[i]] <= pw)) { cur.push_back({hist[sym[i]], sym[i], -1}); i++; }
            else { cur.push_back({pw, -1, 2 * j}); j++; }
        }
    }
    // expand the chosen entries level by level: `take` entries of level d
    // contribute one unit of length to every leaf below them
    std::vector<int> count(256, 0);
    int take = 2 * (n - 1);
    for (int d = lmax - 1; d >= 0 && take > 0; d--) {
        int packages = 0;
        for (int k = 0; k < take; k++) {
            const Entry &e = level[d][k];
            if (e.leaf >= 0) count[e.leaf]++;
            else packages++;
        }
        take = 2 * packages;   // packages at level d use the first 2*packages of level d-1
    }
    int maxlen = 0;
    for (int s = 0; s < 256; s++) { len[s] = (uint8_t)count[s]; maxlen = std::max(maxlen, count[s]); }
    return maxlen;
}

// rotate an exponent right by one bit: the low exponent bit lands in bit 7
inline uint32_t rot_exp(uint32_t e) { return ((e >> 1) | (e << 7)) & 0xFFu; }

}  // namespace

namespace df11 {

// Canonical codes, RFC 1951 3.2.2 style: count codes per length, derive the
// first code of every length, hand out codes in exponent order.
void canonical_codes(const uint8_t *len, uint32_t *code)
{
    uint32_t bl_count[DF11_MAX_LEN + 2] = {0};
    uint64_t next_code[DF11_MAX_LEN + 2] = {0};
    for (int s = 0; s < 256; s++) if (len[s]) bl_count[len[s]]++;
    uint64_t c = 0;
    for (int bits = 1; bits <= DF11_MAX_LEN; bits++) {
        c = (c + bl_count[bits - 1]) << 1;
        next_code[bits] = c;
    }
    for (int s = 0; s < 256; s++) code[s] = len[s] ? (uint32_t)next_code[len[s]]++ : 0;
}

// Decode the first code of a left-aligned 32-bit window by walking chain[].
// Returns the entry that ends the walk (a leaf or an "invalid" leaf).
uint16_t chain_walk(const uint16_t *chain, uint32_t window)
{
    uint32_t t = 0;
    for (int level = 0; level < 4; level++) {
        uint16_t e = chain[t * 256 + ((window >> (24 - 8 * level)) & 0xFF)];
        if (!(e & 0x8000)) return e;
        t = e & 0x7FFF;
    }
    return (uint16_t)(32u << 8);
}

int build_tables(df11_codebook *cb)
{
    // hierarchical tables: table 0 covers the first 8 bits; a code longer
    // than 8(level+1) bits links through one more table per 8 bits
    std::memset(cb->chain, 0, sizeof(cb->chain));
    int ntab = 1;
    std::vector<uint8_t> filled(DF11_MAX_TABLES * 256, 0);
    for (int s = 0; s < 256; s++) {
        int L = cb->len[s];
        if (!L) continue;
        uint32_t c = cb->code[s];
        uint32_t t = 0;
        int level = 0;
        while (L > 8 * (level + 1)) {
            uint32_t idx = (c >> (L - 8 * (level + 1))) & 0xFF;
            uint16_t &e = cb->chain[t * 256 + idx];
            if (!filled[t * 256 + idx]) {
                if (ntab >= DF11_MAX_TABLES) return fail(DF11_E_CODE_LEN, "code needs more than %d lookup tables", DF11_MAX_TABLES);
                e = (uint16_t)(0x8000u | (uint32_t)ntab);
                filled[t * 256 + idx] = 1;
                ntab++;
            }
            t = e & 0x7FFF;
            level++;
        }
        int rem = L - 8 * level;               // 1..8 bits left in this table
        uint32_t lo = (c & ((1u << rem) - 1)) << (8 - rem);
        for (uint32_t k = 0; k < (1u << (8 - rem)); k++) {
            cb->chain[t * 256 + lo + k] = (uint16_t)((uint32_t)s | ((uint32_t)L << 8));
            filled[t * 256 + lo + k] = 1;
        }
    }
    // entries no code reaches (an incomplete code, e.g. one symbol) become
    // leaves that consume 32 bits, so every walk terminates
    for (int t = 0; t < ntab; t++)
        for (int k = 0; k < 256; k++)
            if (!filled[t * 256 + k]) cb->chain[t * 256 + k] = (uint16_t)(32u << 8);
    cb->n_tables = (uint32_t)ntab;

    // multi-code table: up to 4 whole codes inside the next fast_bits bits
    const uint32_t K = cb->fast_bits;
    for (uint32_t idx = 0; idx < (1u << K); idx++) {
        uint32_t window = idx << (32 - K);
        uint32_t used = 0, cnt = 0, syms = 0;
        while (cnt < 4) {
            uint32_t w = used < 32 ? window << used : 0;
            uint16_t e = chain_walk(cb->chain, w);
            uint32_t L = (e >> 8) & 0x3F;
            uint32_t s = e & 0xFF;
            if (!cb->len[s] || cb->len[s] != L || L == 0 || used + L > K) break;
            if (((cb->code[s] << (32 - L)) ^ w) >> (32 - L)) break;   // not this code
            syms |= rot_exp(s) << (8 * cnt);
            used += L;
            cnt++;
        }
        cb->fast[2 * idx + 0] = syms;
        cb->fast[2 * idx + 1] = cnt ? ((cnt << 16) - used) : 0u;
    }
    return DF11_OK;
}

}  // namespace df11

extern "C" int df11_codebook_build(const uint64_t hist[256], uint32_t max_len, uint32_t fast_bits,
                                   df11_codebook *cb)
{
    if (!hist || !cb) return fail(DF11_E_ARG, "df11_codebook_build: null pointer");
    if (max_len < 1 || max_len > DF11_MAX_LEN)
        return fail(DF11_E_CODE_LEN, "max_len %u outside 1..%d", max_len, DF11_MAX_LEN);
    if (fast_bits < DF11_FAST_BITS_MIN || fast_bits > DF11_FAST_BITS_MAX)
        return fail(DF11_E_ARG, "fast_bits %u outside %d..%d", fast_bits, DF11_FAST_BITS_MIN, DF11_FAST_BITS_MAX);
    std::memset(cb, 0, sizeof(*cb));
    cb->fast_bits = fast_bits;
    int m = huffman_lengths(hist, cb->len);
    if (m > (int)max_len) {
        m = limited_lengths(hist, (int)max_len, cb->len);
        if (m < 0) return fail(DF11_E_CODE_LEN, "max_len %u too small for the number of exponents", max_len);
    }
    uint32_t nsym = 0, mn = 0;
    for (int s = 0; s < 256; s++)
        if (cb->len[s]) { nsym++; if (!mn || cb->len[s] < mn) mn = cb->len[s]; }
    cb->n_symbols = nsym;
    cb->max_len = (uint32_t)std::max(m, 0);
    cb->min_len = mn;
    canonical_codes(cb->len, cb->code);
    return build_tables(cb);
}
