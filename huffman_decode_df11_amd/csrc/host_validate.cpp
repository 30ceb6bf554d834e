// df11_validate: O(n) CPU structural check of an encoded tensor.  It rebuilds
// the tables from the code lengths, walks every segment's codes and compares
// the gaps and segment records with what the walk finds.  It never produces
// decoded weights; decoding is the GPU's job.
#include <cstring>
#include <vector>

#include "df11_internal.h"

using namespace df11;

namespace {

inline uint32_t window_at(const uint32_t *w, uint64_t nwords, uint64_t pos)
{
    uint64_t i = pos >> 5, off = pos & 31;
    uint64_t hi = i < nwords ? w[i] : 0, lo = i + 1 < nwords ? w[i + 1] : 0;
    return (uint32_t)(((hi << 32) | lo) << off >> 32);
}

}  // namespace

extern "C" int df11_validate(const df11_view *v, const df11_codebook *cb)
{
    if (!v || !cb) return fail(DF11_E_ARG, "df11_validate: null pointer");
    if (v->n && (!v->exp_words || !v->sm || !v->gaps || (v->n_counts && !v->counts) || !v->segs || !v->chain || !v->fast))
        return fail(DF11_E_ARG, "df11_validate: null array in view");
    // codebook: lengths, Kraft sum, canonical codes and tables
    uint64_t kraft = 0;   // in units of 2^-32
    for (int s = 0; s < 256; s++) {
        if (cb->len[s] > DF11_MAX_LEN) return fail(DF11_E_FORMAT, "length %u of exponent %d > 32", cb->len[s], s);
        if (cb->len[s]) kraft += 1ull << (32 - cb->len[s]);
    }
    if (kraft > (1ull << 32)) return fail(DF11_E_FORMAT, "code lengths violate the Kraft inequality");
    df11_codebook ref;
    std::memcpy(ref.len, cb->len, sizeof ref.len);
    ref.fast_bits = cb->fast_bits;
    if (ref.fast_bits < DF11_FAST_BITS_MIN || ref.fast_bits > DF11_FAST_BITS_MAX)
        return fail(DF11_E_FORMAT, "fast_bits %u out of range", ref.fast_bits);
    canonical_codes(ref.len, ref.code);
    if (std::memcmp(ref.code, cb->code, sizeof ref.code)) return fail(DF11_E_FORMAT, "codes are not the canonical codes of the lengths");
    if (build_tables(&ref)) return fail(DF11_E_FORMAT, "tables cannot be built");
    if (v->n_tables != ref.n_tables || v->n_chain != (uint64_t)ref.n_tables * 256 ||
        std::memcmp(v->chain, ref.chain, sizeof(uint16_t) * ref.n_tables * 256))
        return fail(DF11_E_FORMAT, "hierarchical tables differ from the codebook's");
    if (v->fast_bits != ref.fast_bits || v->n_fast != (2ull << ref.fast_bits) ||
        std::memcmp(v->fast, ref.fast, sizeof(uint32_t) * (2ull << ref.fast_bits)))
        return fail(DF11_E_FORMAT, "multi-code table differs from the codebook's");

    // sizes
    if (v->seg_lanes != DF11_SEG_LANES || v->chunk_bytes < 4 || v->chunk_bytes > 32 || v->chunk_bytes % 4)
        return fail(DF11_E_FORMAT, "layout chunk_bytes %u / seg_lanes %u", v->chunk_bytes, v->seg_lanes);
    const uint64_t chunk_bits = 8ull * v->chunk_bytes, lanes = v->seg_lanes;
    const uint64_t seg_bits = chunk_bits * lanes, seg_words = seg_bits / 32;
    if (v->n_segments != (v->total_bits + seg_bits - 1) / seg_bits)
        return fail(DF11_E_FORMAT, "n_segments %llu does not match total_bits", (unsigned long long)v->n_segments);
    if (v->n_exp_words < v->n_segments * seg_words + 2 || v->n_sm < (v->n + 15) / 16 * 16 ||
        v->n_gaps != v->n_segments * lanes || (v->n_counts && v->n_counts != v->n_segments * lanes) ||
        v->n_segs != v->n_segments + 1)
        return fail(DF11_E_FORMAT, "array sizes do not match n and n_segments");
    if (v->segs[0].elem_off != 0 || v->segs[v->n_segments].elem_off != v->n)
        return fail(DF11_E_FORMAT, "first/last segment record must be 0 / n");

    // aligned blocks: each block's first element opens its first segment
    if (v->align_elems) {
        const uint64_t nb = (v->n + v->align_elems - 1) / v->align_elems;
        if (v->n_block_seg != nb + 1 || !v->block_seg) return fail(DF11_E_FORMAT, "block_seg size");
        if (v->block_seg[nb] != v->n_segments) return fail(DF11_E_FORMAT, "block_seg must end with n_segments");
        for (uint64_t b = 0; b < nb; b++) {
            const uint64_t s = v->block_seg[b];
            if (s > v->block_seg[b + 1] || s >= v->n_segments || v->segs[s].elem_off != b * v->align_elems ||
                v->gaps[s * lanes] != 0)
                return fail(DF11_E_FORMAT, "block %llu does not open segment %llu", (unsigned long long)b,
                            (unsigned long long)s);
        }
    } else if (v->n_block_seg) {
        return fail(DF11_E_FORMAT, "block_seg given without align_elems");
    }
    // walk every segment
    std::vector<uint32_t> count(lanes);
    for (uint64_t s = 0; s < v->n_segments; s++) {
        const uint64_t s0 = s * seg_bits;
        const df11_segment &sg = v->segs[s];
        if (sg.elem_off > v->segs[s + 1].elem_off)
            return fail(DF11_E_FORMAT, "segment %llu: element offsets decrease", (unsigned long long)s);
        if (sg.nbits > seg_bits) return fail(DF11_E_FORMAT, "segment %llu: nbits > segment size", (unsigned long long)s);
        const uint64_t want = v->segs[s + 1].elem_off - sg.elem_off;
        const uint64_t vend = s0 + sg.nbits;
        uint64_t got = 0;
        for (uint64_t l = 0; l < lanes; l++) {
            const uint64_t c0 = s0 + l * chunk_bits, c1 = c0 + chunk_bits;
            const uint32_t gap = v->gaps[s * lanes + l];
            if (c0 >= vend) {
                if (gap) return fail(DF11_E_FORMAT, "segment %llu lane %llu: gap past the segment's codes", (unsigned long long)s, (unsigned long long)l);
                if (v->n_counts && v->counts[s * lanes + l])
                    return fail(DF11_E_FORMAT, "segment %llu lane %llu: count past the segment's codes", (unsigned long long)s, (unsigned long long)l);
                continue;
            }
            if (gap >= 32) return fail(DF11_E_FORMAT, "segment %llu lane %llu: gap %u >= 32", (unsigned long long)s, (unsigned long long)l, gap);
            // the previous lane's last code must end exactly where this lane starts
            uint64_t p = c0 + gap;
            const uint64_t end = c1 < vend ? c1 : vend;
            const uint64_t got0 = got;
            while (p < end) {
                uint16_t e = chain_walk(v->chain, window_at(v->exp_words, v->n_exp_words, p));
                uint32_t L = (e >> 8) & 0x3F;
                if (!L || cb->len[e & 0xFF] != L)
                    return fail(DF11_E_FORMAT, "segment %llu: bit %llu starts no code", (unsigned long long)s, (unsigned long long)p);
                p += L;
                got++;
            }
            if (v->n_counts && got - got0 != v->counts[s * lanes + l])
                return fail(DF11_E_FORMAT, "segment %llu lane %llu: %llu codes start in the chunk, count says %u",
                            (unsigned long long)s, (unsigned long long)l, (unsigned long long)(got - got0),
                            v->counts[s * lanes + l]);
            if (l + 1 < lanes && c1 < vend && p != c1 + v->gaps[s * lanes + l + 1])
                return fail(DF11_E_FORMAT, "segment %llu lane %llu: codes do not meet the next lane's gap", (unsigned long long)s, (unsigned long long)l);
            if (c1 >= vend && sg.nbits < seg_bits && p != vend)
                return fail(DF11_E_FORMAT, "segment %llu: last code does not end at nbits", (unsigned long long)s);
        }
        if (want > v->max_seg_elems)
            return fail(DF11_E_FORMAT, "segment %llu holds more codes than max_seg_elems", (unsigned long long)s);
        if (got != want)
            return fail(DF11_E_FORMAT, "segment %llu holds %llu codes but its records say %llu",
                        (unsigned long long)s, (unsigned long long)got, (unsigned long long)want);
    }
    return DF11_OK;
}
