// Device building blocks shared by the decode and fused decode+GEMM kernels.
//
// One 64-lane wavefront decodes one segment of the exponent stream:
//   stage   the segment's words go to LDS in reversed word order;
//   locate  every lane counts the codes that start in its chunk ([P3]
//           "DFloat11重新定义LLM无损压缩的技术边界" 2.2 Phase 1), reading the
//           multi-code table and, for long codes, the hierarchical tables;
//   scan    a wavefront prefix sum turns counts into output positions
//           ([P3] 2.2 prefix sum);
//   emit    every lane decodes its chunk again and writes each exponent
//           (rotated right by one bit) to its output slot in LDS ([P3] 2.2
//           Phase 2);
// after which the caller merges the staged exponents with the sign+mantissa
// bytes ([P1] "DFloat11无损压缩技术：基于哈夫曼编码的BFloat16大模型显存优化方案"
// 2.2 item 2) into BF16.
//
// Bit cursor.  A lane keeps one 32-bit state word: bits 0..15 hold
// kM0 - p for stream position p (bits from the segment start) and bits
// 16..31 hold a count or an LDS byte address.  A multi-code table entry's
// meta = (codes << 16) - bits, so `state += meta` advances both halves.
// With the segment's words stored reversed in LDS, the 32-bit window at p is
// alignbit(word[(p-1)>>5], word[((p-1)>>5)+1], -p), whose two words are
// adjacent in LDS at an address linear in (state >> 5) & 0x7FF.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace df11dev {

constexpr uint32_t kM0 = 65504;          // multiple of 32, above any segment size
constexpr uint32_t kQ = kM0 / 32;

__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }

// LDS byte pointer helpers (generic pointers into __shared__ memory)
__device__ __forceinline__ uint32_t lds_u32(const uint8_t *lds, uint32_t byte_addr)
{
    return *reinterpret_cast<const uint32_t *>(lds + byte_addr);
}

struct SegWindow {
    const uint8_t *lds;    // base of dynamic LDS
    uint32_t rbase;        // byte address such that word[(p-1)>>5] sits at rbase + 4*((state>>5)&0x7FF) + 4
    __device__ __forceinline__ uint32_t operator()(uint32_t st) const
    {
        const uint32_t d = __builtin_amdgcn_ubfe(st, 5, 11);
        const uint32_t a = rbase + 4u * d;
        const uint32_t w_next = lds_u32(lds, a);        // word[a'+1]
        const uint32_t w_cur = lds_u32(lds, a + 4);     // word[a']
        return __builtin_amdgcn_alignbit(w_cur, w_next, st);
    }
};

// First code of a window through the hierarchical tables in LDS.  Returns
// exponent | length << 8; a malformed walk yields length 32.
__device__ __forceinline__ uint32_t chain_decode(const uint16_t *chain, uint32_t win)
{
    uint32_t e = chain[win >> 24];
    if (e & 0x8000u) {
        e = chain[(e & 0x7FFFu) * 256u + ((win >> 16) & 0xFFu)];
        if (e & 0x8000u) {
            e = chain[(e & 0x7FFFu) * 256u + ((win >> 8) & 0xFFu)];
            if (e & 0x8000u) {
                e = chain[(e & 0x7FFFu) * 256u + (win & 0xFFu)];
                if (e & 0x8000u) e = 32u << 8;
            }
        }
    }
    if (!(e & 0x3F00u)) e = 32u << 8;   // never advance by zero bits
    return e;
}

__device__ __forceinline__ uint32_t rot_exp(uint32_t e) { return ((e >> 1) | (e << 7)) & 0xFFu; }

// Stage one segment's words into LDS in reversed order.  region: LDS byte
// offset of a (seg_words + 8)-word, 16-byte aligned region.  Word i of the
// segment lands at word index K0 - i with K0 = region/4 + 3 + seg_words;
// word seg_words (the next segment's first word, read as look-ahead) at
// region/4 + 3 and the guard word[-1] at K0 + 1.  Returns rbase.
template <int CB>
__device__ __forceinline__ uint32_t stage_segment(uint8_t *lds, uint32_t region,
                                                  const uint32_t *__restrict__ words,
                                                  uint64_t seg)
{
    constexpr uint32_t kWordsPerLane = CB / 4;
    constexpr uint32_t kSegWords = 64 * kWordsPerLane;
    const uint32_t lane = lane_id();
    const uint32_t *src = words + seg * kSegWords + lane * kWordsPerLane;
    const uint32_t k0 = region / 4 + 3 + kSegWords;
    uint32_t *ldsw = reinterpret_cast<uint32_t *>(lds);
    if constexpr (kWordsPerLane == 4) {
        const uint4 v = *reinterpret_cast<const uint4 *>(src);
        // words 4l..4l+3 go to k0-4l-3 .. k0-4l, i.e. reversed inside the uint4
        *reinterpret_cast<uint4 *>(ldsw + (k0 - 4 * lane - 3)) = make_uint4(v.w, v.z, v.y, v.x);
    } else {
#pragma unroll
        for (uint32_t i = 0; i < kWordsPerLane; i++) ldsw[k0 - kWordsPerLane * lane - i] = src[i];
    }
    if (lane == 0) {
        ldsw[k0 - kSegWords] = words[(seg + 1) * kSegWords];
        ldsw[k0 + 1] = 0;
    }
    // word[a'] for state st is at k0 - (kQ - 1 - d); the pair read starts one word lower
    return 4u * (k0 - kQ);
}

// Wavefront-scope ordering of LDS traffic between lanes of one wave.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Locate: number of codes starting in [p0, end).
template <int K>
__device__ __forceinline__ uint32_t count_codes(const SegWindow &win, const uint2 *fast,
                                                const uint16_t *chain, uint32_t p0, uint32_t end)
{
    uint32_t st = kM0 - p0;
    const uint32_t lim = kM0 - end;            // p < end  <=>  (st & 0xFFFF) > lim
    uint32_t meta = 0;
    while ((st & 0xFFFFu) > lim) {
        const uint32_t w = win(st);
        meta = fast[w >> (32 - K)].y;
        if (meta == 0) meta = (1u << 16) - ((chain_decode(chain, w) >> 8) & 0x3Fu);
        st += meta;
    }
    // the last lookup may have counted codes that start at or past `end`:
    // step back and redo it one code at a time
    st -= meta;
    while ((st & 0xFFFFu) > lim) {
        const uint32_t w = win(st);
        st += (1u << 16) - ((chain_decode(chain, w) >> 8) & 0x3Fu);
    }
    return st >> 16;
}

// Emit: decode `cnt` codes from p0 and write their rotated exponents to LDS
// bytes [wpos, wpos + cnt).  wpos + cnt must be below 65536.
template <int K>
__device__ __forceinline__ void emit_codes(const SegWindow &win, const uint2 *fast,
                                           const uint16_t *chain, uint8_t *lds, uint32_t p0,
                                           uint32_t wpos, uint32_t cnt)
{
    uint32_t st = (kM0 - p0) | (wpos << 16);
    const uint32_t bound = (wpos + cnt - 3u) << 16;   // st < bound <=> at least 4 codes left
    while (st < bound) {
        const uint32_t w = win(st);
        const uint2 f = fast[w >> (32 - K)];
        uint32_t syms = f.x, meta = f.y;
        if (meta == 0) {
            const uint32_t e = chain_decode(chain, w);
            syms = rot_exp(e & 0xFFu);
            meta = (1u << 16) - ((e >> 8) & 0x3Fu);
        }
        uint8_t *dst = lds + (st >> 16);
        dst[0] = (uint8_t)syms;
        dst[1] = (uint8_t)(syms >> 8);
        dst[2] = (uint8_t)(syms >> 16);
        dst[3] = (uint8_t)(syms >> 24);
        st += meta;
    }
    const uint32_t lend = wpos + cnt;
    while ((st >> 16) < lend) {
        const uint32_t e = chain_decode(chain, win(st));
        lds[st >> 16] = (uint8_t)rot_exp(e & 0xFFu);
        st += (1u << 16) - ((e >> 8) & 0x3Fu);
    }
}

// Exclusive prefix sum over the wavefront; *total receives the sum.
__device__ __forceinline__ uint32_t wave_exclusive_scan(uint32_t x, uint32_t *total)
{
    const uint32_t lane = lane_id();
    uint32_t v = x;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t y = __shfl_up(v, d, 64);
        if (lane >= (uint32_t)d) v += y;
    }
    *total = __builtin_amdgcn_readlane(v, 63);
    return v - x;
}

// Merge 4 sign+mantissa bytes with 4 rotated exponents into 4 BF16 words.
__device__ __forceinline__ uint2 assemble4(uint32_t sm, uint32_t rx)
{
    const uint32_t hi = (sm & 0x80808080u) | (rx & 0x7F7F7F7Fu);   // sign | exponent >> 1
    const uint32_t lo = (rx & 0x80808080u) | (sm & 0x7F7F7F7Fu);   // exponent bit 0 | mantissa
    return make_uint2(__builtin_amdgcn_perm(hi, lo, 0x05010400u), __builtin_amdgcn_perm(hi, lo, 0x07030602u));
}

__device__ __forceinline__ uint16_t assemble1(uint32_t sm, uint32_t rx)
{
    const uint32_t hi = (sm & 0x80u) | (rx & 0x7Fu);
    const uint32_t lo = (rx & 0x80u) | (sm & 0x7Fu);
    return (uint16_t)((hi << 8) | lo);
}

}  // namespace df11dev
