// Device building blocks shared by the decode and fused decode+GEMM kernels.
//
// One 64-lane wavefront decodes one segment of the exponent stream:
//   load    every lane holds its chunk of four stream words plus the next
//           chunk's first word (160 bits) in registers;
//   locate  every lane learns how many codes start in its chunk ([P3]
//           "DFloat11重新定义LLM无损压缩的技术边界" 2.2 Phase 1): the count
//           stored with the chunk's gap, or, for an encoding without
//           counts, by walking the chunk through the multi-code table and,
//           for long codes, the hierarchical tables (count_codes);
//   scan    a wavefront prefix sum turns counts into output positions
//           ([P3] 2.2 prefix sum);
//   emit    every lane decodes its chunk again and writes each exponent
//           (rotated right by one bit) to its output slot in LDS ([P3] 2.2
//           Phase 2);
// after which the caller merges the staged exponents with the sign+mantissa
// bytes ([P1] "DFloat11无损压缩技术：基于哈夫曼编码的BFloat16大模型显存优化方案"
// 2.2 item 2) into BF16.
//
// Bit window.  The chunk plus one look-ahead word live in registers, most
// significant first (160 bits in five registers for 16-byte chunks);
// consuming b bits shifts them all left with v_alignbit_b32 by (32 - b) mod 32,
// which is exactly the low five bits of the table word meta = (codes << 16) - b,
// so a lookup costs one LDS read and no address arithmetic on the stream.
// Cursor.  A lane keeps one 32-bit state word: bits 0..15 hold kM0 - p for
// the bit position p in its chunk, bits 16..31 a count or an LDS byte
// address; `state += meta` advances both halves at once.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace df11dev {

constexpr uint32_t kM0 = 65504;          // multiple of 32, above any chunk size
constexpr uint32_t kQ = kM0 / 32;

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef uint32_t v2u32 __attribute__((ext_vector_type(2)));
typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v2u32 lds_u2;
typedef __attribute__((address_space(3))) v4u32 lds_u4;

// LDS accesses by 32-bit byte address
__device__ __forceinline__ uint32_t ld32(uint32_t a) { return *(const lds_u32 *)(size_t)a; }
__device__ __forceinline__ uint16_t ld16(uint32_t a) { return *(const lds_u16 *)(size_t)a; }
__device__ __forceinline__ uint2 ld64(uint32_t a)
{
    const v2u32 v = *(const lds_u2 *)(size_t)a;
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint4 ld128(uint32_t a)
{
    const v4u32 v = *(const lds_u4 *)(size_t)a;
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st8(uint32_t a, uint32_t v) { *(lds_u8 *)(size_t)a = (uint8_t)v; }
__device__ __forceinline__ void st32(uint32_t a, uint32_t v) { *(lds_u32 *)(size_t)a = v; }

// a * (1 << sh) + b as one v_lshl_add_u32 (kept out of the compiler's reach:
// it would otherwise rewrite the bitfield extract as shift + and + add)
template <int SH>
__device__ __forceinline__ uint32_t lshl_add(uint32_t a, uint32_t b)
{
    uint32_t r;
    asm("v_lshl_add_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "i"(SH), "v"(b));
    return r;
}

// the same with a wave-uniform b held in a scalar register
template <int SH>
__device__ __forceinline__ uint32_t lshl_add_s(uint32_t a, uint32_t b)
{
    uint32_t r;
    asm("v_lshl_add_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "i"(SH), "s"(b));
    return r;
}

__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }

// A lane's stream window of 32 * NW bits, first stream bit in bit 31 of
// w[0]: its chunk's NW - 1 words and the next chunk's first word (five
// registers for 16-byte chunks, three for 8-byte chunks).
template <int NW>
struct Window {
    uint32_t w[NW];
    // consume b bits (1 <= b <= 32) where sh holds (32 - b) mod 32 in its low five bits
    __device__ __forceinline__ void consume(uint32_t sh)
    {
#pragma unroll
        for (int i = 0; i + 1 < NW; i++) w[i] = __builtin_amdgcn_alignbit(w[i], w[i + 1], sh);
        w[NW - 1] = __builtin_amdgcn_alignbit(w[NW - 1], 0u, sh);
    }
};

__device__ __forceinline__ Window<5> make_window(uint4 own, uint32_t next, uint32_t gap)
{
    Window<5> w{{own.x, own.y, own.z, own.w, next}};
    if (gap) w.consume(0u - gap);
    return w;
}

__device__ __forceinline__ Window<3> make_window(uint2 own, uint32_t next, uint32_t gap)
{
    Window<3> w{{own.x, own.y, next}};
    if (gap) w.consume(0u - gap);
    return w;
}

// First code of a window through the hierarchical tables at LDS byte
// address `chain`.  Returns exponent | length << 8; a malformed walk yields
// length 32 so that every step advances.
__device__ __forceinline__ uint32_t chain_decode(uint32_t chain, uint32_t win)
{
    uint32_t e = ld16(lshl_add_s<1>(win >> 24, chain));
    if (e & 0x8000u) {
        e = ld16(chain + 2u * ((e & 0x7FFFu) * 256u + ((win >> 16) & 0xFFu)));
        if (e & 0x8000u) {
            e = ld16(chain + 2u * ((e & 0x7FFFu) * 256u + ((win >> 8) & 0xFFu)));
            if (e & 0x8000u) {
                e = ld16(chain + 2u * ((e & 0x7FFFu) * 256u + (win & 0xFFu)));
                if (e & 0x8000u) e = 32u << 8;
            }
        }
    }
    if (!(e & 0x3F00u)) e = 32u << 8;
    return e;
}

__device__ __forceinline__ uint32_t rot_exp(uint32_t e) { return ((e >> 1) | (e << 7)) & 0xFFu; }

// Wavefront-scope ordering of LDS traffic between lanes of one wave.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Locate: number of codes starting in [p0, end) of the lane's chunk; w is
// the window at p0.  Multi-code lookups run while a whole table window
// (K bits) lies before `end`, so every code they count starts inside the
// chunk; the last bits are then walked one code at a time.
template <int K, int NW>
__device__ __forceinline__ uint32_t count_codes(Window<NW> w, uint32_t fast, uint32_t chain, uint32_t p0,
                                                uint32_t end)
{
    uint32_t st = kM0 - p0;
    const uint32_t lim = kM0 - end;            // p < end      <=>  (st & 0xFFFF) > lim
    const uint32_t limk = lim + K;             // p + K <= end <=>  (st & 0xFFFF) >= limk
    while ((st & 0xFFFFu) >= limk) {
        uint32_t meta = ld32(lshl_add_s<3>(w.w[0] >> (32 - K), fast) + 4);
        if (meta == 0) meta = (1u << 16) - ((chain_decode(chain, w.w[0]) >> 8) & 0x3Fu);
        w.consume(meta);
        st += meta;
    }
    while ((st & 0xFFFFu) > lim) {
        const uint32_t step = (1u << 16) - ((chain_decode(chain, w.w[0]) >> 8) & 0x3Fu);
        w.consume(step);
        st += step;
    }
    return st >> 16;
}

// Emit: decode `cnt` codes from the window w and write their rotated
// exponents to LDS bytes [wpos, wpos + cnt).  wpos + cnt must be below 65536.
template <int K, int NW>
__device__ __forceinline__ void emit_codes(Window<NW> w, uint32_t fast, uint32_t chain, uint32_t wpos,
                                           uint32_t cnt)
{
    uint32_t st = (wpos << 16) | kM0;   // the low half only has to keep borrowing
    const uint32_t bound = (wpos + cnt - 3u) << 16;   // st < bound <=> at least 4 codes left
    while (st < bound) {
        const uint2 f = ld64(lshl_add_s<3>(w.w[0] >> (32 - K), fast));
        uint32_t syms = f.x, meta = f.y;
        if (meta == 0) {
            const uint32_t e = chain_decode(chain, w.w[0]);
            syms = rot_exp(e & 0xFFu);
            meta = (1u << 16) - ((e >> 8) & 0x3Fu);
        }
        // bytes 0 and 2 of syms and of syms >> 8 (stores of a high half
        // need no shift)
        const uint32_t a = st >> 16;
        uint32_t t = syms >> 8;
        asm("" : "+v"(t));   // keeps t >> 16 from being folded into syms >> 24
        st8(a, syms);
        st8(a + 1, t);
        st8(a + 2, syms >> 16);
        st8(a + 3, t >> 16);
        w.consume(meta);
        st += meta;
    }
    const uint32_t lend = wpos + cnt;
    while ((st >> 16) < lend) {
        const uint32_t e = chain_decode(chain, w.w[0]);
        const uint32_t step = (1u << 16) - ((e >> 8) & 0x3Fu);
        st8(st >> 16, rot_exp(e & 0xFFu));
        w.consume(step);
        st += step;
    }
}

// Exclusive prefix sum over the wavefront; *total receives the sum.  DPP
// row shifts scan each row of 16 lanes, then the row totals are broadcast
// to the rows above them (gfx9 row_bcast:15 and row_bcast:31).
__device__ __forceinline__ uint32_t wave_exclusive_scan(uint32_t x, uint32_t *total)
{
    uint32_t v = x;
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);   // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);   // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);   // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);   // row_shr:8
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);   // row_bcast:15
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);   // row_bcast:31
    *total = __builtin_amdgcn_readlane(v, 63);
    return v - x;
}

// Copy the multi-code table (8 << K bytes) and the hierarchical tables
// (n_chain uint16 entries) from global memory into LDS at fast_lds and
// chain_lds, with 16-byte accesses; every load of the first pass is issued
// before the first LDS store.  Both global arrays are 16-byte aligned and
// n_chain is a multiple of 8 (256 entries per table).
template <int K, uint32_t THREADS>
__device__ __forceinline__ void stage_tables(uint32_t fast_lds, uint32_t chain_lds, const uint32_t *fast,
                                             const uint16_t *chain, uint32_t n_chain)
{
    constexpr uint32_t kFast4 = (8u << K) / 16;
    constexpr uint32_t kPer = (kFast4 + THREADS - 1) / THREADS;
    const uint4 *f4 = reinterpret_cast<const uint4 *>(fast);
    const uint4 *c4 = reinterpret_cast<const uint4 *>(chain);
    const uint32_t nc4 = n_chain / 8, tid = threadIdx.x;
    uint4 v[kPer];
#pragma unroll
    for (uint32_t i = 0; i < kPer; i++) {
        const uint32_t idx = tid + i * THREADS;
        v[i] = idx < kFast4 ? f4[idx] : make_uint4(0, 0, 0, 0);
    }
    const uint4 c = tid < nc4 ? c4[tid] : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (uint32_t i = 0; i < kPer; i++) {
        const uint32_t idx = tid + i * THREADS;
        if (idx < kFast4) *(lds_u4 *)(size_t)(fast_lds + 16 * idx) = v4u32{v[i].x, v[i].y, v[i].z, v[i].w};
    }
    if (tid < nc4) *(lds_u4 *)(size_t)(chain_lds + 16 * tid) = v4u32{c.x, c.y, c.z, c.w};
    for (uint32_t idx = tid + THREADS; idx < nc4; idx += THREADS) {
        const uint4 w = c4[idx];
        *(lds_u4 *)(size_t)(chain_lds + 16 * idx) = v4u32{w.x, w.y, w.z, w.w};
    }
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
