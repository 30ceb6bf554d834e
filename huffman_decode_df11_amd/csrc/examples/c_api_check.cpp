// The C ABI on its own, with no Python and no PyTorch: a host program that
// builds a codebook, encodes a weight, copies the encoded arrays to the GPU
// with plain HIP runtime calls, decodes it, and runs the fused product, each
// result checked here.  Usage: c_api_check [--host-only]
//   --host-only   histogram, codebook, encode and validate only (no GPU).
// Prints one line starting with "c-api ok" and exits 0 when every check
// passes; otherwise prints what failed and exits 1.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "df11.h"

namespace {

#define CHECK_DF11(call)                                                                         \
    do {                                                                                         \
        int rc_ = (call);                                                                        \
        if (rc_ != DF11_OK) {                                                                    \
            std::fprintf(stderr, "%s failed: %s (%s)\n", #call, df11_status_string(rc_), df11_last_error()); \
            return 1;                                                                            \
        }                                                                                        \
    } while (0)

#define CHECK_HIP(call)                                                                          \
    do {                                                                                         \
        hipError_t e_ = (call);                                                                  \
        if (e_ != hipSuccess) {                                                                  \
            std::fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));              \
            return 1;                                                                            \
        }                                                                                        \
    } while (0)

// float -> BF16 bits, round to nearest, ties to even (finite inputs here)
uint16_t to_bf16(float f)
{
    uint32_t u;
    std::memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

float from_bf16(uint16_t h)
{
    const uint32_t u = (uint32_t)h << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

// N(0, sigma) BF16 values from a 64-bit linear congruential generator and
// the Box-Muller transform
std::vector<uint16_t> normal_bf16(uint64_t n, double sigma, uint64_t seed)
{
    std::vector<uint16_t> out(n);
    uint64_t x = seed * 0x9E3779B97F4A7C15ull + 1;
    auto uniform = [&x]() {
        x = x * 6364136223846793005ull + 1442695040888963407ull;
        return ((x >> 11) + 0.5) * (1.0 / 9007199254740992.0);
    };
    for (uint64_t i = 0; i < n; i += 2) {
        const double r = std::sqrt(-2.0 * std::log(uniform())), t = 6.283185307179586 * uniform();
        out[i] = to_bf16((float)(sigma * r * std::cos(t)));
        if (i + 1 < n) out[i + 1] = to_bf16((float)(sigma * r * std::sin(t)));
    }
    return out;
}

// Device copies of every array of a host view; the returned view points at
// them.  Allocations are appended to `keep` (freed by the caller).
template <class T>
int upload(const T *host, uint64_t count, const T **dev, std::vector<void *> &keep)
{
    *dev = nullptr;
    if (!count) return 0;
    void *p = nullptr;
    CHECK_HIP(hipMalloc(&p, count * sizeof(T)));
    keep.push_back(p);
    CHECK_HIP(hipMemcpy(p, host, count * sizeof(T), hipMemcpyHostToDevice));
    *dev = static_cast<const T *>(p);
    return 0;
}

int to_device(const df11_view &h, df11_view *d, std::vector<void *> &keep)
{
    *d = h;
    if (upload(h.exp_words, h.n_exp_words, &d->exp_words, keep) || upload(h.sm, h.n_sm, &d->sm, keep) ||
        upload(h.gaps, h.n_gaps, &d->gaps, keep) || upload(h.segs, h.n_segs, &d->segs, keep) ||
        upload(h.chain, h.n_chain, &d->chain, keep) || upload(h.fast, h.n_fast, &d->fast, keep) ||
        upload(h.block_seg, h.n_block_seg, &d->block_seg, keep) || upload(h.counts, h.n_counts, &d->counts, keep))
        return 1;
    return 0;
}

}  // namespace

int main(int argc, char **argv)
{
    const bool host_only = argc > 1 && std::strcmp(argv[1], "--host-only") == 0;
    const uint64_t R = 256, C = 2048, n = R * C;   // an [R, C] weight (8 row blocks of the fused tiles)
    const std::vector<uint16_t> w = normal_bf16(n, 0.02, 7);

    // host: histogram, codebook, two encodings (row-major and the fused kernel's tile order)
    uint64_t hist[256] = {0};
    CHECK_DF11(df11_hist_accumulate(w.data(), n, hist));
    df11_codebook *cb = static_cast<df11_codebook *>(std::calloc(1, sizeof(df11_codebook)));
    if (!cb) return 1;
    CHECK_DF11(df11_codebook_build(hist, DF11_MAX_LEN, DF11_FAST_BITS_DEFAULT, cb));
    df11_encoded *enc = nullptr, *genc = nullptr;
    CHECK_DF11(df11_encode(w.data(), n, cb, nullptr, &enc));
    df11_layout gl;
    CHECK_DF11(df11_gemm_layout(R, C, &gl));
    CHECK_DF11(df11_encode(w.data(), n, cb, &gl, &genc));
    df11_view hv, hgv;
    CHECK_DF11(df11_encoded_view(enc, &hv));
    CHECK_DF11(df11_encoded_view(genc, &hgv));
    CHECK_DF11(df11_validate(&hv, cb));
    CHECK_DF11(df11_validate(&hgv, cb));
    const double bpw = 8.0 * (double)((hv.total_bits + 7) / 8 + hv.n + hv.n_gaps + hv.n_counts +
                                      hv.n_segs * sizeof(df11_segment)) / (double)n;
    // an error is reported as a status with a message, not a crash
    if (df11_encode(nullptr, 5, cb, nullptr, &enc) != DF11_E_ARG || !df11_last_error()[0]) {
        std::fprintf(stderr, "null input not rejected\n");
        return 1;
    }
    if (host_only) {
        std::printf("c-api ok (host only): %llu elements, %u coded exponents, codes up to %u bits, %.3f bits per weight, "
                    "%llu segments, library %s\n", (unsigned long long)n, cb->n_symbols, cb->max_len, bpw,
                    (unsigned long long)hv.n_segments, df11_version());
        df11_encoded_free(enc);
        df11_encoded_free(genc);
        std::free(cb);
        return 0;
    }

    // device: the arrays copied by hand, then decode and the fused product
    std::vector<void *> keep;
    df11_view dv, dgv;
    if (to_device(hv, &dv, keep) || to_device(hgv, &dgv, keep)) return 1;
    hipStream_t st;
    CHECK_HIP(hipStreamCreate(&st));
    uint16_t *dout = nullptr;
    CHECK_HIP(hipMalloc((void **)&dout, (n + 64) * 2));
    CHECK_HIP(hipMemsetAsync(dout, 0x55, (n + 64) * 2, st));
    CHECK_DF11(df11_decode(&dv, dout, st));
    std::vector<uint16_t> got(n + 64);
    CHECK_HIP(hipMemcpyAsync(got.data(), dout, (n + 64) * 2, hipMemcpyDeviceToHost, st));
    CHECK_HIP(hipStreamSynchronize(st));
    uint64_t bad = 0;
    for (uint64_t i = 0; i < n; i++) bad += got[i] != w[i];
    for (uint64_t i = n; i < n + 64; i++) bad += got[i] != 0x5555;
    if (bad) {
        std::fprintf(stderr, "decode: %llu elements differ\n", (unsigned long long)bad);
        return 1;
    }

    const uint32_t B = 8;
    const std::vector<uint16_t> x = normal_bf16((uint64_t)B * C, 1.0, 11);
    uint16_t *dx = nullptr;
    float *dy = nullptr;
    uint16_t *dy16 = nullptr;
    CHECK_HIP(hipMalloc((void **)&dx, x.size() * 2));
    CHECK_HIP(hipMalloc((void **)&dy, (size_t)B * R * 4));
    CHECK_HIP(hipMalloc((void **)&dy16, (size_t)B * R * 2));
    CHECK_HIP(hipMemcpyAsync(dx, x.data(), x.size() * 2, hipMemcpyHostToDevice, st));
    CHECK_DF11(df11_decode_gemm(&dgv, dx, B, dy, nullptr, st));
    CHECK_DF11(df11_decode_gemm_out(&dgv, dx, B, dy16, DF11_Y_BF16, nullptr, st));
    std::vector<float> y((size_t)B * R);
    std::vector<uint16_t> y16((size_t)B * R);
    CHECK_HIP(hipMemcpyAsync(y.data(), dy, y.size() * 4, hipMemcpyDeviceToHost, st));
    CHECK_HIP(hipMemcpyAsync(y16.data(), dy16, y16.size() * 2, hipMemcpyDeviceToHost, st));
    CHECK_HIP(hipStreamSynchronize(st));
    double num = 0, den = 0, worst16 = 0;
    for (uint32_t b = 0; b < B; b++)
        for (uint64_t r = 0; r < R; r++) {
            double ref = 0;
            for (uint64_t k = 0; k < C; k++) ref += (double)from_bf16(x[b * C + k]) * from_bf16(w[r * C + k]);
            const double d = y[b * R + r] - ref;
            num += d * d;
            den += ref * ref;
            // BF16 y: within one BF16 step of the exact product
            const double step = std::ldexp(1.0, std::ilogb(std::fabs(ref) > 0 ? ref : 1.0) - 7);
            worst16 = std::fmax(worst16, std::fabs(from_bf16(y16[b * R + r]) - ref) / step);
        }
    const double rel = std::sqrt(num / den);
    if (!(rel < 2e-3) || !(worst16 <= 1.0)) {
        std::fprintf(stderr, "fused product: relative error %.3g, BF16 y off by %.2f steps\n", rel, worst16);
        return 1;
    }
    std::printf("c-api ok: %llu elements decoded bit-exact from hand-copied device arrays, %.3f bits per weight; "
                "fused [%u x %llu] x [%llu x %llu]^T relative error %.2e, BF16 y within %.2f steps\n",
                (unsigned long long)n, bpw, B, (unsigned long long)C, (unsigned long long)R, (unsigned long long)C,
                rel, worst16);
    for (void *p : keep) (void)hipFree(p);
    (void)hipFree(dout);
    (void)hipFree(dx);
    (void)hipFree(dy);
    (void)hipFree(dy16);
    (void)hipStreamDestroy(st);
    df11_encoded_free(enc);
    df11_encoded_free(genc);
    std::free(cb);
    return 0;
}
