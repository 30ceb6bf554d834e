// df11_decode_gemm: fused decode + matrix product (placeholder until the
// fused kernel lands; reports E_UNSUPPORTED).
#include <hip/hip_runtime.h>

#include "df11_internal.h"

extern "C" int df11_decode_gemm(const df11_view *w, const uint16_t *x, uint32_t B, float *y,
                                uint16_t *w_debug, void *stream)
{
    (void)w; (void)x; (void)B; (void)y; (void)w_debug; (void)stream;
    return df11::fail(DF11_E_UNSUPPORTED, "df11_decode_gemm: not built yet");
}
