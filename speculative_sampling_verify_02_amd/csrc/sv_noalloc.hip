// spec_verify for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc): the workspace is a
// file-scope device array of fixed size instead of a caller buffer.  The kernels and
// their results are spec_verify's.
//
// Each GPU holds its own copy of the array, at its own address, for the life of the
// process.  Host code never passes the array's name to a kernel or a copy (in host
// code that name is a stand-in, not a device address): the address is looked up once
// per device with hipGetSymbolAddress and kept.
#include <mutex>
#include <stdint.h>

#include "spec_verify.h"
#include "sv_internal.h"

namespace {

static_assert(SPEC_VERIFY_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size must keep 256-byte alignment");
static __device__ __align__(256) unsigned char scratch[SPEC_VERIFY_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices] = {};

// This device's copy of the scratch array (looked up on the first call on the device,
// with that device current).
sv_status scratch_for(int dev, void **out)
{
    if (dev < 0 || dev >= kMaxDevices) return SV_EHIP;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch[dev] == nullptr) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return SV_EHIP;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return SV_EHIP;
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || p == nullptr) return SV_EHIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return SV_OK;
}

}  // namespace

extern "C" sv_status spec_verify_noalloc(const void *target_logits, const void *draft_logits, int32_t dtype,
                                         int64_t vocab, int32_t batch, int64_t n_target_rows,
                                         const int32_t *draft_tokens, const float *uniforms,
                                         const float *temperature, const int32_t *gamma_per_row,
                                         int32_t gamma_uniform, int32_t mode, int32_t *n_accepted,
                                         int32_t *emitted_tokens, const sv_diag *diag, void *hip_stream)
{
    if (dtype != SV_BF16 && dtype != SV_F32) return SV_EDTYPE;
    const size_t need = spec_verify_workspace_bytes(batch, n_target_rows, vocab, dtype);
    if (need == 0) return SV_EINVAL;
    if (need > (size_t)SPEC_VERIFY_NOALLOC_SCRATCH_BYTES) return SV_ESCRATCH;
    if (batch == 0) return n_target_rows == 0 ? SV_OK : SV_EINVAL;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    int dev = -1;
    if (s != nullptr) {
        if (hipStreamGetDevice(s, &dev) != hipSuccess) return SV_EHIP;
    } else if (hipGetDevice(&dev) != hipSuccess) {
        return SV_EHIP;
    }
    void *ws = nullptr;
    const sv_status st = scratch_for(dev, &ws);
    if (st != SV_OK) return st;
    return spec_verify(target_logits, draft_logits, dtype, vocab, batch, n_target_rows, draft_tokens, uniforms,
                       temperature, gamma_per_row, gamma_uniform, mode, n_accepted, emitted_tokens, diag, ws,
                       (size_t)SPEC_VERIFY_NOALLOC_SCRATCH_BYTES, hip_stream);
}
