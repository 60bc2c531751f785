// GroupNorm(32) + SiLU for callers that cannot allocate memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid allocation):
// vae_groupnorm_silu with its workspace -- the per-group partial sums of the
// statistics pass -- in a static device array of the library instead of a
// caller buffer.  The kernels are the same as vae_groupnorm_silu's.
//
// The array `scratch` exists once per GPU the library runs on and lives until
// the process ends.  Host code never passes its name to a kernel (on the host
// the name is only a stand-in for the symbol): the first call on a device
// looks up that device's address with hipGetSymbolAddress, with the device
// current, and every later call on it uses the stored address.  Every call
// on a GPU shares its array; the statistics pass writes every partial sum
// the normalisation pass reads, so nothing has to start at zero, but calls
// that overlap in time on one GPU (on different streams) race on it.

#include <mutex>

#include "vae_internal.h"

namespace {

// Largest workspace any GroupNorm needs: 32 groups x at most 64 parts x 2
// doubles of partial sums, 32 doubles of shifts and 32 (mean, rstd) pairs
// (33,280 bytes).
constexpr size_t kScratchBytes = 36 * 1024;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices];   // the array's address on each device, once looked up

// The current device's copy of `scratch`.
int32_t scratch_on_current_device(void **out) {
    int dev = 0;
    int32_t rc = vae::hip_status(hipGetDevice(&dev), "vae_groupnorm_silu_noalloc: hipGetDevice");
    if (rc) return rc;
    if (dev < 0 || dev >= kMaxDevices) {
        vae::set_error("vae_groupnorm_silu_noalloc: device %d beyond the %d the library tracks", dev, kMaxDevices);
        return VAE_ERR_UNSUPPORTED;
    }
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        rc = vae::hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)),
                             "vae_groupnorm_silu_noalloc: hipGetSymbolAddress(scratch)");
        if (rc) return rc;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return VAE_OK;
}

}  // namespace

extern "C" int32_t vae_groupnorm_silu_noalloc(const float *x, int32_t c, int64_t spatial, const vae_norm *norm,
                                              int32_t apply_silu, const float *residual, float *y, void *stream) {
    int32_t rc = vae::check_groupnorm_args("vae_groupnorm_silu_noalloc", x, c, spatial, norm, y);
    if (rc) return rc;
    const size_t need = vae::groupnorm_ws_bytes(c, spatial);
    if (need > kScratchBytes) {
        vae::set_error("vae_groupnorm_silu_noalloc: needs %zu bytes of scratch, the static buffer holds %zu", need,
                       kScratchBytes);
        return VAE_ERR_UNSUPPORTED;
    }
    void *ws = nullptr;
    if ((rc = scratch_on_current_device(&ws))) return rc;
    return vae::launch_groupnorm(x, c, spatial, norm->gamma, norm->beta, apply_silu ? 1 : 0, residual, y, ws,
                                 static_cast<hipStream_t>(stream));
}
