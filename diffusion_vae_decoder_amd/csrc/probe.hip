// Measurement probes: kernels of known work that measure the FP32 MFMA and
// HBM ceilings of the GPU the library runs on, so that the decoder's kernels
// can be read against measured ceilings beside the published ones.  They
// compute nothing of the decoder; the caller times them with events on the
// stream it passes.

#include "vae_internal.h"

namespace vae {

namespace {

constexpr int kProbeThreads = 256;   // four waves
constexpr int kProbeChains = 8;      // independent accumulator chains per wave

// Every wave runs `iters` rounds of kProbeChains independent
// v_mfma_f32_32x32x2_f32 (2 * 32 * 32 * 2 FLOPs each) on operands held in
// registers, so nothing but the matrix pipe bounds it.  Lane l supplies
// A[m = l % 32][k = l / 32] = a(l) and B[k = l / 32][n = l % 32] = b(l), so
// every round adds sum_k a(m + 32k) b(n + 32k) to C[m][n]; each thread
// writes the sum of its accumulators, which keeps the work live.
__global__ __launch_bounds__(kProbeThreads) void probe_mfma_f32(int iters, float *out) {
    const int lane = threadIdx.x & 63;
    const float a = 1.0f + (float)lane * (1.0f / 64.0f);
    const float b = 1.0f - (float)lane * (1.0f / 128.0f);
    floatx16 acc[kProbeChains];
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
    for (int i = 0; i < iters; ++i)
#pragma unroll
        for (int c = 0; c < kProbeChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[c], 0, 0, 0);
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[c][e];
    out[(long long)blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

// The HBM probes stream contiguous chunks of 256 x kProbeBatch float4s (16
// KB), one chunk per workgroup step, grid-stride over the chunks; each thread
// has kProbeBatch 16-byte loads in flight.  Measured on MI355X this layout
// outran a grid-stride over single float4s by 10-25%.
constexpr int kProbeBatch = 4;
constexpr long long kProbeChunk = (long long)kProbeThreads * kProbeBatch;   // float4s

// Reads x once; each thread writes the sum of what it read.
__global__ __launch_bounds__(kProbeThreads) void probe_hbm_read(const floatx4 *__restrict__ x, long long n4,
                                                                float *__restrict__ out) {
    floatx4 s = {0.f, 0.f, 0.f, 0.f};
    for (long long c0 = (long long)blockIdx.x * kProbeChunk; c0 < n4; c0 += (long long)gridDim.x * kProbeChunk) {
        if (c0 + kProbeChunk <= n4) {
            floatx4 v[kProbeBatch];
#pragma unroll
            for (int k = 0; k < kProbeBatch; ++k) v[k] = x[c0 + k * kProbeThreads + threadIdx.x];
#pragma unroll
            for (int k = 0; k < kProbeBatch; ++k) s += v[k];
        } else {
            for (long long i = c0 + threadIdx.x; i < n4; i += kProbeThreads) s += x[i];
        }
    }
    out[(long long)blockIdx.x * kProbeThreads + threadIdx.x] = (s[0] + s[1]) + (s[2] + s[3]);
}

// Copies x to y, a thread's loads of a chunk issued before its stores.
__global__ __launch_bounds__(kProbeThreads) void probe_hbm_copy(const floatx4 *__restrict__ x, long long n4,
                                                                floatx4 *__restrict__ y) {
    for (long long c0 = (long long)blockIdx.x * kProbeChunk; c0 < n4; c0 += (long long)gridDim.x * kProbeChunk) {
        if (c0 + kProbeChunk <= n4) {
            floatx4 v[kProbeBatch];
#pragma unroll
            for (int k = 0; k < kProbeBatch; ++k) v[k] = x[c0 + k * kProbeThreads + threadIdx.x];
#pragma unroll
            for (int k = 0; k < kProbeBatch; ++k) y[c0 + k * kProbeThreads + threadIdx.x] = v[k];
        } else {
            for (long long i = c0 + threadIdx.x; i < n4; i += kProbeThreads) y[i] = x[i];
        }
    }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

template <typename... A>
int32_t bad_arg(const char *fmt, A... a) {
    set_error(fmt, a...);
    return VAE_ERR_INVALID_ARG;
}

}  // namespace

}  // namespace vae

extern "C" {

int32_t vae_probe_mfma_f32(int32_t blocks, int32_t iters, float *out, size_t out_floats, double *flops,
                           void *stream) {
    const char *who = "vae_probe_mfma_f32";
    if (!out || !flops) return vae::bad_arg("%s: NULL pointer", who);
    if (blocks < 1 || blocks > 65535 || iters < 1 || iters > (1 << 20))
        return vae::bad_arg("%s: blocks %d (1..65535) or iters %d (1..2^20) out of range", who, blocks, iters);
    const size_t need = (size_t)blocks * vae::kProbeThreads;
    if (out_floats < need) return vae::bad_arg("%s: out holds %zu floats < %zu", who, out_floats, need);
    *flops = (double)blocks * (vae::kProbeThreads / 64) * iters * vae::kProbeChains * (2.0 * 32 * 32 * 2);
    hipLaunchKernelGGL(vae::probe_mfma_f32, dim3((unsigned)blocks), dim3(vae::kProbeThreads), 0,
                       static_cast<hipStream_t>(stream), (int)iters, out);
    return vae::check_launch(who);
}

int32_t vae_probe_hbm(const float *x, size_t n, float *y, int32_t blocks, float *out, size_t out_floats,
                      void *stream) {
    const char *who = "vae_probe_hbm";
    if (!x || (!y && !out)) return vae::bad_arg("%s: NULL pointer", who);
    if (n == 0 || n % 4 || !vae::aligned16(x) || (y && !vae::aligned16(y)))
        return vae::bad_arg("%s: n = %zu must be a positive multiple of 4, buffers 16-byte aligned", who, n);
    if (blocks < 1 || blocks > 65535) return vae::bad_arg("%s: blocks %d (1..65535)", who, blocks);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const long long n4 = (long long)(n / 4);
    if (y) {
        hipLaunchKernelGGL(vae::probe_hbm_copy, dim3((unsigned)blocks), dim3(vae::kProbeThreads), 0, s,
                           reinterpret_cast<const vae::floatx4 *>(x), n4, reinterpret_cast<vae::floatx4 *>(y));
    } else {
        const size_t need = (size_t)blocks * vae::kProbeThreads;
        if (out_floats < need) return vae::bad_arg("%s: out holds %zu floats < %zu", who, out_floats, need);
        hipLaunchKernelGGL(vae::probe_hbm_read, dim3((unsigned)blocks), dim3(vae::kProbeThreads), 0, s,
                           reinterpret_cast<const vae::floatx4 *>(x), n4, out);
    }
    return vae::check_launch(who);
}

}  // extern "C"
