// Pieces shared by the two Winograd forms of the 3x3 conv (conv_wino.hip,
// conv_wino4.hip): the launch parameters, buffer resources and direct
// global -> LDS loads, the step cursor over (time tap, channel quad), and the
// pairwise merge of GroupNorm statistics.
#pragma once

#include "vae_internal.h"

namespace vae {
namespace wino {

constexpr int kWCh = 4;             // input channels per step (the K of v_mfma_f32_16x16x4_f32)
constexpr int kWOOB = 0x7FFFFFF0;   // buffer offset past every range: reads 0

struct WParams {
    const float *x;         // input [cin, T, Hin, Win]
    const float *u;         // packed U
    const float *bias, *res;
    const float *gn_coef;   // GroupNorm + SiLU on load: (mean, scale, beta, -) per input channel
    float *y;
    float *part;            // split-K partial sums [ksplit][cout][T][H][W]
    floatx4 *gn_rec;        // GroupNorm records of y, [32 groups][gn_nrec]
    int cin, cout, H, W, Hin, Win, kt, nquads, tiles_x, ncb, ksplit, gn_cpg, gn_nrec;
    int nub;                // packed U blocks (of the packing's output-channel block)
    long long in_cstride, in_fstride, out_cstride, out_fstride, part_stride;
};

__device__ __attribute__((always_inline)) inline __amdgpu_buffer_rsrc_t wino_rsrc(const float *base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __attribute__((always_inline)) inline const float *wino_frame(const WParams &p, int frame, int dt) {
    int fr = frame + dt - (p.kt - 1);
    fr = fr < 0 ? 0 : fr;
    return p.x + (long long)fr * p.in_fstride;
}

// The next step to stage: time tap dt and channel quad, and the quad's first
// channel in the tap's frame.  Advanced by additions only.
struct WCursor {
    int quad, dt;
    const float *x;
};

__device__ __attribute__((always_inline)) inline void wino_next(const WParams &p, int frame, WCursor &c) {
    if (++c.quad == p.nquads) {
        c.quad = 0;
        ++c.dt;
        c.x = wino_frame(p, frame, c.dt);
    } else {
        c.x += kWCh * p.in_cstride;
    }
}

__device__ __attribute__((always_inline)) inline WCursor wino_cursor(const WParams &p, int frame, int s0) {
    WCursor c;
    c.dt = s0 / p.nquads;
    c.quad = s0 - c.dt * p.nquads;
    c.x = wino_frame(p, frame, c.dt) + (long long)kWCh * c.quad * p.in_cstride;
    return c;
}

// Direct global -> LDS load: lane i's 4 (16) bytes land at lds + i (float or
// float4); an offset past the buffer's range writes 0.
__device__ __attribute__((always_inline)) inline void wino_dma4(__amdgpu_buffer_rsrc_t r, float *lds, int voffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 4, voffset, 0, 0, 0);
}
__device__ __attribute__((always_inline)) inline void wino_dma16(__amdgpu_buffer_rsrc_t r, floatx4 *lds, int voffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, voffset, 0, 0, 0);
}

// (n, mean, M2) of a set merged with (nb, mb, qb) of another (pairwise update
// of Chan, Golub and LeVeque); empty sets (n = 0) merge as the identity.
__device__ __attribute__((always_inline)) inline void wino_chan_merge(float (&a)[3], float nb, float mb, float qb) {
    const float nt = a[0] + nb;
    const float delta = mb - a[1];
    // counts are whole numbers: a hardware reciprocal (1 ulp) instead of a
    // full-precision division, which costs about ten instructions
    const float fb = nt > 0.f ? nb * __builtin_amdgcn_rcpf(nt) : 0.f;
    a[2] = (a[2] + qb) + delta * delta * a[0] * fb;
    a[1] = a[1] + delta * fb;
    a[0] = nt;
}

}  // namespace wino
}  // namespace vae
