// Convolutions of the FLUX-class VAE decoder on gfx950.
//
// conv3x3_mfma: 3x3 (and causal 3x3x3) stride-1 convolution as an implicit
// GEMM on FP32 MFMA (v_mfma_f32_32x32x2_f32).  The GEMM is
//     Y[o, p] = sum_k Wp[o, k] * X[k, p] + bias[o] (+ R[o, p])
// with o the output channel, p the output pixel and k = (input channel,
// tap): the "GPU plan" of the VAE decode -> GPU handoff note (im2col then
// one GEMM per layer), but the im2col matrix is never formed.  Instead each
// workgroup stages, per chunk of 4 input channels, the input tile plus a
// one-pixel halo in LDS; one staged pixel then feeds all nine taps.  The
// nearest-x2 upsample (cortiq-engine 0.7.7 `vae`, VaeUpRef) and the latent
// de-normalisation (VaeDecoder) are applied while staging, so neither is
// ever written to memory.  Bias and the resnet skip (VaeResnetRef) are added
// in the epilogue.
//
// Workgroup: 256 threads = 4 waves in a 2 x 2 grid; each wave owns a 64 x 64
// block of the 128 (channels) x 128 (pixels) tile as 2 x 2 MFMA 32x32 tiles.
// In every MFMA the two lane halves carry two different K indices; K within
// a chunk is ordered (channel, tap) and lane half h takes the channels
// [2h, 2h + 2), so both LDS operand reads are one row of 32 consecutive
// floats per half-wave, and the strides are padded so the two halves fall in
// different LDS banks.  The halo and weight tiles are double-buffered (48 KB),
// so three workgroups (three waves per SIMD) share a CU and hide each other's
// staging.  The halo is gathered with raw buffer loads: padding and channels
// past cin read as 0 from out-of-range offsets, with no branch.
//
// Shapes that yield fewer workgroups than the GPU holds are split along K;
// each split writes partial sums that splitk_reduce adds in a fixed order.
//
// When the output is normalised next (a GroupNorm of the following layer),
// the epilogue (or splitk_reduce) also writes per-group records (count,
// mean, sum of squared deviations) of the tile, which the normalisation
// merges instead of making a statistics pass over the output.
//
// MODE_GNSILU (optional, off in the decoder by default) applies GroupNorm +
// SiLU of the input while staging it, from per-channel coefficients held in
// an LDS table.  It removes the separate normalisation pass but costs about
// 10% of the conv on MI355X, more than that pass.
//
// By default the 3x3 convs run in the Winograd form (conv_wino.hip); this
// implicit GEMM serves conv_in, whose gather de-normalises the latent, and
// every 3x3 conv when the implicit-GEMM form is selected
// (vae_set_conv3x3_algorithm).  The decoder's conv_out (3 output channels)
// runs on conv3x3_direct in conv_direct.hip.

#include <atomic>
#include <cstdio>

#include "vae_internal.h"

namespace vae {

namespace {

constexpr int kThreads = 256;
constexpr int kCK = kConvCC * 9;         // K per chunk (36)
constexpr int kSteps = kCK / 2;          // MFMA k-steps per chunk (18)
constexpr int kHalfC = kConvCC / 2;      // channels per lane half

// Smallest stride >= base, a multiple of `align`, with (mult * stride) % 64 == 32:
// the two lane halves of a wave then read disjoint halves of a 64-bank LDS.
constexpr int bank_split_stride(int base, int mult, int align) {
    for (int s = base; s < base + 512; ++s)
        if (s % align == 0 && (mult * s) % 64 == 32) return s;
    return -1;
}

constexpr int kLdaW = bank_split_stride(kConvBM, kHalfC * 9, 4);   // weight row stride (144)
static_assert(kLdaW > 0, "no bank-split stride for the weight tile");

template <int TC>
struct Geom {
    static constexpr int TR = kConvBN / TC;                 // tile rows
    static constexpr int HWD = TC + 2;                       // halo row width
    static constexpr int HP = (TR + 2) * HWD;                // halo plane
    static constexpr int PLANE = bank_split_stride(HP, kHalfC, 1);
    static constexpr int HALO = kConvCC * HP;                // staged halo floats
    static constexpr int HALO_PER_T = (HALO + kThreads - 1) / kThreads;
    static_assert(PLANE > 0, "no bank-split stride for the halo tile");
};

constexpr int kW4 = kCK * kConvBM / 4;                      // float4s of one weight chunk
constexpr int kW4_PER_T = (kW4 + kThreads - 1) / kThreads;
constexpr int kGnMaxChannels = kDirectGnMaxChannels;   // input channels a GroupNorm-on-load table holds

struct Params {
    const float *x, *wpk, *bias, *res;
    const float *gn_coef;   // MODE_GNSILU: (mean, scale, beta, -) per input channel
    float *y;
    float *part;            // split-K partial sums [ksplit][cout][T][H][W] (ksplit > 1)
    floatx4 *gn_rec;        // if set: GroupNorm records of y, [32 groups][gn_nrec] (count, mean, M2, 0)
    int cin, cout, H, W, Win, kt, n_cb, tiles_x, ksplit, gn_cpg, gn_nrec;
    long long in_cstride, in_fstride, out_cstride, out_fstride, part_stride;
    float dn_scale, dn_shift;
};

enum { MODE_PLAIN = 0, MODE_UPSAMPLE = 1, MODE_DENORM = 2, MODE_GNSILU = 3 };

// Offset that lies outside every buffer range below: a buffer load from it
// returns 0 without touching memory (the zero padding of the halo).
constexpr int kOOB = 0x7FFFFFF0;

__device__ __attribute__((always_inline)) inline __amdgpu_buffer_rsrc_t make_rsrc(const float *base,
                                                                                 unsigned bytes) {
    // raw buffer (stride 0), range `bytes`, gfx9 resource word 3
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), (short)0, (int)bytes, 0x00020000);
}

// The K chunk a workgroup stages next: time tap dt, channel block cb, the
// chunk's packed weights and its first input channel in the time tap's
// frame.  Advanced by additions only; the frame is recomputed when the time
// tap changes (at most kt - 1 times).
struct Cursor {
    int dt, cb;
    const float *w;    // packed weight chunk
    const float *x;    // input channel cb * 4 of frame max(frame + dt - (kt - 1), 0)
};

__device__ __attribute__((always_inline)) inline const float *frame_base(const Params &p, int frame, int dt) {
    int fr = frame + dt - (p.kt - 1);
    fr = fr < 0 ? 0 : fr;
    return p.x + (long long)fr * p.in_fstride;
}

__device__ __attribute__((always_inline)) inline Cursor cursor_at(const Params &p, const float *wbase, int it,
                                                                 int frame) {
    Cursor c;
    c.dt = it / p.n_cb;
    c.cb = it - c.dt * p.n_cb;
    c.w = wbase + (size_t)it * (kCK * kConvBM);
    c.x = frame_base(p, frame, c.dt) + (long long)c.cb * kConvCC * p.in_cstride;
    return c;
}

__device__ __attribute__((always_inline)) inline void cursor_next(const Params &p, int frame, Cursor &c) {
    c.w += kCK * kConvBM;
    if (++c.cb == p.n_cb) {
        c.cb = 0;
        ++c.dt;
        c.x = frame_base(p, frame, c.dt);
    } else {
        c.x += kConvCC * p.in_cstride;
    }
}

// Global -> registers: the chunk at cursor `cur` of the packed weights and of
// the input halo.  The halo buffer range covers only the chunk's valid
// channels, so channels past cin and padding positions (offset kOOB) both
// read as 0 with no branch.
template <int TC, int MODE>
__device__ __attribute__((always_inline)) inline void stage_load(
    const Params &p, const Cursor &cur, const int (&h_boff)[Geom<TC>::HALO_PER_T],
    const int (&h_c)[Geom<TC>::HALO_PER_T], floatx4 (&wreg)[kW4_PER_T],
    float (&xreg)[Geom<TC>::HALO_PER_T], bool (&vmask)[Geom<TC>::HALO_PER_T]) {
    using G = Geom<TC>;
    const int tid = threadIdx.x;
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(cur.w, kCK * kConvBM * 4);
#pragma unroll
    for (int i = 0; i < kW4_PER_T; ++i) {
        const int idx = tid + i * kThreads;
        if (kW4 % kThreads == 0 || (i + 1) * kThreads <= kW4 || idx < kW4)
            wreg[i] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(wr, idx * 16, 0, 0));
    }
    const int c0 = cur.cb * kConvCC;
    const int nc = p.cin - c0 < kConvCC ? p.cin - c0 : kConvCC;
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(cur.x, (unsigned)(nc * p.in_cstride * 4));
#pragma unroll
    for (int i = 0; i < G::HALO_PER_T; ++i) {
        float v = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(xr, h_boff[i], 0, 0));
        if (MODE == MODE_DENORM) v = (h_boff[i] != kOOB && h_c[i] < nc) ? v / p.dn_scale + p.dn_shift : 0.f;
        if (MODE == MODE_GNSILU) vmask[i] = h_boff[i] != kOOB && h_c[i] < nc;
        xreg[i] = v;
    }
}

// Registers -> LDS buffer.  MODE_GNSILU applies GroupNorm + SiLU here, after
// the MFMA phase, with the per-channel coefficients (mean, scale, beta) of
// chunk channel c0 + c read from the LDS table `lc`.
template <int TC, int MODE>
__device__ __attribute__((always_inline)) inline void stage_store(
    float *lw, float *lx, const int (&h_lds)[Geom<TC>::HALO_PER_T], const floatx4 (&wreg)[kW4_PER_T],
    float (&xreg)[Geom<TC>::HALO_PER_T], const bool (&vmask)[Geom<TC>::HALO_PER_T],
    const int (&h_c)[Geom<TC>::HALO_PER_T], const float *lc, int c0) {
    if (MODE == MODE_GNSILU) {
#pragma unroll
        for (int i = 0; i < Geom<TC>::HALO_PER_T; ++i) {
            const float *cf = lc + 3 * (c0 + h_c[i]);
            float t = (xreg[i] - cf[0]) * cf[1] + cf[2];
            t = t * __builtin_amdgcn_rcpf(1.f + __expf(-t));
            xreg[i] = vmask[i] ? t : 0.f;
        }
    }
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < kW4_PER_T; ++i) {
        const int idx = tid + i * kThreads;
        if (kW4 % kThreads == 0 || (i + 1) * kThreads <= kW4 || idx < kW4) {
            const int row = idx >> 5, c4 = idx & 31;
            *reinterpret_cast<floatx4 *>(&lw[row * kLdaW + c4 * 4]) = wreg[i];
        }
    }
#pragma unroll
    for (int i = 0; i < Geom<TC>::HALO_PER_T; ++i)
        if ((i + 1) * kThreads <= Geom<TC>::HALO || h_lds[i] >= 0) lx[h_lds[i]] = xreg[i];
}

// Sum each value over the 32 lanes of its lane half (butterfly within 32).
__device__ __attribute__((always_inline)) inline void half_wave_sum(float (&q)[2][4]) {
#pragma unroll
    for (int o = 1; o < 32; o <<= 1)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) q[i][rq] += __shfl_xor(q[i][rq], o, 64);
}

template <int TC, int MODE, bool RES, bool SPLIT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void conv3x3_mfma(Params p) {
    using G = Geom<TC>;
    __shared__ __attribute__((aligned(16))) float lds_w[2][kCK * kLdaW];
    __shared__ float lds_x[2][kConvCC * G::PLANE];
    // GroupNorm coefficients of every input channel (MODE_GNSILU): 3 floats each
    __shared__ float lds_c[MODE == MODE_GNSILU ? 3 * (kGnMaxChannels + kConvCC) : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int half = lane >> 5, l32 = lane & 31;

    // Workgroups are dealt to the 8 XCDs round-robin by linear id.  When the
    // tile count is a multiple of 8 (then the linear id and blockIdx.x agree
    // mod 8), renumber so each XCD walks one contiguous band of tiles: tiles
    // that share halo rows and columns then share one L2.
    int tile = blockIdx.x;
    if ((gridDim.x & 7) == 0) tile = (tile & 7) * (gridDim.x >> 3) + (tile >> 3);
    const int ty = tile / p.tiles_x;
    const int tx = tile - ty * p.tiles_x;
    const int y0 = ty * G::TR, x0 = tx * TC;
    const int ob = blockIdx.y;
    // blockIdx.z = frame * ksplit + split: split s accumulates the K chunks
    // [s * n / ksplit, (s + 1) * n / ksplit) of the n = kt * n_cb chunks.
    const int frame = SPLIT ? blockIdx.z / p.ksplit : blockIdx.z;
    const int split = SPLIT ? blockIdx.z - frame * p.ksplit : 0;

    // Per-thread halo elements: their LDS slot, channel within the chunk and
    // byte offset from the chunk's first channel (kOOB = zero padding).  They
    // are the same for every chunk.
    int h_lds[G::HALO_PER_T], h_boff[G::HALO_PER_T], h_c[G::HALO_PER_T];
#pragma unroll
    for (int i = 0; i < G::HALO_PER_T; ++i) {
        const int e = tid + i * kThreads;
        h_lds[i] = -1;
        h_boff[i] = kOOB;
        h_c[i] = 0;
        if (e < G::HALO) {
            const int c = e / G::HP;
            const int rem = e - c * G::HP;
            const int rr = rem / G::HWD;
            const int cc = rem - rr * G::HWD;
            const int yy = y0 - 1 + rr, xx = x0 - 1 + cc;
            h_lds[i] = c * G::PLANE + rr * G::HWD + cc;
            h_c[i] = c;
            if (yy >= 0 && yy < p.H && xx >= 0 && xx < p.W) {
                const int sp = (MODE == MODE_UPSAMPLE) ? (yy >> 1) * p.Win + (xx >> 1) : yy * p.W + xx;
                h_boff[i] = (c * (int)p.in_cstride + sp) * 4;
            }
        }
    }

    const int n_iter = p.kt * p.n_cb;
    const int it0 = SPLIT ? (int)((long long)split * n_iter / p.ksplit) : 0;
    const int it1 = SPLIT ? (int)((long long)(split + 1) * n_iter / p.ksplit) : n_iter;
    const float *wbase = p.wpk + (size_t)ob * n_iter * (kCK * kConvBM);

    floatx4 wreg[kW4_PER_T];
    float xreg[G::HALO_PER_T];
    bool vmask[G::HALO_PER_T];
    if (MODE == MODE_GNSILU) {
        // channels past cin (up to the chunk's end) get zeros; their values are masked anyway
        for (int e = tid; e < 3 * (p.n_cb * kConvCC); e += kThreads) {
            const int c = e / 3, k = e - 3 * (e / 3);
            lds_c[e] = c < p.cin ? p.gn_coef[4 * c + k] : 0.f;
        }
        __syncthreads();
    }

    // Operand addresses of this lane (the per-step parts are immediates).
    int a_off[2], b_off[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) a_off[i] = half * (kHalfC * 9) * kLdaW + wm * 64 + i * 32 + l32;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int n = wn * 64 + j * 32 + l32;
        const int r = n / TC, col = n - (n / TC) * TC;
        b_off[j] = half * kHalfC * G::PLANE + r * G::HWD + col;
    }

    floatx16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    Cursor cur = cursor_at(p, wbase, it0, frame);
    stage_load<TC, MODE>(p, cur, h_boff, h_c, wreg, xreg, vmask);
    stage_store<TC, MODE>(lds_w[0], lds_x[0], h_lds, wreg, xreg, vmask, h_c, lds_c, cur.cb * kConvCC);
    __syncthreads();

    for (int it = it0; it < it1; ++it) {
        const int buf = (it - it0) & 1;
        if (it + 1 < it1) {
            cursor_next(p, frame, cur);
            stage_load<TC, MODE>(p, cur, h_boff, h_c, wreg, xreg, vmask);
        }
        const float *A = lds_w[buf];
        const float *B = lds_x[buf];
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            const int cl = s / 9, tap = s % 9;
            const int boff = cl * G::PLANE + (tap / 3) * G::HWD + (tap % 3);
            const float a0 = A[a_off[0] + s * kLdaW];
            const float a1 = A[a_off[1] + s * kLdaW];
            const float b0 = B[b_off[0] + boff];
            const float b1 = B[b_off[1] + boff];
            acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc[0][0], 0, 0, 0);
            acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, acc[0][1], 0, 0, 0);
            acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, acc[1][0], 0, 0, 0);
            acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc[1][1], 0, 0, 0);
        }
        if (it + 1 < it1) stage_store<TC, MODE>(lds_w[buf ^ 1], lds_x[buf ^ 1], h_lds, wreg, xreg, vmask, h_c, lds_c, cur.cb * kConvCC);
        __syncthreads();
    }

    // Epilogue: D[i][j] of a 32x32 MFMA tile sits in lane j + 32*((i/4)%2),
    // register (i%4) + 4*(i/8).
    const long long fo = (long long)frame * p.out_fstride;
    bool pv[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int n = wn * 64 + j * 32 + l32;
        pv[j] = y0 + n / TC < p.H && x0 + (n - (n / TC) * TC) < p.W;
    }
    // Per 32-row half of the wave's block, the residual (conv2 of a resnet)
    // is read first, 32 values with no branch (positions outside the image
    // read an in-bounds neighbour and are never stored), then added and stored.
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        float rv[2][16];
        if (RES && !SPLIT) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int n = wn * 64 + j * 32 + l32;
                const int yy = min(y0 + n / TC, p.H - 1), xx = min(x0 + (n - (n / TC) * TC), p.W - 1);
                const long long sp = fo + (long long)yy * p.W + xx;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int o = min(ob * kConvBM + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3), p.cout - 1);
                    rv[j][r] = p.res[(long long)o * p.out_cstride + sp];
                }
            }
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            if (!pv[j]) continue;
            const int n = wn * 64 + j * 32 + l32;
            const long long sp = fo + (long long)(y0 + n / TC) * p.W + x0 + (n - (n / TC) * TC);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                const int o = ob * kConvBM + m;
                if (o < p.cout) {
                    const long long off = (long long)o * p.out_cstride + sp;
                    if (SPLIT) {
                        p.part[split * p.part_stride + off] = acc[i][j][r];
                    } else {
                        float v = acc[i][j][r] + p.bias[o];
                        if (RES) v += rv[j][r];
                        p.y[off] = v;
                        acc[i][j][r] = v;
                    }
                }
            }
        }
    }
    if (!SPLIT && p.gn_rec) {
        // GroupNorm statistics of this tile's outputs for the layer that
        // normalises them next: per group (count, mean, sum of squared
        // deviations from that mean), two passes over the registers.  The
        // host enables this only for cout % 128 == 0 and channels per group a
        // multiple of 4, so a group is a whole number of the 4-channel row
        // quads the MFMA layout gives each lane half.  The staging buffers
        // are free after the main loop's last barrier.
        float *red = lds_x[0];          // [2 column waves][32 quads]
        float *gmean = lds_x[0] + 64;   // [32 quads]: mean of the quad's group
        const int qpg = p.gn_cpg >> 2;
        const int npx = (p.H - y0 < G::TR ? p.H - y0 : G::TR) * (p.W - x0 < TC ? p.W - x0 : TC);
        const float cnt = (float)(npx * p.gn_cpg);
        float q[2][4];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                float t = 0.f;
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    if (pv[j])
                        t += (acc[i][j][4 * rq] + acc[i][j][4 * rq + 1]) + (acc[i][j][4 * rq + 2] + acc[i][j][4 * rq + 3]);
                q[i][rq] = t;
            }
        half_wave_sum(q);
        if (l32 == 0)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) red[wn * 32 + wm * 16 + i * 8 + 2 * rq + half] = q[i][rq];
        __syncthreads();
        if (tid < 32) {
            const int g0 = (tid / qpg) * qpg;
            float t = 0.f;
            for (int k = 0; k < qpg; ++k) t += red[g0 + k] + red[32 + g0 + k];
            gmean[tid] = t / cnt;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const float mu = gmean[wm * 16 + i * 8 + 2 * rq + half];
                float t = 0.f;
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    if (pv[j])
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float d = acc[i][j][4 * rq + e] - mu;
                            t += d * d;
                        }
                q[i][rq] = t;
            }
        half_wave_sum(q);
        if (l32 == 0)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) red[wn * 32 + wm * 16 + i * 8 + 2 * rq + half] = q[i][rq];
        __syncthreads();
        const int gpb = kConvBM / p.gn_cpg;   // groups in this output-channel block
        if (tid < gpb) {
            float m2 = 0.f;
            for (int k = 0; k < qpg; ++k) m2 += red[tid * qpg + k] + red[32 + tid * qpg + k];
            const long long rec = (long long)(ob * gpb + tid) * p.gn_nrec + (long long)frame * gridDim.x + tile;
            p.gn_rec[rec] = floatx4{cnt, gmean[tid * qpg], m2, 0.f};
        }
    }
}

// Packed layout: [ob][dt][cb][k = c_local * 9 + tap][m], m in [0, 128);
// zero where the output channel or input channel is out of range.  One
// workgroup per chunk (ob, dt, cb): the 128 output channels' 36 weights are
// read along their rows (contiguous in [cout, cin, (kt,) 3, 3]) into LDS and
// written back transposed, so both sides are coalesced.
constexpr int kPackLd = kCK + 1;   // odd row stride: the transposed LDS reads hit distinct banks
__global__ __launch_bounds__(kThreads) void pack_conv3x3_kernel(const float *__restrict__ w, float *__restrict__ dst,
                                                                int cout, int cin, int kt, int n_cb) {
    __shared__ float t[kConvBM * kPackLd];
    const int cb = blockIdx.x, dt = blockIdx.y, ob = blockIdx.z;
    for (int e = threadIdx.x; e < kConvBM * kCK; e += kThreads) {
        const int m = e / kCK, k = e - (e / kCK) * kCK;
        const int o = ob * kConvBM + m, c = cb * kConvCC + k / 9, tap = k % 9;
        float v = 0.f;
        if (o < cout && c < cin) v = w[(((long long)o * cin + c) * kt + dt) * 9 + tap];
        t[m * kPackLd + k] = v;
    }
    __syncthreads();
    float *out = dst + (((long long)ob * kt + dt) * n_cb + cb) * (kCK * kConvBM);
    for (int e = threadIdx.x; e < kCK * kConvBM; e += kThreads) {
        const int k = e / kConvBM, m = e - (e / kConvBM) * kConvBM;
        out[e] = t[m * kPackLd + k];
    }
}

// y[o, :] = bias[o] + sum_s part[s, o, :] (+ res[o, :]), summed in split order.
constexpr int kRedElems = 4096;   // elements per workgroup

// Sum over the 256 threads of a workgroup; every thread gets the result.
__device__ inline float block_sum(float v, float *scratch) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    __syncthreads();   // scratch may still be read from a previous call
    if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
    __syncthreads();
    return (scratch[0] + scratch[1]) + (scratch[2] + scratch[3]);
}

// With gn_rec set, each workgroup also writes the GroupNorm record (count,
// mean, sum of squared deviations) of the elements it produced: record
// (o % cpg) * gridDim.x + blockIdx.x of group o / cpg.
template <bool VEC, bool RES>
__global__ __launch_bounds__(kThreads) void splitk_reduce(const float *__restrict__ part, long long part_stride,
                                                          int ksplit, const float *__restrict__ bias,
                                                          const float *res, float *y, long long plane,
                                                          floatx4 *__restrict__ gn_rec, int gn_cpg) {
    __shared__ float scratch[4];
    const int o = blockIdx.y;
    const long long base = (long long)o * plane;
    const long long lo = (long long)blockIdx.x * kRedElems;
    long long hi = lo + kRedElems;
    if (hi > plane) hi = plane;
    const float b = bias[o];
    float sum = 0.f;
    if (VEC) {
        for (long long i = lo / 4 + threadIdx.x; i < hi / 4; i += kThreads) {
            floatx4 v = {b, b, b, b};
            for (int sp = 0; sp < ksplit; ++sp)
                v += reinterpret_cast<const floatx4 *>(part + sp * part_stride + base)[i];
            if (RES) v += reinterpret_cast<const floatx4 *>(res + base)[i];
            reinterpret_cast<floatx4 *>(y + base)[i] = v;
            sum += (v[0] + v[1]) + (v[2] + v[3]);
        }
    } else {
        for (long long i = lo + threadIdx.x; i < hi; i += kThreads) {
            float v = b;
            for (int sp = 0; sp < ksplit; ++sp) v += part[sp * part_stride + base + i];
            if (RES) v += res[base + i];
            y[base + i] = v;
            sum += v;
        }
    }
    if (!gn_rec) return;   // uniform over the workgroup
    // Second pass over this thread's own outputs (program order: no barrier needed).
    const float cnt = (float)(hi - lo);
    const float mean = block_sum(sum, scratch) / cnt;
    float m2 = 0.f;
    if (VEC) {
        for (long long i = lo / 4 + threadIdx.x; i < hi / 4; i += kThreads) {
            const floatx4 d = reinterpret_cast<const floatx4 *>(y + base)[i] - mean;
            m2 += (d[0] * d[0] + d[1] * d[1]) + (d[2] * d[2] + d[3] * d[3]);
        }
    } else {
        for (long long i = lo + threadIdx.x; i < hi; i += kThreads) {
            const float d = y[base + i] - mean;
            m2 += d * d;
        }
    }
    m2 = block_sum(m2, scratch);
    if (threadIdx.x == 0) {
        const long long nrec = (long long)gn_cpg * gridDim.x;
        gn_rec[(long long)(o / gn_cpg) * nrec + (long long)(o % gn_cpg) * gridDim.x + blockIdx.x] =
            floatx4{cnt, mean, m2, 0.f};
    }
}

template <int TC, int MODE, bool RES>
void launch_t(const Params &p, bool split, dim3 grid, hipStream_t s) {
    if (split) hipLaunchKernelGGL((conv3x3_mfma<TC, MODE, false, true>), grid, dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL((conv3x3_mfma<TC, MODE, RES, false>), grid, dim3(kThreads), 0, s, p);
}

template <int TC>
void launch_tc(const Params &p, int mode, bool res, bool split, dim3 grid, hipStream_t s) {
    if (mode == MODE_UPSAMPLE) {
        if (res) launch_t<TC, MODE_UPSAMPLE, true>(p, split, grid, s);
        else launch_t<TC, MODE_UPSAMPLE, false>(p, split, grid, s);
    } else if (mode == MODE_DENORM) {
        if (res) launch_t<TC, MODE_DENORM, true>(p, split, grid, s);
        else launch_t<TC, MODE_DENORM, false>(p, split, grid, s);
    } else if (mode == MODE_GNSILU) {
        if (res) launch_t<TC, MODE_GNSILU, true>(p, split, grid, s);
        else launch_t<TC, MODE_GNSILU, false>(p, split, grid, s);
    } else {
        if (res) launch_t<TC, MODE_PLAIN, true>(p, split, grid, s);
        else launch_t<TC, MODE_PLAIN, false>(p, split, grid, s);
    }
}

}  // namespace

size_t conv3x3_packed_floats(int cout, int cin, int kt) {
    const size_t n_ob = (size_t)(cout + kConvBM - 1) / kConvBM;
    const size_t n_cb = (size_t)(cin + kConvCC - 1) / kConvCC;
    return n_ob * (size_t)kt * n_cb * kCK * kConvBM;
}

int32_t pack_conv3x3(const float *w, int cout, int cin, int kt, float *dst, hipStream_t s) {
    const int n_cb = (cin + kConvCC - 1) / kConvCC;
    const int n_ob = (cout + kConvBM - 1) / kConvBM;
    hipLaunchKernelGGL(pack_conv3x3_kernel, dim3((unsigned)n_cb, (unsigned)kt, (unsigned)n_ob), dim3(kThreads), 0, s,
                       w, dst, cout, cin, kt, n_cb);
    return check_launch("pack_conv3x3");
}

namespace {
std::atomic<int32_t> g_conv3x3_algorithm{VAE_CONV3X3_WINOGRAD_4X4};
}  // namespace

int32_t set_conv3x3_algorithm(int32_t algorithm) {
    if (algorithm != VAE_CONV3X3_WINOGRAD_2X2 && algorithm != VAE_CONV3X3_IMPLICIT_GEMM &&
        algorithm != VAE_CONV3X3_WINOGRAD_4X4) {
        set_error("vae_set_conv3x3_algorithm: unknown algorithm %d", algorithm);
        return VAE_ERR_INVALID_ARG;
    }
    g_conv3x3_algorithm.store(algorithm);
    return VAE_OK;
}

int32_t get_conv3x3_algorithm() { return g_conv3x3_algorithm.load(); }

int conv3x3_layout(int denorm, int upsample) {
    const int32_t alg = g_conv3x3_algorithm.load();
    if (denorm || alg == VAE_CONV3X3_IMPLICIT_GEMM) return 0;
    if (alg == VAE_CONV3X3_WINOGRAD_4X4) return upsample ? 4 : 3;
    return upsample ? 2 : 1;
}

bool conv3x3_layout_gn_on_load(int layout) { return layout <= 1; }

size_t conv3x3_pack_floats(int layout, int cout, int cin, int kt) {
    if (layout == 0) return conv3x3_packed_floats(cout, cin, kt);
    if (layout <= 2) return conv3x3_wino_packed_floats(cout, cin, kt, layout == 2);
    return conv3x3_wino4_packed_floats(cout, cin, kt, layout == 4);
}

size_t conv3x3_pack_floats_max(int cout, int cin, int kt) {
    size_t n = 0;
    for (int layout = 0; layout <= 4; ++layout) {
        const size_t m = conv3x3_pack_floats(layout, cout, cin, kt);
        if (m > n) n = m;
    }
    return n;
}

int32_t pack_conv3x3_layout(int layout, const float *w, int cout, int cin, int kt, float *dst, hipStream_t s) {
    if (layout == 0) return pack_conv3x3(w, cout, cin, kt, dst, s);
    if (layout <= 2) return pack_conv3x3_wino(w, cout, cin, kt, layout == 2, dst, s);
    return pack_conv3x3_wino4(w, cout, cin, kt, layout == 4, dst, s);
}

namespace {
int conv_tc(int W) { return W > 16 ? 32 : (W > 8 ? 16 : 8); }
constexpr int kSlots = 256 * 3;   // CUs x resident conv workgroups per CU
}  // namespace

namespace {
int mfma_ksplit(int cout, int cin, int kt, int H, int W, int T) {
    const int TC = conv_tc(W), TR = kConvBN / TC;
    const long long base = (long long)((W + TC - 1) / TC) * ((H + TR - 1) / TR) *
                           ((cout + kConvBM - 1) / kConvBM) * T;
    if (base >= kSlots) return 1;
    const int n_iter = kt * ((cin + kConvCC - 1) / kConvCC);
    long long s = (2 * kSlots + base - 1) / base;   // about two rounds of workgroups
    if (s > n_iter / 8) s = n_iter / 8;              // each split keeps >= 8 K chunks
    if (s > 16) s = 16;
    if (s * T > 65535) s = 65535 / T;
    return s < 1 ? 1 : (int)s;
}

}  // namespace

int conv3x3_ksplit(const ConvLaunch &a) {
    if (a.wino >= 3) return conv3x3_wino4_ksplit(a);
    return a.wino ? conv3x3_wino_ksplit(a) : mfma_ksplit(a.cout, a.cin, a.kt, a.H, a.W, a.T);
}

size_t conv3x3_partial_floats(const ConvLaunch &a) {
    const int ks = conv3x3_ksplit(a);
    return ks > 1 ? (size_t)ks * a.cout * a.T * (size_t)a.H * a.W : 0;
}

int conv3x3_gn_records(const ConvLaunch &a) {
    if (a.cout % 32 != 0) return 0;
    const long long plane = (long long)a.T * a.H * a.W;
    if (conv3x3_ksplit(a) > 1)
        return (int)((a.cout / 32) * ((plane + kRedElems - 1) / kRedElems));
    if (a.wino >= 3) return conv3x3_wino4_gn_records(a);
    if (a.wino) return conv3x3_wino_gn_records(a);
    if (a.cout % kConvBM != 0 || (a.cout / 32) % 4 != 0) return 0;
    const int TC = conv_tc(a.W), TR = kConvBN / TC;
    return ((a.W + TC - 1) / TC) * ((a.H + TR - 1) / TR) * a.T;
}

const char *conv3x3_kernel_name(const ConvLaunch &a) {
    static const char *algos[3] = {"mfma", "wino", "wino4"};
    static const char *tcs[4] = {"32", "16", "8", "4"};
    static const char *modes[4] = {"plain", "up2x", "denorm", "gnsilu"};
    static const char *tails[3] = {"", ",res", ",splitk"};
    static char names[3][4][4][3][48];
    static bool init = false;
    if (!init) {
        for (int g = 0; g < 3; ++g)
            for (int t = 0; t < 4; ++t)
                for (int m = 0; m < 4; ++m)
                    for (int k = 0; k < 3; ++k)
                        snprintf(names[g][t][m][k], sizeof names[g][t][m][k], "conv3x3_%s<%s,%s%s>", algos[g], tcs[t],
                                 modes[m], tails[k]);
        init = true;
    }
    // column tile width: the implicit GEMM's output columns, the Winograd form's tiles per row
    const int tc = a.wino >= 3 ? conv3x3_wino4_tcw(a) : (a.wino ? conv3x3_wino_tcw(a) : conv_tc(a.W));
    const int ti = tc == 32 ? 0 : (tc == 16 ? 1 : (tc == 8 ? 2 : 3));
    const int mi = a.upsample ? 1 : (a.denorm ? 2 : (a.gn_coef ? 3 : 0));
    const int si = conv3x3_ksplit(a) > 1 ? 2 : (a.res ? 1 : 0);
    return names[a.wino >= 3 ? 2 : (a.wino ? 1 : 0)][ti][mi][si];
}

int32_t launch_conv3x3_main(const ConvLaunch &a, hipStream_t s) {
    if (a.wino >= 3) return launch_conv3x3_wino4_main(a, s);
    if (a.wino) return launch_conv3x3_wino_main(a, s);
    Params p;
    p.x = a.x;
    p.wpk = a.wpk;
    p.bias = a.bias;
    p.res = a.res;
    p.y = a.y;
    p.cin = a.cin;
    p.cout = a.cout;
    p.H = a.H;
    p.W = a.W;
    p.Win = a.upsample ? a.W / 2 : a.W;
    const int Hin = a.upsample ? a.H / 2 : a.H;
    p.kt = a.kt;
    p.n_cb = (a.cin + kConvCC - 1) / kConvCC;
    p.in_fstride = (long long)Hin * p.Win;
    p.in_cstride = p.in_fstride * a.T;
    p.out_fstride = (long long)a.H * a.W;
    p.out_cstride = p.out_fstride * a.T;
    p.dn_scale = a.dn_scale;
    p.dn_shift = a.dn_shift;
    const int TC = conv_tc(a.W);
    const int TR = kConvBN / TC;
    p.tiles_x = (a.W + TC - 1) / TC;
    const int tiles_y = (a.H + TR - 1) / TR;
    p.ksplit = mfma_ksplit(a.cout, a.cin, a.kt, a.H, a.W, a.T);
    p.part = a.part;
    p.part_stride = p.out_cstride * a.cout;
    if (p.ksplit > 1 && !a.part) {
        set_error("conv3x3: split-K needs a partial-sum workspace");
        return VAE_ERR_WORKSPACE;
    }
    // byte offsets inside one channel chunk are 32-bit
    if (p.in_cstride * kConvCC * 4 >= (1LL << 31)) {
        set_error("conv3x3: input plane of %lld elements is too large", p.in_cstride);
        return VAE_ERR_UNSUPPORTED;
    }
    const dim3 grid((unsigned)(p.tiles_x * tiles_y), (unsigned)((a.cout + kConvBM - 1) / kConvBM),
                    (unsigned)(a.T * p.ksplit));
    if (a.gn_coef && (a.upsample || a.denorm || a.cin > kGnMaxChannels)) {
        set_error("conv3x3: GroupNorm-on-load needs a plain input of at most %d channels", kGnMaxChannels);
        return VAE_ERR_UNSUPPORTED;
    }
    p.gn_coef = a.gn_coef;
    p.gn_rec = nullptr;
    p.gn_cpg = 0;
    p.gn_nrec = 0;
    if (a.gn_rec && p.ksplit == 1) {
        if (conv3x3_gn_records(a) == 0) {
            set_error("conv3x3: GroupNorm records in the epilogue need out_channels %% 128 == 0");
            return VAE_ERR_UNSUPPORTED;
        }
        p.gn_rec = a.gn_rec;
        p.gn_cpg = a.cout / 32;
        p.gn_nrec = (int)(grid.x * grid.z);
    }
    const int mode = a.upsample ? MODE_UPSAMPLE : (a.denorm ? MODE_DENORM : (a.gn_coef ? MODE_GNSILU : MODE_PLAIN));
    const bool res = a.res != nullptr;
    const bool split = p.ksplit > 1;
    if (TC == 32) launch_tc<32>(p, mode, res, split, grid, s);
    else if (TC == 16) launch_tc<16>(p, mode, res, split, grid, s);
    else launch_tc<8>(p, mode, res, split, grid, s);
    return check_launch("conv3x3_mfma");
}

int32_t launch_conv3x3_reduce(const ConvLaunch &a, hipStream_t s) {
    const int ksplit = conv3x3_ksplit(a);
    if (ksplit == 1) return VAE_OK;
    const long long plane = (long long)a.T * a.H * a.W;
    const long long part_stride = plane * a.cout;
    const bool res = a.res != nullptr;
    const dim3 rgrid((unsigned)((plane + kRedElems - 1) / kRedElems), (unsigned)a.cout);
    floatx4 *rec = a.gn_rec;
    const int cpg = a.cout / 32;
    if (rec && a.cout % 32 != 0) {
        set_error("splitk_reduce: GroupNorm records need out_channels %% 32 == 0");
        return VAE_ERR_UNSUPPORTED;
    }
    const bool vec = plane % 4 == 0 && (reinterpret_cast<uintptr_t>(a.y) & 15) == 0 &&
                     (reinterpret_cast<uintptr_t>(a.part) & 15) == 0 &&
                     (!res || (reinterpret_cast<uintptr_t>(a.res) & 15) == 0);
    if (vec) {
        if (res) hipLaunchKernelGGL((splitk_reduce<true, true>), rgrid, dim3(kThreads), 0, s, a.part, part_stride, ksplit, a.bias, a.res, a.y, plane, rec, cpg);
        else hipLaunchKernelGGL((splitk_reduce<true, false>), rgrid, dim3(kThreads), 0, s, a.part, part_stride, ksplit, a.bias, a.res, a.y, plane, rec, cpg);
    } else {
        if (res) hipLaunchKernelGGL((splitk_reduce<false, true>), rgrid, dim3(kThreads), 0, s, a.part, part_stride, ksplit, a.bias, a.res, a.y, plane, rec, cpg);
        else hipLaunchKernelGGL((splitk_reduce<false, false>), rgrid, dim3(kThreads), 0, s, a.part, part_stride, ksplit, a.bias, a.res, a.y, plane, rec, cpg);
    }
    return check_launch("splitk_reduce");
}

int32_t launch_conv3x3(const ConvLaunch &a, hipStream_t s) {
    int32_t rc = launch_conv3x3_main(a, s);
    if (rc != VAE_OK) return rc;
    return launch_conv3x3_reduce(a, s);
}

int32_t launch_rows_reduce(const float *part, long long part_stride, int splits, const float *bias, float *y,
                           long long plane, int rows, hipStream_t s) {
    const dim3 rgrid((unsigned)((plane + kRedElems - 1) / kRedElems), (unsigned)rows);
    const bool vec = plane % 4 == 0 && (reinterpret_cast<uintptr_t>(y) & 15) == 0 &&
                     (reinterpret_cast<uintptr_t>(part) & 15) == 0 && part_stride % 4 == 0;
    if (vec)
        hipLaunchKernelGGL((splitk_reduce<true, false>), rgrid, dim3(kThreads), 0, s, part, part_stride, splits,
                           bias, nullptr, y, plane, nullptr, 0);
    else
        hipLaunchKernelGGL((splitk_reduce<false, false>), rgrid, dim3(kThreads), 0, s, part, part_stride, splits,
                           bias, nullptr, y, plane, nullptr, 0);
    return check_launch("splitk_reduce");
}

}  // namespace vae
