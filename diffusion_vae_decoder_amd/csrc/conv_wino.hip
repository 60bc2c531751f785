// Winograd F(2x2, 3x3) form of the decoder's 3x3 convolutions on FP32 MFMA.
//
// The conv (cortiq-engine 0.7.7 `vae`, VaeConvRef: stride 1, zero padding
// 1, cross-correlation) computes each 2 x 2 block of outputs from the 4 x 4
// input patch d around it.  With the minimal filtering algorithm of Lavin and
// Gray (Fast Algorithms for Convolutional Neural Networks, 2016),
//     Y = A^T [ sum_c (G g_c G^T) . (B^T d_c B) ] A        (. elementwise)
//     B^T = [1 0 -1 0; 0 1 1 0; 0 -1 1 0; 0 1 0 -1]
//     G   = [1 0 0; 1/2 1/2 1/2; 1/2 -1/2 1/2; 0 0 1]
//     A^T = [1 1 1 0; 0 1 -1 -1]
// the sum over input channels c becomes 16 independent GEMMs, one per point
// xi of the 4 x 4 transform: M_xi[o, tile] = sum_c U_xi[o, c] V_xi[c, tile],
// with 16 multiplies per 2 x 2 outputs and channel pair instead of 36.
// U = G g G^T is formed once, in double precision, when the weights are
// packed.  The result equals the direct conv up to rounding (about 1e-6 of
// the output's magnitude in float32 at the decoder's shapes).
//
// Nearest-x2 upsampled input (VaeUpRef): a 2 x 2 output block at even
// coordinates reads the upsampled rows 2i-1, 2i, 2i+1, 2i+2, which are the
// source rows i-1, i, i, i+1.  Rows 1 and 2 of d coincide, so row (and
// column) 2 of B^T d B vanishes and 9 of the 16 points remain; rows 1 of
// B^T d B double.  The kernel reads the 3 x 3 source patch directly and the
// factors 2 are folded into U (exact).  That is 9 multiplies per 2 x 2
// outputs and channel pair instead of 36.
//
// Workgroup: 4 waves; wave w owns output channels [32w, 32w + 32) of the
// workgroup's 128 and all 32 tiles (2 x 2 output blocks) of the workgroup's
// 4 x 32, 8 x 16 or 16 x 8 output block.  Each lane transforms one
// (channel, tile) patch per step in registers: lane l takes tile l % 32 and
// channel l / 32 of the step's channel pair, which is exactly the B operand
// of v_mfma_f32_32x32x2_f32 for every point xi, so the input needs no LDS and
// the kernel no barrier in its main loop.  The transformed weights U are
// packed per (32-channel block, step, lane) and read straight into
// registers.  All 16 (or 9) accumulators of a lane hold the same (output
// channel, tile) entries, so the output transform is lane-local.  The 256
// accumulator registers allow one wave per SIMD; loads run two steps ahead.

#include <cstdio>

#include "vae_internal.h"

namespace vae {

namespace {

constexpr int kWThreads = 256;
constexpr int kWavesOut = 32;               // output channels per wave
constexpr int kWOOB = 0x7FFFFFF0;           // buffer offset past every range: reads 0
constexpr int kWPrefetch = 2;               // steps loaded ahead

template <bool UP>
struct WinoShape {
    static constexpr int NX = UP ? 9 : 16;      // transform points
    static constexpr int NXP = UP ? 12 : 16;    // packed floats per lane and step
    static constexpr int NP = UP ? 3 : 4;       // input rows (and columns) of a tile's patch
    static constexpr int NQ = NXP / 4;          // float4 loads of U per step
};

struct WParams {
    const float *x;         // input [cin, T, Hin, Win]
    const float *u;         // packed U
    const float *bias, *res;
    const float *gn_coef;   // GroupNorm + SiLU on load: (mean, scale, beta, -) per input channel
    float *y;
    float *part;            // split-K partial sums [ksplit][cout][T][H][W]
    floatx4 *gn_rec;        // GroupNorm records of y, as for the implicit-GEMM conv
    int cin, cout, H, W, Hin, Win, kt, npairs, tiles_x, ksplit, gn_cpg, gn_nrec;
    long long in_cstride, in_fstride, out_cstride, out_fstride, part_stride;
};

__device__ __attribute__((always_inline)) inline __amdgpu_buffer_rsrc_t wino_rsrc(const float *base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), (short)0, (int)bytes, 0x00020000);
}

// Next step to load: time tap dt, channel pair, the pair's first channel in
// the tap's frame and the lane's packed U.  Advanced by additions only.
struct WCursor {
    int pair, dt;
    const float *x;
    const floatx4 *u;
};

__device__ __attribute__((always_inline)) inline const float *wino_frame(const WParams &p, int frame, int dt) {
    int fr = frame + dt - (p.kt - 1);
    fr = fr < 0 ? 0 : fr;
    return p.x + (long long)fr * p.in_fstride;
}

// One step's operands in registers: the lane's input patch, its packed U
// and, for GroupNorm on load, the coefficients of the lane's channel.
template <bool UP, bool GN>
struct WSlot {
    float d[WinoShape<UP>::NP * WinoShape<UP>::NP];
    floatx4 u[WinoShape<UP>::NQ];
    floatx4 cf;
    bool cok;   // the lane's channel is below cin
};

template <bool UP, bool GN>
__device__ __attribute__((always_inline)) inline void wino_load(const WParams &p, const WCursor &c, int h,
                                                               const int (&boff)[WinoShape<UP>::NP * WinoShape<UP>::NP],
                                                               WSlot<UP, GN> &sl) {
    using S = WinoShape<UP>;
    const int rem = p.cin - 2 * c.pair;
    const int nc = rem < 2 ? rem : 2;
    const __amdgpu_buffer_rsrc_t xr = wino_rsrc(c.x, (unsigned)(nc * p.in_cstride * 4));
#pragma unroll
    for (int i = 0; i < S::NP * S::NP; ++i)
        sl.d[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(xr, boff[i], 0, 0));
#pragma unroll
    for (int i = 0; i < S::NQ; ++i) sl.u[i] = c.u[i];
    if (GN) {
        const int ch = 2 * c.pair + h;
        sl.cok = ch < p.cin;
        sl.cf = *reinterpret_cast<const floatx4 *>(p.gn_coef + 4 * (ch < p.cin ? ch : p.cin - 1));
    }
}

__device__ __attribute__((always_inline)) inline void wino_next(const WParams &p, int frame, int ustep, WCursor &c) {
    c.u += ustep;
    if (++c.pair == p.npairs) {
        c.pair = 0;
        ++c.dt;
        c.x = wino_frame(p, frame, c.dt);
    } else {
        c.x += 2 * p.in_cstride;
    }
}

// Input transform of the lane's patch and the step's MFMAs.
// GN: the patch is first normalised, silu((x - mean) * scale + beta), with
// padding positions (bit clear in vmask) and channels past cin kept at 0.
template <bool UP, bool GN>
__device__ __attribute__((always_inline)) inline void wino_step(const WSlot<UP, GN> &sl, unsigned vmask,
                                                               floatx16 (&acc)[WinoShape<UP>::NX]) {
    constexpr int NPP = WinoShape<UP>::NP * WinoShape<UP>::NP;
    float d[NPP];
#pragma unroll
    for (int i = 0; i < NPP; ++i) {
        if (GN) {
            float t = (sl.d[i] - sl.cf[0]) * sl.cf[1] + sl.cf[2];
            t = t * __builtin_amdgcn_rcpf(1.f + __expf(-t));
            d[i] = (((vmask >> i) & 1u) && sl.cok) ? t : 0.f;
        } else {
            d[i] = sl.d[i];
        }
    }
    const floatx4 (&u)[WinoShape<UP>::NQ] = sl.u;
    float v[WinoShape<UP>::NX];
    if (!UP) {
        float t[4][4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            t[0][q] = d[q] - d[8 + q];
            t[1][q] = d[4 + q] + d[8 + q];
            t[2][q] = d[8 + q] - d[4 + q];
            t[3][q] = d[4 + q] - d[12 + q];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            v[4 * r + 0] = t[r][0] - t[r][2];
            v[4 * r + 1] = t[r][1] + t[r][2];
            v[4 * r + 2] = t[r][2] - t[r][1];
            v[4 * r + 3] = t[r][1] - t[r][3];
        }
    } else {
        // source patch e (3 x 3): transform points (0, 1, 3) of each axis, the
        // factor 2 of point 1 being in U
        float t[3][3];
#pragma unroll
        for (int q = 0; q < 3; ++q) {
            t[0][q] = d[q] - d[3 + q];
            t[1][q] = d[3 + q];
            t[2][q] = d[3 + q] - d[6 + q];
        }
#pragma unroll
        for (int r = 0; r < 3; ++r) {
            v[3 * r + 0] = t[r][0] - t[r][1];
            v[3 * r + 1] = t[r][1];
            v[3 * r + 2] = t[r][1] - t[r][2];
        }
    }
#pragma unroll
    for (int k = 0; k < WinoShape<UP>::NX; ++k)
        acc[k] = __builtin_amdgcn_mfma_f32_32x32x2f32(u[k >> 2][k & 3], v[k], acc[k], 0, 0, 0);
}

// Output transform of register r of every accumulator: the lane's 2 x 2 outputs.
template <bool UP>
__device__ __attribute__((always_inline)) inline void wino_out(const floatx16 (&acc)[WinoShape<UP>::NX], int r,
                                                              float (&y)[2][2]) {
    if (!UP) {
        float s[2][4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            s[0][c] = (acc[c][r] + acc[4 + c][r]) + acc[8 + c][r];
            s[1][c] = (acc[4 + c][r] - acc[8 + c][r]) - acc[12 + c][r];
        }
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            y[a][0] = (s[a][0] + s[a][1]) + s[a][2];
            y[a][1] = (s[a][1] - s[a][2]) - s[a][3];
        }
    } else {
        float s[2][3];
#pragma unroll
        for (int c = 0; c < 3; ++c) {
            s[0][c] = acc[c][r] + acc[3 + c][r];
            s[1][c] = acc[3 + c][r] - acc[6 + c][r];
        }
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            y[a][0] = s[a][0] + s[a][1];
            y[a][1] = s[a][1] - s[a][2];
        }
    }
}

// (n, mean, M2) of a set merged with (nb, mb, qb) of another (pairwise update
// of Chan, Golub and LeVeque); empty sets (n = 0) merge as the identity.
__device__ __attribute__((always_inline)) inline void wino_chan_merge(float (&a)[3], float nb, float mb, float qb) {
    const float nt = a[0] + nb;
    const float delta = mb - a[1];
    const float fb = nt > 0.f ? nb / nt : 0.f;
    a[2] = (a[2] + qb) + delta * delta * a[0] * fb;
    a[1] = a[1] + delta * fb;
    a[0] = nt;
}

template <int TC, bool UP, bool GN, bool RES, bool SPLIT>
__global__ __launch_bounds__(kWThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void conv3x3_wino(WParams p) {
    using S = WinoShape<UP>;
    constexpr int TCT = TC / 2;            // tiles per row
    constexpr int TRT = 32 / TCT;          // rows of tiles
    constexpr int TR = 2 * TRT;            // output rows of the block

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, n = lane & 31;

    // XCD-aware renumbering, as in the implicit-GEMM conv.
    int tile = blockIdx.x;
    if ((gridDim.x & 7) == 0) tile = (tile & 7) * (gridDim.x >> 3) + (tile >> 3);
    const int ty = tile / p.tiles_x;
    const int tx = tile - ty * p.tiles_x;
    const int y0 = ty * TR, x0 = tx * TC;
    const int ob = blockIdx.y;
    const int frame = SPLIT ? blockIdx.z / p.ksplit : blockIdx.z;
    const int split = SPLIT ? blockIdx.z - frame * p.ksplit : 0;

    const int tr = n / TCT, tc = n - (n / TCT) * TCT;
    const int Y0 = y0 + 2 * tr, X0 = x0 + 2 * tc;   // the lane's tile (top-left output)

    // Byte offsets of the lane's patch from its channel pair's first channel
    // (kWOOB for zero padding); the same for every step.
    int boff[S::NP * S::NP];
    unsigned vmask = 0;   // bit i: patch element i lies in the image
    {
        const int ry = UP ? (Y0 >> 1) - 1 : Y0 - 1;
        const int rx = UP ? (X0 >> 1) - 1 : X0 - 1;
        const int Hs = UP ? p.Hin : p.H, Ws = UP ? p.Win : p.W;
#pragma unroll
        for (int r = 0; r < S::NP; ++r)
#pragma unroll
            for (int q = 0; q < S::NP; ++q) {
                const int yy = ry + r, xx = rx + q;
                const bool ok = yy >= 0 && yy < Hs && xx >= 0 && xx < Ws;
                boff[r * S::NP + q] = ok ? (int)((h * p.in_cstride + (long long)yy * Ws + xx) * 4) : kWOOB;
                vmask |= (ok ? 1u : 0u) << (r * S::NP + q);
            }
    }

    const int nsteps = p.kt * p.npairs;
    const int s0 = SPLIT ? (int)((long long)split * nsteps / p.ksplit) : 0;
    const int s1 = SPLIT ? (int)((long long)(split + 1) * nsteps / p.ksplit) : nsteps;
    constexpr int USTEP = 64 * S::NQ;    // float4s of U per step (all lanes)
    const int cb32 = ob * (kConvBM / kWavesOut) + wave;

    WCursor cur;
    cur.dt = s0 / p.npairs;
    cur.pair = s0 - cur.dt * p.npairs;
    cur.x = wino_frame(p, frame, cur.dt) + 2LL * cur.pair * p.in_cstride;
    cur.u = reinterpret_cast<const floatx4 *>(p.u) + ((size_t)cb32 * nsteps + s0) * USTEP + lane * S::NQ;

    floatx16 acc[S::NX];
#pragma unroll
    for (int k = 0; k < S::NX; ++k)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[k][r] = 0.f;

    constexpr int NB = kWPrefetch + 1;
    WSlot<UP, GN> sl[NB];
#pragma unroll
    for (int j = 0; j < kWPrefetch; ++j)
        if (s0 + j < s1) {
            wino_load<UP, GN>(p, cur, h, boff, sl[j]);
            wino_next(p, frame, USTEP, cur);
        }
    // Steady state: groups of NB steps whose prefetches all lie in range, with
    // no branch around a load (step s uses register slot (s - s0) % NB).
    int s = s0;
    for (; s + NB + kWPrefetch <= s1; s += NB) {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            wino_load<UP, GN>(p, cur, h, boff, sl[(j + kWPrefetch) % NB]);
            wino_next(p, frame, USTEP, cur);
            wino_step<UP, GN>(sl[j], vmask, acc);
        }
    }
    // The last (fewer than NB + kWPrefetch) steps.
#pragma unroll
    for (int j = 0; j < NB + kWPrefetch - 1; ++j) {
        if (s + j < s1) {
            if (s + j + kWPrefetch < s1) {
                wino_load<UP, GN>(p, cur, h, boff, sl[(j + kWPrefetch) % NB]);
                wino_next(p, frame, USTEP, cur);
            }
            wino_step<UP, GN>(sl[j % NB], vmask, acc);
        }
    }

    // Epilogue: register r of a 32x32 MFMA tile is output channel
    // 8 (r / 4) + 4 h + r % 4 of the wave's block, for the lane's tile n.
    const long long fo = (long long)frame * p.out_fstride;
    const int obase = ob * kConvBM + wave * kWavesOut + 4 * h;
    bool pv[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) pv[a][b] = Y0 + a < p.H && X0 + b < p.W;
    // in-image position of each output, clamped (branch-free residual reads)
    long long sp[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
            sp[a][b] = fo + (long long)min(Y0 + a, p.H - 1) * p.W + min(X0 + b, p.W - 1);
    const float nval = (float)((pv[0][0] + pv[0][1] + pv[1][0] + pv[1][1]) * 4);

    // Per 4-channel quad rq of the lane: its 16 outputs, and, for GroupNorm
    // records, their count, mean and sum of squared deviations (st).
    float st[4][3];
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
        float rv[4][4];
        if (RES && !SPLIT) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int o = min(obase + 8 * rq + k, p.cout - 1);
#pragma unroll
                for (int e = 0; e < 4; ++e) rv[k][e] = p.res[(long long)o * p.out_cstride + sp[e >> 1][e & 1]];
            }
        }
        float val[4][4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int r = 4 * rq + k;
            const int o = obase + 8 * rq + k;
            float yv[2][2];
            wino_out<UP>(acc, r, yv);
            const long long base = (long long)min(o, p.cout - 1) * p.out_cstride;
            const float bo = SPLIT ? 0.f : p.bias[min(o, p.cout - 1)];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float v = yv[e >> 1][e & 1] + bo;
                if (RES && !SPLIT) v += rv[k][e];
                val[k][e] = v;
                if (o < p.cout && pv[e >> 1][e & 1]) {
                    if (SPLIT) p.part[split * p.part_stride + base + sp[e >> 1][e & 1]] = v;
                    else p.y[base + sp[e >> 1][e & 1]] = v;
                }
            }
        }
        if (!SPLIT && p.gn_rec) {
            float t = 0.f;
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (pv[e >> 1][e & 1]) t += val[k][e];
            const float mean = nval > 0.f ? t / nval : 0.f;
            float m2 = 0.f;
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (pv[e >> 1][e & 1]) {
                        const float dv = val[k][e] - mean;
                        m2 += dv * dv;
                    }
            st[rq][0] = nval;
            st[rq][1] = mean;
            st[rq][2] = m2;
        }
    }

    if (!SPLIT && p.gn_rec) {
        // GroupNorm records of the workgroup's outputs: per group (count, mean,
        // sum of squared deviations from that mean), merged pairwise (Chan,
        // Golub and LeVeque) over the 32 tiles of a lane half, then over the
        // quads of a group.  The host enables this only for cout % 128 == 0 and
        // channels per group a multiple of 4: a group is then a whole number of
        // quads.
        __shared__ float qst[32][3];   // per quad of the workgroup's 128 channels
#pragma unroll
        for (int o = 1; o < 32; o <<= 1)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const float nb = __shfl_xor(st[rq][0], o, 64);
                const float mb = __shfl_xor(st[rq][1], o, 64);
                const float qb = __shfl_xor(st[rq][2], o, 64);
                wino_chan_merge(st[rq], nb, mb, qb);
            }
        if (n == 0)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const int qd = wave * 8 + 2 * rq + h;
                qst[qd][0] = st[rq][0];
                qst[qd][1] = st[rq][1];
                qst[qd][2] = st[rq][2];
            }
        __syncthreads();
        const int qpg = p.gn_cpg >> 2;
        const int gpb = kConvBM / p.gn_cpg;
        if (tid < gpb) {
            float g[3] = {qst[tid * qpg][0], qst[tid * qpg][1], qst[tid * qpg][2]};
            for (int k = 1; k < qpg; ++k) wino_chan_merge(g, qst[tid * qpg + k][0], qst[tid * qpg + k][1], qst[tid * qpg + k][2]);
            const long long rec = (long long)(ob * gpb + tid) * p.gn_nrec + (long long)frame * gridDim.x + tile;
            p.gn_rec[rec] = floatx4{g[0], g[1], g[2], 0.f};
        }
    }
}


// Packed U: [cout block of 32][step = (dt, channel pair)][lane][NXP], lane =
// (channel of the pair) * 32 + (output channel in the block); zero where the
// output or input channel is out of range.  One thread per (block, step, lane).
template <bool UP>
__global__ __launch_bounds__(256) void pack_wino_kernel(const float *__restrict__ w, float *__restrict__ dst, int cout,
                                                        int cin, int kt, int npairs, long long total) {
    using S = WinoShape<UP>;
    const long long id = (long long)blockIdx.x * 256 + threadIdx.x;
    if (id >= total) return;
    const int lane = (int)(id & 63);
    const long long bs = id >> 6;
    const int nsteps = kt * npairs;
    const int cb32 = (int)(bs / nsteps);
    const int s = (int)(bs - (long long)cb32 * nsteps);
    const int dt = s / npairs, pair = s - dt * npairs;
    const int o = cb32 * kWavesOut + (lane & 31);
    const int c = 2 * pair + (lane >> 5);
    double g[3][3];
#pragma unroll
    for (int i = 0; i < 9; ++i)
        g[i / 3][i % 3] = (o < cout && c < cin) ? (double)w[(((long long)o * cin + c) * kt + dt) * 9 + i] : 0.0;
    // U = G g G^T
    const double G[4][3] = {{1.0, 0.0, 0.0}, {0.5, 0.5, 0.5}, {0.5, -0.5, 0.5}, {0.0, 0.0, 1.0}};
    double t[4][3];
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int j = 0; j < 3; ++j) t[x][j] = G[x][0] * g[0][j] + G[x][1] * g[1][j] + G[x][2] * g[2][j];
    float *out = dst + id * S::NXP;
    if (!UP) {
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
            for (int y = 0; y < 4; ++y) out[4 * x + y] = (float)(t[x][0] * G[y][0] + t[x][1] * G[y][1] + t[x][2] * G[y][2]);
    } else {
        const int pts[3] = {0, 1, 3};
#pragma unroll
        for (int ix = 0; ix < 3; ++ix)
#pragma unroll
            for (int iy = 0; iy < 3; ++iy) {
                const int x = pts[ix], y = pts[iy];
                const double f = (ix == 1 ? 2.0 : 1.0) * (iy == 1 ? 2.0 : 1.0);
                out[3 * ix + iy] = (float)(f * (t[x][0] * G[y][0] + t[x][1] * G[y][1] + t[x][2] * G[y][2]));
            }
#pragma unroll
        for (int k = 9; k < S::NXP; ++k) out[k] = 0.f;
    }
}

int wino_tc(int W) { return W > 16 ? 32 : (W > 8 ? 16 : 8); }

template <int TC, bool UP, bool GN>
void wino_launch_t(const WParams &p, bool res, bool split, dim3 grid, hipStream_t s) {
    if (split) hipLaunchKernelGGL((conv3x3_wino<TC, UP, GN, false, true>), grid, dim3(kWThreads), 0, s, p);
    else if (res) hipLaunchKernelGGL((conv3x3_wino<TC, UP, GN, true, false>), grid, dim3(kWThreads), 0, s, p);
    else hipLaunchKernelGGL((conv3x3_wino<TC, UP, GN, false, false>), grid, dim3(kWThreads), 0, s, p);
}

template <int TC>
void wino_launch_tc(const WParams &p, bool up, bool gn, bool res, bool split, dim3 grid, hipStream_t s) {
    if (up) wino_launch_t<TC, true, false>(p, res, split, grid, s);
    else if (gn) wino_launch_t<TC, false, true>(p, res, split, grid, s);
    else wino_launch_t<TC, false, false>(p, res, split, grid, s);
}

}  // namespace

size_t conv3x3_wino_packed_floats(int cout, int cin, int kt, int up) {
    const size_t ncb32 = (size_t)((cout + kConvBM - 1) / kConvBM) * (kConvBM / kWavesOut);
    const size_t nsteps = (size_t)kt * ((cin + 1) / 2);
    return ncb32 * nsteps * 64 * (up ? WinoShape<true>::NXP : WinoShape<false>::NXP);
}

int32_t pack_conv3x3_wino(const float *w, int cout, int cin, int kt, int up, float *dst, hipStream_t s) {
    const int npairs = (cin + 1) / 2;
    const long long ncb32 = (long long)((cout + kConvBM - 1) / kConvBM) * (kConvBM / kWavesOut);
    const long long total = ncb32 * kt * npairs * 64;
    const dim3 grid((unsigned)((total + 255) / 256));
    if (up) hipLaunchKernelGGL(pack_wino_kernel<true>, grid, dim3(256), 0, s, w, dst, cout, cin, kt, npairs, total);
    else hipLaunchKernelGGL(pack_wino_kernel<false>, grid, dim3(256), 0, s, w, dst, cout, cin, kt, npairs, total);
    return check_launch("pack_conv3x3_wino");
}

int32_t launch_conv3x3_wino_main(const ConvLaunch &a, hipStream_t s) {
    if (a.denorm || (a.gn_coef && a.upsample)) {
        set_error("conv3x3_wino: no de-normalisation, and no GroupNorm on load of an upsampled input");
        return VAE_ERR_UNSUPPORTED;
    }
    if ((a.wino == 2) != (a.upsample != 0)) {
        set_error("conv3x3_wino: weights packed for %s input", a.wino == 2 ? "an upsampled" : "a plain");
        return VAE_ERR_INVALID_ARG;
    }
    if (a.gn_coef && (reinterpret_cast<uintptr_t>(a.gn_coef) & 15)) {
        set_error("conv3x3_wino: GroupNorm coefficients must be 16-byte aligned");
        return VAE_ERR_INVALID_ARG;
    }
    WParams p;
    p.x = a.x;
    p.u = a.wpk;
    p.bias = a.bias;
    p.res = a.res;
    p.gn_coef = a.gn_coef;
    p.y = a.y;
    p.cin = a.cin;
    p.cout = a.cout;
    p.H = a.H;
    p.W = a.W;
    p.Hin = a.upsample ? a.H / 2 : a.H;
    p.Win = a.upsample ? a.W / 2 : a.W;
    p.kt = a.kt;
    p.npairs = (a.cin + 1) / 2;
    p.in_fstride = (long long)p.Hin * p.Win;
    p.in_cstride = p.in_fstride * a.T;
    p.out_fstride = (long long)a.H * a.W;
    p.out_cstride = p.out_fstride * a.T;
    const int TC = wino_tc(a.W);
    const int TR = 128 / TC;
    p.tiles_x = (a.W + TC - 1) / TC;
    const int tiles_y = (a.H + TR - 1) / TR;
    p.ksplit = conv3x3_ksplit(a.cout, a.cin, a.kt, a.H, a.W, a.T);
    p.part = a.part;
    p.part_stride = p.out_cstride * a.cout;
    if (p.ksplit > 1 && !a.part) {
        set_error("conv3x3_wino: split-K needs a partial-sum workspace");
        return VAE_ERR_WORKSPACE;
    }
    if (p.in_cstride * 2 * 4 >= (1LL << 31)) {
        set_error("conv3x3_wino: input plane of %lld elements is too large", p.in_cstride);
        return VAE_ERR_UNSUPPORTED;
    }
    if (a.upsample && ((a.H | a.W) & 1)) {
        set_error("conv3x3_wino: an upsampled input has even sizes");
        return VAE_ERR_INVALID_ARG;
    }
    const dim3 grid((unsigned)(p.tiles_x * tiles_y), (unsigned)((a.cout + kConvBM - 1) / kConvBM),
                    (unsigned)(a.T * p.ksplit));
    p.gn_rec = nullptr;
    p.gn_cpg = 0;
    p.gn_nrec = 0;
    if (a.gn_rec && p.ksplit == 1) {
        if (conv3x3_gn_records(a) == 0) {
            set_error("conv3x3_wino: GroupNorm records in the epilogue need out_channels %% 128 == 0");
            return VAE_ERR_UNSUPPORTED;
        }
        p.gn_rec = a.gn_rec;
        p.gn_cpg = a.cout / 32;
        p.gn_nrec = (int)(grid.x * grid.z);
    }
    const bool up = a.upsample != 0, gn = a.gn_coef != nullptr, res = a.res != nullptr, split = p.ksplit > 1;
    if (TC == 32) wino_launch_tc<32>(p, up, gn, res, split, grid, s);
    else if (TC == 16) wino_launch_tc<16>(p, up, gn, res, split, grid, s);
    else wino_launch_tc<8>(p, up, gn, res, split, grid, s);
    return check_launch("conv3x3_wino");
}

}  // namespace vae
