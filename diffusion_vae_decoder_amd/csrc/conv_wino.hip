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
// with 16 multiplies per 2 x 2 outputs and input channel instead of 36.
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
// outputs and input channel instead of 36.
//
// Workgroup: 4 waves, one block of 32 output channels and 64 tiles (2 x 2
// output blocks; 256 outputs); wave w owns tiles [16w, 16w + 16).  A step is
// four input channels: every lane transforms one (channel, tile) patch in
// registers (lane l: tile l % 16, channel l / 16), which is exactly the B
// operand of v_mfma_f32_16x16x4_f32 for every point xi; each point takes two
// MFMAs (output channels 0-15 and 16-31 of the block, A operand from U).
// All accumulators of a lane hold the same (output channels, tile) entries,
// so the output transform is lane-local.  The 128 accumulator registers let
// two waves share a SIMD (two workgroups per CU), so one wave's transform,
// LDS and memory work overlaps the other's MFMAs.  The input tile with its
// halo and the block's U are staged through LDS, kWStage steps at a time and
// double-buffered: step j of a stage also loads step j of the next stage
// and stores step j - 1 of it, with one barrier per stage.

#include <cstdio>

#include "wino_common.h"

namespace vae {

namespace {

using namespace wino;

constexpr int kWThreads = 256;
constexpr int kWOut = 32;        // output channels per workgroup (two MFMA row blocks of 16)
constexpr int kWTiles = 64;      // tiles per workgroup (16 per wave)
constexpr int kWStage = 2;       // steps per LDS stage

template <bool UP>
struct WinoShape {
    static constexpr int NX = UP ? 9 : 16;                 // transform points
    static constexpr int NQ = (2 * NX + 3) / 4;            // float4s of U per lane and step (2 row blocks per point)
    static constexpr int NP = UP ? 3 : 4;                  // input rows (and columns) of a tile's patch
};

// Channel-plane stride of a staged step.  Plain input: 8-byte patch reads,
// 32 lanes (two channels x 16 tiles) per LDS cycle; upsampled: 4-byte reads,
// all four channels in one cycle.  The stride puts those channels in
// distinct bank ranges.
constexpr int wino_plane(int n, bool up) {
    for (int p = n; p < n + 64; ++p)
        if (p % 64 == (up ? 16 : 32)) return p;
    return -1;
}

template <int TCW, bool UP>
struct WGeom {
    static constexpr int TRW = kWTiles / TCW;          // tile rows of the block
    static constexpr int OR = 2 * TRW, OC = 2 * TCW;   // output rows, columns of the block
    static constexpr int HR = UP ? TRW + 2 : OR + 2;   // staged rows (source rows when upsampled)
    static constexpr int HC = UP ? TCW + 2 : OC + 2;   // staged columns
    static constexpr int HCP = HC;   // row stride: contiguous rows (HC is even for plain input: 8-byte reads)
    static constexpr int NCH = (HR * HC + 63) / 64;       // 64-element chunks of a staged plane
    static constexpr int PLANE = wino_plane(NCH * 64, UP);
    static constexpr int EPT = (HR * HC + kWThreads - 1) / kWThreads;   // staged elements per thread and plane
    static constexpr int XSTEP = kWCh * PLANE;                           // floats of input per step
    static constexpr int USTEP = WinoShape<UP>::NQ * 64;                 // float4s of U per step
    static constexpr int UPT = (USTEP + kWThreads - 1) / kWThreads;      // U float4s per thread and step
    static_assert(PLANE > 0, "no LDS layout");
};






// One step's staging in registers on its way to LDS: this thread's elements
// of the step's four channel planes, its float4s of U and, for GroupNorm on
// load, the channels' coefficients.
template <int TCW, bool UP, bool GN>
struct WStep {
    float x[kWCh][WGeom<TCW, UP>::EPT];
    floatx4 u[WGeom<TCW, UP>::UPT];
    floatx4 cf[kWCh];
    bool cok[kWCh];
};

// Global -> registers for the step at the cursor, with no branch (a branch
// around a load makes the compiler wait for every load in flight).  Channels
// past cin, the zero padding and dead steps (live false) read 0 from the
// buffer range check; `ustep` is a live step's U (the caller clamps it), and
// indices past the step's float4s read its last one (not stored).
template <int TCW, bool UP, bool GN>
__device__ __attribute__((always_inline)) inline void wino_step_load(const WParams &p, int frame, bool live,
                                                                    WCursor &cur, const floatx4 *ustep,
                                                                    const int (&soff)[WGeom<TCW, UP>::EPT],
                                                                    WStep<TCW, UP, GN> &st) {
    using G = WGeom<TCW, UP>;
#pragma unroll
    for (int c = 0; c < kWCh; ++c) {
        const int ch = kWCh * cur.quad + c;
        const bool ok = live && ch < p.cin;
        const __amdgpu_buffer_rsrc_t xr = wino_rsrc(cur.x + c * p.in_cstride, ok ? (unsigned)(p.in_cstride * 4) : 0u);
#pragma unroll
        for (int i = 0; i < G::EPT; ++i)
            st.x[c][i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(xr, soff[i], 0, 0));
        if (GN) {
            st.cok[c] = ok;
            st.cf[c] = *reinterpret_cast<const floatx4 *>(p.gn_coef + 4 * (ch < p.cin ? ch : p.cin - 1));
        }
    }
    wino_next(p, frame, cur);
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < G::UPT; ++i) {
        const int e = t + i * kWThreads;
        st.u[i] = ustep[e < G::USTEP ? e : G::USTEP - 1];
    }
}

// Registers -> LDS slot j of a stage buffer (GroupNorm + SiLU applied here;
// padding and channels past cin stay 0).  A dead step is stored as zeros
// (input and U), so every stage runs all its kWStage steps and those add
// exactly 0.  Elements a thread does not own go to its word of `dummy`.
template <int TCW, bool UP, bool GN>
__device__ __attribute__((always_inline)) inline void wino_step_store(float *lx, floatx4 *lu, float *dummy,
                                                                     floatx4 *udummy, int j, bool live,
                                                                     const int (&soff)[WGeom<TCW, UP>::EPT],
                                                                     const int (&loff)[WGeom<TCW, UP>::EPT],
                                                                     const WStep<TCW, UP, GN> &st) {
    using G = WGeom<TCW, UP>;
    const int t = threadIdx.x;
#pragma unroll
    for (int c = 0; c < kWCh; ++c)
#pragma unroll
        for (int i = 0; i < G::EPT; ++i) {
            float v = st.x[c][i];
            if (GN) {
                const floatx4 cf = st.cf[c];
                float tt = (v - cf[0]) * cf[1] + cf[2];
                tt = tt * __builtin_amdgcn_rcpf(1.f + __expf(-tt));
                v = (st.cok[c] && soff[i] != kWOOB) ? tt : 0.f;
            }
            float *dst = loff[i] >= 0 ? lx + j * G::XSTEP + c * G::PLANE + loff[i] : dummy + t;
            *dst = live ? v : 0.f;
        }
#pragma unroll
    for (int i = 0; i < G::UPT; ++i) {
        const int e = t + i * kWThreads;
        floatx4 *ud = e < G::USTEP ? lu + j * G::USTEP + e : udummy + (t & 63);
        *ud = live ? st.u[i] : floatx4{0.f, 0.f, 0.f, 0.f};
    }
}


// Issue the direct loads of one stage (kWStage steps from sb) into (lx, lu):
// wave w takes chunks w, w + 4, ... of every channel plane and float4 rows
// w, w + 4, ... of every step's U.  Channels past cin, the zero padding and
// dead steps (from s1 on: zero-range buffers) land as zeros, so every stage
// runs all its steps and those add exactly 0.
template <int TCW, bool UP>
__device__ __attribute__((always_inline)) inline void wino_stage_dma(const WParams &p, int frame, int sb, int s1,
                                                                    WCursor &cur, const floatx4 *ublock, float *lx,
                                                                    floatx4 *lu,
                                                                    const int (&soffd)[(WGeom<TCW, UP>::NCH + 3) / 4]) {
    using G = WGeom<TCW, UP>;
    // the wave index is uniform: held in a scalar register, the chunk tests
    // are scalar branches and the LDS destinations scalar sums
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < kWStage; ++j) {
        const bool live = sb + j < s1;
#pragma unroll
        for (int c = 0; c < kWCh; ++c) {
            const int ch = kWCh * cur.quad + c;
            const bool ok = live && ch < p.cin;
            const __amdgpu_buffer_rsrc_t xr = wino_rsrc(cur.x + c * p.in_cstride, ok ? (unsigned)(p.in_cstride * 4) : 0u);
#pragma unroll
            for (int i = 0; i < (G::NCH + 3) / 4; ++i) {
                const int ck = w + 4 * i;
                if (ck < G::NCH) wino_dma4(xr, lx + j * G::XSTEP + c * G::PLANE + 64 * ck, soffd[i]);
            }
        }
        wino_next(p, frame, cur);
        const int s = live ? sb + j : s1 - 1;
        const __amdgpu_buffer_rsrc_t ur = wino_rsrc(reinterpret_cast<const float *>(ublock + (size_t)s * G::USTEP),
                                                    live ? (unsigned)(G::USTEP * 16) : 0u);
#pragma unroll
        for (int i = 0; i < (WinoShape<UP>::NQ + 3) / 4; ++i) {
            const int q = w + 4 * i;
            if (q < WinoShape<UP>::NQ) wino_dma16(ur, lu + j * G::USTEP + q * 64, (q * 64 + lane) * 16);
        }
    }
}

// One step from LDS: the lane's patch of its channel, its input transform and
// the step's 2 NX MFMAs (A operand: U of point k and row block b is float4
// (2k + b) / 4, component (2k + b) % 4).
template <int TCW, bool UP>
__device__ __attribute__((always_inline)) inline void wino_step(const float *lx, const floatx4 *lu, int j, int pbase,
                                                               int lane, floatx4 (&acc)[WinoShape<UP>::NX][2]) {
    using G = WGeom<TCW, UP>;
    using S = WinoShape<UP>;
    const float *pl = lx + j * G::XSTEP + pbase;
    float v[S::NX];
    if (!UP) {
        float d[16];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const floatx2 a = *reinterpret_cast<const floatx2 *>(pl + r * G::HCP);
            const floatx2 b = *reinterpret_cast<const floatx2 *>(pl + r * G::HCP + 2);
            d[4 * r + 0] = a[0];
            d[4 * r + 1] = a[1];
            d[4 * r + 2] = b[0];
            d[4 * r + 3] = b[1];
        }
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
        // source patch (3 x 3): transform points (0, 1, 3) of each axis, the
        // factor 2 of point 1 being in U
        float d[9];
#pragma unroll
        for (int r = 0; r < 3; ++r)
#pragma unroll
            for (int q = 0; q < 3; ++q) d[3 * r + q] = pl[r * G::HCP + q];
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
    const floatx4 *ul = lu + j * G::USTEP + lane;
#pragma unroll
    for (int q = 0; q < S::NQ; ++q) {
        const floatx4 u = ul[q * 64];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int kb = 4 * q + e;
            if (kb < 2 * S::NX)
                acc[kb >> 1][kb & 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(u[e], v[kb >> 1], acc[kb >> 1][kb & 1], 0, 0, 0);
        }
    }
}

// Output transform of register i of row block b of every accumulator: the
// lane's 2 x 2 outputs.
template <bool UP>
__device__ __attribute__((always_inline)) inline void wino_out(const floatx4 (&acc)[WinoShape<UP>::NX][2], int b, int i,
                                                              float (&y)[2][2]) {
    if (!UP) {
        float s[2][4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            s[0][c] = (acc[c][b][i] + acc[4 + c][b][i]) + acc[8 + c][b][i];
            s[1][c] = (acc[4 + c][b][i] - acc[8 + c][b][i]) - acc[12 + c][b][i];
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
            s[0][c] = acc[c][b][i] + acc[3 + c][b][i];
            s[1][c] = acc[3 + c][b][i] - acc[6 + c][b][i];
        }
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            y[a][0] = s[a][0] + s[a][1];
            y[a][1] = s[a][1] - s[a][2];
        }
    }
}


template <int TCW, bool UP, bool GN, bool RES, bool SPLIT>
__global__ __launch_bounds__(kWThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void conv3x3_wino(WParams p) {
    using G = WGeom<TCW, UP>;
    using S = WinoShape<UP>;
    // Two stage buffers, declared apart: the compiler then knows that LDS
    // reads of one buffer do not wait for direct loads into the other.
    __shared__ __attribute__((aligned(16))) float lx0[kWStage * G::XSTEP];
    __shared__ __attribute__((aligned(16))) float lx1[kWStage * G::XSTEP];
    __shared__ floatx4 lu0[kWStage * G::USTEP];
    __shared__ floatx4 lu1[kWStage * G::USTEP];
    // GroupNorm on load: stores of staged elements a thread does not own
    __shared__ float lds_dummy[GN ? kWThreads : 1];
    __shared__ floatx4 lds_udummy[GN ? 64 : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int g4 = lane >> 4;   // the lane's channel of a step, and its 4-row group of an MFMA output

    // blockIdx.x enumerates (tile block, 32-channel output block) with the
    // channel block fastest.  Workgroups are dealt to the 8 XCDs round-robin by
    // linear id; when their count is a multiple of 8 they are renumbered so each
    // XCD walks one contiguous band: all channel blocks of a tile then run
    // together on one XCD and read the tile's input from HBM once.
    int lin = blockIdx.x;
    if ((gridDim.x & 7) == 0) lin = (lin & 7) * (gridDim.x >> 3) + (lin >> 3);
    const int tile = lin / p.ncb;
    const int cb = lin - tile * p.ncb;   // block of 32 output channels
    const int ty = tile / p.tiles_x;
    const int tx = tile - ty * p.tiles_x;
    const int y0 = ty * G::OR, x0 = tx * G::OC;
    const int frame = SPLIT ? blockIdx.z / p.ksplit : blockIdx.z;
    const int split = SPLIT ? blockIdx.z - frame * p.ksplit : 0;

    // The lane's tile and the offset of its patch in a staged step.
    const int n = wave * 16 + (lane & 15);
    const int tr = n / TCW, tc = n - (n / TCW) * TCW;
    const int Y0 = y0 + 2 * tr, X0 = x0 + 2 * tc;   // top-left output of the tile
    const int pbase = g4 * G::PLANE + (UP ? tr * G::HCP + tc : 2 * tr * G::HCP + 2 * tc);

    // GroupNorm on load: this thread's staged elements of a plane, their byte
    // offset in the channel (kWOOB for zero padding) and LDS offset in the
    // plane (-1: none).
    int soff[G::EPT], loff[G::EPT];
    if (GN) {
        const int ry = UP ? (y0 >> 1) - 1 : y0 - 1;
        const int rx = UP ? (x0 >> 1) - 1 : x0 - 1;
        const int Hs = UP ? p.Hin : p.H, Ws = UP ? p.Win : p.W;
#pragma unroll
        for (int i = 0; i < G::EPT; ++i) {
            const int e = tid + i * kWThreads;
            soff[i] = kWOOB;
            loff[i] = -1;
            if (e < G::HR * G::HC) {
                const int r = e / G::HC, q = e - (e / G::HC) * G::HC;
                const int yy = ry + r, xx = rx + q;
                loff[i] = r * G::HCP + q;
                if (yy >= 0 && yy < Hs && xx >= 0 && xx < Ws) soff[i] = (yy * Ws + xx) * 4;
            }
        }
    }

    const int nsteps = p.kt * p.nquads;
    const int s0 = SPLIT ? (int)((long long)split * nsteps / p.ksplit) : 0;
    const int s1 = SPLIT ? (int)((long long)(split + 1) * nsteps / p.ksplit) : nsteps;
    const floatx4 *ublock = reinterpret_cast<const floatx4 *>(p.u) + (size_t)cb * nsteps * G::USTEP;
    auto ustep = [&](int s) { return ublock + (size_t)(s < s1 ? s : s1 - 1) * G::USTEP; };

    WCursor cur = wino_cursor(p, frame, s0);

    floatx4 acc[S::NX][2];
#pragma unroll
    for (int k = 0; k < S::NX; ++k)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[k][b] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int nst = (s1 - s0 + kWStage - 1) / kWStage;
    if constexpr (!GN) {
        // Direct loads: per-lane offsets of this wave's chunks of a staged plane.
        int soffd[(G::NCH + 3) / 4];
        {
            const int ry = UP ? (y0 >> 1) - 1 : y0 - 1;
            const int rx = UP ? (x0 >> 1) - 1 : x0 - 1;
            const int Hs = UP ? p.Hin : p.H, Ws = UP ? p.Win : p.W;
#pragma unroll
            for (int i = 0; i < (G::NCH + 3) / 4; ++i) {
                const int e = 64 * (wave + 4 * i) + lane;
                const int r = e / G::HC, q = e - (e / G::HC) * G::HC;
                const int yy = ry + r, xx = rx + q;
                soffd[i] = (e < G::HR * G::HC && yy >= 0 && yy < Hs && xx >= 0 && xx < Ws) ? (yy * Ws + xx) * 4 : kWOOB;
            }
        }
        // Stage k + 1 is loaded while stage k is computed; the loop is unrolled
        // by two so each buffer is named statically.
        wino_stage_dma<TCW, UP>(p, frame, s0, s1, cur, ublock, lx0, lu0, soffd);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        int k = 0;
        for (; k + 2 <= nst; k += 2) {
            const int sb = s0 + k * kWStage;
            wino_stage_dma<TCW, UP>(p, frame, sb + kWStage, s1, cur, ublock, lx1, lu1, soffd);
#pragma unroll
            for (int j = 0; j < kWStage; ++j) wino_step<TCW, UP>(lx0, lu0, j, pbase, lane, acc);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (k + 2 < nst) wino_stage_dma<TCW, UP>(p, frame, sb + 2 * kWStage, s1, cur, ublock, lx0, lu0, soffd);
#pragma unroll
            for (int j = 0; j < kWStage; ++j) wino_step<TCW, UP>(lx1, lu1, j, pbase, lane, acc);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
        if (k < nst) {   // an odd stage count: the last stage is in buffer 0
#pragma unroll
            for (int j = 0; j < kWStage; ++j) wino_step<TCW, UP>(lx0, lu0, j, pbase, lane, acc);
        }
    } else {
        // GroupNorm on load: staged through registers, where each element is
        // normalised.
        WStep<TCW, UP, GN> rs[kWStage];
        // stage 0: all its loads in flight, then the stores
#pragma unroll
        for (int j = 0; j < kWStage; ++j)
            wino_step_load<TCW, UP, GN>(p, frame, s0 + j < s1, cur, ustep(s0 + j), soff, rs[j]);
#pragma unroll
        for (int j = 0; j < kWStage; ++j)
            wino_step_store<TCW, UP, GN>(lx0, lu0, lds_dummy, lds_udummy, j, s0 + j < s1, soff, loff, rs[j]);
        __syncthreads();
        // Stages but the last: step j also loads step j of the next stage and
        // stores step j - 1 of it.
        int k = 0;
        for (; k + 1 < nst; ++k) {
            const int buf = k & 1;
            const int nb = s0 + (k + 1) * kWStage;
#pragma unroll
            for (int j = 0; j < kWStage; ++j) {
                wino_step_load<TCW, UP, GN>(p, frame, nb + j < s1, cur, ustep(nb + j), soff, rs[j]);
                wino_step<TCW, UP>(buf ? lx1 : lx0, buf ? lu1 : lu0, j, pbase, lane, acc);
                if (j >= 1)
                    wino_step_store<TCW, UP, GN>(buf ? lx0 : lx1, buf ? lu0 : lu1, lds_dummy, lds_udummy, j - 1,
                                                 nb + j - 1 < s1, soff, loff, rs[j - 1]);
            }
            wino_step_store<TCW, UP, GN>(buf ? lx0 : lx1, buf ? lu0 : lu1, lds_dummy, lds_udummy, kWStage - 1,
                                         nb + kWStage - 1 < s1, soff, loff, rs[kWStage - 1]);
            __syncthreads();
        }
#pragma unroll
        for (int j = 0; j < kWStage; ++j)
            wino_step<TCW, UP>((k & 1) ? lx1 : lx0, (k & 1) ? lu1 : lu0, j, pbase, lane, acc);
    }

    // Epilogue: register i of row block b of a 16x16 MFMA tile is output
    // channel 16 b + 4 g4 + i of the block, for the lane's tile.
    const long long fo = (long long)frame * p.out_fstride;
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

    // Per row block b (the lane's quad of 4 output channels): its 16 outputs,
    // and, for GroupNorm records, their count, mean and sum of squared
    // deviations (gs).
    float gs[2][3];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int obase = cb * kWOut + 16 * b + 4 * g4;
        float rv[4][4];
        if (RES && !SPLIT) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int o = min(obase + i, p.cout - 1);
#pragma unroll
                for (int e = 0; e < 4; ++e) rv[i][e] = p.res[(long long)o * p.out_cstride + sp[e >> 1][e & 1]];
            }
        }
        float val[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int o = obase + i;
            float yv[2][2];
            wino_out<UP>(acc, b, i, yv);
            const long long base = (long long)min(o, p.cout - 1) * p.out_cstride;
            const float bo = SPLIT ? 0.f : p.bias[min(o, p.cout - 1)];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float v = yv[e >> 1][e & 1] + bo;
                if (RES && !SPLIT) v += rv[i][e];
                val[i][e] = v;
                if (o < p.cout && pv[e >> 1][e & 1]) {
                    if (SPLIT) p.part[split * p.part_stride + base + sp[e >> 1][e & 1]] = v;
                    else p.y[base + sp[e >> 1][e & 1]] = v;
                }
            }
        }
        if (!SPLIT && p.gn_rec) {
            float t = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (pv[e >> 1][e & 1]) t += val[i][e];
            const float mean = nval > 0.f ? t / nval : 0.f;
            float m2 = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (pv[e >> 1][e & 1]) {
                        const float dv = val[i][e] - mean;
                        m2 += dv * dv;
                    }
            gs[b][0] = nval;
            gs[b][1] = mean;
            gs[b][2] = m2;
        }
    }

    if (!SPLIT && p.gn_rec) {
        // GroupNorm records of the block: per group (count, mean, sum of
        // squared deviations from that mean), merged pairwise (Chan, Golub and
        // LeVeque) over the 16 tiles of a lane group, then over the four waves
        // and the quads of a group, in a fixed order.  Quad 4 b + g4 holds
        // output channels 16 b + 4 g4 + (0..3) of the block.  The host enables
        // this only when a group is a whole number of quads within 32 channels
        // (cout % 128 == 0, cout <= 1024).
        __syncthreads();   // the staging buffers are reused below
        float *qst = lx0;   // [wave][quad of 8][3]
#pragma unroll
        for (int o = 1; o < 16; o <<= 1)
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const float nb = __shfl_xor(gs[b][0], o, 64);
                const float mb = __shfl_xor(gs[b][1], o, 64);
                const float qb = __shfl_xor(gs[b][2], o, 64);
                wino_chan_merge(gs[b], nb, mb, qb);
            }
        if ((lane & 15) == 0)
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                float *d = qst + (wave * 8 + 4 * b + g4) * 3;
                d[0] = gs[b][0];
                d[1] = gs[b][1];
                d[2] = gs[b][2];
            }
        __syncthreads();
        const int qpg = p.gn_cpg >> 2;
        const int gpb = kWOut / p.gn_cpg;
        if (tid < gpb) {
            float g[3] = {0.f, 0.f, 0.f};
            for (int w = 0; w < 4; ++w)
                for (int q = 0; q < qpg; ++q) {
                    const float *d = qst + (w * 8 + tid * qpg + q) * 3;
                    wino_chan_merge(g, d[0], d[1], d[2]);
                }
            const long long rec = (long long)(cb * gpb + tid) * p.gn_nrec + (long long)frame * (gridDim.x / p.ncb) + tile;
            p.gn_rec[rec] = floatx4{g[0], g[1], g[2], 0.f};
        }
    }
}

// Packed U: [32-channel output block][step = (dt, channel quad)][q][lane][4]
// with lane = (channel of the quad) * 16 + (output channel within its row
// block) and float4 component e of q holding transform point (4q + e) / 2 of
// row block (4q + e) % 2; zero where the output or input channel is out of
// range and in the padding.  One thread per (block, step, lane).
template <bool UP>
__global__ __launch_bounds__(256) void pack_wino_kernel(const float *__restrict__ w, float *__restrict__ dst, int cout,
                                                        int cin, int kt, int nquads, long long total) {
    using S = WinoShape<UP>;
    const long long id = (long long)blockIdx.x * 256 + threadIdx.x;
    if (id >= total) return;
    const int lane = (int)(id & 63);
    const long long bs = id >> 6;   // block * nsteps + step
    const int nsteps = kt * nquads;
    const int cb = (int)(bs / nsteps);
    const int s = (int)(bs - (long long)cb * nsteps);
    const int dt = s / nquads, quad = s - dt * nquads;
    const int c = kWCh * quad + (lane >> 4);
    const double G[4][3] = {{1.0, 0.0, 0.0}, {0.5, 0.5, 0.5}, {0.5, -0.5, 0.5}, {0.0, 0.0, 1.0}};
    float u[2][16];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int o = cb * kWOut + 16 * b + (lane & 15);
        double g[3][3];
#pragma unroll
        for (int i = 0; i < 9; ++i)
            g[i / 3][i % 3] = (o < cout && c < cin) ? (double)w[(((long long)o * cin + c) * kt + dt) * 9 + i] : 0.0;
        // U = G g G^T
        double t[4][3];
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
            for (int j = 0; j < 3; ++j) t[x][j] = G[x][0] * g[0][j] + G[x][1] * g[1][j] + G[x][2] * g[2][j];
        if (!UP) {
#pragma unroll
            for (int x = 0; x < 4; ++x)
#pragma unroll
                for (int y = 0; y < 4; ++y)
                    u[b][4 * x + y] = (float)(t[x][0] * G[y][0] + t[x][1] * G[y][1] + t[x][2] * G[y][2]);
        } else {
            const int pts[3] = {0, 1, 3};
#pragma unroll
            for (int ix = 0; ix < 3; ++ix)
#pragma unroll
                for (int iy = 0; iy < 3; ++iy) {
                    const int x = pts[ix], y = pts[iy];
                    const double f = (ix == 1 ? 2.0 : 1.0) * (iy == 1 ? 2.0 : 1.0);
                    u[b][3 * ix + iy] = (float)(f * (t[x][0] * G[y][0] + t[x][1] * G[y][1] + t[x][2] * G[y][2]));
                }
        }
    }
    float *out = dst + bs * (S::NQ * 64 * 4) + lane * 4;
#pragma unroll
    for (int q = 0; q < S::NQ; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int kb = 4 * q + e;
            out[q * 256 + e] = kb < 2 * S::NX ? u[kb & 1][kb >> 1] : 0.f;
        }
}

int wino_tcw(int W) { return W > 16 ? 16 : (W > 8 ? 8 : 4); }

struct WinoGrid {
    int tcw, tiles_x, tiles_y, ncb;
};

WinoGrid wino_grid(int cout, int H, int W) {
    WinoGrid g;
    g.tcw = wino_tcw(W);
    const int oc = 2 * g.tcw, orr = 2 * (kWTiles / g.tcw);
    g.tiles_x = (W + oc - 1) / oc;
    g.tiles_y = (H + orr - 1) / orr;
    g.ncb = (cout + kWOut - 1) / kWOut;
    return g;
}

template <int TCW, bool UP, bool GN>
void wino_launch_t(const WParams &p, bool res, bool split, dim3 grid, hipStream_t s) {
    if (split) hipLaunchKernelGGL((conv3x3_wino<TCW, UP, GN, false, true>), grid, dim3(kWThreads), 0, s, p);
    else if (res) hipLaunchKernelGGL((conv3x3_wino<TCW, UP, GN, true, false>), grid, dim3(kWThreads), 0, s, p);
    else hipLaunchKernelGGL((conv3x3_wino<TCW, UP, GN, false, false>), grid, dim3(kWThreads), 0, s, p);
}

template <int TCW>
void wino_launch_tc(const WParams &p, bool up, bool gn, bool res, bool split, dim3 grid, hipStream_t s) {
    if (up) wino_launch_t<TCW, true, false>(p, res, split, grid, s);
    else if (gn) wino_launch_t<TCW, false, true>(p, res, split, grid, s);
    else wino_launch_t<TCW, false, false>(p, res, split, grid, s);
}

constexpr int kWSlots = 512;   // resident workgroups: two per CU

}  // namespace

size_t conv3x3_wino_packed_floats(int cout, int cin, int kt, int up) {
    const size_t ncb = (size_t)(cout + kWOut - 1) / kWOut;
    const size_t nsteps = (size_t)kt * ((cin + kWCh - 1) / kWCh);
    return ncb * nsteps * 64 * 4 * (up ? WinoShape<true>::NQ : WinoShape<false>::NQ);
}

int32_t pack_conv3x3_wino(const float *w, int cout, int cin, int kt, int up, float *dst, hipStream_t s) {
    const int nquads = (cin + kWCh - 1) / kWCh;
    const long long ncb = (cout + kWOut - 1) / kWOut;
    const long long total = ncb * kt * nquads * 64;
    const dim3 grid((unsigned)((total + 255) / 256));
    if (up) hipLaunchKernelGGL(pack_wino_kernel<true>, grid, dim3(256), 0, s, w, dst, cout, cin, kt, nquads, total);
    else hipLaunchKernelGGL(pack_wino_kernel<false>, grid, dim3(256), 0, s, w, dst, cout, cin, kt, nquads, total);
    return check_launch("pack_conv3x3_wino");
}

int conv3x3_wino_ksplit(const ConvLaunch &a) {
    const WinoGrid g = wino_grid(a.cout, a.H, a.W);
    const long long base = (long long)g.tiles_x * g.tiles_y * g.ncb * a.T;
    if (base >= 2 * kWSlots) return 1;
    const int nsteps = a.kt * ((a.cin + kWCh - 1) / kWCh);
    long long s = (2 * kWSlots + base - 1) / base;     // about two rounds of workgroups
    if (s > nsteps / (2 * kWStage)) s = nsteps / (2 * kWStage);   // each split keeps >= 2 stages
    if (s > 16) s = 16;
    if (s * a.T > 65535) s = 65535 / a.T;
    return s < 1 ? 1 : (int)s;
}

int conv3x3_wino_gn_records(const ConvLaunch &a) {
    if (a.cout % 128 != 0 || a.cout > 32 * kWOut) return 0;
    const WinoGrid g = wino_grid(a.cout, a.H, a.W);
    return g.tiles_x * g.tiles_y * a.T;
}

int conv3x3_wino_tcw(const ConvLaunch &a) { return wino_tcw(a.W); }

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
    if (a.upsample && ((a.H | a.W) & 1)) {
        set_error("conv3x3_wino: an upsampled input has even sizes");
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
    p.nquads = (a.cin + kWCh - 1) / kWCh;
    p.in_fstride = (long long)p.Hin * p.Win;
    p.in_cstride = p.in_fstride * a.T;
    p.out_fstride = (long long)a.H * a.W;
    p.out_cstride = p.out_fstride * a.T;
    const WinoGrid g = wino_grid(a.cout, a.H, a.W);
    p.tiles_x = g.tiles_x;
    p.ncb = g.ncb;
    p.ksplit = conv3x3_wino_ksplit(a);
    p.part = a.part;
    p.part_stride = p.out_cstride * a.cout;
    if (p.ksplit > 1 && !a.part) {
        set_error("conv3x3_wino: split-K needs a partial-sum workspace");
        return VAE_ERR_WORKSPACE;
    }
    // byte offsets within one channel are 32-bit
    if (p.in_cstride * 4 >= (1LL << 31)) {
        set_error("conv3x3_wino: input channel of %lld elements is too large", p.in_cstride);
        return VAE_ERR_UNSUPPORTED;
    }
    const long long nwg = (long long)g.tiles_x * g.tiles_y * g.ncb;
    if (nwg >= (1LL << 31)) {
        set_error("conv3x3_wino: %lld workgroups exceed the grid limit", nwg);
        return VAE_ERR_UNSUPPORTED;
    }
    const dim3 grid((unsigned)nwg, 1u, (unsigned)(a.T * p.ksplit));
    p.gn_rec = nullptr;
    p.gn_cpg = 0;
    p.gn_nrec = 0;
    if (a.gn_rec && p.ksplit == 1) {
        if (conv3x3_wino_gn_records(a) == 0) {
            set_error("conv3x3_wino: GroupNorm records in the epilogue need out_channels %% 128 == 0 (<= 1024)");
            return VAE_ERR_UNSUPPORTED;
        }
        p.gn_rec = a.gn_rec;
        p.gn_cpg = a.cout / 32;
        p.gn_nrec = g.tiles_x * g.tiles_y * (int)grid.z;
    }
    const bool up = a.upsample != 0, gn = a.gn_coef != nullptr, res = a.res != nullptr, split = p.ksplit > 1;
    switch (g.tcw) {
    case 16: wino_launch_tc<16>(p, up, gn, res, split, grid, s); break;
    case 8: wino_launch_tc<8>(p, up, gn, res, split, grid, s); break;
    default: wino_launch_tc<4>(p, up, gn, res, split, grid, s); break;
    }
    return check_launch("conv3x3_wino");
}

}  // namespace vae
