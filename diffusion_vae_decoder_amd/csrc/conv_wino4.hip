// Winograd F(4x4, 3x3) form of the decoder's 3x3 convolutions on FP32 MFMA.
//
// The conv (cortiq-engine 0.7.7 `vae`, VaeConvRef: stride 1, zero padding
// 1, cross-correlation) computes each 4 x 4 block of outputs from the 6 x 6
// input patch d around it.  With the minimal filtering algorithm of Lavin and
// Gray (Fast Algorithms for Convolutional Neural Networks, 2016), built on the
// interpolation points 0, 1, -1, 2, -2 and infinity,
//     Y = A^T [ sum_c (G g_c G^T) . (B^T d_c B) ] A        (. elementwise)
//     B^T = [4 0 -5 0 1 0; 0 -4 -4 1 1 0; 0 4 -4 -1 1 0;
//            0 -2 -1 2 1 0; 0 2 -1 -2 1 0; 0 4 0 -5 0 1]
//     G   = [1/4 0 0; -1/6 -1/6 -1/6; -1/6 1/6 -1/6;
//            1/24 1/12 1/6; 1/24 -1/12 1/6; 0 0 1]
//     A^T = [1 1 1 1 1 0; 0 1 -1 2 -2 0; 0 1 1 4 4 0; 0 1 -1 8 -8 1]
// the sum over input channels becomes 36 independent GEMMs, one per point of
// the 6 x 6 transform: 36 multiplies per 4 x 4 outputs and input channel
// instead of 144 (F(2x2, 3x3): 64).  U = G g G^T is formed once, in double
// precision, when the weights are packed.  The result equals the direct conv
// up to rounding: about 1e-5 of the output's magnitude in float32 at the
// decoder's shapes (the larger transform coefficients cost about one decimal
// digit against F(2x2, 3x3)).
//
// Nearest-x2 upsampled input (VaeUpRef): the 6 x 6 patch of a 4 x 4 output
// block at multiples of 4 reads upsampled rows 4i-1 .. 4i+4, i.e. source rows
// 2i-1, 2i, 2i, 2i+1, 2i+1, 2i+2.  On that repetition B^T collapses to four
// rows over the 4 source rows s: (4 -5 1 0), (0 -8 2 0), (0 1 -1 0) and
// (0 4 -5 1); point 2 vanishes and point 3 is -3 times point 4.  The 4 x 4
// source patch transforms to 16 values, and the 25 products of points
// {0, 1, 3, 4, 5}^2 use them with the factors -3 folded into U (exact in
// double precision before rounding): 25 multiplies per 4 x 4 outputs and
// channel instead of 144 (F(2x2, 3x3): 36).
//
// On MI355X a SIMD does not overlap FP32 vector instructions with FP32 MFMA
// execution, so the input transform's VALU work adds to the MFMA time; the
// layout below spends as little of it per MFMA as the registers allow.
// Workgroup: 4 waves, 32 output channels (two MFMA row blocks) and 32 tiles
// (4 x 4 output blocks) in two groups of 16.  The two waves of a tile group
// split the transform's points: wave half h takes columns 3h .. 3h + 2 of
// B^T d B (18 points; on an upsampled input 13 and 12 of the 25 products)
// for both row blocks, so each transformed value feeds two MFMAs and the
// first transform pass computes only the outputs the half uses.  A step is four input channels: every lane
// transforms one (channel, tile) patch (lane l: tile l % 16, channel l / 16),
// which is the B operand of v_mfma_f32_16x16x4_f32; the A operand is U of the
// point.  Accumulators: 2 row blocks x 18 points x 4 = 144 registers, so two
// waves share a SIMD (two workgroups per CU).  The input tile with its halo
// and the workgroup's U are staged by direct global -> LDS loads,
// double-buffered, one barrier per step.  In the epilogue each wave applies
// A^T to its half and the two halves exchange partial outputs through LDS.

#include <cstdio>

#include "wino_common.h"

namespace vae {

namespace {

using namespace wino;

constexpr int kW4Blk = 16;               // output channels of an MFMA row block
constexpr int kW4RB = 2;                 // row blocks of a wave and of a workgroup
constexpr int kW4TG = 2;                 // tile groups (of 16 tiles) of a workgroup
constexpr int kW4Waves = 2 * kW4TG;      // a wave pair (point halves) per tile group
constexpr int kW4Threads = 64 * kW4Waves;

// Products of a point half, and float4 rows of U per row block and step (a
// plain input: 18 per half in 5 float4s each; an upsampled one: 13 and 12 in
// 4 and 3 float4s).
template <bool UP>
struct W4Shape {
    static constexpr int NX = UP ? 13 : 18;      // accumulators per row block (the larger half)
    static constexpr int Q1 = UP ? 4 : 5;        // first float4 row of half 1
    static constexpr int UQ = UP ? 7 : 10;       // float4 rows per row block
};
constexpr int kW4Slots = 512;            // resident workgroups: two per CU

// Staged columns: column x of a row sits at position w4_pos(x).  Layout 1
// moves columns 32..63 up by two and puts columns 64 and 65 (the right halo
// of 16 tiles of 4) in the two freed positions 32 and 33, so that tiles 8..15
// read other banks than tiles 0..7; w4_col inverts it (-1: a free position).
constexpr int w4_pos(int x, int lay) { return lay == 0 || x < 32 ? x : (x < 64 ? x + 2 : x - 32); }
constexpr int w4_col(int q, int lay, int hc) {
    const int x = lay == 0 || q < 32 ? q : (q < 34 ? q + 32 : q - 2);
    return x < hc ? x : -1;
}

// LDS bank check of the patch reads: pair h (columns 2h, 2h + 1 of a patch
// row) of every lane, `nl` lanes served together from `nb` four-byte banks
// (a patch starts every 4 staged columns, every 2 on an upsampled input).
constexpr bool w4_reads_ok(int tcw, bool up, int hcp, int lay, int plane, int nb, int nl) {
    const int stride = up ? 2 : 4;
    for (int h = 0; h < (up ? 2 : 3); ++h)
        for (int g0 = 0; g0 < 64; g0 += nl) {
            bool used[64] = {};
            for (int l = g0; l < g0 + nl; ++l) {
                const int ch = l / 16, t = l % 16;
                const int addr = ch * plane + stride * (t / tcw) * hcp + w4_pos(stride * (t % tcw) + 2 * h, lay);
                for (int k = 0; k < 2; ++k) {
                    const int b = (addr + k) % nb;
                    if (used[b]) return false;
                    used[b] = true;
                }
            }
        }
    return true;
}

struct W4Layout {
    int lay, hcp, plane;
};

// The first column layout, then smallest even row stride and channel-plane
// stride (whole 64-element chunks for the direct loads), whose patch reads
// are free of bank conflicts both with 32 banks serving 16 lanes and with 64
// banks serving 32; failing that (fewer than 16 tiles per row, whose tile
// rows a 4-row stride cannot separate in 32 banks), free of them with 64.
constexpr W4Layout w4_layout(int tcw, bool up, int hr, int hc) {
    for (int strict = 1; strict >= 0; --strict)
        for (int lay = 0; lay < (hc <= 66 ? 2 : 1); ++lay) {
            int width = 0;
            for (int x = 0; x < hc; ++x) width = w4_pos(x, lay) + 1 > width ? w4_pos(x, lay) + 1 : width;
            for (int hcp = width + (width & 1); hcp < width + 64; hcp += 2) {
                const int base = (hr * hcp + 63) / 64 * 64;
                for (int plane = base; plane < base + 64; plane += 2)
                    if ((!strict || w4_reads_ok(tcw, up, hcp, lay, plane, 32, 16)) &&
                        w4_reads_ok(tcw, up, hcp, lay, plane, 64, 32))
                        return W4Layout{lay, hcp, plane};
            }
        }
    return W4Layout{-1, -1, -1};
}

template <int TCW, bool UP>
struct W4Geom {
    static constexpr int TILES = 16 * kW4TG;            // tiles of the block
    static constexpr int TRW = TILES / TCW;             // tile rows of the block
    static constexpr int OR = 4 * TRW, OC = 4 * TCW;    // output rows, columns of the block
    static constexpr int HR = UP ? 2 * TRW + 2 : OR + 2;   // staged rows (source rows when upsampled)
    static constexpr int HC = UP ? 2 * TCW + 2 : OC + 2;   // staged columns
    static constexpr W4Layout L = w4_layout(TCW, UP, HR, HC);
    static constexpr int LAY = L.lay;                   // column layout (w4_pos)
    static constexpr int HCP = L.hcp;                   // row stride
    static constexpr int PLANE = L.plane;               // channel-plane stride
    static constexpr int NCH = (HR * HCP + 63) / 64;    // 64-element chunks of a staged plane
    static constexpr int XSTEP = kWCh * PLANE;          // floats of input per step
    static constexpr int UROWS = kW4RB * W4Shape<UP>::UQ;   // 64-lane float4 rows of U per step
    static constexpr int USTEP = UROWS * 64;            // float4s of U per step
    // wave w loads chunks w, w + 4, ... of every channel plane and U rows
    // w, w + 4, ...
    static constexpr int CPW = (NCH + kW4Waves - 1) / kW4Waves;
    static constexpr int UPW = (UROWS + kW4Waves - 1) / kW4Waves;
    static_assert(HCP > 0, "no LDS layout");
    static_assert(TILES % TCW == 0 && TCW <= 16, "tile rows");
};

// One axis of B^T on a 6-point line.
__device__ __attribute__((always_inline)) inline void w4_bt(float d0, float d1, float d2, float d3, float d4, float d5,
                                                           float (&v)[6]) {
    v[0] = fmaf(4.f, d0, fmaf(-5.f, d2, d4));
    const float s12 = d1 + d2, s34 = d3 + d4;
    v[1] = fmaf(-4.f, s12, s34);
    const float d12 = d1 - d2, d43 = d4 - d3;
    v[2] = fmaf(4.f, d12, d43);
    const float d31 = d3 - d1, d42 = d4 - d2;
    v[3] = fmaf(2.f, d31, d42);
    v[4] = fmaf(-2.f, d31, d42);
    v[5] = fmaf(4.f, d1, fmaf(-5.f, d3, d5));
}

// One axis of B^T on the repeated source line s0 s1 s1 s2 s2 s3: points 0, 1,
// 4 and 5 (point 3 is -3 times point 4, point 2 is zero).
__device__ __attribute__((always_inline)) inline void w4_btu(float s0, float s1, float s2, float s3, float (&w)[4]) {
    w[0] = fmaf(4.f, s0, fmaf(-5.f, s1, s2));
    w[1] = fmaf(-8.f, s1, 2.f * s2);
    w[2] = s1 - s2;
    w[3] = fmaf(4.f, s1, fmaf(-5.f, s2, s3));
}

// Points 3H .. 3H + 2 of B^T on a 6-point line.
template <int H>
__device__ __attribute__((always_inline)) inline void w4_bt_half(const float (&d)[6], float &a, float &b, float &c) {
    if (H == 0) {
        a = fmaf(4.f, d[0], fmaf(-5.f, d[2], d[4]));
        b = fmaf(-4.f, d[1] + d[2], d[3] + d[4]);
        c = fmaf(4.f, d[1] - d[2], d[4] - d[3]);
    } else {
        const float d31 = d[3] - d[1], d42 = d[4] - d[2];
        a = fmaf(2.f, d31, d42);
        b = fmaf(-2.f, d31, d42);
        c = fmaf(4.f, d[1], fmaf(-5.f, d[3], d[5]));
    }
}

// One axis of A^T: six points to four outputs.
__device__ __attribute__((always_inline)) inline void w4_at(float m0, float m1, float m2, float m3, float m4, float m5,
                                                           float (&o)[4]) {
    const float s12 = m1 + m2, d12 = m1 - m2, s34 = m3 + m4, d34 = m3 - m4;
    o[0] = (m0 + s12) + s34;
    o[1] = fmaf(2.f, d34, d12);
    o[2] = fmaf(4.f, s34, s12);
    o[3] = fmaf(8.f, d34, d12) + m5;
}

// Issue the direct loads of the step at the cursor into (lx, lu).  Channels
// past cin, the zero padding and dead steps (from s1 on) land as zeros, so
// those add exactly 0.  `soffd` holds the lane's byte offsets of the wave's
// input chunks; `ublk` is the workgroup's packed U (a step's rows are
// contiguous).
template <int TCW, bool UP>
__device__ __attribute__((always_inline)) inline void w4_stage(const WParams &p, int frame, int sb, int s1,
                                                              const float *ublk, WCursor &cur, float *lx, floatx4 *lu,
                                                              const int (&soffd)[W4Geom<TCW, UP>::CPW]) {
    using G = W4Geom<TCW, UP>;
    // the wave index is uniform: in a scalar register the load tests are
    // scalar branches and the LDS destinations scalar sums
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    __builtin_assume(w >= 0 && w < kW4Waves);
    const bool live = sb < s1;
#pragma unroll
    for (int c = 0; c < kWCh; ++c) {
        const bool ok = live && kWCh * cur.quad + c < p.cin;
        const __amdgpu_buffer_rsrc_t xr = wino_rsrc(cur.x + c * p.in_cstride, ok ? (unsigned)(p.in_cstride * 4) : 0u);
#pragma unroll
        for (int i = 0; i < G::CPW; ++i) {
            const int ck = w + kW4Waves * i;
            if (kW4Waves * (i + 1) <= G::NCH || ck < G::NCH) wino_dma4(xr, lx + c * G::PLANE + 64 * ck, soffd[i]);
        }
    }
    wino_next(p, frame, cur);
    const int s = live ? sb : s1 - 1;
    const __amdgpu_buffer_rsrc_t ur = wino_rsrc(ublk + (size_t)s * (G::UROWS * 256), live ? G::UROWS * 1024u : 0u);
#pragma unroll
    for (int i = 0; i < G::UPW; ++i) {
        const int qq = w + kW4Waves * i;
        if (kW4Waves * (i + 1) <= G::UROWS || qq < G::UROWS)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ur, (__attribute__((address_space(3))) void *)(lu + qq * 64), 16,
                                                     lane * 16, qq * 1024, 0, 0);
    }
}

// One step from LDS for point half H of a plain input: the lane's patch of
// its channel, the half's transform and its 2 x 18 MFMAs.  Every LDS read of
// the step (the 6 x 6 patch and the half's U) is issued first, so their
// latency is paid once per step and the transform consumes the values in the
// order they arrive (left to the compiler, the U reads went out just before
// their MFMAs into reused registers, each with a wait of its own).  The patch
// rows pass through B^T for the half's three columns, then each column is
// finished and multiplied at once.  Product k = 6 c + r of the half is point
// (r, 3H + c); its A operand for row block b is component k % 4 of float4
// b * 10 + 5 H + k / 4.
template <int TCW, int H>
__device__ __attribute__((always_inline)) inline void w4_step(const float *lx, const floatx4 *lu, const int (&pb)[3],
                                                             int lane, floatx4 (&acc)[kW4RB][W4Shape<false>::NX]) {
    using G = W4Geom<TCW, false>;
    using S = W4Shape<false>;
    static_assert(S::NX == 4 * (S::Q1 - 1) + 2, "products 16 and 17 fill half of the last float4");
    float d[6][6];
#pragma unroll
    for (int r = 0; r < 6; ++r)
#pragma unroll
        for (int h = 0; h < 3; ++h) {
            const floatx2 a = *reinterpret_cast<const floatx2 *>(lx + pb[h] + r * G::HCP);
            d[r][2 * h] = a[0];
            d[r][2 * h + 1] = a[1];
        }
    // the last float4 of a row block is read as its used half, so the
    // compiler does not reuse the other half's registers (which would make it
    // wait for every read in flight first)
    const floatx4 *ul = lu + H * S::Q1 * 64 + lane;
    floatx4 u[kW4RB][S::Q1 - 1];
    floatx2 ulast[kW4RB];
#pragma unroll
    for (int b = 0; b < kW4RB; ++b) {
#pragma unroll
        for (int q = 0; q < S::Q1 - 1; ++q) u[b][q] = ul[(b * S::UQ + q) * 64];
        ulast[b] = *reinterpret_cast<const floatx2 *>(ul + (b * S::UQ + S::Q1 - 1) * 64);
    }
    __builtin_amdgcn_sched_barrier(0);
    float t[6][3];   // d B, the half's columns
#pragma unroll
    for (int r = 0; r < 6; ++r) w4_bt_half<H>(d[r], t[r][0], t[r][1], t[r][2]);
    // The two waves of a SIMD (from two workgroups) share its datapath; with
    // the MFMA phase at the higher priority, one wave's MFMAs go first while
    // the other's transform, loads and barrier wait fill the gaps, instead of
    // both alternating instruction by instruction (measured 2-8% per plain
    // layer of the 1024x1024 decode; the whole step at the higher priority,
    // or the upsampled step's MFMA phase, measured slower).
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int c = 0; c < 3; ++c) {
        float v[6];
        w4_bt(t[0][c], t[1][c], t[2][c], t[3][c], t[4][c], t[5][c], v);
#pragma unroll
        for (int r = 0; r < 6; ++r) {
            const int k = 6 * c + r;
#pragma unroll
            for (int b = 0; b < kW4RB; ++b) {
                const float ua = k / 4 == S::Q1 - 1 ? ulast[b][k & 1] : u[b][k / 4 < S::Q1 - 1 ? k / 4 : 0][k % 4];
                acc[b][k] = __builtin_amdgcn_mfma_f32_16x16x4f32(ua, v[r], acc[b][k], 0, 0, 0);
            }
        }
    }
    __builtin_amdgcn_s_setprio(0);
}

// The 25 products of an upsampled input, over rows a and columns c indexing
// the points P = {0, 1, 3, 4, 5}: half 0 takes columns 0 and 1 and rows 0..2
// of column 2 (13 products), half 1 rows 3 and 4 of column 2 and columns 3 and
// 4 (12).  Product k of half H is (w4u_row(H, k), w4u_col(H, k)); a point
// index reads value w4u_src(a) of a source line's transform.
constexpr int w4u_col(int h, int k) { return h == 0 ? (k < 10 ? k / 5 : 2) : (k < 2 ? 2 : 3 + (k - 2) / 5); }
constexpr int w4u_row(int h, int k) { return h == 0 ? (k < 10 ? k % 5 : k - 10) : (k < 2 ? 3 + k : (k - 2) % 5); }
constexpr int w4u_count(int h) { return h == 0 ? 13 : 12; }
constexpr int w4u_src(int a) { return a <= 1 ? a : (a <= 3 ? 2 : 3); }

// One step from LDS for point half H of an upsampled input: the lane's 4 x 4
// source patch, the half's share of its transform (first pass: the half's
// distinct columns of each source row; then each distinct column, whose four
// values serve every product of it) and its 2 x 13 (12) MFMAs.  The A operand
// of product k for row block b is component k % 4 of float4 b * 7 + 4 H + k / 4.
// As in the plain step, every LDS read is issued first (left to itself the
// compiler read each U float4 just before its MFMAs; hoisted: the upsample
// convs of a 1024x1024 decode 4.84 -> 4.66 ms).
template <int TCW, int H>
__device__ __attribute__((always_inline)) inline void w4_step_up(const float *lx, const floatx4 *lu, const int (&pb)[2],
                                                                int lane, floatx4 (&acc)[kW4RB][W4Shape<true>::NX]) {
    using G = W4Geom<TCW, true>;
    using S = W4Shape<true>;
    constexpr int C0 = H == 0 ? 0 : 2, NC = H == 0 ? 3 : 2;   // the half's distinct columns C0 .. C0 + NC - 1
    float t[4][NC];
    // every LDS read of the step first: the patch rows, then the half's U
    // float4s of both row blocks
    floatx2 pa[4], pbv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        pa[r] = *reinterpret_cast<const floatx2 *>(lx + pb[0] + r * G::HCP);
        pbv[r] = *reinterpret_cast<const floatx2 *>(lx + pb[1] + r * G::HCP);
    }
    const floatx4 *ul = lu + H * S::Q1 * 64 + lane;
    constexpr int NQ = (w4u_count(H) + 3) / 4;
    floatx4 u[kW4RB][4];
#pragma unroll
    for (int b = 0; b < kW4RB; ++b)
#pragma unroll
        for (int q = 0; q < NQ; ++q) u[b][q] = ul[(b * S::UQ + q) * 64];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const floatx2 a = pa[r];
        const floatx2 b = pbv[r];
        if (H == 0) {
            t[r][0] = fmaf(4.f, a[0], fmaf(-5.f, a[1], b[0]));
            t[r][1] = fmaf(-8.f, a[1], 2.f * b[0]);
            t[r][2] = a[1] - b[0];
        } else {
            t[r][0] = a[1] - b[0];
            t[r][1] = fmaf(4.f, a[1], fmaf(-5.f, b[0], b[1]));
        }
    }
#pragma unroll
    for (int dc = 0; dc < NC; ++dc) {
        float w[4];
        w4_btu(t[0][dc], t[1][dc], t[2][dc], t[3][dc], w);
#pragma unroll
        for (int k = 0; k < w4u_count(H); ++k) {
            if (w4u_src(w4u_col(H, k)) != C0 + dc) continue;
#pragma unroll
            for (int b = 0; b < kW4RB; ++b) {
                acc[b][k] = __builtin_amdgcn_mfma_f32_16x16x4f32(u[b][k / 4][k % 4], w[w4u_src(w4u_row(H, k))], acc[b][k],
                                                                0, 0, 0);
            }
        }
    }
}

// The half's share of the output transform of register i of a row block:
// y[a][x] = sum over the half's products (r, c) of A^T[a][r] M[r][c] A^T[x][c].
template <int H>
__device__ __attribute__((always_inline)) inline void w4_out_half(const floatx4 (&acc)[W4Shape<false>::NX], int i,
                                                                 float (&y)[4][4]) {
    float s[4][3];
#pragma unroll
    for (int c = 0; c < 3; ++c) {
        float o[4];
        w4_at(acc[6 * c][i], acc[6 * c + 1][i], acc[6 * c + 2][i], acc[6 * c + 3][i], acc[6 * c + 4][i],
              acc[6 * c + 5][i], o);
#pragma unroll
        for (int a = 0; a < 4; ++a) s[a][c] = o[a];
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        if (H == 0) {   // columns 0, 1, 2 of A^T: (1 0 0 0), (1 1 1 1), (1 -1 1 -1)
            const float sp = s[a][1] + s[a][2], sm = s[a][1] - s[a][2];
            y[a][0] = s[a][0] + sp;
            y[a][1] = sm;
            y[a][2] = sp;
            y[a][3] = sm;
        } else {        // columns 3, 4, 5: (1 2 4 8), (1 -2 4 -8), (0 0 0 1)
            const float sp = s[a][0] + s[a][1], sm = s[a][0] - s[a][1];
            y[a][0] = sp;
            y[a][1] = 2.f * sm;
            y[a][2] = 4.f * sp;
            y[a][3] = fmaf(8.f, sm, s[a][2]);
        }
    }
}

// The same for an upsampled input's half (point 2 of M is zero; columns of
// A^T for the points {0, 1, 3, 4, 5}: (1 0 0 0), (1 1 1 1), (1 2 4 8),
// (1 -2 4 -8), (0 0 0 1)).
template <int H>
__device__ __attribute__((always_inline)) inline void w4_out_half_up(const floatx4 (&acc)[W4Shape<true>::NX], int i,
                                                                    float (&y)[4][4]) {
    constexpr float AC[5][4] = {{1.f, 0.f, 0.f, 0.f}, {1.f, 1.f, 1.f, 1.f}, {1.f, 2.f, 4.f, 8.f},
                                {1.f, -2.f, 4.f, -8.f}, {0.f, 0.f, 0.f, 1.f}};
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int x = 0; x < 4; ++x) y[a][x] = 0.f;
#pragma unroll
    for (int c = 0; c < 5; ++c) {
        float m[5] = {0.f, 0.f, 0.f, 0.f, 0.f};   // the half's products in column c
        bool any = false;
#pragma unroll
        for (int k = 0; k < w4u_count(H); ++k)
            if (w4u_col(H, k) == c) {
                m[w4u_row(H, k)] = acc[k][i];
                any = true;
            }
        if (!any) continue;
        float o[4];
        w4_at(m[0], m[1], 0.f, m[2], m[3], m[4], o);
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int x = 0; x < 4; ++x)
                if (AC[c][x] != 0.f) y[a][x] = fmaf(AC[c][x], o[a], y[a][x]);
    }
}

// The workgroup's work for the waves of point half H (H is the wave's index
// mod 2, so the two instantiations run side by side through the same
// barriers).
template <int TCW, bool UP, int H, bool RES, bool SPLIT>
__device__ __attribute__((always_inline)) inline void w4_body(const WParams &p, float *lx0, float *lx1, floatx4 *lu0,
                                                             floatx4 *lu1, float *lxb) {
    using G = W4Geom<TCW, UP>;
    using S = W4Shape<UP>;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wtg = wave >> 1;   // the wave's tile group
    const int g4 = lane >> 4;    // the lane's channel of a step, and its 4-row group of an MFMA output

    // blockIdx.x enumerates (tile block, channel block) with the channel block
    // fastest; when the count is a multiple of 8 each XCD walks one contiguous
    // band, so all channel blocks of a tile run on one XCD and share its input
    // through that XCD's L2.
    int lin = blockIdx.x;
    if ((gridDim.x & 7) == 0) lin = (lin & 7) * (gridDim.x >> 3) + (lin >> 3);
    const int tile = lin / p.ncb;
    const int cb = lin - tile * p.ncb;
    const int ty = tile / p.tiles_x;
    const int tx = tile - ty * p.tiles_x;
    const int y0 = ty * G::OR, x0 = tx * G::OC;
    const int frame = SPLIT ? blockIdx.z / p.ksplit : blockIdx.z;
    const int split = SPLIT ? blockIdx.z - frame * p.ksplit : 0;

    // The lane's tile and the offsets of its patch's column pairs.
    const int n = wtg * 16 + (lane & 15);
    const int tr = n / TCW, tc = n - (n / TCW) * TCW;
    const int Y0 = y0 + 4 * tr, X0 = x0 + 4 * tc;   // top-left output of the tile
    constexpr int NPAIR = UP ? 2 : 3, STRIDE = UP ? 2 : 4;   // column pairs of a patch row; tile spacing when staged
    int pb[NPAIR];
#pragma unroll
    for (int h = 0; h < NPAIR; ++h) pb[h] = g4 * G::PLANE + STRIDE * tr * G::HCP + w4_pos(STRIDE * tc + 2 * h, G::LAY);

    const int nsteps = p.kt * p.nquads;
    const int s0 = SPLIT ? (int)((long long)split * nsteps / p.ksplit) : 0;
    const int s1 = SPLIT ? (int)((long long)(split + 1) * nsteps / p.ksplit) : nsteps;
    WCursor cur = wino_cursor(p, frame, s0);

    floatx4 acc[kW4RB][S::NX];
#pragma unroll
    for (int b = 0; b < kW4RB; ++b)
#pragma unroll
        for (int k = 0; k < S::NX; ++k) acc[b][k] = floatx4{0.f, 0.f, 0.f, 0.f};

    // Per-lane byte offsets of this wave's chunks of a staged plane (the same
    // for every plane).
    int soffd[G::CPW];
#pragma unroll
    for (int i = 0; i < G::CPW; ++i) {
        const int e = 64 * (wave + kW4Waves * i) + lane;
        const int r = e / G::HCP, q = e - (e / G::HCP) * G::HCP;
        const int x = w4_col(q, G::LAY, G::HC);   // staged column at position q (-1: none)
        const int yy = (UP ? y0 >> 1 : y0) - 1 + r, xx = (UP ? x0 >> 1 : x0) - 1 + x;
        soffd[i] = (r < G::HR && x >= 0 && yy >= 0 && yy < p.Hin && xx >= 0 && xx < p.Win) ? (yy * p.Win + xx) * 4
                                                                                          : kWOOB;
    }

    // Step k + 1 is loaded while step k is computed.  The loop is unrolled by
    // two so each buffer is named statically; the step count is rounded up to
    // an even number with a dead step (zeros, adding exactly 0), which keeps
    // the loop free of a tail copy.
    const int nst = (s1 - s0 + 1) / 2 * 2;
    const float *ublk = p.u + (size_t)cb * nsteps * (G::UROWS * 256);
    // The barrier between steps orders only direct loads (each wave has
    // waited for its own) and LDS reads, so it needs no memory fence: a
    // compiler-only barrier keeps the accesses on their side of it.  The
    // scheduling barriers pin the order of the whole step: the next step's
    // loads are issued before any of this step's MFMAs, and the wait for them
    // comes after the last one (left free, the scheduler moves the wait and the
    // barrier, which touch no registers, into the middle of the MFMAs and the
    // loads down to just before the wait, exposing their latency every step).
    auto next = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };
    auto step = [&](const float *lx, const floatx4 *lu) {
        if constexpr (UP) w4_step_up<TCW, H>(lx, lu, pb, lane, acc);
        else w4_step<TCW, H>(lx, lu, pb, lane, acc);
    };
    w4_stage<TCW, UP>(p, frame, s0, s1, ublk, cur, lx0, lu0, soffd);
    next();
    for (int k = 0; k < nst; k += 2) {
        w4_stage<TCW, UP>(p, frame, s0 + k + 1, s1, ublk, cur, lx1, lu1, soffd);
        __builtin_amdgcn_sched_barrier(0);
        step(lx0, lu0);
        next();
        w4_stage<TCW, UP>(p, frame, s0 + k + 2, s1, ublk, cur, lx0, lu0, soffd);
        __builtin_amdgcn_sched_barrier(0);
        step(lx1, lu1);
        next();
    }

    // Epilogue, per row block b: register i of the block's 16 x 16 MFMA tile
    // is output channel 4 g4 + i of the block, for the lane's tile.  Each
    // wave applies its half of A^T, hands the other half's rows of the 4 x 4
    // block to its partner through LDS (half 0 finishes rows 0 and 1, half 1
    // rows 2 and 3) and adds the partner's share to its own rows.
    const long long fo = (long long)frame * p.out_fstride;
    const bool rowvec = (p.W & 3) == 0 && X0 < p.W;   // 4 outputs of a row in range, 16-byte aligned
    const bool full = Y0 + 2 * H + 1 < p.H && X0 + 3 < p.W;   // the lane's two rows of 4 outputs in range
    // [receiving half][i][row][col][lane]: a U buffer, or the upsampled kernel's own exchange area
    float *xb = UP ? lxb + wtg * (2 * 4 * 8 * 64) : reinterpret_cast<float *>(wtg == 0 ? lu0 : lu1);
    float gs[kW4RB][3];   // per row block: (count, mean, sum of squared deviations) of the lane's outputs
#pragma unroll
    for (int b = 0; b < kW4RB; ++b) {
        // the row block's residual rows are requested before its output
        // transform, so their latency overlaps that arithmetic
        floatx4 r4[4][2];
        if (RES && !SPLIT && rowvec) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int o = (cb * kW4RB + b) * kW4Blk + 4 * g4 + i;
                const long long cbase = (long long)(o < p.cout ? o : p.cout - 1) * p.out_cstride + fo;
#pragma unroll
                for (int a = 0; a < 2; ++a)
                    r4[i][a] = *reinterpret_cast<const floatx4 *>(p.res + cbase +
                                                                 (long long)min(Y0 + 2 * H + a, p.H - 1) * p.W + X0);
            }
        }
        float y[4][4][4];   // [i][row][col]
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (UP) w4_out_half_up<H>(acc[b], i, y[i]);
            else w4_out_half<H>(acc[b], i, y[i]);
        }
        // the partner's rows to LDS
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int x = 0; x < 4; ++x)
                    xb[(((1 - H) * 4 + i) * 8 + a * 4 + x) * 64 + lane] = y[i][2 * (1 - H) + a][x];
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int x = 0; x < 4; ++x) y[i][2 * H + a][x] += xb[((H * 4 + i) * 8 + a * 4 + x) * 64 + lane];
        __syncthreads();   // xb is rewritten by the next row block

        gs[b][0] = gs[b][1] = gs[b][2] = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int o = (cb * kW4RB + b) * kW4Blk + 4 * g4 + i;
            const bool ovalid = o < p.cout;
            const int oc = ovalid ? o : p.cout - 1;
            const float bo = SPLIT ? 0.f : p.bias[oc];
            const long long cbase = (long long)oc * p.out_cstride + fo;
            float v[2][4];
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                const int yy = Y0 + 2 * H + a;
                const bool rv = ovalid && yy < p.H;
                const long long rb = cbase + (long long)min(yy, p.H - 1) * p.W;
#pragma unroll
                for (int x = 0; x < 4; ++x) v[a][x] = y[i][2 * H + a][x] + bo;
                if (rowvec) {
                    if (RES && !SPLIT) {
#pragma unroll
                        for (int x = 0; x < 4; ++x) v[a][x] += r4[i][a][x];
                    }
                    if (rv) {
                        float *dst = SPLIT ? p.part + split * p.part_stride + rb + X0 : p.y + rb + X0;
                        *reinterpret_cast<floatx4 *>(dst) = floatx4{v[a][0], v[a][1], v[a][2], v[a][3]};
                    }
                } else {
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        const int xx = X0 + x;
                        const long long at = rb + min(xx, p.W - 1);
                        if (RES && !SPLIT) v[a][x] += p.res[at];
                        if (rv && xx < p.W) {
                            if (SPLIT) p.part[split * p.part_stride + at] = v[a][x];
                            else p.y[at] = v[a][x];
                        }
                    }
                }
            }
            if (!SPLIT && p.gn_rec) {
                // the channel's valid outputs among the wave's rows of the tile:
                // all 8 of them away from the bottom and right edges
                float cnt = 0.f, sum = 0.f, m2 = 0.f, mean = 0.f;
                if (ovalid && full) {
                    cnt = 8.f;
#pragma unroll
                    for (int a = 0; a < 2; ++a)
#pragma unroll
                        for (int x = 0; x < 4; ++x) sum += v[a][x];
                    mean = sum * 0.125f;
#pragma unroll
                    for (int a = 0; a < 2; ++a)
#pragma unroll
                        for (int x = 0; x < 4; ++x) {
                            const float dv = v[a][x] - mean;
                            m2 += dv * dv;
                        }
                } else {
#pragma unroll
                    for (int a = 0; a < 2; ++a)
#pragma unroll
                        for (int x = 0; x < 4; ++x)
                            if (ovalid && Y0 + 2 * H + a < p.H && X0 + x < p.W) {
                                cnt += 1.f;
                                sum += v[a][x];
                            }
                    mean = cnt > 0.f ? sum * __builtin_amdgcn_rcpf(cnt) : 0.f;
#pragma unroll
                    for (int a = 0; a < 2; ++a)
#pragma unroll
                        for (int x = 0; x < 4; ++x)
                            if (ovalid && Y0 + 2 * H + a < p.H && X0 + x < p.W) {
                                const float dv = v[a][x] - mean;
                                m2 += dv * dv;
                            }
                }
                wino_chan_merge(gs[b], cnt, mean, m2);
            }
        }
    }

    if (!SPLIT && p.gn_rec) {
        // GroupNorm records of the workgroup: per group (count, mean, sum of
        // squared deviations from that mean), merged pairwise (Chan, Golub
        // and LeVeque) over the 16 tiles of a lane group, then over the four
        // waves and the quads of a group, in a fixed order.  Quad 4 b + g4
        // holds output channels 16 b + 4 g4 + (0..3) of the workgroup.  The
        // host enables this only when a group is a whole number of quads
        // within the workgroup's 32 channels.
        float *qst = lx0;   // [wave][row block][quad][3]
#pragma unroll
        for (int o = 1; o < 16; o <<= 1)
#pragma unroll
            for (int b = 0; b < kW4RB; ++b) {
                const float nb = __shfl_xor(gs[b][0], o, 64);
                const float mb = __shfl_xor(gs[b][1], o, 64);
                const float qb = __shfl_xor(gs[b][2], o, 64);
                wino_chan_merge(gs[b], nb, mb, qb);
            }
        if ((lane & 15) == 0)
#pragma unroll
            for (int b = 0; b < kW4RB; ++b) {
                float *d = qst + ((wave * kW4RB + b) * 4 + g4) * 3;
                d[0] = gs[b][0];
                d[1] = gs[b][1];
                d[2] = gs[b][2];
            }
        __syncthreads();
        const int qpg = p.gn_cpg >> 2;
        const int gpb = kW4RB * kW4Blk / p.gn_cpg;
        if (tid < gpb) {
            float g[3] = {0.f, 0.f, 0.f};
            for (int w = 0; w < kW4Waves; ++w)
                for (int q = 0; q < qpg; ++q) {
                    const float *d = qst + (w * kW4RB * 4 + tid * qpg + q) * 3;
                    wino_chan_merge(g, d[0], d[1], d[2]);
                }
            const long long rec = (long long)(cb * gpb + tid) * p.gn_nrec + (long long)frame * (gridDim.x / p.ncb) + tile;
            p.gn_rec[rec] = floatx4{g[0], g[1], g[2], 0.f};
        }
    }
}

template <int TCW, bool UP, bool RES, bool SPLIT>
__global__ __launch_bounds__(kW4Threads) __attribute__((amdgpu_waves_per_eu(2, 2))) void conv3x3_wino4(WParams p) {
    using G = W4Geom<TCW, UP>;
    // Two stage buffers, declared apart: the compiler then knows that LDS
    // reads of one buffer do not wait for direct loads into the other.
    __shared__ __attribute__((aligned(16))) float lx0[G::XSTEP];
    __shared__ __attribute__((aligned(16))) float lx1[G::XSTEP];
    __shared__ floatx4 lu0[G::USTEP];
    __shared__ floatx4 lu1[G::USTEP];
    // the epilogue exchange of a wave pair: a U buffer, or (upsampled input,
    // whose U buffers are smaller) an area of its own
    __shared__ float lxb[UP ? kW4TG * 2 * 4 * 8 * 64 : 1];
    static_assert(UP || G::USTEP * 4 >= 2 * 4 * 8 * 64, "the epilogue exchange of a wave pair fits a U buffer");
    static_assert(G::XSTEP >= kW4Waves * kW4RB * 4 * 3, "the GroupNorm quads fit an input buffer");
    if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) & 1) w4_body<TCW, UP, 1, RES, SPLIT>(p, lx0, lx1, lu0, lu1, lxb);
    else w4_body<TCW, UP, 0, RES, SPLIT>(p, lx0, lx1, lu0, lu1, lxb);
}

// Packed U: [workgroup block of 32 output channels][step = (dt, channel
// quad)][row block b][q][lane][4] with lane = (channel of the quad) * 16 +
// (output channel within the row block).  A plain input's float4s q = 5 H +
// k / 4 hold product k = 6 c + r of half H, i.e. point (r, 3 H + c) of the
// transform, in component k % 4 (the two components past product 17 are
// zero); an upsampled input's float4s q = 4 H + k / 4 hold product k of half
// H (w4u_row, w4u_col over the points {0, 1, 3, 4, 5}), scaled by -3 for each
// index that is point 3.  Zero where the output or input channel is out of
// range and in the padding, so a workgroup's rows of one step are
// contiguous.  One thread per (block, step, row block, lane).
template <bool UP>
__global__ __launch_bounds__(256) void pack_wino4_kernel(const float *__restrict__ w, float *__restrict__ dst, int cout,
                                                         int cin, int kt, int nquads, long long total) {
    using S = W4Shape<UP>;
    const long long id = (long long)blockIdx.x * 256 + threadIdx.x;
    if (id >= total) return;
    const int lane = (int)(id & 63);
    const long long bsb = id >> 6;   // (block * nsteps + step) * kW4RB + row block
    const int nsteps = kt * nquads;
    const int b = (int)(bsb % kW4RB);
    const long long bs = bsb / kW4RB;
    const int blk = (int)(bs / nsteps);
    const int s = (int)(bs - (long long)blk * nsteps);
    const int dt = s / nquads, quad = s - dt * nquads;
    const int c = kWCh * quad + (lane >> 4);
    const int o = (blk * kW4RB + b) * kW4Blk + (lane & 15);
    const double G[6][3] = {{1.0 / 4, 0.0, 0.0},           {-1.0 / 6, -1.0 / 6, -1.0 / 6}, {-1.0 / 6, 1.0 / 6, -1.0 / 6},
                            {1.0 / 24, 1.0 / 12, 1.0 / 6}, {1.0 / 24, -1.0 / 12, 1.0 / 6}, {0.0, 0.0, 1.0}};
    double g[3][3];
#pragma unroll
    for (int i = 0; i < 9; ++i)
        g[i / 3][i % 3] = (o < cout && c < cin) ? (double)w[(((long long)o * cin + c) * kt + dt) * 9 + i] : 0.0;
    // U = G g G^T
    double t[6][3];
#pragma unroll
    for (int x = 0; x < 6; ++x)
#pragma unroll
        for (int j = 0; j < 3; ++j) t[x][j] = G[x][0] * g[0][j] + G[x][1] * g[1][j] + G[x][2] * g[2][j];
    auto U = [&](int x, int y) { return t[x][0] * G[y][0] + t[x][1] * G[y][1] + t[x][2] * G[y][2]; };
    float u[S::UQ * 4];
#pragma unroll
    for (int k = 0; k < S::UQ * 4; ++k) u[k] = 0.f;
    if (!UP) {
#pragma unroll
        for (int x = 0; x < 6; ++x)
#pragma unroll
            for (int y = 0; y < 6; ++y) {
                const int h = y / 3, k = 6 * (y % 3) + x;   // half, product of the half
                u[4 * S::Q1 * h + k] = (float)U(x, y);
            }
    } else {
        const int pts[5] = {0, 1, 3, 4, 5};
        const double f[5] = {1.0, 1.0, -3.0, 1.0, 1.0};   // point 3 reads -3 x the transformed input of point 4
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int k = 0; k < w4u_count(h); ++k) {
                const int a = w4u_row(h, k), cc = w4u_col(h, k);
                u[4 * S::Q1 * h + k] = (float)(f[a] * f[cc] * U(pts[a], pts[cc]));
            }
    }
    float *out = dst + bsb * (S::UQ * 256) + lane * 4;
#pragma unroll
    for (int q = 0; q < S::UQ; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) out[q * 256 + e] = u[4 * q + e];
}

int w4_tcw(int W) { return W > 32 ? 16 : (W > 16 ? 8 : 4); }

struct W4Grid {
    int tcw, tiles_x, tiles_y, ncb;
};

W4Grid w4_grid(int cout, int H, int W) {
    W4Grid g;
    g.tcw = w4_tcw(W);
    const int oc = 4 * g.tcw, orr = 4 * (16 * kW4TG / g.tcw);
    g.tiles_x = (W + oc - 1) / oc;
    g.tiles_y = (H + orr - 1) / orr;
    g.ncb = (cout + kW4RB * kW4Blk - 1) / (kW4RB * kW4Blk);
    return g;
}

template <int TCW, bool UP>
void w4_launch_t(const WParams &p, bool res, bool split, dim3 grid, hipStream_t s) {
    if (split) hipLaunchKernelGGL((conv3x3_wino4<TCW, UP, false, true>), grid, dim3(kW4Threads), 0, s, p);
    else if (res) hipLaunchKernelGGL((conv3x3_wino4<TCW, UP, true, false>), grid, dim3(kW4Threads), 0, s, p);
    else hipLaunchKernelGGL((conv3x3_wino4<TCW, UP, false, false>), grid, dim3(kW4Threads), 0, s, p);
}

template <int TCW>
void w4_launch_tc(const WParams &p, bool up, bool res, bool split, dim3 grid, hipStream_t s) {
    if (up) w4_launch_t<TCW, true>(p, res, split, grid, s);
    else w4_launch_t<TCW, false>(p, res, split, grid, s);
}

}  // namespace

size_t conv3x3_wino4_packed_floats(int cout, int cin, int kt, int up) {
    const size_t blocks = (size_t)(cout + kW4RB * kW4Blk - 1) / (kW4RB * kW4Blk);
    const size_t nsteps = (size_t)kt * ((cin + kWCh - 1) / kWCh);
    return blocks * nsteps * kW4RB * (up ? W4Shape<true>::UQ : W4Shape<false>::UQ) * 256;
}

int32_t pack_conv3x3_wino4(const float *w, int cout, int cin, int kt, int up, float *dst, hipStream_t s) {
    const int nquads = (cin + kWCh - 1) / kWCh;
    const long long blocks = (cout + kW4RB * kW4Blk - 1) / (kW4RB * kW4Blk);
    const long long total = blocks * kt * nquads * kW4RB * 64;
    const dim3 grid((unsigned)((total + 255) / 256));
    if (up) hipLaunchKernelGGL(pack_wino4_kernel<true>, grid, dim3(256), 0, s, w, dst, cout, cin, kt, nquads, total);
    else hipLaunchKernelGGL(pack_wino4_kernel<false>, grid, dim3(256), 0, s, w, dst, cout, cin, kt, nquads, total);
    return check_launch("pack_conv3x3_wino4");
}

int conv3x3_wino4_ksplit(const ConvLaunch &a) {
    const W4Grid g = w4_grid(a.cout, a.H, a.W);
    const long long base = (long long)g.tiles_x * g.tiles_y * g.ncb * a.T;
    const int nsteps = a.kt * ((a.cin + kWCh - 1) / kWCh);
    auto cap = [&](long long s) {
        if (s > nsteps / 4) s = nsteps / 4;            // each split keeps >= 4 steps
        if (s > 16) s = 16;
        if (s * a.T > 65535) s = 65535 / a.T;
        return s < 1 ? 1LL : s;
    };
    // Candidates: the fewest splits that fill one round of resident workgroups,
    // and twice that.  Cost, in full-K workgroup times: rounds of workgroups
    // over splits, with the doubled split charged 15% for its partial sums and
    // their reduction (measured 7-32% per doubling at equal rounds per split).
    const long long s1 = cap(base >= kW4Slots ? 1 : (kW4Slots + base - 1) / base);
    const long long s2 = cap(2 * s1);
    auto cost = [&](long long s) {
        return (double)((base * s + kW4Slots - 1) / kW4Slots) / (double)s * (s > s1 ? 1.15 : 1.0);
    };
    return (int)(cost(s2) < cost(s1) ? s2 : s1);
}

int conv3x3_wino4_gn_records(const ConvLaunch &a) {
    if (a.cout % 128 != 0 || a.cout / 32 > kW4RB * kW4Blk) return 0;
    const W4Grid g = w4_grid(a.cout, a.H, a.W);
    return g.tiles_x * g.tiles_y * a.T;
}

int conv3x3_wino4_tcw(const ConvLaunch &a) { return w4_tcw(a.W); }

int32_t launch_conv3x3_wino4_main(const ConvLaunch &a, hipStream_t s) {
    if (a.denorm || a.gn_coef) {
        set_error("conv3x3_wino4: no de-normalisation or GroupNorm on load");
        return VAE_ERR_UNSUPPORTED;
    }
    if ((a.wino == 4) != (a.upsample != 0) || a.wino < 3) {
        set_error("conv3x3_wino4: weights not packed by pack_conv3x3_wino4 for %s input",
                  a.upsample ? "an upsampled" : "a plain");
        return VAE_ERR_INVALID_ARG;
    }
    if (a.upsample && ((a.H | a.W) & 1)) {
        set_error("conv3x3_wino4: an upsampled input has even sizes");
        return VAE_ERR_INVALID_ARG;
    }
    WParams p;
    p.x = a.x;
    p.u = a.wpk;
    p.bias = a.bias;
    p.res = a.res;
    p.gn_coef = nullptr;
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
    const W4Grid g = w4_grid(a.cout, a.H, a.W);
    p.tiles_x = g.tiles_x;
    p.ncb = g.ncb;
    p.nub = g.ncb * kW4RB;
    p.ksplit = conv3x3_wino4_ksplit(a);
    p.part = a.part;
    p.part_stride = p.out_cstride * a.cout;
    if (p.ksplit > 1 && !a.part) {
        set_error("conv3x3_wino4: split-K needs a partial-sum workspace");
        return VAE_ERR_WORKSPACE;
    }
    // byte offsets within one channel are 32-bit
    if (p.in_cstride * 4 >= (1LL << 31)) {
        set_error("conv3x3_wino4: input channel of %lld elements is too large", p.in_cstride);
        return VAE_ERR_UNSUPPORTED;
    }
    const long long nwg = (long long)g.tiles_x * g.tiles_y * g.ncb;
    if (nwg >= (1LL << 31)) {
        set_error("conv3x3_wino4: %lld workgroups exceed the grid limit", nwg);
        return VAE_ERR_UNSUPPORTED;
    }
    const dim3 grid((unsigned)nwg, 1u, (unsigned)(a.T * p.ksplit));
    p.gn_rec = nullptr;
    p.gn_cpg = 0;
    p.gn_nrec = 0;
    if (a.gn_rec && p.ksplit == 1) {
        if (conv3x3_wino4_gn_records(a) == 0) {
            set_error("conv3x3_wino4: GroupNorm records in the epilogue need out_channels %% 128 == 0 (<= %d)",
                      32 * kW4RB * kW4Blk);
            return VAE_ERR_UNSUPPORTED;
        }
        p.gn_rec = a.gn_rec;
        p.gn_cpg = a.cout / 32;
        p.gn_nrec = g.tiles_x * g.tiles_y * (int)grid.z;
    }
    const bool up = a.upsample != 0, res = a.res != nullptr, split = p.ksplit > 1;
    switch (g.tcw) {
    case 16: w4_launch_tc<16>(p, up, res, split, grid, s); break;
    case 8: w4_launch_tc<8>(p, up, res, split, grid, s); break;
    default: w4_launch_tc<4>(p, up, res, split, grid, s); break;
    }
    return check_launch("conv3x3_wino4");
}

}  // namespace vae
