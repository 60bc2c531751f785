// Direct 3x3 convolution for a handful of output channels: the decoder's
// conv_out, 128 -> 3 (cortiq-engine 0.7.7 `vae`, VaeDecoder).  With three
// output channels the GEMM is far too thin for MFMA; this kernel streams the
// input once with float4 loads, keeps the weights in the scalar cache and
// does the 27 (or 81, for the causal 3x3x3 conv of a clip) multiply-adds
// per input value on the vector ALUs.  The decoder's norm_out GroupNorm +
// SiLU is applied while the input is loaded, so the normalised tensor is
// never written.

#include "vae_internal.h"

namespace vae {

namespace {

constexpr int kThreads = 256;
constexpr int kGnMaxChannels = kDirectGnMaxChannels;
constexpr int kDirectSlots = 1024;   // about 4 conv_out workgroups per CU

// Direct 3x3 conv for a handful of output channels.  Workgroup tile: 8 rows x
// 128 columns; thread (r, g) computes pixels 4g..4g+3 of row r for every
// output channel.  Input channels go in chunks of 4: the chunk's halo tile
// [4][10][128 + 2] is loaded into registers (float4 loads for the 128
// interior columns, one scalar per row edge) while the previous chunk is
// being used, then written to LDS.  The weights are the same for the whole
// workgroup and are read through the scalar cache.
constexpr int kDR = 8;                 // tile rows
constexpr int kDC = 128;               // tile columns
constexpr int kDCC = 4;                // input channels per chunk
constexpr int kDRow = kDC + 8;         // LDS row: [pad x3][left][128 interior][right][pad x3]
constexpr int kDRows = kDR + 2;
constexpr int kDQuads = kDCC * kDRows * (kDC / 4);            // float4 items per chunk (1280)
constexpr int kDQPerT = (kDQuads + kThreads - 1) / kThreads;  // 5
constexpr int kDEdges = kDCC * kDRows * 2;                    // scalar edge items per chunk (80)

// A clip [cin, T, H, W] with KT = 3 time taps is the causal 3x3x3 conv
// (frame index clamped at 0, i.e. frame 0 repeated in front): the chunks
// then run over (time tap, 4 channels) and blockIdx.z is the output frame.
// blockIdx.y = split: with several splits, split s sums the chunks
// [s * n / splits, (s + 1) * n / splits) into part[s] (no bias) and
// splitk_reduce adds the splits in order.
template <int COUT, bool GN, int KT>
__global__ __launch_bounds__(kThreads) void conv3x3_direct(const float *__restrict__ x,
                                                           const float *__restrict__ w,
                                                           const float *__restrict__ bias,
                                                           float *__restrict__ y, int cin, int H,
                                                           int W, int tiles_x,
                                                           const float *__restrict__ gn_coef,
                                                           float *__restrict__ part) {
    __shared__ __attribute__((aligned(16))) float halo[kDCC * kDRows * kDRow];
    __shared__ float lc[GN ? 3 * (kGnMaxChannels + kDCC) : 1];
    const int tid = threadIdx.x;
    const int ty = blockIdx.x / tiles_x, tx = blockIdx.x - (blockIdx.x / tiles_x) * tiles_x;
    const int y0 = ty * kDR, x0 = tx * kDC;
    const int r = tid >> 5, g = tid & 31;
    const long long plane = (long long)H * W;
    const int T = gridDim.z, t = blockIdx.z;
    const long long cstride = plane * T;   // channel stride of x and y
    // interior columns of this tile all inside the image and rows 16-byte aligned
    const bool vec = (W & 3) == 0 && x0 + kDC <= W && (reinterpret_cast<uintptr_t>(x) & 15) == 0;
    const bool vec_out = (W & 3) == 0 && x0 + kDC <= W &&
                         (reinterpret_cast<uintptr_t>(part ? part : y) & 15) == 0;
    const int n_cb = (cin + kDCC - 1) / kDCC;
    const int n_chunks = KT * n_cb;   // chunk q = (time tap q / n_cb, channels 4 (q % n_cb) ..)
    const int cb0 = (int)((long long)blockIdx.y * n_chunks / gridDim.y);
    const int cb1 = (int)((long long)(blockIdx.y + 1) * n_chunks / gridDim.y);

    if (GN) {
        for (int e = tid; e < 3 * n_cb * kDCC; e += kThreads) {
            const int c = e / 3, k = e - 3 * (e / 3);
            lc[e] = c < cin ? gn_coef[4 * c + k] : 0.f;
        }
    }

    floatx4 q[kDQPerT];
    float edge = 0.f;
    auto gn = [&](float v, int c) {
        const float *cf = lc + 3 * c;
        const float t = (v - cf[0]) * cf[1] + cf[2];
        return t * __builtin_amdgcn_rcpf(1.f + __expf(-t));
    };
    // global -> registers for chunk qc: time tap qc / n_cb, channels from c0
    auto load = [&](int qc) {
        const int dt = qc / n_cb, c0 = (qc - dt * n_cb) * kDCC;
        int fr = t + dt - (KT - 1);
        fr = fr < 0 ? 0 : fr;
        const float *xf = x + fr * plane;
#pragma unroll
        for (int j = 0; j < kDQPerT; ++j) {
            const int k = tid + j * kThreads;
            floatx4 v = {0.f, 0.f, 0.f, 0.f};
            if (k < kDQuads) {
                const int c = k / (kDRows * 32), rem = k - c * (kDRows * 32);
                const int row = rem >> 5, qq = rem & 31;
                const int ch = c0 + c, yy = y0 - 1 + row, xx = x0 + 4 * qq;
                if (ch < cin && yy >= 0 && yy < H) {
                    const float *src = xf + ch * cstride + (long long)yy * W + xx;
                    if (vec) {
                        v = *reinterpret_cast<const floatx4 *>(src);
                        if (GN) {
                            v[0] = gn(v[0], ch);
                            v[1] = gn(v[1], ch);
                            v[2] = gn(v[2], ch);
                            v[3] = gn(v[3], ch);
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (xx + e < W) v[e] = GN ? gn(src[e], ch) : src[e];
                    }
                }
            }
            q[j] = v;
        }
        if (tid < kDEdges) {
            const int c = tid / (2 * kDRows), rem = tid - c * (2 * kDRows);
            const int row = rem >> 1, side = rem & 1;
            const int ch = c0 + c, yy = y0 - 1 + row, xx = side ? x0 + kDC : x0 - 1;
            float v = 0.f;
            if (ch < cin && yy >= 0 && yy < H && xx >= 0 && xx < W) {
                v = xf[ch * cstride + (long long)yy * W + xx];
                if (GN) v = gn(v, ch);
            }
            edge = v;
        }
    };
    auto store = [&]() {
#pragma unroll
        for (int j = 0; j < kDQPerT; ++j) {
            const int k = tid + j * kThreads;
            if (k < kDQuads) {
                const int c = k / (kDRows * 32), rem = k - c * (kDRows * 32);
                const int row = rem >> 5, qq = rem & 31;
                *reinterpret_cast<floatx4 *>(&halo[(c * kDRows + row) * kDRow + 4 + 4 * qq]) = q[j];
            }
        }
        if (tid < kDEdges) {
            const int c = tid / (2 * kDRows), rem = tid - c * (2 * kDRows);
            const int row = rem >> 1, side = rem & 1;
            halo[(c * kDRows + row) * kDRow + (side ? 4 + kDC : 3)] = edge;
        }
    };

    float acc[COUT][4];
#pragma unroll
    for (int o = 0; o < COUT; ++o)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[o][e] = 0.f;

    if (GN) __syncthreads();   // coefficient table
    load(cb0);
    for (int qc = cb0; qc < cb1; ++qc) {
        const int dt = qc / n_cb, c0 = (qc - dt * n_cb) * kDCC;
        store();
        __syncthreads();
        if (qc + 1 < cb1) load(qc + 1);
#pragma unroll
        for (int c = 0; c < kDCC; ++c) {
            const int ch = c0 + c;
            if (ch >= cin) break;
#pragma unroll
            for (int dy = 0; dy < 3; ++dy) {
                const float *row = &halo[(c * kDRows + r + dy) * kDRow + 4 * g + 3];
                const floatx4 mid = *reinterpret_cast<const floatx4 *>(row + 1);
                const float v[6] = {row[0], mid[0], mid[1], mid[2], mid[3], row[5]};
#pragma unroll
                for (int dx = 0; dx < 3; ++dx)
#pragma unroll
                    for (int o = 0; o < COUT; ++o) {
                        const float wv = w[(((long long)o * cin + ch) * KT + dt) * 9 + dy * 3 + dx];
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[o][e] = fmaf(wv, v[e + dx], acc[o][e]);
                    }
            }
        }
        __syncthreads();
    }
    const int yy = y0 + r;
    if (yy >= H) return;
    const int xx = x0 + 4 * g;
    float *out = (part ? part + (long long)blockIdx.y * COUT * cstride : y) + t * plane;
#pragma unroll
    for (int o = 0; o < COUT; ++o) {
        const float b = part ? 0.f : bias[o];
        float *dst = out + o * cstride + (long long)yy * W + xx;
        if (vec_out) {
            *reinterpret_cast<floatx4 *>(dst) = floatx4{acc[o][0] + b, acc[o][1] + b, acc[o][2] + b, acc[o][3] + b};
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (xx + e < W) dst[e] = acc[o][e] + b;
        }
    }
}

}  // namespace


int conv3x3_direct_splits(int cin, int kt, int H, int W, int T) {
    const long long tiles = (long long)((W + kDC - 1) / kDC) * ((H + kDR - 1) / kDR) * T;
    const int n_chunks = kt * ((cin + kDCC - 1) / kDCC);
    if (tiles * 2 >= kDirectSlots) return 1;
    long long s = (kDirectSlots + tiles - 1) / tiles;
    if (s > n_chunks / 4) s = n_chunks / 4;   // each split keeps >= 4 chunks (16 channels)
    if (s > 16) s = 16;
    return s < 2 ? 1 : (int)s;
}

size_t conv3x3_direct_partial_floats(int cout, int cin, int kt, int H, int W, int T) {
    const int sp = conv3x3_direct_splits(cin, kt, H, W, T);
    return sp > 1 ? (size_t)sp * cout * T * H * W : 0;
}

int32_t launch_conv3x3_direct(const float *x, const float *w, const float *bias, float *y, int cin,
                              int cout, int H, int W, hipStream_t s, const float *gn_coef, float *part, int T,
                              int kt) {
    if (gn_coef && cin > kGnMaxChannels) {
        set_error("conv3x3_direct: GroupNorm-on-load holds at most %d input channels", kGnMaxChannels);
        return VAE_ERR_UNSUPPORTED;
    }
    if ((kt != 1 && kt != 3) || T < 1 || T > 65535) {
        set_error("conv3x3_direct: %d time taps over %d frames unsupported", kt, T);
        return VAE_ERR_UNSUPPORTED;
    }
    const int splits = conv3x3_direct_splits(cin, kt, H, W, T);
    if (splits > 1 && !part) {
        set_error("conv3x3_direct: a split shape needs a partial-sum workspace");
        return VAE_ERR_WORKSPACE;
    }
    float *pp = splits > 1 ? part : nullptr;
    const int tiles_x = (W + kDC - 1) / kDC;
    const int tiles_y = (H + kDR - 1) / kDR;
    const dim3 grid((unsigned)(tiles_x * tiles_y), (unsigned)splits, (unsigned)T);
#define VAE_DIRECT_KT(N, G, K) \
    hipLaunchKernelGGL((conv3x3_direct<N, G, K>), grid, dim3(kThreads), 0, s, x, w, bias, y, cin, H, W, tiles_x, gn_coef, pp);
#define VAE_DIRECT(N)                                                     \
    if (kt == 3) {                                                        \
        if (gn_coef) VAE_DIRECT_KT(N, true, 3) else VAE_DIRECT_KT(N, false, 3) \
    } else {                                                              \
        if (gn_coef) VAE_DIRECT_KT(N, true, 1) else VAE_DIRECT_KT(N, false, 1) \
    }
    switch (cout) {
        case 1: VAE_DIRECT(1) break;
        case 2: VAE_DIRECT(2) break;
        case 3: VAE_DIRECT(3) break;
        case 4: VAE_DIRECT(4) break;
        default: set_error("conv3x3_direct: out_channels %d > 4", cout); return VAE_ERR_UNSUPPORTED;
    }
#undef VAE_DIRECT
#undef VAE_DIRECT_KT
    int32_t rc = check_launch("conv3x3_direct");
    if (rc != VAE_OK || splits == 1) return rc;
    const long long plane = (long long)T * H * W;
    return launch_rows_reduce(part, plane * cout, splits, bias, y, plane, cout, s);
}
}  // namespace vae
