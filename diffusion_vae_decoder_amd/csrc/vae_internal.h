// Internal declarations shared by the HIP sources of libvae.so.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <string>

#include "../../include/vae.h"

namespace vae {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ errors
void set_error(const char *fmt, ...);
int32_t hip_status(hipError_t e, const char *what);
int32_t check_launch(const char *what);
// Argument checks of the GroupNorm entry points (NULLs, sizes, channel count,
// c % 32); sets the message under `who` and returns its code.
int32_t check_groupnorm_args(const char *who, const float *x, int c, long long spatial, const vae_norm *norm,
                             const float *y);

// ------------------------------------------------------------------ conv
// Geometry of the implicit-GEMM 3x3 conv: a workgroup computes 128 output
// channels x 128 output pixels (TR rows x TC columns of one frame).
constexpr int kConvBM = 128;
constexpr int kConvBN = 128;
constexpr int kConvCC = 4;   // input channels per K chunk (K chunk = 4 x 9 taps)

struct ConvLaunch {
    const float *x;        // input activations
    const float *wpk;      // packed weights, in the layout `wino` names
    const float *bias;     // [cout]
    const float *res;      // residual [cout, (T,) H, W] or nullptr
    float *y;              // output  [cout, (T,) H, W]
    int cin, cout;
    int H, W;              // output height/width (the conv's own input size after upsampling)
    int T;                 // frames (1 for 2-D)
    int kt;                // time taps (1 for 2-D, 3 for causal 3-D)
    int upsample;          // input is the nearest-x2 upsample of x
    int denorm;            // input is x / dn_scale + dn_shift (padding stays 0)
    float dn_scale, dn_shift;
    float *part;           // split-K partial sums, conv3x3_partial_floats() floats (or nullptr if 0)
    const float *gn_coef;  // if set: the input is silu((x - c[0]) * c[1] + c[2]) with c = gn_coef[4*channel..]
                           // (GroupNorm + SiLU applied on load; padding stays 0)
    floatx4 *gn_rec;       // if set: GroupNorm(32) records of y for the normalisation that follows,
                           // [32][conv3x3_gn_records()] of (count, mean, M2, 0); M2 is the sum of
                           // squared deviations from the record's own mean
    int wino;              // wpk layout: 0 pack_conv3x3 (implicit GEMM); 1, 2 pack_conv3x3_wino
                           // (Winograd F(2x2,3x3)) for a plain, an upsampled input; 3, 4
                           // pack_conv3x3_wino4 (Winograd F(4x4,3x3)) for a plain, an upsampled input
};

// Bytes of the packed weights for a conv with `cout` x `cin` x (kt x 3 x 3).
size_t conv3x3_packed_floats(int cout, int cin, int kt);
// Enqueue the repacking of raw weights [cout, cin, (kt,) 3, 3] into `dst`.
int32_t pack_conv3x3(const float *w, int cout, int cin, int kt, float *dst, hipStream_t s);
// Enqueue one implicit-GEMM conv: the conv kernel, then (for a K-split
// shape) the reduction of its partial sums with bias and residual.
int32_t launch_conv3x3(const ConvLaunch &a, hipStream_t s);
int32_t launch_conv3x3_main(const ConvLaunch &a, hipStream_t s);
int32_t launch_conv3x3_reduce(const ConvLaunch &a, hipStream_t s);
// K-split factor launch_conv3x3 uses for `a` (its shape and weight layout;
// 1 = none), and the partial-sum workspace it then needs (floats, 0 when not
// split).
int conv3x3_ksplit(const ConvLaunch &a);
size_t conv3x3_partial_floats(const ConvLaunch &a);
// GroupNorm records per group that launch_conv3x3 writes for `a` when
// a.gn_rec is set; 0 if this launch cannot produce them (then normalise with
// a separate statistics pass).
int conv3x3_gn_records(const ConvLaunch &a);
// Name of the kernel instantiation launch_conv3x3 picks for `a`.
const char *conv3x3_kernel_name(const ConvLaunch &a);

// Winograd F(2x2, 3x3) form of the same conv (conv_wino.hip): weights packed
// by pack_conv3x3_wino (`up`: for a nearest-x2 upsampled input, which only
// this packing may then be used with).  Same split-K factor, partial-sum
// workspace, reduction and GroupNorm records as the implicit GEMM; no
// de-normalisation, and GroupNorm on load only of a plain input.
size_t conv3x3_wino_packed_floats(int cout, int cin, int kt, int up);
int32_t pack_conv3x3_wino(const float *w, int cout, int cin, int kt, int up, float *dst, hipStream_t s);
int32_t launch_conv3x3_wino_main(const ConvLaunch &a, hipStream_t s);
int conv3x3_wino_ksplit(const ConvLaunch &a);
int conv3x3_wino_gn_records(const ConvLaunch &a);
int conv3x3_wino_tcw(const ConvLaunch &a);   // tiles per row of its workgroup block

// Winograd F(4x4, 3x3) form (conv_wino4.hip): weights packed by
// pack_conv3x3_wino4 (`up`: for an upsampled input, which only this packing
// may then be used with); same split-K workspace, reduction and GroupNorm
// records as the forms above; no de-normalisation or GroupNorm on load.
size_t conv3x3_wino4_packed_floats(int cout, int cin, int kt, int up);
int32_t pack_conv3x3_wino4(const float *w, int cout, int cin, int kt, int up, float *dst, hipStream_t s);
int32_t launch_conv3x3_wino4_main(const ConvLaunch &a, hipStream_t s);
int conv3x3_wino4_ksplit(const ConvLaunch &a);
int conv3x3_wino4_gn_records(const ConvLaunch &a);
int conv3x3_wino4_tcw(const ConvLaunch &a);
// The ConvLaunch::wino layout a conv's weights are packed in now: the form
// the process-wide setting (set_conv3x3_algorithm) selects, for a plain or
// an upsampled input; the implicit GEMM for an input de-normalised on load.
// Then its packed floats and the packing; conv3x3_pack_floats_max bounds
// every layout.  conv3x3_layout_gn_on_load: whether a layout's kernel can
// apply GroupNorm + SiLU while loading its input.
int conv3x3_layout(int denorm, int upsample);
bool conv3x3_layout_gn_on_load(int layout);
int32_t set_conv3x3_algorithm(int32_t algorithm);
int32_t get_conv3x3_algorithm();
size_t conv3x3_pack_floats(int layout, int cout, int cin, int kt);
size_t conv3x3_pack_floats_max(int cout, int cin, int kt);
int32_t pack_conv3x3_layout(int layout, const float *w, int cout, int cin, int kt, float *dst, hipStream_t s);

// y[o, :] = bias[o] + sum_s part[s * part_stride + o * plane + :] over `splits`
// partial-sum slices, in slice order, for `rows` rows of `plane` elements.
int32_t launch_rows_reduce(const float *part, long long part_stride, int splits, const float *bias, float *y,
                           long long plane, int rows, hipStream_t s);

// Direct conv for out_channels <= 4 (conv_out); gn_coef as in ConvLaunch (may be nullptr,
// else at most kDirectGnMaxChannels input channels).
constexpr int kDirectGnMaxChannels = 512;
// Shapes with too few tiles split the input channels; the partial sums then
// need conv3x3_direct_partial_floats() floats in `part`.  kt = 3: the causal
// 3x3x3 conv of a clip of T frames, weights [cout, cin, 3, 3, 3].
int32_t launch_conv3x3_direct(const float *x, const float *w, const float *bias, float *y,
                              int cin, int cout, int H, int W, hipStream_t s,
                              const float *gn_coef, float *part, int T = 1, int kt = 1);
size_t conv3x3_direct_partial_floats(int cout, int cin, int kt, int H, int W, int T);

// ------------------------------------------------------------------ GEMM
// C[m, n] = alpha * sum_k A(m, k) B(k, n) + bias[m] (+ R[m, n]).
// A(m, k) = a_km ? A[k * lda + m] : A[m * lda + k]
// B(k, n) = b_nk ? B[n * ldb + k] : B[k * ldb + n]
struct GemmLaunch {
    const float *A;
    const float *B;
    const float *bias;   // [M] or nullptr
    const float *R;      // [M, N] with ldr, or nullptr
    float *C;
    int M, N, K;
    long long lda, ldb, ldc, ldr;
    int a_km, b_nk;
    float alpha;
    // Row softmax split over two products (attention only; see gemm.hip):
    float *colstat;        // if set: C holds exp(c - mb) with mb the maximum of column n over its
                           // 128-row block, and colstat the (mb, sum exp(c - mb)) of each block,
                           // [ceil(M / 128)][N] pairs; needs a_km, KN B and no residual
    const float *bsoft;    // if set: B(k, n) -> B(k, n) * exp(blk - bsoft[2n]) * bsoft[2n + 1], with
                           // blk = bsoft_blk[2 ((k / 128) N + n)]; needs MK A, KN B
    const float *bsoft_blk;
    float *part;           // K-split partial sums, gemm_partial_floats() floats (nullptr if 0); C's ldc must be N
};
int32_t launch_gemm(const GemmLaunch &g, hipStream_t s);
// K-split factor launch_gemm uses (1 = none; never with colstat) and the
// partial-sum floats it then needs.
int gemm_ksplit(int M, int N, int K, bool colstat);
size_t gemm_partial_floats(int M, int N, int K, bool colstat);

// ------------------------------------------------------------------ norm
size_t groupnorm_ws_bytes(int c, long long spatial);
// y = silu?(GroupNorm(x)) (+ res).  With `rec` (nrec records per group, as a
// producer wrote them in ConvLaunch::gn_rec) the statistics are merged from
// the records instead of a pass over x.
int32_t launch_groupnorm(const float *x, int c, long long spatial, const float *gamma,
                         const float *beta, int silu, const float *res, float *y, void *ws,
                         hipStream_t s, const floatx4 *rec = nullptr, int nrec = 0);
// Statistics only: writes coef[4*c + {0,1,2}] = (mean of c's group, rstd * gamma[c], beta[c])
// for a consumer that normalises while loading.  ws and rec as for launch_groupnorm.
int32_t launch_groupnorm_coef(const float *x, int c, long long spatial, const float *gamma, const float *beta,
                              void *ws, float *coef, hipStream_t s, const floatx4 *rec = nullptr,
                              int nrec = 0);

// ------------------------------------------------------------------ misc
int32_t launch_upsample2x(const float *x, int c, int h, int w, float *y, hipStream_t s);

// Attention on x [c, n] with packed qkv weights [3c, c] and bias [3c].
size_t attention_ws_bytes(int c, long long n);
int32_t launch_attention(const float *x, int c, int h, int w, const float *gn_gamma,
                         const float *gn_beta, const float *wqkv, const float *bqkv,
                         const float *wo, const float *bo, float *y, void *ws, hipStream_t s);

// The streaming-softmax form of the same attention (attention_flash.hip):
// c in {32, 64, 128, 256, 512}; the key-range count it splits n tokens into;
// the core on Q, V [c, n] and K^T [n, c] (Op/ml: per-range partials, used when
// the range count is above 1); and the whole layer.
bool attention_flash_supported(int c);
int attention_flash_ranges(long long n);
int32_t launch_attention_flash_core(const float *Q, const float *KT, const float *V, float *O, float *Op,
                                    float *ml, int c, long long n, hipStream_t s);
size_t attention_streaming_ws_bytes(int c, long long n);
int32_t launch_attention_streaming(const float *x, int c, int h, int w, const float *gn_gamma,
                                   const float *gn_beta, const float *wqkv, const float *bqkv,
                                   const float *wo, const float *bo, float *y, void *ws, hipStream_t s);

}  // namespace vae
