/*
 * vae.h -- C ABI of libvae.so, an MI355X (gfx950) FLUX-class VAE decoder.
 *
 * The library decodes a FLUX-class AutoencoderKL latent [16, h, w] into RGB
 * [3, 8h, 8w] (docs.rs, cortiq-engine 0.7.7, module `vae`: module doc and
 * struct VaeDecoder) and exports the decoder's layers one by one.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are float32, batch 1, channel-major (NCHW without the N, or
 *    C,T,H,W for the 3-D conv), densely packed, in DEVICE memory of the
 *    current HIP device.  Pointers are borrowed: the caller owns and frees
 *    every buffer, including workspaces.  The library allocates nothing.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues work on it and returns; nothing is synchronised.  Inputs must
 *    stay alive and unmodified until that work has run.
 *  - Outputs must not overlap inputs unless a function says otherwise.
 *  - Return value: VAE_OK (0) or a negative VAE_ERR_* code.  On error nothing
 *    has been enqueued, except for VAE_ERR_HIP, which reports a failed
 *    launch.  vae_last_error() then returns a message (per calling thread).
 *  - Every size is validated before any launch: non-positive sizes, NULL
 *    required pointers, a workspace that is too small, and shapes the
 *    kernels do not support are reported, never run.
 */
#ifndef VAE_H_
#define VAE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VAE_ABI_VERSION 11

#define VAE_OK 0
#define VAE_ERR_INVALID_ARG (-1) /* NULL pointer, non-positive size, mismatched channels */
#define VAE_ERR_UNSUPPORTED (-2) /* a shape the kernels do not handle (e.g. C % 32 != 0) */
#define VAE_ERR_WORKSPACE (-3)   /* workspace smaller than the matching *_workspace_bytes */
#define VAE_ERR_HIP (-4)         /* a HIP launch or runtime call failed */

/* One convolution: weight [out_channels, in_channels, k, k] row-major
 * (k x k x k for the 3-D conv), bias [out_channels]; stride 1, zero padding
 * k/2 (cortiq-engine 0.7.7 `vae`, structs Conv2d and VaeConvRef).  A conv
 * with weight == NULL is "absent" where the struct is optional. */
typedef struct vae_conv {
    const float *weight;
    const float *bias;
    int32_t out_channels;
    int32_t in_channels;
    int32_t kernel; /* 1 or 3 */
} vae_conv;

/* GroupNorm(32 groups, eps 1e-6) affine parameters gamma[c], beta[c]
 * (cortiq-engine 0.7.7 `vae`, structs GroupNorm and VaeNormRef). */
typedef struct vae_norm {
    const float *gamma;
    const float *beta;
    int32_t channels;
} vae_norm;

/* x + conv2(silu(norm2(conv1(silu(norm1(x)))))), the skip going through the
 * 1x1 `shortcut` when the block changes the channel count (VaeResnetRef).
 * shortcut.weight == NULL means the identity skip. */
typedef struct vae_resnet {
    vae_norm norm1;
    vae_conv conv1;
    vae_norm norm2;
    vae_conv conv2;
    vae_conv shortcut;
} vae_resnet;

/* Mid-block single-head spatial attention (VaeAttnRef): GroupNorm, then
 * token-major Linear q, k, v ([c, c] row-major out x in, + bias, given as
 * kernel-1 convs), softmax(q k^T / sqrt(c)) v, Linear `out` + bias, residual
 * add onto the block input. */
typedef struct vae_attn {
    vae_norm norm;
    vae_conv q, k, v, out;
} vae_attn;

/* One up block (VaeUpRef): its resnets in order, then, if upsample.weight is
 * not NULL, nearest x2 upsampling followed by the 3x3 `upsample` conv. */
typedef struct vae_up {
    int32_t n_resnets;
    const vae_resnet *resnets;
    vae_conv upsample;
} vae_up;

/* The whole decoder in execution order (VaeChainArgs): conv_in -> mid_res0 ->
 * mid_attn -> mid_res1 -> ups[0..n_up) -> norm_out + SiLU -> conv_out, with
 * the latent de-normalised first as z / scaling_factor + shift_factor
 * (VaeDecoder). */
typedef struct vae_weights {
    vae_conv conv_in;
    vae_resnet mid_res0;
    vae_attn mid_attn;
    vae_resnet mid_res1;
    int32_t n_up;
    const vae_up *ups;
    vae_norm norm_out;
    vae_conv conv_out;
    float scaling_factor;
    float shift_factor;
} vae_weights;

/* Message of the last failing call on this thread ("" if none). */
const char *vae_last_error(void);
int32_t vae_abi_version(void);

/* The form of the 3x3 convolutions (every 3x3 conv but conv_in, which always
 * runs as an implicit GEMM that de-normalises the latent while loading it):
 *   VAE_CONV3X3_WINOGRAD_4X4   (default) Winograd F(4x4, 3x3) on FP32 MFMA:
 *                              36 of the direct conv's 144 multiplies per 4x4
 *                              outputs and input channel (25 on a nearest-x2
 *                              input), results within about 1e-5 of the
 *                              output's magnitude of the exact conv;
 *   VAE_CONV3X3_WINOGRAD_2X2   Winograd F(2x2, 3x3) on FP32 MFMA for every
 *                              conv: 16 of 36 multiplies per 2x2 outputs and
 *                              input channel (9 on a nearest-x2 input); about
 *                              1e-6;
 *   VAE_CONV3X3_IMPLICIT_GEMM  the direct conv as an implicit GEMM (all 36;
 *                              about 2e-7).
 * All stay within the decoder's per-layer bound of 1e-4 (normwise).  The
 * setting is process-wide and read when weights are packed: by
 * vae_decoder_create / vae_decoder3d_create (a decoder keeps the form it was
 * created with) and by each per-layer call.  GroupNorm applied on load
 * (vae_decoder_set_groupnorm_fusion) needs a decoder created with the F(2x2)
 * form or the implicit GEMM.  VAE_ERR_INVALID_ARG for other values. */
#define VAE_CONV3X3_WINOGRAD_2X2 0
#define VAE_CONV3X3_IMPLICIT_GEMM 1
#define VAE_CONV3X3_WINOGRAD_4X4 2
int32_t vae_set_conv3x3_algorithm(int32_t algorithm);
int32_t vae_get_conv3x3_algorithm(void);

/* ---------------------------------------------------------------- layers */

/* Workspace (device bytes) needed by vae_conv2d / vae_conv_in for `conv` on an
 * input of h x w (upsampled to 2h x 2w when upsample2x): the weights repacked
 * for the kernel and, for shapes too small to fill the GPU, the partial sums
 * of a split along K (input channels x taps).  Kernel-1 convs and convs with
 * at most 4 outputs need only the partial sums (0 for large images). */
int32_t vae_conv2d_workspace_bytes(const vae_conv *conv, int32_t h, int32_t w, int32_t upsample2x,
                                   size_t *bytes);

/* 2-D convolution (Conv2d / VaeConvRef): y = conv(u) + bias [+ residual].
 *   x        [cin, h, w]
 *   u        = x, or its nearest-x2 upsample [cin, 2h, 2w] when upsample2x
 *              (VaeUpRef; the upsampled tensor is never formed in memory)
 *   y        [cout, H, W] with (H, W) = (h, w), or (2h, 2w) when upsample2x
 *   residual NULL or [cout, H, W], added after the bias (the resnet skip)
 *   conv     kernel 1 or 3; conv->in_channels must equal cin
 *   ws       >= vae_conv2d_workspace_bytes(conv, h, w, upsample2x) device bytes (may be NULL if 0)
 * A convolution with out_channels <= 4 (the decoder's conv_out) runs on a
 * direct kernel; other 3x3 convolutions run in the form set by
 * vae_set_conv3x3_algorithm, on FP32 MFMA.
 * upsample2x requires kernel 3.  y may not alias x; it may alias residual. */
int32_t vae_conv2d(const float *x, int32_t cin, int32_t h, int32_t w, const vae_conv *conv,
                   int32_t upsample2x, const float *residual, float *y,
                   void *ws, size_t ws_bytes, void *stream);

/* conv_in with the latent de-normalisation folded into its input gather
 * (VaeDecoder): y = conv(z / scaling_factor + shift_factor) + bias, where
 * the zero padding stays zero.  z [cin, h, w], y [cout, h, w], kernel 3. */
int32_t vae_conv_in(const float *z, int32_t cin, int32_t h, int32_t w, const vae_conv *conv,
                    float scaling_factor, float shift_factor, float *y,
                    void *ws, size_t ws_bytes, void *stream);

/* Workspace for vae_groupnorm_silu on x [c, spatial]: per-group partial sums. */
int32_t vae_groupnorm_workspace_bytes(int32_t c, int64_t spatial, size_t *bytes);

/* GroupNorm(32, eps 1e-6, affine) (GroupNorm / VaeNormRef) over x [c, spatial]
 * (spatial = h*w, or t*h*w for the 3-D stack), then SiLU v/(1+exp(-v)) if
 * apply_silu, then + residual [c, spatial] if residual != NULL.
 * Statistics: the group mean and biased variance, accumulated in float64.
 * c % 32 == 0.  y may alias x (in place) and/or residual. */
int32_t vae_groupnorm_silu(const float *x, int32_t c, int64_t spatial, const vae_norm *norm,
                           int32_t apply_silu, const float *residual, float *y,
                           void *ws, size_t ws_bytes, void *stream);

/* vae_groupnorm_silu without a workspace argument, for callers that cannot
 * allocate memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, kernels and results as
 * vae_groupnorm_silu; its partial sums live in a static device buffer of the
 * library (36 KiB per GPU, held until the process ends; every GroupNorm
 * needs at most 33,280 bytes of it, and a larger need is refused with
 * VAE_ERR_UNSUPPORTED).  The buffer is looked up on the first call on each
 * device (the current device) and shared by every later call on that GPU:
 * calls that overlap in time on one GPU race on it, so callers serialise
 * them (one stream, or events).  Nothing is allocated, by the library or
 * through torch. */
int32_t vae_groupnorm_silu_noalloc(const float *x, int32_t c, int64_t spatial, const vae_norm *norm,
                                   int32_t apply_silu, const float *residual, float *y, void *stream);

/* Workspace for vae_conv2d_groupnorm_silu (same arguments as
 * vae_conv2d_workspace_bytes; kernel 3, out_channels % 32 == 0). */
int32_t vae_conv2d_groupnorm_workspace_bytes(const vae_conv *conv, int32_t h, int32_t w, int32_t upsample2x,
                                             size_t *bytes);

/* A 3x3 convolution followed by GroupNorm(32) (+ SiLU) of its output: the
 * conv -> norm pairs of VaeResnetRef (conv1 -> norm2, and conv2 -> the next
 * resnet's norm1).
 *   y = conv(u) + bias [+ residual]      exactly as vae_conv2d (kernel 3)
 *   z = GroupNorm(y), then SiLU if apply_silu, as vae_groupnorm_silu
 * The conv's epilogue records per-group statistics of the tiles it writes
 * (count, mean, sum of squared deviations), so the normalisation needs no
 * separate statistics pass over y.  norm->channels == conv->out_channels,
 * a multiple of 32.  y may not alias x; y may alias residual; z may alias
 * any argument (it is written last). */
int32_t vae_conv2d_groupnorm_silu(const float *x, int32_t cin, int32_t h, int32_t w, const vae_conv *conv,
                                  int32_t upsample2x, const float *residual, const vae_norm *norm,
                                  int32_t apply_silu, float *y, float *z, void *ws, size_t ws_bytes,
                                  void *stream);

/* Nearest x2 upsample (VaeUpRef): y[c, Y, X] = x[c, Y/2, X/2];
 * x [c, h, w] -> y [c, 2h, 2w].  Exact copy. */
int32_t vae_upsample_nearest2x(const float *x, int32_t c, int32_t h, int32_t w, float *y,
                               void *stream);

/* Workspace for vae_attention on x [c, h, w]: the normalised input, q/k/v,
 * the [h*w, h*w] score matrix and the attention output. */
int32_t vae_attention_workspace_bytes(int32_t c, int32_t h, int32_t w, size_t *bytes);

/* Mid-block attention (VaeAttnRef) on x [c, h, w] -> y [c, h, w]; tokens are
 * the h*w positions in row-major order.  c % 32 == 0; q, k, v, out are
 * kernel-1 convs with c in and c out channels.  y may not alias x. */
int32_t vae_attention(const float *x, int32_t c, int32_t h, int32_t w, const vae_attn *attn,
                      float *y, void *ws, size_t ws_bytes, void *stream);

/* The same attention with a streaming softmax (VaeAttnRef; the online softmax
 * of Milakov and Gimelshein, 2018): the scores of a query stay in the
 * registers of the wave that computes them, so the [h*w, h*w] score matrix is
 * never formed in memory, and the workspace holds only the normalised input,
 * q, v, k (token-major), the attention output and, when the keys are split
 * into ranges to fill the GPU, per-range partial outputs.  Same arguments and
 * results (up to rounding) as vae_attention; c must be 128, 256 or 512
 * (VAE_ERR_UNSUPPORTED otherwise).  The key bias is not applied: it adds one
 * constant to all scores of a query, which the softmax removes exactly. */
int32_t vae_attention_streaming_workspace_bytes(int32_t c, int32_t h, int32_t w, size_t *bytes);
int32_t vae_attention_streaming(const float *x, int32_t c, int32_t h, int32_t w, const vae_attn *attn,
                                float *y, void *ws, size_t ws_bytes, void *stream);

/* Workspace for vae_conv3d_causal on [cin, t, h, w]: the repacked 3x3x3
 * weights (and split-K partial sums for small shapes). */
int32_t vae_conv3d_causal_workspace_bytes(const vae_conv *conv, int32_t t, int32_t h, int32_t w,
                                          size_t *bytes);

/* Causal 3-D convolution (VAE decode -> GPU handoff, "The CPU VAE code" and
 * "GPU plan": LTX's 3-D causal conv with causal padding on time):
 * x [cin, t, h, w] -> y [cout, t, h, w]; weight [cout, cin, 3, 3, 3];
 * time padded at the front with two copies of frame 0, h and w zero-padded
 * by 1; stride 1.  y may not alias x. */
int32_t vae_conv3d_causal(const float *x, int32_t cin, int32_t t, int32_t h, int32_t w,
                          const vae_conv *conv, float *y, void *ws, size_t ws_bytes,
                          void *stream);

/* The causal 3-D conv followed by GroupNorm(32) (+ SiLU) of its output and an
 * optional residual added after it: one layer of the LTX-style causal stack
 * (VAE decode -> GPU handoff, "The CPU VAE code").
 *   y = conv3d_causal(x)                                as vae_conv3d_causal
 *   z = SiLU?(GroupNorm(y)) [+ residual]                statistics over
 *       (C/32) x t x h x w, taken from the conv's epilogue records, so the
 *       normalisation needs no separate statistics pass over y
 * norm->channels == conv->out_channels, a multiple of 32.  y may not alias x
 * or the residual; z may alias y (it is written last) or the residual. */
int32_t vae_conv3d_causal_groupnorm_workspace_bytes(const vae_conv *conv, int32_t t, int32_t h, int32_t w,
                                                    size_t *bytes);
int32_t vae_conv3d_causal_groupnorm_silu(const float *x, int32_t cin, int32_t t, int32_t h, int32_t w,
                                         const vae_conv *conv, const vae_norm *norm, int32_t apply_silu,
                                         const float *residual, float *y, float *z, void *ws, size_t ws_bytes,
                                         void *stream);

/* --------------------------------------------------------------- decoder */

typedef struct vae_decoder vae_decoder; /* opaque; created and freed by the library */

/* Device bytes of the decoder's own weight copy ("pack") for `w`. */
int32_t vae_decoder_pack_bytes(const vae_weights *w, size_t *bytes);

/* Validates the chain, then copies and repacks every weight of `w` into the
 * caller's device buffer `pack` (>= vae_decoder_pack_bytes) on `stream`.
 * The decoder keeps using `pack` (which the caller must keep alive until
 * vae_decoder_destroy); the arrays `w` points to may be freed once the
 * enqueued copies have run.  This is the weight cache keyed by the decoder
 * handle (VaeChainArgs: a key stable for the life of the decoder). */
int32_t vae_decoder_create(vae_decoder **out, const vae_weights *w, void *pack, size_t pack_bytes,
                           void *stream);

/* Workspace for one vae_decode of a [latent_channels, h, w] latent. */
int32_t vae_decoder_workspace_bytes(const vae_decoder *d, int32_t h, int32_t w, size_t *bytes);

/* latent [latent_channels, h, w] -> rgb [out_channels, 8h, 8w] (for four up
 * blocks), raw conv_out values.  Every activation stays in `ws`; only the
 * caller's rgb buffer is written.  Calls on one decoder must not overlap in
 * time on different streams (they share the handle's profiling state). */
int32_t vae_decode(vae_decoder *d, const float *latent, int32_t h, int32_t w, float *rgb,
                   void *ws, size_t ws_bytes, void *stream);

/* The causal 3-D decoder (VAE decode -> GPU handoff, "The CPU VAE code": the
 * LTX decoder is a 3-D causal conv decode, causal padding on time).  The same
 * chain and the same vae_weights layout, read as a video decoder: every
 * kernel-3 conv holds [cout, cin, 3, 3, 3] weights and runs as a causal
 * 3x3x3 conv (time front-padded with two copies of frame 0, h and w
 * zero-padded), kernel-1 convs are 1x1x1 ([cout, cin]); GroupNorm statistics
 * span (C/32) x T x H x W; the mid attention runs over all t*h*w positions
 * (row-major over t, y, x); upsampling doubles h and w only.  The handle is
 * used with vae_decoder3d_workspace_bytes / vae_decode3d (the 2-D calls
 * reject it and vice versa); destroy, output shape, GroupNorm mode and
 * profiling calls are shared. */
int32_t vae_decoder3d_pack_bytes(const vae_weights *w, size_t *bytes);
int32_t vae_decoder3d_create(vae_decoder **out, const vae_weights *w, void *pack, size_t pack_bytes,
                             void *stream);
int32_t vae_decoder3d_workspace_bytes(const vae_decoder *d, int32_t t, int32_t h, int32_t w, size_t *bytes);
/* latent [latent_channels, t, h, w] -> rgb [out_channels, t, 8h, 8w]. */
int32_t vae_decode3d(vae_decoder *d, const float *latent, int32_t t, int32_t h, int32_t w, float *rgb,
                     void *ws, size_t ws_bytes, void *stream);

/* Tiled decode: the tiling of the video VAE in cortiq-engine 0.8.78
 * `vae3d.rs` (constants TILE = 256 and TILE_OVERLAP_MIN = 64, split_tiles,
 * VideoVae::decode_clip, blend) applied to this 2-D decoder, for outputs whose
 * whole-image workspace is too large.  Along each axis of the [8h, 8w] output
 * the tiles are `tile` pixels long (one tile if the axis is no longer); their
 * count is the fewest that cover the axis with neighbours overlapping by
 * `overlap` pixels, and the length left over widens the overlaps one latent
 * cell (8 pixels) at a time, from the first overlap on, cycling.  Each tile's
 * latent block is decoded on its own (vae_decode, graph mode and attention
 * form as set on `d`); tile (i, j) then cross-fades its first rows into the
 * last rows of the decoded tile above, weight k/e for row k of an overlap of
 * e rows, and its first columns likewise into the decoded tile to its left,
 * and keeps the part before the next tiles start (the last tile of a row or
 * column keeps the rest), so each output pixel is written once.
 *   latent [latent_channels, h, w], rgb [out_channels, 8h, 8w] (device);
 *   tile, overlap  pixels, multiples of 8, 0 <= overlap < tile (the pages:
 *                  256 and 64); at most 64 tiles per axis;
 *   ws   >= vae_decoder_tiled_workspace_bytes(...) device bytes: every
 *        decoded tile (ny x nx x out_channels x tile x tile floats), a staging
 *        tile, and for each of three concurrent tile decodes a latent block and
 *        a decode workspace; owned by the caller.
 * With graph mode and profiling off and `stream` not being captured, the tiles
 * decode three at a time on streams the handle creates on first use (default
 * priority, destroyed with the handle), forked from and joined back to
 * `stream` by events, so the call is ordered on `stream` like any other; else
 * one after another on `stream`.  Calls on one handle from several host
 * threads at once race.
 * A 2-D decoder only.  VAE_ERR_INVALID_ARG for bad sizes, VAE_ERR_UNSUPPORTED
 * beyond 64 tiles per axis, VAE_ERR_WORKSPACE for a short workspace, all
 * before any launch.  A single tile (tile >= 8h and 8w) gives vae_decode's
 * result exactly. */
int32_t vae_decoder_tiled_workspace_bytes(const vae_decoder *d, int32_t h, int32_t w, int32_t tile, int32_t overlap,
                                          size_t *bytes);
int32_t vae_decode_tiled(vae_decoder *d, const float *latent, int32_t h, int32_t w, int32_t tile, int32_t overlap,
                         float *rgb, void *ws, size_t ws_bytes, void *stream);

/* Output spatial scale of the chain (8 for four up blocks) and its channels. */
int32_t vae_decoder_output_shape(const vae_decoder *d, int32_t h, int32_t w, int32_t *c,
                                 int32_t *ho, int32_t *wo);

void vae_decoder_destroy(vae_decoder *d);

/* on != 0: apply each conv input's GroupNorm + SiLU while the conv loads it,
 * from per-channel coefficients computed by a statistics-only pass, instead
 * of a separate normalisation pass that writes the normalised tensor (the
 * default).  Same results up to rounding.  On MI355X the separate pass is
 * faster, so the default is off.  VAE_ERR_UNSUPPORTED if a normalised conv
 * has more than 512 input channels, or if the decoder's 3x3 convs were
 * packed in the F(4x4) Winograd form (VAE_CONV3X3_WINOGRAD_4X4). */
int32_t vae_decoder_set_groupnorm_fusion(vae_decoder *d, int32_t on);

/* The form of the decoder's mid-block attention:
 *   VAE_ATTENTION_SPLIT_SOFTMAX  the score matrix in the workspace, the softmax
 *                                split across the two products around it
 *                                (vae_attention);
 *   VAE_ATTENTION_STREAMING      streaming softmax, no score matrix
 *                                (vae_attention_streaming; 128, 256 or 512
 *                                channels, else VAE_ERR_UNSUPPORTED).
 * The decode workspace follows the form set when it is sized.
 * VAE_ERR_INVALID_ARG for other values. */
#define VAE_ATTENTION_SPLIT_SOFTMAX 0
#define VAE_ATTENTION_STREAMING 1
int32_t vae_decoder_set_attention(vae_decoder *d, int32_t form);
int32_t vae_decoder_get_attention(const vae_decoder *d);

/* on != 0: vae_decode / vae_decode3d capture their launch sequence into a HIP
 * graph on the first call with a given (latent, rgb, workspace, sizes,
 * stream, GroupNorm mode) and replay the graph on later calls with the same
 * arguments; other arguments capture a new graph (one is cached).  The
 * graph reads the buffers when it runs, so new contents in the same buffers
 * are decoded; the caller keeps them allocated while the graph is cached (or
 * turns graphs off, which frees it).  Plain launches are used while
 * profiling, on the null stream, and while the caller captures the stream
 * itself.  Off by default. */
int32_t vae_decoder_set_graph(vae_decoder *d, int32_t on);

/* ------------------------------------------------------------- profiling */

/* One kernel launch (or one composite layer: GroupNorm = stats + apply,
 * attention = its GEMMs and softmax) of a profiled vae_decode. */
typedef struct vae_prof_record {
    char kernel[40];   /* kernel class, e.g. "conv3x3_mfma" */
    char layer[72];    /* decoder layer, e.g. "up_blocks.3.resnets.1.conv2" */
    float ms;          /* launch duration from HIP events on the decode stream */
    double flops;      /* algorithmic FLOPs of the launch (direct-conv count) */
    double bytes;      /* algorithmic HBM bytes of the launch (one read of each input, one write) */
} vae_prof_record;

/* Clears the recorded launches.  on != 0: the following vae_decode calls
 * bracket every launch with HIP events on their stream and append one
 * record per launch (events are created on first use; a failure to create
 * one is reported as VAE_ERR_HIP by vae_decode).  The events only time: they
 * are recorded without a system-scope memory fence, so they order nothing for
 * the host; synchronise the stream before reading the decode's output. */
int32_t vae_decoder_set_profiling(vae_decoder *d, int32_t on);

/* Synchronises on the recorded events and copies up to `max` records
 * (oldest first) into `out`; *n receives the number recorded since the last
 * vae_decoder_set_profiling call. */
int32_t vae_decoder_profile(vae_decoder *d, vae_prof_record *out, int32_t max, int32_t *n);

/* ------------------------------------------------------------ measurement */

/* Measurement only, no step of the decode: probes of known work that
 * measure the GPU's own ceilings, so the kernels above (the convs bound by
 * the FP32 matrix units, the normalisation and upsample by HBM) can be read
 * against measured peaks beside the published ones.  They only enqueue on
 * `stream`; the caller times them with events there.
 *
 * vae_probe_mfma_f32: `blocks` workgroups of 256 threads, each wave running
 * `iters` rounds of 8 independent v_mfma_f32_32x32x2_f32 on register
 * operands; *flops receives the launch's FLOPs (blocks x 4 waves x iters x 8
 * x 4096).  Lane l of every wave feeds a(l) = 1 + l/64 as the A operand
 * (A[l % 32][l / 32]) and b(l) = 1 - l/128 as the B operand (B[l / 32][l % 32]),
 * and each thread writes the sum of its accumulators to out[block * 256 +
 * thread], so a wave's 64 outputs sum to 8 x iters x sum_k A_k B_k with A_k =
 * sum_m a(m + 32k), B_k = sum_n b(n + 32k), up to float32 rounding.
 *   out  >= blocks x 256 floats (device); 1 <= blocks <= 65535,
 *        1 <= iters <= 2^20.
 * vae_probe_hbm: y == NULL: reads x [n] once and writes each thread's sum of
 * what it read to out (>= blocks x 256 floats; the outputs sum to sum(x) up
 * to rounding); y != NULL: copies x to y (out unused).  n a positive multiple
 * of 4, x and y 16-byte aligned, 1 <= blocks <= 65535; workgroups of 256
 * threads stream contiguous 16 KB chunks, grid-stride over the chunks, four
 * 16-byte loads in flight per thread.
 * Both return VAE_ERR_INVALID_ARG for bad arguments, before any launch. */
int32_t vae_probe_mfma_f32(int32_t blocks, int32_t iters, float *out, size_t out_floats, double *flops,
                           void *stream);
int32_t vae_probe_hbm(const float *x, size_t n, float *y, int32_t blocks, float *out, size_t out_floats,
                      void *stream);

#ifdef __cplusplus
}
#endif

#endif /* VAE_H_ */
