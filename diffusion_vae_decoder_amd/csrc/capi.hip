// C ABI of libvae.so: per-layer entry points and error reporting.  Every
// entry point validates its arguments completely before enqueuing anything.

#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cstring>

#include "vae_internal.h"

namespace vae {

namespace {
thread_local char g_err[512] = "";
}

void set_error(const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
}

int32_t hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return VAE_OK;
    set_error("%s: %s", what, hipGetErrorString(e));
    return VAE_ERR_HIP;
}

int32_t check_launch(const char *what) { return hip_status(hipGetLastError(), what); }

int32_t check_groupnorm_args(const char *who, const float *x, int c, long long spatial, const vae_norm *norm,
                             const float *y) {
    if (!x || !y || !norm || !norm->gamma || !norm->beta) {
        set_error("%s: NULL pointer", who);
        return VAE_ERR_INVALID_ARG;
    }
    if (c <= 0 || spatial <= 0) {
        set_error("%s: sizes must be positive", who);
        return VAE_ERR_INVALID_ARG;
    }
    if (norm->channels != c) {
        set_error("%s: norm has %d channels, tensor %d", who, norm->channels, c);
        return VAE_ERR_INVALID_ARG;
    }
    if (c % 32) {
        set_error("%s: channels %d not divisible by 32", who, c);
        return VAE_ERR_UNSUPPORTED;
    }
    if ((long long)c * spatial > (1LL << 34)) {
        set_error("%s: tensor too large", who);
        return VAE_ERR_UNSUPPORTED;
    }
    return VAE_OK;
}

}  // namespace vae

using namespace vae;

namespace {

constexpr long long kMaxElems = 1LL << 34;   // per tensor; offsets inside kernels are 64-bit
constexpr long long kMaxPlane = 1LL << 30;   // h*w per plane; plane offsets are 32-bit

int32_t bad(const char *fmt, ...) {
    char buf[400];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    set_error("%s", buf);
    return VAE_ERR_INVALID_ARG;
}

int32_t unsupported(const char *fmt, ...) {
    char buf[400];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    set_error("%s", buf);
    return VAE_ERR_UNSUPPORTED;
}

int32_t check_conv(const char *who, const vae_conv *c, int kernel_required /* 0 = 1 or 3 */) {
    if (!c) return bad("%s: conv is NULL", who);
    if (!c->weight || !c->bias) return bad("%s: conv weight/bias is NULL", who);
    if (c->out_channels <= 0 || c->in_channels <= 0)
        return bad("%s: conv channels must be positive (out %d, in %d)", who, c->out_channels, c->in_channels);
    if (kernel_required ? c->kernel != kernel_required : (c->kernel != 1 && c->kernel != 3))
        return unsupported("%s: unsupported kernel size %d", who, c->kernel);
    return VAE_OK;
}

int32_t check_plane(const char *who, long long c, long long h, long long w) {
    if (c <= 0 || h <= 0 || w <= 0) return bad("%s: sizes must be positive (c %lld, h %lld, w %lld)", who, c, h, w);
    if (h * w > kMaxPlane || c * h * w > kMaxElems)
        return unsupported("%s: tensor [%lld, %lld, %lld] too large", who, c, h, w);
    return VAE_OK;
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// Workspace of a 3x3 conv producing [cout, T, H, W]: the repacked weights (room
// for any layout), then the split-K partial sums (if the shape is split).
// Split-K partial sums of the conv in the weight layout it runs with; the
// workspace sizes below take the larger of the two layouts, so one size
// serves vae_conv2d and vae_conv_in alike.
size_t conv_partial_floats(const vae_conv *c, int kt, int T, int H, int W, int layout) {
    ConvLaunch a{};
    a.cin = c->in_channels; a.cout = c->out_channels; a.H = H; a.W = W; a.T = T; a.kt = kt; a.wino = layout;
    return conv3x3_partial_floats(a);
}

size_t conv_ws(const vae_conv *c, int kt, int T, int H, int W) {
    if (c->kernel == 1) return gemm_partial_floats(c->out_channels, H * W, c->in_channels, false) * sizeof(float);
    const size_t part = std::max({conv_partial_floats(c, kt, T, H, W, 0), conv_partial_floats(c, kt, T, H, W, 1),
                                  conv_partial_floats(c, kt, T, H, W, 3)});
    const size_t packed = align256(conv3x3_pack_floats_max(c->out_channels, c->in_channels, kt) * sizeof(float)) +
                          part * sizeof(float);
    if (kt == 1 && c->out_channels <= 4)   // direct kernel (or, with upsample / residual, the packed path)
        return std::max(conv3x3_direct_partial_floats(c->out_channels, c->in_channels, 1, H, W, 1) * sizeof(float),
                        packed);
    return packed;
}

float *conv_ws_part(const vae_conv *c, int kt, void *ws) {
    return reinterpret_cast<float *>(static_cast<char *>(ws) +
                                     align256(conv3x3_pack_floats_max(c->out_channels, c->in_channels, kt) * sizeof(float)));
}

}  // namespace

extern "C" {

const char *vae_last_error(void) { return g_err; }

int32_t vae_abi_version(void) { return VAE_ABI_VERSION; }

int32_t vae_set_conv3x3_algorithm(int32_t algorithm) { return set_conv3x3_algorithm(algorithm); }

int32_t vae_get_conv3x3_algorithm(void) { return get_conv3x3_algorithm(); }

int32_t vae_conv2d_workspace_bytes(const vae_conv *conv, int32_t h, int32_t w, int32_t upsample2x,
                                   size_t *bytes) {
    int32_t rc = check_conv("vae_conv2d_workspace_bytes", conv, 0);
    if (rc) return rc;
    if (!bytes) return bad("vae_conv2d_workspace_bytes: bytes is NULL");
    if ((rc = check_plane("vae_conv2d_workspace_bytes", conv->out_channels, upsample2x ? 2LL * h : h,
                          upsample2x ? 2LL * w : w))) return rc;
    *bytes = conv_ws(conv, 1, 1, upsample2x ? 2 * h : h, upsample2x ? 2 * w : w);
    return VAE_OK;
}

int32_t vae_conv2d(const float *x, int32_t cin, int32_t h, int32_t w, const vae_conv *conv,
                   int32_t upsample2x, const float *residual, float *y, void *ws, size_t ws_bytes,
                   void *stream) {
    int32_t rc = check_conv("vae_conv2d", conv, 0);
    if (rc) return rc;
    if (!x || !y) return bad("vae_conv2d: x or y is NULL");
    const int H = upsample2x ? 2 * h : h, W = upsample2x ? 2 * w : w;
    if ((rc = check_plane("vae_conv2d", cin, h, w))) return rc;
    if ((rc = check_plane("vae_conv2d", conv->out_channels, H, W))) return rc;
    if (conv->in_channels != cin)
        return bad("vae_conv2d: conv expects %d input channels, got %d", conv->in_channels, cin);
    if (x == y) return bad("vae_conv2d: y may not alias x");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (conv->kernel == 1) {
        if (upsample2x) return unsupported("vae_conv2d: upsample2x needs a 3x3 conv");
        GemmLaunch g{};
        g.A = conv->weight; g.lda = cin; g.a_km = 0;
        g.B = x; g.ldb = (long long)h * w; g.b_nk = 0;
        g.bias = conv->bias; g.R = residual; g.ldr = (long long)h * w;
        g.C = y; g.ldc = (long long)h * w;
        g.M = conv->out_channels; g.N = h * w; g.K = cin; g.alpha = 1.f;
        const size_t need = conv_ws(conv, 1, 1, h, w);
        if (need && (!ws || ws_bytes < need))
            return set_error("vae_conv2d: workspace %zu bytes < %zu", ws_bytes, need), VAE_ERR_WORKSPACE;
        g.part = static_cast<float *>(ws);
        return launch_gemm(g, s);
    }
    const size_t need = conv_ws(conv, 1, 1, H, W);
    if (conv->out_channels <= 4 && !upsample2x && !residual) {
        if (need && (!ws || ws_bytes < need))
            return set_error("vae_conv2d: workspace %zu bytes < %zu", ws_bytes, need), VAE_ERR_WORKSPACE;
        return launch_conv3x3_direct(x, conv->weight, conv->bias, y, cin, conv->out_channels, h, w, s, nullptr,
                                     static_cast<float *>(ws));
    }
    if (!ws || ws_bytes < need)
        return set_error("vae_conv2d: workspace %zu bytes < %zu", ws_bytes, need), VAE_ERR_WORKSPACE;
    ConvLaunch a{};
    a.wino = conv3x3_layout(0, upsample2x);
    if ((rc = pack_conv3x3_layout(a.wino, conv->weight, conv->out_channels, cin, 1, static_cast<float *>(ws), s)))
        return rc;
    a.x = x; a.wpk = static_cast<const float *>(ws); a.bias = conv->bias; a.res = residual; a.y = y;
    a.part = conv_ws_part(conv, 1, ws);
    a.cin = cin; a.cout = conv->out_channels; a.H = H; a.W = W; a.T = 1; a.kt = 1;
    a.upsample = upsample2x ? 1 : 0;
    return launch_conv3x3(a, s);
}

int32_t vae_conv_in(const float *z, int32_t cin, int32_t h, int32_t w, const vae_conv *conv,
                    float scaling_factor, float shift_factor, float *y, void *ws, size_t ws_bytes,
                    void *stream) {
    int32_t rc = check_conv("vae_conv_in", conv, 3);
    if (rc) return rc;
    if (!z || !y) return bad("vae_conv_in: z or y is NULL");
    if ((rc = check_plane("vae_conv_in", cin, h, w))) return rc;
    if ((rc = check_plane("vae_conv_in", conv->out_channels, h, w))) return rc;
    if (conv->in_channels != cin) return bad("vae_conv_in: conv expects %d input channels, got %d", conv->in_channels, cin);
    if (!(scaling_factor != 0.f)) return bad("vae_conv_in: scaling_factor must be non-zero");
    if (z == y) return bad("vae_conv_in: y may not alias z");
    const size_t need = conv_ws(conv, 1, 1, h, w);
    if (!ws || ws_bytes < need)
        return set_error("vae_conv_in: workspace %zu bytes < %zu", ws_bytes, need), VAE_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((rc = pack_conv3x3(conv->weight, conv->out_channels, cin, 1, static_cast<float *>(ws), s))) return rc;
    ConvLaunch a{};
    a.x = z; a.wpk = static_cast<const float *>(ws); a.bias = conv->bias; a.y = y;
    a.part = conv_ws_part(conv, 1, ws);
    a.cin = cin; a.cout = conv->out_channels; a.H = h; a.W = w; a.T = 1; a.kt = 1;
    a.denorm = 1; a.dn_scale = scaling_factor; a.dn_shift = shift_factor;
    return launch_conv3x3(a, s);
}

int32_t vae_groupnorm_workspace_bytes(int32_t c, int64_t spatial, size_t *bytes) {
    if (!bytes) return bad("vae_groupnorm_workspace_bytes: bytes is NULL");
    if (c <= 0 || spatial <= 0) return bad("vae_groupnorm_workspace_bytes: sizes must be positive");
    if (c % 32) return unsupported("vae_groupnorm_workspace_bytes: channels %d not divisible by 32", c);
    *bytes = groupnorm_ws_bytes(c, spatial);
    return VAE_OK;
}

int32_t vae_groupnorm_silu(const float *x, int32_t c, int64_t spatial, const vae_norm *norm,
                           int32_t apply_silu, const float *residual, float *y, void *ws,
                           size_t ws_bytes, void *stream) {
    int32_t rc = check_groupnorm_args("vae_groupnorm_silu", x, c, spatial, norm, y);
    if (rc) return rc;
    const size_t need = groupnorm_ws_bytes(c, spatial);
    if (!ws || ws_bytes < need)
        return set_error("vae_groupnorm_silu: workspace %zu bytes < %zu", ws_bytes, need), VAE_ERR_WORKSPACE;
    return launch_groupnorm(x, c, spatial, norm->gamma, norm->beta, apply_silu ? 1 : 0, residual, y, ws,
                            static_cast<hipStream_t>(stream));
}

namespace {
// Workspace of vae_conv2d_groupnorm_silu: the conv's workspace, then the
// GroupNorm records of its output, then the GroupNorm partial sums.
size_t conv_gn_records_bytes(const vae_conv *c, int cin, int H, int W, int upsample, int T = 1, int kt = 1) {
    ConvLaunch a{};
    a.cin = cin; a.cout = c->out_channels; a.H = H; a.W = W; a.T = T; a.kt = kt;
    a.upsample = upsample;
    int n = 0;   // the most records any form writes, so the size holds whatever the setting
    for (int layout : {0, upsample ? 2 : 1, upsample ? 4 : 3}) {
        a.wino = layout;
        n = std::max(n, conv3x3_gn_records(a));
    }
    return (size_t)32 * n * sizeof(floatx4);
}
size_t conv_gn_ws(const vae_conv *c, int H, int W, int upsample, int T = 1, int kt = 1) {
    return align256(conv_ws(c, kt, T, H, W)) + align256(conv_gn_records_bytes(c, c->in_channels, H, W, upsample, T, kt)) +
           groupnorm_ws_bytes(c->out_channels, (long long)T * H * W);
}
}  // namespace

int32_t vae_conv2d_groupnorm_workspace_bytes(const vae_conv *conv, int32_t h, int32_t w, int32_t upsample2x,
                                             size_t *bytes) {
    int32_t rc = check_conv("vae_conv2d_groupnorm_workspace_bytes", conv, 3);
    if (rc) return rc;
    if (!bytes) return bad("vae_conv2d_groupnorm_workspace_bytes: bytes is NULL");
    const long long H = upsample2x ? 2LL * h : h, W = upsample2x ? 2LL * w : w;
    if ((rc = check_plane("vae_conv2d_groupnorm_workspace_bytes", conv->out_channels, H, W))) return rc;
    if (conv->out_channels % 32)
        return unsupported("vae_conv2d_groupnorm_workspace_bytes: out_channels %d not divisible by 32",
                           conv->out_channels);
    *bytes = conv_gn_ws(conv, (int)H, (int)W, upsample2x ? 1 : 0);
    return VAE_OK;
}

int32_t vae_conv2d_groupnorm_silu(const float *x, int32_t cin, int32_t h, int32_t w, const vae_conv *conv,
                                  int32_t upsample2x, const float *residual, const vae_norm *norm,
                                  int32_t apply_silu, float *y, float *z, void *ws, size_t ws_bytes,
                                  void *stream) {
    int32_t rc = check_conv("vae_conv2d_groupnorm_silu", conv, 3);
    if (rc) return rc;
    if (!x || !y || !z) return bad("vae_conv2d_groupnorm_silu: x, y or z is NULL");
    if (!norm || !norm->gamma || !norm->beta) return bad("vae_conv2d_groupnorm_silu: norm missing");
    const int H = upsample2x ? 2 * h : h, W = upsample2x ? 2 * w : w;
    if ((rc = check_plane("vae_conv2d_groupnorm_silu", cin, h, w))) return rc;
    if ((rc = check_plane("vae_conv2d_groupnorm_silu", conv->out_channels, H, W))) return rc;
    if (conv->in_channels != cin)
        return bad("vae_conv2d_groupnorm_silu: conv expects %d input channels, got %d", conv->in_channels, cin);
    if (norm->channels != conv->out_channels)
        return bad("vae_conv2d_groupnorm_silu: norm has %d channels, conv output %d", norm->channels,
                   conv->out_channels);
    if (conv->out_channels % 32)
        return unsupported("vae_conv2d_groupnorm_silu: out_channels %d not divisible by 32", conv->out_channels);
    if (x == y) return bad("vae_conv2d_groupnorm_silu: y may not alias x");
    const size_t need = conv_gn_ws(conv, H, W, upsample2x ? 1 : 0);
    if (!ws || ws_bytes < need)
        return set_error("vae_conv2d_groupnorm_silu: workspace %zu bytes < %zu", ws_bytes, need), VAE_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    char *base = static_cast<char *>(ws);
    ConvLaunch a{};
    a.wino = conv3x3_layout(0, upsample2x);
    if ((rc = pack_conv3x3_layout(a.wino, conv->weight, conv->out_channels, cin, 1, reinterpret_cast<float *>(base), s)))
        return rc;
    a.x = x; a.wpk = reinterpret_cast<const float *>(base); a.bias = conv->bias; a.res = residual; a.y = y;
    a.part = conv_ws_part(conv, 1, ws);
    a.cin = cin; a.cout = conv->out_channels; a.H = H; a.W = W; a.T = 1; a.kt = 1;
    a.upsample = upsample2x ? 1 : 0;
    char *recs = base + align256(conv_ws(conv, 1, 1, H, W));
    void *gws = recs + align256(conv_gn_records_bytes(conv, cin, H, W, upsample2x ? 1 : 0));
    const int nrec = conv3x3_gn_records(a);
    a.gn_rec = nrec > 0 ? reinterpret_cast<floatx4 *>(recs) : nullptr;
    if ((rc = launch_conv3x3(a, s))) return rc;
    return launch_groupnorm(y, conv->out_channels, (long long)H * W, norm->gamma, norm->beta, apply_silu ? 1 : 0,
                            nullptr, z, gws, s, a.gn_rec, nrec);
}

int32_t vae_conv3d_causal_groupnorm_workspace_bytes(const vae_conv *conv, int32_t t, int32_t h, int32_t w,
                                                    size_t *bytes) {
    const char *who = "vae_conv3d_causal_groupnorm_workspace_bytes";
    int32_t rc = check_conv(who, conv, 3);
    if (rc) return rc;
    if (!bytes) return bad("%s: bytes is NULL", who);
    if (t <= 0) return bad("%s: t must be positive", who);
    if (t > 65535) return unsupported("%s: t %d exceeds the grid limit", who, t);
    if ((rc = check_plane(who, (long long)conv->out_channels * t, h, w))) return rc;
    if (conv->out_channels % 32) return unsupported("%s: out_channels %d not divisible by 32", who, conv->out_channels);
    *bytes = conv_gn_ws(conv, h, w, 0, t, 3);
    return VAE_OK;
}

int32_t vae_conv3d_causal_groupnorm_silu(const float *x, int32_t cin, int32_t t, int32_t h, int32_t w,
                                         const vae_conv *conv, const vae_norm *norm, int32_t apply_silu,
                                         const float *residual, float *y, float *z, void *ws, size_t ws_bytes,
                                         void *stream) {
    const char *who = "vae_conv3d_causal_groupnorm_silu";
    int32_t rc = check_conv(who, conv, 3);
    if (rc) return rc;
    if (!x || !y || !z) return bad("%s: x, y or z is NULL", who);
    if (!norm || !norm->gamma || !norm->beta) return bad("%s: norm missing", who);
    if (t <= 0) return bad("%s: t must be positive", who);
    if (t > 65535) return unsupported("%s: t %d exceeds the grid limit", who, t);
    if ((rc = check_plane(who, (long long)cin * t, h, w))) return rc;
    if ((rc = check_plane(who, (long long)conv->out_channels * t, h, w))) return rc;
    if (conv->in_channels != cin) return bad("%s: conv expects %d input channels, got %d", who, conv->in_channels, cin);
    if (norm->channels != conv->out_channels)
        return bad("%s: norm has %d channels, conv output %d", who, norm->channels, conv->out_channels);
    if (conv->out_channels % 32) return unsupported("%s: out_channels %d not divisible by 32", who, conv->out_channels);
    if (x == y) return bad("%s: y may not alias x", who);
    if (residual == y) return bad("%s: the residual may not alias y", who);
    const size_t need = conv_gn_ws(conv, h, w, 0, t, 3);
    if (!ws || ws_bytes < need)
        return set_error("%s: workspace %zu bytes < %zu", who, ws_bytes, need), VAE_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    char *base = static_cast<char *>(ws);
    ConvLaunch a{};
    a.wino = conv3x3_layout(0, 0);
    if ((rc = pack_conv3x3_layout(a.wino, conv->weight, conv->out_channels, cin, 3, reinterpret_cast<float *>(base), s)))
        return rc;
    a.x = x; a.wpk = reinterpret_cast<const float *>(base); a.bias = conv->bias; a.y = y;
    a.part = conv_ws_part(conv, 3, ws);
    a.cin = cin; a.cout = conv->out_channels; a.H = h; a.W = w; a.T = t; a.kt = 3;
    char *recs = base + align256(conv_ws(conv, 3, t, h, w));
    void *gws = recs + align256(conv_gn_records_bytes(conv, cin, h, w, 0, t, 3));
    const int nrec = conv3x3_gn_records(a);
    a.gn_rec = nrec > 0 ? reinterpret_cast<floatx4 *>(recs) : nullptr;
    if ((rc = launch_conv3x3(a, s))) return rc;
    return launch_groupnorm(y, conv->out_channels, (long long)t * h * w, norm->gamma, norm->beta, apply_silu ? 1 : 0,
                            residual, z, gws, s, a.gn_rec, nrec);
}

int32_t vae_upsample_nearest2x(const float *x, int32_t c, int32_t h, int32_t w, float *y, void *stream) {
    if (!x || !y) return bad("vae_upsample_nearest2x: NULL pointer");
    int32_t rc = check_plane("vae_upsample_nearest2x", c, 2LL * h, 2LL * w);
    if (rc) return rc;
    if (x == y) return bad("vae_upsample_nearest2x: y may not alias x");
    return launch_upsample2x(x, c, h, w, y, static_cast<hipStream_t>(stream));
}

int32_t vae_attention_workspace_bytes(int32_t c, int32_t h, int32_t w, size_t *bytes) {
    if (!bytes) return bad("vae_attention_workspace_bytes: bytes is NULL");
    int32_t rc = check_plane("vae_attention_workspace_bytes", c, h, w);
    if (rc) return rc;
    if (c % 32) return unsupported("vae_attention_workspace_bytes: channels %d not divisible by 32", c);
    // plus room for the concatenated q/k/v weights and biases
    *bytes = attention_ws_bytes(c, (long long)h * w) + (((size_t)3 * c * c + 3 * c) * 4 + 512);
    return VAE_OK;
}

namespace {
// Checks shared by the two attention entry points; `streaming` adds the
// channel counts the streaming kernel supports.
int32_t check_attention(const char *who, const float *x, int32_t c, int32_t h, int32_t w, const vae_attn *attn,
                        const float *y, bool streaming) {
    if (!x || !y || !attn) return bad("%s: NULL pointer", who);
    int32_t rc = check_plane(who, c, h, w);
    if (rc) return rc;
    if ((long long)h * w > (1LL << 31) / 2) return unsupported("%s: too many tokens", who);
    if (c % 32) return unsupported("%s: channels %d not divisible by 32", who, c);
    if (streaming && !attention_flash_supported(c))
        return unsupported("%s: %d channels; the streaming form supports 128, 256 and 512", who, c);
    if (streaming && (long long)c * h * w * 4 >= (1LL << 31))
        return unsupported("%s: %d x %d tokens of %d channels exceed 2 GiB per operand", who, h, w, c);
    if (!attn->norm.gamma || !attn->norm.beta || attn->norm.channels != c)
        return bad("%s: norm missing or has %d channels (want %d)", who, attn->norm.channels, c);
    const vae_conv *lin[4] = {&attn->q, &attn->k, &attn->v, &attn->out};
    for (int i = 0; i < 4; ++i) {
        if ((rc = check_conv(who, lin[i], 1))) return rc;
        if (lin[i]->in_channels != c || lin[i]->out_channels != c)
            return bad("%s: projection %d is %dx%d, want %dx%d", who, i, lin[i]->out_channels, lin[i]->in_channels,
                       c, c);
    }
    if (x == y) return bad("%s: y may not alias x", who);
    return VAE_OK;
}

// q, k, v weights and biases concatenated at `dst` ([3c, c] then [3c]).
int32_t copy_qkv(const vae_attn *attn, int c, float *wqkv, hipStream_t s, const char *who) {
    float *bqkv = wqkv + (size_t)3 * c * c;
    const vae_conv *lin[3] = {&attn->q, &attn->k, &attn->v};
    const size_t cc = (size_t)c * c * 4;
    int32_t rc;
    for (int i = 0; i < 3; ++i) {
        if ((rc = hip_status(hipMemcpyAsync(wqkv + (size_t)i * c * c, lin[i]->weight, cc, hipMemcpyDeviceToDevice, s), who))) return rc;
        if ((rc = hip_status(hipMemcpyAsync(bqkv + (size_t)i * c, lin[i]->bias, (size_t)c * 4, hipMemcpyDeviceToDevice, s), who))) return rc;
    }
    return VAE_OK;
}
}  // namespace

int32_t vae_attention(const float *x, int32_t c, int32_t h, int32_t w, const vae_attn *attn, float *y,
                      void *ws, size_t ws_bytes, void *stream) {
    int32_t rc = check_attention("vae_attention", x, c, h, w, attn, y, false);
    if (rc) return rc;
    size_t need = 0;
    vae_attention_workspace_bytes(c, h, w, &need);
    if (!ws || ws_bytes < need)
        return set_error("vae_attention: workspace %zu bytes < %zu", ws_bytes, need), VAE_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    float *wqkv = reinterpret_cast<float *>(static_cast<char *>(ws) + attention_ws_bytes(c, (long long)h * w));
    if ((rc = copy_qkv(attn, c, wqkv, s, "vae_attention: copy"))) return rc;
    return launch_attention(x, c, h, w, attn->norm.gamma, attn->norm.beta, wqkv, wqkv + (size_t)3 * c * c,
                            attn->out.weight, attn->out.bias, y, ws, s);
}

int32_t vae_attention_streaming_workspace_bytes(int32_t c, int32_t h, int32_t w, size_t *bytes) {
    if (!bytes) return bad("vae_attention_streaming_workspace_bytes: bytes is NULL");
    int32_t rc = check_plane("vae_attention_streaming_workspace_bytes", c, h, w);
    if (rc) return rc;
    if (!attention_flash_supported(c))
        return unsupported("vae_attention_streaming_workspace_bytes: %d channels; supported: 128, 256, 512", c);
    *bytes = attention_streaming_ws_bytes(c, (long long)h * w) + (((size_t)3 * c * c + 3 * c) * 4 + 512);
    return VAE_OK;
}

int32_t vae_attention_streaming(const float *x, int32_t c, int32_t h, int32_t w, const vae_attn *attn, float *y,
                                void *ws, size_t ws_bytes, void *stream) {
    int32_t rc = check_attention("vae_attention_streaming", x, c, h, w, attn, y, true);
    if (rc) return rc;
    size_t need = 0;
    vae_attention_streaming_workspace_bytes(c, h, w, &need);
    if (!ws || ws_bytes < need)
        return set_error("vae_attention_streaming: workspace %zu bytes < %zu", ws_bytes, need), VAE_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    float *wqkv = reinterpret_cast<float *>(static_cast<char *>(ws) + attention_streaming_ws_bytes(c, (long long)h * w));
    if ((rc = copy_qkv(attn, c, wqkv, s, "vae_attention_streaming: copy"))) return rc;
    return launch_attention_streaming(x, c, h, w, attn->norm.gamma, attn->norm.beta, wqkv, wqkv + (size_t)3 * c * c,
                                      attn->out.weight, attn->out.bias, y, ws, s);
}

int32_t vae_conv3d_causal_workspace_bytes(const vae_conv *conv, int32_t t, int32_t h, int32_t w,
                                          size_t *bytes) {
    int32_t rc = check_conv("vae_conv3d_causal_workspace_bytes", conv, 3);
    if (rc) return rc;
    if (!bytes) return bad("vae_conv3d_causal_workspace_bytes: bytes is NULL");
    if (t <= 0) return bad("vae_conv3d_causal_workspace_bytes: t must be positive");
    if (t > 65535) return unsupported("vae_conv3d_causal_workspace_bytes: t %d exceeds the grid limit", t);
    if ((rc = check_plane("vae_conv3d_causal_workspace_bytes", (long long)conv->out_channels * t, h, w))) return rc;
    *bytes = conv_ws(conv, 3, t, h, w);
    return VAE_OK;
}

int32_t vae_conv3d_causal(const float *x, int32_t cin, int32_t t, int32_t h, int32_t w,
                          const vae_conv *conv, float *y, void *ws, size_t ws_bytes, void *stream) {
    int32_t rc = check_conv("vae_conv3d_causal", conv, 3);
    if (rc) return rc;
    if (!x || !y) return bad("vae_conv3d_causal: x or y is NULL");
    if (t <= 0) return bad("vae_conv3d_causal: t must be positive");
    if ((rc = check_plane("vae_conv3d_causal", (long long)cin * t, h, w))) return rc;
    if ((rc = check_plane("vae_conv3d_causal", (long long)conv->out_channels * t, h, w))) return rc;
    if (t > 65535) return unsupported("vae_conv3d_causal: t %d exceeds the grid limit", t);
    if (conv->in_channels != cin) return bad("vae_conv3d_causal: conv expects %d input channels, got %d", conv->in_channels, cin);
    if (x == y) return bad("vae_conv3d_causal: y may not alias x");
    const size_t need = conv_ws(conv, 3, t, h, w);
    if (!ws || ws_bytes < need)
        return set_error("vae_conv3d_causal: workspace %zu bytes < %zu", ws_bytes, need), VAE_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    ConvLaunch a{};
    a.wino = conv3x3_layout(0, 0);
    if ((rc = pack_conv3x3_layout(a.wino, conv->weight, conv->out_channels, cin, 3, static_cast<float *>(ws), s)))
        return rc;
    a.x = x; a.wpk = static_cast<const float *>(ws); a.bias = conv->bias; a.y = y;
    a.part = conv_ws_part(conv, 3, ws);
    a.cin = cin; a.cout = conv->out_channels; a.H = h; a.W = w; a.T = t; a.kt = 3;
    return launch_conv3x3(a, s);
}

}  // extern "C"
