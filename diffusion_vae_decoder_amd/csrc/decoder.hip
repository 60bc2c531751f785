// The decoder chain (cortiq-engine 0.7.7 `vae`, VaeChainArgs / VaeDecoder):
// conv_in (with the latent de-normalisation in its gather) -> mid resnet ->
// mid attention -> mid resnet -> up blocks (resnets, then nearest x2 folded
// into the upsample conv) -> GroupNorm + SiLU -> conv_out.
//
// The causal 3-D decoder (VAE decode -> GPU handoff, "The CPU VAE code": the
// LTX decoder is a 3-D causal conv decode) is the same chain on a clip
// [c, T, h, w]: every 3x3 conv becomes a causal 3x3x3 conv (time front-padded
// with two copies of frame 0), GroupNorm spans (C/32) x T x H x W, the
// attention runs over all T*H*W positions and upsampling is spatial only.
// It runs on the same kernels with three time taps and T frames.
//
// vae_decoder_create copies every weight once into the caller's `pack`
// buffer (3x3 weights already in the conv kernel's layout, q/k/v
// concatenated), so a decode launches kernels only.  All activations live in
// the caller's workspace, reused across layers:
//   X (block input) | Y (block output) | T, U (resnet temporaries) | S (1x1 skip)
// each sized for the largest activation of the chain, plus GroupNorm
// partials and the attention workspace.

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "vae_internal.h"

using namespace vae;

namespace {

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

struct DConv {
    const float *w = nullptr;   // packed (3x3, in ConvLaunch::wino layout `layout`) or raw [cout, cin] (1x1)
    const float *b = nullptr;
    int cout = 0, cin = 0, k = 0;
    int layout = 0;
    bool present = false;
};
struct DNorm {
    const float *g = nullptr, *b = nullptr;
    int c = 0;
};
struct DRes {
    DNorm n1, n2;
    DConv c1, c2, sc;
    std::string name;
};
struct DAttn {
    DNorm n;
    const float *wqkv = nullptr, *bqkv = nullptr, *wo = nullptr, *bo = nullptr;
    int c = 0;
};
struct DUp {
    std::vector<DRes> res;
    DConv up;
};

struct ProfEntry {
    hipEvent_t start = nullptr, stop = nullptr;
    std::string kernel, layer;
    double flops = 0, bytes = 0;
};

// Walks the weights once to size the pack (dst == nullptr) or to fill it.
struct Packer {
    char *dst;
    size_t off = 0;
    hipStream_t s;
    int kt = 1;   // time taps of the 3x3 convs (3: causal 3-D)
    int32_t rc = VAE_OK;

    const float *take(size_t floats) {
        const size_t at = off;
        off += align256(floats * 4);
        return dst ? reinterpret_cast<const float *>(dst + at) : nullptr;
    }
    const float *copy(const float *src, size_t floats) {
        const float *d = take(floats);
        if (dst && rc == VAE_OK)
            rc = hip_status(hipMemcpyAsync(const_cast<float *>(d), src, floats * 4, hipMemcpyDeviceToDevice, s),
                            "vae_decoder_create: copy");
        return d;
    }
    // raw3: keep a 3x3 weight in its own [cout, cin, 3, 3] layout (the
    // direct conv_out kernel reads that); otherwise 3x3 weights are repacked
    // for the conv's input: de-normalised on load (conv_in), upsampled or plain.
    DConv conv(const vae_conv &c, bool raw3 = false, bool denorm = false, bool upsample = false) {
        DConv d;
        d.present = true;
        d.cout = c.out_channels;
        d.cin = c.in_channels;
        d.k = c.kernel;
        if (c.kernel == 3 && raw3) {
            d.w = copy(c.weight, (size_t)c.out_channels * c.in_channels * 9 * kt);
        } else if (c.kernel == 3) {
            d.layout = conv3x3_layout(denorm, upsample);
            const float *p = take(conv3x3_pack_floats(d.layout, c.out_channels, c.in_channels, kt));
            if (dst && rc == VAE_OK)
                rc = pack_conv3x3_layout(d.layout, c.weight, c.out_channels, c.in_channels, kt, const_cast<float *>(p), s);
            d.w = p;
        } else {
            d.w = copy(c.weight, (size_t)c.out_channels * c.in_channels);
        }
        d.b = copy(c.bias, c.out_channels);
        return d;
    }
    DNorm norm(const vae_norm &n) {
        DNorm d;
        d.c = n.channels;
        d.g = copy(n.gamma, n.channels);
        d.b = copy(n.beta, n.channels);
        return d;
    }
    DRes resnet(const vae_resnet &r, const std::string &name) {
        DRes d;
        d.name = name;
        d.n1 = norm(r.norm1);
        d.c1 = conv(r.conv1);
        d.n2 = norm(r.norm2);
        d.c2 = conv(r.conv2);
        if (r.shortcut.weight) d.sc = conv(r.shortcut);
        return d;
    }
    DAttn attn(const vae_attn &a) {
        DAttn d;
        d.c = a.norm.channels;
        d.n = norm(a.norm);
        const size_t cc = (size_t)d.c * d.c;
        float *wqkv = const_cast<float *>(take(3 * cc));
        float *bqkv = const_cast<float *>(take(3 * (size_t)d.c));
        if (dst) {
            const vae_conv *qkv[3] = {&a.q, &a.k, &a.v};
            for (int i = 0; i < 3 && rc == VAE_OK; ++i) {
                rc = hip_status(hipMemcpyAsync(wqkv + i * cc, qkv[i]->weight, cc * 4, hipMemcpyDeviceToDevice, s), "vae_decoder_create: copy");
                if (rc == VAE_OK)
                    rc = hip_status(hipMemcpyAsync(bqkv + (size_t)i * d.c, qkv[i]->bias, (size_t)d.c * 4, hipMemcpyDeviceToDevice, s), "vae_decoder_create: copy");
            }
        }
        d.wqkv = wqkv;
        d.bqkv = bqkv;
        d.wo = copy(a.out.weight, cc);
        d.bo = copy(a.out.bias, d.c);
        return d;
    }
};

int32_t fail(int32_t code, const char *fmt, ...) {
    char buf[400];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    set_error("%s", buf);
    return code;
}

int32_t check_conv_shape(const char *what, const vae_conv &c, int k, int cin, int cout) {
    if (!c.weight || !c.bias) return fail(VAE_ERR_INVALID_ARG, "vae_decoder_create: %s weight/bias is NULL", what);
    if (c.kernel != k) return fail(VAE_ERR_UNSUPPORTED, "vae_decoder_create: %s kernel %d, want %d", what, c.kernel, k);
    if (c.in_channels != cin || (cout > 0 && c.out_channels != cout))
        return fail(VAE_ERR_INVALID_ARG, "vae_decoder_create: %s is %d->%d, want %d->%d", what, c.in_channels,
                    c.out_channels, cin, cout);
    if (c.out_channels <= 0) return fail(VAE_ERR_INVALID_ARG, "vae_decoder_create: %s has no outputs", what);
    return VAE_OK;
}

int32_t check_norm(const char *what, const vae_norm &n, int c) {
    if (!n.gamma || !n.beta) return fail(VAE_ERR_INVALID_ARG, "vae_decoder_create: %s gamma/beta is NULL", what);
    if (n.channels != c) return fail(VAE_ERR_INVALID_ARG, "vae_decoder_create: %s has %d channels, want %d", what, n.channels, c);
    if (c % 32) return fail(VAE_ERR_UNSUPPORTED, "vae_decoder_create: %s channels %d not divisible by 32", what, c);
    return VAE_OK;
}

int32_t check_resnet(const std::string &name, const vae_resnet &r, int cin, int *cout) {
    int32_t rc;
    const int co = r.conv1.out_channels;
    if ((rc = check_norm((name + ".norm1").c_str(), r.norm1, cin))) return rc;
    if ((rc = check_conv_shape((name + ".conv1").c_str(), r.conv1, 3, cin, -1))) return rc;
    if ((rc = check_norm((name + ".norm2").c_str(), r.norm2, co))) return rc;
    if ((rc = check_conv_shape((name + ".conv2").c_str(), r.conv2, 3, co, co))) return rc;
    if (r.shortcut.weight) {
        if ((rc = check_conv_shape((name + ".conv_shortcut").c_str(), r.shortcut, 1, cin, co))) return rc;
    } else if (cin != co) {
        return fail(VAE_ERR_INVALID_ARG, "vae_decoder_create: %s changes channels %d->%d without a shortcut",
                    name.c_str(), cin, co);
    }
    *cout = co;
    return VAE_OK;
}

int32_t validate(const vae_weights *w) {
    if (!w) return fail(VAE_ERR_INVALID_ARG, "vae_decoder_create: weights is NULL");
    int32_t rc;
    const int zc = w->conv_in.in_channels;
    if (zc <= 0) return fail(VAE_ERR_INVALID_ARG, "vae_decoder_create: conv_in has no inputs");
    if ((rc = check_conv_shape("conv_in", w->conv_in, 3, zc, -1))) return rc;
    if (!(w->scaling_factor != 0.f)) return fail(VAE_ERR_INVALID_ARG, "vae_decoder_create: scaling_factor is 0");
    int c = w->conv_in.out_channels;
    if ((rc = check_resnet("mid_block.resnets.0", w->mid_res0, c, &c))) return rc;
    if ((rc = check_norm("mid_block.attentions.0.group_norm", w->mid_attn.norm, c))) return rc;
    const vae_conv *lin[4] = {&w->mid_attn.q, &w->mid_attn.k, &w->mid_attn.v, &w->mid_attn.out};
    for (int i = 0; i < 4; ++i)
        if ((rc = check_conv_shape("mid_block.attentions.0 projection", *lin[i], 1, c, c))) return rc;
    if ((rc = check_resnet("mid_block.resnets.1", w->mid_res1, c, &c))) return rc;
    if (w->n_up <= 0 || !w->ups) return fail(VAE_ERR_INVALID_ARG, "vae_decoder_create: no up blocks");
    for (int i = 0; i < w->n_up; ++i) {
        const vae_up &u = w->ups[i];
        if (u.n_resnets <= 0 || !u.resnets) return fail(VAE_ERR_INVALID_ARG, "vae_decoder_create: up block %d has no resnets", i);
        for (int j = 0; j < u.n_resnets; ++j) {
            const std::string name = "up_blocks." + std::to_string(i) + ".resnets." + std::to_string(j);
            if ((rc = check_resnet(name, u.resnets[j], c, &c))) return rc;
        }
        if (u.upsample.weight)
            if ((rc = check_conv_shape("upsample conv", u.upsample, 3, c, c))) return rc;
    }
    if ((rc = check_norm("conv_norm_out", w->norm_out, c))) return rc;
    if ((rc = check_conv_shape("conv_out", w->conv_out, 3, c, -1))) return rc;
    return VAE_OK;
}

}  // namespace

struct vae_decoder {
    DConv conv_in;
    DRes mid0, mid1;
    DAttn attn;
    std::vector<DUp> ups;
    DNorm norm_out;
    DConv conv_out;
    float scaling = 1.f, shift = 0.f;
    int latent_c = 0;
    int kt = 1;              // 3: the causal 3-D decoder
    bool direct_out = false; // conv_out kept raw for the direct kernel
    bool gn_fused = false;   // GroupNorm + SiLU applied while the consuming conv loads its input
    int attn_form = VAE_ATTENTION_SPLIT_SOFTMAX;
    // HIP-graph replay of the decode's launch sequence (vae_decoder_set_graph)
    struct Graph {
        bool on = false;
        hipGraphExec_t exec = nullptr;
        const float *latent = nullptr;
        float *rgb = nullptr;
        void *ws = nullptr;
        size_t ws_bytes = 0;
        int T = 0, h = 0, w = 0;
        hipStream_t stream = nullptr;
        bool gn_fused = false;
        int attn_form = 0;
    } graph;
    // profiling
    bool profiling = false;
    std::vector<ProfEntry> prof;
    size_t prof_used = 0;
    // streams of the tiled decode's concurrent tiles (created on first use,
    // default priority), and the events that fork them from and join them to
    // the caller's stream
    static constexpr int kTileStreams = 3;
    struct TileStreams {
        bool made = false;
        hipStream_t s[kTileStreams] = {};
        hipEvent_t fork = nullptr, join[kTileStreams] = {};
    } tiles;
};

namespace {

struct Buffers {
    float *X, *Y, *T, *U, *S;
    float *part;   // split-K partial sums of the small convs
    float *coef;   // GroupNorm coefficients (mean, rstd*gamma, beta, -) per channel, for the next conv
    floatx4 *rec;  // GroupNorm records a conv wrote for the normalisation of its output
    void *gn;
    void *attn;
};

// The chain's spatial plan for a latent of (h, w): largest activation (floats),
// largest GroupNorm workspace, attention workspace.
struct Plan {
    size_t act = 0, gn = 0, attn = 0, part = 0, coef = 0, rec = 0;
};

ConvLaunch launch_shape(const DConv &c, long long H, long long W, int T, int kt) {
    ConvLaunch a{};
    a.cin = c.cin;
    a.cout = c.cout;
    a.H = (int)H;
    a.W = (int)W;
    a.T = T;
    a.kt = kt;
    a.wino = c.layout;
    a.upsample = c.layout == 2;
    return a;
}

// Sizes for a clip of T frames (T = 1 for images).
Plan plan_for(const vae_decoder *d, int T, int h, int w) {
    Plan p;
    const int kt = d->kt;
    auto act = [&](long long c, long long H, long long W) {
        const size_t n = (size_t)(c * T * H * W);
        if (n > p.act) p.act = n;
    };
    auto gn = [&](long long c, long long H, long long W) {
        const size_t b = groupnorm_ws_bytes((int)c, (long long)T * H * W);
        if (b > p.gn) p.gn = b;
        if ((size_t)c * 16 > p.coef) p.coef = (size_t)c * 16;
    };
    auto part = [&](const DConv &c, long long H, long long W) {
        const size_t n = conv3x3_partial_floats(launch_shape(c, H, W, T, kt));
        if (n > p.part) p.part = n;
        const size_t r = (size_t)32 * conv3x3_gn_records(launch_shape(c, H, W, T, kt)) * sizeof(floatx4);
        if (r > p.rec) p.rec = r;
    };
    long long H = h, W = w;
    act(d->latent_c, H, W);
    act(d->conv_in.cout, H, W);
    part(d->conv_in, H, W);
    auto res = [&](const DRes &r) {
        if (r.sc.present) {
            const size_t n = gemm_partial_floats(r.sc.cout, (int)(T * H * W), r.sc.cin, false);
            if (n > p.part) p.part = n;
        }
        gn(r.c1.cin, H, W);
        gn(r.c1.cout, H, W);
        act(r.c1.cin, H, W);
        act(r.c1.cout, H, W);
        part(r.c1, H, W);
        part(r.c2, H, W);
    };
    res(d->mid0);
    p.attn = d->attn_form == VAE_ATTENTION_STREAMING ? attention_streaming_ws_bytes(d->attn.c, (long long)T * H * W)
                                                     : attention_ws_bytes(d->attn.c, (long long)T * H * W);
    res(d->mid1);
    for (const DUp &u : d->ups) {
        for (const DRes &r : u.res) res(r);
        if (u.up.present) {
            H *= 2;
            W *= 2;
            act(u.up.cout, H, W);
            part(u.up, H, W);
        }
    }
    gn(d->norm_out.c, H, W);
    if (d->direct_out) {
        const size_t n = conv3x3_direct_partial_floats(d->conv_out.cout, d->conv_out.cin, kt, (int)H, (int)W, T);
        if (n > p.part) p.part = n;
    } else {
        part(d->conv_out, H, W);
    }
    return p;
}

// Algorithmic FLOPs of a conv over an H x W frame (times the time taps for 3x3 kernels).
double conv_flops(const DConv &c, long long H, long long W, int kt) {
    return 2.0 * c.cout * c.cin * c.k * c.k * (c.k == 3 ? kt : 1) * (double)(H * W);
}

struct Runner {
    vae_decoder *d;
    hipStream_t s;
    float *part = nullptr;
    int T = 1;   // frames
    int32_t rc = VAE_OK;

    ProfEntry *begin(const char *kernel, const std::string &layer, double flops, double bytes) {
        if (!d->profiling || rc != VAE_OK) return nullptr;
        if (d->prof_used == d->prof.size()) {
            // timing-only events: no system-scope fence when they are recorded (a
            // cache writeback per event would stall the stream between launches);
            // their times are read only after the caller has synchronised the device
            ProfEntry e;
            if ((rc = hip_status(hipEventCreateWithFlags(&e.start, hipEventDisableSystemFence),
                                 "hipEventCreateWithFlags")) != VAE_OK) return nullptr;
            if ((rc = hip_status(hipEventCreateWithFlags(&e.stop, hipEventDisableSystemFence),
                                 "hipEventCreateWithFlags")) != VAE_OK) return nullptr;
            d->prof.push_back(e);
        }
        ProfEntry *e = &d->prof[d->prof_used++];
        e->kernel = kernel;
        e->layer = layer;
        e->flops = flops;
        e->bytes = bytes;
        rc = hip_status(hipEventRecord(e->start, s), "hipEventRecord");
        return e;
    }
    void end(ProfEntry *e) {
        if (e && rc == VAE_OK) rc = hip_status(hipEventRecord(e->stop, s), "hipEventRecord");
    }

    float *coef = nullptr;
    // GroupNorm records of the activation rec_of (written by the last conv
    // asked for them), consumed by the next normalisation of that activation.
    floatx4 *rec = nullptr;
    const float *rec_of = nullptr;
    int rec_n = 0;

    void conv3(const std::string &layer, const DConv &c, const float *x, int H, int W, bool up,
               const float *res, float *y, bool denorm = false, bool gn = false, bool stats = false) {
        if (rc != VAE_OK) return;
        rec_of = nullptr;
        ConvLaunch a{};
        a.x = x;
        a.wpk = c.w;
        a.bias = c.b;
        a.res = res;
        a.y = y;
        a.cin = c.cin;
        a.cout = c.cout;
        a.H = H;
        a.W = W;
        a.T = T;
        a.kt = d->kt;
        a.upsample = up ? 1 : 0;
        a.denorm = denorm ? 1 : 0;
        a.dn_scale = d->scaling;
        a.dn_shift = d->shift;
        a.part = part;
        a.gn_coef = gn ? coef : nullptr;
        a.wino = c.layout;
        const int nrec = stats && c.cout % 32 == 0 ? conv3x3_gn_records(a) : 0;
        a.gn_rec = nrec > 0 ? rec : nullptr;
        const double in_elems = (double)c.cin * T * H * W / (up ? 4.0 : 1.0);
        const double out_elems = (double)c.cout * T * H * W;
        const double bytes = 4.0 * (in_elems + out_elems * (res ? 2.0 : 1.0));
        const int ks = conv3x3_ksplit(a);
        ProfEntry *e = begin(conv3x3_kernel_name(a), layer, conv_flops(c, H, W, d->kt) * T,
                             ks > 1 ? 4.0 * (in_elems + out_elems * ks) : bytes);
        if (rc != VAE_OK) return;
        rc = launch_conv3x3_main(a, s);
        end(e);
        if (rc == VAE_OK && ks > 1) {
            e = begin("splitk_reduce", layer, 0.0, 4.0 * out_elems * (ks + 1 + (res ? 1 : 0)));
            if (rc != VAE_OK) return;
            rc = launch_conv3x3_reduce(a, s);
            end(e);
        }
        if (rc == VAE_OK && a.gn_rec) {
            rec_of = y;
            rec_n = nrec;
        }
    }
    // Records for x if the last conv wrote them (then they are used up).
    const floatx4 *take_rec(const float *x, int *n) {
        const floatx4 *r = (x == rec_of) ? rec : nullptr;
        *n = r ? rec_n : 0;
        rec_of = nullptr;
        return r;
    }
    void conv1(const std::string &layer, const DConv &c, const float *x, int H, int W, float *y) {
        if (rc != VAE_OK) return;
        GemmLaunch g{};
        g.A = c.w;
        g.lda = c.cin;
        const long long n = (long long)T * H * W;
        g.B = x;
        g.ldb = n;
        g.bias = c.b;
        g.C = y;
        g.ldc = n;
        g.M = c.cout;
        g.N = (int)n;
        g.K = c.cin;
        g.alpha = 1.f;
        g.part = part;
        ProfEntry *e = begin("gemm_mfma", layer, conv_flops(c, H, W, 1) * T, 4.0 * (c.cin + c.cout) * (double)n);
        if (rc != VAE_OK) return;
        rc = launch_gemm(g, s);
        end(e);
    }
    // GroupNorm statistics of x -> per-channel coefficients in `coef`; the
    // next conv applies the normalisation and SiLU while loading x.
    void gnc(const std::string &layer, const DNorm &n, const float *x, long long spatial, void *ws) {
        if (rc != VAE_OK) return;
        int nr = 0;
        const floatx4 *r = take_rec(x, &nr);
        ProfEntry *e = begin(r ? "groupnorm_merge" : "groupnorm_stats", layer, 0.0, r ? 0.0 : 4.0 * n.c * (double)spatial);
        if (rc != VAE_OK) return;
        rc = launch_groupnorm_coef(x, n.c, spatial, n.g, n.b, ws, coef, s, r, nr);
        end(e);
    }
    void gn(const std::string &layer, const DNorm &n, const float *x, long long spatial, float *y, void *ws) {
        if (rc != VAE_OK) return;
        int nr = 0;
        const floatx4 *r = take_rec(x, &nr);
        ProfEntry *e = begin("groupnorm_silu", layer, 0.0, 8.0 * n.c * (double)spatial);
        if (rc != VAE_OK) return;
        rc = launch_groupnorm(x, n.c, spatial, n.g, n.b, 1, nullptr, y, ws, s, r, nr);
        end(e);
    }
    // X -> Y; uses T, U (and S for a 1x1 skip).  out_stats: the output is
    // normalised next, so conv2 records its GroupNorm statistics.
    void resnet(const DRes &r, Buffers &b, int H, int W, bool out_stats) {
        const long long sp = (long long)T * H * W;
        if (!d->gn_fused) {
            gn(r.name + ".norm1", r.n1, b.X, sp, b.T, b.gn);
            conv3(r.name + ".conv1", r.c1, b.T, H, W, false, nullptr, b.U, false, false, true);
            gn(r.name + ".norm2", r.n2, b.U, sp, b.U, b.gn);
            const float *skip = b.X;
            if (r.sc.present) {
                conv1(r.name + ".conv_shortcut", r.sc, b.X, H, W, b.S);
                skip = b.S;
            }
            conv3(r.name + ".conv2", r.c2, b.U, H, W, false, skip, b.Y, false, false, out_stats);
            return;
        }
        gnc(r.name + ".norm1", r.n1, b.X, sp, b.gn);
        conv3(r.name + ".conv1", r.c1, b.X, H, W, false, nullptr, b.U, false, true, true);
        gnc(r.name + ".norm2", r.n2, b.U, sp, b.gn);
        const float *skip = b.X;
        if (r.sc.present) {
            conv1(r.name + ".conv_shortcut", r.sc, b.X, H, W, b.S);
            skip = b.S;
        }
        conv3(r.name + ".conv2", r.c2, b.U, H, W, false, skip, b.Y, false, true, out_stats);
    }
};

}  // namespace

namespace {

int32_t pack_bytes_kt(const vae_weights *w, int kt, size_t *bytes, const char *who) {
    int32_t rc = validate(w);
    if (rc) return rc;
    if (!bytes) return fail(VAE_ERR_INVALID_ARG, "%s: bytes is NULL", who);
    Packer p{nullptr, 0, nullptr};
    p.kt = kt;
    p.conv(w->conv_in, false, /*denorm=*/true);
    p.resnet(w->mid_res0, "");
    p.attn(w->mid_attn);
    p.resnet(w->mid_res1, "");
    for (int i = 0; i < w->n_up; ++i) {
        for (int j = 0; j < w->ups[i].n_resnets; ++j) p.resnet(w->ups[i].resnets[j], "");
        if (w->ups[i].upsample.weight) p.conv(w->ups[i].upsample, false, false, /*upsample=*/true);
    }
    p.norm(w->norm_out);
    p.conv(w->conv_out, w->conv_out.out_channels <= 4);
    *bytes = p.off;
    return VAE_OK;
}

int32_t create_kt(vae_decoder **out, const vae_weights *w, int kt, void *pack, size_t pack_bytes, void *stream,
                  const char *who) {
    if (!out) return fail(VAE_ERR_INVALID_ARG, "%s: out is NULL", who);
    *out = nullptr;
    size_t need = 0;
    int32_t rc = pack_bytes_kt(w, kt, &need, who);
    if (rc) return rc;
    if (!pack || pack_bytes < need) return fail(VAE_ERR_WORKSPACE, "%s: pack buffer %zu bytes < %zu", who, pack_bytes, need);
    if (reinterpret_cast<uintptr_t>(pack) & 255)
        return fail(VAE_ERR_INVALID_ARG, "%s: pack buffer must be 256-byte aligned", who);
    vae_decoder *d = new vae_decoder();
    d->kt = kt;
    d->direct_out = w->conv_out.out_channels <= 4;
    Packer p{static_cast<char *>(pack), 0, static_cast<hipStream_t>(stream)};
    p.kt = kt;
    d->conv_in = p.conv(w->conv_in, false, /*denorm=*/true);
    d->mid0 = p.resnet(w->mid_res0, "mid_block.resnets.0");
    d->attn = p.attn(w->mid_attn);
    d->mid1 = p.resnet(w->mid_res1, "mid_block.resnets.1");
    for (int i = 0; i < w->n_up; ++i) {
        DUp u;
        for (int j = 0; j < w->ups[i].n_resnets; ++j)
            u.res.push_back(p.resnet(w->ups[i].resnets[j], "up_blocks." + std::to_string(i) + ".resnets." + std::to_string(j)));
        if (w->ups[i].upsample.weight) u.up = p.conv(w->ups[i].upsample, false, false, /*upsample=*/true);
        d->ups.push_back(u);
    }
    d->norm_out = p.norm(w->norm_out);
    d->conv_out = p.conv(w->conv_out, d->direct_out);
    d->scaling = w->scaling_factor;
    d->shift = w->shift_factor;
    d->latent_c = w->conv_in.in_channels;
    if (p.rc != VAE_OK) {
        delete d;
        return p.rc;
    }
    *out = d;
    return VAE_OK;
}

int32_t workspace_bytes_t(const vae_decoder *d, int T, int h, int w, size_t *bytes, const char *who) {
    if (!d || !bytes) return fail(VAE_ERR_INVALID_ARG, "%s: NULL pointer", who);
    if (T <= 0 || h <= 0 || w <= 0) return fail(VAE_ERR_INVALID_ARG, "%s: sizes must be positive", who);
    int32_t c, ho, wo;
    vae_decoder_output_shape(d, h, w, &c, &ho, &wo);
    if ((long long)T * ho * wo > (1LL << 30) || (long long)T * h * w > (1LL << 20))
        return fail(VAE_ERR_UNSUPPORTED, "%s: latent %dx%dx%d too large", who, T, h, w);
    if (T > 65535) return fail(VAE_ERR_UNSUPPORTED, "%s: %d frames exceed the grid limit", who, T);
    const Plan p = plan_for(d, T, h, w);
    *bytes = 5 * align256(p.act * 4) + align256(p.gn) + align256(p.attn) + align256(p.part * 4) +
             align256(p.coef) + align256(p.rec);
    return VAE_OK;
}

// Enqueues every launch of one decode on `stream` (arguments validated).
int32_t run_chain(vae_decoder *d, const float *latent, int T, int h, int w, float *rgb, void *ws, void *stream) {
    const Plan pl = plan_for(d, T, h, w);
    char *base = static_cast<char *>(ws);
    const size_t a = align256(pl.act * 4);
    Buffers b;
    b.X = reinterpret_cast<float *>(base);
    b.Y = reinterpret_cast<float *>(base + a);
    b.T = reinterpret_cast<float *>(base + 2 * a);
    b.U = reinterpret_cast<float *>(base + 3 * a);
    b.S = reinterpret_cast<float *>(base + 4 * a);
    char *q = base + 5 * a;
    b.gn = q;
    q += align256(pl.gn);
    b.attn = q;
    q += align256(pl.attn);
    b.part = reinterpret_cast<float *>(q);
    q += align256(pl.part * 4);
    b.coef = reinterpret_cast<float *>(q);
    q += align256(pl.coef);
    b.rec = reinterpret_cast<floatx4 *>(q);

    Runner r{d, static_cast<hipStream_t>(stream), b.part};
    r.T = T;
    r.coef = b.coef;
    r.rec = b.rec;
    int H = h, W = w;
    r.conv3("conv_in", d->conv_in, latent, H, W, false, nullptr, b.X, /*denorm=*/true, false, /*stats=*/true);
    r.resnet(d->mid0, b, H, W, /*out_stats=*/false);   // the attention normalises its own input
    std::swap(b.X, b.Y);
    if (r.rc == VAE_OK) {
        // tokens: the T*H*W positions, row-major over (t, y, x)
        const double n = (double)T * H * W, c = d->attn.c;
        const bool streaming = d->attn_form == VAE_ATTENTION_STREAMING;
        // algorithmic bytes: the input read and the output written, plus (split
        // softmax) the score matrix written and read once
        ProfEntry *e = r.begin(streaming ? "attention_streaming" : "attention", "mid_block.attentions.0",
                               8.0 * n * c * c + 4.0 * n * n * c,
                               4.0 * (2.0 * c * n + (streaming ? 0.0 : 2.0 * n * n)));
        if (r.rc == VAE_OK) {
            r.rc = streaming ? launch_attention_streaming(b.X, d->attn.c, T * H, W, d->attn.n.g, d->attn.n.b,
                                                          d->attn.wqkv, d->attn.bqkv, d->attn.wo, d->attn.bo, b.Y,
                                                          b.attn, r.s)
                             : launch_attention(b.X, d->attn.c, T * H, W, d->attn.n.g, d->attn.n.b, d->attn.wqkv,
                                                d->attn.bqkv, d->attn.wo, d->attn.bo, b.Y, b.attn, r.s);
            r.end(e);
        }
    }
    std::swap(b.X, b.Y);
    r.resnet(d->mid1, b, H, W, true);
    std::swap(b.X, b.Y);
    for (size_t i = 0; i < d->ups.size(); ++i) {
        const DUp &u = d->ups[i];
        for (size_t j = 0; j < u.res.size(); ++j) {
            // the last resnet before an upsample feeds a conv, not a GroupNorm
            r.resnet(u.res[j], b, H, W, !(j + 1 == u.res.size() && u.up.present));
            std::swap(b.X, b.Y);
        }
        if (u.up.present) {
            H *= 2;
            W *= 2;
            r.conv3("up_blocks." + std::to_string(i) + ".upsamplers.0.conv", u.up, b.X, H, W, true, nullptr, b.Y,
                    false, false, true);
            std::swap(b.X, b.Y);
        }
    }
    // norm_out + SiLU, conv_out.  A conv_out with at most 4 outputs is bound
    // by reading its input: the direct kernel (three time taps for clips)
    // normalises while loading, so only the statistics are computed before
    // it.  A wider conv_out follows the decoder's GroupNorm mode.
    const DConv &c = d->conv_out;
    const long long sp = (long long)T * H * W;
    const bool fused = (c.cout <= 4 && c.cin <= kDirectGnMaxChannels) || d->gn_fused;
    const float *cin_x = fused ? b.X : b.T;
    if (fused) r.gnc("conv_norm_out", d->norm_out, b.X, sp, b.gn);
    else r.gn("conv_norm_out", d->norm_out, b.X, sp, b.T, b.gn);
    if (r.rc == VAE_OK) {
        if (d->direct_out) {
            ProfEntry *e = r.begin("conv3x3_direct", "conv_out", conv_flops(c, H, W, d->kt) * T,
                                   4.0 * (c.cin + c.cout) * (double)T * H * W);
            if (r.rc == VAE_OK) {
                r.rc = launch_conv3x3_direct(cin_x, c.w, c.b, rgb, c.cin, c.cout, H, W, r.s, fused ? b.coef : nullptr,
                                             b.part, T, d->kt);
                r.end(e);
            }
        } else {
            r.conv3("conv_out", c, cin_x, H, W, false, nullptr, rgb, false, fused);
        }
    }
    return r.rc;
}

int32_t decode_t(vae_decoder *d, const float *latent, int T, int h, int w, float *rgb, void *ws, size_t ws_bytes,
                 void *stream, const char *who) {
    if (!d || !latent || !rgb) return fail(VAE_ERR_INVALID_ARG, "%s: NULL pointer", who);
    size_t need = 0;
    int32_t rc = workspace_bytes_t(d, T, h, w, &need, who);
    if (rc) return rc;
    if (!ws || ws_bytes < need) return fail(VAE_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu", who, ws_bytes, need);
    hipStream_t s = static_cast<hipStream_t>(stream);
    vae_decoder::Graph &g = d->graph;
    bool graph = g.on && !d->profiling && s != nullptr;
    if (graph) {
        // a caller that is capturing this stream itself gets the plain launches
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if ((rc = hip_status(hipStreamIsCapturing(s, &cs), "hipStreamIsCapturing"))) return rc;
        graph = cs == hipStreamCaptureStatusNone;
    }
    if (!graph) return run_chain(d, latent, T, h, w, rgb, ws, stream);
    const bool hit = g.exec && g.latent == latent && g.rgb == rgb && g.ws == ws && g.ws_bytes == ws_bytes &&
                     g.T == T && g.h == h && g.w == w && g.stream == s && g.gn_fused == d->gn_fused &&
                     g.attn_form == d->attn_form;
    if (!hit) {
        if (g.exec) {
            (void)hipGraphExecDestroy(g.exec);
            g.exec = nullptr;
        }
        if ((rc = hip_status(hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal), "hipStreamBeginCapture")))
            return rc;
        const int32_t chain_rc = run_chain(d, latent, T, h, w, rgb, ws, stream);
        hipGraph_t graph_def = nullptr;
        rc = hip_status(hipStreamEndCapture(s, &graph_def), "hipStreamEndCapture");
        if (chain_rc == VAE_OK && rc == VAE_OK)
            rc = hip_status(hipGraphInstantiate(&g.exec, graph_def, nullptr, nullptr, 0), "hipGraphInstantiate");
        if (graph_def) (void)hipGraphDestroy(graph_def);
        if (chain_rc != VAE_OK) return chain_rc;
        if (rc != VAE_OK) {
            g.exec = nullptr;
            return rc;
        }
        g.latent = latent;
        g.rgb = rgb;
        g.ws = ws;
        g.ws_bytes = ws_bytes;
        g.T = T;
        g.h = h;
        g.w = w;
        g.stream = s;
        g.gn_fused = d->gn_fused;
        g.attn_form = d->attn_form;
    }
    return hip_status(hipGraphLaunch(g.exec, s), "hipGraphLaunch");
}

}  // namespace

// ---------------------------------------------------------------- tiled decode
// The tiling of the video VAE in cortiq-engine 0.8.78 `vae3d.rs` (the
// constants TILE and TILE_OVERLAP_MIN, split_tiles, VideoVae::decode_clip and
// blend), applied to this decoder: the output plane is cut into tiles of a
// fixed pixel edge along each axis, each tile's latent block is decoded on
// its own, and the decoded tiles are assembled with a linear cross-fade
// across their overlaps.
namespace {

constexpr int kMaxTiles = 64;   // tiles along one axis

// One axis of the schedule (split_tiles): every tile `len` pixels long (one
// tile of the whole axis when it is no longer than a tile); the fewest tiles
// that cover the axis with neighbours overlapping by `ov_min`, the length
// left over then added to the overlaps one latent cell (`step` pixels) at a
// time, from the first overlap on, cycling.  Tile k + 1 starts len - ov[k]
// after tile k.
struct TileAxis {
    int n, len;
    int start[kMaxTiles];
    int ov[kMaxTiles];   // overlap of tile k with tile k + 1
};

int32_t tile_axis(int length, int step, int tile, int ov_min, TileAxis &a, const char *who) {
    a = TileAxis{};
    if (tile >= length) {
        a.n = 1;
        a.len = length;
        return VAE_OK;
    }
    long long n = (length + tile - 1) / tile;
    while (n * tile < (n - 1) * ov_min + length) ++n;
    if (n > kMaxTiles) return fail(VAE_ERR_UNSUPPORTED, "%s: %lld tiles along an axis (at most %d)", who, n, kMaxTiles);
    a.n = (int)n;
    a.len = tile;
    for (int k = 0; k + 1 < a.n; ++k) a.ov[k] = ov_min;
    const long long slack = n * tile - (n - 1) * ov_min - length;   // < tile - ov_min: n is the fewest
    for (long long q = 0; q < slack / step; ++q) a.ov[q % (n - 1)] += step;
    for (int k = 0; k + 1 < a.n; ++k) a.start[k + 1] = a.start[k] + tile - a.ov[k];
    return VAE_OK;
}

// The latent block [c, bh, bw] at (r0, c0) of z [c, h, w].
__global__ __launch_bounds__(256) void tile_extract(const float *__restrict__ z, int c, int h, int w, int r0, int c0,
                                                    int bh, int bw, float *__restrict__ out) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= (long long)c * bh * bw) return;
    const int x = (int)(i % bw);
    const long long r = i / bw;
    const int y = (int)(r % bh), ch = (int)(r / bh);
    out[i] = z[((long long)ch * h + r0 + y) * w + c0 + x];
}

struct TileGrid {
    TileAxis ys, xs;
};

// Output [C, H, W] from the decoded tiles raw[i][j][C][th][tw].  The tiles'
// kept parts partition the plane: tile row i keeps rows [ys.start[i],
// ys.start[i + 1]) (the last one to H), and so on for columns.  A pixel at
// (hh, ww) of tile (i, j): the decoded value; within the overlap e with the
// tile above, (1 - hh/e) * (that tile's row th - e + hh) + (hh/e) * value;
// then within the overlap e' with the tile to the left, (1 - ww/e') * (that
// tile's column tw - e' + ww, as decoded) + (ww/e') * value.  One thread per
// output element; workgroup b covers 256 columns of row b / xchunks (c * H + y).
__global__ __launch_bounds__(256) void tile_assemble(const float *__restrict__ raw, int C, int H, int W, int xchunks,
                                                     TileGrid g, float *__restrict__ out) {
    const int row = blockIdx.x / xchunks;
    const int x = (blockIdx.x - row * xchunks) * 256 + threadIdx.x;
    if (x >= W) return;
    const int c = row / H, y = row - c * H;
    int i = 0, j = 0;
    while (i + 1 < g.ys.n && g.ys.start[i + 1] <= y) ++i;
    while (j + 1 < g.xs.n && g.xs.start[j + 1] <= x) ++j;
    const int th = g.ys.len, tw = g.xs.len;
    const int hh = y - g.ys.start[i], ww = x - g.xs.start[j];
    const long long plane = (long long)th * tw;
    auto tile = [&](int ti, int tj) { return raw + ((long long)(ti * g.xs.n + tj) * C + c) * plane; };
    float v = tile(i, j)[(long long)hh * tw + ww];
    if (i > 0 && hh < g.ys.ov[i - 1]) {
        const int e = g.ys.ov[i - 1];
        const float wb = (float)hh / (float)e, wa = 1.f - wb;
        v = tile(i - 1, j)[(long long)(th - e + hh) * tw + ww] * wa + v * wb;
    }
    if (j > 0 && ww < g.xs.ov[j - 1]) {
        const int e = g.xs.ov[j - 1];
        const float wb = (float)ww / (float)e, wa = 1.f - wb;
        v = tile(i, j - 1)[(long long)hh * tw + tw - e + ww] * wa + v * wb;
    }
    out[(long long)row * W + x] = v;
}

// Workspace: the decoded tiles, a staging tile, and per concurrent stream a
// latent block and a decode workspace.
struct TilePlan {
    TileGrid g;
    int scale, lat_c, out_c, bh, bw;   // a tile's latent block is bh x bw
    size_t lat, stage, raw, dec;       // workspace segments (bytes; lat and dec per stream)
    size_t total() const { return raw + stage + vae_decoder::kTileStreams * (lat + dec); }
};

int32_t tile_plan(const vae_decoder *d, int h, int w, int tile, int overlap, TilePlan &tp, const char *who) {
    if (!d) return fail(VAE_ERR_INVALID_ARG, "%s: NULL decoder", who);
    if (d->kt != 1) return fail(VAE_ERR_INVALID_ARG, "%s: a 3-D decoder", who);
    if (h <= 0 || w <= 0) return fail(VAE_ERR_INVALID_ARG, "%s: sizes must be positive", who);
    int32_t c, H, W;
    vae_decoder_output_shape(d, h, w, &c, &H, &W);
    const int scale = H / h;
    if (tile <= 0 || overlap < 0 || overlap >= tile || tile % scale || overlap % scale)
        return fail(VAE_ERR_INVALID_ARG,
                    "%s: tile %d and overlap %d must be multiples of %d pixels with 0 <= overlap < tile", who, tile,
                    overlap, scale);
    int32_t rc;
    if ((rc = tile_axis(H, scale, tile, overlap, tp.g.ys, who)) || (rc = tile_axis(W, scale, tile, overlap, tp.g.xs, who)))
        return rc;
    tp.scale = scale;
    tp.lat_c = d->latent_c;
    tp.out_c = c;
    tp.bh = tp.g.ys.len / scale;
    tp.bw = tp.g.xs.len / scale;
    const size_t tpx = (size_t)tp.g.ys.len * tp.g.xs.len;
    tp.lat = align256((size_t)tp.lat_c * tp.bh * tp.bw * 4);
    tp.stage = align256((size_t)c * tpx * 4);
    tp.raw = align256((size_t)tp.g.ys.n * tp.g.xs.n * c * tpx * 4);
    return workspace_bytes_t(d, 1, tp.bh, tp.bw, &tp.dec, who);
}

}  // namespace

extern "C" {

int32_t vae_decoder_pack_bytes(const vae_weights *w, size_t *bytes) {
    return pack_bytes_kt(w, 1, bytes, "vae_decoder_pack_bytes");
}

int32_t vae_decoder_create(vae_decoder **out, const vae_weights *w, void *pack, size_t pack_bytes, void *stream) {
    return create_kt(out, w, 1, pack, pack_bytes, stream, "vae_decoder_create");
}

int32_t vae_decoder3d_pack_bytes(const vae_weights *w, size_t *bytes) {
    return pack_bytes_kt(w, 3, bytes, "vae_decoder3d_pack_bytes");
}

int32_t vae_decoder3d_create(vae_decoder **out, const vae_weights *w, void *pack, size_t pack_bytes, void *stream) {
    return create_kt(out, w, 3, pack, pack_bytes, stream, "vae_decoder3d_create");
}

int32_t vae_decoder_output_shape(const vae_decoder *d, int32_t h, int32_t w, int32_t *c, int32_t *ho, int32_t *wo) {
    if (!d || !c || !ho || !wo) return fail(VAE_ERR_INVALID_ARG, "vae_decoder_output_shape: NULL pointer");
    long long H = h, W = w;
    for (const DUp &u : d->ups)
        if (u.up.present) {
            H *= 2;
            W *= 2;
        }
    *c = d->conv_out.cout;
    *ho = (int32_t)H;
    *wo = (int32_t)W;
    return VAE_OK;
}

int32_t vae_decoder_workspace_bytes(const vae_decoder *d, int32_t h, int32_t w, size_t *bytes) {
    if (d && d->kt != 1) return fail(VAE_ERR_INVALID_ARG, "vae_decoder_workspace_bytes: a 3-D decoder; use vae_decoder3d_workspace_bytes");
    return workspace_bytes_t(d, 1, h, w, bytes, "vae_decoder_workspace_bytes");
}

int32_t vae_decoder3d_workspace_bytes(const vae_decoder *d, int32_t t, int32_t h, int32_t w, size_t *bytes) {
    if (d && d->kt != 3) return fail(VAE_ERR_INVALID_ARG, "vae_decoder3d_workspace_bytes: not a 3-D decoder");
    return workspace_bytes_t(d, t, h, w, bytes, "vae_decoder3d_workspace_bytes");
}

int32_t vae_decode(vae_decoder *d, const float *latent, int32_t h, int32_t w, float *rgb, void *ws, size_t ws_bytes,
                   void *stream) {
    if (d && d->kt != 1) return fail(VAE_ERR_INVALID_ARG, "vae_decode: a 3-D decoder; use vae_decode3d");
    return decode_t(d, latent, 1, h, w, rgb, ws, ws_bytes, stream, "vae_decode");
}

int32_t vae_decode3d(vae_decoder *d, const float *latent, int32_t t, int32_t h, int32_t w, float *rgb, void *ws,
                     size_t ws_bytes, void *stream) {
    if (d && d->kt != 3) return fail(VAE_ERR_INVALID_ARG, "vae_decode3d: not a 3-D decoder");
    return decode_t(d, latent, t, h, w, rgb, ws, ws_bytes, stream, "vae_decode3d");
}

int32_t vae_decoder_tiled_workspace_bytes(const vae_decoder *d, int32_t h, int32_t w, int32_t tile, int32_t overlap,
                                          size_t *bytes) {
    if (!bytes) return fail(VAE_ERR_INVALID_ARG, "vae_decoder_tiled_workspace_bytes: NULL pointer");
    TilePlan tp;
    const int32_t rc = tile_plan(d, h, w, tile, overlap, tp, "vae_decoder_tiled_workspace_bytes");
    if (rc) return rc;
    *bytes = tp.total();
    return VAE_OK;
}

int32_t vae_decode_tiled(vae_decoder *d, const float *latent, int32_t h, int32_t w, int32_t tile, int32_t overlap,
                         float *rgb, void *ws, size_t ws_bytes, void *stream) {
    const char *who = "vae_decode_tiled";
    if (!latent || !rgb) return fail(VAE_ERR_INVALID_ARG, "%s: NULL pointer", who);
    TilePlan tp;
    int32_t rc = tile_plan(d, h, w, tile, overlap, tp, who);
    if (rc) return rc;
    const size_t need = tp.total();
    if (!ws || ws_bytes < need) return fail(VAE_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu", who, ws_bytes, need);
    char *base = static_cast<char *>(ws);
    float *raw = reinterpret_cast<float *>(base);
    float *stage = reinterpret_cast<float *>(base + tp.raw);
    auto lat = [&](int k) { return reinterpret_cast<float *>(base + tp.raw + tp.stage + k * (tp.lat + tp.dec)); };
    auto dws = [&](int k) { return static_cast<void *>(base + tp.raw + tp.stage + k * (tp.lat + tp.dec) + tp.lat); };
    hipStream_t s = static_cast<hipStream_t>(stream);
    const TileGrid &g = tp.g;
    const int ntiles = g.ys.n * g.xs.n;
    const size_t tile_bytes = (size_t)tp.out_c * g.ys.len * g.xs.len * 4;
    const long long lat_elems = (long long)tp.lat_c * tp.bh * tp.bw;
    auto slot = [&](int t) { return reinterpret_cast<float *>(reinterpret_cast<char *>(raw) + (size_t)t * tile_bytes); };
    auto extract = [&](int t, float *dst, hipStream_t st) {
        const int i = t / g.xs.n, j = t - i * g.xs.n;
        hipLaunchKernelGGL(tile_extract, dim3((unsigned)((lat_elems + 255) / 256)), dim3(256), 0, st, latent,
                           tp.lat_c, h, w, g.ys.start[i] / tp.scale, g.xs.start[j] / tp.scale, tp.bh, tp.bw, dst);
        return check_launch("tile_extract");
    };
    // Tiles decode concurrently on the decoder's own streams unless the
    // decode is profiled (the records are the handle's), graph replay is on
    // (one graph serves the tiles) or the caller's stream is being captured.
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (s && (rc = hip_status(hipStreamIsCapturing(s, &cs), "hipStreamIsCapturing"))) return rc;
    const int nk = (d->profiling || d->graph.on || cs != hipStreamCaptureStatusNone || ntiles < 2)
                       ? 1 : (ntiles < vae_decoder::kTileStreams ? ntiles : vae_decoder::kTileStreams);
    if (nk == 1) {
        // every tile decodes from one block buffer into one staging buffer
        // (one HIP graph serves them all when graphs are on), then moves to its slot
        for (int t = 0; t < ntiles; ++t) {
            if ((rc = extract(t, lat(0), s))) return rc;
            if ((rc = decode_t(d, lat(0), 1, tp.bh, tp.bw, stage, dws(0), tp.dec, stream, who))) return rc;
            if ((rc = hip_status(hipMemcpyAsync(slot(t), stage, tile_bytes, hipMemcpyDeviceToDevice, s),
                                 "hipMemcpyAsync")))
                return rc;
        }
    } else {
        vae_decoder::TileStreams &ts = d->tiles;
        if (!ts.made) {
            for (int k = 0; k < vae_decoder::kTileStreams && rc == VAE_OK; ++k) {
                rc = hip_status(hipStreamCreateWithFlags(&ts.s[k], hipStreamNonBlocking), "hipStreamCreateWithFlags");
                if (rc == VAE_OK)
                    rc = hip_status(hipEventCreateWithFlags(&ts.join[k], hipEventDisableTiming), "hipEventCreateWithFlags");
            }
            if (rc == VAE_OK)
                rc = hip_status(hipEventCreateWithFlags(&ts.fork, hipEventDisableTiming), "hipEventCreateWithFlags");
            if (rc) {   // release what was made; the next call tries again
                for (int k = 0; k < vae_decoder::kTileStreams; ++k) {
                    if (ts.s[k]) (void)hipStreamDestroy(ts.s[k]);
                    if (ts.join[k]) (void)hipEventDestroy(ts.join[k]);
                    ts.s[k] = nullptr;
                    ts.join[k] = nullptr;
                }
                if (ts.fork) (void)hipEventDestroy(ts.fork);
                ts.fork = nullptr;
                return rc;
            }
            ts.made = true;
        }
        if ((rc = hip_status(hipEventRecord(ts.fork, s), "hipEventRecord"))) return rc;
        for (int k = 0; k < nk; ++k)
            if ((rc = hip_status(hipStreamWaitEvent(ts.s[k], ts.fork, 0), "hipStreamWaitEvent"))) return rc;
        // tile t on stream t % nk, decoded straight into its slot; the
        // caller's stream joins the streams even after a failed launch, so
        // nothing that was enqueued outlives the caller's view of the call
        for (int t = 0; t < ntiles && rc == VAE_OK; ++t) {
            const int k = t % nk;
            rc = extract(t, lat(k), ts.s[k]);
            if (rc == VAE_OK) rc = run_chain(d, lat(k), 1, tp.bh, tp.bw, slot(t), dws(k), ts.s[k]);
        }
        for (int k = 0; k < nk; ++k) {
            int32_t jr = hip_status(hipEventRecord(ts.join[k], ts.s[k]), "hipEventRecord");
            if (jr == VAE_OK) jr = hip_status(hipStreamWaitEvent(s, ts.join[k], 0), "hipStreamWaitEvent");
            if (jr != VAE_OK && rc == VAE_OK) rc = jr;
        }
        if (rc) return rc;
    }
    const int H = h * tp.scale, W = w * tp.scale, xchunks = (W + 255) / 256;
    hipLaunchKernelGGL(tile_assemble, dim3((unsigned)((long long)tp.out_c * H * xchunks)), dim3(256), 0, s, raw, tp.out_c,
                       H, W, xchunks, g, rgb);
    return check_launch("tile_assemble");
}

int32_t vae_decoder_set_graph(vae_decoder *d, int32_t on) {
    if (!d) return fail(VAE_ERR_INVALID_ARG, "vae_decoder_set_graph: NULL decoder");
    d->graph.on = on != 0;
    if (!d->graph.on && d->graph.exec) {
        int32_t rc = hip_status(hipGraphExecDestroy(d->graph.exec), "hipGraphExecDestroy");
        d->graph.exec = nullptr;
        if (rc) return rc;
    }
    return VAE_OK;
}

void vae_decoder_destroy(vae_decoder *d) {
    if (!d) return;
    if (d->graph.exec) (void)hipGraphExecDestroy(d->graph.exec);
    if (d->tiles.made) {
        for (int k = 0; k < vae_decoder::kTileStreams; ++k) {
            (void)hipStreamSynchronize(d->tiles.s[k]);
            (void)hipStreamDestroy(d->tiles.s[k]);
            (void)hipEventDestroy(d->tiles.join[k]);
        }
        (void)hipEventDestroy(d->tiles.fork);
    }
    for (ProfEntry &e : d->prof) {
        if (e.start) (void)hipEventDestroy(e.start);
        if (e.stop) (void)hipEventDestroy(e.stop);
    }
    delete d;
}

int32_t vae_decoder_set_groupnorm_fusion(vae_decoder *d, int32_t on) {
    if (!d) return fail(VAE_ERR_INVALID_ARG, "vae_decoder_set_groupnorm_fusion: NULL decoder");
    if (on) {
        // the conv's coefficient table holds 512 input channels, and its
        // kernel must normalise while loading (not the F(4x4) Winograd form)
        bool wide = false, form = false;
        auto check = [&](const DConv &c) {
            wide = wide || c.cin > 512;
            form = form || !conv3x3_layout_gn_on_load(c.layout);
        };
        check(d->conv_out);
        for (const DRes *r : {&d->mid0, &d->mid1}) check(r->c1), check(r->c2);
        for (const DUp &u : d->ups)
            for (const DRes &r : u.res) check(r.c1), check(r.c2);
        if (wide) return fail(VAE_ERR_UNSUPPORTED, "vae_decoder_set_groupnorm_fusion: a conv has more than 512 inputs");
        if (form)
            return fail(VAE_ERR_UNSUPPORTED,
                        "vae_decoder_set_groupnorm_fusion: the decoder's 3x3 convs use the F(4x4) Winograd form, "
                        "which does not apply GroupNorm on load (create it with the F(2x2) form or the implicit GEMM)");
    }
    d->gn_fused = on != 0;
    return VAE_OK;
}

int32_t vae_decoder_set_attention(vae_decoder *d, int32_t form) {
    if (!d) return fail(VAE_ERR_INVALID_ARG, "vae_decoder_set_attention: NULL decoder");
    if (form != VAE_ATTENTION_SPLIT_SOFTMAX && form != VAE_ATTENTION_STREAMING)
        return fail(VAE_ERR_INVALID_ARG, "vae_decoder_set_attention: unknown form %d", form);
    if (form == VAE_ATTENTION_STREAMING && !attention_flash_supported(d->attn.c))
        return fail(VAE_ERR_UNSUPPORTED, "vae_decoder_set_attention: the streaming form supports 128, 256 or 512 "
                                         "channels, the attention has %d", d->attn.c);
    d->attn_form = form;
    return VAE_OK;
}

int32_t vae_decoder_get_attention(const vae_decoder *d) { return d ? d->attn_form : VAE_ERR_INVALID_ARG; }

int32_t vae_decoder_set_profiling(vae_decoder *d, int32_t on) {
    if (!d) return fail(VAE_ERR_INVALID_ARG, "vae_decoder_set_profiling: NULL decoder");
    d->profiling = on != 0;
    d->prof_used = 0;   // records restart; decodes append until the next call
    return VAE_OK;
}

int32_t vae_decoder_profile(vae_decoder *d, vae_prof_record *out, int32_t max, int32_t *n) {
    if (!d || !n || (max > 0 && !out)) return fail(VAE_ERR_INVALID_ARG, "vae_decoder_profile: NULL pointer");
    *n = (int32_t)d->prof_used;
    for (size_t i = 0; i < d->prof_used && (int32_t)i < max; ++i) {
        ProfEntry &e = d->prof[i];
        int32_t rc = hip_status(hipEventSynchronize(e.stop), "hipEventSynchronize");
        if (rc) return rc;
        float ms = 0.f;
        if ((rc = hip_status(hipEventElapsedTime(&ms, e.start, e.stop), "hipEventElapsedTime"))) return rc;
        vae_prof_record &o = out[i];
        memset(&o, 0, sizeof o);
        snprintf(o.kernel, sizeof o.kernel, "%s", e.kernel.c_str());
        snprintf(o.layer, sizeof o.layer, "%s", e.layer.c_str());
        o.ms = ms;
        o.flops = e.flops;
        o.bytes = e.bytes;
    }
    return VAE_OK;
}

}  // extern "C"
