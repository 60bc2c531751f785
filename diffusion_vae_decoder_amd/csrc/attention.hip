// Mid-block single-head spatial attention (cortiq-engine 0.7.7 `vae`,
// VaeAttnRef) on x [c, n], n = h*w tokens in row-major order:
//   xn  = GroupNorm(x)                                   (gn_stats/gn_apply)
//   QKV = Wqkv xn + bqkv,   Wqkv = [Wq; Wk; Wv]  [3c, c]  (one GEMM, [3c, n])
//   St  = (K^T Q) / sqrt(c)                      [n, n]   St[u, t] = score of query t, key u
//   P   = softmax over u of St[:, t] for every query t
//   O   = V P^T                                  [c, n]   O[:, t] = sum_u V[:, u] P[t, u]
//   y   = x + Wo O + bo                                   (GEMM, residual epilogue)
// The channel-major layout of the decoder's activations makes every product a
// plain GEMM with no transposition in memory.
//
// The softmax never gets a pass of its own.  The scores are produced
// transposed, so the 32 scores of one query in an MFMA tile sit in one lane:
// the score GEMM's epilogue reduces them to (max, sum of exp(s - max)) per
// query and 128-key block and stores exp(s - block max) in place of the
// scores; softmax_merge combines the blocks of every query in a fixed order
// into (max, 1 / sum); and the P V GEMM rescales each 128-key block of those
// exponentials to the query's max and sum as it loads them (one multiply per
// score).  The n x n matrix is written once and read once.
//
// Workspace: xn [c, n] | QKV [3c, n] | St [n, n] | O [c, n] |
//            column statistics [ceil(n/128)][n] x 2 | merged [n] x 2 | GroupNorm partials |
//            K-split partial sums of the small products.

#include "vae_internal.h"

namespace vae {

namespace {
size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t split_floats(int c, long long n) {
    size_t f = gemm_partial_floats(3 * c, (int)n, c, false);
    const size_t pv = gemm_partial_floats(c, (int)n, (int)n, false);
    const size_t out = gemm_partial_floats(c, (int)n, c, false);
    if (pv > f) f = pv;
    if (out > f) f = out;
    return f;
}

// stat[t] = (m, 1/l): the online-softmax combination, in block order, of the
// blocks' (max, sum exp(s - max)) for query t.
__global__ __launch_bounds__(256) void softmax_merge(const floatx2 *__restrict__ colstat, int blocks, int n,
                                                     floatx2 *__restrict__ stat) {
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= n) return;
    float m = -INFINITY, l = 0.f;
    for (int b = 0; b < blocks; ++b) {
        const floatx2 v = colstat[(long long)b * n + t];
        const float mn = fmaxf(m, v[0]);
        l = l * __expf(m - mn) + v[1] * __expf(v[0] - mn);
        m = mn;
    }
    stat[t] = floatx2{m, 1.0f / l};
}
}  // namespace

size_t attention_ws_bytes(int c, long long n) {
    const long long blocks = (n + 127) / 128;
    size_t b = 0;
    b += align256((size_t)c * n * 4);        // xn
    b += align256((size_t)3 * c * n * 4);    // qkv
    b += align256((size_t)n * n * 4);        // St
    b += align256((size_t)c * n * 4);        // O
    b += align256((size_t)blocks * n * 8);   // column statistics
    b += align256((size_t)n * 8);            // merged statistics
    b += align256(groupnorm_ws_bytes(c, n)); // GroupNorm partials
    b += align256(split_floats(c, n) * 4);   // K-split partial sums
    return b;
}

int32_t launch_attention(const float *x, int c, int h, int w, const float *gn_gamma,
                         const float *gn_beta, const float *wqkv, const float *bqkv,
                         const float *wo, const float *bo, float *y, void *ws, hipStream_t s) {
    const long long n = (long long)h * w;
    const int blocks = (int)((n + 127) / 128);
    char *p = static_cast<char *>(ws);
    float *xn = reinterpret_cast<float *>(p);
    p += align256((size_t)c * n * 4);
    float *qkv = reinterpret_cast<float *>(p);
    p += align256((size_t)3 * c * n * 4);
    float *St = reinterpret_cast<float *>(p);
    p += align256((size_t)n * n * 4);
    float *O = reinterpret_cast<float *>(p);
    p += align256((size_t)c * n * 4);
    float *colstat = reinterpret_cast<float *>(p);
    p += align256((size_t)blocks * n * 8);
    float *stat = reinterpret_cast<float *>(p);
    p += align256((size_t)n * 8);
    void *gnws = p;
    p += align256(groupnorm_ws_bytes(c, n));
    float *part = reinterpret_cast<float *>(p);

    int32_t rc = launch_groupnorm(x, c, n, gn_gamma, gn_beta, /*silu=*/0, nullptr, xn, gnws, s);
    if (rc != VAE_OK) return rc;

    GemmLaunch g{};
    // QKV[3c, n] = Wqkv[3c, c] . xn[c, n] + bqkv
    g.A = wqkv; g.lda = c; g.a_km = 0;
    g.B = xn; g.ldb = n; g.b_nk = 0;
    g.bias = bqkv; g.R = nullptr;
    g.C = qkv; g.ldc = n;
    g.M = 3 * c; g.N = (int)n; g.K = c; g.alpha = 1.f;
    g.part = part;
    if ((rc = launch_gemm(g, s)) != VAE_OK) return rc;

    const float *Q = qkv, *K = qkv + (size_t)c * n, *V = qkv + (size_t)2 * c * n;
    // s[u, t] = sum_ch K[ch, u] Q[ch, t] / sqrt(c); St[u, t] = exp(s[u, t] - mb) with mb the max
    // of query t's scores over u's 128-key block, and per-(key block, query) (mb, sum)
    g = GemmLaunch{};
    g.A = K; g.lda = n; g.a_km = 1;
    g.B = Q; g.ldb = n; g.b_nk = 0;
    g.C = St; g.ldc = n;
    g.M = (int)n; g.N = (int)n; g.K = c; g.alpha = (float)(1.0 / sqrt((double)c));
    g.colstat = colstat;
    if ((rc = launch_gemm(g, s)) != VAE_OK) return rc;

    hipLaunchKernelGGL(softmax_merge, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       reinterpret_cast<const floatx2 *>(colstat), blocks, (int)n, reinterpret_cast<floatx2 *>(stat));
    if ((rc = check_launch("softmax_merge")) != VAE_OK) return rc;

    // O[ch, t] = sum_u V[ch, u] P[t, u], P[t, u] = St[u, t] exp(mb - m_t) / l_t applied on load
    g = GemmLaunch{};
    g.A = V; g.lda = n; g.a_km = 0;
    g.B = St; g.ldb = n; g.b_nk = 0;
    g.C = O; g.ldc = n;
    g.M = c; g.N = (int)n; g.K = (int)n; g.alpha = 1.f;
    g.bsoft = stat;
    g.bsoft_blk = colstat;
    g.part = part;
    if ((rc = launch_gemm(g, s)) != VAE_OK) return rc;

    // y = x + Wo O + bo
    g = GemmLaunch{};
    g.A = wo; g.lda = c; g.a_km = 0;
    g.B = O; g.ldb = n; g.b_nk = 0;
    g.bias = bo; g.R = x; g.ldr = n;
    g.C = y; g.ldc = n;
    g.M = c; g.N = (int)n; g.K = c; g.alpha = 1.f;
    g.part = part;
    return launch_gemm(g, s);
}

// ---------------------------------------------------------------------------
// The streaming-softmax form (attention_flash.hip): the scores never reach
// memory.  Workspace: xn [c, n] | Q [c, n] | V [c, n] | K^T [n, c] | O [c, n] |
// per-range outputs [R][c][n] and (m, l) [R][n] (R > 1) | GroupNorm partials |
// K-split partial sums of the projections.
//
// K^T is produced without the key bias: it adds q . b_k to every score of
// query q, a per-query constant that the softmax removes exactly.

namespace {
size_t flash_split_floats(int c, long long n) {
    size_t f = gemm_partial_floats(c, (int)n, c, false);                     // Q, V, output projection
    const size_t kt = gemm_partial_floats((int)n, c, c, false);              // K^T
    return f > kt ? f : kt;
}
}  // namespace

size_t attention_streaming_ws_bytes(int c, long long n) {
    const int R = attention_flash_ranges(n);
    size_t b = 0;
    b += 5 * align256((size_t)c * n * 4);                         // xn, Q, V, K^T, O
    if (R > 1) b += align256((size_t)R * c * n * 4) + align256((size_t)R * n * 8);
    b += align256(groupnorm_ws_bytes(c, n));
    b += align256(flash_split_floats(c, n) * 4);
    return b;
}

int32_t launch_attention_streaming(const float *x, int c, int h, int w, const float *gn_gamma,
                                   const float *gn_beta, const float *wqkv, const float *bqkv,
                                   const float *wo, const float *bo, float *y, void *ws, hipStream_t s) {
    const long long n = (long long)h * w;
    if (!attention_flash_supported(c)) {
        set_error("attention (streaming): %d channels; supported: 128, 256, 512", c);
        return VAE_ERR_UNSUPPORTED;
    }
    if ((long long)c * n * 4 >= (1LL << 31)) {
        set_error("attention (streaming): %lld tokens of %d channels exceed 2 GiB per operand", n, c);
        return VAE_ERR_UNSUPPORTED;
    }
    const int R = attention_flash_ranges(n);
    const size_t a = align256((size_t)c * n * 4);
    char *p = static_cast<char *>(ws);
    float *xn = reinterpret_cast<float *>(p);
    float *Q = reinterpret_cast<float *>(p + a);
    float *V = reinterpret_cast<float *>(p + 2 * a);
    float *KT = reinterpret_cast<float *>(p + 3 * a);
    float *O = reinterpret_cast<float *>(p + 4 * a);
    p += 5 * a;
    float *Op = nullptr, *ml = nullptr;
    if (R > 1) {
        Op = reinterpret_cast<float *>(p);
        p += align256((size_t)R * c * n * 4);
        ml = reinterpret_cast<float *>(p);
        p += align256((size_t)R * n * 8);
    }
    void *gnws = p;
    p += align256(groupnorm_ws_bytes(c, n));
    float *part = reinterpret_cast<float *>(p);

    int32_t rc = launch_groupnorm(x, c, n, gn_gamma, gn_beta, /*silu=*/0, nullptr, xn, gnws, s);
    if (rc != VAE_OK) return rc;
    const size_t cc = (size_t)c * c;
    // Q = Wq xn + bq and V = Wv xn + bv, channel-major [c, n]
    for (int which : {0, 2}) {
        GemmLaunch g{};
        g.A = wqkv + which * cc; g.lda = c; g.a_km = 0;
        g.B = xn; g.ldb = n; g.b_nk = 0;
        g.bias = bqkv + (size_t)which * c;
        g.C = which == 0 ? Q : V; g.ldc = n;
        g.M = c; g.N = (int)n; g.K = c; g.alpha = 1.f;
        g.part = part;
        if ((rc = launch_gemm(g, s)) != VAE_OK) return rc;
    }
    // K^T[t, ch] = sum_k xn[k, t] Wk[ch, k], token-major [n, c]
    {
        GemmLaunch g{};
        g.A = xn; g.lda = n; g.a_km = 1;
        g.B = wqkv + cc; g.ldb = c; g.b_nk = 1;
        g.C = KT; g.ldc = c;
        g.M = (int)n; g.N = c; g.K = c; g.alpha = 1.f;
        g.part = part;
        if ((rc = launch_gemm(g, s)) != VAE_OK) return rc;
    }
    if ((rc = launch_attention_flash_core(Q, KT, V, O, Op, ml, c, n, s)) != VAE_OK) return rc;
    // y = x + Wo O + bo
    GemmLaunch g{};
    g.A = wo; g.lda = c; g.a_km = 0;
    g.B = O; g.ldb = n; g.b_nk = 0;
    g.bias = bo; g.R = x; g.ldr = n;
    g.C = y; g.ldc = n;
    g.M = c; g.N = (int)n; g.K = c; g.alpha = 1.f;
    g.part = part;
    return launch_gemm(g, s);
}

}  // namespace vae
