// Mid-block single-head spatial attention (cortiq-engine 0.7.7 `vae`,
// VaeAttnRef) on x [c, n], n = h*w tokens in row-major order:
//   xn  = GroupNorm(x)                                   (gn_stats/gn_apply)
//   QKV = Wqkv xn + bqkv,   Wqkv = [Wq; Wk; Wv]  [3c, c]  (one GEMM, [3c, n])
//   S   = (Q^T K) / sqrt(c)                      [n, n]   (GEMM, A read KM)
//   P   = softmax over each row of S                      (in place)
//   O   = V P^T                                  [c, n]   (GEMM, B read NK)
//   y   = x + Wo O + bo                                   (GEMM, residual epilogue)
// The channel-major layout of the decoder's activations makes every product a
// plain GEMM with no transposition in memory.
//
// Workspace: xn [c, n] | QKV [3c, n] | S [n, n] | O [c, n] | GroupNorm partials.

#include "vae_internal.h"

namespace vae {

namespace {
size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }
}  // namespace

size_t attention_ws_bytes(int c, long long n) {
    size_t b = 0;
    b += align256((size_t)c * n * 4);        // xn
    b += align256((size_t)3 * c * n * 4);    // qkv
    b += align256((size_t)n * n * 4);        // S
    b += align256((size_t)c * n * 4);        // O
    b += align256(groupnorm_ws_bytes(c, n)); // partials
    return b;
}

int32_t launch_attention(const float *x, int c, int h, int w, const float *gn_gamma,
                         const float *gn_beta, const float *wqkv, const float *bqkv,
                         const float *wo, const float *bo, float *y, void *ws, hipStream_t s) {
    const long long n = (long long)h * w;
    char *p = static_cast<char *>(ws);
    float *xn = reinterpret_cast<float *>(p);
    p += align256((size_t)c * n * 4);
    float *qkv = reinterpret_cast<float *>(p);
    p += align256((size_t)3 * c * n * 4);
    float *S = reinterpret_cast<float *>(p);
    p += align256((size_t)n * n * 4);
    float *O = reinterpret_cast<float *>(p);
    p += align256((size_t)c * n * 4);
    void *gnws = p;

    int32_t rc = launch_groupnorm(x, c, n, gn_gamma, gn_beta, /*silu=*/0, nullptr, xn, gnws, s);
    if (rc != VAE_OK) return rc;

    GemmLaunch g{};
    // QKV[3c, n] = Wqkv[3c, c] . xn[c, n] + bqkv
    g.A = wqkv; g.lda = c; g.a_km = 0;
    g.B = xn; g.ldb = n; g.b_nk = 0;
    g.bias = bqkv; g.R = nullptr;
    g.C = qkv; g.ldc = n;
    g.M = 3 * c; g.N = (int)n; g.K = c; g.alpha = 1.f;
    if ((rc = launch_gemm(g, s)) != VAE_OK) return rc;

    const float *Q = qkv, *K = qkv + (size_t)c * n, *V = qkv + (size_t)2 * c * n;
    // S[t, u] = sum_ch Q[ch, t] K[ch, u] / sqrt(c)
    g = GemmLaunch{};
    g.A = Q; g.lda = n; g.a_km = 1;
    g.B = K; g.ldb = n; g.b_nk = 0;
    g.C = S; g.ldc = n;
    g.M = (int)n; g.N = (int)n; g.K = c; g.alpha = (float)(1.0 / sqrt((double)c));
    if ((rc = launch_gemm(g, s)) != VAE_OK) return rc;

    if ((rc = launch_softmax_rows(S, (int)n, (int)n, s)) != VAE_OK) return rc;

    // O[ch, t] = sum_u V[ch, u] P[t, u]
    g = GemmLaunch{};
    g.A = V; g.lda = n; g.a_km = 0;
    g.B = S; g.ldb = n; g.b_nk = 1;
    g.C = O; g.ldc = n;
    g.M = c; g.N = (int)n; g.K = (int)n; g.alpha = 1.f;
    if ((rc = launch_gemm(g, s)) != VAE_OK) return rc;

    // y = x + Wo O + bo
    g = GemmLaunch{};
    g.A = wo; g.lda = c; g.a_km = 0;
    g.B = O; g.ldb = n; g.b_nk = 0;
    g.bias = bo; g.R = x; g.ldr = n;
    g.C = y; g.ldc = n;
    g.M = c; g.N = (int)n; g.K = c; g.alpha = 1.f;
    return launch_gemm(g, s);
}

}  // namespace vae
