// FP32-MFMA GEMM for the decoder's dense contractions that are not 3x3
// convolutions: the 1x1 resnet shortcut (cortiq-engine 0.7.7 `vae`,
// VaeResnetRef), and in the mid-block attention (VaeAttnRef) the q/k/v
// projections, q . k^T, P . v and the output projection.
//
//   C[m, n] = alpha * sum_k A(m, k) * B(k, n) + bias[m] (+ R[m, n])
//
// A(m, k) is read from A[k*lda + m] ("KM", m contiguous) or A[m*lda + k]
// ("MK"); B(k, n) from B[k*ldb + n] ("KN") or B[n*ldb + k] ("NK").  Tiles of
// 128 x 128 outputs per 256-thread workgroup, K in chunks of 16 staged in LDS
// as [k][m] / [k][n] rows (double-buffered); each wave computes 64 x 64 as
// 2 x 2 v_mfma_f32_32x32x2_f32 tiles.  Lane half h of a wave carries the K
// indices [8h, 8h + 8) of a chunk.

#include "vae_internal.h"

namespace vae {

namespace {

constexpr int kThreads = 256;
constexpr int BM = 128, BN = 128, BK = 16;
constexpr int LD = 132;   // row stride: 8 * 132 = 1056 = 32 (mod 64), lane halves split the banks
static_assert((8 * LD) % 64 == 32 && LD % 4 == 0, "bad LDS stride");

struct Params {
    const float *A, *B, *bias, *R;
    float *C;
    int M, N, K;
    long long lda, ldb, ldc, ldr;
    float alpha;
};

// Loads one 16 x 128 operand tile (rows k, columns i = m or n) into registers.
// TRANS = false: element (k, i) at P[k*ld + i] (i contiguous);
// TRANS = true : element (k, i) at P[i*ld + k] (k contiguous).
template <bool TRANS, bool VEC>
__device__ __attribute__((always_inline)) inline void tile_load(const float *P, long long ld, int k0,
                                                                int i0, int K, int I,
                                                                floatx4 (&r)[2]) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int idx = tid + q * kThreads;
        int kk, ii;
        if (!TRANS) { kk = idx >> 5; ii = (idx & 31) * 4; }   // 16 rows x 32 float4
        else { ii = idx >> 2; kk = (idx & 3) * 4; }           // 128 rows x 4 float4
        const int k = k0 + kk, i = i0 + ii;
        floatx4 v = {0.f, 0.f, 0.f, 0.f};
        if (!TRANS) {
            if (VEC) {
                if (k < K && i < I) v = *reinterpret_cast<const floatx4 *>(P + (long long)k * ld + i);
            } else if (k < K) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (i + j < I) v[j] = P[(long long)k * ld + i + j];
            }
        } else {
            if (VEC) {
                if (k < K && i < I) v = *reinterpret_cast<const floatx4 *>(P + (long long)i * ld + k);
            } else if (i < I) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (k + j < K) v[j] = P[(long long)i * ld + k + j];
            }
        }
        r[q] = v;
    }
}

template <bool TRANS>
__device__ __attribute__((always_inline)) inline void tile_store(float *lds, const floatx4 (&r)[2]) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int idx = tid + q * kThreads;
        if (!TRANS) {
            const int kk = idx >> 5, ii = (idx & 31) * 4;
            *reinterpret_cast<floatx4 *>(&lds[kk * LD + ii]) = r[q];
        } else {
            const int ii = idx >> 2, kk = (idx & 3) * 4;
#pragma unroll
            for (int j = 0; j < 4; ++j) lds[(kk + j) * LD + ii] = r[q][j];
        }
    }
}

template <bool A_MK, bool B_NK, bool VEC, bool RES>
__global__ __launch_bounds__(kThreads) void gemm_mfma(Params p) {
    __shared__ __attribute__((aligned(16))) float As[2][BK * LD];
    __shared__ __attribute__((aligned(16))) float Bs[2][BK * LD];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int half = lane >> 5, l32 = lane & 31;
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;

    floatx4 ra[2], rb[2];
    floatx16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int n_iter = (p.K + BK - 1) / BK;
    tile_load<A_MK, VEC>(p.A, p.lda, 0, m0, p.K, p.M, ra);
    tile_load<B_NK, VEC>(p.B, p.ldb, 0, n0, p.K, p.N, rb);
    tile_store<A_MK>(As[0], ra);
    tile_store<B_NK>(Bs[0], rb);
    __syncthreads();

    const int a_off = half * 8 * LD + wm * 64 + l32;
    const int b_off = half * 8 * LD + wn * 64 + l32;
    for (int it = 0; it < n_iter; ++it) {
        const int buf = it & 1;
        if (it + 1 < n_iter) {
            tile_load<A_MK, VEC>(p.A, p.lda, (it + 1) * BK, m0, p.K, p.M, ra);
            tile_load<B_NK, VEC>(p.B, p.ldb, (it + 1) * BK, n0, p.K, p.N, rb);
        }
        const float *a = As[buf];
        const float *b = Bs[buf];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const float a0 = a[a_off + s * LD], a1 = a[a_off + s * LD + 32];
            const float b0 = b[b_off + s * LD], b1 = b[b_off + s * LD + 32];
            acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc[0][0], 0, 0, 0);
            acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, acc[0][1], 0, 0, 0);
            acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, acc[1][0], 0, 0, 0);
            acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc[1][1], 0, 0, 0);
        }
        if (it + 1 < n_iter) {
            tile_store<A_MK>(As[buf ^ 1], ra);
            tile_store<B_NK>(Bs[buf ^ 1], rb);
        }
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = n0 + wn * 64 + j * 32 + l32;
            if (n >= p.N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                if (m < p.M) {
                    float v = p.alpha * acc[i][j][r];
                    if (p.bias) v += p.bias[m];
                    if (RES) v += p.R[(long long)m * p.ldr + n];
                    p.C[(long long)m * p.ldc + n] = v;
                }
            }
        }
    }
}

template <bool A_MK, bool B_NK, bool VEC>
void launch3(const Params &p, bool res, dim3 grid, hipStream_t s) {
    if (res) hipLaunchKernelGGL((gemm_mfma<A_MK, B_NK, VEC, true>), grid, dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL((gemm_mfma<A_MK, B_NK, VEC, false>), grid, dim3(kThreads), 0, s, p);
}

template <bool A_MK, bool B_NK>
void launch2(const Params &p, bool vec, bool res, dim3 grid, hipStream_t s) {
    if (vec) launch3<A_MK, B_NK, true>(p, res, grid, s);
    else launch3<A_MK, B_NK, false>(p, res, grid, s);
}

bool aligned16(const void *ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; }

}  // namespace

int32_t launch_gemm(const GemmLaunch &g, hipStream_t s) {
    Params p;
    p.A = g.A;
    p.B = g.B;
    p.bias = g.bias;
    p.R = g.R;
    p.C = g.C;
    p.M = g.M;
    p.N = g.N;
    p.K = g.K;
    p.lda = g.lda;
    p.ldb = g.ldb;
    p.ldc = g.ldc;
    p.ldr = g.ldr;
    p.alpha = g.alpha;
    // In this kernel's terms the A tile is "transposed" when A is stored MK.
    const bool a_mk = !g.a_km;
    const bool b_nk = g.b_nk != 0;
    // float4 loads need the contiguous extent and the leading dimension to be
    // multiples of 4 and 16-byte aligned bases.
    const int a_contig = a_mk ? g.K : g.M;
    const int b_contig = b_nk ? g.K : g.N;
    const bool vec = a_contig % 4 == 0 && b_contig % 4 == 0 && g.lda % 4 == 0 && g.ldb % 4 == 0 &&
                     aligned16(g.A) && aligned16(g.B);
    const dim3 grid((unsigned)((g.N + BN - 1) / BN), (unsigned)((g.M + BM - 1) / BM));
    const bool res = g.R != nullptr;
    if (a_mk) {
        if (b_nk) launch2<true, true>(p, vec, res, grid, s);
        else launch2<true, false>(p, vec, res, grid, s);
    } else {
        if (b_nk) launch2<false, true>(p, vec, res, grid, s);
        else launch2<false, false>(p, vec, res, grid, s);
    }
    return check_launch("gemm_mfma");
}

}  // namespace vae
