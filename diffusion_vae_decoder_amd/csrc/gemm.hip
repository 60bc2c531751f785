// FP32-MFMA GEMM for the decoder's dense contractions that are not 3x3
// convolutions: the 1x1 resnet shortcut (cortiq-engine 0.7.7 `vae`,
// VaeResnetRef), and in the mid-block attention (VaeAttnRef) the q/k/v
// projections, the scores k^T q, P v and the output projection.
//
//   C[m, n] = alpha * sum_k A(m, k) * B(k, n) + bias[m] (+ R[m, n])
//
// A(m, k) is read from A[k*lda + m] ("KM", m contiguous) or A[m*lda + k]
// ("MK"); B(k, n) from B[k*ldb + n] ("KN") or B[n*ldb + k] ("NK").  Tiles of
// 128 x 128 outputs per 256-thread workgroup, K in chunks of 16 staged in LDS
// as [k][m] / [k][n] rows (double-buffered); each wave computes 64 x 64 as
// 2 x 2 v_mfma_f32_32x32x2_f32 tiles.  Lane half h of a wave carries the K
// indices [8h, 8h + 8) of a chunk.  When every tile is full (M, N multiples
// of 128, K of 16, float4-aligned operands and bias) the operand loads walk
// precomputed pointers with no bounds checks, each 2-deep K step's LDS
// operands are read while the previous step's MFMAs run, and the epilogue
// stores through buffer resources (row offsets in scalar registers).
//
// Problems whose tiles cannot fill the GPU (the small attentions) split K
// into ranges of at least 8 chunks; each split stores raw partial sums and
// gemm_splitk_reduce adds them in split order with alpha, bias and residual.
//
// Two attention-only variants split a row softmax across the two products
// that surround it (the score matrix is written once and read once):
//   - EPI_COLSTAT: each workgroup takes, for every column n of its tile, the
//     maximum mb over its valid rows m, stores exp(c - mb) in place of c (the
//     exponentials are needed here for the sums anyway) and writes (mb, sum of
//     exp(c - mb)) at colstat[blockIdx.y * N + n];
//   - B_SOFTMAX: such a B(k, n) (KN) is scaled on load by exp(mb - mx[n]) *
//     inv[n], with (mx, inv) = bsoft[n] the merged statistics of column n and
//     mb = bsblk[(k / 128) * N + n] the maximum of k's 128-row block: one
//     multiply per element, the factor recomputed once per 128 rows.

#include "vae_internal.h"

namespace vae {

namespace {

constexpr int kThreads = 256;
constexpr int BM = 128, BN = 128, BK = 16;
constexpr int LD = 132;   // row stride: 8 * 132 = 1056 = 32 (mod 64), lane halves split the banks
static_assert((8 * LD) % 64 == 32 && LD % 4 == 0, "bad LDS stride");

enum { EPI_STORE = 0, EPI_COLSTAT = 1 };

struct Params {
    const float *A, *B, *bias, *R;
    float *C;
    floatx2 *colstat;
    const floatx2 *bsoft;
    const floatx2 *bsblk;   // B_SOFTMAX: the block statistics EPI_COLSTAT wrote for B
    float *part;       // split K: partial sums [ksplit][M][N]
    int M, N, K, ksplit;
    int buf_epi;       // full tiles: C (and R) within 32-bit byte offsets of a tile's first row
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

// Full tiles: this thread's two element pointers, advanced by a fixed stride
// after every K chunk.
template <bool TRANS>
__device__ __attribute__((always_inline)) inline void tile_ptrs(const float *P, long long ld, int i0,
                                                                const float *(&ptr)[2]) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int idx = tid + q * kThreads;
        if (!TRANS) ptr[q] = P + (long long)(idx >> 5) * ld + i0 + (idx & 31) * 4;
        else ptr[q] = P + (long long)(i0 + (idx >> 2)) * ld + (idx & 3) * 4;
    }
}

__device__ __attribute__((always_inline)) inline void tile_load_full(const float *(&ptr)[2], long long step,
                                                                     floatx4 (&r)[2]) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        r[q] = *reinterpret_cast<const floatx4 *>(ptr[q]);
        ptr[q] += step;
    }
}

// B_SOFTMAX: this thread's four columns n0 + (tid & 31) * 4 + e are the same
// for every chunk, and a chunk's 16 rows lie in one 128-row block, whose
// factors f are current; entries outside the matrix become 0.
template <bool FULL>
__device__ __attribute__((always_inline)) inline void softmax_on_load(floatx4 (&r)[2], int k0, int n,
                                                                      int K, int N, const float (&f)[4]) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int k = k0 + ((threadIdx.x + q * kThreads) >> 5);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float v = r[q][e] * f[e];
            r[q][e] = (FULL || (k < K && n + e < N)) ? v : 0.f;
        }
    }
}

// The factors exp(mb - mx) * inv of the thread's four columns for the 128-row
// block of B that holds row k0.
__device__ __attribute__((always_inline)) inline void softmax_factors(const floatx2 *bsblk, int k0, int n, int N,
                                                                      const float (&mx)[4], const float (&inv)[4],
                                                                      float (&f)[4]) {
    const long long row = (long long)(k0 >> 7) * N;
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = __expf(bsblk[row + (n + e < N ? n + e : N - 1)][0] - mx[e]) * inv[e];
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

// Four waves per SIMD (four workgroups per CU): the accumulators then live in
// the architectural VGPRs (left free, the compiler put them in AGPRs and the
// kernel ran three waves per SIMD, 6-9% slower on the decoder's shapes).
template <bool A_MK, bool B_NK, bool VEC, bool RES, bool FULL, int EPI, bool BSM, bool SPLIT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void gemm_mfma(Params p) {
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

    float smx[4], sinv[4];
    const int sn = n0 + (tid & 31) * 4;
    if (BSM) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const floatx2 st = p.bsoft[sn + e < p.N ? sn + e : p.N - 1];
            smx[e] = st[0];
            sinv[e] = st[1];
        }
    }

    // K chunks [c0, c1) of this workgroup (all of them unless K is split)
    const int n_chunks = (p.K + BK - 1) / BK;
    const int split = SPLIT ? blockIdx.z : 0;
    const int c0 = SPLIT ? (int)((long long)split * n_chunks / p.ksplit) : 0;
    const int c1 = SPLIT ? (int)((long long)(split + 1) * n_chunks / p.ksplit) : n_chunks;
    const int n_iter = c1 - c0;
    const int kb = c0 * BK;
    const float *pa[2], *pb[2];
    const long long sa = A_MK ? BK : BK * p.lda, sb = B_NK ? BK : BK * p.ldb;
    if (FULL) {
        tile_ptrs<A_MK>(p.A, p.lda, m0, pa);
        tile_ptrs<B_NK>(p.B, p.ldb, n0, pb);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            pa[q] += (long long)c0 * sa;
            pb[q] += (long long)c0 * sb;
        }
        tile_load_full(pa, sa, ra);
        tile_load_full(pb, sb, rb);
    } else {
        tile_load<A_MK, VEC>(p.A, p.lda, kb, m0, p.K, p.M, ra);
        tile_load<B_NK, VEC>(p.B, p.ldb, kb, n0, p.K, p.N, rb);
    }
    float sf[4];          // B_SOFTMAX factors of the current 128-row block of B
    int sblk = kb >> 7;
    if (BSM) {
        softmax_factors(p.bsblk, kb, sn, p.N, smx, sinv, sf);
        softmax_on_load<FULL>(rb, kb, sn, p.K, p.N, sf);
    }
    tile_store<A_MK>(As[0], ra);
    tile_store<B_NK>(Bs[0], rb);
    __syncthreads();

    const int a_off = half * 8 * LD + wm * 64 + l32;
    const int b_off = half * 8 * LD + wn * 64 + l32;
    for (int it = 0; it < n_iter; ++it) {
        const int buf = it & 1;
        if (it + 1 < n_iter) {
            if (FULL) {
                tile_load_full(pa, sa, ra);
                tile_load_full(pb, sb, rb);
            } else {
                tile_load<A_MK, VEC>(p.A, p.lda, kb + (it + 1) * BK, m0, p.K, p.M, ra);
                tile_load<B_NK, VEC>(p.B, p.ldb, kb + (it + 1) * BK, n0, p.K, p.N, rb);
            }
        }
        const float *a = As[buf];
        const float *b = Bs[buf];
        // the operands of step s + 1 are read while step s's MFMAs run (left
        // to itself the compiler read each step's operands into the same four
        // registers and waited for them right before its MFMAs)
        float a0 = a[a_off], a1 = a[a_off + 32], b0 = b[b_off], b1 = b[b_off + 32];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            float a0n = 0.f, a1n = 0.f, b0n = 0.f, b1n = 0.f;
            if (s < 7) {
                a0n = a[a_off + (s + 1) * LD];
                a1n = a[a_off + (s + 1) * LD + 32];
                b0n = b[b_off + (s + 1) * LD];
                b1n = b[b_off + (s + 1) * LD + 32];
            }
            acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc[0][0], 0, 0, 0);
            acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, acc[0][1], 0, 0, 0);
            acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, acc[1][0], 0, 0, 0);
            acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc[1][1], 0, 0, 0);
            a0 = a0n; a1 = a1n; b0 = b0n; b1 = b1n;
        }
        // order: the reads of steps 0 and 1, then per step its four MFMAs
        // followed by the reads of the step after next
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int s = 0; s < 7; ++s) {
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            if (s < 6) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        if (it + 1 < n_iter) {
            if (BSM) {
                const int k1 = kb + (it + 1) * BK;
                if ((k1 >> 7) != sblk) {
                    sblk = k1 >> 7;
                    softmax_factors(p.bsblk, k1, sn, p.N, smx, sinv, sf);
                }
                softmax_on_load<FULL>(rb, k1, sn, p.K, p.N, sf);
            }
            tile_store<A_MK>(As[buf ^ 1], ra);
            tile_store<B_NK>(Bs[buf ^ 1], rb);
        }
        __syncthreads();
    }

    // Epilogue: D[i][j] of a 32x32 MFMA tile sits in lane j + 32*((i/4)%2),
    // register (i%4) + 4*(i/8).
    // full tiles: the lane's 32 bias values as float4s (rows m .. m + 3 of a
    // register quad), one load each instead of one per output row
    floatx4 bq[2][4];
    if (FULL && !SPLIT) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                bq[i][g] = p.bias ? *reinterpret_cast<const floatx4 *>(p.bias + m0 + wm * 64 + i * 32 + 8 * g + 4 * half)
                                  : floatx4{0.f, 0.f, 0.f, 0.f};
    }
    if constexpr (FULL && !SPLIT && EPI == EPI_STORE) {
        if (p.buf_epi) {
            // stores through buffer resources: the row offset of each
            // register (uniform) in a scalar offset, the lane's column and
            // row half in the vector offset, no per-element address arithmetic
            const long long r0 = m0 + wm * 64, c0 = n0 + wn * 64;
            const __amdgpu_buffer_rsrc_t cr = __builtin_amdgcn_make_buffer_rsrc(
                p.C + r0 * p.ldc + c0, (short)0, (int)((64 * p.ldc + 64) * 4), 0x00020000);
            __amdgpu_buffer_rsrc_t rr = cr;
            if (RES)
                rr = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(p.R) + r0 * p.ldr + c0, (short)0,
                                                       (int)((64 * p.ldr + 64) * 4), 0x00020000);
            const int vc = (int)((4 * half * p.ldc + l32) * 4), vr = RES ? (int)((4 * half * p.ldr + l32) * 4) : 0;
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = i * 32 + 8 * (r >> 2) + (r & 3);
                        float v = p.alpha * acc[i][j][r] + bq[i][r >> 2][r & 3];
                        if (RES)
                            v += __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                                rr, vr, (int)((row * p.ldr + j * 32) * 4), 0));
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), cr, vc,
                                                                  (int)((row * p.ldc + j * 32) * 4), 0);
                    }
            return;
        }
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
                if (m < p.M && SPLIT) {
                    p.part[((long long)split * p.M + m) * p.N + n] = acc[i][j][r];
                } else if (m < p.M) {
                    float v = p.alpha * acc[i][j][r];
                    if (FULL) v += bq[i][r >> 2][r & 3];
                    else if (p.bias) v += p.bias[m];
                    if (RES) v += p.R[(long long)m * p.ldr + n];
                    if (EPI != EPI_COLSTAT) p.C[(long long)m * p.ldc + n] = v;   // COLSTAT stores below
                    acc[i][j][r] = v;
                }
            }
        }
    }
    if (EPI == EPI_COLSTAT) {
        // Column statistics over this tile's valid rows.  A lane holds 32 rows
        // of each of its two columns; the other lane half and the other row
        // wave hold the rest.  The staging buffers are free after the last
        // barrier of the main loop.
        float *red = As[0];          // [2 row waves][128 columns]: max, then sum
        float *red2 = As[0] + 256;
        float mx[2] = {-INFINITY, -INFINITY};
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                if (FULL || m < p.M) {
                    mx[0] = fmaxf(mx[0], acc[i][0][r]);
                    mx[1] = fmaxf(mx[1], acc[i][1][r]);
                }
            }
#pragma unroll
        for (int j = 0; j < 2; ++j) mx[j] = fmaxf(mx[j], __shfl_xor(mx[j], 32, 64));
        if (half == 0) {
            red[wm * 128 + wn * 64 + l32] = mx[0];
            red[wm * 128 + wn * 64 + 32 + l32] = mx[1];
        }
        __syncthreads();
        float cm[2], sm[2] = {0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int nl = wn * 64 + j * 32 + l32;
            cm[j] = fmaxf(red[nl], red[128 + nl]);
        }
        // C holds exp(c - column maximum of the block); the sums are of those
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                if (FULL || m < p.M) {
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int n = n0 + wn * 64 + j * 32 + l32;
                        const float e = __expf(acc[i][j][r] - cm[j]);
                        sm[j] += e;
                        if (FULL || n < p.N) p.C[(long long)m * p.ldc + n] = e;
                    }
                }
            }
#pragma unroll
        for (int j = 0; j < 2; ++j) sm[j] += __shfl_xor(sm[j], 32, 64);
        if (half == 0) {
            red2[wm * 128 + wn * 64 + l32] = sm[0];
            red2[wm * 128 + wn * 64 + 32 + l32] = sm[1];
        }
        __syncthreads();
        if (tid < BN && n0 + tid < p.N)
            p.colstat[(long long)blockIdx.y * p.N + n0 + tid] =
                floatx2{fmaxf(red[tid], red[128 + tid]), red2[tid] + red2[128 + tid]};
    }
}

// C[m, n] = alpha * sum_s part[s, m, n] (split order) + bias[m] (+ R[m, n]).
__global__ __launch_bounds__(kThreads) void gemm_splitk_reduce(Params p) {
    const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
    const long long mn = (long long)p.M * p.N;
    if (i >= mn) return;
    const int m = (int)(i / p.N), n = (int)(i - (long long)m * p.N);
    float t = 0.f;
    for (int sp = 0; sp < p.ksplit; ++sp) t += p.part[sp * mn + i];
    float v = p.alpha * t;
    if (p.bias) v += p.bias[m];
    if (p.R) v += p.R[(long long)m * p.ldr + n];
    p.C[(long long)m * p.ldc + n] = v;
}

template <bool A_MK, bool B_NK, bool VEC, bool FULL>
void launch4(const Params &p, bool res, dim3 grid, hipStream_t s) {
    if (p.ksplit > 1) hipLaunchKernelGGL((gemm_mfma<A_MK, B_NK, VEC, false, FULL, EPI_STORE, false, true>), grid, dim3(kThreads), 0, s, p);
    else if (res) hipLaunchKernelGGL((gemm_mfma<A_MK, B_NK, VEC, true, FULL, EPI_STORE, false, false>), grid, dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL((gemm_mfma<A_MK, B_NK, VEC, false, FULL, EPI_STORE, false, false>), grid, dim3(kThreads), 0, s, p);
}

template <bool A_MK, bool B_NK>
void launch2(const Params &p, bool vec, bool full, bool res, dim3 grid, hipStream_t s) {
    if (full) launch4<A_MK, B_NK, true, true>(p, res, grid, s);
    else if (vec) launch4<A_MK, B_NK, true, false>(p, res, grid, s);
    else launch4<A_MK, B_NK, false, false>(p, res, grid, s);
}

bool aligned16(const void *ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; }

constexpr int kSlots = 256 * 3;   // CUs x resident GEMM workgroups per CU

}  // namespace

int gemm_ksplit(int M, int N, int K, bool colstat) {
    const long long tiles = (long long)((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    if (colstat || tiles * 2 >= kSlots) return 1;
    const int n_chunks = (K + BK - 1) / BK;
    long long s = (kSlots + tiles - 1) / tiles;
    if (s > n_chunks / 8) s = n_chunks / 8;   // each split keeps >= 8 K chunks
    if (s > 16) s = 16;
    return s < 2 ? 1 : (int)s;
}

size_t gemm_partial_floats(int M, int N, int K, bool colstat) {
    const int s = gemm_ksplit(M, N, K, colstat);
    return s > 1 ? (size_t)s * M * N : 0;
}

int32_t launch_gemm(const GemmLaunch &g, hipStream_t s) {
    Params p;
    p.A = g.A;
    p.B = g.B;
    p.bias = g.bias;
    p.R = g.R;
    p.C = g.C;
    p.colstat = reinterpret_cast<floatx2 *>(g.colstat);
    p.part = g.part;
    p.ksplit = gemm_ksplit(g.M, g.N, g.K, g.colstat != nullptr);
    if (p.ksplit > 1 && !g.part) {
        set_error("gemm: a K-split shape needs a partial-sum workspace");
        return VAE_ERR_WORKSPACE;
    }
    p.bsoft = reinterpret_cast<const floatx2 *>(g.bsoft);
    p.bsblk = reinterpret_cast<const floatx2 *>(g.bsoft_blk);
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
    const bool full = vec && g.M % BM == 0 && g.N % BN == 0 && g.K % BK == 0 && (!g.bias || aligned16(g.bias));
    p.buf_epi = g.ldc * 256 + 256 < (1LL << 31) && (!g.R || g.ldr * 256 + 256 < (1LL << 31));
    const dim3 grid((unsigned)((g.N + BN - 1) / BN), (unsigned)((g.M + BM - 1) / BM), (unsigned)p.ksplit);
    const bool res = g.R != nullptr;
    if (g.colstat || g.bsoft) {
        // the two halves of the attention softmax: scores k^T q (A = k stored KM,
        // B = q stored KN) and P v (A = v stored MK, B = the scores stored KN)
        if (res || b_nk || (g.colstat && g.bsoft) || (g.colstat && a_mk) || (g.bsoft && !a_mk) ||
            (g.bsoft && !g.bsoft_blk)) {
            set_error("gemm: unsupported softmax-split configuration");
            return VAE_ERR_UNSUPPORTED;
        }
#define VAE_GEMM_SM(AMK, E, B, S)                                                                                 \
    if (full) hipLaunchKernelGGL((gemm_mfma<AMK, false, true, false, true, E, B, S>), grid, dim3(kThreads), 0, s, p); \
    else if (vec) hipLaunchKernelGGL((gemm_mfma<AMK, false, true, false, false, E, B, S>), grid, dim3(kThreads), 0, s, p); \
    else hipLaunchKernelGGL((gemm_mfma<AMK, false, false, false, false, E, B, S>), grid, dim3(kThreads), 0, s, p);
        if (g.colstat) {
            VAE_GEMM_SM(false, EPI_COLSTAT, false, false)
        } else if (p.ksplit > 1) {
            VAE_GEMM_SM(true, EPI_STORE, true, true)
        } else {
            VAE_GEMM_SM(true, EPI_STORE, true, false)
        }
#undef VAE_GEMM_SM
    } else if (a_mk) {
        if (b_nk) launch2<true, true>(p, vec, full, res, grid, s);
        else launch2<true, false>(p, vec, full, res, grid, s);
    } else {
        if (b_nk) launch2<false, true>(p, vec, full, res, grid, s);
        else launch2<false, false>(p, vec, full, res, grid, s);
    }
    int32_t rc = check_launch("gemm_mfma");
    if (rc != VAE_OK || p.ksplit == 1) return rc;
    const long long mn = (long long)g.M * g.N;
    hipLaunchKernelGGL(gemm_splitk_reduce, dim3((unsigned)((mn + kThreads - 1) / kThreads)), dim3(kThreads), 0, s, p);
    return check_launch("gemm_splitk_reduce");
}

}  // namespace vae
