// Streaming-softmax form of the mid-block attention (cortiq-engine 0.7.7
// `vae`, VaeAttnRef): softmax(q k^T / sqrt(c)) v for every query, with the
// scores of a query never leaving the registers of the wave that owns it.
//
// Each workgroup takes 64 queries (16 per wave) and a range of keys, in blocks
// of 16 keys.  Per block a wave forms its 16 x 16 tile of transposed scores
// S^T[key, query] on v_mfma_f32_16x16x4_f32, updates the running maximum m
// and sum l of each query's exponentials (the online softmax of Milakov and
// Gimelshein, 2018), rescales its output accumulator by exp(m_old - m_new)
// and adds V P^T for the block.  The labelling of the contraction index makes
// every operand local to its lane:
//   - scores: MFMA step (t, j) of the channel sum pairs lane group g with
//     channel 16 t + 4 g + j, in the A operand (K^T) and in the B operand (Q);
//   - P V: step j of a key block pairs lane group g with key 4 g + j, which
//     is exactly where the score tile's output layout left P[key, query]
//     (register j of lane group g), so P is the B operand as it stands.
// Q of the wave's queries, scaled by 1 / sqrt(c), stays in registers (c / 4
// per lane); the output accumulator holds c x 16 values (c / 4 per lane).
// K is read token-major (K^T, [n, c]: a key block is one contiguous run) and
// V channel-major ([c, n]); both blocks are brought into LDS by direct
// global -> LDS loads, double-buffered, with the 16-byte slots of each row
// permuted (XOR with the row index) so that the MFMA operand reads of 16
// lanes fall on distinct banks.
//
// Key ranges: when the query blocks alone cannot fill the GPU the keys are
// split into R ranges; each range writes its unnormalised output and (m, l)
// per query, and attn_flash_merge combines the ranges of a query in range
// order: O = sum_r exp(m_r - M) O_r / sum_r exp(m_r - M) l_r, M = max_r m_r.
// With one range the kernel divides by l and writes O itself.

#include "wino_common.h"

namespace vae {

namespace {

constexpr int kFQ = 64;       // queries per workgroup: 16 per wave pair
constexpr int kFK = 16;       // keys per block
constexpr int kFWaves = 8;    // 4 query tiles x 2 channel halves
constexpr int kFThreads = 64 * kFWaves;
constexpr int kFSlots = 256;  // resident workgroups: one per CU (two waves per SIMD)

template <int C>
struct FGeom {
    static constexpr int T = C / 16;                  // 16-channel groups
    static constexpr int TH = T / 2;                  // groups of a channel half
    static constexpr int KQ = C / 4;                  // 16-byte slots per K^T row
    static constexpr int KSLOTS = kFK * KQ;           // slots of a K^T block
    static constexpr int VSLOTS = C * kFK / 4;        // slots of a V block
    static constexpr int KDMA = KSLOTS / 64;          // 64-slot direct loads per block
    static constexpr int VDMA = VSLOTS / 64;
    static_assert(C % 128 == 0 && C <= 512, "channel count: 128, 256 or 512");
};

// Row r of a K^T block keeps logical slot q at physical slot q ^ (r & 15);
// row r (a channel) of a V block keeps slot q at q ^ ((r >> 2) & 3).

// Direct loads of key block `kb` (keys kb*16 ..) into (lk, lv).  Keys past n
// read zeros (K^T) or finite values of the next channel row, or zeros past
// the buffer (V): their probabilities are exactly 0.
template <int C>
__device__ __attribute__((always_inline)) inline void flash_stage(__amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr,
                                                                 int kb, int n, floatx4 *lk, floatx4 *lv) {
    using G = FGeom<C>;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int key0 = kb * kFK;
#pragma unroll
    for (int i = 0; i < G::KDMA / kFWaves; ++i) {
        const int d = w + kFWaves * i;
        const int p = 64 * d + lane;
        const int r = p / G::KQ, pq = p - r * G::KQ;
        const int lq = pq ^ (r & 15);
        const int off = key0 + r < n ? ((key0 + r) * C + 4 * lq) * 4 : wino::kWOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (__attribute__((address_space(3))) void *)(lk + 64 * d), 16, off,
                                                 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < G::VDMA / kFWaves; ++i) {
        const int d = w + kFWaves * i;
        const int p = 64 * d + lane;
        const int r = p >> 2, pq = p & 3;
        const int lq = pq ^ ((r >> 2) & 3);
        const int off = (r * n + key0 + 4 * lq) * 4;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (__attribute__((address_space(3))) void *)(lv + 64 * d), 16, off,
                                                 0, 0, 0);
    }
}

// Q [C, n] and V [C, n] channel-major, KT [n, C] token-major.  Range r of R
// covers key blocks [r nb / R, (r + 1) nb / R).  R == 1: O [C, n] normalised;
// else Op [R][C][n] unnormalised and ml [R][n] = (m, l).
//
// Wave w: query tile w >> 1 (16 queries), channel half w & 1.  Each wave of a
// pair sums the scores over its half of the channels; the pair exchanges the
// partial tiles through LDS and adds them in half order, so both hold the
// same scores, maxima, sums and probabilities.  Each then adds V P^T for its
// half of the output channels.
template <int C>
__global__ __launch_bounds__(kFThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_flash(
    const float *__restrict__ Q, const float *__restrict__ KT, const float *__restrict__ V, float *__restrict__ O,
    float *__restrict__ Op, floatx2 *__restrict__ ml, int n, int R, float scale) {
    using G = FGeom<C>;
    __shared__ floatx4 lk0[G::KSLOTS];
    __shared__ floatx4 lk1[G::KSLOTS];
    __shared__ floatx4 lv0[G::VSLOTS];
    __shared__ floatx4 lv1[G::VSLOTS];
    __shared__ floatx4 xs[kFWaves * 64];   // each wave's partial score tile

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int half = wave & 1;
    const int g = lane >> 4, m16 = lane & 15;
    const int q = blockIdx.x * kFQ + 16 * (wave >> 1) + m16;   // the lane's query (column of its tiles)
    const int qc = q < n ? q : n - 1;
    const int r = blockIdx.y;
    const int nb = (n + kFK - 1) / kFK;
    const int b0 = (int)((long long)r * nb / R), b1 = (int)((long long)(r + 1) * nb / R);
    const int t0 = half * G::TH;   // first channel group of the wave's half

    const __amdgpu_buffer_rsrc_t kr = wino::wino_rsrc(KT, (unsigned)((long long)n * C * 4));
    const __amdgpu_buffer_rsrc_t vr = wino::wino_rsrc(V, (unsigned)((long long)n * C * 4));
    flash_stage<C>(kr, vr, b0, n, lk0, lv0);

    // Q of the lane's query over the wave's half, scaled:
    // qr[t][j] = scale * Q[16 (t0 + t) + 4 g + j, q]
    float qr[G::TH][4];
    {
        const float *qp = Q + (long long)(16 * t0 + 4 * g) * n + qc;
#pragma unroll
        for (int t = 0; t < G::TH; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) qr[t][j] = scale * qp[(long long)(16 * t + j) * n];
    }

    floatx4 acc[G::TH];   // O[16 (t0 + T) + 4 g + i, q] in register i of tile T
#pragma unroll
    for (int t = 0; t < G::TH; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
    float mrun = -INFINITY, lrun = 0.f;

    // Operand reads come in chunks of 4 channel groups, each chunk's reads
    // issued while the previous chunk's MFMAs run (scheduling barriers keep
    // the compiler from hoisting every read of the block).  Slot
    // (4 tt + g) ^ m16 of K^T row m16 is 4 (tt ^ a) + (g ^ b), a = m16 >> 2,
    // b = m16 & 3: four per-lane bases (tt mod 4) plus the constant
    // 4 (tt - tt mod 4); t0 is a multiple of 4.  V row 16 tt + m16 is a
    // per-lane base plus the constant 64 tt.
    constexpr int CH = 4;
    constexpr int NCH = G::TH / CH;
    int koff[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) koff[u] = m16 * G::KQ + 4 * (u ^ (m16 >> 2)) + (g ^ (m16 & 3)) + 4 * t0;
    const int voff = m16 * 4 + (g ^ ((m16 >> 2) & 3)) + 64 * t0;

    // the wave's partial scores of key block kb, to xs
    auto scores = [&](const floatx4 *lk) {
        floatx4 sp[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) sp[a] = floatx4{0.f, 0.f, 0.f, 0.f};
        floatx4 kv[2][CH];
#pragma unroll
        for (int u = 0; u < CH; ++u) kv[0][u] = lk[koff[u] + 4 * (u & ~3)];   // K^T[key m16, 16 (t0 + u) + 4 g + j]
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            if (c + 1 < NCH) {
#pragma unroll
                for (int u = 0; u < CH; ++u) {
                    const int t = CH * (c + 1) + u;
                    kv[(c + 1) & 1][u] = lk[koff[t & 3] + 4 * (t & ~3)];
                }
            }
#pragma unroll
            for (int u = 0; u < CH; ++u) {
                const int t = CH * c + u;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    sp[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[c & 1][u][j], qr[t][j], sp[j], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        floatx4 part;
#pragma unroll
        for (int i = 0; i < 4; ++i) part[i] = (sp[0][i] + sp[1][i]) + (sp[2][i] + sp[3][i]);
        xs[wave * 64 + lane] = part;
    };
    // softmax update from the pair's partial scores, then O += V P^T
    auto update = [&](int kb, const floatx4 *lv) {
        const floatx4 p0 = xs[(wave & ~1) * 64 + lane], p1 = xs[(wave | 1) * 64 + lane];
        float s[4];
        const int key0 = kb * kFK + 4 * g;
        const int kend = kb < b1 ? n : 0;   // a dead block (past the range) masks every key
#pragma unroll
        for (int i = 0; i < 4; ++i) s[i] = key0 + i < kend ? p0[i] + p1[i] : -INFINITY;
        float bm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
        bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
        bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
        const float mnew = fmaxf(mrun, bm);
        const float alpha = __expf(mrun - mnew);   // 0 on the first block (mrun = -inf)
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s[i] = __expf(s[i] - mnew);
            ps += s[i];
        }
        ps += __shfl_xor(ps, 16, 64);
        ps += __shfl_xor(ps, 32, 64);
        lrun = lrun * alpha + ps;
        mrun = mnew;
        // once the maxima settle most blocks leave every query's maximum as it
        // was (alpha == 1 in all lanes), and the rescale is skipped
        if (__ballot(alpha != 1.f)) {
#pragma unroll
            for (int t = 0; t < G::TH; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[t][i] *= alpha;
        }
        __builtin_amdgcn_sched_barrier(0);
        floatx4 vv[2][CH];
#pragma unroll
        for (int u = 0; u < CH; ++u) vv[0][u] = lv[voff + 64 * u];   // V[16 (t0 + u) + m16, keys 4 g + j]
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            if (c + 1 < NCH) {
#pragma unroll
                for (int u = 0; u < CH; ++u) vv[(c + 1) & 1][u] = lv[voff + 64 * (CH * (c + 1) + u)];
            }
#pragma unroll
            for (int u = 0; u < CH; ++u) {
                const int t = CH * c + u;
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(vv[c & 1][u][j], s[j], acc[t], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // Block start: this block's loads (issued a block earlier) have landed and
    // every wave is done with the other buffer, which then receives the next
    // block.  Mid-block: the partial scores are in LDS (the direct loads in
    // flight are not waited for).
    auto sync = [&]() {
        __builtin_amdgcn_s_waitcnt(0);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    auto sync_lds = [&]() {
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0) only
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    // The block count is rounded up to an even number with a dead block (all
    // keys masked: it adds exactly 0 and leaves m and l as they are), so the
    // loop has no exit between its two halves; its staging reads keys of the
    // next range or zeros.
    const int b1e = b0 + (b1 - b0 + 1) / 2 * 2;
    for (int kb = b0; kb < b1e; kb += 2) {
        sync();
        flash_stage<C>(kr, vr, kb + 1, n, lk1, lv1);
        scores(lk0);
        sync_lds();
        update(kb, lv0);
        sync();
        if (kb + 2 < b1e) flash_stage<C>(kr, vr, kb + 2, n, lk0, lv0);
        scores(lk1);
        sync_lds();
        update(kb + 1, lv1);
    }

    if (q >= n) return;
    if (R == 1) {
        const float inv = 1.f / lrun;
#pragma unroll
        for (int t = 0; t < G::TH; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) O[(long long)(16 * (t0 + t) + 4 * g + i) * n + q] = acc[t][i] * inv;
    } else {
        float *dst = Op + (long long)r * C * n;
#pragma unroll
        for (int t = 0; t < G::TH; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[(long long)(16 * (t0 + t) + 4 * g + i) * n + q] = acc[t][i];
        if (g == 0 && half == 0) ml[(long long)r * n + q] = floatx2{mrun, lrun};
    }
}

// O[ch, q] = sum_r w_r Op[r, ch, q], w_r = exp(m_r - M) / sum_r exp(m_r - M) l_r,
// ranges in order.  One thread per query and 16 channels.
__global__ __launch_bounds__(256) void attn_flash_merge(const float *__restrict__ Op, const floatx2 *__restrict__ ml,
                                                        float *__restrict__ O, int c, int n, int R) {
    const int q = blockIdx.x * 256 + threadIdx.x;
    if (q >= n) return;
    float M = -INFINITY;
    for (int r = 0; r < R; ++r) M = fmaxf(M, ml[(long long)r * n + q][0]);
    float L = 0.f;
    for (int r = 0; r < R; ++r) {
        const floatx2 v = ml[(long long)r * n + q];
        L += __expf(v[0] - M) * v[1];
    }
    const float invL = 1.f / L;
    const int c0 = blockIdx.y * 16;
    for (int ch = c0; ch < c0 + 16 && ch < c; ++ch) {
        float s = 0.f;
        for (int r = 0; r < R; ++r)
            s += __expf(ml[(long long)r * n + q][0] - M) * Op[((long long)r * c + ch) * n + q];
        O[(long long)ch * n + q] = s * invL;
    }
}

template <int C>
void flash_launch(const float *Q, const float *KT, const float *V, float *O, float *Op, floatx2 *ml, int n, int R,
                  float scale, hipStream_t s) {
    const dim3 grid((unsigned)((n + kFQ - 1) / kFQ), (unsigned)R);
    hipLaunchKernelGGL(attn_flash<C>, grid, dim3(kFThreads), 0, s, Q, KT, V, O, Op, ml, n, R, scale);
}

}  // namespace

bool attention_flash_supported(int c) { return c == 128 || c == 256 || c == 512; }

int attention_flash_ranges(long long n) {
    const long long qb = (n + kFQ - 1) / kFQ;
    const long long nb = (n + kFK - 1) / kFK;
    // fewest rounds of resident workgroups per unit of work, ranges charged
    // 2% each for their partial outputs and merge; each range keeps >= 4 blocks
    int best = 1;
    double best_cost = 1e30;
    for (int r = 1; r <= 32 && (long long)r * 4 <= (nb > 4 ? nb : 4); ++r) {
        const double cost = (double)((qb * r + kFSlots - 1) / kFSlots) / r * (1.0 + 0.02 * (r - 1));
        if (cost < best_cost - 1e-9) {
            best_cost = cost;
            best = r;
        }
    }
    return best;
}

int32_t launch_attention_flash_core(const float *Q, const float *KT, const float *V, float *O, float *Op,
                                    float *ml, int c, long long n, hipStream_t s) {
    const int R = attention_flash_ranges(n);
    const float scale = (float)(1.0 / sqrt((double)c));
    floatx2 *m2 = reinterpret_cast<floatx2 *>(ml);
    switch (c) {
    case 128: flash_launch<128>(Q, KT, V, O, Op, m2, (int)n, R, scale, s); break;
    case 256: flash_launch<256>(Q, KT, V, O, Op, m2, (int)n, R, scale, s); break;
    case 512: flash_launch<512>(Q, KT, V, O, Op, m2, (int)n, R, scale, s); break;
    default:
        set_error("attention (streaming): %d channels; supported: 128, 256, 512", c);
        return VAE_ERR_UNSUPPORTED;
    }
    int32_t rc = check_launch("attn_flash");
    if (rc != VAE_OK || R == 1) return rc;
    hipLaunchKernelGGL(attn_flash_merge, dim3((unsigned)((n + 255) / 256), (unsigned)((c + 15) / 16)), dim3(256), 0, s,
                       Op, m2, O, c, (int)n, R);
    return check_launch("attn_flash_merge");
}

}  // namespace vae
