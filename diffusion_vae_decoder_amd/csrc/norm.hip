// GroupNorm(32, eps 1e-6, affine) + SiLU (cortiq-engine 0.7.7 `vae`,
// GroupNorm / VaeNormRef; cortiq-engine 0.8.78 vae3d.rs GroupNorm::apply for
// the statistics: group mean and biased variance) and nearest x2 upsample
// (VaeUpRef).
//
// GroupNorm needs the group statistics before it can write anything.  In the
// decoder they come from the producing conv, which writes per-group records
// (count, mean, sum of squared deviations) of every tile it stores; gn_merge
// sums the records in float64 in a fixed order (or, for a short list, each
// gn_apply workgroup does).  Without records (standalone calls, the input of
// the attention) gn_stats makes the statistics pass: a grid of (parts, 32
// groups) workgroups each reduces one contiguous slice of a group to (sum d,
// sum d^2) with d = x - x_first (the group's first value, a shift that keeps
// the variance free of cancellation); float32 per float4, float64 across
// float4s and threads.  gn_apply: a grid of (spatial chunks, channels); each
// workgroup merges its group's statistics in a fixed order (deterministic),
// then streams y = silu((x - mean) * rstd * gamma + beta) [+ residual] with
// float4 loads and stores.

#include "vae_internal.h"

namespace vae {

namespace {

constexpr int kThreads = 256;
constexpr int kGroups = 32;
constexpr int kMaxParts = 64;
constexpr long long kPartElems = 16384;   // group elements per stats workgroup, at least
constexpr int kApplyElems = 4096;         // elements per apply workgroup (16 per thread)
constexpr int kApplyBatch = kApplyElems / (4 * kThreads);   // float4 loads in flight per apply thread
constexpr int kStatsBatch = 8;            // float4 loads in flight per statistics thread
constexpr int kInlineRecords = 512;       // producer records per group an apply workgroup merges itself

int parts_for(long long gsize) {
    long long p = (gsize + kPartElems - 1) / kPartElems;
    if (p < 1) p = 1;
    if (p > kMaxParts) p = kMaxParts;
    return (int)p;
}

__device__ inline double warp_sum(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_down(v, o, 64);
    return v;
}

// Sum over the 256 threads of a workgroup in a fixed order; result valid in thread 0.
__device__ inline void block_sum2(double &a, double &b, double *scratch) {
    a = warp_sum(a);
    b = warp_sum(b);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) {
        scratch[wave] = a;
        scratch[4 + wave] = b;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        a = (scratch[0] + scratch[1]) + (scratch[2] + scratch[3]);
        b = (scratch[4] + scratch[5]) + (scratch[6] + scratch[7]);
    }
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void gn_stats(const float *__restrict__ x, long long gsize,
                                                     int parts, double *__restrict__ part,
                                                     double *__restrict__ shift_out) {
    __shared__ double scratch[8];
    const int g = blockIdx.y, pi = blockIdx.x;
    const float *base = x + (long long)g * gsize;
    const float shift = base[0];
    long long chunk = (gsize + parts - 1) / parts;
    chunk = (chunk + 3) & ~3LL;
    const long long lo = (long long)pi * chunk;
    long long hi = lo + chunk;
    if (hi > gsize) hi = gsize;
    double s1 = 0.0, s2 = 0.0;
    if (VEC) {
        const floatx4 *b4 = reinterpret_cast<const floatx4 *>(base);
        auto add = [&](const floatx4 &v) {
            const float d0 = v[0] - shift, d1 = v[1] - shift, d2 = v[2] - shift, d3 = v[3] - shift;
            s1 += (double)((d0 + d1) + (d2 + d3));
            s2 += (double)((d0 * d0 + d1 * d1) + (d2 * d2 + d3 * d3));
        };
        // kStatsBatch loads in flight per thread (one at a time, each waited
        // for, leaves the pass latency-bound); the float4s are added in the
        // same order as by the plain loop
        long long i = lo / 4 + threadIdx.x;
        const long long e = hi / 4;
        for (; i + (kStatsBatch - 1) * kThreads < e; i += kStatsBatch * kThreads) {
            floatx4 v[kStatsBatch];
#pragma unroll
            for (int k = 0; k < kStatsBatch; ++k) v[k] = b4[i + k * kThreads];
#pragma unroll
            for (int k = 0; k < kStatsBatch; ++k) add(v[k]);
        }
        for (; i < e; i += kThreads) add(b4[i]);
    } else {
        for (long long i = lo + threadIdx.x; i < hi; i += kThreads) {
            const float d = base[i] - shift;
            s1 += (double)d;
            s2 += (double)d * (double)d;
        }
    }
    block_sum2(s1, s2, scratch);
    if (threadIdx.x == 0) {
        part[2 * ((long long)g * parts + pi)] = s1;
        part[2 * ((long long)g * parts + pi) + 1] = s2;
        if (pi == 0) shift_out[g] = (double)shift;
    }
}

// With `rec` set (a short list of producer records per group) or `part` (the
// statistics pass's partial sums) each workgroup merges its group's
// statistics itself; otherwise it reads the group's (mean, rstd) that gn_merge
// wrote.
template <bool VEC, bool SILU, bool RES>
__global__ __launch_bounds__(kThreads) void gn_apply(const float *x, long long spatial, int cpg,
                                                     const floatx2 *__restrict__ gstat,
                                                     const double *__restrict__ part, int parts,
                                                     const double *__restrict__ shifts,
                                                     const float *__restrict__ gamma,
                                                     const float *__restrict__ beta,
                                                     const float *res, float *y,
                                                     const floatx4 *__restrict__ rec, int nrec) {
    __shared__ double scratch[8];
    __shared__ float stat[2];
    const int c = blockIdx.y;
    const int g = c / cpg;
    float mean, scale;
    if (rec || part) {
        // the workgroup merges its group's statistics itself: producer records,
        // or the statistics pass's shifted partial sums, in a fixed order
        double s1 = 0.0, s2 = 0.0;
        if (rec) {
            for (int i = threadIdx.x; i < nrec; i += kThreads) {
                const floatx4 v = rec[(long long)g * nrec + i];
                const double n = v[0], m = v[1];
                s1 += n * m;
                s2 += (double)v[2] + n * m * m;
            }
        } else if (threadIdx.x < parts) {
            s1 = part[2 * ((long long)g * parts + threadIdx.x)];
            s2 = part[2 * ((long long)g * parts + threadIdx.x) + 1];
        }
        block_sum2(s1, s2, scratch);
        if (threadIdx.x == 0) {
            const double n = (double)spatial * cpg;
            double mu, var;
            if (rec) {   // s1 = sum n m, s2 = sum (M2 + n m^2) over the records
                mu = s1 / n;
                var = (s2 - s1 * mu) / n;
            } else {     // shifted sums d = x - shift
                const double md = s1 / n;
                var = s2 / n - md * md;
                mu = shifts[g] + md;
            }
            if (var < 0.0) var = 0.0;
            stat[0] = (float)mu;
            stat[1] = (float)(1.0 / sqrt(var + 1e-6) * (double)gamma[c]);
        }
        __syncthreads();
        mean = stat[0];
        scale = stat[1];
    } else {
        const floatx2 st = gstat[g];
        mean = st[0];
        scale = st[1] * gamma[c];
    }
    const float b = beta[c];
    const long long cbase = (long long)c * spatial;
    const long long lo = (long long)blockIdx.x * kApplyElems;
    long long hi = lo + kApplyElems;
    if (hi > spatial) hi = spatial;
    auto f = [&](float v) {
        float t = (v - mean) * scale + b;
        if (SILU) t = t / (1.0f + __expf(-t));
        return t;
    };
    if (VEC) {
        const floatx4 *x4 = reinterpret_cast<const floatx4 *>(x + cbase);
        const floatx4 *r4 = reinterpret_cast<const floatx4 *>(res + cbase);
        floatx4 *y4 = reinterpret_cast<floatx4 *>(y + cbase);
        auto out = [&](const floatx4 &v, const floatx4 &r) {
            floatx4 o;
            o[0] = f(v[0]);
            o[1] = f(v[1]);
            o[2] = f(v[2]);
            o[3] = f(v[3]);
            if (RES) {
                o[0] += r[0];
                o[1] += r[1];
                o[2] += r[2];
                o[3] += r[3];
            }
            return o;
        };
        // all of a thread's loads of a full chunk are issued before its first
        // store (a wait for a load also waits for the stores before it); each
        // element is still read before the same thread writes it, so y may be x
        long long i = lo / 4 + threadIdx.x;
        const long long e = hi / 4;
        for (; i + (kApplyBatch - 1) * kThreads < e; i += kApplyBatch * kThreads) {
            floatx4 v[kApplyBatch], r[kApplyBatch];
#pragma unroll
            for (int k = 0; k < kApplyBatch; ++k) {
                v[k] = x4[i + k * kThreads];
                if (RES) r[k] = r4[i + k * kThreads];
            }
#pragma unroll
            for (int k = 0; k < kApplyBatch; ++k) y4[i + k * kThreads] = out(v[k], r[k]);
        }
        for (; i < e; i += kThreads) y4[i] = out(x4[i], RES ? r4[i] : floatx4{});
    } else {
        for (long long i = lo + threadIdx.x; i < hi; i += kThreads) {
            float t = f(x[cbase + i]);
            if (RES) t += res[cbase + i];
            y[cbase + i] = t;
        }
    }
}

// (mean, rstd) of each group from the statistics pass's shifted partial sums,
// added in part order (deterministic): one thread per group.
__global__ __launch_bounds__(64) void gn_finalize(long long gsize, int parts, const double *__restrict__ part,
                                                  const double *__restrict__ shifts, floatx2 *__restrict__ gstat) {
    const int g = threadIdx.x;
    if (g >= kGroups) return;
    double s1 = 0.0, s2 = 0.0;
    for (int i = 0; i < parts; ++i) {
        s1 += part[2 * ((long long)g * parts + i)];
        s2 += part[2 * ((long long)g * parts + i) + 1];
    }
    const double n = (double)gsize;
    const double md = s1 / n;
    double var = s2 / n - md * md;
    if (var < 0.0) var = 0.0;
    gstat[g] = floatx2{(float)(shifts[g] + md), (float)(1.0 / sqrt(var + 1e-6))};
}

// Per-channel coefficients of GroupNorm for a consumer that normalises on
// load: coef[c] = (mean_g, rstd_g * gamma[c], beta[c], 0).
__global__ __launch_bounds__(kThreads) void gn_coef(int c, int cpg, const floatx2 *__restrict__ gstat,
                                                    const float *__restrict__ gamma,
                                                    const float *__restrict__ beta, float *__restrict__ coef) {
    const int ch = blockIdx.x * kThreads + threadIdx.x;
    if (ch >= c) return;
    const floatx2 st = gstat[ch / cpg];
    reinterpret_cast<floatx4 *>(coef)[ch] = floatx4{st[0], st[1] * gamma[ch], beta[ch], 0.f};
}

// One workgroup per group merges the group's records (count n, mean m, M2)
// into float64 sums S0 = sum n, S1 = sum n m and S2 = sum (M2 + n m^2), in a
// fixed order (a strided pass per thread, then a fixed tree), and stores the
// group's mean S1 / S0 and rstd 1 / sqrt((S2 - S1^2 / S0) / S0 + eps).  The records' own
// centring keeps M2 accurate in float32; the float64 sums then lose nothing
// to cancellation unless the mean exceeds the spread by ~1e6.
__global__ __launch_bounds__(kThreads) void gn_merge(const floatx4 *__restrict__ rec, int nrec,
                                                     floatx2 *__restrict__ gstat) {
    __shared__ double sh[3 * 4];
    const int g = blockIdx.x;
    const floatx4 *r = rec + (long long)g * nrec;
    double s0 = 0.0, s1 = 0.0, s2 = 0.0;
#pragma unroll 4
    for (int i = threadIdx.x; i < nrec; i += kThreads) {
        const floatx4 v = r[i];
        const double n = v[0], m = v[1];
        s0 += n;
        s1 += n * m;
        s2 += (double)v[2] + n * m * m;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        s0 += __shfl_down(s0, o, 64);
        s1 += __shfl_down(s1, o, 64);
        s2 += __shfl_down(s2, o, 64);
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) {
        sh[3 * wave] = s0;
        sh[3 * wave + 1] = s1;
        sh[3 * wave + 2] = s2;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const double n = (sh[0] + sh[3]) + (sh[6] + sh[9]);
        const double t1 = (sh[1] + sh[4]) + (sh[7] + sh[10]);
        const double t2 = (sh[2] + sh[5]) + (sh[8] + sh[11]);
        const double mean = t1 / n;
        double m2 = t2 - t1 * mean;
        if (m2 < 0.0) m2 = 0.0;
        gstat[g] = floatx2{(float)mean, (float)(1.0 / sqrt(m2 / n + 1e-6))};
    }
}

struct ApplyStats {
    const floatx2 *gstat;                  // merged (mean, rstd) per group, or
    const double *part; int parts;         // the statistics pass's partial sums, or
    const double *shifts;
    const floatx4 *rec; int nrec;          // producer records
};

template <bool VEC, bool SILU>
void apply2(bool res, dim3 grid, hipStream_t s, const float *x, long long spatial, int cpg, const ApplyStats &st,
            const float *gamma, const float *beta, const float *r, float *y) {
    if (res)
        hipLaunchKernelGGL((gn_apply<VEC, SILU, true>), grid, dim3(kThreads), 0, s, x, spatial, cpg, st.gstat, st.part,
                           st.parts, st.shifts, gamma, beta, r, y, st.rec, st.nrec);
    else
        hipLaunchKernelGGL((gn_apply<VEC, SILU, false>), grid, dim3(kThreads), 0, s, x, spatial, cpg, st.gstat,
                           st.part, st.parts, st.shifts, gamma, beta, r, y, st.rec, st.nrec);
}

// ------------------------------------------------------------- upsample x2
__global__ void upsample2x_pairs(const float *__restrict__ x, float *__restrict__ y, int h, int w,
                                 long long total_pairs) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total_pairs) return;
    const int half_w = w >> 1;
    const long long row = i / half_w;        // (c, yy) input row
    const int q = (int)(i - row * half_w);
    const float a = x[row * w + 2 * q];
    const float b = x[row * w + 2 * q + 1];
    const long long c = row / h;
    const int yy = (int)(row - c * h);
    const long long obase = (c * 2 * h + 2 * yy) * (long long)(2 * w) + 4 * q;
    const floatx4 v = {a, a, b, b};
    *reinterpret_cast<floatx4 *>(y + obase) = v;
    *reinterpret_cast<floatx4 *>(y + obase + 2 * w) = v;
}

__global__ void upsample2x_scalar(const float *__restrict__ x, float *__restrict__ y, int h, int w,
                                  long long total) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int W2 = 2 * w, H2 = 2 * h;
    const int xx = (int)(i % W2);
    const long long r = i / W2;
    const int yy = (int)(r % H2);
    const long long c = r / H2;
    y[i] = x[(c * h + (yy >> 1)) * w + (xx >> 1)];
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// The statistics pass over x: shifted partial sums of each group's slices
// into ws (parts per group), and each group's shift.
int32_t groupnorm_pass(const float *x, int c, long long spatial, void *ws, hipStream_t s) {
    const long long gsize = (long long)(c / kGroups) * spatial;
    const int parts = parts_for(gsize);
    double *part = reinterpret_cast<double *>(ws);
    double *shifts = part + 2 * kGroups * parts;
    if (gsize % 4 == 0 && aligned16(x))
        hipLaunchKernelGGL(gn_stats<true>, dim3(parts, kGroups), dim3(kThreads), 0, s, x, gsize, parts, part, shifts);
    else
        hipLaunchKernelGGL(gn_stats<false>, dim3(parts, kGroups), dim3(kThreads), 0, s, x, gsize, parts, part, shifts);
    return check_launch("gn_stats");
}

// Statistics of x's 32 groups: (mean, rstd) per group into `gstat`, from the
// records a producer wrote or from a pass over x (partial sums in ws).
int32_t groupnorm_stats(const float *x, int c, long long spatial, void *ws, floatx2 *gstat, hipStream_t s,
                        const floatx4 *rec, int nrec) {
    if (rec) {
        hipLaunchKernelGGL(gn_merge, dim3(kGroups), dim3(kThreads), 0, s, rec, nrec, gstat);
        return check_launch("gn_merge");
    }
    int32_t rc = groupnorm_pass(x, c, spatial, ws, s);
    if (rc != VAE_OK) return rc;
    const long long gsize = (long long)(c / kGroups) * spatial;
    const int parts = parts_for(gsize);
    const double *part = reinterpret_cast<const double *>(ws);
    hipLaunchKernelGGL(gn_finalize, dim3(1), dim3(64), 0, s, gsize, parts, part, part + 2 * kGroups * parts, gstat);
    return check_launch("gn_finalize");
}

}  // namespace

// Workspace: the statistics pass's partial sums and shifts, then (mean, rstd)
// per group.
size_t groupnorm_ws_bytes(int c, long long spatial) {
    const long long gsize = (long long)(c / kGroups) * spatial;
    return (size_t)kGroups * parts_for(gsize) * 2 * sizeof(double) + kGroups * sizeof(double) +
           kGroups * sizeof(floatx2);
}

namespace {
floatx2 *gstat_of(void *ws, int c, long long spatial) {
    const long long gsize = (long long)(c / kGroups) * spatial;
    return reinterpret_cast<floatx2 *>(static_cast<char *>(ws) +
                                       (size_t)kGroups * parts_for(gsize) * 2 * sizeof(double) +
                                       kGroups * sizeof(double));
}
}  // namespace

int32_t launch_groupnorm(const float *x, int c, long long spatial, const float *gamma,
                         const float *beta, int silu, const float *res, float *y, void *ws,
                         hipStream_t s, const floatx4 *rec, int nrec) {
    const int cpg = c / kGroups;
    ApplyStats st{};
    int32_t rc = VAE_OK;
    if (rec && nrec <= kInlineRecords) {
        // a few records per group: every apply workgroup merges its group's own
        st.rec = rec;
        st.nrec = nrec;
    } else if (rec) {
        st.gstat = gstat_of(ws, c, spatial);
        rc = groupnorm_stats(x, c, spatial, ws, const_cast<floatx2 *>(st.gstat), s, rec, nrec);
    } else {
        // every apply workgroup merges the statistics pass's partial sums
        // (cheaper than a launch that merges them once)
        rc = groupnorm_pass(x, c, spatial, ws, s);
        st.parts = parts_for((long long)cpg * spatial);
        st.part = reinterpret_cast<const double *>(ws);
        st.shifts = st.part + 2 * kGroups * st.parts;
    }
    if (rc != VAE_OK) return rc;
    const bool vec = spatial % 4 == 0 && aligned16(x) && aligned16(y) && (!res || aligned16(res));
    const dim3 grid((unsigned)((spatial + kApplyElems - 1) / kApplyElems), (unsigned)c);
    if (vec) {
        if (silu) apply2<true, true>(res, grid, s, x, spatial, cpg, st, gamma, beta, res, y);
        else apply2<true, false>(res, grid, s, x, spatial, cpg, st, gamma, beta, res, y);
    } else {
        if (silu) apply2<false, true>(res, grid, s, x, spatial, cpg, st, gamma, beta, res, y);
        else apply2<false, false>(res, grid, s, x, spatial, cpg, st, gamma, beta, res, y);
    }
    return check_launch("gn_apply");
}

int32_t launch_groupnorm_coef(const float *x, int c, long long spatial, const float *gamma, const float *beta,
                              void *ws, float *coef, hipStream_t s, const floatx4 *rec, int nrec) {
    floatx2 *gstat = gstat_of(ws, c, spatial);
    int32_t rc = groupnorm_stats(x, c, spatial, ws, gstat, s, rec, nrec);
    if (rc != VAE_OK) return rc;
    hipLaunchKernelGGL(gn_coef, dim3((unsigned)((c + kThreads - 1) / kThreads)), dim3(kThreads), 0, s, c,
                       c / kGroups, gstat, gamma, beta, coef);
    return check_launch("gn_coef");
}

int32_t launch_upsample2x(const float *x, int c, int h, int w, float *y, hipStream_t s) {
    const int threads = 256;
    if (w % 2 == 0 && aligned16(y)) {
        const long long pairs = (long long)c * h * (w / 2);
        hipLaunchKernelGGL(upsample2x_pairs, dim3((unsigned)((pairs + threads - 1) / threads)),
                           dim3(threads), 0, s, x, y, h, w, pairs);
    } else {
        const long long total = (long long)c * 4 * h * w;
        hipLaunchKernelGGL(upsample2x_scalar, dim3((unsigned)((total + threads - 1) / threads)),
                           dim3(threads), 0, s, x, y, h, w, total);
    }
    return check_launch("upsample2x");
}


}  // namespace vae
