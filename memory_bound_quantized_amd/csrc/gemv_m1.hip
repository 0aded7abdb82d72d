// gemv_m1.hip -- single-token matrix-vector product for block-quantized weights.
//
// y[n] (+)= sum_k w[n][k] x[k], the weight stream of one decode token
// ([roofline-holds] "The Math": each weight is read once and used for two
// sums, so the product is bound by memory, not by arithmetic).
//
// Geometry (gfx950, wave64):
//   * a workgroup of 4 waves stages x (fp32) once into LDS, together with the
//     per-block sums of x that fold the code offset out of the inner loop;
//   * each wave owns R rows at a time; lane l reads chunk c*64 + l of each row
//     (16 code bytes + its scales), so one load instruction of a wave is a
//     1 KiB coalesced burst ([mountain-runs] section 3);
//   * chunks are double-buffered in registers: the loads of the next chunk are
//     issued before the current one is unpacked, and the first chunk's loads
//     are issued before x is staged, so bytes are in flight from the first
//     cycles ([roofline-holds] "Little and Volkov": a kernel must keep
//     bandwidth x latency bytes in flight);
//   * the R row sums are reduced across the wave and written by lanes 0..R-1.
// Gathered experts reuse the kernel with an output-row -> weight-row map.
#include "device_common.h"
#include "formats.h"
#include "kernels.h"

namespace mbq {

// Stage x[0..K) into LDS (swizzled per chunk) and write the folded block
// sums  mbs[i] = -offset * sum(x over block-sum group i).
template <int FMT>
__device__ __forceinline__ void stage_x(const float* __restrict__ x, int K, float4* xs,
                                        float* mbs) {
    using T = Traits<FMT>;
    const int nf4 = K >> 2;
    for (int base = 0; base < nf4; base += kBlock) {
        const int f = base + (int)threadIdx.x;
        const bool ok = f < nf4;
        const float4 v = ok ? ((const float4*)x)[f] : make_float4(0.f, 0.f, 0.f, 0.f);
        if (ok) xs[x_slot<FMT>(f / T::F4, f % T::F4)] = v;
        if constexpr (T::NBS > 0) {
            const float s = group_sum<T::BSG>((v.x + v.y) + (v.z + v.w));
            if (ok && (f % T::BSG) == 0) mbs[f / T::BSG] = -T::OFF * s;
        }
    }
}

template <int FMT>
__device__ __forceinline__ void read_x(const float4* xs, const float* mbs, int b, float* xv,
                                       float* mb) {
    using T = Traits<FMT>;
#pragma unroll
    for (int j = 0; j < T::F4; j++) {
        const float4 v = xs[x_slot<FMT>(b, j)];
        xv[4 * j + 0] = v.x;
        xv[4 * j + 1] = v.y;
        xv[4 * j + 2] = v.z;
        xv[4 * j + 3] = v.w;
    }
#pragma unroll
    for (int i = 0; i < (T::NBS > 0 ? T::NBS : 1); i++) mb[i] = T::NBS > 0 ? mbs[T::NBS * b + i] : 0.f;
}

template <int FMT, int R, bool GATHER>
__global__ __launch_bounds__(kBlock) void gemv_m1_kernel(DevPlanes P, int64_t N, int K,
                                                         const float* __restrict__ x,
                                                         float* __restrict__ y, int accumulate,
                                                         int groups,
                                                         const int32_t* __restrict__ gidx,
                                                         int rpe) {
    using T = Traits<FMT>;
    using Row = typename T::Row;
    extern __shared__ float4 smem[];
    float4* xs = smem;
    float* mbs = (float*)(smem + (K >> 2));

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int nchunks = K / T::WPC;
    const int C = (nchunks + kWave - 1) / kWave;   // chunk steps per row
    const int U = groups * C;                      // units (group, chunk) per wave
    const int64_t row0 = (int64_t)blockIdx.x * groups * (kWavesPerBlock * R) + wave * R;

    // Weight-row bases of the group whose chunks are being loaded.  Output
    // rows past N re-read row N-1 (their results are not stored).
    DevPlanes base[R];
    auto set_rows = [&](int g) {
        const int64_t nb = row0 + (int64_t)g * (kWavesPerBlock * R);
#pragma unroll
        for (int r = 0; r < R; r++) {
            int64_t n = nb + r < N ? nb + r : N - 1;
            if constexpr (GATHER) {
                const int e = (int)(n / rpe);
                n = (int64_t)gidx[e] * rpe + (n - (int64_t)e * rpe);
            }
            base[r] = T::base(P, n, K);
        }
    };
    auto load_unit = [&](Row* u, int c) {
        const int b = c * kWave + lane;
        const int bb = b < nchunks ? b : 0;
#pragma unroll
        for (int r = 0; r < R; r++) T::load(u[r], base[r], bb);
    };

    Row bufA[R], bufB[R];
    float acc[R], yold[R];
    set_rows(0);
    load_unit(bufA, 0);
    stage_x<FMT>(x, K, xs, mbs);
    __syncthreads();

    int g = 0, c = 0;
    auto step = [&](Row* cur, Row* nxt, int u) {
        int gn = g, cn = c + 1;
        if (cn == C) {
            cn = 0;
            gn = g + 1;
        }
        if (u + 1 < U) {
            if (cn == 0) set_rows(gn);
            load_unit(nxt, cn);
        }
        const int64_t nb = row0 + (int64_t)g * (kWavesPerBlock * R);
        if (c == 0) {
#pragma unroll
            for (int r = 0; r < R; r++) {
                acc[r] = 0.f;
                yold[r] = 0.f;
                if (accumulate && lane == r && nb + r < N) yold[r] = y[nb + r];
            }
        }
        const int b = c * kWave + lane;
        const bool ok = b < nchunks;
        float xv[T::WPC];
        float mb[T::NBS > 0 ? T::NBS : 1];
        read_x<FMT>(xs, mbs, ok ? b : 0, xv, mb);
#pragma unroll
        for (int r = 0; r < R; r++) {
            const float v = T::dot(cur[r], xv, mb);
            acc[r] += ok ? v : 0.f;
        }
        if (c == C - 1) {
#pragma unroll
            for (int r = 0; r < R; r++) {
                const float s = wave_sum(acc[r]);
                if (lane == r && nb + r < N) y[nb + r] = yold[r] + s;
            }
        }
        g = gn;
        c = cn;
    };
    for (int u = 0; u < U; u += 2) {
        step(bufA, bufB, u);
        if (u + 1 < U) step(bufB, bufA, u + 1);
    }
}

template <int FMT, int R, bool GATHER>
static hipError_t launch_frg(DevPlanes P, int64_t N, int64_t K, const float* x, float* y,
                             int accumulate, const int32_t* gidx, int64_t rpe, int groups,
                             hipStream_t stream) {
    using T = Traits<FMT>;
    const int64_t rows_per_wg = (int64_t)groups * kWavesPerBlock * R;
    const int64_t grid = (N + rows_per_wg - 1) / rows_per_wg;
    const size_t lds = (size_t)K * 4 + (size_t)(T::NBS > 0 ? (K / T::WPC) * T::NBS : 0) * 4;
    auto kern = gemv_m1_kernel<FMT, R, GATHER>;
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)kern,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kBlock), lds, stream, P, N, (int)K, x,
                       y, accumulate, groups, gidx, (int)rpe);
    return hipGetLastError();
}

template <int FMT, int R>
static hipError_t launch_fr(DevPlanes P, int64_t N, int64_t K, const float* x, float* y,
                            int accumulate, const int32_t* gidx, int64_t rpe, int groups,
                            hipStream_t stream) {
    if (gidx) return launch_frg<FMT, R, true>(P, N, K, x, y, accumulate, gidx, rpe, groups, stream);
    return launch_frg<FMT, R, false>(P, N, K, x, y, accumulate, gidx, rpe, groups, stream);
}

template <int FMT>
static hipError_t launch_f(DevPlanes P, int64_t N, int64_t K, const float* x, float* y,
                           int accumulate, const int32_t* gidx, int64_t rpe, GemvGeom geom,
                           hipStream_t stream) {
    switch (geom.rows_per_wave) {
    case 1: return launch_fr<FMT, 1>(P, N, K, x, y, accumulate, gidx, rpe, geom.groups_per_wg, stream);
    case 2: return launch_fr<FMT, 2>(P, N, K, x, y, accumulate, gidx, rpe, geom.groups_per_wg, stream);
    default: return launch_fr<FMT, 4>(P, N, K, x, y, accumulate, gidx, rpe, geom.groups_per_wg, stream);
    }
}

GemvGeom gemv_m1_default_geom(int fmt, int64_t N, int64_t K) {
    (void)fmt;
    (void)K;
    GemvGeom g;
    if (N >= 8192) {
        g.rows_per_wave = 4;
        g.groups_per_wg = N >= 65536 ? 4 : 1;
    } else if (N >= 2048) {
        g.rows_per_wave = 2;
        g.groups_per_wg = 1;
    } else {
        g.rows_per_wave = 1;
        g.groups_per_wg = 1;
    }
    return g;
}

hipError_t launch_gemv_m1(int fmt, DevPlanes P, int64_t N_out, int64_t K, const float* x,
                          float* y, int accumulate, const int32_t* gidx, int64_t rpe,
                          GemvGeom geom, hipStream_t stream) {
    switch (fmt) {
    case kQ45: return launch_f<kQ45>(P, N_out, K, x, y, accumulate, gidx, rpe, geom, stream);
    case kQ65: return launch_f<kQ65>(P, N_out, K, x, y, accumulate, gidx, rpe, geom, stream);
    case kQ25: return launch_f<kQ25>(P, N_out, K, x, y, accumulate, gidx, rpe, geom, stream);
    case kBF16: return launch_f<kBF16>(P, N_out, K, x, y, accumulate, gidx, rpe, geom, stream);
    }
    return hipErrorInvalidValue;
}

// y[m][n] = 0, n < N (the K == 0 product).
__global__ __launch_bounds__(kBlock) void fill_zero_kernel(float* y, int64_t M, int64_t N,
                                                           int64_t ldy) {
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i < M * N) y[(i / N) * ldy + (i % N)] = 0.f;
}

hipError_t launch_fill_zero(float* y, int64_t M, int64_t N, int64_t ldy, hipStream_t stream) {
    const int64_t total = M * N;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((total + kBlock - 1) / kBlock)),
                       dim3(kBlock), 0, stream, y, M, N, ldy);
    return hipGetLastError();
}

}  // namespace mbq
