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

// x staging.  Each thread moves XR float4 of x per round from global memory
// into LDS.  The first round's loads are issued before any weight load, so
// waiting for them never waits for weights (vector-memory counters retire in
// order).  A round is XR/(GX/4) groups of GX values per thread, four threads
// per chunk.  For the quantized formats each group is rounded to 24-bit fixed
// point with the chunk's exponent and written as digit words (formats.h); the
// chunk's exponent and offset terms come from lane shuffles.  For BF16 x is
// stored as fp32.  Dword d of chunk b lives at b * Stride::DW + d.
constexpr int XR = 4;

template <int FMT>
__device__ __forceinline__ void x_load(const float* __restrict__ x, int nf4, int round, float4* xr) {
    constexpr int GF4 = Traits<FMT>::GX / 4;     // float4 per group
    constexpr int XG = XR / GF4;                 // groups per thread per round
#pragma unroll
    for (int i = 0; i < XG; i++) {
        const int og = (round * XG + i) * kBlock + (int)threadIdx.x;
#pragma unroll
        for (int j = 0; j < GF4; j++) {
            const int f = og * GF4 + j;
            xr[i * GF4 + j] = f < nf4 ? ((const float4*)x)[f] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
}

template <int FMT>
__device__ __forceinline__ void lds_put(uint32_t* xs, int b, int d, uint32_t v) {
    xs[Stride<FMT>::DW * b + d] = v;
}

template <int FMT>
__device__ __forceinline__ void x_store(int nf4, int round, const float4* xr, uint32_t* xs) {
    using T = Traits<FMT>;
    constexpr int GX = T::GX, GF4 = GX / 4, XG = XR / GF4;
    const int ngroups = nf4 / GF4;
#pragma unroll
    for (int i = 0; i < XG; i++) {
        const int og = (round * XG + i) * kBlock + (int)threadIdx.x;
        const bool ok = og < ngroups;
        const float* v = (const float*)(xr + i * GF4);
        constexpr int GPC = T::WPC / GX;      // groups per chunk: 4 (1 for BF16)
        const int b = og / GPC, gi = og % GPC;   // chunk, group within chunk
        if constexpr (!T::INT) {
#pragma unroll
            for (int j = 0; j < GX; j++)
                if (ok) lds_put<FMT>(xs, b, GX * gi + j, __builtin_bit_cast(uint32_t, v[j]));
        } else {
            float amax = 0.f;
#pragma unroll
            for (int k = 0; k < GX; k++) amax = fmaxf(amax, fabsf(v[k]));
            amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
            amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
            const int e = chunk_exp(amax);
            const float up = pow2f(e);
            int32_t n[GX];
#pragma unroll
            for (int k = 0; k < GX; k++) n[k] = round_fixed(v[k], up);
            // digit words of the group's code vectors
            constexpr int NV = GX / 4;            // code vectors per group
            uint32_t dg[3 * NV];
#pragma unroll
            for (int m = 0; m < NV; m++) {
                // Q45/Q65 octet: vector 0 = even values, 1 = odd values.
                // Q25 group of 16: vector m = values m, 4+m, 8+m, 12+m.
                const int s0 = (GX == 8) ? m : m, st = (GX == 8) ? 2 : 4;
                digit_words(n[s0], n[s0 + st], n[s0 + 2 * st], n[s0 + 3 * st], dg + 3 * m);
            }
            // digit sums of the group, then of its offset block
            int32_t S[3] = {0, 0, 0};
#pragma unroll
            for (int m = 0; m < NV; m++) {
                S[0] += (int32_t)udot4(dg[3 * m], 0x01010101u, 0u);
                S[1] += (int32_t)udot4(dg[3 * m + 1], 0x01010101u, 0u);
                S[2] = sdot4(dg[3 * m + 2], 0x01010101u, S[2]);
            }
            int32_t B01[3], B23[3];
#pragma unroll
            for (int p = 0; p < 3; p++) {
                B01[p] = S[p] + __shfl_xor(S[p], 1, kWave);     // groups 0+1 (or 2+3)
                B23[p] = __shfl_xor(B01[p], 2, kWave);         // the other pair
            }
            if (ok) {
                uint32_t* dst = xs + Stride<FMT>::DW * b + 3 * NV * gi;   // 8-byte aligned
#pragma unroll
                for (int t = 0; t < 3 * NV; t += 2) *(uint2*)(dst + t) = make_uint2(dg[t], dg[t + 1]);
                if (gi == 0) {
                    lds_put<FMT>(xs, b, T::META, __builtin_bit_cast(uint32_t, pow2f(-e)));
                    if constexpr (T::BLK == 32 && T::WPC == 32) {   // one block per chunk
#pragma unroll
                        for (int p = 0; p < 3; p++)
                            lds_put<FMT>(xs, b, T::META + 1 + p, (uint32_t)(-T::OFF * (B01[p] + B23[p])));
                    } else {                                          // two blocks per chunk
#pragma unroll
                        for (int p = 0; p < 3; p++) {
                            lds_put<FMT>(xs, b, T::META + 1 + p, (uint32_t)(-T::OFF * B01[p]));
                            lds_put<FMT>(xs, b, T::META + 4 + p, (uint32_t)(-T::OFF * B23[p]));
                        }
                    }
                }
            }
        }
    }
}

template <int FMT>
__device__ __forceinline__ void read_x(const uint32_t* xs, int b, uint32_t* xv) {
    using T = Traits<FMT>;
    const uint32_t* src = xs + Stride<FMT>::DW * b;
#pragma unroll
    for (int j = 0; j < T::F4; j++) {
        const uint4 v = *(const uint4*)(src + 4 * j);
        xv[4 * j + 0] = v.x;
        xv[4 * j + 1] = v.y;
        xv[4 * j + 2] = v.z;
        xv[4 * j + 3] = v.w;
    }
}

// One prefetch slot: a chunk of R rows.
template <int FMT, int R>
struct Slot {
    typename Traits<FMT>::Row row[R];
};

template <int FMT, int R, int D, bool GATHER>
__global__ __launch_bounds__(kBlock) void gemv_m1_kernel(DevPlanes P, int64_t N, int K,
                                                         const float* __restrict__ x,
                                                         float* __restrict__ y, int accumulate,
                                                         int groups,
                                                         const int32_t* __restrict__ gidx,
                                                         int rpe) {
    using T = Traits<FMT>;
    extern __shared__ float4 smem[];
    uint32_t* xs = (uint32_t*)smem;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int nf4 = K >> 2;
    const int nchunks = K / T::WPC;
    const int C = (nchunks + kWave - 1) / kWave;   // chunk steps per row
    const int U = groups * C;                      // units (group, chunk) per wave
    const int64_t row0 = (int64_t)blockIdx.x * groups * (kWavesPerBlock * R) + wave * R;
    const int64_t gstride = kWavesPerBlock * R;

    float4 xr[XR];
    x_load<FMT>(x, nf4, 0, xr);

    // ---- load cursor: weight-row bases of the group being loaded.  Output
    // rows past N re-read row N-1 (their results are not stored).
    // When the load cursor enters a group, the y values an accumulating
    // product adds to are requested before that group's weights, so waiting
    // for them never waits for weight loads.
    DevPlanes base[R];
    float ynext[R];
    int lg = 0, lc = 0;
    auto set_rows = [&](int g) {
        const int64_t nb = row0 + (int64_t)g * gstride;
#pragma unroll
        for (int r = 0; r < R; r++) {
            int64_t n = nb + r < N ? nb + r : N - 1;
            ynext[r] = (accumulate && lane == r && nb + r < N) ? y[nb + r] : 0.f;
            if constexpr (GATHER) {
                const int e = (int)(n / rpe);
                n = (int64_t)gidx[e] * rpe + (n - (int64_t)e * rpe);
            }
            base[r] = T::base(P, n, K);
        }
    };
    auto load_next = [&](Slot<FMT, R>& sl) {
        const int b = lc * kWave + lane;
        const int bb = b < nchunks ? b : 0;
#pragma unroll
        for (int r = 0; r < R; r++) T::load(sl.row[r], base[r], bb);
        if (++lc == C) {
            lc = 0;
            if (++lg < groups) set_rows(lg);
        }
    };

    Slot<FMT, R> buf[D];
    set_rows(0);
#pragma unroll
    for (int d = 0; d < D; d++)
        if (d < U) load_next(buf[d]);

    const int rounds = (nf4 + XR * kBlock - 1) / (XR * kBlock);
    x_store<FMT>(nf4, 0, xr, xs);
    for (int rd = 1; rd < rounds; rd++) {
        x_load<FMT>(x, nf4, rd, xr);
        x_store<FMT>(nf4, rd, xr, xs);
    }
    __syncthreads();

    // ---- compute cursor
    int g = 0, c = 0;
    float acc[R], yold[R];
#pragma unroll
    for (int r = 0; r < R; r++) yold[r] = 0.f;
    auto compute = [&](const Slot<FMT, R>& sl) {
        if (c == 0) {
            // With C >= D the load cursor is still inside this group, so
            // ynext holds its y; otherwise it has moved on and y is read now.
            const int64_t nb = row0 + (int64_t)g * gstride;
#pragma unroll
            for (int r = 0; r < R; r++) {
                acc[r] = 0.f;
                if (C >= D)
                    yold[r] = ynext[r];
                else
                    yold[r] = (accumulate && lane == r && nb + r < N) ? y[nb + r] : 0.f;
            }
        }
        const int b = c * kWave + lane;
        const bool ok = b < nchunks;
        uint32_t xv[4 * T::F4];
        read_x<FMT>(xs, ok ? b : 0, xv);
        if constexpr (T::INT) {
            // lanes past the last chunk contribute exactly zero (scale 0)
            xv[T::META] = ok ? xv[T::META] : 0u;
#pragma unroll
            for (int r = 0; r < R; r++) acc[r] += T::dot(sl.row[r], xv);
        } else {
#pragma unroll
            for (int r = 0; r < R; r++) {
                const float v = T::dot(sl.row[r], xv);
                acc[r] += ok ? v : 0.f;
            }
        }
        if (c == C - 1) {
            const int64_t nb = row0 + (int64_t)g * gstride;
#pragma unroll
            for (int r = 0; r < R; r++) {
                const float s = wave_sum_dpp(acc[r]);
                if (lane == r && nb + r < N) y[nb + r] = yold[r] + s;
            }
        }
        if (++c == C) {
            c = 0;
            ++g;
        }
    };
    for (int u = 0; u < U; u += D) {
#pragma unroll
        for (int d = 0; d < D; d++) {
            if (u + d < U) {
                compute(buf[d]);
                if (u + d + D < U) load_next(buf[d]);
            }
        }
    }
}

template <int FMT, int R, int D, bool GATHER>
static hipError_t launch_frg(DevPlanes P, int64_t N, int64_t K, const float* x, float* y,
                             int accumulate, const int32_t* gidx, int64_t rpe, int groups,
                             hipStream_t stream) {
    using T = Traits<FMT>;
    const int64_t rows_per_wg = (int64_t)groups * kWavesPerBlock * R;
    const int64_t grid = (N + rows_per_wg - 1) / rows_per_wg;
    const size_t lds = (size_t)(K / T::WPC) * Stride<FMT>::DW * 4;
    auto kern = gemv_m1_kernel<FMT, R, D, GATHER>;
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)kern,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kBlock), lds, stream, P, N, (int)K, x,
                       y, accumulate, groups, gidx, (int)rpe);
    return hipGetLastError();
}

template <int FMT, int R, int D>
static hipError_t launch_frd(DevPlanes P, int64_t N, int64_t K, const float* x, float* y,
                             int accumulate, const int32_t* gidx, int64_t rpe, int groups,
                             hipStream_t stream) {
    if (gidx) return launch_frg<FMT, R, D, true>(P, N, K, x, y, accumulate, gidx, rpe, groups, stream);
    return launch_frg<FMT, R, D, false>(P, N, K, x, y, accumulate, gidx, rpe, groups, stream);
}

template <int FMT, int R>
static hipError_t launch_fr(DevPlanes P, int64_t N, int64_t K, const float* x, float* y,
                            int accumulate, const int32_t* gidx, int64_t rpe, int groups,
                            int prefetch, hipStream_t stream) {
    if (prefetch >= 4) return launch_frd<FMT, R, 4>(P, N, K, x, y, accumulate, gidx, rpe, groups, stream);
    return launch_frd<FMT, R, 2>(P, N, K, x, y, accumulate, gidx, rpe, groups, stream);
}

template <int FMT>
static hipError_t launch_f(DevPlanes P, int64_t N, int64_t K, const float* x, float* y,
                           int accumulate, const int32_t* gidx, int64_t rpe, GemvGeom geom,
                           hipStream_t stream) {
    const int G = geom.groups_per_wg, D = geom.prefetch;
    switch (geom.rows_per_wave) {
    case 1: return launch_fr<FMT, 1>(P, N, K, x, y, accumulate, gidx, rpe, G, D, stream);
    case 2: return launch_fr<FMT, 2>(P, N, K, x, y, accumulate, gidx, rpe, G, D, stream);
    default: return launch_fr<FMT, 4>(P, N, K, x, y, accumulate, gidx, rpe, G, D, stream);
    }
}

// Default geometry, from cold-cache sweeps on MI355X (rows per wave R, row
// groups per workgroup G, units in flight D): many small workgroups hide
// latency better than few large ones, so R = 2 above 2048 rows.
GemvGeom gemv_m1_default_geom(int fmt, int64_t N, int64_t K) {
    (void)fmt;
    (void)K;
    GemvGeom g;
    g.prefetch = 2;
    g.groups_per_wg = 1;
    g.rows_per_wave = N >= 2048 ? 2 : 1;
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
