// gemv_m1.hip -- single-token matrix-vector product for block-quantized weights.
//
// y[n] (+)= sum_k w[n][k] x[k], the weight stream of one decode token
// ([roofline-holds] "The Math": each weight is read once and used for two
// sums, so the product is bound by memory, not by arithmetic).
//
// Geometry (gfx950, wave64):
//   * a workgroup of 4 waves puts x into LDS in its staged form (staging.h):
//     either staging fp32 x itself, or copying x that a producer kernel
//     already staged (XQ), which leaves the workgroup only the dot products;
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
#include "staging.h"

namespace mbq {

// One prefetch slot: a chunk of R rows.
template <int FMT, int R>
struct Slot {
    typename Traits<FMT>::Row row[R];
};

// Pieces of x each thread loads before the first weight load.
constexpr int kXPre = 12;

// Each wave computes R consecutive output rows; lane l takes chunk
// c * 64 + l of each row for c = 0 .. C-1.  CS > 0 fixes C = CS at compile time
// (K = 64 * CS * WPC exactly): every loop is unrolled and every load is
// unconditional, so each wait for loaded data names exactly the loads it
// needs (vector-memory counters retire in order) -- x never waits for
// weights and a chunk never waits for the chunks prefetched after it.
// CS == 0 handles any K with the same steps in runtime loops.
//
// Fusions (static K, fp32 x only):
//   PRO == kProRms: x is replaced by RMSNorm(x) * gamma before staging; each
//     workgroup normalises the whole row in registers (one block-wide sum)
//     while its first weight loads are in flight, so the norm costs no launch
//     ([roofline-holds] "Hiding, fusing, and keeping the sums busy").
//   EPI == kEpiSilu: rows 2i and 2i+1 are the gate and up rows of output i;
//     the wave that computes both writes y[i] = silu(gate) * up.
constexpr int kProNone = 0, kProRms = 1;
constexpr int kEpiStore = 0, kEpiSilu = 1;

template <int FMT, int R, int CS, bool GATHER, bool XQ, int PRO = kProNone, int EPI = kEpiStore>
__global__ __launch_bounds__(kBlock) void gemv_m1_kernel(DevPlanes P, int64_t N, int K,
                                                         const void* __restrict__ xsrc,
                                                         float* __restrict__ y, int accumulate,
                                                         const int32_t* __restrict__ gidx,
                                                         int rpe, const float* __restrict__ gamma,
                                                         float eps) {
    using T = Traits<FMT>;
    static_assert(PRO == kProNone || (CS > 0 && !XQ), "the norm prologue needs static K, fp32 x");
    static_assert(EPI == kEpiStore || R == 2, "the silu epilogue pairs two rows per wave");
    using XP = XPieces<FMT, XQ>;
    constexpr int D = 2;                                      // chunk steps in flight
    extern __shared__ float4 smem[];
    uint32_t* xs = (uint32_t*)smem;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int nchunks = K / T::WPC;
    const int C = CS > 0 ? CS : (nchunks + kWave - 1) / kWave;
    const int64_t row0 = ((int64_t)blockIdx.x * kWavesPerBlock + wave) * R;

    // ---- x: the first pieces, before any weight load
    const uint4* xsrc4 = (const uint4*)xsrc;
    const int npieces = XP::count(K);
    constexpr int GF4 = XP::GF4;
    constexpr int NR = 4;                                     // pieces per runtime round
    // pieces per thread: all of them (static K), or the first round
    constexpr int NX = CS > 0 ? (XQ ? CS * T::F4 / 4 : CS * T::WPC / 16) : NR;
    static_assert(NX <= kXPre && NX % GF4 == 0, "x pieces per thread");
    uint4 xr[NX];
#pragma unroll
    for (int i = 0; i < NX; i++) xr[i] = XP::load(xsrc4, i, npieces);
    uint4 gr[PRO == kProRms ? NX : 1];
    if constexpr (PRO == kProRms) {
#pragma unroll
        for (int i = 0; i < NX; i++) gr[i] = XP::load((const uint4*)gamma, i, npieces);
    }

    // ---- y for an accumulating product (one load per lane, unconditional)
    const int64_t yrow = row0 + (lane < R ? lane : 0);
    const float yin = y[yrow < N ? yrow : N - 1];

    // ---- weight rows: rows past N re-read row N-1 (their results are not stored)
    DevPlanes base[R];
#pragma unroll
    for (int r = 0; r < R; r++) {
        int64_t n = row0 + r < N ? row0 + r : N - 1;
        if constexpr (GATHER) {
            const int e = (int)(n / rpe);
            n = (int64_t)gidx[e] * rpe + (n - (int64_t)e * rpe);
        }
        base[r] = T::base(P, n, K);
    }
    auto load = [&](Slot<FMT, R>& sl, int c) {
        const int b = c * kWave + lane;
        const int bb = b < nchunks ? b : 0;
#pragma unroll
        for (int r = 0; r < R; r++) T::load(sl.row[r], base[r], bb);
    };

    float acc[R];
#pragma unroll
    for (int r = 0; r < R; r++) acc[r] = 0.f;
    auto compute = [&](const Slot<FMT, R>& sl, int c) {
        const int b = c * kWave + lane;
        const bool ok = b < nchunks;
        uint32_t xv[4 * T::F4];
        read_x<FMT>(xs, ok ? b : 0, xv);
        if constexpr (T::INT) {
            xv[T::META] = ok ? xv[T::META] : 0u;    // lanes past the row add exactly 0
#pragma unroll
            for (int r = 0; r < R; r++) acc[r] += T::dot(sl.row[r], xv);
        } else {
#pragma unroll
            for (int r = 0; r < R; r++) {
                const float v = T::dot(sl.row[r], xv);
                acc[r] += ok ? v : 0.f;
            }
        }
    };

    if constexpr (CS > 0) {
        // All of the row's chunks in flight when they fit (C <= 2), else D.
        constexpr int DD = CS <= 2 ? CS : D;
        Slot<FMT, R> buf[DD];
#pragma unroll
        for (int d = 0; d < DD; d++) load(buf[d], d);
        if constexpr (PRO == kProRms) {
            // RMSNorm of the row, as the stand-alone kernel: y = g * (x * inv)
            __shared__ float red[kWavesPerBlock];
            float ss = 0.f;
#pragma unroll
            for (int i = 0; i < NX; i++) {
                const float4 v = __builtin_bit_cast(float4, xr[i]);
                ss = fmaf(v.x, v.x, ss);
                ss = fmaf(v.y, v.y, ss);
                ss = fmaf(v.z, v.z, ss);
                ss = fmaf(v.w, v.w, ss);
            }
            const float inv = 1.0f / sqrtf(block_sum(ss, red) / (float)K + eps);
#pragma unroll
            for (int i = 0; i < NX; i++) {
                const float4 v = __builtin_bit_cast(float4, xr[i]);
                const float4 g = __builtin_bit_cast(float4, gr[i]);
                xr[i] = __builtin_bit_cast(uint4, make_float4(g.x * (v.x * inv), g.y * (v.y * inv),
                                                              g.z * (v.z * inv), g.w * (v.w * inv)));
            }
        }
        XP::template store<NX, true>(xr, 0, npieces, xs);
        __syncthreads();
#pragma unroll
        for (int c = 0; c < CS; c++) {
            compute(buf[c % DD], c);
            if (c + DD < CS) load(buf[c % DD], c + DD);
        }
    } else {
        Slot<FMT, R> buf[D];
#pragma unroll
        for (int d = 0; d < D; d++) load(buf[d], d < C ? d : 0);
        XP::template store<NX, false>(xr, 0, npieces, xs);
        // later rounds of x (their loads follow the weights' in the queue)
        const int npt = XQ ? (npieces + kBlock - 1) / kBlock
                           : (npieces / GF4 + kBlock - 1) / kBlock * GF4;
        for (int i0 = NX; i0 < npt; i0 += NR) {
            uint4 xt[NR];
#pragma unroll
            for (int i = 0; i < NR; i++) xt[i] = XP::load(xsrc4, i0 + i, npieces);
            XP::template store<NR, false>(xt, i0, npieces, xs);
        }
        __syncthreads();
        for (int c = 0; c < C; c += D) {
#pragma unroll
            for (int d = 0; d < D; d++) {
                if (c + d < C) {
                    compute(buf[d], c + d);
                    load(buf[d], c + d + D < C ? c + d + D : 0);
                }
            }
        }
    }

    if constexpr (EPI == kEpiSilu) {
        const float g = wave_sum_dpp(acc[0]), u = wave_sum_dpp(acc[1]);
        if (lane == 0 && row0 + 1 < N) y[row0 / 2] = g / (1.0f + expf(-g)) * u;
    } else {
#pragma unroll
        for (int r = 0; r < R; r++) {
            const float s = wave_sum_dpp(acc[r]);
            if (lane == r && row0 + r < N) y[row0 + r] = (accumulate ? yin : 0.f) + s;
        }
    }
}

// Chunk steps per row fixed at compile time for the decode shapes: K = 4096
// and 12288 for the 32-weight chunks, 4096 for Q25 and BF16.
template <int FMT>
constexpr int static_steps(int64_t K) {
    constexpr int per = 64 * Traits<FMT>::WPC;
    if (FMT == kQ45 || FMT == kQ65) return K == 2 * per ? 2 : K == 6 * per ? 6 : 0;
    if (FMT == kQ25) return K == per ? 1 : 0;
    return K == 8 * per ? 8 : 0;
}

struct M1Args {
    DevPlanes P;
    int64_t N, K;
    const void* x;
    float* y;
    int accumulate;
    const int32_t* gidx;
    int64_t rpe;
    const float* gamma;
    float eps;
};

template <int FMT, int R, int CS, bool GATHER, bool XQ, int PRO = kProNone, int EPI = kEpiStore>
static hipError_t launch_k(const M1Args& a, hipStream_t stream) {
    using T = Traits<FMT>;
    const int64_t rows_per_wg = (int64_t)kWavesPerBlock * R;
    const int64_t grid = (a.N + rows_per_wg - 1) / rows_per_wg;
    const size_t lds = (size_t)(a.K / T::WPC) * Stride<FMT>::DW * 4;
    auto kern = gemv_m1_kernel<FMT, R, CS, GATHER, XQ, PRO, EPI>;
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)kern,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kBlock), lds, stream, a.P, a.N, (int)a.K,
                       a.x, a.y, a.accumulate, a.gidx, (int)a.rpe, a.gamma, a.eps);
    return hipGetLastError();
}

template <int FMT, int R, int CS>
static hipError_t launch_c(const M1Args& a, bool xq, hipStream_t s) {
    // BF16's staged x is x itself (fp32, chunks back to back).
    if constexpr (Traits<FMT>::INT) {
        if (xq) return a.gidx ? launch_k<FMT, R, CS, true, true>(a, s) : launch_k<FMT, R, CS, false, true>(a, s);
    }
    return a.gidx ? launch_k<FMT, R, CS, true, false>(a, s) : launch_k<FMT, R, CS, false, false>(a, s);
}

template <int FMT, int R>
static hipError_t launch_r(const M1Args& a, bool xq, hipStream_t s) {
    switch (static_steps<FMT>(a.K)) {
    case 1: if constexpr (FMT == kQ25) return launch_c<FMT, R, 1>(a, xq, s); break;
    case 2: if constexpr (FMT == kQ45 || FMT == kQ65) return launch_c<FMT, R, 2>(a, xq, s); break;
    case 6: if constexpr (FMT == kQ45 || FMT == kQ65) return launch_c<FMT, R, 6>(a, xq, s); break;
    case 8: if constexpr (FMT == kBF16) return launch_c<FMT, R, 8>(a, xq, s); break;
    default: break;
    }
    return launch_c<FMT, R, 0>(a, xq, s);
}

template <int FMT>
static hipError_t launch_f(const M1Args& a, bool xq, GemvGeom geom, hipStream_t s) {
    switch (geom.rows_per_wave) {
    case 1: return launch_r<FMT, 1>(a, xq, s);
    case 2: return launch_r<FMT, 2>(a, xq, s);
    default: return launch_r<FMT, 4>(a, xq, s);
    }
}

// Default rows per wave, from cold-cache sweeps on MI355X: many small
// workgroups hide latency better than few large ones, so R = 2 only for the
// larger tables.
GemvGeom gemv_m1_default_geom(int fmt, int64_t N, int64_t K) {
    (void)fmt;
    GemvGeom g;
    g.rows_per_wave = N >= 65536 ? 4 : N * K >= ((int64_t)32 << 20) ? 2 : 1;
    return g;
}

hipError_t launch_gemv_m1(int fmt, DevPlanes P, int64_t N_out, int64_t K, const void* x,
                          bool x_staged, float* y, int accumulate, const int32_t* gidx,
                          int64_t rpe, GemvGeom geom, hipStream_t stream) {
    const M1Args a{P, N_out, K, x, y, accumulate, gidx, rpe, nullptr, 0.f};
    switch (fmt) {
    case kQ45: return launch_f<kQ45>(a, x_staged, geom, stream);
    case kQ65: return launch_f<kQ65>(a, x_staged, geom, stream);
    case kQ25: return launch_f<kQ25>(a, x_staged, geom, stream);
    case kBF16: return launch_f<kBF16>(a, x_staged, geom, stream);
    }
    return hipErrorInvalidValue;
}

// ---- fused products ---------------------------------------------------
template <int FMT, int CS, int PRO>
static hipError_t launch_fused_cs(const M1Args& a, bool silu, int rows, hipStream_t s) {
    if (silu) return launch_k<FMT, 2, CS, false, false, PRO, kEpiSilu>(a, s);
    switch (rows) {
    case 1: return launch_k<FMT, 1, CS, false, false, PRO, kEpiStore>(a, s);
    case 2: return launch_k<FMT, 2, CS, false, false, PRO, kEpiStore>(a, s);
    default: return launch_k<FMT, 4, CS, false, false, PRO, kEpiStore>(a, s);
    }
}

template <int FMT>
static hipError_t launch_fused_f(const M1Args& a, bool norm, bool silu, int rows, hipStream_t s) {
    switch (static_steps<FMT>(a.K)) {
    case 2:
        return norm ? launch_fused_cs<FMT, 2, kProRms>(a, silu, rows, s)
                    : launch_fused_cs<FMT, 2, kProNone>(a, silu, rows, s);
    case 6:
        return norm ? launch_fused_cs<FMT, 6, kProRms>(a, silu, rows, s)
                    : launch_fused_cs<FMT, 6, kProNone>(a, silu, rows, s);
    default: return hipErrorNotSupported;
    }
}

bool gemv_fused_supported(int fmt, int64_t K) {
    if (fmt == kQ45) return static_steps<kQ45>(K) == 2 || static_steps<kQ45>(K) == 6;
    if (fmt == kQ65) return static_steps<kQ65>(K) == 2 || static_steps<kQ65>(K) == 6;
    return false;
}

hipError_t launch_gemv_fused(int fmt, DevPlanes P, int64_t N, int64_t K, const float* x,
                             const float* gamma, float eps, bool silu, float* y, int accumulate,
                             GemvGeom geom, hipStream_t stream) {
    const M1Args a{P, N, K, x, y, accumulate, nullptr, 1, gamma, eps};
    const bool norm = gamma != nullptr;
    switch (fmt) {
    case kQ45: return launch_fused_f<kQ45>(a, norm, silu, geom.rows_per_wave, stream);
    case kQ65: return launch_fused_f<kQ65>(a, norm, silu, geom.rows_per_wave, stream);
    }
    return hipErrorNotSupported;
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
