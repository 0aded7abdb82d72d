// gemv_smallm.hip -- Y[m][n] (+)= W[n] . X[m] for 2 <= M <= 8 tokens, on the
// vector units.
//
// Several tokens against one weight stream: each weight read from memory
// serves M sums, so the bytes per token fall as 1/M until the arithmetic
// catches up with the memory ([roofline-holds] "The Math": the crossover
// M* = (w/16)(R/BW); below it memory is the wall).  The kernel is the M = 1
// kernel with the unpack hoisted out of the token loop: a wave unpacks its R
// rows' codes once per chunk and runs the integer-digit dot products
// (formats.h) against the staged x of every token, all M x chunks staged in
// LDS.
#include "device_common.h"
#include "formats.h"
#include "kernels.h"
#include "staging.h"

namespace mbq {

template <int FMT, int R>
struct SlotM {
    typename Traits<FMT>::Row row[R];
};

// CS > 0: K = 64 * CS * WPC, every loop unrolled (see gemv_m1.hip).  Row sums
// follow the single-token kernel's order, so each token's row is bit-identical
// to its M = 1 product.
template <int FMT, int R, int M, int CS, bool XQ>
__global__ __launch_bounds__(kBlock) void gemv_smallm_kernel(DevPlanes P, int64_t N, int K,
                                                             const void* __restrict__ xsrc,
                                                             int64_t ldx, float* __restrict__ y,
                                                             int64_t ldy, int accumulate) {
    using T = Traits<FMT>;
    using XP = XPieces<FMT, XQ>;
    constexpr int D = 2;
    constexpr int GF4 = XP::GF4;
    extern __shared__ float4 smem[];
    uint32_t* xs = (uint32_t*)smem;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int nchunks = K / T::WPC;
    const int C = CS > 0 ? CS : (nchunks + kWave - 1) / kWave;
    const int64_t row0 = ((int64_t)blockIdx.x * kWavesPerBlock + wave) * R;
    const int npieces = XP::count(K);
    const int xs_row = nchunks * Stride<FMT>::DW;       // LDS dwords per token
    // 16-byte pieces of token m: fp32 rows ldx floats apart, staged rows K dwords apart
    auto xrow = [&](int m) {
        return (const uint4*)xsrc + (XQ ? (int64_t)m * K / 4 : (int64_t)m * ldx / 4);
    };

    // ---- x of every token: static K loads all pieces before the weights
    constexpr int NX = CS > 0 ? (XQ ? CS * T::F4 / 4 : CS * T::WPC / 16) : 4;
    constexpr bool PRE = CS > 0 && NX * M <= 32;
    uint4 xr[PRE ? NX * M : 1];
    if constexpr (PRE) {
#pragma unroll
        for (int m = 0; m < M; m++)
#pragma unroll
            for (int i = 0; i < NX; i++) xr[m * NX + i] = XP::load(xrow(m), i, npieces);
    }

    const BufPlanes B = T::planes(P, N, K);
    RowOff ro[R];
#pragma unroll
    for (int r = 0; r < R; r++) ro[r] = T::row_off(row0 + r < N ? row0 + r : N - 1, K);
    auto load = [&](SlotM<FMT, R>& sl, int c) {
        const int b = c * kWave + lane;
        const int bb = b < nchunks ? b : 0;
#pragma unroll
        for (int r = 0; r < R; r++) T::load(sl.row[r], B, ro[r], bb);
    };

    SlotM<FMT, R> buf[D];
#pragma unroll
    for (int d = 0; d < D; d++)
        if (CS == 0 || d < CS) load(buf[d], d < C ? d : 0);

    if constexpr (PRE) {
#pragma unroll
        for (int m = 0; m < M; m++) XP::template store<NX, true>(xr + m * NX, 0, npieces, xs + m * xs_row);
    } else {
        const int npt = XQ ? (npieces + kBlock - 1) / kBlock : (npieces / GF4 + kBlock - 1) / kBlock * GF4;
        for (int m = 0; m < M; m++) {
            for (int i0 = 0; i0 < npt; i0 += 4) {
                uint4 xt[4];
#pragma unroll
                for (int i = 0; i < 4; i++) xt[i] = XP::load(xrow(m), i0 + i, npieces);
                XP::template store<4, false>(xt, i0, npieces, xs + m * xs_row);
            }
        }
    }
    __syncthreads();

    float acc[R][M];
#pragma unroll
    for (int r = 0; r < R; r++)
#pragma unroll
        for (int m = 0; m < M; m++) acc[r][m] = 0.f;
    auto compute = [&](const SlotM<FMT, R>& sl, int c) {
        const int b = c * kWave + lane;
        const bool ok = b < nchunks;
        uint32_t v[R][T::NVEC];
#pragma unroll
        for (int r = 0; r < R; r++) T::unpack(sl.row[r], v[r]);
#pragma unroll
        for (int m = 0; m < M; m++) {
            uint32_t xv[4 * T::F4];
            read_x<FMT>(xs + m * xs_row, ok ? b : 0, xv);
            if constexpr (T::INT) {
                xv[T::META] = ok ? xv[T::META] : 0u;
#pragma unroll
                for (int r = 0; r < R; r++) acc[r][m] += T::dot_vec(sl.row[r], v[r], xv);
            } else {
#pragma unroll
                for (int r = 0; r < R; r++) {
                    const float t = T::dot_vec(sl.row[r], v[r], xv);
                    acc[r][m] += ok ? t : 0.f;
                }
            }
        }
    };

    // Six-step K sums as the single-token kernel does: per two-step slice
    // across the wave, then the slices in order.
    constexpr int SL = CS == 6 ? 2 : CS;
    float tot[R][M];
    if constexpr (CS > 0) {
#pragma unroll
        for (int c = 0; c < CS; c++) {
            compute(buf[c % D], c);
            if (c + D < CS) load(buf[c % D], c + D);
            if (SL < CS && (c + 1) % SL == 0) {
#pragma unroll
                for (int r = 0; r < R; r++)
#pragma unroll
                    for (int m = 0; m < M; m++) {
                        const float w = wave_sum_dpp(acc[r][m]);
                        tot[r][m] = c + 1 == SL ? w : tot[r][m] + w;
                        acc[r][m] = 0.f;
                    }
            }
        }
    } else {
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

    // lane r * M + m stores Y[m][row0 + r]
#pragma unroll
    for (int r = 0; r < R; r++)
#pragma unroll
        for (int m = 0; m < M; m++) {
            const float s = SL < CS ? tot[r][m] : wave_sum_dpp(acc[r][m]);
            if (lane == r * M + m && row0 + r < N) {
                float* dst = y + (int64_t)m * ldy + row0 + r;
                *dst = accumulate ? *dst + s : s;
            }
        }
}

// LDS bytes of M staged tokens of K values.
template <int FMT>
static size_t smallm_lds(int64_t M, int64_t K) {
    return (size_t)M * (size_t)(K / Traits<FMT>::WPC) * Stride<FMT>::DW * 4;
}

template <int FMT, int R, int M, int CS, bool XQ>
static hipError_t launch_sk(DevPlanes P, int64_t N, int64_t K, const void* x, int64_t ldx,
                            float* y, int64_t ldy, int accumulate, hipStream_t stream) {
    const int64_t grid = (N + kWavesPerBlock * R - 1) / (kWavesPerBlock * R);
    const size_t lds = smallm_lds<FMT>(M, K);
    auto kern = gemv_smallm_kernel<FMT, R, M, CS, XQ>;
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)kern,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kBlock), lds, stream, P, N, (int)K, x, ldx,
                       y, ldy, accumulate);
    return hipGetLastError();
}

template <int FMT, int M, int CS>
static hipError_t launch_sc(DevPlanes P, int64_t N, int64_t K, const void* x, int64_t ldx,
                            bool xq, float* y, int64_t ldy, int accumulate, hipStream_t s) {
    constexpr int R = 2;
    if constexpr (Traits<FMT>::INT) {
        if (xq) return launch_sk<FMT, R, M, CS, true>(P, N, K, x, ldx, y, ldy, accumulate, s);
    }
    return launch_sk<FMT, R, M, CS, false>(P, N, K, x, ldx, y, ldy, accumulate, s);
}

template <int FMT, int M>
static hipError_t launch_sm(DevPlanes P, int64_t N, int64_t K, const void* x, int64_t ldx,
                            bool xq, float* y, int64_t ldy, int accumulate, hipStream_t s) {
    constexpr int per = 64 * Traits<FMT>::WPC;
    if constexpr (FMT == kQ45 || FMT == kQ65) {
        if (K == 2 * per) return launch_sc<FMT, M, 2>(P, N, K, x, ldx, xq, y, ldy, accumulate, s);
        if (K == 6 * per) return launch_sc<FMT, M, 6>(P, N, K, x, ldx, xq, y, ldy, accumulate, s);
    }
    if constexpr (FMT == kQ25) {
        if (K == per) return launch_sc<FMT, M, 1>(P, N, K, x, ldx, xq, y, ldy, accumulate, s);
    }
    return launch_sc<FMT, M, 0>(P, N, K, x, ldx, xq, y, ldy, accumulate, s);
}

template <int FMT>
static hipError_t launch_smf(DevPlanes P, int64_t N, int64_t K, const void* x, int64_t M,
                             int64_t ldx, bool xq, float* y, int64_t ldy, int accumulate,
                             hipStream_t s) {
    switch (M) {
    case 2: return launch_sm<FMT, 2>(P, N, K, x, ldx, xq, y, ldy, accumulate, s);
    case 3: return launch_sm<FMT, 3>(P, N, K, x, ldx, xq, y, ldy, accumulate, s);
    case 4: return launch_sm<FMT, 4>(P, N, K, x, ldx, xq, y, ldy, accumulate, s);
    case 5: return launch_sm<FMT, 5>(P, N, K, x, ldx, xq, y, ldy, accumulate, s);
    case 6: return launch_sm<FMT, 6>(P, N, K, x, ldx, xq, y, ldy, accumulate, s);
    case 7: return launch_sm<FMT, 7>(P, N, K, x, ldx, xq, y, ldy, accumulate, s);
    case 8: return launch_sm<FMT, 8>(P, N, K, x, ldx, xq, y, ldy, accumulate, s);
    }
    return hipErrorInvalidValue;
}

bool gemv_smallm_fits(int fmt, int64_t M, int64_t K) {
    const size_t cap = 160 * 1024;
    switch (fmt) {
    case kQ45: return smallm_lds<kQ45>(M, K) <= cap;
    case kQ65: return smallm_lds<kQ65>(M, K) <= cap;
    case kQ25: return smallm_lds<kQ25>(M, K) <= cap;
    case kBF16: return smallm_lds<kBF16>(M, K) <= cap;
    }
    return false;
}

hipError_t launch_gemv_smallm(int fmt, DevPlanes P, int64_t N, int64_t K, const void* x,
                              bool x_staged, int64_t M, int64_t ldx, float* y, int64_t ldy,
                              int accumulate, hipStream_t stream) {
    switch (fmt) {
    case kQ45: return launch_smf<kQ45>(P, N, K, x, M, ldx, x_staged, y, ldy, accumulate, stream);
    case kQ65: return launch_smf<kQ65>(P, N, K, x, M, ldx, x_staged, y, ldy, accumulate, stream);
    case kQ25: return launch_smf<kQ25>(P, N, K, x, M, ldx, x_staged, y, ldy, accumulate, stream);
    case kBF16: return launch_smf<kBF16>(P, N, K, x, M, ldx, x_staged, y, ldy, accumulate, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace mbq
