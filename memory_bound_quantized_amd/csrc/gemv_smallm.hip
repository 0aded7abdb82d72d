// gemv_smallm.hip -- Y[m][n] (+)= W[n] . X[m] for 2 <= M <= 8 tokens, on the
// vector units.
//
// Several tokens against one weight stream: each weight read from memory
// serves M sums, so the bytes per token fall as 1/M until the arithmetic
// catches up with the memory ([roofline-holds] "The Math": the crossover
// M* = (w/16)(R/BW); below it memory is the wall).  The arithmetic is the
// single-token kernel's: a wave unpacks its R rows' codes once per chunk and
// runs the integer-digit dot products (formats.h) against the staged x of
// every token.
//
// Geometry.  The staged x of M tokens takes M x 4.5 bytes per value of LDS
// (147 KB for eight 4096-wide tokens), so a CU holds one or two workgroups.
// A workgroup is therefore 16 waves (1024 threads), which keeps four waves
// per SIMD on one copy of x, and it stays resident for G row groups:
// wave w computes rows ((blk * G + g) * 16 + w) * R + r, g < G, so x is
// staged once per G * 16 * R rows.  The weight loads run two chunk steps
// ahead of the arithmetic across group boundaries.  Row sums go to LDS and
// the workgroup writes its block of Y once, coalesced.
//
// Each token's row is bit-identical to its M = 1 product: the per-lane
// sums, the wave reductions (per 4096-wide slice where the single-token
// kernel slices K = 12288), their order and the final add are the same.
#include "device_common.h"
#include "formats.h"
#include "kernels.h"
#include "staging.h"

namespace mbq {

constexpr int kSmWaves = 16;                       // waves per workgroup
constexpr int kSmBlock = kSmWaves * kWave;         // 1024 threads
constexpr int kSmOutBytes = 8192;                  // LDS for the row sums of a workgroup

template <int FMT, int R>
struct SlotM {
    typename Traits<FMT>::Row row[R];
};

// LDS bytes of M staged tokens of K values.
template <int FMT>
static size_t smallm_x_lds(int64_t M, int64_t K) {
    return (size_t)M * (size_t)(K / Traits<FMT>::WPC) * Stride<FMT>::DW * 4;
}

// Chunk steps per wave reduction: the single-token kernel reduces K = 12288
// (six steps of the 32-weight formats) per two-step slice, everything else
// once per row.
template <int FMT>
static int slice_steps(int64_t K, int C) {
    if constexpr (FMT == kQ45 || FMT == kQ65) {
        if (K == 6 * 64 * Traits<FMT>::WPC) return 2;
    }
    return C;
}

// Chunk steps of weight loads in flight per wave (four measured 4-8 %
// slower than two at M = 2..8: more registers, no more bandwidth).
constexpr int kSmDepth = 2;

template <int FMT, int R, int M, bool XQ, int PD = kSmDepth>
__global__ __launch_bounds__(kSmBlock) void gemv_smallm_kernel(DevPlanes P, int64_t N, int K,
                                                               const void* __restrict__ xsrc,
                                                               int64_t ldx, float* __restrict__ y,
                                                               int64_t ldy, int accumulate,
                                                               int groups, int sl) {
    using T = Traits<FMT>;
    using XP = XPieces<FMT, XQ, kSmBlock>;
    constexpr int GF4 = XP::GF4;
    static_assert(R * M <= kWave, "one storing lane per row and token");
    extern __shared__ float4 smem[];
    uint32_t* xs = (uint32_t*)smem;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int nchunks = K / T::WPC;
    const int C = (nchunks + kWave - 1) / kWave;       // chunk steps per row
    const int G = groups;
    const int npieces = XP::count(K);
    const int xs_row = nchunks * Stride<FMT>::DW;       // LDS dwords per token
    float* outs = (float*)(xs + M * xs_row);            // [G * 16 * R rows][M]
    const int rows_wg = G * kSmWaves * R;
    const int64_t rwg = (int64_t)blockIdx.x * rows_wg;  // first row of the workgroup

    // ---- weight rows: rows past N re-read row N-1 (their sums are not stored)
    const BufPlanes B = T::planes(P, N, K);
    const int n32 = (int)N;
    RowOff ro[R];
    auto set_rows = [&](int g) {
#pragma unroll
        for (int r = 0; r < R; r++) {
            const int rr = (int)rwg + (g * kSmWaves + wave) * R + r;
            ro[r] = T::row_off(rr < n32 ? rr : n32 - 1, K);
        }
    };
    // Loads walk (group, step) in order; past the last step the last one is
    // reloaded (never used).  No branch sits between loads (cursors advance by
    // selects), so each wait for loaded data names only the loads it needs.
    int lg = 0, lc = 0;
    set_rows(0);
    auto next_load = [&](SlotM<FMT, R>& sl) {
        const int b = lc * kWave + lane;
        const int bb = b < nchunks ? b : 0;
#pragma unroll
        for (int r = 0; r < R; r++) T::load(sl.row[r], B, ro[r], bb);
        const bool wrap = lc + 1 >= C;
        const bool last = wrap && lg + 1 >= G;
        lc = last ? lc : (wrap ? 0 : lc + 1);
        lg = wrap && !last ? lg + 1 : lg;
        set_rows(lg);
    };
    SlotM<FMT, R> buf[PD];
#pragma unroll
    for (int d = 0; d < PD; d++) next_load(buf[d]);

    // ---- x of every token into LDS, in rounds of 4 pieces per thread
    auto xrow = [&](int m) {
        return (const uint4*)xsrc + (XQ ? (int64_t)m * K / 4 : (int64_t)m * ldx / 4);
    };
    {
        constexpr int NR = 4;
        const int npt = XQ ? (npieces + kSmBlock - 1) / kSmBlock
                           : (npieces / GF4 + kSmBlock - 1) / kSmBlock * GF4;
        for (int m = 0; m < M; m++) {
            for (int i0 = 0; i0 < npt; i0 += NR) {
                uint4 xt[NR];
#pragma unroll
                for (int i = 0; i < NR; i++) xt[i] = XP::load(xrow(m), i0 + i, npieces);
                XP::template store<NR, false>(xt, i0, npieces, xs + m * xs_row);
            }
        }
    }
    __syncthreads();

    float acc[R][M], tot[R][M];
#pragma unroll
    for (int r = 0; r < R; r++)
#pragma unroll
        for (int m = 0; m < M; m++) acc[r][m] = 0.f, tot[r][m] = 0.f;
    auto compute = [&](const SlotM<FMT, R>& sl, int c) {
        const int b = c * kWave + lane;
        const bool ok = b < nchunks;
        uint32_t v[R][T::NVEC];
#pragma unroll
        for (int r = 0; r < R; r++) T::unpack(sl.row[r], v[r]);
#pragma unroll
        for (int m = 0; m < M; m++) {
            // One token's x at a time: the chunk index of token m carries an
            // (empty) dependence on token m - 1's sum, so its LDS reads cannot
            // be issued ahead and the registers hold one token's x, not M.
            int bi = ok ? b : 0;
            if (m > 0) {
#pragma unroll
                for (int r = 0; r < R; r++) asm volatile("" : "+v"(bi) : "v"(acc[r][m - 1]));
            }
            uint32_t xv[4 * T::F4];
            read_x<FMT>(xs + m * xs_row, bi, xv);
            if constexpr (T::INT) {
                T::mask_meta(xv, ok);
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
    // after step c of a row: close a slice, and at the row's end store its sums
    auto after_step = [&](int g, int c) {
        if ((c + 1) % sl == 0) {
#pragma unroll
            for (int r = 0; r < R; r++)
#pragma unroll
                for (int m = 0; m < M; m++) {
                    const float w = wave_sum_dpp(acc[r][m]);
                    tot[r][m] = c + 1 == sl ? w : tot[r][m] + w;
                    acc[r][m] = 0.f;
                }
        }
        if (c + 1 == C && g < G) {
#pragma unroll
            for (int r = 0; r < R; r++)
#pragma unroll
                for (int m = 0; m < M; m++)
                    if (lane == r * M + m) outs[((g * kSmWaves + wave) * R + r) * M + m] = tot[r][m];
        }
    };

    // Steps in whole rounds of PD: a round past the last step computes the
    // reloaded last step again, and its sums are not stored.
    const int total = G * C;
    const int rounds = (total + PD - 1) / PD;
    int cg = 0, cc = 0;
    for (int j = 0; j < rounds; j++) {
#pragma unroll
        for (int d = 0; d < PD; d++) {
            compute(buf[d], cc);
            next_load(buf[d]);
            after_step(cg, cc);
            const bool wrap = cc + 1 >= C;
            cc = wrap ? 0 : cc + 1;
            cg = wrap ? cg + 1 : cg;
        }
    }
    __syncthreads();

    // ---- the workgroup's block of Y: token-major, consecutive rows per thread
    for (int t = threadIdx.x; t < rows_wg * M; t += kSmBlock) {
        const int m = t / rows_wg, rl = t - m * rows_wg;
        const int64_t n = rwg + rl;
        if (n < N) {
            float* dst = y + (int64_t)m * ldy + n;
            *dst = (accumulate ? *dst : 0.f) + outs[rl * M + m];
        }
    }
}

template <int FMT, int R, int M, bool XQ>
static hipError_t launch_sk(DevPlanes P, int64_t N, int64_t K, const void* x, int64_t ldx,
                            float* y, int64_t ldy, int accumulate, int G, hipStream_t stream) {
    const int64_t rows_wg = (int64_t)G * kSmWaves * R;
    const int64_t grid = (N + rows_wg - 1) / rows_wg;
    const size_t lds = smallm_x_lds<FMT>(M, K) + (size_t)rows_wg * M * 4;
    const int nchunks = (int)(K / Traits<FMT>::WPC);
    const int sl = slice_steps<FMT>(K, (nchunks + kWave - 1) / kWave);
    auto kern = gemv_smallm_kernel<FMT, R, M, XQ>;
    if (hipError_t e = ensure_lds<gemv_smallm_kernel<FMT, R, M, XQ>>(lds)) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kSmBlock), lds, stream, P, N, (int)K, x, ldx,
                       y, ldy, accumulate, G, sl);
    return hipGetLastError();
}

template <int FMT, int M, bool XQ>
static hipError_t launch_smr(DevPlanes P, int64_t N, int64_t K, const void* x, int64_t ldx,
                             float* y, int64_t ldy, int accumulate, GemvGeom g, hipStream_t s) {
    switch (g.rows_per_wave) {
    case 1: return launch_sk<FMT, 1, M, XQ>(P, N, K, x, ldx, y, ldy, accumulate, g.groups, s);
    case 2: return launch_sk<FMT, 2, M, XQ>(P, N, K, x, ldx, y, ldy, accumulate, g.groups, s);
    default: return launch_sk<FMT, 3, M, XQ>(P, N, K, x, ldx, y, ldy, accumulate, g.groups, s);
    }
}

template <int FMT, int M>
static hipError_t launch_sm(DevPlanes P, int64_t N, int64_t K, const void* x, int64_t ldx,
                            bool xq, float* y, int64_t ldy, int accumulate, GemvGeom g,
                            hipStream_t s) {
    if constexpr (Traits<FMT>::INT) {
        if (xq) return launch_smr<FMT, M, true>(P, N, K, x, ldx, y, ldy, accumulate, g, s);
    }
    return launch_smr<FMT, M, false>(P, N, K, x, ldx, y, ldy, accumulate, g, s);
}

template <int FMT>
static hipError_t launch_smf(DevPlanes P, int64_t N, int64_t K, const void* x, int64_t M,
                             int64_t ldx, bool xq, float* y, int64_t ldy, int accumulate,
                             GemvGeom g, hipStream_t s) {
    switch (M) {
    case 2: return launch_sm<FMT, 2>(P, N, K, x, ldx, xq, y, ldy, accumulate, g, s);
    case 3: return launch_sm<FMT, 3>(P, N, K, x, ldx, xq, y, ldy, accumulate, g, s);
    case 4: return launch_sm<FMT, 4>(P, N, K, x, ldx, xq, y, ldy, accumulate, g, s);
    case 5: return launch_sm<FMT, 5>(P, N, K, x, ldx, xq, y, ldy, accumulate, g, s);
    case 6: return launch_sm<FMT, 6>(P, N, K, x, ldx, xq, y, ldy, accumulate, g, s);
    case 7: return launch_sm<FMT, 7>(P, N, K, x, ldx, xq, y, ldy, accumulate, g, s);
    case 8: return launch_sm<FMT, 8>(P, N, K, x, ldx, xq, y, ldy, accumulate, g, s);
    }
    return hipErrorInvalidValue;
}

bool gemv_smallm_fits(int fmt, int64_t M, int64_t K) {
    const size_t cap = 160 * 1024 - kSmOutBytes;
    switch (fmt) {
    case kQ45: return smallm_x_lds<kQ45>(M, K) <= cap;
    case kQ65: return smallm_x_lds<kQ65>(M, K) <= cap;
    case kQ25: return smallm_x_lds<kQ25>(M, K) <= cap;
    case kBF16: return smallm_x_lds<kBF16>(M, K) <= cap;
    }
    return false;
}

// Default geometry: one row per wave and as many row groups as make one
// workgroup per CU (G = N / (16 * 256)), within the row-sum buffer.  Measured
// on the 12288 x 4096 tables: every geometry of 256 workgroups (16 waves x 1
// row x 3 groups, 12 x 2 x 2, 8 x 2 x 3, 8 x 3 x 2) lands within 5 % at
// M = 2, 4 and 8; more workgroups queue behind the LDS (one copy of x per
// CU from five tokens on) and fewer leave CUs idle.
GemvGeom gemv_smallm_default_geom(int fmt, int64_t M, int64_t N) {
    (void)fmt;
    GemvGeom g;
    g.rows_per_wave = 1;
    const int64_t per_wg = 256 * kSmWaves;
    const int64_t G = (N + per_wg - 1) / per_wg;
    const int64_t gmax = kSmOutBytes / (4 * kSmWaves * M);
    g.groups = (int)(G < 1 ? 1 : G > gmax ? gmax : G);
    return g;
}

bool gemv_smallm_geom_ok(int64_t M, GemvGeom g) {
    return g.rows_per_wave >= 1 && g.rows_per_wave <= 3 && g.groups >= 1 &&
           (int64_t)g.groups * kSmWaves * g.rows_per_wave * M * 4 <= kSmOutBytes;
}

hipError_t launch_gemv_smallm(int fmt, DevPlanes P, int64_t N, int64_t K, const void* x,
                              bool x_staged, int64_t M, int64_t ldx, float* y, int64_t ldy,
                              int accumulate, GemvGeom g, hipStream_t stream) {
    if (!gemv_smallm_geom_ok(M, g)) return hipErrorInvalidValue;
    switch (fmt) {
    case kQ45: return launch_smf<kQ45>(P, N, K, x, M, ldx, x_staged, y, ldy, accumulate, g, stream);
    case kQ65: return launch_smf<kQ65>(P, N, K, x, M, ldx, x_staged, y, ldy, accumulate, g, stream);
    case kQ25: return launch_smf<kQ25>(P, N, K, x, M, ldx, x_staged, y, ldy, accumulate, g, stream);
    case kBF16: return launch_smf<kBF16>(P, N, K, x, M, ldx, x_staged, y, ldy, accumulate, g, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace mbq
