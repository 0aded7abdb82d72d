// gemv_m1.hip -- single-token matrix-vector product for block-quantized weights.
//
// y[n] (+)= sum_k w[n][k] x[k], the weight stream of one decode token
// ([roofline-holds] "The Math": every weight crosses the memory bus once per
// token and enters a single multiply-add, a handful of flops per byte where
// the chip could do hundreds, so the memory system sets the pace).
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

// Row groups and K slices (static K of 2 or 6 chunk steps, or 1 for Q25).
// A workgroup holds S x 4 waves; wave w works on K slice w / 4 (chunk steps
// [CSS * s, CSS * (s + 1)) of every row, CSS = CS / S) and on row block w % 4
// of each of its G row groups.  x is staged once per workgroup for all of
// them.  Six-step K (12288) takes S = 3 slices of two steps, so each wave
// keeps the short, register-resident loop of the K = 4096 tables; the slice
// partial sums meet in LDS and are added in slice order.
constexpr bool grouped_form(int CS) { return CS == 1 || CS == 2 || CS == 6; }
constexpr int k_slices(int CS) { return CS == 6 ? 3 : 1; }

template <int FMT, int R, int CS, bool GATHER, bool XQ, int PRO = kProNone, int EPI = kEpiStore>
__global__ __launch_bounds__(kBlock * k_slices(CS)) void gemv_m1_kernel(DevPlanes P, int64_t N, int K,
                                                         const void* __restrict__ xsrc,
                                                         float* __restrict__ y, int accumulate,
                                                         const int32_t* __restrict__ gidx,
                                                         int rpe, const float* __restrict__ gamma,
                                                         float eps, int groups, int64_t nw) {
    using T = Traits<FMT>;
    static_assert(PRO == kProNone || (grouped_form(CS) && !XQ),
                  "the norm prologue needs the grouped form (static K), fp32 x");
    static_assert(EPI == kEpiStore || R == 2, "the silu epilogue pairs two rows per wave");
    constexpr bool GROUPED = grouped_form(CS);
    constexpr int S = k_slices(CS);                           // K slices per workgroup
    constexpr int CSS = CS / S;                               // chunk steps per slice
    constexpr int NT = kBlock * S;                            // threads per workgroup
    using XP = XPieces<FMT, XQ, NT>;
    // chunk steps in flight: two for a runtime K; a static K outside the
    // grouped form (BF16, 8 steps) keeps its whole row in flight at 1 or 2
    // rows per wave, half of it at 4
    constexpr int D = CS > 0 && !GROUPED ? (R <= 2 ? CS : CS / 2) : 2;
    extern __shared__ float4 smem[];
    uint32_t* xs = (uint32_t*)smem;

    const int lane = threadIdx.x & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int wave = wid % kWavesPerBlock;                    // row block of the wave
    const int slice = wid / kWavesPerBlock;                   // K slice of the wave
    const int c0 = slice * CSS;                               // its first chunk step
    const int nchunks = K / T::WPC;
    const int C = CS > 0 ? CS : (nchunks + kWave - 1) / kWave;
    const int G = GROUPED ? groups : 1;
    const int64_t row0 = ((int64_t)blockIdx.x * G * kWavesPerBlock + wave) * R;

    // ---- x: the first pieces, before any weight load
    const uint4* xsrc4 = (const uint4*)xsrc;
    const int npieces = XP::count(K);
    constexpr int GF4 = XP::GF4;
    constexpr int NR = 4;                                     // pieces per runtime round
    // pieces per thread: all of them (static K), or the first round
    constexpr int NX = CS > 0 ? (XQ ? CSS * T::F4 / 4 : CSS * T::WPC / 16) : NR;
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
    auto y_of = [&](int64_t r0) {
        const int64_t yrow = r0 + (lane < R ? lane : 0);
        return y[yrow < N ? yrow : N - 1];
    };
    float yin = y_of(row0);

    // ---- weight rows: rows past N re-read row N-1 (their results are not stored)
    const BufPlanes B = T::planes(P, nw, K);
    RowOff ro[R];
    // Row indices fit in 32 bits (N < 2^31), which keeps the clamps on the
    // scalar unit.
    const int n32 = (int)N;
    auto set_rows = [&](int64_t r0) {
#pragma unroll
        for (int r = 0; r < R; r++) {
            const int rr = (int)r0 + r;
            int n = rr < n32 ? rr : n32 - 1;
            if constexpr (GATHER) {
                const int e = n / rpe;
                n = gidx[e] * rpe + (n - e * rpe);
            }
            ro[r] = T::row_off(n, K);
        }
    };
    set_rows(row0);
    auto load = [&](Slot<FMT, R>& sl, int c) {
        const int b = (c0 + c) * kWave + lane;
        const int bb = b < nchunks ? b : 0;
#pragma unroll
        for (int r = 0; r < R; r++) T::load(sl.row[r], B, ro[r], bb);
    };

    float acc[R];
#pragma unroll
    for (int r = 0; r < R; r++) acc[r] = 0.f;
    auto compute = [&](const Slot<FMT, R>& sl, int c) {
        const int b = (c0 + c) * kWave + lane;
        const bool ok = b < nchunks;
        uint32_t xv[4 * T::F4];
        read_x<FMT>(xs, ok ? b : 0, xv);
        if constexpr (T::INT) {
            T::mask_meta(xv, ok);    // lanes past the row add exactly 0
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
        // All of a slice's chunks in flight in the grouped form, else D.
        constexpr int DD = GROUPED ? CSS : D;
        Slot<FMT, R> buf[DD];
#pragma unroll
        for (int d = 0; d < DD; d++) load(buf[d], d);
        // Row groups (see below): group g of this wave is rows
        // ((blk * G + g) * 4 + wave) * R.  With the norm prologue, and for
        // Q25 (one chunk per lane and group), the second group's loads are
        // issued before x is staged as well, so that two groups of weights
        // are in flight while x is normalised and staged.  A gather takes
        // its rows through an index load first, and is slower so.
        constexpr bool EARLY = GROUPED && (PRO == kProRms || (FMT == kQ25 && !GATHER));
        const int64_t gstride = (int64_t)kWavesPerBlock * R;
        const int64_t rbase = row0;
        Slot<FMT, R> alt[DD];
        auto load_group = [&](Slot<FMT, R>* b, int g) {
            const int gc = g < G ? g : G - 1;
            set_rows(rbase + (int64_t)gc * gstride);
#pragma unroll
            for (int d = 0; d < DD; d++) load(b[d], d);
        };
        if constexpr (EARLY) load_group(alt, 1);
        // RMSNorm of the row, y = g * (x * inv).  With a store or accumulate
        // epilogue the prologue stages g * x and leaves each wave's share of
        // sum(x^2) in LDS; inv = 1 / rms is formed from those shares, added
        // in wave order, after the staging barrier and scales each row's
        // total at the end (W (g x) inv), so no barrier of its own sits
        // between the x loads and the staging.  The silu product, whose
        // long row-group loop measured slower so, scales x by inv first.
        constexpr bool DEFER = PRO == kProRms && EPI != kEpiSilu;
        __shared__ float red[PRO == kProRms ? kWavesPerBlock * S : 1];
        float inv = 1.0f;
        if constexpr (PRO == kProRms) {
            float ss = 0.f;
#pragma unroll
            for (int i = 0; i < NX; i++) {
                const float4 v = __builtin_bit_cast(float4, xr[i]);
                ss = fmaf(v.x, v.x, ss);
                ss = fmaf(v.y, v.y, ss);
                ss = fmaf(v.z, v.z, ss);
                ss = fmaf(v.w, v.w, ss);
            }
            if constexpr (DEFER) {
                ss = wave_sum_dpp(ss);
                if (lane == 0) red[wid] = ss;
            } else {
                inv = 1.0f / sqrtf(block_sum<kWavesPerBlock * S, false>(ss, red) / (float)K + eps);
            }
            const float sx = DEFER ? 1.0f : inv;
#pragma unroll
            for (int i = 0; i < NX; i++) {
                const float4 v = __builtin_bit_cast(float4, xr[i]);
                const float4 g = __builtin_bit_cast(float4, gr[i]);
                xr[i] = __builtin_bit_cast(uint4, make_float4(g.x * (v.x * sx), g.y * (v.y * sx),
                                                              g.z * (v.z * sx), g.w * (v.w * sx)));
            }
        }
        XP::template store<NX, true>(xr, 0, npieces, xs);
        __syncthreads();
        if constexpr (DEFER) {
            float t = red[0];
#pragma unroll
            for (int w = 1; w < kWavesPerBlock * S; w++) t += red[w];
            inv = 1.0f / sqrtf(t / (float)K + eps);
        }
        if constexpr (GROUPED) {
            // Row groups: the workgroup's rows are one contiguous block.  Each group's
            // chunks (of the wave's slice) are all in flight, two groups deep:
            // the loads of group g + 1 are issued before group g is computed
            // (the last group reloads itself; that copy is never used).  Slice
            // sums go to LDS and the block is written once at the end,
            // coalesced, so no store sits between the loads of the loop.
            // G * 4 * R <= 1024 rows per workgroup (G <= 64, R <= 4)
            __shared__ float outs[S][kWavesPerBlock * 4 * 64];
            auto finish = [&](int g) {
#pragma unroll
                for (int r = 0; r < R; r++) {
                    const float sr = wave_sum_dpp(acc[r]);
                    if (lane == r) outs[slice][g * kWavesPerBlock * R + wave * R + r] = sr;
                    acc[r] = 0.f;
                }
            };
            for (int g = 0; g < G; g += 2) {
                if (!EARLY || g > 0) load_group(alt, g + 1);
#pragma unroll
                for (int c = 0; c < CSS; c++) compute(buf[c], c);
                finish(g);
                if (g + 1 >= G) break;
                load_group(buf, g + 2);
#pragma unroll
                for (int c = 0; c < CSS; c++) compute(alt[c], c);
                finish(g + 1);
            }
            __syncthreads();
            // the workgroup's rows [blk G 4R, +G 4R): slice sums in slice order
            const int per = G * kWavesPerBlock * R;
            const int64_t rwg = (int64_t)blockIdx.x * per;
            if constexpr (EPI == kEpiSilu) {
                // rows 2t and 2t + 1 of the block are the gate and up rows of output rwg / 2 + t
                for (int t = threadIdx.x; t < per / 2; t += NT) {
                    float gs = outs[0][2 * t], us = outs[0][2 * t + 1];
#pragma unroll
                    for (int q = 1; q < S; q++) {
                        gs += outs[q][2 * t];
                        us += outs[q][2 * t + 1];
                    }
                    const int64_t n = rwg / 2 + t;
                    if (n < N / 2) y[n] = (accumulate ? y[n] : 0.f) + gs / (1.0f + expf(-gs)) * us;
                }
            } else {
                for (int t = threadIdx.x; t < per; t += NT) {
                    float v = outs[0][t];
#pragma unroll
                    for (int q = 1; q < S; q++) v += outs[q][t];
                    if constexpr (DEFER) v *= inv;
                    const int64_t n = rwg + t;
                    if (n < N) y[n] = (accumulate ? y[n] : 0.f) + v;
                }
            }
            return;
        } else {
#pragma unroll
            for (int c = 0; c < CS; c++) {
                compute(buf[c % DD], c);
                if (c + DD < CS) load(buf[c % DD], c + DD);
            }
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
    int groups;          // row groups per wave (static K with C <= 2 only)
    int64_t nw;          // rows of the weight table (N, or all experts for a gather)
};

template <int FMT, int R, int CS, bool GATHER, bool XQ, int PRO = kProNone, int EPI = kEpiStore>
static hipError_t launch_k(const M1Args& a, hipStream_t stream) {
    using T = Traits<FMT>;
    const int G = grouped_form(CS) ? (a.groups > 0 ? a.groups : 1) : 1;
    const int64_t rows_per_wg = (int64_t)kWavesPerBlock * R * G;
    const int64_t grid = (a.N + rows_per_wg - 1) / rows_per_wg;
    const size_t lds = (size_t)(a.K / T::WPC) * Stride<FMT>::DW * 4;
    auto kern = gemv_m1_kernel<FMT, R, CS, GATHER, XQ, PRO, EPI>;
    if (hipError_t e = ensure_lds<gemv_m1_kernel<FMT, R, CS, GATHER, XQ, PRO, EPI>>(lds)) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kBlock * k_slices(CS)), lds, stream, a.P, a.N, (int)a.K,
                       a.x, a.y, a.accumulate, a.gidx, (int)a.rpe, a.gamma, a.eps, G, a.nw);
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

// Default geometry, from cold-weight sweeps on MI355X.  Tables whose K
// takes at most two unrolled chunk steps use row groups: about 512
// workgroups of 4 waves (N / 2048 rows per wave, at most 4) beat both many
// small workgroups, which each stage x again, and few large ones, which
// leave CUs idle at the tail.  The largest tables (a vocabulary head) take
// 8 rows per wave.  Six-step K (12288) runs three K slices per workgroup
// and N / 1024 single-row groups, at most 4.
// Other K keep one group and 1, 2 or 4 rows per wave.  The silu product
// (pairs) takes its rows two at a time in N / 2048 groups, which is 256
// workgroups (N / 4096 groups, 512 workgroups, past 8 groups; at most 8).
// A Q45 product with the RMSNorm prologue at K = 4096 (below vocabulary
// size) takes 2 rows per wave and N / 2048 groups up to 6: about 256
// workgroups, so each CU normalises and stages x once (7-17 % faster for
// N = 2048 ... 24576; Q65 at 2 rows per wave holds 202 VGPRs and gains
// nothing).  Q25 at K = 4096 (one chunk per lane, plain or gathered)
// takes 2 rows per wave and N / 4096 groups up to 6, about 512 workgroups
// (10-20 % faster at 12288 and 24576 rows).
GemvGeom gemv_m1_default_geom(int fmt, int64_t N, int64_t K, bool pairs, bool norm) {
    GemvGeom g;
    g.groups = 1;
    int steps = 0;
    switch (fmt) {
    case kQ45: steps = static_steps<kQ45>(K); break;
    case kQ65: steps = static_steps<kQ65>(K); break;
    case kQ25: steps = static_steps<kQ25>(K); break;
    case kBF16: steps = static_steps<kBF16>(K); break;
    }
    if (!grouped_form(steps)) {
        // A runtime K of 16384 or more fills most of a CU's LDS with staged
        // x (one 4-wave workgroup per CU), so each wave takes 4 rows to keep
        // enough weight bytes in flight.
        const bool big = N * K >= ((int64_t)32 << 20);
        g.rows_per_wave = N >= 65536 || (big && K >= 16384) ? 4 : big ? 2 : 1;
        return g;
    }
    if (pairs) {
        g.rows_per_wave = 2;
        int64_t gg = N / 2048;
        if (gg > 8) gg = N / 4096;
        g.groups = gg < 1 ? 1 : gg > 8 ? 8 : (int)gg;
        return g;
    }
    if (fmt == kQ25 && steps == 1 && N < 65536) {
        g.rows_per_wave = 2;
        g.groups = N / 4096 < 1 ? 1 : N / 4096 > 6 ? 6 : (int)(N / 4096);
        return g;
    }
    if (norm && fmt == kQ45 && steps == 2 && N < 65536) {
        g.rows_per_wave = 2;
        g.groups = N / 2048 < 1 ? 1 : N / 2048 > 6 ? 6 : (int)(N / 2048);
        return g;
    }
    g.rows_per_wave = 1;
    if (steps == 6) {
        g.groups = N / 1024 < 1 ? 1 : N / 1024 > 4 ? 4 : (int)(N / 1024);
        return g;
    }
    if (N >= 65536) {
        g.groups = 8;
        return g;
    }
    g.groups = N / 2048 < 1 ? 1 : N / 2048 > 4 ? 4 : (int)(N / 2048);
    return g;
}

hipError_t launch_gemv_m1(int fmt, DevPlanes P, int64_t N_out, int64_t K, const void* x,
                          bool x_staged, float* y, int accumulate, const int32_t* gidx,
                          int64_t rpe, GemvGeom geom, hipStream_t stream, int64_t n_weight_rows) {
    const M1Args a{P, N_out, K, x, y, accumulate, gidx, rpe, nullptr, 0.f, geom.groups,
                   n_weight_rows > 0 ? n_weight_rows : N_out};
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
    // the silu epilogue takes its gate/up rows in pairs (R = 2): keep the
    // rows per wave of the geometry asked for
    int groups = geom.groups;
    if (silu && geom.rows_per_wave != 2) groups = (groups * geom.rows_per_wave + 1) / 2;
    const M1Args a{P, N, K, x, y, accumulate, nullptr, 1, gamma, eps, groups, N};
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
