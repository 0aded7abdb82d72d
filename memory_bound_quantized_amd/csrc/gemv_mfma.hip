// gemv_mfma.hip -- Y[m][n] (+)= W[n] . X[m] for M >= 16 tokens of a Q45
// matrix on the matrix cores (v_mfma_f32_16x16x32_f16).
//
// With 16 or more tokens the sums per weight byte pass what the vector units
// sustain, so the contraction goes to the matrix units ([roofline-holds]
// "The Math": above M* = (w/16)(R/BW) the sums, not the memory, are the wall;
// "Two different problems").  Exactness is kept as in the vector kernels:
//   * A (weights): a Q45 code q becomes the fp16 value q - 8 exactly (the
//     bits 0x6400 | q are 1024 + q; subtracting 1032 is exact);
//   * B (tokens): each token is scaled by a power of two 2^e (its largest |x|
//     lands in [2^14, 2^15)) and split into fp16 hi + lo, 22 bits of x;
//   * one MFMA covers exactly one 32-weight block, so the block's fp16 scale
//     multiplies the fp32 block result in the epilogue: acc = fma(s, D, acc).
//
// Staged tile form ("xt", written by stage_x_mfma_kernel): for token tile tt
// (16 tokens) and block b, 2 KB = [hi, lo] x 64 lanes x 8 halfs, lane
// j + 16 g holding token 16 tt + j at k = 32 b + 8 g + {0,4,1,5,2,6,3,7} (the
// order in which a lane unpacks the 8 codes of one dword); then one float per
// token slot, 2^-e (0 for slots past M).
//
// fp32 x form (F32X, for mbq_gemv_q, one token tile per launch): the
// workgroup converts fp32 x into the same slab layout while it fills LDS,
// with one power of two per 32-weight block and token (the block's largest
// |x| lands in [2^14, 2^15)) instead of one per token.  The block's factor
// 2^-e joins its weight scale, so there is no staging launch and no staging
// buffer.
//
// Kernel geometry: TR row tiles x S K parts of waves per workgroup (below).
#include "device_common.h"
#include "formats.h"
#include "kernels.h"

namespace mbq {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef float f4v __attribute__((ext_vector_type(4)));
// Native vector types for the register arrays (HIP's uint4 is a union-based
// struct that keeps arrays of it out of registers here).
typedef uint32_t u4v __attribute__((ext_vector_type(4)));
typedef uint32_t u2v __attribute__((ext_vector_type(2)));

constexpr int kGB = 4;                  // blocks per weight load (one per lane)
constexpr int kScrStride = 20;          // dwords per row of the transpose scratch

__device__ __forceinline__ int64_t xt_tile_bytes(int64_t K) { return (K / 32) * 2048; }

// ---- staging: one workgroup per token slot and 1024-value chunk of K ------
// Each workgroup finds its token's largest |x| over the whole row (the row is
// read from L2 by every chunk's workgroup) and converts its own chunk, so
// the staging of 16 tokens runs on 16 x K / 1024 workgroups.
constexpr int kStageChunk = 1024;

__global__ __launch_bounds__(kBlock) void stage_x_mfma_kernel(const float* __restrict__ x,
                                                              int64_t ldx, int M, int K,
                                                              uint8_t* __restrict__ xt,
                                                              float* __restrict__ tscale) {
    __shared__ float red[kWavesPerBlock];
    const int m = blockIdx.x;                       // token slot
    const int k0 = blockIdx.y * kStageChunk;        // this workgroup's chunk
    const int tt = m / 16, j = m % 16;
    const int nb = K / 32;
    const bool real = m < M;
    const float* xr = x + (int64_t)(real ? m : 0) * ldx;
    float amax = 0.f;
    for (int k = 4 * (int)threadIdx.x; k < K; k += 4 * kBlock) {
        const float4 v = *(const float4*)(xr + k);
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    // 2^e puts the largest |x| into [2^14, 2^15); e within the normal range
    int e = 141 - (int)((__builtin_bit_cast(uint32_t, amax) >> 23) & 0xFFu);
    e = e > 126 ? 126 : (e < -126 ? -126 : e);
    const float up = __builtin_bit_cast(float, (uint32_t)(e + 127) << 23);
    if (threadIdx.x == 0 && blockIdx.y == 0)
        tscale[m] = real ? __builtin_bit_cast(float, (uint32_t)(127 - e) << 23) : 0.f;
    // half slot of weight m8 = k % 8 within a lane's 8 values
    constexpr int kSlot[8] = {0, 2, 4, 6, 1, 3, 5, 7};
    _Float16* base = (_Float16*)(xt + (int64_t)tt * nb * 2048);
    const int k1 = k0 + kStageChunk < K ? k0 + kStageChunk : K;
    for (int k = k0 + 4 * (int)threadIdx.x; k < k1; k += 4 * kBlock) {
        float4 v = real ? *(const float4*)(xr + k) : make_float4(0.f, 0.f, 0.f, 0.f);
        const float vv[4] = {v.x, v.y, v.z, v.w};
        const int b = k / 32, g = (k % 32) / 8, lane = j + 16 * g;
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const float xs = vv[q] * up;
            const _Float16 hi = (_Float16)xs;
            const _Float16 lo = (_Float16)(xs - (float)hi);
            const int slot = kSlot[(k + q) % 8];
            _Float16* p = base + (int64_t)b * 1024 + lane * 8 + slot;
            p[0] = hi;          // part 0
            p[512] = lo;        // part 1 (1024 bytes on)
        }
    }
}

int64_t xt_bytes(int64_t M, int64_t K) {
    const int64_t TT = (M + 15) / 16;
    return TT * (K / 32) * 2048 + TT * 16 * 4;
}

hipError_t launch_stage_x_mfma(const float* x, int64_t M, int64_t ldx, int64_t K, void* xt,
                               hipStream_t stream) {
    const int64_t TT = (M + 15) / 16;
    uint8_t* p = (uint8_t*)xt;
    float* ts = (float*)(p + TT * (K / 32) * 2048);
    const unsigned chunks = (unsigned)((K + kStageChunk - 1) / kStageChunk);
    hipLaunchKernelGGL(stage_x_mfma_kernel, dim3((unsigned)(TT * 16), chunks), dim3(kBlock), 0, stream,
                       x, ldx, (int)M, (int)K, p, ts);
    return hipGetLastError();
}

// ---- the product ---------------------------------------------------------
// Compile-time loop: f(IC<I>{}) for I = B .. E-1, so indices into register
// arrays are constants (the ring slots stay in registers).
template <int V>
struct IC {
    static constexpr int value = V;
};
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(IC<B>{});
        static_for<B + 1, E>(f);
    }
}

// 8 codes of one dword as fp16 (q - 8), in the order {0,4,1,5,2,6,3,7}.
__device__ __forceinline__ h8 codes_to_a(uint32_t a) {
    const h2v off = {(_Float16)1032.0f, (_Float16)1032.0f};
    h2v w[4];
#pragma unroll
    for (int s = 0; s < 4; s++)
        w[s] = __builtin_bit_cast(h2v, ((a >> (4 * s)) & 0x000F000Fu) | 0x64006400u) - off;
    return h8{w[0][0], w[0][1], w[1][0], w[1][1], w[2][0], w[2][1], w[3][0], w[3][1]};
}

// Workgroup = TR row tiles x S K parts of waves (TR * S waves).  Wave w takes
// row tile w % TR (16 rows) over K part w / TR (nb / S blocks); the waves of
// one K part share its xt slabs (SB blocks of every token tile), which the
// workgroup copies into LDS one step ahead (double-buffered).  Each wave
// streams its rows' codes as 16-byte loads (one block per lane, 4 blocks per
// row per load), kPG loads ahead, and turns them into MFMA A operands through
// a small per-wave LDS transpose.  The S partial tiles of a row tile are
// added in part order through LDS at the end.
//
// Requires K % 1024 == 0 and (nb / S) a multiple of kPG * kGB and of SB.
constexpr int kPG = 4;                   // weight loads in flight per wave

// One (block, token) item of an fp32-x slab: 32 values of token m from k0,
// as hi/lo fp16 halves of x * 2^e in the lane order of the tile form.
struct XItem {
    float4 v[8];
};
__device__ __forceinline__ void xitem_load(XItem& it, const float* __restrict__ x, int64_t ldx,
                                           int m, int M, int k0) {
    const float4* src = (const float4*)(x + (int64_t)(m < M ? m : 0) * ldx + k0);
#pragma unroll
    for (int q = 0; q < 8; q++) it.v[q] = m < M ? src[q] : make_float4(0.f, 0.f, 0.f, 0.f);
}
// Store item (t, lb, j) of part p into slab buffer sb: the hi and lo u4v of
// lanes j + 16 g (g = 0..3), and 2^-e into ie.
__device__ __forceinline__ void xitem_store(const XItem& it, u4v* sb, float* ie) {
    float amax = 0.f;
#pragma unroll
    for (int q = 0; q < 8; q++)
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(it.v[q].x), fabsf(it.v[q].y)),
                                 fmaxf(fabsf(it.v[q].z), fabsf(it.v[q].w))));
    int e = 141 - (int)((__builtin_bit_cast(uint32_t, amax) >> 23) & 0xFFu);
    e = e > 126 ? 126 : (e < -126 ? -126 : e);
    const float up = __builtin_bit_cast(float, (uint32_t)(e + 127) << 23);
    *ie = __builtin_bit_cast(float, (uint32_t)(127 - e) << 23);
#pragma unroll
    for (int g = 0; g < 4; g++) {
        // values k = 8 g + {0, 4, 1, 5, 2, 6, 3, 7}
        const float4 a = it.v[2 * g], b = it.v[2 * g + 1];
        const float w[8] = {a.x, b.x, a.y, b.y, a.z, b.z, a.w, b.w};
        h8 hi, lo;
#pragma unroll
        for (int q = 0; q < 8; q++) {
            const float xs = w[q] * up;
            hi[q] = (_Float16)xs;
            lo[q] = (_Float16)(xs - (float)hi[q]);
        }
        sb[16 * g] = __builtin_bit_cast(u4v, hi);
        sb[64 + 16 * g] = __builtin_bit_cast(u4v, lo);
    }
}

template <int TT, int TR, int S, int SB, bool F32X>
__global__ __launch_bounds__(kWave * TR * S) void gemv_mfma_q45_kernel(
        DevPlanes P, int64_t N, int K, const u4v* __restrict__ xt, const float* __restrict__ tscale,
        const float* __restrict__ xf, int64_t ldx,
        int M, float* __restrict__ y, int64_t ldy, int accumulate) {
    constexpr int NW = TR * S;
    constexpr int NT = kWave * NW;
    constexpr int XSB = TT * SB * 128;                // uint4 per slab of one K part
    constexpr int XALL = S * XSB;                     // uint4 per slab step, all parts
    constexpr int XPT = F32X ? 1 : (XALL + NT - 1) / NT;   // per thread (last round guarded)
    // fp32 x: items (part, tile, block, token) per slab step, per thread
    constexpr int XIT = S * TT * SB * 16;
    constexpr int IPT = F32X ? (XIT + NT - 1) / NT : 1;
    constexpr int GPS = SB / kGB;                     // weight groups per slab
    constexpr int kUS = kPG / GPS > 0 ? kPG / GPS : 1;   // slabs per unrolled body
    constexpr int RING = kUS * GPS;                  // ring slots (>= kPG)
    static_assert(SB % kGB == 0 && RING >= kPG, "slab and ring geometry");
    extern __shared__ u4v lds[];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int tr = wave % TR, part = wave / TR;
    const int i = lane & 15, g = lane >> 4;
    uint32_t* scr = (uint32_t*)(lds + 2 * XALL) + wave * 16 * kScrStride;
    // fp32 x: 2^-e of each (part, tile, block, token) of the two slab buffers
    float* iex = (float*)(lds + 2 * XALL) + NW * 16 * kScrStride;
    const int nb = K / 32, nbp = nb / S;              // blocks per K part
    const int ngroups = nbp / kGB, nslab = nbp / SB;
    const int b0 = part * nbp;                        // first block of this wave's part
    const int64_t row0 = ((int64_t)blockIdx.x * TR + tr) * 16;

    // A side: row i's codes from block b0, 16 bytes (one block) per lane per load
    const int64_t ra = row0 + i < N ? row0 + i : N - 1;
    const u4v* wq = (const u4v*)(P.p0 + ra * (K >> 1)) + b0;
    // D side: the scales of rows 4g + v, 4 blocks (8 bytes) per load
    const u2v* sq[4];
#pragma unroll
    for (int v = 0; v < 4; v++) {
        const int64_t rs = row0 + 4 * g + v < N ? row0 + 4 * g + v : N - 1;
        sq[v] = (const u2v*)(P.p2 + rs * (K >> 5) * 2) + b0 / kGB;
    }
    // slab step s: element e of the step is part e / XSB, tile (e % XSB) / (SB * 128)
    auto xt_el = [&](int st, int e) {
        const int p = e / XSB, r = e - p * XSB;
        const int t = r / (SB * 128), w = r - t * (SB * 128);
        return xt + (int64_t)t * nb * 128 + (int64_t)(p * nbp + st * SB) * 128 + w;
    };

    u4v xr[XPT];
    XItem xi[IPT];
    // item it of slab step st: part, tile, block in slab, token
    auto item_k0 = [&](int st, int it, int& m) {
        const int p = it / (TT * SB * 16), r = it - p * (TT * SB * 16);
        const int t = r / (SB * 16), r2 = r - t * (SB * 16);
        const int lb = r2 / 16, j = r2 - lb * 16;
        m = 16 * t + j;
        return 32 * (p * nbp + st * SB + lb);
    };
    auto load_x = [&](int st) {
        if constexpr (F32X) {
#pragma unroll
            for (int q = 0; q < IPT; q++) {
                const int it = q * NT + tid;
                if (XIT % NT == 0 || it < XIT) {
                    int m;
                    const int k0 = item_k0(st, it, m);
                    xitem_load(xi[q], xf, ldx, m, M, k0);
                }
            }
        } else {
#pragma unroll
            for (int q = 0; q < XPT; q++) {
                const int e = q * NT + tid;
                if (XALL % NT == 0 || e < XALL) xr[q] = *xt_el(st, e);
            }
        }
    };
    auto store_x = [&](int bsel) {
        if constexpr (F32X) {
#pragma unroll
            for (int q = 0; q < IPT; q++) {
                const int it = q * NT + tid;
                if (XIT % NT == 0 || it < XIT) {
                    const int p = it / (TT * SB * 16), r = it - p * (TT * SB * 16);
                    const int t = r / (SB * 16), r2 = r - t * (SB * 16);
                    const int lb = r2 / 16, j = r2 - lb * 16;
                    u4v* sb = lds + bsel * XALL + p * XSB + (t * SB + lb) * 128 + j;
                    xitem_store(xi[q], sb, iex + bsel * XIT + it);
                }
            }
        } else {
#pragma unroll
            for (int q = 0; q < XPT; q++) {
                const int e = q * NT + tid;
                if (XALL % NT == 0 || e < XALL) lds[bsel * XALL + e] = xr[q];
            }
        }
    };
    load_x(0);
    u4v wr[RING];
    u2v sr[RING][4];
#pragma unroll
    for (int t = 0; t < kPG; t++) {
        const int tc = t < ngroups ? t : ngroups - 1;
        wr[t] = wq[kGB * tc + g];
#pragma unroll
        for (int v = 0; v < 4; v++) sr[t][v] = sq[v][tc];
    }
    store_x(0);
    __syncthreads();

    f4v acc[TT];
#pragma unroll
    for (int tt = 0; tt < TT; tt++) acc[tt] = f4v{0.f, 0.f, 0.f, 0.f};
    const f4v zero = {0.f, 0.f, 0.f, 0.f};

    for (int s0 = 0; s0 < nslab; s0 += kUS) {
        static_for<0, kUS>([&](auto su_c) {
            constexpr int su = decltype(su_c)::value;
            const int st = s0 + su;
            constexpr int buf = su & 1;
            // next slab step (the last one reloads itself; it is not stored)
            const int sn = st + 1 < nslab ? st + 1 : st;
            load_x(sn);
            static_for<0, GPS>([&](auto tg_c) {
                constexpr int tg = decltype(tg_c)::value;
                constexpr int tl = (su * GPS + tg) % RING;          // ring slot
                constexpr int tf = (su * GPS + tg + kPG) % RING;  // slot of the group kPG ahead
                const int t = st * GPS + tg;                        // weight group
                // transpose: lane (i, g) holds block 4t + g of row i; each
                // MFMA needs dword g of one block from every lane of row i
                *(u4v*)(scr + i * kScrStride + 4 * g) = wr[tl];
                u2v sc[4];
#pragma unroll
                for (int v = 0; v < 4; v++) sc[v] = sr[tl][v];
                const int tn = t + kPG < ngroups ? t + kPG : ngroups - 1;
                wr[tf] = wq[kGB * tn + g];
#pragma unroll
                for (int v = 0; v < 4; v++) sr[tf][v] = sq[v][tn];
#pragma unroll
                for (int b4 = 0; b4 < kGB; b4++) {
                    const h8 a = codes_to_a(scr[i * kScrStride + 4 * b4 + g]);
                    float sv[4];
#pragma unroll
                    for (int v = 0; v < 4; v++)
                        sv[v] = h2f((b4 < 2 ? sc[v].x : sc[v].y) >> (16 * (b4 & 1)));
                    const int lb = tg * kGB + b4;                   // block within the slab
#pragma unroll
                    for (int tt = 0; tt < TT; tt++) {
                        const u4v* bp = lds + buf * XALL + part * XSB + (tt * SB + lb) * 128;
                        const h8 bh = __builtin_bit_cast(h8, bp[lane]);
                        const h8 bl = __builtin_bit_cast(h8, bp[64 + lane]);
                        f4v d = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bh, zero, 0, 0, 0);
                        d = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bl, d, 0, 0, 0);
                        if constexpr (F32X) {
                            // the block's 2^-e for this lane's token column
                            const float ie = iex[buf * XIT + ((part * TT + tt) * SB + lb) * 16 + (lane & 15)];
#pragma unroll
                            for (int v = 0; v < 4; v++) acc[tt][v] = fmaf(sv[v] * ie, d[v], acc[tt][v]);
                        } else {
#pragma unroll
                            for (int v = 0; v < 4; v++) acc[tt][v] = fmaf(sv[v], d[v], acc[tt][v]);
                        }
                    }
                }
                // fp32 x: convert the next slab into the other buffer (read
                // only after the barrier below) between this step's matrix
                // instructions
                if constexpr (F32X && tg == (GPS - 1) / 2) store_x(buf ^ 1);
            });
            if constexpr (!F32X) store_x(buf ^ 1);
            __syncthreads();
        });
    }

    // K parts 1 .. S-1 leave their tiles in LDS (the slab area is free now);
    // part 0 adds them in part order.
    f4v* red = (f4v*)lds;                              // [S - 1][TR][TT][64]
    if constexpr (S > 1) {
        if (part > 0) {
#pragma unroll
            for (int tt = 0; tt < TT; tt++) red[(((part - 1) * TR + tr) * TT + tt) * kWave + lane] = acc[tt];
        }
        __syncthreads();
        if (part > 0) return;
#pragma unroll
        for (int q = 1; q < S; q++)
#pragma unroll
            for (int tt = 0; tt < TT; tt++) {
                const f4v o = red[(((q - 1) * TR + tr) * TT + tt) * kWave + lane];
#pragma unroll
                for (int v = 0; v < 4; v++) acc[tt][v] += o[v];
            }
    }

    // lane j + 16 g holds rows 4g + v of token column j
    const int j = lane & 15;
#pragma unroll
    for (int tt = 0; tt < TT; tt++) {
        const int m = 16 * tt + j;
        if (m >= M) continue;
        const float ts = F32X ? 1.0f : tscale[m];
#pragma unroll
        for (int v = 0; v < 4; v++) {
            const int64_t n = row0 + 4 * g + v;
            if (n < N) {
                float* dst = y + (int64_t)m * ldy + n;
                const float val = acc[tt][v] * ts;
                *dst = accumulate ? *dst + val : val;
            }
        }
    }
}

template <int TT, int TR, int S, int SB, bool F32X>
static hipError_t launch_mfma_k(DevPlanes P, int64_t N, int64_t K, const u4v* xt, const float* ts,
                                const float* xf, int64_t ldx, int M, float* y, int64_t ldy,
                                int accumulate, hipStream_t stream) {
    const size_t lds = (size_t)2 * S * TT * SB * 128 * 16 + (size_t)TR * S * 16 * kScrStride * 4 +
                       (F32X ? (size_t)2 * S * TT * SB * 16 * 4 : 0);
    auto kern = gemv_mfma_q45_kernel<TT, TR, S, SB, F32X>;
    if (hipError_t e = ensure_lds<gemv_mfma_q45_kernel<TT, TR, S, SB, F32X>>(lds)) return e;
    const int64_t grid = (N + 16 * TR - 1) / (16 * TR);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kWave * TR * S), lds, stream, P, N, (int)K,
                       xt, ts, xf, ldx, M, y, ldy, accumulate);
    return hipGetLastError();
}

// K parts and slab size (LDS: 2 * S * TT * SB * 2 KB <= 128 KB): one or two
// token tiles take S = 4 parts when a workgroup has at most two row tiles,
// else 2; three or four token tiles take 2; K = 1024 (32 blocks) takes 2.
// MBQ_MFMA_S = 2 forces two parts (tuning sweeps).
template <int TT, int TR, bool F32X>
static hipError_t launch_mfma_tr(DevPlanes P, int64_t N, int64_t K, const u4v* xt, const float* ts,
                                 const float* xf, int64_t ldx, int M, float* y, int64_t ldy,
                                 int accumulate, hipStream_t s) {
    bool four = TT <= 2 && TR <= 2 && (K / 32) % 64 == 0;
    if (const char* e = tuning_var("MBQ_MFMA_S")) four = TT <= 2 && (K / 32) % 64 == 0 && atoi(e) == 4;
    if constexpr (TT == 1) {
        if (four) return launch_mfma_k<1, TR, 4, 8, F32X>(P, N, K, xt, ts, xf, ldx, M, y, ldy, accumulate, s);
        return launch_mfma_k<1, TR, 2, 8, F32X>(P, N, K, xt, ts, xf, ldx, M, y, ldy, accumulate, s);
    } else if constexpr (TT == 2) {
        if (four) return launch_mfma_k<2, TR, 4, 4, F32X>(P, N, K, xt, ts, xf, ldx, M, y, ldy, accumulate, s);
        return launch_mfma_k<2, TR, 2, 4, F32X>(P, N, K, xt, ts, xf, ldx, M, y, ldy, accumulate, s);
    } else {
        return launch_mfma_k<TT, TR, 2, 4, F32X>(P, N, K, xt, ts, xf, ldx, M, y, ldy, accumulate, s);
    }
}

// Row tiles per workgroup, from sweeps on MI355X (N = 4096 and 12288).
// * One token tile: N / 4096 tiles, so 12288 rows take three and fill 256
//   workgroups (16.0 us at 16 tokens, against 19.3 us with four tiles on 192
//   workgroups).
// * Two token tiles: one workgroup per 192 tiles' worth of rows.
// * More: one per 128.
// At most 4.  Three tiles keep their registers only with one or three token
// tiles (two or four spill), so elsewhere three becomes four.  MBQ_MFMA_TR
// overrides (tuning sweeps).
template <int TT, bool F32X>
static hipError_t launch_mfma_tt(DevPlanes P, int64_t N, int64_t K, const u4v* xt, const float* ts,
                                 const float* xf, int64_t ldx, int M, float* y, int64_t ldy,
                                 int accumulate, hipStream_t s) {
    int64_t tr = TT == 1 ? N / (16 * 256) : TT == 2 ? N / (16 * 192) : N / (16 * 128);
    if (const char* e = tuning_var("MBQ_MFMA_TR")) tr = atoi(e);
    if (tr == 3 && (TT == 2 || TT == 4)) tr = 4;
    switch (tr <= 1 ? 1 : tr == 2 ? 2 : tr == 3 ? 3 : 4) {
    case 1: return launch_mfma_tr<TT, 1, F32X>(P, N, K, xt, ts, xf, ldx, M, y, ldy, accumulate, s);
    case 2: return launch_mfma_tr<TT, 2, F32X>(P, N, K, xt, ts, xf, ldx, M, y, ldy, accumulate, s);
    case 3: return launch_mfma_tr<TT, 3, F32X>(P, N, K, xt, ts, xf, ldx, M, y, ldy, accumulate, s);
    default: return launch_mfma_tr<TT, 4, F32X>(P, N, K, xt, ts, xf, ldx, M, y, ldy, accumulate, s);
    }
}

template <bool F32X>
static hipError_t launch_tt(int tt, DevPlanes P, int64_t N, int64_t K, const u4v* xt,
                            const float* ts, const float* xf, int64_t ldx, int M, float* y,
                            int64_t ldy, int accumulate, hipStream_t s) {
    switch (tt) {
    case 1: return launch_mfma_tt<1, F32X>(P, N, K, xt, ts, xf, ldx, M, y, ldy, accumulate, s);
    case 2: return launch_mfma_tt<2, F32X>(P, N, K, xt, ts, xf, ldx, M, y, ldy, accumulate, s);
    case 3: return launch_mfma_tt<3, F32X>(P, N, K, xt, ts, xf, ldx, M, y, ldy, accumulate, s);
    default: return launch_mfma_tt<4, F32X>(P, N, K, xt, ts, xf, ldx, M, y, ldy, accumulate, s);
    }
}

// Tokens in groups of 64 (four tiles) per launch.
hipError_t launch_gemv_mfma_q45(DevPlanes P, int64_t N, int64_t K, const void* xt, int64_t M,
                                float* y, int64_t ldy, int accumulate, hipStream_t stream) {
    const int64_t TT = (M + 15) / 16;
    const uint8_t* base = (const uint8_t*)xt;
    const float* ts = (const float*)(base + TT * (K / 32) * 2048);
    for (int64_t m0 = 0; m0 < M; m0 += 64) {
        const int mg = (int)(M - m0 < 64 ? M - m0 : 64);
        const u4v* xg = (const u4v*)(base + (m0 / 16) * (K / 32) * 2048);
        const hipError_t e = launch_tt<false>((mg + 15) / 16, P, N, K, xg, ts + m0, nullptr, 0, mg,
                                              y + m0 * ldy, ldy, accumulate, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// fp32 x: passes of 16 tokens (one token tile).  With more tiles the
// converted slab items and the weight ring outgrow the registers.
hipError_t launch_gemv_mfma_q45_f32x(DevPlanes P, int64_t N, int64_t K, const float* x,
                                     int64_t ldx, int64_t M, float* y, int64_t ldy,
                                     int accumulate, hipStream_t stream) {
    for (int64_t m0 = 0; m0 < M; m0 += 16) {
        const int mg = (int)(M - m0 < 16 ? M - m0 : 16);
        const hipError_t e = launch_mfma_tt<1, true>(P, N, K, nullptr, nullptr, x + m0 * ldx, ldx,
                                                     mg, y + m0 * ldy, ldy, accumulate, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace mbq
