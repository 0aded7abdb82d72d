// gemv_mfma.hip -- Y[m][n] (+)= W[n] . X[m] for batches of tokens on a Q45
// matrix, on the matrix cores (v_mfma_f32_16x16x32_f16).
//
// Past M* = (w/16)(R/BW) the sums, not the bytes, bound a product of many
// tokens, and the matrix units carry the sums ([roofline-holds] "The Math";
// "Two different problems": decode and prefill).  The arithmetic keeps the
// weights exact and x to 22 bits, as the vector kernels do:
//   * B (weights): a Q45 code q becomes the fp16 value q - 8 exactly (the
//     bits 0x6400 | q are 1024 + q; subtracting 1032 is exact);
//   * A (tokens): each 32-value block of each token is scaled by its own
//     power of two 2^e (the block's largest |x| lands in [2^14, 2^15)) and
//     split into fp16 high and low parts, 22 bits relative to the block;
//   * one pair of instructions (high part, then low part into the same
//     accumulator) covers exactly one 32-weight block, so its fp32 result D
//     takes the block's weight scale and 2^-e in the epilogue:
//     acc = fma(s, ldexp(D, -e), acc).
//
// Tile form of x (written by stage_x_mfma_kernel for the staged entry
// points; the fp32-x entry point converts into LDS the same way).  Per tile
// of 16 tokens:
//   blocks b = 0 .. K/32-1, 2 KB each: [high part 1 KB][low part 1 KB]; lane
//       l = 16 g + t of an instruction's A operand holds token t at
//       k = 32 b + 8 g + {0, 4, 1, 5, 2, 6, 3, 7} (the order in which a lane
//       unpacks the 8 codes of one dword), 16 bytes at 16 l;
//   then per quad of blocks u = 0 .. K/128-1, 64 bytes of exponents: byte
//       16 g + 4 i + r holds -e of token 4 g + r in block 4 u + i (int8).
//
// Kernel geometry: a workgroup of 8 waves covers RW row tiles (16 rows each)
// and TT token tiles.  K runs in chunks of 8 QW quads (128 values each): the
// chunk's x is brought into LDS once (QW quads per wave, TT tiles), and each
// wave multiplies its QW quads of the chunk against every row tile.  The
// weights of the next chunk are in flight while a chunk computes; they are
// the only vector-memory loads of the inner loop.  The 8 waves' partial tiles
// are added in wave order through LDS at the end.
#include "device_common.h"
#include "formats.h"
#include "kernels.h"

namespace mbq {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef float f4v __attribute__((ext_vector_type(4)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));
typedef uint32_t u2v __attribute__((ext_vector_type(2)));
typedef float f4g __attribute__((ext_vector_type(4)));

constexpr int kMW = 8;                        // waves per workgroup
constexpr int kMT = kMW * kWave;              // threads per workgroup
constexpr int kTileBlockBytes = 2048;         // one block of one token tile: high + low

// Bytes of the tile form of one token tile of K values.
__host__ __device__ __forceinline__ int64_t xt_tile_bytes(int64_t K) {
    return (K / 32) * kTileBlockBytes + (K / 128) * 64;
}

int64_t xt_bytes(int64_t M, int64_t K) { return (M + 15) / 16 * xt_tile_bytes(K); }

// ---- conversion of x into the tile form ---------------------------------
// One item = the 8 values of token t, block b, k-group g.  The four items of
// a (t, b) sit in four adjacent lanes (g = lane % 4), which combine their
// largest |x| with two lane exchanges.
struct XConv {
    u4v hi, lo;
    int ne;     // -e
};
__device__ __forceinline__ XConv convert_item(f4g a, f4g b) {
    float amax = fmaxf(fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))),
                       fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w))));
    amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
    amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
    // 2^e puts the largest |x| into [2^14, 2^15); e within the normal range
    int e = 141 - (int)((__builtin_bit_cast(uint32_t, amax) >> 23) & 0xFFu);
    e = e > 126 ? 126 : (e < -126 ? -126 : e);
    const float up = __builtin_bit_cast(float, (uint32_t)(e + 127) << 23);
    const float w[8] = {a.x, b.x, a.y, b.y, a.z, b.z, a.w, b.w};
    h8 hi, lo;
#pragma unroll
    for (int q = 0; q < 8; q++) {
        const float xs = w[q] * up;
        hi[q] = (_Float16)xs;
        lo[q] = (_Float16)(xs - (float)hi[q]);
    }
    return XConv{__builtin_bit_cast(u4v, hi), __builtin_bit_cast(u4v, lo), -e};
}

// Item index i of a region of nbt blocks per tile: g = i % 4, token t =
// (i / 4) % 16, block (i / 64) % nbt, tile i / (64 nbt).  Its destinations:
// the 16-byte slot of lane 16 g + t in the block's high and low kilobytes,
// and the exponent byte (within the tile's exponent area).
__device__ __forceinline__ int xt_slot(int b, int g, int t) { return b * kTileBlockBytes + (16 * g + t) * 16; }
__device__ __forceinline__ int xt_exp_byte(int b, int t) {
    return (b >> 2) * 64 + (t >> 2) * 16 + (b & 3) * 4 + (t & 3);
}

// ---- staging launch: fp32 x [M][ldx] -> tile form -------------------------
__global__ __launch_bounds__(kBlock) void stage_x_mfma_kernel(const float* __restrict__ x,
                                                              int64_t ldx, int M, int K,
                                                              uint8_t* __restrict__ xt,
                                                              int64_t nitems) {
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    const int nb = K / 32;
    // every lane of a quad takes part in the exchanges; items past the end
    // (only in the last workgroup) load nothing and store nothing
    const bool ok = i < nitems;
    const int g = (int)(i & 3), t = (int)((i >> 2) & 15);
    const int64_t r = i >> 6;
    const int b = (int)(r % nb);
    const int64_t tt = r / nb;
    const int64_t m = tt * 16 + t;
    f4g a = {0.f, 0.f, 0.f, 0.f}, c = {0.f, 0.f, 0.f, 0.f};
    if (ok && m < M) {
        const f4g* src = (const f4g*)(x + m * ldx + 32 * b + 8 * g);
        a = src[0];
        c = src[1];
    }
    const XConv v = convert_item(a, c);
    if (ok) {
        uint8_t* tile = xt + tt * xt_tile_bytes(K);
        *(u4v*)(tile + xt_slot(b, g, t)) = v.hi;
        *(u4v*)(tile + xt_slot(b, g, t) + 1024) = v.lo;
        if (g == 0) tile[(int64_t)nb * kTileBlockBytes + xt_exp_byte(b, t)] = (uint8_t)(int8_t)v.ne;
    }
}

hipError_t launch_stage_x_mfma(const float* x, int64_t M, int64_t ldx, int64_t K, void* xt,
                               hipStream_t stream) {
    const int64_t TTn = (M + 15) / 16;
    const int64_t nitems = TTn * (K / 32) * 64;
    const unsigned grid = (unsigned)((nitems + kBlock - 1) / kBlock);
    hipLaunchKernelGGL(stage_x_mfma_kernel, dim3(grid), dim3(kBlock), 0, stream, x, ldx, (int)M,
                       (int)K, (uint8_t*)xt, nitems);
    return hipGetLastError();
}

// ---- the product -----------------------------------------------------------
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
__device__ __forceinline__ h8 codes_to_b(uint32_t a) {
    const h2v off = {(_Float16)1032.0f, (_Float16)1032.0f};
    h2v w[4];
#pragma unroll
    for (int s = 0; s < 4; s++)
        w[s] = __builtin_bit_cast(h2v, ((a >> (4 * s)) & 0x000F000Fu) | 0x64006400u) - off;
    return h8{w[0][0], w[0][1], w[1][0], w[1][1], w[2][0], w[2][1], w[3][0], w[3][1]};
}

// Lane 16 g + j loaded 16 bytes = block 4u + g of row j (dword i = its
// k-group i).  After the exchange lane 16 g + j holds dword g of blocks
// 4u + 0 .. 4u + 3 of row j: the B operand of each of the 4 blocks.  Two
// rounds of swaps, across halves of the wave and across 16-lane rows.
__device__ __forceinline__ u4v quad_transpose(u4v d) {
    auto s02 = __builtin_amdgcn_permlane32_swap(d[0], d[2], false, false);
    auto s13 = __builtin_amdgcn_permlane32_swap(d[1], d[3], false, false);
    auto s01 = __builtin_amdgcn_permlane16_swap(s02[0], s13[0], false, false);
    auto s23 = __builtin_amdgcn_permlane16_swap(s02[1], s13[1], false, false);
    return u4v{s01[0], s01[1], s23[0], s23[1]};
}

typedef const void __attribute__((address_space(1)))* gvoid;
typedef void __attribute__((address_space(3)))* lvoid;

// s_waitcnt with vmcnt = n and the other counters left alone (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int n>
__device__ __forceinline__ void wait_vm() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// NCH: chunks of K, known at compile time for the common widths (the whole
// pipeline is then straight-line code and every wait names exactly the loads
// it needs); 0 when K is known only at run time.
template <int TT, int RW, int QW, int NCH, bool F32X>
__global__ __launch_bounds__(kMT) void gemv_mfma_q45_kernel(
        DevPlanes P, int N, int K, const uint8_t* __restrict__ xt, const float* __restrict__ xf,
        int64_t ldx, int M, float* __restrict__ y, int64_t ldy, int accumulate) {
    constexpr int QPC = kMW * QW;                 // quads per chunk
    constexpr int NBC = 4 * QPC;                  // blocks per chunk
    constexpr int XB = TT * NBC * kTileBlockBytes;   // LDS bytes of x per chunk
    // weight slots in registers: chunks whose loads are in flight or done
    constexpr int NS = NCH == 0 ? 2 : (NCH < (F32X ? 2 : 3) ? NCH : (F32X ? 2 : 3));
    constexpr int WLOADS = QW * RW * 2;           // load instructions of one chunk's weights
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int g = lane >> 4, j = lane & 15;
    const int nq = K / 128, nb = K / 32;
    const int nchunks = NCH > 0 ? NCH : (nq + QPC - 1) / QPC;
    const int row0 = blockIdx.x * (16 * RW);
    const int tt0 = blockIdx.y * TT;               // first token tile
    const int ntt = (M + 15) / 16;

    // weights: one resource per plane; lane (g, j) reads row j's block
    // 4u + g (16 bytes) and the 4 scales of quad u (8 bytes)
    const uint64_t nk = (uint64_t)N * (uint64_t)K;
    const Rsrc rc = make_rsrc(P.p0, nk / 2), rs = make_rsrc(P.p2, nk / 16);
    uint32_t co[RW], so[RW];
#pragma unroll
    for (int rt = 0; rt < RW; rt++) {
        const int row = min(row0 + 16 * rt + j, N - 1);
        co[rt] = (uint32_t)row * (uint32_t)(K / 2) + 16u * g;
        so[rt] = (uint32_t)row * (uint32_t)(K / 16);
    }
    u4v wc[NS][QW][RW];
    u2v ws[NS][QW][RW];
    auto load_w = [&](auto slot_c, int c) __attribute__((always_inline)) {
        constexpr int sl = decltype(slot_c)::value;
#pragma unroll
        for (int i = 0; i < QW; i++) {
            const int u = min(c * QPC + wave * QW + i, nq - 1);
#pragma unroll
            for (int rt = 0; rt < RW; rt++) {
                wc[sl][i][rt] = bload<u4v, true>(rc, co[rt], 64u * (uint32_t)u);
                ws[sl][i][rt] = bload<u2v, true>(rs, so[rt], 8u * (uint32_t)u);
            }
        }
    };

    // x of chunk c into LDS: [tt][block][2 KB], then [tt][quad][64 B].  The
    // copy is issued (fill_issue) and completed (fill_finish) in two steps,
    // so that loads issued between them stay in flight.
    constexpr int ITEMS = TT * NBC * 64;
    constexpr int IPT = F32X ? ITEMS / kMT : 1;
    static_assert(!F32X || ITEMS % kMT == 0, "items per thread");
    f4g va[IPT], vb[IPT];
    // Every workgroup reads the same x: each starts at its own piece or
    // block, so the workgroups of an XCD do not all ask one L2 channel for
    // the same lines at the same moment.
    const int rotb = (int)((blockIdx.x * 5u) % (unsigned)NBC);
    auto blk = [&](int i) __attribute__((always_inline)) { const int b = (i >> 6) % NBC + rotb; return b < NBC ? b : b - NBC; };
    auto fill_issue = [&](int c) __attribute__((always_inline)) {
        const int nbc = min(NBC, nb - c * NBC);        // valid blocks of this chunk
        if constexpr (F32X) {
#pragma unroll
            for (int s = 0; s < IPT; s++) {
                const int i = s * kMT + tid;
                const int gg = i & 3, t = (i >> 2) & 15, b = blk(i), tt = (i >> 6) / NBC;
                const int m = (tt0 + tt) * 16 + t;
                va[s] = f4g{0.f, 0.f, 0.f, 0.f};
                vb[s] = va[s];
                if (m < M && b < nbc) {
                    const f4g* src = (const f4g*)(xf + (int64_t)m * ldx + (int64_t)(c * NBC + b) * 32 + 8 * gg);
                    va[s] = src[0];
                    vb[s] = src[1];
                }
            }
        } else {
            // copies of 1 KB pieces (one per wave instruction), straight into LDS
            const int pieces_x = nbc * 2;                  // per tile
            const int pieces_e = (nbc * 16 + 1023) / 1024;   // exponent bytes per tile: 16 per block
            const int npc = TT * (pieces_x + pieces_e);
            const int rot = (int)((blockIdx.x * 37u) % (unsigned)npc);
#pragma unroll 1
            for (int p0 = wave; p0 < npc; p0 += kMW) {
                const int p = p0 + rot < npc ? p0 + rot : p0 + rot - npc;
                const int tt = p / (pieces_x + pieces_e), q = p % (pieces_x + pieces_e);
                const int ttg = min(tt0 + tt, ntt - 1);
                const uint8_t* tile = xt + (int64_t)ttg * xt_tile_bytes(K);
                if (q < pieces_x) {
                    __builtin_amdgcn_global_load_lds((gvoid)(tile + (int64_t)(c * NBC) * kTileBlockBytes + q * 1024 + 16 * lane),
                                                     (lvoid)(lds + tt * (NBC * kTileBlockBytes) + q * 1024), 16, 0, 0);
                } else {
                    const int e0 = (q - pieces_x) * 1024 + 16 * lane;   // byte within the chunk's exponents
                    if (e0 < nbc * 16)
                        __builtin_amdgcn_global_load_lds((gvoid)(tile + (int64_t)nb * kTileBlockBytes + (int64_t)(c * NBC) * 16 + e0),
                                                         (lvoid)(lds + XB + tt * (NBC * 16) + (q - pieces_x) * 1024), 16, 0, 0);
                }
            }
        }
    };
    // PEND: weight loads issued after fill_issue that may stay in flight.
    auto fill_finish = [&](auto pend_c) __attribute__((always_inline)) {
        constexpr int PEND = decltype(pend_c)::value;
        if constexpr (F32X) {
#pragma unroll
            for (int s = 0; s < IPT; s++) {
                const int i = s * kMT + tid;
                const int gg = i & 3, t = (i >> 2) & 15, b = blk(i), tt = (i >> 6) / NBC;
                const XConv v = convert_item(va[s], vb[s]);
                uint8_t* tile = lds + tt * (NBC * kTileBlockBytes);
                *(u4v*)(tile + xt_slot(b, gg, t)) = v.hi;
                *(u4v*)(tile + xt_slot(b, gg, t) + 1024) = v.lo;
                if (gg == 0) lds[XB + tt * (NBC * 16) + xt_exp_byte(b, t)] = (uint8_t)(int8_t)v.ne;
            }
        } else {
            wait_vm<PEND>();
        }
    };
    auto fill = [&](int c) __attribute__((always_inline)) {
        fill_issue(c);
        fill_finish(IC<0>{});
    };

    f4v acc[RW][TT];
#pragma unroll
    for (int rt = 0; rt < RW; rt++)
#pragma unroll
        for (int tt = 0; tt < TT; tt++) acc[rt][tt] = f4v{0.f, 0.f, 0.f, 0.f};
    const f4v zero = {0.f, 0.f, 0.f, 0.f};

    auto compute = [&](auto slot_c, int c) __attribute__((always_inline)) {
        constexpr int sl = decltype(slot_c)::value;
        const int nqc = NCH > 0 ? QPC : min(QPC, nq - c * QPC);   // quads of this chunk
#pragma unroll
        for (int i = 0; i < QW; i++) {
            const int ql = wave * QW + i;                  // quad within the chunk
            if (NCH == 0 && ql >= nqc) break;              // the same in every lane
            u4v cb[RW];
#pragma unroll
            for (int rt = 0; rt < RW; rt++) cb[rt] = quad_transpose(wc[sl][i][rt]);
            u4v ed[TT];
#pragma unroll
            for (int tt = 0; tt < TT; tt++) ed[tt] = *(const u4v*)(lds + XB + tt * (NBC * 16) + ql * 64 + 16 * g);
#pragma unroll
            for (int b = 0; b < 4; b++) {
                const int bl = 4 * ql + b;
                h8 xh[TT], xl[TT];
                int ne[TT][4];
#pragma unroll
                for (int tt = 0; tt < TT; tt++) {
                    const uint8_t* xb = lds + tt * (NBC * kTileBlockBytes) + bl * kTileBlockBytes + 16 * lane;
                    xh[tt] = __builtin_bit_cast(h8, *(const u4v*)xb);
                    xl[tt] = __builtin_bit_cast(h8, *(const u4v*)(xb + 1024));
#pragma unroll
                    for (int r = 0; r < 4; r++) ne[tt][r] = ((int32_t)(ed[tt][b] << (24 - 8 * r))) >> 24;
                }
#pragma unroll
                for (int rt = 0; rt < RW; rt++) {
                    const h8 bw = codes_to_b(cb[rt][b]);
                    const float sv = h2f(ws[sl][i][rt][b >> 1] >> (16 * (b & 1)));
#pragma unroll
                    for (int tt = 0; tt < TT; tt++) {
                        f4v d = __builtin_amdgcn_mfma_f32_16x16x32_f16(xh[tt], bw, zero, 0, 0, 0);
                        d = __builtin_amdgcn_mfma_f32_16x16x32_f16(xl[tt], bw, d, 0, 0, 0);
#pragma unroll
                        for (int r = 0; r < 4; r++)
                            acc[rt][tt][r] = fmaf(sv, __builtin_ldexpf(d[r], ne[tt][r]), acc[rt][tt][r]);
                    }
                }
            }
        }
    };

    if constexpr (NCH > 0) {
        // straight-line pipeline: NS chunks of weights in flight from the
        // start; after chunk c computes, chunk c + 1's x is copied in and
        // the slot chunk c used refills with chunk c + NS, whose loads go out
        // after the copy so that completing the copy does not wait for them
#pragma unroll
        for (int c = 0; c < NS; c++) {
            if (c == 0) load_w(IC<0>{}, 0);
            if (c == 1) load_w(IC<1 % NS>{}, 1);
            if (c == 2) load_w(IC<2 % NS>{}, 2);
        }
        fill(0);
        __syncthreads();
        static_for<0, NCH>([&](auto cc) __attribute__((always_inline)) {
            constexpr int c = decltype(cc)::value;
            compute(IC<c % NS>{}, c);
            if constexpr (c + 1 < NCH) {
                __syncthreads();
                fill_issue(c + 1);
                if constexpr (c + NS < NCH) {
                    load_w(IC<c % NS>{}, c + NS);
                    fill_finish(IC<WLOADS>{});
                } else {
                    fill_finish(IC<0>{});
                }
                __syncthreads();
            }
        });
    } else {
        // K known only at run time: two slots, chunk c + 1's weights load
        // while chunk c computes
        load_w(IC<0>{}, 0);
        fill(0);
        __syncthreads();
#pragma unroll 1
        for (int c = 0; c < nchunks; c += 2) {
            if (c + 1 < nchunks) load_w(IC<1>{}, c + 1);
            compute(IC<0>{}, c);
            if (c + 1 >= nchunks) break;
            __syncthreads();
            fill(c + 1);
            __syncthreads();
            if (c + 2 < nchunks) load_w(IC<0>{}, c + 2);
            compute(IC<1>{}, c + 1);
            if (c + 2 >= nchunks) break;
            __syncthreads();
            fill(c + 2);
            __syncthreads();
        }
    }

    // the 8 waves' partial tiles, added in wave order
    __syncthreads();
    f4v* red = (f4v*)lds;                                  // [wave][rt][tt][lane]
#pragma unroll
    for (int rt = 0; rt < RW; rt++)
#pragma unroll
        for (int tt = 0; tt < TT; tt++) red[((wave * RW + rt) * TT + tt) * kWave + lane] = acc[rt][tt];
    __syncthreads();
#pragma unroll 1
    for (int u = wave; u < RW * TT; u += kMW) {
        const int rt = u / TT, tt = u % TT;
        f4v s = red[(rt * TT + tt) * kWave + lane];
#pragma unroll
        for (int w = 1; w < kMW; w++) {
            const f4v o = red[((w * RW + rt) * TT + tt) * kWave + lane];
            s += o;
        }
        // lane 16 g + j holds tokens 4 g + r of the tile, row j of the row tile
        const int n = row0 + 16 * rt + j;
        if (n >= N) continue;
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int m = (tt0 + tt) * 16 + 4 * g + r;
            if (m < M) {
                float* dst = y + (int64_t)m * ldy + n;
                *dst = accumulate ? *dst + s[r] : s[r];
            }
        }
    }
}

template <int TT, int RW, int QW, int NCH, bool F32X>
static hipError_t launch_k(DevPlanes P, int64_t N, int64_t K, const uint8_t* xt, const float* xf,
                           int64_t ldx, int64_t M, float* y, int64_t ldy, int accumulate,
                           hipStream_t stream) {
    constexpr int NBC = 4 * kMW * QW;
    constexpr size_t xl = (size_t)TT * NBC * kTileBlockBytes + (size_t)TT * NBC * 16;
    constexpr size_t rl = (size_t)kMW * RW * TT * kWave * 16;
    constexpr size_t lds = xl > rl ? xl : rl;
    auto kern = gemv_mfma_q45_kernel<TT, RW, QW, NCH, F32X>;
    if (hipError_t e = ensure_lds<gemv_mfma_q45_kernel<TT, RW, QW, NCH, F32X>>(lds)) return e;
    const int64_t ntt = (M + 15) / 16;
    const dim3 grid((unsigned)((N + 16 * RW - 1) / (16 * RW)), (unsigned)((ntt + TT - 1) / TT));
    hipLaunchKernelGGL(kern, grid, dim3(kMT), lds, stream, P, (int)N, (int)K, xt, xf, ldx, (int)M, y,
                       ldy, accumulate);
    return hipGetLastError();
}

template <int TT, int RW, bool F32X>
static hipError_t launch_rw(DevPlanes P, int64_t N, int64_t K, const uint8_t* xt, const float* xf,
                            int64_t ldx, int64_t M, float* y, int64_t ldy, int accumulate,
                            hipStream_t s) {
    constexpr int QW = TT == 1 ? 2 : 1;    // chunk of x: 128 KB of LDS
    constexpr int KC = kMW * QW * 128;     // values per chunk
    // fp32 x keeps the run-time loop: unrolled, its conversion registers and
    // the weight slots outgrow the register file
    if (F32X) return launch_k<TT, RW, QW, 0, F32X>(P, N, K, xt, xf, ldx, M, y, ldy, accumulate, s);
    if (K == 4096) return launch_k<TT, RW, QW, 4096 / KC, F32X>(P, N, K, xt, xf, ldx, M, y, ldy, accumulate, s);
    if (K == 12288) return launch_k<TT, RW, QW, 12288 / KC, F32X>(P, N, K, xt, xf, ldx, M, y, ldy, accumulate, s);
    return launch_k<TT, RW, QW, 0, F32X>(P, N, K, xt, xf, ldx, M, y, ldy, accumulate, s);
}

// Row tiles per workgroup: about 256 workgroups per token-tile group (one
// per compute unit), at most 4 tiles; MBQ_MFMA_RW overrides (tuning).
template <int TT, bool F32X>
static hipError_t launch_tt(DevPlanes P, int64_t N, int64_t K, const uint8_t* xt, const float* xf,
                            int64_t ldx, int64_t M, float* y, int64_t ldy, int accumulate,
                            hipStream_t s) {
    int64_t rw = (N + 16 * 256 - 1) / (16 * 256);
    if (const char* e = tuning_var("MBQ_MFMA_RW")) rw = atoi(e);
    switch (rw <= 1 ? 1 : rw == 2 ? 2 : rw == 3 ? 3 : 4) {
    case 1: return launch_rw<TT, 1, F32X>(P, N, K, xt, xf, ldx, M, y, ldy, accumulate, s);
    case 2: return launch_rw<TT, 2, F32X>(P, N, K, xt, xf, ldx, M, y, ldy, accumulate, s);
    case 3: return launch_rw<TT, 3, F32X>(P, N, K, xt, xf, ldx, M, y, ldy, accumulate, s);
    default: return launch_rw<TT, 4, F32X>(P, N, K, xt, xf, ldx, M, y, ldy, accumulate, s);
    }
}

// One or two token tiles per workgroup: one tile up to 16 tokens, else two
// (the grid covers the rest); MBQ_MFMA_TT = 1 forces one (tuning).
static int pick_tt(int64_t M) {
    int tt = M <= 16 ? 1 : 2;
    if (const char* e = tuning_var("MBQ_MFMA_TT")) tt = atoi(e) == 1 ? 1 : 2;
    return tt;
}

hipError_t launch_gemv_mfma_q45(DevPlanes P, int64_t N, int64_t K, const void* xt, int64_t M,
                                float* y, int64_t ldy, int accumulate, hipStream_t stream) {
    const uint8_t* x = (const uint8_t*)xt;
    return pick_tt(M) == 1 ? launch_tt<1, false>(P, N, K, x, nullptr, 0, M, y, ldy, accumulate, stream)
                           : launch_tt<2, false>(P, N, K, x, nullptr, 0, M, y, ldy, accumulate, stream);
}

hipError_t launch_gemv_mfma_q45_f32x(DevPlanes P, int64_t N, int64_t K, const float* x,
                                     int64_t ldx, int64_t M, float* y, int64_t ldy,
                                     int accumulate, hipStream_t stream) {
    return pick_tt(M) == 1 ? launch_tt<1, true>(P, N, K, nullptr, x, ldx, M, y, ldy, accumulate, stream)
                           : launch_tt<2, true>(P, N, K, nullptr, x, ldx, M, y, ldy, accumulate, stream);
}

}  // namespace mbq
