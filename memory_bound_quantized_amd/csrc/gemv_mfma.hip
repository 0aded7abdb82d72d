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
// points; the fp32-x entry point converts in registers the same way).  Per tile
// of 16 tokens:
//   blocks b = 0 .. K/32-1, 2 KB each: [high part 1 KB][low part 1 KB]; lane
//       l = 16 g + t of an instruction's A operand holds token t at
//       k = 32 b + 8 g + {0, 4, 1, 5, 2, 6, 3, 7} (the order in which a lane
//       unpacks the 8 codes of one dword), 16 bytes at 16 l;
//   then per quad of blocks u = 0 .. K/128-1, 64 bytes of exponents: byte
//       16 g + 4 i + r holds -e of token 4 g + r in block 4 u + i (int8).
//
// Kernel geometry: a workgroup of MW waves (16 for one token tile, 8 for
// two) covers RW row tiles (16 rows each) and TT token tiles; the waves
// split K.  Wave w takes quads (128 values of K) w, w + MW, w + 2 MW, ...:
// for each it reads the RW row tiles' codes and scales and the TT tiles' x
// straight into registers and multiplies every row tile by every token tile,
// so each byte of x reaches the compute unit once and is used RW times, each
// weight once and used TT times.  There is no barrier in the stream: the
// next quad's weights are loaded as soon as the current ones are transposed,
// and each block of its x as soon as the same block of the current quad is
// used.  The waves' partial tiles are added in wave order through LDS at the
// end, so the sums depend on MW but not on RW or TT.
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
    amax = fmaxf(amax, lane_xor1(amax));
    amax = fmaxf(amax, lane_xor2(amax));
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

// (v & mask) | bits in one instruction.  Written out because the compiler
// splits it into an and and an or whenever both constants are literals.
__device__ __forceinline__ uint32_t and_or(uint32_t v, uint32_t mask, uint32_t bits) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(v), "s"(mask), "v"(bits));
    return r;
}

// 8 codes of one dword as fp16 (q - 8), in the order {0,4,1,5,2,6,3,7}:
// each pair of nibbles becomes the halves 1024 + q (bits 0x6400 | q), and
// one packed subtraction of 1032 leaves q - 8 exactly.
__device__ __forceinline__ h8 codes_to_b(uint32_t a, uint32_t exp_bits) {
    const h2v off = {(_Float16)1032.0f, (_Float16)1032.0f};
    h2v w[4];
#pragma unroll
    for (int s = 0; s < 4; s++)
        w[s] = __builtin_bit_cast(h2v, and_or(a >> (4 * s), 0x000F000Fu, exp_bits)) - off;
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

// 4 x 4 transpose within each quad of lanes: register r of lane 4 q + i
// becomes register i of lane 4 q + r.  Two rounds of 2 x 2 exchanges, with
// the partner lane's value brought in by DPP (lane ^ 1, then lane ^ 2).
__device__ __forceinline__ u4v lane_quad_transpose(u4v x, int lane) {
    constexpr int kXor1 = 0xB1, kXor2 = 0x4E;     // quad_perm [1,0,3,2], [2,3,0,1]
    const bool o1 = lane & 1, o2 = lane & 2;
    auto dpp = [](uint32_t v, auto ctrl_c) __attribute__((always_inline)) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, decltype(ctrl_c)::value, 0xF, 0xF, false);
    };
    // lane bit 0 <-> register bit 0
    const uint32_t a0 = dpp(x[0], IC<kXor1>{}), a1 = dpp(x[1], IC<kXor1>{});
    const uint32_t a2 = dpp(x[2], IC<kXor1>{}), a3 = dpp(x[3], IC<kXor1>{});
    const uint32_t t0 = o1 ? a1 : x[0], t1 = o1 ? x[1] : a0;
    const uint32_t t2 = o1 ? a3 : x[2], t3 = o1 ? x[3] : a2;
    // lane bit 1 <-> register bit 1
    const uint32_t b0 = dpp(t0, IC<kXor2>{}), b1 = dpp(t1, IC<kXor2>{});
    const uint32_t b2 = dpp(t2, IC<kXor2>{}), b3 = dpp(t3, IC<kXor2>{});
    return u4v{o2 ? b2 : t0, o2 ? b3 : t1, o2 ? t2 : b0, o2 ? t3 : b1};
}

// A copy of v that the compiler cannot prove equal to v.  The swaps below
// take the same value twice, and the compiler folds a swap of two equal
// operands into two equal results, which drops the exchange across lanes.
__device__ __forceinline__ uint32_t opaque_copy(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}

// Largest of the non-negative floats with bits v over lanes l, l ^ 16,
// l ^ 32, l ^ 48 (the four k-groups of one token's block in the A-operand
// layout).  Swapping a value with itself across halves, then rows, hands
// each lane its own and its partner's value.  The maximum is taken on the
// bits (for non-negative floats the same order): compiled as a float
// maximum, the compiler dropped the swap's second result.
__device__ __forceinline__ uint32_t max_over_rows(uint32_t v) {
    auto h = __builtin_amdgcn_permlane32_swap(v, opaque_copy(v), false, false);
    v = h[0] > h[1] ? h[0] : h[1];
    auto q = __builtin_amdgcn_permlane16_swap(v, opaque_copy(v), false, false);
    return q[0] > q[1] ? q[0] : q[1];
}

// The conversion of convert_item for a lane that holds token t's k-group g of
// one block (lane 16 g + t): the block maximum combines the four lanes of
// the token across 16-lane rows.  Same values, same results.
__device__ __forceinline__ XConv convert_lane(f4g a, f4g b) {
    float amax = fmaxf(fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))),
                       fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w))));
    const uint32_t mbits = max_over_rows(__builtin_bit_cast(uint32_t, amax));
    int e = 141 - (int)((mbits >> 23) & 0xFFu);
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

// Sign-extended byte i of w.
__device__ __forceinline__ int sbyte(uint32_t w, int i) { return ((int32_t)(w << (24 - 8 * i))) >> 24; }

// One wave's operands for one quad (128 values of K): the codes and scales
// of RW row tiles and, per token tile, the exponents and the 4 blocks of x
// (high and low parts; fp32 x in two halves before conversion).
template <int TT, int RW, bool F32X>
struct QuadOps {
    u4v wc[RW];
    u2v ws[RW];
    u4v ed[TT];
    u4v x0[4][TT], x1[4][TT];
};

// NSTEP: quads per wave when K is known at compile time (K = 1024 NSTEP),
// so that the whole stream is straight-line code; 0 for K known only at run
// time.
// MW waves per workgroup, one workgroup per compute unit: MW / 4 waves per
// SIMD is the occupancy it needs.  Telling the compiler so keeps it from
// sinking the next quad's loads next to their uses to save registers for an
// occupancy the grid never reaches.
template <int MW, int TT, int RW, int NSTEP, bool F32X, int S>
__global__ __launch_bounds__(MW * kWave) __attribute__((amdgpu_waves_per_eu(MW / 4, MW / 4))) void gemv_mfma_q45_kernel(
        DevPlanes P, int N, int K, const uint8_t* __restrict__ xt, const float* __restrict__ xf,
        int64_t ldx, int M, float* __restrict__ y, int64_t ldy, int accumulate,
        float* __restrict__ part, uint32_t* __restrict__ ctr) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int g = lane >> 4, j = lane & 15;
    // K split S ways (gridDim.z = S): workgroup z takes quads z nq .. z nq + nq - 1
    const int z = S > 1 ? (int)blockIdx.z : 0;
    const int nq = K / 128 / S, qbase = z * nq;
    const int nstep = NSTEP > 0 ? NSTEP : (nq + MW - 1) / MW;
    const int row0 = blockIdx.x * (16 * RW);
    const int tt0 = blockIdx.y * TT;               // first token tile
    const int ntt = (M + 15) / 16;

    // codes: a quad of lanes 4 a + b reads 64 contiguous bytes, blocks
    // b = 0..3 of quad u of row tau(a) = 4 (a & 3) + (a >> 2) of the row tile
    // (one cache line access per 4 lanes).  lane_quad_transpose then
    // quad_transpose (lane bits 1..0 and 5..4 exchanged with the register
    // index) leave lane 16 g + j with dword g of the 4 blocks of row j.
    const uint64_t nk = (uint64_t)N * (uint64_t)K;
    const Rsrc rc = make_rsrc(P.p0, nk / 2);
    uint32_t co[RW];
    {
        const int a = lane >> 2, tau = 4 * (a & 3) + (a >> 2);
#pragma unroll
        for (int rt = 0; rt < RW; rt++) {
            const int row = min(row0 + 16 * rt + tau, N - 1);
            co[rt] = (uint32_t)row * (uint32_t)(K / 2) + 16u * (uint32_t)(lane & 3);
        }
    }
    // scales: lane (g, j) reads the 4 scales of quad u of row j (8 bytes)
    const Rsrc rs = make_rsrc(P.p2, nk / 16);
    uint32_t so[RW];
#pragma unroll
    for (int rt = 0; rt < RW; rt++) so[rt] = (uint32_t)min(row0 + 16 * rt + j, N - 1) * (uint32_t)(K / 16);
    // x: staged, one resource per token tile (lane l reads the 16 bytes at
    // 16 l of each kilobyte); fp32, lane (g, t) reads token t's 8 values of
    // k-group g (rows past M repeat row M - 1: their sums are never stored)
    Rsrc rx[TT];
    const float* xr[TT];
#pragma unroll
    for (int tt = 0; tt < TT; tt++) {
        const int ttg = min(tt0 + tt, ntt - 1);
        if constexpr (F32X) {
            const int m = min(ttg * 16 + j, M - 1);
            xr[tt] = xf + (int64_t)m * ldx + 8 * g;
        } else {
            const int64_t tb = xt_tile_bytes(K);
            rx[tt] = make_rsrc(xt + (int64_t)ttg * tb, (uint64_t)tb);
        }
    }
    const uint32_t eoff = (uint32_t)(K / 32) * kTileBlockBytes + 16u * g;

    typedef QuadOps<TT, RW, F32X> Q;
    // quad of step s: the waves interleave, so that two adjacent waves read
    // the two halves of each 128-byte line of a row at about the same time;
    // past the end (run-time K only) the last quad is read again and not used
    auto quad = [&](int s) __attribute__((always_inline)) { return qbase + min(wave + MW * s, nq - 1); };
    auto load_w = [&](Q& q, int u) __attribute__((always_inline)) {
#pragma unroll
        for (int rt = 0; rt < RW; rt++) {
            q.wc[rt] = bload<u4v, true>(rc, co[rt], 64u * (uint32_t)u);
            q.ws[rt] = bload<u2v, true>(rs, so[rt], 8u * (uint32_t)u);
        }
        if constexpr (!F32X) {
#pragma unroll
            for (int tt = 0; tt < TT; tt++) q.ed[tt] = bload<u4v, true>(rx[tt], eoff, 64u * (uint32_t)u);
        }
    };
    auto load_x = [&](Q& q, int b, int u) __attribute__((always_inline)) {
#pragma unroll
        for (int tt = 0; tt < TT; tt++) {
            if constexpr (F32X) {
                const f4g* src = (const f4g*)(xr[tt] + 32 * (4 * u + b));
                q.x0[b][tt] = __builtin_bit_cast(u4v, src[0]);
                q.x1[b][tt] = __builtin_bit_cast(u4v, src[1]);
            } else {
                const uint32_t off = (uint32_t)(4 * u + b) * kTileBlockBytes + 16u * lane;
                q.x0[b][tt] = bload<u4v, true>(rx[tt], off, 0u);
                q.x1[b][tt] = bload<u4v, true>(rx[tt], off + 1024u, 0u);
            }
        }
    };

    f4v acc[RW][TT];
#pragma unroll
    for (int rt = 0; rt < RW; rt++)
#pragma unroll
        for (int tt = 0; tt < TT; tt++) acc[rt][tt] = f4v{0.f, 0.f, 0.f, 0.f};
    const f4v zero = {0.f, 0.f, 0.f, 0.f};
    const uint32_t exp_bits = opaque_copy(0x64006400u);    // kept in a register for and_or

    // One step: multiply quad q (in cur) and load quad un into cur: the
    // weights and exponents first (their registers are free once copied),
    // then each block of x right after the same block of cur is used.
    // LOAD false: the last step of a compile-time stream loads nothing.
    auto step = [&](auto load_c, Q& cur, bool use, int un) __attribute__((always_inline)) {
        constexpr bool LOAD = decltype(load_c)::value;
        u4v cb[RW];
        u2v sc[RW];
#pragma unroll
        for (int rt = 0; rt < RW; rt++) {
            cb[rt] = lane_quad_transpose(quad_transpose(cur.wc[rt]), lane);
            sc[rt] = cur.ws[rt];
        }
        u4v ed[TT];
#pragma unroll
        for (int tt = 0; tt < TT; tt++) ed[tt] = cur.ed[tt];
        if constexpr (LOAD) load_w(cur, un);
#pragma unroll
        for (int b = 0; b < 4; b++) {
            h8 xh[TT], xl[TT];
            int ne[TT][4];
#pragma unroll
            for (int tt = 0; tt < TT; tt++) {
                if constexpr (F32X) {
                    const XConv v = convert_lane(__builtin_bit_cast(f4g, cur.x0[b][tt]),
                                                 __builtin_bit_cast(f4g, cur.x1[b][tt]));
                    xh[tt] = __builtin_bit_cast(h8, v.hi);
                    xl[tt] = __builtin_bit_cast(h8, v.lo);
                    // -e of tokens 4 g + r sit in lanes 4 g + r
#pragma unroll
                    for (int r = 0; r < 4; r++) ne[tt][r] = __shfl(v.ne, 4 * g + r, kWave);
                } else {
                    xh[tt] = __builtin_bit_cast(h8, cur.x0[b][tt]);
                    xl[tt] = __builtin_bit_cast(h8, cur.x1[b][tt]);
#pragma unroll
                    for (int r = 0; r < 4; r++) ne[tt][r] = sbyte(ed[tt][b], r);
                }
            }
            if constexpr (LOAD) load_x(cur, b, un);
            if (!use) continue;                        // the same in every lane
#pragma unroll
            for (int rt = 0; rt < RW; rt++) {
                const h8 bw = codes_to_b(cb[rt][b], exp_bits);
                const float sv = h2f(sc[rt][b >> 1] >> (16 * (b & 1)));
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
    };

    Q cur;
    load_w(cur, quad(0));
#pragma unroll
    for (int b = 0; b < 4; b++) load_x(cur, b, quad(0));
    if constexpr (NSTEP > 0) {
        // every wave has exactly NSTEP quads
        static_for<0, NSTEP>([&](auto ss) __attribute__((always_inline)) {
            constexpr int s = decltype(ss)::value;
            step(IC<(s + 1 < NSTEP)>{}, cur, true, quad(s + 1 < NSTEP ? s + 1 : s));
        });
    } else {
#pragma unroll 1
        for (int s = 0; s < nstep; s++) step(IC<1>{}, cur, wave + MW * s < nq, quad(s + 1));
    }

    // the waves' partial tiles, added in wave order
    f4v* red = (f4v*)lds;                                  // [wave][rt][tt][lane]
#pragma unroll
    for (int rt = 0; rt < RW; rt++)
#pragma unroll
        for (int tt = 0; tt < TT; tt++) red[((wave * RW + rt) * TT + tt) * kWave + lane] = acc[rt][tt];
    __syncthreads();
#pragma unroll 1
    for (int u = wave; u < RW * TT; u += MW) {
        const int rt = u / TT, tt = u % TT;
        f4v s = red[(rt * TT + tt) * kWave + lane];
#pragma unroll
        for (int w = 1; w < MW; w++) {
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
                if constexpr (S > 1) {
                    __hip_atomic_store(part + ((int64_t)z * M + m) * N + n, s[r], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                } else {
                    float* dst = y + (int64_t)m * ldy + n;
                    *dst = accumulate ? *dst + s[r] : s[r];
                }
            }
        }
    }
    if constexpr (S > 1) {
        // K split: the last of the S workgroups of this tile to finish adds
        // the partial tiles in split order (the sums do not depend on which
        // one is last), then zeroes them and the tile's counter, so that
        // every call leaves the workspace as it found it: all zero.
        // Ordering without cache maintenance: the partials and the counter
        // are only ever accessed as agent-scope atomics, which the compiler
        // makes coherent across the compute dies by writing through and
        // reading past their L2s; each wave waits for its partial stores to
        // complete before the barrier that precedes the counter increment,
        // and the last workgroup reads the partials only after the increment
        // returns.  An agent-scope release/acquire pair would do the same by
        // writing back and invalidating each die's whole L2, which throws
        // away the L2-resident x of every other workgroup on that die.
        __builtin_amdgcn_s_waitcnt(0);                   // every counter, stores included
        __syncthreads();
        uint32_t* c = ctr + (blockIdx.y * gridDim.x + blockIdx.x);
        __shared__ int last;
        if (tid == 0)
            last = __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(S - 1);
        __syncthreads();
        if (!last) return;
        // each thread's NOUT outputs: every load issued before any is used
        // (one memory round trip); rows and tokens past the end read a
        // clamped address of this tile and store nothing
        constexpr int NOUT = 16 * RW * 16 * TT / (MW * kWave);
        static_assert(NOUT * MW * kWave == 16 * RW * 16 * TT, "tile not a multiple of the workgroup");
        float t[NOUT][S], y0[NOUT];
        int64_t pi[NOUT], yi[NOUT];
        bool ok[NOUT];
#pragma unroll
        for (int i = 0; i < NOUT; i++) {
            const int o = tid + i * MW * kWave;
            const int n = row0 + o % (16 * RW), m = tt0 * 16 + o / (16 * RW);
            ok[i] = n < N && m < M;
            const int nc = min(n, N - 1), mc = min(m, M - 1);
            pi[i] = (int64_t)mc * N + nc;
            yi[i] = (int64_t)mc * ldy + nc;
#pragma unroll
            for (int zz = 0; zz < S; zz++)
                t[i][zz] = __hip_atomic_load(part + pi[i] + (int64_t)zz * M * N, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
            y0[i] = accumulate ? y[yi[i]] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < NOUT; i++) {
            if (!ok[i]) continue;
            float v = t[i][0];
#pragma unroll
            for (int zz = 1; zz < S; zz++) v += t[i][zz];
#pragma unroll
            for (int zz = 0; zz < S; zz++)
                __hip_atomic_store(part + pi[i] + (int64_t)zz * M * N, 0.f, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            y[yi[i]] = accumulate ? y0[i] + v : v;
        }
        if (tid == 0) __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <int MW, int TT, int RW, int NSTEP, bool F32X, int S = 1>
static hipError_t launch_k(DevPlanes P, int64_t N, int64_t K, const uint8_t* xt, const float* xf,
                           int64_t ldx, int64_t M, float* y, int64_t ldy, int accumulate,
                           hipStream_t stream, float* part = nullptr, uint32_t* ctr = nullptr) {
    constexpr size_t lds = (size_t)MW * RW * TT * kWave * 16;
    auto kern = gemv_mfma_q45_kernel<MW, TT, RW, NSTEP, F32X, S>;
    if (hipError_t e = ensure_lds<gemv_mfma_q45_kernel<MW, TT, RW, NSTEP, F32X, S>>(lds)) return e;
    const int64_t ntt = (M + 15) / 16;
    const dim3 grid((unsigned)((N + 16 * RW - 1) / (16 * RW)), (unsigned)((ntt + TT - 1) / TT), (unsigned)S);
    hipLaunchKernelGGL(kern, grid, dim3(MW * kWave), lds, stream, P, (int)N, (int)K, xt, xf, ldx,
                       (int)M, y, ldy, accumulate, part, ctr);
    return hipGetLastError();
}

// Waves per workgroup: 16 for one token tile (4 per SIMD) where the
// registers fit 128 without spilling (up to 3 row tiles, 4 at K = 4096),
// else 8 (2 per SIMD); 4 (one per SIMD, up to 512 registers) for four token
// tiles.  MBQ_MFMA_MW = 8 forces 8 for one tile (tuning).
template <int TT, int RW, bool F32X>
static hipError_t launch_rw(DevPlanes P, int64_t N, int64_t K, const uint8_t* xt, const float* xf,
                            int64_t ldx, int64_t M, float* y, int64_t ldy, int accumulate,
                            hipStream_t s) {
    if constexpr (TT == 1) {
        bool mw16 = K == 4096 || (K == 12288 && RW <= 3) || RW <= 2;
        if (const char* e = tuning_var("MBQ_MFMA_MW")) mw16 = mw16 && atoi(e) != 8;
        if (mw16) {
            constexpr int MW = 16, KS = MW * 128;      // values per step of the workgroup
            if (K == 4096) return launch_k<MW, TT, RW, 4096 / KS, F32X>(P, N, K, xt, xf, ldx, M, y, ldy, accumulate, s);
            if constexpr (RW <= 3)
                if (K == 12288) return launch_k<MW, TT, RW, 12288 / KS, F32X>(P, N, K, xt, xf, ldx, M, y, ldy, accumulate, s);
            if constexpr (RW <= 2) return launch_k<MW, TT, RW, 0, F32X>(P, N, K, xt, xf, ldx, M, y, ldy, accumulate, s);
        }
    }
    constexpr int MW = TT == 4 ? 4 : 8, KS = MW * 128;
    if (K == 4096) return launch_k<MW, TT, RW, 4096 / KS, F32X>(P, N, K, xt, xf, ldx, M, y, ldy, accumulate, s);
    // four token tiles: the 24-step stream of K = 12288 takes minutes to
    // compile for little gain over the loop
    if constexpr (TT < 4)
        if (K == 12288) return launch_k<MW, TT, RW, 12288 / KS, F32X>(P, N, K, xt, xf, ldx, M, y, ldy, accumulate, s);
    return launch_k<MW, TT, RW, 0, F32X>(P, N, K, xt, xf, ldx, M, y, ldy, accumulate, s);
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

// Token tiles per workgroup: one up to 16 tokens, two up to 32, else four
// (the grid covers the rest): each code a workgroup converts serves TT
// tiles.  MBQ_MFMA_TT overrides (tuning).
static int pick_tt(int64_t M) {
    int tt = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
    if (const char* e = tuning_var("MBQ_MFMA_TT")) {
        const int v = atoi(e);
        tt = v <= 1 ? 1 : (v == 2 ? 2 : 4);
    }
    return tt;
}

hipError_t launch_gemv_mfma_q45(DevPlanes P, int64_t N, int64_t K, const void* xt, int64_t M,
                                float* y, int64_t ldy, int accumulate, hipStream_t stream) {
    const uint8_t* x = (const uint8_t*)xt;
    switch (pick_tt(M)) {
    case 1: return launch_tt<1, false>(P, N, K, x, nullptr, 0, M, y, ldy, accumulate, stream);
    case 2: return launch_tt<2, false>(P, N, K, x, nullptr, 0, M, y, ldy, accumulate, stream);
    default: return launch_tt<4, false>(P, N, K, x, nullptr, 0, M, y, ldy, accumulate, stream);
    }
}

// ---- the K split (the workspace-taking entry point) -------------------------
// Every compute unit of the stream above reads all of x for its rows.  Split
// S ways along K, a workgroup covers S times the rows over 1/S of K, so it
// reads 1/S of the x for the same weights; the S partial tiles meet in the
// workspace, and the last workgroup of a tile adds them (about 2 us of
// memory round trips at the end).  Shapes by the unsplit row tiles per
// workgroup, rw1 = N / 4096 rounded up: rw1 = 1 splits in 4 (4 row tiles),
// rw1 = 2 or 3 in 2 (4 or 6 row tiles), more rows not at all.  Where it
// pays, measured on the 36-layer model's tables (graphs of cold launches,
// warmed clocks, best of two in alternating order; us at 16 / 64 / 512
// tokens, K whole -> split):
//   rw1 = 1: K >= 12288 (4096 x 12288: 18.8 -> 15.3, 46.1 -> 32.8,
//            309 -> 217), or more than 32 tokens (4096 x 4096: 16.2 ->
//            15.7 and 98.8 -> 87.9; 8.0 -> 8.4 at 16, where each part has
//            one step per wave);
//   rw1 = 2: more than 32 tokens (6144 x 4096: 20.4 -> 20.2, 104 -> 101;
//            10.0 -> 11.3 at 16);
//   rw1 = 3: K >= 12288 and more than 32 tokens (12288 x 12288: 76.4 ->
//            76.0, 556 -> 548; 12288 x 4096 is slower split at every
//            batch, 13.2 -> 15.7, 26.7 -> 33.6, 184 -> 223).
// It also needs K / 128 to be a whole number of steps of every part.
// MBQ_MFMA_SPLIT (tuning): 1 never splits, 2 splits every shape that has a
// split form.
SplitPlan mfma_split_plan(int64_t N, int64_t K, int64_t M) {
    SplitPlan p{1, 0, 0, 0};
    const int64_t ntt = (M + 15) / 16;
    const int tt = pick_tt(M);
    const int mw = tt == 4 ? 4 : 8;
    const int64_t rw1 = (N + 16 * 256 - 1) / (16 * 256);
    const int64_t nq = K / 128;
    int S = rw1 == 1 ? 4 : (rw1 <= 3 ? 2 : 1);
    bool want = rw1 == 1 ? (K >= 12288 || M > 32) : rw1 == 2 ? M > 32 : (K >= 12288 && M > 32);
    if (const char* e = tuning_var("MBQ_MFMA_SPLIT")) {
        const int v = atoi(e);
        if (v == 1) want = false;
        if (v == 2) want = true;
    }
    // two token tiles of 6 row tiles spill in the run-time-K loop
    if (tt == 2 && rw1 == 3 && K != 4096 && K != 12288) want = false;
    if (want && S > 1 && N > 0 && M > 0 && nq % (S * mw) == 0) {
        p.S = S;
        p.RW = (int)(S * rw1);
        p.gx = (N + 16 * p.RW - 1) / (16 * p.RW);
        p.gy = (ntt + tt - 1) / tt;
    }
    return p;
}

// Workspace: one counter per output tile, then the partial tiles
// [S][M][N] fp32 from the next 256-byte boundary.
static size_t split_ctr_bytes(const SplitPlan& p) {
    return ((size_t)p.gx * (size_t)p.gy * 4 + 255) / 256 * 256;
}

size_t mfma_split_workspace_bytes(int64_t N, int64_t K, int64_t M) {
    const SplitPlan p = mfma_split_plan(N, K, M);
    if (p.S == 1) return 0;
    return split_ctr_bytes(p) + (size_t)p.S * (size_t)M * (size_t)N * 4;
}

template <int TT, int RW, int S>
static hipError_t launch_split_s(DevPlanes P, int64_t N, int64_t K, const uint8_t* xt, int64_t M, float* y,
                                 int64_t ldy, int accumulate, hipStream_t s, float* part, uint32_t* ctr) {
    constexpr int MW = TT == 4 ? 4 : 8, KS = S * MW * 128;   // values per step of all S parts
    // four token tiles of 6 row tiles spill as a straight-line stream
    if constexpr (TT == 4 && RW == 6) {
        return launch_k<MW, TT, RW, 0, false, S>(P, N, K, xt, nullptr, 0, M, y, ldy, accumulate, s, part, ctr);
    } else {
        if constexpr (4096 % KS == 0)
            if (K == 4096) return launch_k<MW, TT, RW, 4096 / KS, false, S>(P, N, K, xt, nullptr, 0, M, y, ldy, accumulate, s, part, ctr);
        if constexpr (TT < 4 && 12288 % KS == 0)
            if (K == 12288) return launch_k<MW, TT, RW, 12288 / KS, false, S>(P, N, K, xt, nullptr, 0, M, y, ldy, accumulate, s, part, ctr);
        return launch_k<MW, TT, RW, 0, false, S>(P, N, K, xt, nullptr, 0, M, y, ldy, accumulate, s, part, ctr);
    }
}

template <int TT>
static hipError_t launch_split_tt(DevPlanes P, int64_t N, int64_t K, const uint8_t* xt, int64_t M, float* y,
                                  int64_t ldy, int accumulate, hipStream_t s, float* part, uint32_t* ctr,
                                  const SplitPlan& p) {
    if (p.RW == 6) return launch_split_s<TT, 6, 2>(P, N, K, xt, M, y, ldy, accumulate, s, part, ctr);
    if (p.S == 2) return launch_split_s<TT, 4, 2>(P, N, K, xt, M, y, ldy, accumulate, s, part, ctr);
    return launch_split_s<TT, 4, 4>(P, N, K, xt, M, y, ldy, accumulate, s, part, ctr);
}

hipError_t launch_gemv_mfma_q45_ws(DevPlanes P, int64_t N, int64_t K, const void* xt, int64_t M, float* y,
                                   int64_t ldy, int accumulate, void* ws, hipStream_t stream) {
    const SplitPlan p = mfma_split_plan(N, K, M);
    if (p.S == 1) return launch_gemv_mfma_q45(P, N, K, xt, M, y, ldy, accumulate, stream);
    const uint8_t* x = (const uint8_t*)xt;
    uint32_t* ctr = (uint32_t*)ws;
    float* part = (float*)((uint8_t*)ws + split_ctr_bytes(p));
    switch (pick_tt(M)) {
    case 1: return launch_split_tt<1>(P, N, K, x, M, y, ldy, accumulate, stream, part, ctr, p);
    case 2: return launch_split_tt<2>(P, N, K, x, M, y, ldy, accumulate, stream, part, ctr, p);
    default: return launch_split_tt<4>(P, N, K, x, M, y, ldy, accumulate, stream, part, ctr, p);
    }
}

// fp32 x converts every token tile in every workgroup, and that vector work
// runs better at two waves per SIMD (two token tiles, 8 waves) than at one
// (four tiles, 4 waves) wherever a workgroup covers two or more row tiles:
// 12288 x 4096 at 64 tokens 47.5 us against 52.6, at 512 356 against 399.
// With one row tile (4096 rows) four tiles stay slightly ahead (95.1
// against 96.6 at 64 tokens on 4096 x 12288).
static int pick_tt_f32x(int64_t N, int64_t M) {
    const int tt = pick_tt(M);
    if (tuning_var("MBQ_MFMA_TT")) return tt;
    const int64_t rw = (N + 16 * 256 - 1) / (16 * 256);
    return tt == 4 && rw >= 2 ? 2 : tt;
}

hipError_t launch_gemv_mfma_q45_f32x(DevPlanes P, int64_t N, int64_t K, const float* x,
                                     int64_t ldx, int64_t M, float* y, int64_t ldy,
                                     int accumulate, hipStream_t stream) {
    switch (pick_tt_f32x(N, M)) {
    case 1: return launch_tt<1, true>(P, N, K, nullptr, x, ldx, M, y, ldy, accumulate, stream);
    case 2: return launch_tt<2, true>(P, N, K, nullptr, x, ldx, M, y, ldy, accumulate, stream);
    default: return launch_tt<4, true>(P, N, K, nullptr, x, ldx, M, y, ldy, accumulate, stream);
    }
}

}  // namespace mbq
