// formats.h -- per-format lane chunks: load, in-register unpack, dot product.
//
// A lane owns one "chunk" of a row at a time: 16 bytes of plane 0, which is
// 32 weights for Q45 and Q65, 64 for Q25 and 8 for BF16, plus the matching
// bytes of the other planes.  Consecutive lanes own consecutive chunks, so a
// wave's plane-0 load is one fully coalesced 1 KiB burst ([mountain-runs]
// section 3: lanes read consecutive 16-byte chunks).
//
// Codes are unpacked in registers and never stored ([roofline-holds]
// "Hiding, fusing, and keeping the sums busy", Dtypes).  For the quantized
// formats the unpack masks four codes at once into the four bytes of a dword
// ("code vector").  x is held per chunk as 24-bit fixed point: each value is
// rounded to the integer n = rint(x * 2^e), e chosen per chunk so that the
// chunk's largest |x| maps into [2^21, 2^22), and n is split into its three
// two's-complement bytes n = b2 * 2^16 + b1 * 2^8 + b0 (b0, b1 unsigned, b2
// signed).  One v_dot4_u32_u8 per low byte and one v_dot4_i32_i8 per top byte
// then form the exact integer sums  sum_k q_k * b_p(k)  of four weights each,
// so the whole chunk's  sum_k (q_k - offset) n_k  is exact; the offset term
// -offset * sum_k b_p(k) is precomputed per block and starts the sums.  The
// only rounding is x to 22 bits relative to its chunk maximum (the same
// relative precision as the fp16 high/low split of an fp32 value) and the
// final conversion of each chunk's integer to fp32.
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace mbq {

__device__ __forceinline__ uint32_t udot4(uint32_t a, uint32_t b, uint32_t c) {
    return __builtin_amdgcn_udot4(a, b, c, false);
}
__device__ __forceinline__ int32_t sdot4(uint32_t a, uint32_t b, int32_t c) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// Sums of the three digit planes of a code vector's chunk, started at the
// precomputed offset terms i0, i1, i2 (held as raw 32-bit words).
struct Acc3 {
    uint32_t a0, a1;
    int32_t a2;
};

__device__ __forceinline__ void acc_vec(Acc3& s, uint32_t codes, const uint32_t* dig) {
    s.a0 = udot4(codes, dig[0], s.a0);
    s.a1 = udot4(codes, dig[1], s.a1);
    s.a2 = sdot4(codes, dig[2], s.a2);
}

// The chunk's integer  sum (q - offset) n  as fp32:  a2 * 2^16 + (a1 * 2^8 + a0).
__device__ __forceinline__ float acc_value(const Acc3& s) {
    const int32_t lo = (int32_t)(s.a1 * 256u + s.a0);
    return fmaf((float)s.a2, 65536.f, (float)lo);
}

// Load from device memory through a global (address space 1) pointer, so the
// access is a global load even where the plane pointer came from memory (a
// generic pointer would be a flat load).
typedef uint32_t gu4 __attribute__((ext_vector_type(4)));
typedef uint32_t gu2 __attribute__((ext_vector_type(2)));
typedef const uint8_t __attribute__((address_space(1)))* gbyte;
// base (uniform) + off (per lane, 32-bit): the form of a scalar-base global load
template <class V>
__device__ __forceinline__ V gload(const uint8_t* base, uint32_t off) {
    const gbyte p = (gbyte)base + off;
    if constexpr (sizeof(V) == 16) {
        return __builtin_bit_cast(V, *(const __attribute__((address_space(1))) gu4*)p);
    } else if constexpr (sizeof(V) == 8) {
        return __builtin_bit_cast(V, *(const __attribute__((address_space(1))) gu2*)p);
    } else {
        return *(const __attribute__((address_space(1))) V*)p;
    }
}
template <class V>
__device__ __forceinline__ V gload(const uint8_t* p) {
    return gload<V>(p, 0u);
}

// ---- buffer loads ----------------------------------------------------------
// Weight planes are read through buffer resources: a scalar descriptor per
// plane, the row's byte offset in a scalar register and the lane's 32-bit
// offset in a vector register.  No 64-bit per-lane address is ever formed.
// Every plane must be smaller than 4 GiB.
typedef __amdgpu_buffer_rsrc_t Rsrc;
struct BufPlanes {
    Rsrc p0, p1, p2, p3;
};
// Byte offset of one row in each plane.
struct RowOff {
    uint32_t o0, o1, o2, o3;
};
__device__ __forceinline__ Rsrc make_rsrc(const uint8_t* p, uint64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0,
                                             (int)(bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : bytes),
                                             0x00020000);
}
// UNI: soff is the same in every lane (scalar offset); otherwise it is added
// to the lane's offset.
template <class V, bool UNI>
__device__ __forceinline__ V bload(Rsrc r, uint32_t voff, uint32_t soff) {
    const uint32_t vo = UNI ? voff : voff + soff;
    const uint32_t so = UNI ? soff : 0u;
    if constexpr (sizeof(V) == 16) {
        return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b128(r, vo, so, 0));
    } else if constexpr (sizeof(V) == 8) {
        return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b64(r, vo, so, 0));
    } else if constexpr (sizeof(V) == 4) {
        return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b32(r, vo, so, 0));
    } else {
        return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b16(r, vo, so, 0));
    }
}

template <int FMT>
struct Traits;

// Staged x per chunk (dwords, LDS): for every code vector of the chunk its
// three digit words, then the chunk's metadata.  Vector order per 8 weights
// (Q45, Q65): the even weights (0, 2, 4, 6) then the odd ones (1, 3, 5, 7).

// ----------------------------------------------------------------- Q45 ----
// codes dword: byte j = weight 2j (low nibble), 2j+1 (high nibble).
// Chunk x layout: 4 octets x {E digits 0-2, O digits 0-2} = 24 dwords, then
// meta [24] = 2^-e (float bits), [25..27] = -8 * (block sums of digits 0-2).
template <>
struct Traits<kQ45> {
    static constexpr int WPC = 32;   // weights per chunk
    static constexpr int F4 = 8;     // 16-byte LDS slots per chunk
    static constexpr int GX = 8;     // x values per staging group
    static constexpr int BLK = 32;   // weights per offset block
    static constexpr int OFF = 8;
    static constexpr int META = 24;  // dword index of the metadata
    static constexpr bool INT = true;
    struct Row {
        uint4 c;
        uint32_t s;
    };
    // Resources of the planes the format uses, for an N x K matrix.
    __device__ static __forceinline__ BufPlanes planes(const DevPlanes& P, int64_t N, int64_t K) {
        const uint64_t nk = (uint64_t)N * (uint64_t)K;
        return BufPlanes{make_rsrc(P.p0, nk / 2), make_rsrc(P.p0, 0), make_rsrc(P.p2, nk / 16),
                         make_rsrc(P.p0, 0)};
    }
    // Start of one row in each plane.
    __device__ static __forceinline__ RowOff row_off(int64_t row, int64_t K) {
        return RowOff{(uint32_t)(row * (K >> 1)), 0u, (uint32_t)(row * (K >> 4)), 0u};
    }
    template <bool UNI = true>
    __device__ static __forceinline__ void load(Row& r, const BufPlanes& B, const RowOff& o, int b) {
        r.c = bload<uint4, UNI>(B.p0, 16u * (uint32_t)b, o.o0);
        r.s = bload<uint16_t, UNI>(B.p2, 2u * (uint32_t)b, o.o2);
    }
    // code vectors of dword d: even weights, odd weights
    __device__ static __forceinline__ void vectors(uint32_t d, uint32_t& ev, uint32_t& od) {
        ev = d & 0x0F0F0F0Fu;
        od = (d >> 4) & 0x0F0F0F0Fu;
    }
    // Code vectors of the chunk, in the order of the staged digit words.
    static constexpr int NVEC = 8;
    __device__ static __forceinline__ void unpack(const Row& r, uint32_t* v) {
        const uint32_t* c = &r.c.x;
#pragma unroll
        for (int i = 0; i < 4; i++) vectors(c[i], v[2 * i], v[2 * i + 1]);
    }
    // The chunk's contribution to y from its code vectors (xv: the chunk's
    // 32 staged dwords).
    __device__ static __forceinline__ float dot_vec(const Row& r, const uint32_t* v,
                                                    const uint32_t* xv) {
        Acc3 s{xv[META + 1], xv[META + 2], (int32_t)xv[META + 3]};
#pragma unroll
        for (int j = 0; j < NVEC; j++) acc_vec(s, v[j], xv + 3 * j);
        return (h2f(r.s) * as_f(xv[META])) * acc_value(s);
    }
    // Lanes past the row: 2^-e to 0, so they add exactly 0.
    __device__ static __forceinline__ void mask_meta(uint32_t* xv, bool ok) {
        xv[META] = ok ? xv[META] : 0u;
    }
    __device__ static __forceinline__ float dot(const Row& r, const uint32_t* xv) {
        uint32_t v[NVEC];
        unpack(r, v);
        return dot_vec(r, v, xv);
    }
    // integer codes of the chunk, through the same unpack as dot()
    __device__ static __forceinline__ void codes(const Row& r, int* q) {
        const uint32_t* c = &r.c.x;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            uint32_t ev, od;
            vectors(c[i], ev, od);
#pragma unroll
            for (int j = 0; j < 4; j++) {
                q[8 * i + 2 * j] = (int)((ev >> (8 * j)) & 0xFFu);
                q[8 * i + 2 * j + 1] = (int)((od >> (8 * j)) & 0xFFu);
            }
        }
    }
    __device__ static __forceinline__ void weights(const Row& r, float* w) {
        int q[WPC];
        codes(r, q);
        const float s = h2f(r.s);
#pragma unroll
        for (int k = 0; k < WPC; k++) w[k] = s * (float)(q[k] - OFF);
    }
};

// ----------------------------------------------------------------- Q65 ----
// ql dwords as Q45 (low 4 bits).  One qh dword h holds the high 2 bits of a
// 16-weight run whose low bits are ql dwords d0 (weights 0-7) and d1 (8-15):
// byte j of h carries weight 2j in bits 4-5, 2j+1 in bits 2-3, 8+2j in bits
// 0-1 and 8+2j+1 in bits 6-7, so every code vector is one mask (plus at most
// two shifts) away:  q(2j) = lo | (h & 0x30) ...  for the four vectors
//   E0 = even of d0, O0 = odd of d0, E1 = even of d1, O1 = odd of d1.
// Chunk x layout as Q45; meta [24] = 2^-e, [25..27] offset terms of the first
// 16-weight sub-block, [28..30] of the second.
template <>
struct Traits<kQ65> {
    static constexpr int WPC = 32;
    static constexpr int F4 = 8;
    static constexpr int GX = 8;
    static constexpr int BLK = 16;
    static constexpr int OFF = 32;
    static constexpr int META = 24;
    static constexpr bool INT = true;
    struct Row {
        uint4 ql;
        uint2 qh;
        uint32_t sc;   // two int8 sub-scales (low byte: first 16 weights)
        uint32_t d;    // fp16 super-scale of the chunk's 256-weight block
    };
    __device__ static __forceinline__ BufPlanes planes(const DevPlanes& P, int64_t N, int64_t K) {
        const uint64_t nk = (uint64_t)N * (uint64_t)K;
        return BufPlanes{make_rsrc(P.p0, nk / 2), make_rsrc(P.p1, nk / 4), make_rsrc(P.p2, nk / 16),
                         make_rsrc(P.p3, nk / 128)};
    }
    __device__ static __forceinline__ RowOff row_off(int64_t row, int64_t K) {
        return RowOff{(uint32_t)(row * (K >> 1)), (uint32_t)(row * (K >> 2)),
                      (uint32_t)(row * (K >> 4)), (uint32_t)(row * (K >> 7))};
    }
    template <bool UNI = true>
    __device__ static __forceinline__ void load(Row& r, const BufPlanes& B, const RowOff& o, int b) {
        r.ql = bload<uint4, UNI>(B.p0, 16u * (uint32_t)b, o.o0);
        r.qh = bload<uint2, UNI>(B.p1, 8u * (uint32_t)b, o.o1);
        r.sc = bload<uint16_t, UNI>(B.p2, 2u * (uint32_t)b, o.o2);
        r.d = bload<uint16_t, UNI>(B.p3, 2u * ((uint32_t)b >> 3), o.o3);
    }
    __device__ static __forceinline__ void vectors(uint32_t d0, uint32_t d1, uint32_t h,
                                                   uint32_t* v) {
        v[0] = (d0 & 0x0F0F0F0Fu) | (h & 0x30303030u);
        v[1] = ((d0 >> 4) & 0x0F0F0F0Fu) | ((h << 2) & 0x30303030u);
        v[2] = (d1 & 0x0F0F0F0Fu) | ((h << 4) & 0x30303030u);
        v[3] = ((d1 >> 4) & 0x0F0F0F0Fu) | ((h >> 2) & 0x30303030u);
    }
    __device__ static __forceinline__ float sc_f(uint32_t sc, int sb) {
        return (float)(int)(int8_t)((sc >> (8 * sb)) & 0xFFu);
    }
    static constexpr int NVEC = 8;
    __device__ static __forceinline__ void unpack(const Row& r, uint32_t* v) {
        const uint32_t* ql = &r.ql.x;
        const uint32_t* qh = &r.qh.x;
#pragma unroll
        for (int sb = 0; sb < 2; sb++) vectors(ql[2 * sb], ql[2 * sb + 1], qh[sb], v + 4 * sb);
    }
    __device__ static __forceinline__ float dot_vec(const Row& r, const uint32_t* v,
                                                    const uint32_t* xv) {
        float t[2];
#pragma unroll
        for (int sb = 0; sb < 2; sb++) {
            Acc3 s{xv[META + 1 + 3 * sb], xv[META + 2 + 3 * sb], (int32_t)xv[META + 3 + 3 * sb]};
#pragma unroll
            for (int i = 0; i < 4; i++) acc_vec(s, v[4 * sb + i], xv + 12 * sb + 3 * i);
            t[sb] = acc_value(s);
        }
        return (h2f(r.d) * as_f(xv[META])) * fmaf(sc_f(r.sc, 1), t[1], sc_f(r.sc, 0) * t[0]);
    }
    // Lanes past the row: 2^-e to 0, so they add exactly 0.
    __device__ static __forceinline__ void mask_meta(uint32_t* xv, bool ok) {
        xv[META] = ok ? xv[META] : 0u;
    }
    __device__ static __forceinline__ float dot(const Row& r, const uint32_t* xv) {
        uint32_t v[NVEC];
        unpack(r, v);
        return dot_vec(r, v, xv);
    }
    __device__ static __forceinline__ void codes(const Row& r, int* q) {
        const uint32_t* ql = &r.ql.x;
        const uint32_t* qh = &r.qh.x;
#pragma unroll
        for (int sb = 0; sb < 2; sb++) {
            uint32_t v[4];
            vectors(ql[2 * sb], ql[2 * sb + 1], qh[sb], v);
#pragma unroll
            for (int j = 0; j < 4; j++) {
                q[16 * sb + 2 * j] = (int)((v[0] >> (8 * j)) & 0xFFu);
                q[16 * sb + 2 * j + 1] = (int)((v[1] >> (8 * j)) & 0xFFu);
                q[16 * sb + 8 + 2 * j] = (int)((v[2] >> (8 * j)) & 0xFFu);
                q[16 * sb + 8 + 2 * j + 1] = (int)((v[3] >> (8 * j)) & 0xFFu);
            }
        }
    }
    __device__ static __forceinline__ void weights(const Row& r, float* w) {
        int q[WPC];
        codes(r, q);
        const float d = h2f(r.d);
#pragma unroll
        for (int k = 0; k < WPC; k++) w[k] = d * sc_f(r.sc, k >> 4) * (float)(q[k] - OFF);
    }
};

// ----------------------------------------------------------------- Q25 ----
// codes dword: weights 0-15, byte j holds 4j..4j+3 in bits 0-1, 2-3, 4-5, 6-7;
// code vector m (m = 0..3) = (d >> 2m) & 0x03030303 holds weights
// (m, 4+m, 8+m, 12+m).  Chunk x layout: 4 dwords x 4 vectors x 3 digits = 48
// dwords, meta [48] = 2^-e of block 0, [49..51] offset terms of block 0,
// [52..54] those of block 1, [55] = 2^-e of block 1 (each block of 32 values
// keeps 22 bits relative to its own largest |x|).
template <>
struct Traits<kQ25> {
    static constexpr int WPC = 64;
    static constexpr int F4 = 16;
    static constexpr int GX = 16;
    static constexpr int BLK = 32;
    static constexpr int OFF = 2;
    static constexpr int META = 48;
    static constexpr bool INT = true;
    struct Row {
        uint4 c;
        uint32_t s2;   // the chunk's two fp16 scales
    };
    __device__ static __forceinline__ BufPlanes planes(const DevPlanes& P, int64_t N, int64_t K) {
        const uint64_t nk = (uint64_t)N * (uint64_t)K;
        return BufPlanes{make_rsrc(P.p0, nk / 4), make_rsrc(P.p0, 0), make_rsrc(P.p2, nk / 16),
                         make_rsrc(P.p0, 0)};
    }
    __device__ static __forceinline__ RowOff row_off(int64_t row, int64_t K) {
        return RowOff{(uint32_t)(row * (K >> 2)), 0u, (uint32_t)(row * (K >> 4)), 0u};
    }
    template <bool UNI = true>
    __device__ static __forceinline__ void load(Row& r, const BufPlanes& B, const RowOff& o, int b) {
        r.c = bload<uint4, UNI>(B.p0, 16u * (uint32_t)b, o.o0);
        r.s2 = bload<uint32_t, UNI>(B.p2, 4u * (uint32_t)b, o.o2);
    }
    __device__ static __forceinline__ uint32_t vec(uint32_t d, int m) {
        return (d >> (2 * m)) & 0x03030303u;
    }
    static constexpr int NVEC = 16;
    __device__ static __forceinline__ void unpack(const Row& r, uint32_t* v) {
        const uint32_t* c = &r.c.x;
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int m = 0; m < 4; m++) v[4 * i + m] = vec(c[i], m);
    }
    __device__ static __forceinline__ float dot_vec(const Row& r, const uint32_t* v,
                                                    const uint32_t* xv) {
        float t[2];
#pragma unroll
        for (int blk = 0; blk < 2; blk++) {
            Acc3 s{xv[META + 1 + 3 * blk], xv[META + 2 + 3 * blk], (int32_t)xv[META + 3 + 3 * blk]};
#pragma unroll
            for (int j = 0; j < 8; j++) acc_vec(s, v[8 * blk + j], xv + 24 * blk + 3 * j);
            t[blk] = acc_value(s);
        }
        return fmaf(h2f(r.s2 >> 16) * as_f(xv[META + 7]), t[1], (h2f(r.s2) * as_f(xv[META])) * t[0]);
    }
    // Lanes past the row: both blocks' 2^-e to 0, so they add exactly 0.
    __device__ static __forceinline__ void mask_meta(uint32_t* xv, bool ok) {
        xv[META] = ok ? xv[META] : 0u;
        xv[META + 7] = ok ? xv[META + 7] : 0u;
    }
    __device__ static __forceinline__ float dot(const Row& r, const uint32_t* xv) {
        uint32_t v[NVEC];
        unpack(r, v);
        return dot_vec(r, v, xv);
    }
    __device__ static __forceinline__ void codes(const Row& r, int* q) {
        const uint32_t* c = &r.c.x;
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int m = 0; m < 4; m++) {
                const uint32_t v = vec(c[i], m);
#pragma unroll
                for (int j = 0; j < 4; j++) q[16 * i + 4 * j + m] = (int)((v >> (8 * j)) & 0xFFu);
            }
    }
    __device__ static __forceinline__ void weights(const Row& r, float* w) {
        int q[WPC];
        codes(r, q);
        const float s0 = h2f(r.s2), s1 = h2f(r.s2 >> 16);
#pragma unroll
        for (int k = 0; k < WPC; k++) w[k] = (k < 32 ? s0 : s1) * (float)(q[k] - OFF);
    }
};

// ---------------------------------------------------------------- BF16 ----
// 16 bits per weight leave ample arithmetic per byte: x stays fp32 and each
// weight is one shift or mask plus one fp32 FMA.  Chunk x layout: 8 floats.
template <>
struct Traits<kBF16> {
    static constexpr int WPC = 8;
    static constexpr int F4 = 2;
    static constexpr int GX = 8;
    static constexpr int BLK = 8;
    static constexpr int OFF = 0;
    static constexpr int META = 0;
    static constexpr bool INT = false;
    struct Row {
        uint4 w;
    };
    __device__ static __forceinline__ BufPlanes planes(const DevPlanes& P, int64_t N, int64_t K) {
        const uint64_t nk = (uint64_t)N * (uint64_t)K;
        return BufPlanes{make_rsrc(P.p0, 2 * nk), make_rsrc(P.p0, 0), make_rsrc(P.p0, 0),
                         make_rsrc(P.p0, 0)};
    }
    __device__ static __forceinline__ RowOff row_off(int64_t row, int64_t K) {
        return RowOff{(uint32_t)(2 * row * K), 0u, 0u, 0u};
    }
    template <bool UNI = true>
    __device__ static __forceinline__ void load(Row& r, const BufPlanes& B, const RowOff& o, int b) {
        r.w = bload<uint4, UNI>(B.p0, 16u * (uint32_t)b, o.o0);
    }
    static constexpr int NVEC = 8;   // the 8 weights as fp32 bit patterns
    __device__ static __forceinline__ void unpack(const Row& r, uint32_t* v) {
        const uint32_t* c = &r.w.x;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            v[2 * i] = c[i] << 16;
            v[2 * i + 1] = c[i] & 0xFFFF0000u;
        }
    }
    __device__ static __forceinline__ float dot_vec(const Row& r, const uint32_t* v,
                                                    const uint32_t* xv) {
        (void)r;
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            a0 = fmaf(as_f(v[2 * i]), as_f(xv[2 * i]), a0);
            a1 = fmaf(as_f(v[2 * i + 1]), as_f(xv[2 * i + 1]), a1);
        }
        return a0 + a1;
    }
    __device__ static __forceinline__ float dot(const Row& r, const uint32_t* xv) {
        uint32_t v[NVEC];
        unpack(r, v);
        return dot_vec(r, v, xv);
    }
    __device__ static __forceinline__ void weights(const Row& r, float* w) {
        const uint32_t* c = &r.w.x;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            w[2 * i] = as_f(c[i] << 16);
            w[2 * i + 1] = as_f(c[i] & 0xFFFF0000u);
        }
    }
};

}  // namespace mbq
