// staging.h -- x in the form the quantized dot products consume ("staged x").
//
// For the quantized formats x is held per chunk (32 values, 64 for Q25) as
// 24-bit fixed point: n = rint(x * 2^e), e chosen per 32-value block (one
// per chunk, two per Q25 chunk) so that the block's largest |x| maps into
// [2^21, 2^22), and n is split into the bytes
// b0, b1 (unsigned) and b2 (signed) of its two's complement.  The bytes are
// laid out as "digit words" in the order of the format's code vectors
// (formats.h), followed by the chunk's metadata: 2^-e and the offset terms
// -offset * (sum of each digit over an offset block); a Q25 chunk's second
// block keeps its own 2^-e in metadata dword 7.  BF16 keeps x as fp32.
//
// A chunk takes Traits::F4 16-byte slots: 4 bytes per value for every format
// (Q45/Q65: 24 digit dwords + 7 metadata dwords + 1 pad per 32 values; Q25:
// 48 + 7 + 9 pad per 64; BF16: the 8 floats).  In global memory the chunks of
// a row are packed back to back (row stride 4*K bytes).  In LDS each chunk
// takes one more slot, so lanes reading consecutive chunks at that stride hit
// distinct banks for any 16 consecutive lanes.
//
// Staging is computed in groups of GX consecutive values (8, 16 for Q25),
// one group per thread, the GPC groups of a chunk in adjacent lanes; the
// chunk maximum and the block sums are combined with lane shuffles.
#pragma once

#include "device_common.h"
#include "formats.h"

namespace mbq {

// Chunk exponent for a largest |x| with biased exponent E (0: zero or
// subnormal): e = 148 - E maps it into [2^21, 2^22); clamped to <= 126 so
// 2^e and 2^-e are normal floats (values below 2^-126 then round to 0 or
// +-1 units of 2^-126).
__device__ __forceinline__ int chunk_exp(float amax) {
    const int E = (int)((__builtin_bit_cast(uint32_t, amax) >> 23) & 0xFFu);
    const int e = 148 - E;
    return e > 126 ? 126 : e;
}
__device__ __forceinline__ float pow2f(int e) {
    return __builtin_bit_cast(float, (uint32_t)(e + 127) << 23);
}

// Byte p (p = 0, 1, 2) of four 32-bit integers, packed into one word.
__device__ __forceinline__ void digit_words(int32_t n0, int32_t n1, int32_t n2, int32_t n3,
                                            uint32_t* dg) {
    const uint32_t t01 = __builtin_amdgcn_perm((uint32_t)n1, (uint32_t)n0, 0x05010400u);
    const uint32_t t23 = __builtin_amdgcn_perm((uint32_t)n3, (uint32_t)n2, 0x05010400u);
    const uint32_t u01 = __builtin_amdgcn_perm((uint32_t)n1, (uint32_t)n0, 0x06020602u);
    const uint32_t u23 = __builtin_amdgcn_perm((uint32_t)n3, (uint32_t)n2, 0x06020602u);
    dg[0] = __builtin_amdgcn_perm(t23, t01, 0x05040100u);
    dg[1] = __builtin_amdgcn_perm(t23, t01, 0x07060302u);
    dg[2] = __builtin_amdgcn_perm(u23, u01, 0x05040100u);
}

// Round x * 2^e to the nearest integer (ties to even) with one FMA: adding
// 1.5 * 2^23 leaves the integer in the low mantissa bits for |x 2^e| < 2^22.
__device__ __forceinline__ int32_t round_fixed(float v, float up) {
    const float t = fmaf(v, up, 12582912.0f);
    return (int32_t)(__builtin_bit_cast(uint32_t, t) - 0x4B400000u);
}

template <int FMT>
struct Stride {
    static constexpr int GDW = 4 * Traits<FMT>::F4;        // dwords per chunk, global
    static constexpr int SLOTS = Traits<FMT>::F4 + 1;      // 16-byte slots per chunk, LDS
    static constexpr int DW = 4 * SLOTS;                   // dwords per chunk, LDS
};

// Destinations of staged dwords: d is the dword index within chunk b.
template <int FMT>
struct LdsDst {
    uint32_t* xs;
    __device__ uint32_t* at(int b, int d) const { return xs + Stride<FMT>::DW * b + d; }
};
template <int FMT>
struct GlobalDst {
    uint32_t* xq;
    __device__ uint32_t* at(int b, int d) const { return xq + (int64_t)Stride<FMT>::GDW * b + d; }
};

// Stage one group of GX values v (group og of the row; `ok` false for groups
// past the row, which still take part in the lane shuffles).
template <int FMT, class Dst>
__device__ __forceinline__ void stage_group(const float* v, int og, bool ok, const Dst& dst) {
    using T = Traits<FMT>;
    constexpr int GX = T::GX;
    constexpr int GPC = T::WPC / GX;          // groups per chunk: 4 (1 for BF16)
    const int b = og / GPC, gi = og % GPC;    // chunk, group within chunk
    if constexpr (!T::INT) {
        if (ok) {
#pragma unroll
            for (int j = 0; j < GX; j += 4)
                *(uint4*)dst.at(b, GX * gi + j) =
                    make_uint4(__builtin_bit_cast(uint32_t, v[j]), __builtin_bit_cast(uint32_t, v[j + 1]),
                               __builtin_bit_cast(uint32_t, v[j + 2]), __builtin_bit_cast(uint32_t, v[j + 3]));
        }
    } else {
        // one exponent per 32-value block: the chunk's four groups (Q45,
        // Q65: one block), or each pair of groups (Q25: two blocks of 32)
        constexpr bool TWO = T::BLK == 32 && T::WPC == 64;
        float amax = 0.f;
#pragma unroll
        for (int k = 0; k < GX; k++) amax = fmaxf(amax, fabsf(v[k]));
        amax = fmaxf(amax, lane_xor1(amax));
        if constexpr (!TWO) amax = fmaxf(amax, lane_xor2(amax));
        const int e = chunk_exp(amax);
        const int e_hi = TWO ? lane_xor2(e) : e;              // the second block's, in groups 0, 1
        const float up = pow2f(e);
        int32_t n[GX];
#pragma unroll
        for (int k = 0; k < GX; k++) n[k] = round_fixed(v[k], up);
        // digit words of the group's code vectors.  Q45/Q65 octet: vector 0 =
        // even values, 1 = odd values.  Q25 group of 16: vector m = values
        // m, 4+m, 8+m, 12+m.
        constexpr int NV = GX / 4;
        constexpr int ST = (GX == 8) ? 2 : 4;
        uint32_t dg[3 * NV];
#pragma unroll
        for (int m = 0; m < NV; m++)
            digit_words(n[m], n[m + ST], n[m + 2 * ST], n[m + 3 * ST], dg + 3 * m);
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
            B01[p] = S[p] + lane_xor1(S[p]);               // groups 0+1 (or 2+3)
            B23[p] = lane_xor2(B01[p]);                    // the other pair
        }
        if (ok) {
            uint32_t* o = dst.at(b, 3 * NV * gi);            // 8-byte aligned
#pragma unroll
            for (int t = 0; t < 3 * NV; t += 2) *(uint2*)(o + t) = make_uint2(dg[t], dg[t + 1]);
            if (gi == 0) {
                // metadata slots, padding included, so every staged byte is defined
                constexpr int MD = 4 * T::F4 - T::META;
                uint32_t m[MD];
#pragma unroll
                for (int t = 0; t < MD; t++) m[t] = 0u;
                m[0] = __builtin_bit_cast(uint32_t, pow2f(-e));
                if constexpr (TWO) m[7] = __builtin_bit_cast(uint32_t, pow2f(-e_hi));
                if constexpr (T::BLK == 32 && T::WPC == 32) {   // one offset block per chunk
#pragma unroll
                    for (int p = 0; p < 3; p++) m[1 + p] = (uint32_t)(-T::OFF * (B01[p] + B23[p]));
                } else {                                          // two blocks per chunk
#pragma unroll
                    for (int p = 0; p < 3; p++) {
                        m[1 + p] = (uint32_t)(-T::OFF * B01[p]);
                        m[4 + p] = (uint32_t)(-T::OFF * B23[p]);
                    }
                }
                uint32_t* md = dst.at(b, T::META);                // 16-byte aligned
#pragma unroll
                for (int t = 0; t < MD; t += 4) *(uint4*)(md + t) = make_uint4(m[t], m[t + 1], m[t + 2], m[t + 3]);
            }
        }
    }
}

// The staged dwords of chunk b from LDS.
template <int FMT>
__device__ __forceinline__ void read_x(const uint32_t* xs, int b, uint32_t* xv) {
    const uint32_t* src = xs + Stride<FMT>::DW * b;
#pragma unroll
    for (int j = 0; j < Traits<FMT>::F4; j++) {
        const uint4 v = *(const uint4*)(src + 4 * j);
        xv[4 * j + 0] = v.x;
        xv[4 * j + 1] = v.y;
        xv[4 * j + 2] = v.z;
        xv[4 * j + 3] = v.w;
    }
}

// ---- x into LDS, inside a workgroup --------------------------------------
// x arrives as 16-byte pieces: float4 of fp32 x, or 16-byte slots of staged x
// (XQ).  Piece i of a thread (i = 0, 1, ...) of a workgroup of NT threads is
//   staged: slot i * NT + tid of the row (consecutive threads, consecutive
//           slots: coalesced);
//   fp32:   float4 j = i % GF4 of group (i / GF4) * NT + tid, so each thread
//           holds the GF4 float4 of whole groups of GX values.
template <int FMT, bool XQ, int NT = kBlock>
struct XPieces {
    static constexpr int GF4 = Traits<FMT>::GX / 4;
    __device__ static __forceinline__ int index(int i) {
        if constexpr (XQ)
            return i * NT + (int)threadIdx.x;
        else
            return ((i / GF4) * NT + (int)threadIdx.x) * GF4 + i % GF4;
    }
    // pieces in a row of K values
    __device__ static __forceinline__ int count(int K) {
        return XQ ? (K / Traits<FMT>::WPC) * Traits<FMT>::F4 : K / 4;
    }
    // Load piece i (index clamped into the row, so the load is unconditional).
    __device__ static __forceinline__ uint4 load(const uint4* __restrict__ src, int i, int n) {
        const int p = index(i);
        return gload<uint4>((const uint8_t*)src, 16u * (uint32_t)(p < n ? p : n - 1));
    }
    // Store pieces [i0, i0 + NI) (NI a multiple of GF4 for fp32) into LDS.
    // ALL: every piece is known to lie inside the row (no bounds test, so the
    // loads feeding the stores cannot be moved behind a branch).
    template <int NI, bool ALL>
    __device__ static __forceinline__ void store(const uint4* v, int i0, int n, uint32_t* xs) {
        if constexpr (XQ) {
            constexpr int F4 = Traits<FMT>::F4;
#pragma unroll
            for (int i = 0; i < NI; i++) {
                const int p = index(i0 + i);
                if (ALL || p < n) *(uint4*)(xs + Stride<FMT>::DW * (p / F4) + 4 * (p % F4)) = v[i];
            }
        } else {
            const int ngroups = n / GF4;
#pragma unroll
            for (int i = 0; i < NI; i += GF4) {
                const int og = ((i0 + i) / GF4) * NT + (int)threadIdx.x;
                stage_group<FMT>((const float*)(v + i), og, ALL || og < ngroups, LdsDst<FMT>{xs});
            }
        }
    }
};

}  // namespace mbq
