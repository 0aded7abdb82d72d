// formats.h -- per-format lane chunks: load, in-register unpack, dot product.
//
// A lane owns one "chunk" of a row at a time: 16 bytes of plane 0, which is
// 32 weights for Q45 and Q65, 64 for Q25 and 8 for BF16, plus the matching
// bytes of the other planes.  Consecutive lanes own consecutive chunks, so a
// wave's plane-0 load is one fully coalesced 1 KiB burst ([mountain-runs]
// section 3: lanes read consecutive 16-byte chunks).
//
// Codes are unpacked in registers and never stored ([roofline-holds]
// "Hiding, fusing, and keeping the sums busy", Dtypes).  The unpack masks
// codes into bytes and converts each byte with one v_cvt_f32_ubyteN; bytes
// that hold a code times a power of two are accumulated separately and
// rescaled once per block, which is exact.  The block offset is folded out
// of the inner loop:  sum_k s (q_k - o) x_k = s (sum_k q_k x_k - o sum_k x_k),
// with the per-block sums of x computed once per workgroup.
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace mbq {

template <int FMT>
struct Traits;

// ----------------------------------------------------------------- Q45 ----
template <>
struct Traits<kQ45> {
    static constexpr int WPC = 32;   // weights per chunk
    static constexpr int F4 = 8;     // float4 of x per chunk
    static constexpr int NBS = 1;    // block sums per chunk
    static constexpr int BSG = 8;    // float4 per block sum
    static constexpr float OFF = 8.f;
    struct Row {
        uint4 c;
        uint32_t s;
    };
    // Start of one row in each plane the format uses.
    __device__ static __forceinline__ DevPlanes base(const DevPlanes& P, int64_t row, int64_t K) {
        return DevPlanes{P.p0 + row * (K >> 1), nullptr, P.p2 + 2 * row * (K >> 5), nullptr};
    }
    __device__ static __forceinline__ void load(Row& r, const DevPlanes& B, int b) {
        r.c = *(const uint4*)(B.p0 + 16 * b);
        r.s = *(const uint16_t*)(B.p2 + 2 * b);
    }
    // dword i: byte j low nibble = weight 8i+2j, high nibble = weight 8i+2j+1
    __device__ static __forceinline__ uint32_t lo(uint32_t d) { return d & 0x0F0F0F0Fu; }
    __device__ static __forceinline__ uint32_t hi16(uint32_t d) { return d & 0xF0F0F0F0u; }
    // sum over the chunk of w_k x_k; mbs[0] = -8 * (sum of the chunk's x)
    __device__ static __forceinline__ float dot(const Row& r, const float* xv, const float* mbs) {
        float ae = mbs[0], ao = 0.f;
        const uint32_t* c = &r.c.x;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t l = lo(c[i]), h = hi16(c[i]);
            ae = fmaf(ub0(l), xv[8 * i + 0], ae);
            ao = fmaf(ub0(h), xv[8 * i + 1], ao);
            ae = fmaf(ub1(l), xv[8 * i + 2], ae);
            ao = fmaf(ub1(h), xv[8 * i + 3], ao);
            ae = fmaf(ub2(l), xv[8 * i + 4], ae);
            ao = fmaf(ub2(h), xv[8 * i + 5], ao);
            ae = fmaf(ub3(l), xv[8 * i + 6], ae);
            ao = fmaf(ub3(h), xv[8 * i + 7], ao);
        }
        return h2f(r.s) * fmaf(ao, 0.0625f, ae);
    }
    // integer codes of the chunk, through the same unpack as dot()
    __device__ static __forceinline__ void codes(const Row& r, float* q) {
        const uint32_t* c = &r.c.x;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t l = lo(c[i]), h = hi16(c[i]);
            q[8 * i + 0] = ub0(l); q[8 * i + 1] = ub0(h) * 0.0625f;
            q[8 * i + 2] = ub1(l); q[8 * i + 3] = ub1(h) * 0.0625f;
            q[8 * i + 4] = ub2(l); q[8 * i + 5] = ub2(h) * 0.0625f;
            q[8 * i + 6] = ub3(l); q[8 * i + 7] = ub3(h) * 0.0625f;
        }
    }
    __device__ static __forceinline__ void weights(const Row& r, float* w) {
        float q[WPC];
        codes(r, q);
        const float s = h2f(r.s);
#pragma unroll
        for (int k = 0; k < WPC; k++) w[k] = s * (q[k] - OFF);
    }
};

// ----------------------------------------------------------------- Q65 ----
template <>
struct Traits<kQ65> {
    static constexpr int WPC = 32;
    static constexpr int F4 = 8;
    static constexpr int NBS = 2;    // one sum per 16-weight sub-block
    static constexpr int BSG = 4;
    static constexpr float OFF = 32.f;
    struct Row {
        uint4 ql;
        uint2 qh;
        uint32_t sc;   // two int8 sub-scales (low byte: first 16 weights)
        uint32_t d;    // fp16 super-scale of the chunk's 256-weight block
    };
    __device__ static __forceinline__ DevPlanes base(const DevPlanes& P, int64_t row, int64_t K) {
        return DevPlanes{P.p0 + row * (K >> 1), P.p1 + row * (K >> 2), P.p2 + row * (K >> 4),
                         P.p3 + 2 * row * (K >> 8)};
    }
    __device__ static __forceinline__ void load(Row& r, const DevPlanes& B, int b) {
        r.ql = *(const uint4*)(B.p0 + 16 * b);
        r.qh = *(const uint2*)(B.p1 + 8 * b);
        r.sc = *(const uint16_t*)(B.p2 + 2 * b);
        r.d = *(const uint16_t*)(B.p3 + 2 * (b >> 3));
    }
    // One run of 16 weights: low bits in ql dwords d0 (weights 0-7) and d1
    // (8-15), high bits in qh dword h.  Produces four dwords whose byte j holds
    //   E0: q(2j)        O0: 4 q(2j+1)      E1: q(8+2j)      O1: 4 q(8+2j+1)
    __device__ static __forceinline__ void run(uint32_t d0, uint32_t d1, uint32_t h,
                                               uint32_t& E0, uint32_t& O0, uint32_t& E1,
                                               uint32_t& O1) {
        const uint32_t h4 = h << 4;
        E0 = (d0 & 0x0F0F0F0Fu) | (h & 0x30303030u);
        O0 = ((d0 >> 2) & 0x3C3C3C3Cu) | (h & 0xC0C0C0C0u);
        E1 = (d1 & 0x0F0F0F0Fu) | (h4 & 0x30303030u);
        O1 = ((d1 >> 2) & 0x3C3C3C3Cu) | (h4 & 0xC0C0C0C0u);
    }
    __device__ static __forceinline__ float sc_f(uint32_t sc, int sb) {
        return (float)(int)(int8_t)((sc >> (8 * sb)) & 0xFFu);
    }
    // mbs[sb] = -32 * (sum of x over sub-block sb of the chunk)
    __device__ static __forceinline__ float dot(const Row& r, const float* xv, const float* mbs) {
        const uint32_t* ql = &r.ql.x;
        const uint32_t* qh = &r.qh.x;
        float t[2];
#pragma unroll
        for (int sb = 0; sb < 2; sb++) {
            uint32_t E0, O0, E1, O1;
            run(ql[2 * sb], ql[2 * sb + 1], qh[sb], E0, O0, E1, O1);
            const float* xs = xv + 16 * sb;
            float ae = mbs[sb], ao = 0.f;
            ae = fmaf(ub0(E0), xs[0], ae);
            ao = fmaf(ub0(O0), xs[1], ao);
            ae = fmaf(ub1(E0), xs[2], ae);
            ao = fmaf(ub1(O0), xs[3], ao);
            ae = fmaf(ub2(E0), xs[4], ae);
            ao = fmaf(ub2(O0), xs[5], ao);
            ae = fmaf(ub3(E0), xs[6], ae);
            ao = fmaf(ub3(O0), xs[7], ao);
            ae = fmaf(ub0(E1), xs[8], ae);
            ao = fmaf(ub0(O1), xs[9], ao);
            ae = fmaf(ub1(E1), xs[10], ae);
            ao = fmaf(ub1(O1), xs[11], ao);
            ae = fmaf(ub2(E1), xs[12], ae);
            ao = fmaf(ub2(O1), xs[13], ao);
            ae = fmaf(ub3(E1), xs[14], ae);
            ao = fmaf(ub3(O1), xs[15], ao);
            t[sb] = fmaf(ao, 0.25f, ae);
        }
        return h2f(r.d) * fmaf(sc_f(r.sc, 1), t[1], sc_f(r.sc, 0) * t[0]);
    }
    __device__ static __forceinline__ void codes(const Row& r, float* q) {
        const uint32_t* ql = &r.ql.x;
        const uint32_t* qh = &r.qh.x;
#pragma unroll
        for (int sb = 0; sb < 2; sb++) {
            uint32_t E0, O0, E1, O1;
            run(ql[2 * sb], ql[2 * sb + 1], qh[sb], E0, O0, E1, O1);
            float* o = q + 16 * sb;
            o[0] = ub0(E0); o[1] = ub0(O0) * 0.25f; o[2] = ub1(E0); o[3] = ub1(O0) * 0.25f;
            o[4] = ub2(E0); o[5] = ub2(O0) * 0.25f; o[6] = ub3(E0); o[7] = ub3(O0) * 0.25f;
            o[8] = ub0(E1); o[9] = ub0(O1) * 0.25f; o[10] = ub1(E1); o[11] = ub1(O1) * 0.25f;
            o[12] = ub2(E1); o[13] = ub2(O1) * 0.25f; o[14] = ub3(E1); o[15] = ub3(O1) * 0.25f;
        }
    }
    __device__ static __forceinline__ void weights(const Row& r, float* w) {
        float q[WPC];
        codes(r, q);
        const float d = h2f(r.d);
#pragma unroll
        for (int k = 0; k < WPC; k++) w[k] = d * sc_f(r.sc, k >> 4) * (q[k] - OFF);
    }
};

// ----------------------------------------------------------------- Q25 ----
template <>
struct Traits<kQ25> {
    static constexpr int WPC = 64;
    static constexpr int F4 = 16;
    static constexpr int NBS = 2;    // one sum per 32-weight block
    static constexpr int BSG = 8;
    static constexpr float OFF = 2.f;
    struct Row {
        uint4 c;
        uint32_t s2;   // the chunk's two fp16 scales
    };
    __device__ static __forceinline__ DevPlanes base(const DevPlanes& P, int64_t row, int64_t K) {
        return DevPlanes{P.p0 + row * (K >> 2), nullptr, P.p2 + 2 * row * (K >> 5), nullptr};
    }
    __device__ static __forceinline__ void load(Row& r, const DevPlanes& B, int b) {
        r.c = *(const uint4*)(B.p0 + 16 * b);
        r.s2 = *(const uint32_t*)(B.p2 + 4 * b);
    }
    // dword i holds weights 16i..16i+15; byte j holds 16i+4j+{0,1,2,3} in
    // bits {0-1, 2-3, 4-5, 6-7}: masked, the byte is q, 4q, 16q or 64q.
    __device__ static __forceinline__ float dot(const Row& r, const float* xv, const float* mbs) {
        const uint32_t* c = &r.c.x;
        float t[2];
#pragma unroll
        for (int blk = 0; blk < 2; blk++) {
            float a0 = mbs[blk], a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
            for (int ii = 0; ii < 2; ii++) {
                const int i = 2 * blk + ii;
                const uint32_t d = c[i];
                const uint32_t m0 = d & 0x03030303u, m1 = d & 0x0C0C0C0Cu;
                const uint32_t m2 = d & 0x30303030u, m3 = d & 0xC0C0C0C0u;
                const float* xs = xv + 16 * i;
                a0 = fmaf(ub0(m0), xs[0], a0);  a1 = fmaf(ub0(m1), xs[1], a1);
                a2 = fmaf(ub0(m2), xs[2], a2);  a3 = fmaf(ub0(m3), xs[3], a3);
                a0 = fmaf(ub1(m0), xs[4], a0);  a1 = fmaf(ub1(m1), xs[5], a1);
                a2 = fmaf(ub1(m2), xs[6], a2);  a3 = fmaf(ub1(m3), xs[7], a3);
                a0 = fmaf(ub2(m0), xs[8], a0);  a1 = fmaf(ub2(m1), xs[9], a1);
                a2 = fmaf(ub2(m2), xs[10], a2); a3 = fmaf(ub2(m3), xs[11], a3);
                a0 = fmaf(ub3(m0), xs[12], a0); a1 = fmaf(ub3(m1), xs[13], a1);
                a2 = fmaf(ub3(m2), xs[14], a2); a3 = fmaf(ub3(m3), xs[15], a3);
            }
            t[blk] = fmaf(a3, 0.015625f, fmaf(a2, 0.0625f, fmaf(a1, 0.25f, a0)));
        }
        return fmaf(h2f(r.s2 >> 16), t[1], h2f(r.s2) * t[0]);
    }
    __device__ static __forceinline__ void codes(const Row& r, float* q) {
        const uint32_t* c = &r.c.x;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t d = c[i];
            const uint32_t m0 = d & 0x03030303u, m1 = d & 0x0C0C0C0Cu;
            const uint32_t m2 = d & 0x30303030u, m3 = d & 0xC0C0C0C0u;
            float* o = q + 16 * i;
            o[0] = ub0(m0); o[1] = ub0(m1) * 0.25f; o[2] = ub0(m2) * 0.0625f; o[3] = ub0(m3) * 0.015625f;
            o[4] = ub1(m0); o[5] = ub1(m1) * 0.25f; o[6] = ub1(m2) * 0.0625f; o[7] = ub1(m3) * 0.015625f;
            o[8] = ub2(m0); o[9] = ub2(m1) * 0.25f; o[10] = ub2(m2) * 0.0625f; o[11] = ub2(m3) * 0.015625f;
            o[12] = ub3(m0); o[13] = ub3(m1) * 0.25f; o[14] = ub3(m2) * 0.0625f; o[15] = ub3(m3) * 0.015625f;
        }
    }
    __device__ static __forceinline__ void weights(const Row& r, float* w) {
        float q[WPC];
        codes(r, q);
        const float s0 = h2f(r.s2), s1 = h2f(r.s2 >> 16);
#pragma unroll
        for (int k = 0; k < WPC; k++) w[k] = (k < 32 ? s0 : s1) * (q[k] - OFF);
    }
};

// ---------------------------------------------------------------- BF16 ----
template <>
struct Traits<kBF16> {
    static constexpr int WPC = 8;
    static constexpr int F4 = 2;
    static constexpr int NBS = 0;
    static constexpr int BSG = 1;
    static constexpr float OFF = 0.f;
    struct Row {
        uint4 w;
    };
    __device__ static __forceinline__ DevPlanes base(const DevPlanes& P, int64_t row, int64_t K) {
        return DevPlanes{P.p0 + 2 * row * K, nullptr, nullptr, nullptr};
    }
    __device__ static __forceinline__ void load(Row& r, const DevPlanes& B, int b) {
        r.w = *(const uint4*)(B.p0 + 16 * b);
    }
    __device__ static __forceinline__ float dot(const Row& r, const float* xv, const float*) {
        const uint32_t* c = &r.w.x;
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            a0 = fmaf(as_f(c[i] << 16), xv[2 * i], a0);
            a1 = fmaf(as_f(c[i] & 0xFFFF0000u), xv[2 * i + 1], a1);
        }
        return a0 + a1;
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

// Physical float4 slot, within LDS, of float4 j of chunk b.  Lanes read their
// chunk's x at a stride of F4 float4; rotating the slot by the chunk index
// spreads eight consecutive lanes over all banks.
template <int FMT>
__device__ __forceinline__ int x_slot(int b, int j) {
    constexpr int F4 = Traits<FMT>::F4;
    if constexpr (F4 >= 8)
        return F4 * b + (j ^ (b & 7));
    else
        return F4 * b + (j ^ ((b >> 2) & (F4 - 1)));
}

}  // namespace mbq
