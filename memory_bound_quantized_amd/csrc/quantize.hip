// quantize.hip -- fp32 weights [N][K] -> the block formats' planes (Q45,
// Q65, Q25; BF16 by rounding).
//
// The pages fix the formats by their byte budgets only ([roofline-holds]
// "The Math": 4.5 and 6.5625 bits per weight; "The search space": 256
// weights in 144 and 210 bytes); the scale rule is this library's: symmetric
// absmax per block, every integer decision taken in fp32 (correctly rounded
// division, round half to even), scales rounded to binary16 half to even and
// saturated at 65504:
//   Q45, Q25 (blocks of 32): s = half(max|w| / Qmax), Qmax = 7 or 1;
//       q = clamp(rint(w / s) + off, 0, 2^b - 1) (off 8 or 2; off if s = 0).
//   Q65 (super-blocks of 256, sub-blocks of 16): a_j = max_j |w| / 31;
//       d = half(max a_j / 127); sc_j = clamp(rint(a_j / d), -128, 127)
//       (0 if d = 0); q = clamp(rint(w / (d sc_j)) + 32, 0, 63) (32 if
//       d sc_j = 0).
//   BF16: round to nearest even.
// The kernel reads each weight once and writes each plane byte once: an
// HBM-bound pass over 4 bytes per weight in and bits/8 out.
//
// Lanes: a Q45/Q25 block of 32 weights is 4 adjacent lanes of 8 values (the
// block maximum over the 4 by two lane exchanges); a Q65 super-block is 32
// adjacent lanes, sub-block j the lane pair (2j, 2j + 1).
#include "device_common.h"
#include "kernels.h"

namespace mbq {

typedef float qf4 __attribute__((ext_vector_type(4)));
typedef uint32_t qu4 __attribute__((ext_vector_type(4)));

// Bit of a 16-weight run's 32-bit high-bits word that holds weight r of the
// run (the Q65 codes_hi layout of mbq.h).
__constant__ int kQ65HiPos[16] = {4, 2, 12, 10, 20, 18, 28, 26, 0, 6, 8, 14, 16, 22, 24, 30};

__device__ __forceinline__ float half_sat(float t) {
    return (float)(_Float16)fminf(t, 65504.0f);      // t >= 0: RNE, saturating
}
__device__ __forceinline__ uint16_t half_bits(float v) {
    return __builtin_bit_cast(uint16_t, (_Float16)v);   // v is a half already
}
// v, through an empty asm: without it the compiler folds a lane swap of a
// value with itself into two equal results and drops the exchange.
static __device__ __forceinline__ uint32_t distinct_copy(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}

// rint(v / s) with v / s the correctly rounded fp32 quotient, for s > 0 with
// 1/s a normal float (r = v_rcp_f32(s), within 1 ulp of 1/s).  t = v r is
// within 1.5 2^-23 |t| of v / s, and the rounded quotient within 2^-24 |t|;
// for |t| < 64 both errors are below 2^-16, so where t lies more than 2^-14
// from the nearest k + 1/2 the two round to the same integer.  Only near a
// tie (about 2^-13 of uniform quotients) is the exact division taken.
__device__ __forceinline__ float rint_quot(float v, float s, float r) {
    const float t = v * r;
    const float f = rintf(t);
    if (fabsf(t - f) < 0.5f - 0x1p-14f && fabsf(t) < 64.f) return f;
    return rintf(v / s);
}

template <int FMT>
__global__ __launch_bounds__(kBlock) void quantize_kernel(const float* __restrict__ w, int64_t ldw,
                                                          int64_t N, int64_t K, DevPlanes out,
                                                          int64_t nthreads) {
    const int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    // every thread of a block's lane group takes part in the exchanges;
    // threads past the end (last workgroup only) compute on zeros and store
    // nothing
    const bool ok = t < nthreads;
    const int64_t per_row = K / 8;                   // 8-value items per row
    const int64_t row = ok ? t / per_row : 0;
    const int64_t item = ok ? t % per_row : 0;
    const int64_t k0 = 8 * item;
    float v[8];
    {
        const qf4* src = (const qf4*)(w + row * ldw + k0);
        const qf4 a = ok ? src[0] : qf4{0.f, 0.f, 0.f, 0.f};
        const qf4 b = ok ? src[1] : qf4{0.f, 0.f, 0.f, 0.f};
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    uint8_t* p0 = (uint8_t*)out.p0;
    if constexpr (FMT == kBF16) {
        uint32_t h[8];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const uint32_t bits = __builtin_bit_cast(uint32_t, v[i]);
            h[i] = (bits + 0x7FFFu + ((bits >> 16) & 1u)) >> 16;
        }
        if (ok)
            *(qu4*)(p0 + 2 * (row * K + k0)) =
                qu4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
        return;
    }
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 8; i++) m = fmaxf(m, fabsf(v[i]));
    if constexpr (FMT == kQ45 || FMT == kQ25) {
        constexpr float QMAX = FMT == kQ45 ? 7.0f : 1.0f;
        constexpr int OFF = FMT == kQ45 ? 8 : 2, TOP = FMT == kQ45 ? 15 : 3;
        m = fmaxf(m, lane_xor1(m));
        m = fmaxf(m, lane_xor2(m));
        const float s = half_sat(m / QMAX);
        int q[8];
        const float sd = s != 0.f ? s : 1.0f;         // s = 0: every code is the offset
        const float rd = __builtin_amdgcn_rcpf(sd);   // sd >= 2^-24: 1/sd is normal
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int c = s != 0.f ? (int)rint_quot(v[i], sd, rd) + OFF : OFF;
            q[i] = c < 0 ? 0 : (c > TOP ? TOP : c);
        }
        if (!ok) return;
        const int g = (int)(item & 3);
        const int64_t b = item >> 2;                  // block within the row
        if constexpr (FMT == kQ45) {
            uint32_t word = 0;
#pragma unroll
            for (int i = 0; i < 8; i++) word |= (uint32_t)q[i] << (4 * i);
            *(uint32_t*)(p0 + (row * K + k0) / 2) = word;
        } else {
            uint32_t word = 0;
#pragma unroll
            for (int i = 0; i < 8; i++) word |= (uint32_t)q[i] << (2 * i);
            *(uint16_t*)(p0 + (row * K + k0) / 4) = (uint16_t)word;
        }
        if (g == 0) *(uint16_t*)((uint8_t*)out.p2 + 2 * (row * (K / 32) + b)) = half_bits(s);
    } else {   // Q65
        const float a = fmaxf(m, lane_xor1(m)) / 31.0f;   // this sub-block's a_j
        // the maximum over the super-block's 32 lanes: quads, eights and
        // sixteens by DPP (a mirror pairs each half with the other one),
        // then the two halves of the 32 (rows 2i and 2i + 1 of the wave) by
        // a row swap of the value with itself, which hands each lane its
        // partner's value; that maximum is taken on the bits (the same
        // order for non-negative floats)
        float amx = fmaxf(a, lane_xor2(a));
        amx = fmaxf(amx, lane_mirror8(amx));
        amx = fmaxf(amx, lane_mirror16(amx));
        {
            const uint32_t b = __builtin_bit_cast(uint32_t, amx);
            auto h = __builtin_amdgcn_permlane16_swap(b, distinct_copy(b), false, false);
            amx = __builtin_bit_cast(float, h[0] > h[1] ? h[0] : h[1]);
        }
        const float d = half_sat(amx / 127.0f);
        int sc = 0;
        if (d != 0.f) {
            const int r = (int)rintf(a / d);
            sc = r < -128 ? -128 : (r > 127 ? 127 : r);
        }
        const float step = d * (float)sc;             // exact: 11 + 7 significant bits
        int q[8];
        const float stepd = step != 0.f ? step : 1.0f;
        const float rs = __builtin_amdgcn_rcpf(stepd); // stepd in [2^-24, 65504 * 127]
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int c = step != 0.f ? (int)rint_quot(v[i], stepd, rs) + 32 : 32;
            q[i] = c < 0 ? 0 : (c > 63 ? 63 : c);
        }
        const int li = (int)(item & 31);               // lane within the super-block
        const int part = li & 1;                       // run positions 0-7 or 8-15
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            lo |= (uint32_t)(q[i] & 15) << (4 * i);
            hi |= (uint32_t)(q[i] >> 4) << kQ65HiPos[8 * part + i];
        }
        hi |= (uint32_t)lane_xor1((int)hi);
        if (!ok) return;
        *(uint32_t*)(p0 + (row * K + k0) / 2) = lo;
        if (part == 0) {
            const int64_t run = (row * K + k0) / 16;   // 16-weight run = sub-block
            *(uint32_t*)((uint8_t*)out.p1 + 4 * run) = hi;
            ((int8_t*)out.p2)[run] = (int8_t)sc;
        }
        if (li == 0) *(uint16_t*)((uint8_t*)out.p3 + 2 * ((row * K + k0) / 256)) = half_bits(d);
    }
}

hipError_t launch_quantize(int fmt, const float* w, int64_t ldw, int64_t N, int64_t K,
                           DevPlanes out, hipStream_t stream) {
    const int64_t nthreads = N * (K / 8);
    if (nthreads == 0) return hipSuccess;
    const dim3 grid((unsigned)((nthreads + kBlock - 1) / kBlock)), block(kBlock);
    switch (fmt) {
    case kQ45: hipLaunchKernelGGL(quantize_kernel<kQ45>, grid, block, 0, stream, w, ldw, N, K, out, nthreads); break;
    case kQ65: hipLaunchKernelGGL(quantize_kernel<kQ65>, grid, block, 0, stream, w, ldw, N, K, out, nthreads); break;
    case kQ25: hipLaunchKernelGGL(quantize_kernel<kQ25>, grid, block, 0, stream, w, ldw, N, K, out, nthreads); break;
    default: hipLaunchKernelGGL(quantize_kernel<kBF16>, grid, block, 0, stream, w, ldw, N, K, out, nthreads); break;
    }
    return hipGetLastError();
}

}  // namespace mbq
