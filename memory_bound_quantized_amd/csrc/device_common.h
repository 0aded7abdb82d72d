// device_common.h -- small device helpers shared by the libmbq kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mbq {

constexpr int kWave = 64;        // CDNA wavefront width
constexpr int kBlock = 256;      // threads per workgroup for every kernel here
constexpr int kWavesPerBlock = kBlock / kWave;

// Byte j of a dword -> float, one VALU op each (v_cvt_f32_ubyte{0..3}).  The
// compiler folds masks into its own byte extraction when it can see them, so
// the instructions are written out to keep one op per converted code.
__device__ __forceinline__ float ub0(uint32_t v) {
    float r;
    asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(r) : "v"(v));
    return r;
}
__device__ __forceinline__ float ub1(uint32_t v) {
    float r;
    asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(r) : "v"(v));
    return r;
}
__device__ __forceinline__ float ub2(uint32_t v) {
    float r;
    asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(r) : "v"(v));
    return r;
}
__device__ __forceinline__ float ub3(uint32_t v) {
    float r;
    asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(r) : "v"(v));
    return r;
}

// fp16 bit pattern (low 16 bits) -> float (v_cvt_f32_f16, exact).
__device__ __forceinline__ float h2f(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xFFFFu));
}

__device__ __forceinline__ float as_f(uint32_t bits) { return __builtin_bit_cast(float, bits); }

// Sum over the 64 lanes of a wave; every lane receives the total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float v) {
    const int s = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF,
                                              false);
    return v + __builtin_bit_cast(float, s);
}

// Lane exchanges by DPP (a vector move, no LDS traffic).  Every lane of the
// group involved must be active.
template <int CTRL>
__device__ __forceinline__ int dpp_mov(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ int lane_xor1(int v) { return dpp_mov<0xB1>(v); }      // quad_perm [1,0,3,2]
__device__ __forceinline__ int lane_xor2(int v) { return dpp_mov<0x4E>(v); }      // quad_perm [2,3,0,1]
__device__ __forceinline__ int lane_mirror8(int v) { return dpp_mov<0x141>(v); }  // lane 7 - i of 8
__device__ __forceinline__ int lane_mirror16(int v) { return dpp_mov<0x140>(v); } // lane 15 - i of 16
__device__ __forceinline__ float lane_xor1(float v) {
    return __builtin_bit_cast(float, lane_xor1(__builtin_bit_cast(int, v)));
}
__device__ __forceinline__ float lane_xor2(float v) {
    return __builtin_bit_cast(float, lane_xor2(__builtin_bit_cast(int, v)));
}
__device__ __forceinline__ float lane_mirror8(float v) {
    return __builtin_bit_cast(float, lane_mirror8(__builtin_bit_cast(int, v)));
}
__device__ __forceinline__ float lane_mirror16(float v) {
    return __builtin_bit_cast(float, lane_mirror16(__builtin_bit_cast(int, v)));
}

// Sum over the 64 lanes of a wave with DPP row operations; the total is
// returned as a wave-uniform value (read from lane 63).
__device__ __forceinline__ float wave_sum_dpp(float v) {
    v = dpp_add<0xB1, 0xF>(v);    // quad_perm [1,0,3,2]
    v = dpp_add<0x4E, 0xF>(v);    // quad_perm [2,3,0,1]
    v = dpp_add<0x141, 0xF>(v);   // row_half_mirror: 8-lane sums
    v = dpp_add<0x140, 0xF>(v);   // row_mirror: 16-lane sums
    v = dpp_add<0x142, 0xA>(v);   // row_bcast:15 into rows 1, 3
    v = dpp_add<0x143, 0xC>(v);   // row_bcast:31 into rows 2, 3
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Sum over aligned groups of G lanes (G a power of two <= 64).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int o = G / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// Sum over the NW waves of a workgroup: a DPP wave reduction, then the wave
// sums through LDS (red holds NW floats), added in wave order.  Every thread
// receives the total.  A second barrier after the read lets the caller use
// red again; a kernel that sums once passes REUSE = false and skips it.
template <int NW = kWavesPerBlock, bool REUSE = true>
__device__ __forceinline__ float block_sum(float v, float* red) {
    v = wave_sum_dpp(v);
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float t = red[0];
#pragma unroll
    for (int w = 1; w < NW; w++) t += red[w];
    if constexpr (REUSE) __syncthreads();
    return t;
}

}  // namespace mbq
