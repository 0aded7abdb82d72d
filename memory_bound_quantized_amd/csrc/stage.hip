// stage.hip -- kernels that produce staged x (staging.h) in global memory.
//
// A matrix-vector product needs its input in staged form in every workgroup.
// Staging once, in the kernel that produces the vector, leaves the product's
// workgroups only a copy of 4 bytes per value into LDS.  This is the
// pages' fusion of the small kernels between weight reads into the
// neighbouring ones ([roofline-holds] "Hiding, fusing, and keeping the sums
// busy"; "Where the time goes": the norms and adds between weight reads).
#include "device_common.h"
#include "formats.h"
#include "kernels.h"
#include "staging.h"

namespace mbq {

// ---- stand-alone staging: M rows of fp32 x --------------------------------
// grid (ceil(groups / 256), M); one group of GX values per thread.
template <int FMT>
__global__ __launch_bounds__(kBlock) void stage_x_kernel(const float* __restrict__ x, int64_t ldx,
                                                         int K, uint32_t* __restrict__ xq) {
    using T = Traits<FMT>;
    constexpr int GF4 = T::GX / 4;
    const int64_t m = blockIdx.y;
    const int ngroups = K / T::GX;
    const int og = (int)blockIdx.x * kBlock + (int)threadIdx.x;
    const bool ok = og < ngroups;
    const float4* src = (const float4*)(x + m * ldx) + (int64_t)og * GF4;
    float4 v[GF4];
#pragma unroll
    for (int j = 0; j < GF4; j++) v[j] = ok ? src[j] : make_float4(0.f, 0.f, 0.f, 0.f);
    stage_group<FMT>((const float*)v, og, ok, GlobalDst<FMT>{xq + m * K});
}

template <int FMT>
static hipError_t stage_x_f(const float* x, int64_t M, int64_t ldx, int64_t K, void* xq,
                            hipStream_t stream) {
    const int64_t ngroups = K / Traits<FMT>::GX;
    const dim3 grid((unsigned)((ngroups + kBlock - 1) / kBlock), (unsigned)M);
    hipLaunchKernelGGL(stage_x_kernel<FMT>, grid, dim3(kBlock), 0, stream, x, ldx, (int)K,
                       (uint32_t*)xq);
    return hipGetLastError();
}

hipError_t launch_stage_x(int fmt, const float* x, int64_t M, int64_t ldx, int64_t K, void* xq,
                          hipStream_t stream) {
    if (M == 0 || K == 0) return hipSuccess;
    switch (fmt) {
    case kQ45: return stage_x_f<kQ45>(x, M, ldx, K, xq, stream);
    case kQ65: return stage_x_f<kQ65>(x, M, ldx, K, xq, stream);
    case kQ25: return stage_x_f<kQ25>(x, M, ldx, K, xq, stream);
    case kBF16: return stage_x_f<kBF16>(x, M, ldx, K, xq, stream);
    }
    return hipErrorInvalidValue;
}

// ---- RMSNorm of one row, emitting staged output ----------------------------
// As the plain RMSNorm kernel (norms.hip), in the same geometry (norm_geom),
// so y is bit for bit mbq_rmsnorm's: values in registers, one block-wide sum;
// the normalised row then goes through LDS so each thread can stage a group
// of GX consecutive values.  n <= BT * 4 * VEC, n % 4 == 0.
template <int FMT, int VEC, int BT>
__global__ __launch_bounds__(BT) void rmsnorm_xq_kernel(const float* x,
                                                        const float* __restrict__ gamma,
                                                        float eps, int n, float* y,
                                                        uint32_t* __restrict__ xq) {
    using T = Traits<FMT>;
    __shared__ float red[BT / kWave];
    __shared__ float4 row[VEC * BT];
    const int n4 = n >> 2;
    const float4* x4 = (const float4*)x;
    const float4* g4 = (const float4*)gamma;
    float4 v[VEC], g[VEC];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < VEC; i++) {
        const int f = i * BT + (int)threadIdx.x;
        v[i] = f < n4 ? x4[f] : make_float4(0.f, 0.f, 0.f, 0.f);
        g[i] = f < n4 ? g4[f] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int i = 0; i < VEC; i++) {
        ss = fmaf(v[i].x, v[i].x, ss);
        ss = fmaf(v[i].y, v[i].y, ss);
        ss = fmaf(v[i].z, v[i].z, ss);
        ss = fmaf(v[i].w, v[i].w, ss);
    }
    const float tot = block_sum<BT / kWave, false>(ss, red);
    const float inv = 1.0f / sqrtf(tot / (float)n + eps);
#pragma unroll
    for (int i = 0; i < VEC; i++) {
        const int f = i * BT + (int)threadIdx.x;
        const float4 o = make_float4(g[i].x * (v[i].x * inv), g[i].y * (v[i].y * inv),
                                     g[i].z * (v[i].z * inv), g[i].w * (v[i].w * inv));
        row[f] = o;
        if (y != nullptr && f < n4) ((float4*)y)[f] = o;
    }
    __syncthreads();
    constexpr int GF4 = T::GX / 4;
    const int ngroups = n / T::GX;
    const int rounds = (ngroups + BT - 1) / BT;
    for (int rd = 0; rd < rounds; rd++) {
        const int og = rd * BT + (int)threadIdx.x;
        const bool ok = og < ngroups;
        float4 w[GF4];
#pragma unroll
        for (int j = 0; j < GF4; j++) w[j] = ok ? row[og * GF4 + j] : make_float4(0.f, 0.f, 0.f, 0.f);
        stage_group<FMT>((const float*)w, og, ok, GlobalDst<FMT>{xq});
    }
}

template <int FMT>
static hipError_t rmsnorm_xq_f(const float* x, const float* gamma, float eps, int64_t n, float* y,
                               void* xq, hipStream_t stream) {
    const NormGeom ng = norm_geom(n);                // n <= 8192: at most 2 float4s of 1024 threads
    const dim3 grid(1);
    uint32_t* q = (uint32_t*)xq;
    if (ng.bt == 256)
        hipLaunchKernelGGL((rmsnorm_xq_kernel<FMT, 1, 256>), grid, dim3(256), 0, stream, x, gamma, eps, (int)n, y, q);
    else if (ng.vec == 1)
        hipLaunchKernelGGL((rmsnorm_xq_kernel<FMT, 1, 1024>), grid, dim3(1024), 0, stream, x, gamma, eps, (int)n, y, q);
    else
        hipLaunchKernelGGL((rmsnorm_xq_kernel<FMT, 2, 1024>), grid, dim3(1024), 0, stream, x, gamma, eps, (int)n, y, q);
    return hipGetLastError();
}

hipError_t launch_rmsnorm_xq(const float* x, const float* gamma, float eps, int64_t n, float* y,
                             int fmt, void* xq, hipStream_t stream) {
    switch (fmt) {
    case kQ45: return rmsnorm_xq_f<kQ45>(x, gamma, eps, n, y, xq, stream);
    case kQ65: return rmsnorm_xq_f<kQ65>(x, gamma, eps, n, y, xq, stream);
    case kQ25: return rmsnorm_xq_f<kQ25>(x, gamma, eps, n, y, xq, stream);
    case kBF16: return rmsnorm_xq_f<kBF16>(x, gamma, eps, n, y, xq, stream);
    }
    return hipErrorInvalidValue;
}

// ---- silu(g) * u, emitting staged output -----------------------------------
// Same arithmetic as the plain silu_mul kernel; one group per thread.
template <int FMT>
__global__ __launch_bounds__(kBlock) void silu_mul_xq_kernel(const float* __restrict__ g,
                                                             const float* __restrict__ u, int n,
                                                             uint32_t* __restrict__ xq) {
    using T = Traits<FMT>;
    constexpr int GF4 = T::GX / 4;
    const int ngroups = n / T::GX;
    const int og = (int)blockIdx.x * kBlock + (int)threadIdx.x;
    const bool ok = og < ngroups;
    float4 a[GF4], b[GF4];
#pragma unroll
    for (int j = 0; j < GF4; j++) {
        a[j] = ok ? ((const float4*)g)[og * GF4 + j] : make_float4(0.f, 0.f, 0.f, 0.f);
        b[j] = ok ? ((const float4*)u)[og * GF4 + j] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float v[T::GX];
#pragma unroll
    for (int k = 0; k < T::GX; k++) {
        const float t = ((const float*)a)[k];
        v[k] = t / (1.0f + expf(-t)) * ((const float*)b)[k];
    }
    stage_group<FMT>(v, og, ok, GlobalDst<FMT>{xq});
}

template <int FMT>
static hipError_t silu_mul_xq_f(const float* g, const float* u, int64_t n, void* xq,
                                hipStream_t stream) {
    const int64_t ngroups = n / Traits<FMT>::GX;
    hipLaunchKernelGGL(silu_mul_xq_kernel<FMT>, dim3((unsigned)((ngroups + kBlock - 1) / kBlock)),
                       dim3(kBlock), 0, stream, g, u, (int)n, (uint32_t*)xq);
    return hipGetLastError();
}

hipError_t launch_silu_mul_xq(const float* g, const float* u, int64_t n, int fmt, void* xq,
                              hipStream_t stream) {
    if (n == 0) return hipSuccess;
    switch (fmt) {
    case kQ45: return silu_mul_xq_f<kQ45>(g, u, n, xq, stream);
    case kQ65: return silu_mul_xq_f<kQ65>(g, u, n, xq, stream);
    case kQ25: return silu_mul_xq_f<kQ25>(g, u, n, xq, stream);
    case kBF16: return silu_mul_xq_f<kBF16>(g, u, n, xq, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace mbq
