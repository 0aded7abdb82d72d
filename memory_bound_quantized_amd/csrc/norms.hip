// norms.hip -- cooperative row norms and the gated glue.
//
// One 256-thread workgroup per row: each thread sums its share of the row
// (held in registers), the partial sums are combined by a wave shuffle tree
// and then across the 4 waves through LDS ([one-serial-kernel] "One thread":
// the serial one-thread-per-row kernel was replaced by a group of 256 threads
// that each sum their part and combine the parts).  LayerNorm makes two
// passes over the register-resident values: the mean first, then the biased
// variance of the centred values, so no E[x^2] - mean^2 cancellation occurs.
#include "device_common.h"
#include "kernels.h"

namespace mbq {

// BT threads per row (norm_geom): 1024 from 1025 values, so that a single
// row's latency chain (load, sum, scale, store) has as little serial work per
// thread as possible.
template <int VEC, int BT>
__global__ __launch_bounds__(BT) void rmsnorm_vec_kernel(const float* x,
                                                         const float* __restrict__ gamma,
                                                         float eps, int n, float* y) {
    __shared__ float red[BT / kWave];
    const int64_t row = blockIdx.x;
    const int n4 = n >> 2;
    const float4* xr = (const float4*)(x + row * n);
    const float4* g4 = (const float4*)gamma;
    // gamma is requested with x, so no memory round trip follows the
    // block-wide sum on the single-row critical path
    float4 v[VEC], g[VEC];
#pragma unroll
    for (int i = 0; i < VEC; i++) {
        const int f = i * BT + (int)threadIdx.x;
        v[i] = f < n4 ? xr[f] : make_float4(0.f, 0.f, 0.f, 0.f);
        g[i] = f < n4 ? g4[f] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < VEC; i++) {
        ss = fmaf(v[i].x, v[i].x, ss);
        ss = fmaf(v[i].y, v[i].y, ss);
        ss = fmaf(v[i].z, v[i].z, ss);
        ss = fmaf(v[i].w, v[i].w, ss);
    }
    const float tot = block_sum<BT / kWave, false>(ss, red);
    const float inv = 1.0f / sqrtf(tot / (float)n + eps);
    float4* yr = (float4*)(y + row * n);
#pragma unroll
    for (int i = 0; i < VEC; i++) {
        const int f = i * BT + (int)threadIdx.x;
        if (f < n4)
            yr[f] = make_float4(g[i].x * (v[i].x * inv), g[i].y * (v[i].y * inv),
                                g[i].z * (v[i].z * inv), g[i].w * (v[i].w * inv));
    }
}

// Any n and alignment: values re-read from memory for the second pass.
__global__ __launch_bounds__(kBlock) void rmsnorm_any_kernel(const float* x,
                                                             const float* __restrict__ gamma,
                                                             float eps, int64_t n, float* y) {
    __shared__ float red[kWavesPerBlock];
    const int64_t row = blockIdx.x;
    const float* xr = x + row * n;
    float ss = 0.f;
    for (int64_t i = threadIdx.x; i < n; i += kBlock) ss = fmaf(xr[i], xr[i], ss);
    const float tot = block_sum<kWavesPerBlock, false>(ss, red);
    const float inv = 1.0f / sqrtf(tot / (float)n + eps);
    float* yr = y + row * n;
    for (int64_t i = threadIdx.x; i < n; i += kBlock) yr[i] = gamma[i] * (xr[i] * inv);
}

template <int VEC>
__global__ __launch_bounds__(kBlock) void layernorm_vec_kernel(const float* x,
                                                               const float* __restrict__ gamma,
                                                               const float* __restrict__ beta,
                                                               float eps, int n, float* y) {
    __shared__ float red[kWavesPerBlock];
    const int64_t row = blockIdx.x;
    const int n4 = n >> 2;
    const float4* xr = (const float4*)(x + row * n);
    float4 v[VEC];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < VEC; i++) {
        const int f = i * kBlock + (int)threadIdx.x;
        v[i] = f < n4 ? xr[f] : make_float4(0.f, 0.f, 0.f, 0.f);
        s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
    }
    const float mean = block_sum(s, red) / (float)n;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < VEC; i++) {
        const int f = i * kBlock + (int)threadIdx.x;
        if (f < n4) {
            const float a = v[i].x - mean, b = v[i].y - mean, c = v[i].z - mean, d = v[i].w - mean;
            q = fmaf(a, a, q);
            q = fmaf(b, b, q);
            q = fmaf(c, c, q);
            q = fmaf(d, d, q);
        }
    }
    const float var = block_sum<kWavesPerBlock, false>(q, red) / (float)n;
    const float inv = 1.0f / sqrtf(var + eps);
    float4* yr = (float4*)(y + row * n);
    const float4* g4 = (const float4*)gamma;
    const float4* b4 = (const float4*)beta;
#pragma unroll
    for (int i = 0; i < VEC; i++) {
        const int f = i * kBlock + (int)threadIdx.x;
        if (f < n4) {
            const float4 g = g4[f], b = b4[f];
            yr[f] = make_float4(fmaf((v[i].x - mean) * inv, g.x, b.x),
                                fmaf((v[i].y - mean) * inv, g.y, b.y),
                                fmaf((v[i].z - mean) * inv, g.z, b.z),
                                fmaf((v[i].w - mean) * inv, g.w, b.w));
        }
    }
}

// One row per wave for rows of 64 * 4 * NV values (256 ... 4096): lane l
// holds float4s l, l + 64, ... of the row, and both statistics are wave
// reductions (DPP), with no workgroup barrier.  gamma and beta are loaded
// with x, so the row's single round trip covers all three.  Against one
// workgroup per row (µs, 8.4 M values, graphs of cold launches, same run):
// 4096 x 2048 12.65 against 14.3; rows of 256 14.2 against 29.2, of 512
// 12.7 against 19.4, of 1024 12.6 against 14.5, of 4096 13.1 against 14.8.
// MBQ_LN_WAVE=0 (tuning) keeps the workgroup-per-row kernels.
template <int NV>
__global__ __launch_bounds__(kBlock) void layernorm_wave_kernel(const float* x,
                                                                const float* __restrict__ gamma,
                                                                const float* __restrict__ beta,
                                                                float eps, int n, int64_t rows,
                                                                float* y) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t row = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
    if (row >= rows) return;                                  // the whole wave
    const float4* xr = (const float4*)(x + row * n);
    const float4* g4 = (const float4*)gamma;
    const float4* b4 = (const float4*)beta;
    float4 v[NV], g[NV], b[NV];
#pragma unroll
    for (int i = 0; i < NV; i++) v[i] = xr[lane + kWave * i];
#pragma unroll
    for (int i = 0; i < NV; i++) {
        g[i] = g4[lane + kWave * i];
        b[i] = b4[lane + kWave * i];
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NV; i++) s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
    const float mean = wave_sum_dpp(s) / (float)n;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < NV; i++) {
        const float a = v[i].x - mean, c = v[i].y - mean, d = v[i].z - mean, e = v[i].w - mean;
        q = fmaf(a, a, q);
        q = fmaf(c, c, q);
        q = fmaf(d, d, q);
        q = fmaf(e, e, q);
    }
    const float var = wave_sum_dpp(q) / (float)n;
    const float inv = 1.0f / sqrtf(var + eps);
    float4* yr = (float4*)(y + row * n);
#pragma unroll
    for (int i = 0; i < NV; i++)
        yr[lane + kWave * i] = make_float4(fmaf((v[i].x - mean) * inv, g[i].x, b[i].x),
                                           fmaf((v[i].y - mean) * inv, g[i].y, b[i].y),
                                           fmaf((v[i].z - mean) * inv, g[i].z, b[i].z),
                                           fmaf((v[i].w - mean) * inv, g[i].w, b[i].w));
}

__global__ __launch_bounds__(kBlock) void layernorm_any_kernel(const float* x,
                                                               const float* __restrict__ gamma,
                                                               const float* __restrict__ beta,
                                                               float eps, int64_t n, float* y) {
    __shared__ float red[kWavesPerBlock];
    const int64_t row = blockIdx.x;
    const float* xr = x + row * n;
    float s = 0.f;
    for (int64_t i = threadIdx.x; i < n; i += kBlock) s += xr[i];
    const float mean = block_sum(s, red) / (float)n;
    float q = 0.f;
    for (int64_t i = threadIdx.x; i < n; i += kBlock) {
        const float a = xr[i] - mean;
        q = fmaf(a, a, q);
    }
    const float inv = 1.0f / sqrtf(block_sum<kWavesPerBlock, false>(q, red) / (float)n + eps);
    float* yr = y + row * n;
    for (int64_t i = threadIdx.x; i < n; i += kBlock)
        yr[i] = fmaf((xr[i] - mean) * inv, gamma[i], beta[i]);
}

static int vec_for(int64_t n) {
    const int64_t n4 = n >> 2;
    if (n4 <= kBlock) return 1;
    if (n4 <= 2 * kBlock) return 2;
    if (n4 <= 4 * kBlock) return 4;
    if (n4 <= 8 * kBlock) return 8;
    return 0;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

hipError_t launch_rmsnorm(const float* x, const float* gamma, float eps, int64_t rows, int64_t n,
                          float* y, hipStream_t stream) {
    const bool vec = n % 4 == 0 && aligned16(x) && aligned16(y) && aligned16(gamma);
    const NormGeom ng = vec ? norm_geom(n) : NormGeom{0, kBlock};
    const dim3 grid((unsigned)rows);
#define MBQ_RMS(V, B) hipLaunchKernelGGL((rmsnorm_vec_kernel<V, B>), grid, dim3(B), 0, stream, x, gamma, eps, (int)n, y)
    if (ng.vec == 1 && ng.bt == kBlock) MBQ_RMS(1, kBlock);
    else if (ng.vec == 1) MBQ_RMS(1, 1024);
    else if (ng.vec == 2) MBQ_RMS(2, 1024);
    else if (ng.vec == 4) MBQ_RMS(4, 1024);
    else if (ng.vec == 8) MBQ_RMS(8, 1024);
    else hipLaunchKernelGGL(rmsnorm_any_kernel, grid, dim3(kBlock), 0, stream, x, gamma, eps, n, y);
#undef MBQ_RMS
    return hipGetLastError();
}

hipError_t launch_layernorm(const float* x, const float* gamma, const float* beta, float eps,
                            int64_t rows, int64_t n, float* y, hipStream_t stream) {
    const bool al = n % 4 == 0 && aligned16(x) && aligned16(y) && aligned16(gamma) && aligned16(beta);
    const int64_t nv = n / (4 * kWave);
    const bool wave = al && n % (4 * kWave) == 0 && (nv == 1 || nv == 2 || nv == 4 || nv == 8 || nv == 16) &&
                      !(tuning_var("MBQ_LN_WAVE") && atoi(tuning_var("MBQ_LN_WAVE")) == 0);
    if (wave) {
        const dim3 wgrid((unsigned)((rows + kWavesPerBlock - 1) / kWavesPerBlock));
        switch (nv) {
#define MBQ_LNW(V) case V: hipLaunchKernelGGL(layernorm_wave_kernel<V>, wgrid, dim3(kBlock), 0, stream, x, gamma, beta, eps, (int)n, rows, y); break;
        MBQ_LNW(1) MBQ_LNW(2) MBQ_LNW(4) MBQ_LNW(8) MBQ_LNW(16)
#undef MBQ_LNW
        }
        return hipGetLastError();
    }
    const int vec = al ? vec_for(n) : 0;
    const dim3 grid((unsigned)rows), block(kBlock);
    switch (vec) {
    case 1: hipLaunchKernelGGL(layernorm_vec_kernel<1>, grid, block, 0, stream, x, gamma, beta, eps, (int)n, y); break;
    case 2: hipLaunchKernelGGL(layernorm_vec_kernel<2>, grid, block, 0, stream, x, gamma, beta, eps, (int)n, y); break;
    case 4: hipLaunchKernelGGL(layernorm_vec_kernel<4>, grid, block, 0, stream, x, gamma, beta, eps, (int)n, y); break;
    case 8: hipLaunchKernelGGL(layernorm_vec_kernel<8>, grid, block, 0, stream, x, gamma, beta, eps, (int)n, y); break;
    default: hipLaunchKernelGGL(layernorm_any_kernel, grid, block, 0, stream, x, gamma, beta, eps, n, y); break;
    }
    return hipGetLastError();
}

__global__ __launch_bounds__(kBlock) void silu_mul_kernel(const float* g, const float* u, int64_t n,
                                                          float* out) {
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i < n) {
        const float t = g[i];
        out[i] = t / (1.0f + expf(-t)) * u[i];
    }
}

hipError_t launch_silu_mul(const float* g, const float* u, int64_t n, float* out,
                           hipStream_t stream) {
    hipLaunchKernelGGL(silu_mul_kernel, dim3((unsigned)((n + kBlock - 1) / kBlock)), dim3(kBlock),
                       0, stream, g, u, n, out);
    return hipGetLastError();
}

}  // namespace mbq
