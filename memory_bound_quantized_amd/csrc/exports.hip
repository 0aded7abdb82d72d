// exports.hip -- device unpack/dequant exports and the bandwidth probes.
//
// mbq_dequant_f32 / mbq_unpack_codes run the exact in-register unpack the
// GEMV kernels use (formats.h) and write its result out, so the unpack can
// be checked bit for bit against an independent decoder.
//
// The probes measure the memory ceiling instead of quoting it
// ([roofline-holds] "The Math": measure the ceiling; "How I ran it": a large
// copy inside the chip, read and write counted as traffic).
#include "device_common.h"
#include "formats.h"
#include "kernels.h"

namespace mbq {

template <int FMT>
__global__ __launch_bounds__(kBlock) void dequant_kernel(DevPlanes P, int64_t N, int64_t K,
                                                         float* __restrict__ w) {
    using T = Traits<FMT>;
    const int64_t nchunks = K / T::WPC;
    const int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (t >= N * nchunks) return;
    const int64_t row = t / nchunks, b = t - row * nchunks;
    typename T::Row r;
    T::template load<false>(r, T::planes(P, N, K), T::row_off(row, K), (int)b);
    float v[T::WPC];
    T::weights(r, v);
    float4* o = (float4*)(w + row * K + b * T::WPC);
#pragma unroll
    for (int i = 0; i < T::WPC / 4; i++)
        o[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
}

template <int FMT>
__global__ __launch_bounds__(kBlock) void codes_kernel(DevPlanes P, int64_t N, int64_t K,
                                                       uint8_t* __restrict__ out) {
    using T = Traits<FMT>;
    const int64_t nchunks = K / T::WPC;
    const int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (t >= N * nchunks) return;
    const int64_t row = t / nchunks, b = t - row * nchunks;
    typename T::Row r;
    T::template load<false>(r, T::planes(P, N, K), T::row_off(row, K), (int)b);
    int q[T::WPC];
    T::codes(r, q);
    uint8_t* o = out + row * K + b * T::WPC;
#pragma unroll
    for (int k = 0; k < T::WPC; k++) o[k] = (uint8_t)q[k];
}

hipError_t launch_dequant(int fmt, DevPlanes P, int64_t N, int64_t K, float* w,
                          hipStream_t stream) {
    int wpc = 0;
    switch (fmt) {
    case kQ45: wpc = Traits<kQ45>::WPC; break;
    case kQ65: wpc = Traits<kQ65>::WPC; break;
    case kQ25: wpc = Traits<kQ25>::WPC; break;
    case kBF16: wpc = Traits<kBF16>::WPC; break;
    default: return hipErrorInvalidValue;
    }
    const int64_t total = N * (K / wpc);
    if (total == 0) return hipSuccess;
    const dim3 grid((unsigned)((total + kBlock - 1) / kBlock)), block(kBlock);
    switch (fmt) {
    case kQ45: hipLaunchKernelGGL(dequant_kernel<kQ45>, grid, block, 0, stream, P, N, K, w); break;
    case kQ65: hipLaunchKernelGGL(dequant_kernel<kQ65>, grid, block, 0, stream, P, N, K, w); break;
    case kQ25: hipLaunchKernelGGL(dequant_kernel<kQ25>, grid, block, 0, stream, P, N, K, w); break;
    case kBF16: hipLaunchKernelGGL(dequant_kernel<kBF16>, grid, block, 0, stream, P, N, K, w); break;
    }
    return hipGetLastError();
}

hipError_t launch_unpack_codes(int fmt, DevPlanes P, int64_t N, int64_t K, uint8_t* out,
                               hipStream_t stream) {
    int wpc = 0;
    switch (fmt) {
    case kQ45: wpc = Traits<kQ45>::WPC; break;
    case kQ65: wpc = Traits<kQ65>::WPC; break;
    case kQ25: wpc = Traits<kQ25>::WPC; break;
    default: return hipErrorInvalidValue;
    }
    const int64_t total = N * (K / wpc);
    if (total == 0) return hipSuccess;
    const dim3 grid((unsigned)((total + kBlock - 1) / kBlock)), block(kBlock);
    switch (fmt) {
    case kQ45: hipLaunchKernelGGL(codes_kernel<kQ45>, grid, block, 0, stream, P, N, K, out); break;
    case kQ65: hipLaunchKernelGGL(codes_kernel<kQ65>, grid, block, 0, stream, P, N, K, out); break;
    case kQ25: hipLaunchKernelGGL(codes_kernel<kQ25>, grid, block, 0, stream, P, N, K, out); break;
    }
    return hipGetLastError();
}

// ------------------------------------------------------------------ probes

constexpr int kProbeBlocks = 4096;   // sink must hold this many floats

__global__ __launch_bounds__(kBlock) void probe_read_kernel(const uint4* __restrict__ buf,
                                                            int64_t n16, float* sink) {
    uint32_t acc = 0;
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n16; i += stride) {
        const uint4 v = buf[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    const float s = wave_sum((float)(acc & 1u));
    __shared__ float red[kWavesPerBlock];
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = s;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

__global__ __launch_bounds__(kBlock) void probe_copy_kernel(uint4* __restrict__ dst,
                                                            const uint4* __restrict__ src,
                                                            int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n16; i += stride)
        dst[i] = src[i];
}

hipError_t launch_probe_read(const void* buf, size_t bytes, float* sink, hipStream_t stream) {
    const int64_t n16 = (int64_t)(bytes / 16);
    hipLaunchKernelGGL(probe_read_kernel, dim3(kProbeBlocks), dim3(kBlock), 0, stream,
                       (const uint4*)buf, n16, sink);
    return hipGetLastError();
}

hipError_t launch_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
    const int64_t n16 = (int64_t)(bytes / 16);
    hipLaunchKernelGGL(probe_copy_kernel, dim3(kProbeBlocks), dim3(kBlock), 0, stream,
                       (uint4*)dst, (const uint4*)src, n16);
    return hipGetLastError();
}

}  // namespace mbq
