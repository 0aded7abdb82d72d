// exports.hip -- device unpack/dequant exports and the bandwidth probes.
//
// mbq_dequant_f32 / mbq_unpack_codes run the exact in-register unpack the
// GEMV kernels use (formats.h) and write its result out, so the unpack can
// be checked bit for bit against an independent decoder.
//
// The probes measure the ceilings (memory bandwidth and latency, matrix and
// vector issue rates) instead of quoting them.
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
//
// The ceilings the roofline is drawn against, measured on the part instead of
// quoted ([roofline-holds] "The Math" and "How I ran it": a read and an
// in-device copy whose read and write both count; peak loops for the
// arithmetic units; "How the breakouts tie out": the latency that Little's
// law turns into bytes in flight).

constexpr int kProbeBlocks = 4096;   // sink must hold this many floats
constexpr int kProbeU = 8;           // independent 16-byte loads per lane in flight
typedef uint32_t pu4 __attribute__((ext_vector_type(4)));

// Each block walks tiles of kBlock * kProbeU 16-byte words; within a tile,
// load u of thread i is word u * kBlock + i, so every load instruction of a
// wave reads 1 KiB contiguously and a lane keeps kProbeU of them in flight.
__global__ __launch_bounds__(kBlock) void probe_read_kernel(const pu4* __restrict__ buf,
                                                            int64_t n16, float* sink) {
    uint32_t acc = 0;
    constexpr int64_t T = (int64_t)kBlock * kProbeU;
    const int64_t ntile = n16 / T;
    for (int64_t t = blockIdx.x; t < ntile; t += gridDim.x) {
        const pu4* p = buf + t * T + threadIdx.x;
        pu4 v[kProbeU];
#pragma unroll
        for (int u = 0; u < kProbeU; u++) v[u] = __builtin_nontemporal_load(p + u * kBlock);
#pragma unroll
        for (int u = 0; u < kProbeU; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (int64_t i = ntile * T + (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n16;
         i += (int64_t)gridDim.x * kBlock) {
        const pu4 v = buf[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    const float s = wave_sum((float)(acc & 1u));
    __shared__ float red[kWavesPerBlock];
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = s;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

constexpr int kCopyU = 4;

__global__ __launch_bounds__(kBlock) void probe_copy_kernel(pu4* __restrict__ dst,
                                                            const pu4* __restrict__ src,
                                                            int64_t n16) {
    constexpr int64_t T = (int64_t)kBlock * kCopyU;
    const int64_t ntile = n16 / T;
    for (int64_t t = blockIdx.x; t < ntile; t += gridDim.x) {
        const int64_t b = t * T + threadIdx.x;
        pu4 v[kCopyU];
#pragma unroll
        for (int u = 0; u < kCopyU; u++) v[u] = __builtin_nontemporal_load(src + b + u * kBlock);
#pragma unroll
        for (int u = 0; u < kCopyU; u++) __builtin_nontemporal_store(v[u], dst + b + u * kBlock);
    }
    for (int64_t i = ntile * T + (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n16;
         i += (int64_t)gridDim.x * kBlock)
        dst[i] = src[i];
}

// Per-compute-unit streams (one workgroup of 16 waves per unit): workgroup
// b reads `dbytes` of its own region of `distinct` (b * dbytes on) and
// `sbytes` of `shared`, a region every workgroup reads (it stays in L2).
// mode 0: the distinct region only; 1: the shared region only; 2: both, every
// wave interleaving 1 KB of distinct data with its share of shared data;
// 3: both, waves 0-3 on the distinct region and 4-15 on the shared one.
constexpr int kMixThreads = 1024;
__global__ __launch_bounds__(kMixThreads) void probe_mixed_kernel(const pu4* __restrict__ distinct,
                                                                  const pu4* __restrict__ shared,
                                                                  int64_t d16, int64_t s16, int mode,
                                                                  float* __restrict__ sink) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const pu4* db = distinct + (int64_t)blockIdx.x * d16;
    const int64_t dp = d16 / 64, sp = s16 / 64;          // 1 KB pieces
    uint32_t acc = 0;
    auto rd = [&](const pu4* b, int64_t piece) __attribute__((always_inline)) {
        const pu4 v = b[piece * 64 + lane];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    };
    if (mode == 0) {
        for (int64_t p = wave; p < dp; p += 16) rd(db, p);
    } else if (mode == 1) {
        for (int64_t p = wave; p < sp; p += 16) rd(shared, p);
    } else if (mode == 2) {
        const int64_t ratio = dp > 0 ? (sp + dp - 1) / dp : 0;
        for (int64_t p = wave; p < dp; p += 16) {
            rd(db, p);
            for (int64_t r = 0; r < ratio; r++) {
                const int64_t q = p * ratio + r;
                if (q < sp) rd(shared, q);
            }
        }
    } else {
        if (wave < 4) {
            for (int64_t p = wave; p < dp; p += 4) rd(db, p);
        } else {
            for (int64_t p = wave - 4; p < sp; p += 12) rd(shared, p);
        }
    }
    if (acc == 0x9E3779B9u) sink[blockIdx.x] = (float)acc;   // keeps the loads
}

hipError_t launch_probe_mixed(const void* distinct, size_t dbytes, const void* shared, size_t sbytes,
                              int mode, int blocks, float* sink, hipStream_t stream) {
    hipLaunchKernelGGL(probe_mixed_kernel, dim3(blocks), dim3(kMixThreads), 0, stream,
                       (const pu4*)distinct, (const pu4*)shared, (int64_t)(dbytes / 16),
                       (int64_t)(sbytes / 16), mode, sink);
    return hipGetLastError();
}

hipError_t launch_probe_read(const void* buf, size_t bytes, float* sink, hipStream_t stream) {
    const int64_t n16 = (int64_t)(bytes / 16);
    hipLaunchKernelGGL(probe_read_kernel, dim3(kProbeBlocks), dim3(kBlock), 0, stream,
                       (const pu4*)buf, n16, sink);
    return hipGetLastError();
}

hipError_t launch_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
    const int64_t n16 = (int64_t)(bytes / 16);
    hipLaunchKernelGGL(probe_copy_kernel, dim3(kProbeBlocks), dim3(kBlock), 0, stream,
                       (pu4*)dst, (const pu4*)src, n16);
    return hipGetLastError();
}

// Pointer chase: entry i of the chain sits at word 64 i (one entry per 256
// bytes) and holds the next entry, (a i + c) mod n with n a power of two,
// a = 1 mod 4 and c odd: one cycle through all n entries, each hop far from
// the last.  One lane follows it, so each hop is one full memory latency.
constexpr uint32_t kChaseA = 0x9E3779B1u, kChaseC = 0x7F4A7C15u;
constexpr int kChaseStride = 64;   // uint32 words between entries

__global__ __launch_bounds__(kBlock) void chase_init_kernel(uint32_t* __restrict__ buf,
                                                            uint32_t n) {
    const uint32_t mask = n - 1;
    for (uint32_t i = blockIdx.x * kBlock + threadIdx.x; i < n; i += gridDim.x * kBlock)
        buf[(size_t)i * kChaseStride] = (kChaseA * i + kChaseC) & mask;
}

// The chase starts at the entry sink holds (masked into the chain) and leaves
// the entry it reached there, so consecutive launches walk on through the
// cycle instead of revisiting entries a previous launch left in the caches.
__global__ void chase_kernel(const uint32_t* __restrict__ buf, uint32_t n, int64_t hops,
                             uint32_t* sink) {
    uint32_t i = sink[0] & (n - 1);
    for (int64_t h = 0; h < hops; h++) i = __builtin_nontemporal_load(buf + (size_t)i * kChaseStride);
    sink[0] = i;
}

uint32_t chase_entries(size_t bytes) {
    size_t n = bytes / (kChaseStride * 4);
    uint32_t p = 1;
    while ((size_t)p * 2 <= n && p < (1u << 31)) p *= 2;
    return n ? p : 0;
}

hipError_t launch_chase_init(void* buf, size_t bytes, hipStream_t stream) {
    const uint32_t n = chase_entries(bytes);
    hipLaunchKernelGGL(chase_init_kernel, dim3(kProbeBlocks), dim3(kBlock), 0, stream,
                       (uint32_t*)buf, n);
    return hipGetLastError();
}

hipError_t launch_chase(const void* buf, uint32_t n, int64_t hops, uint32_t* sink,
                        hipStream_t stream) {
    hipLaunchKernelGGL(chase_kernel, dim3(1), dim3(1), 0, stream, (const uint32_t*)buf, n, hops, sink);
    return hipGetLastError();
}

// Peak loops: every wave runs kChains independent chains of one instruction
// for `iters` rounds, with no memory traffic inside the loop; the results are
// summed into sink (one float per workgroup) so nothing is dead code.
constexpr int kChains = 8;
constexpr int kPeakBlocks = 2048;   // 8 per compute unit: 8 waves per SIMD
typedef _Float16 ph8 __attribute__((ext_vector_type(8)));
typedef float pf4 __attribute__((ext_vector_type(4)));

// Each chain has its own B operand, so the compiler cannot fold chains
// together or carry one chain's result into another.
template <bool BIG>
__global__ __launch_bounds__(kBlock) void peak_mfma_kernel(int64_t iters, float* sink) {
    const float t = (float)threadIdx.x * 1e-3f;
    ph8 a, b[kChains];
#pragma unroll
    for (int i = 0; i < 8; i++) a[i] = (_Float16)(t + i);
#pragma unroll
    for (int c = 0; c < kChains; c++)
#pragma unroll
        for (int i = 0; i < 8; i++) b[c][i] = (_Float16)(1.0f - t * (i + c));
    typedef float pf16 __attribute__((ext_vector_type(16)));
    float s = 0.f;
    if constexpr (BIG) {
        pf16 acc[kChains];
#pragma unroll
        for (int c = 0; c < kChains; c++)
#pragma unroll
            for (int i = 0; i < 16; i++) acc[c][i] = (float)c;
        for (int64_t r = 0; r < iters; r++) {
#pragma unroll
            for (int c = 0; c < kChains; c++) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b[c], acc[c], 0, 0, 0);
        }
#pragma unroll
        for (int c = 0; c < kChains; c++)
#pragma unroll
            for (int i = 0; i < 16; i++) s += acc[c][i];
    } else {
        // the product kernels' pattern: a pair of instructions from a zero
        // accumulator (the second in place), then a vector add
        pf4 acc[kChains];
        const pf4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < kChains; c++) acc[c] = pf4{0.f, 0.f, 0.f, (float)c};
        for (int64_t r = 0; r < iters; r += 2) {
#pragma unroll
            for (int c = 0; c < kChains; c++) {
                pf4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[c], z, 0, 0, 0);
                d = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[(c + 1) % kChains], d, 0, 0, 0);
                acc[c] += d;
            }
        }
#pragma unroll
        for (int c = 0; c < kChains; c++) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    }
    s = wave_sum(s);
    __shared__ float red[kWavesPerBlock];
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = s;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

__global__ __launch_bounds__(kBlock) void peak_fma_kernel(int64_t iters, float* sink) {
    const float t = (float)threadIdx.x * 1e-7f;
    float acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; c++) acc[c] = t + (float)c;
    const float m = 1.0f - t, d = t * 0.5f;
    for (int64_t r = 0; r < iters; r++) {
#pragma unroll
        for (int c = 0; c < kChains; c++) acc[c] = fmaf(acc[c], m, d);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kChains; c++) s += acc[c];
    s = wave_sum(s);
    __shared__ float red[kWavesPerBlock];
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = s;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

__global__ __launch_bounds__(kBlock) void peak_dot4_kernel(int64_t iters, float* sink) {
    const uint32_t t = threadIdx.x * 0x01010101u;
    uint32_t acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; c++) acc[c] = t + (uint32_t)c;
    const uint32_t a = 0x03050709u ^ t, b = 0x0B0D0F11u;
    for (int64_t r = 0; r < iters; r++) {
#pragma unroll
        for (int c = 0; c < kChains; c++) acc[c] = __builtin_amdgcn_udot4(a, b ^ acc[c], acc[c], false);
    }
    uint32_t s = 0;
#pragma unroll
    for (int c = 0; c < kChains; c++) s ^= acc[c];
    const float f = wave_sum((float)(s & 0xFFu));
    __shared__ float red[kWavesPerBlock];
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = f;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

// kind 0: fp16 matrix instructions 16x16x32 (2 * 16 * 16 * 32 flops each);
// 1: fp32 FMA (2 flops per lane); 2: int8 dot4 (8 ops per lane); 3: fp16
// matrix instructions 32x32x16 (2 * 32 * 32 * 16 flops each).
int64_t peak_ops(int kind, int64_t iters) {
    const int64_t waves = (int64_t)kPeakBlocks * kWavesPerBlock;
    if (kind == 0) iters = (iters + 1) / 2 * 2;    // rounds run in pairs
    const int64_t per = kind == 0 || kind == 3 ? 2 * 16 * 16 * 32 * (kind == 3 ? 2 : 1)
                                               : (kind == 1 ? 2 * kWave : 8 * kWave);
    return waves * iters * kChains * per;
}

hipError_t launch_peak(int kind, int64_t iters, float* sink, hipStream_t stream) {
    switch (kind) {
    case 0: hipLaunchKernelGGL(peak_mfma_kernel<false>, dim3(kPeakBlocks), dim3(kBlock), 0, stream, iters, sink); break;
    case 3: hipLaunchKernelGGL(peak_mfma_kernel<true>, dim3(kPeakBlocks), dim3(kBlock), 0, stream, iters, sink); break;
    case 1: hipLaunchKernelGGL(peak_fma_kernel, dim3(kPeakBlocks), dim3(kBlock), 0, stream, iters, sink); break;
    default: hipLaunchKernelGGL(peak_dot4_kernel, dim3(kPeakBlocks), dim3(kBlock), 0, stream, iters, sink); break;
    }
    return hipGetLastError();
}

}  // namespace mbq
