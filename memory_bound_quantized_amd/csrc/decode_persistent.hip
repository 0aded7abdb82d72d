// decode_persistent.hip -- one token through the decoder stack in one launch.
//
// The pages' unbuilt kernel ([one-serial-kernel] "The kernel that was never
// built": one kernel doing the token's work without returning to the host
// between steps; [roofline-holds] "Where the time goes": a fixed toll per
// weight kernel, and fusion as its cure).  Weights never depend on
// activations, so each wave issues the loads of its next table before it
// waits for the grid-wide barrier that publishes that table's input: the
// barrier's latency, the x staging and the norm overlap with the weight
// stream instead of adding to it.
//
// Grid: every workgroup resident at once (cooperative launch), a few per
// compute unit.  Per layer four phases separated by grid barriers:
//   P1  a = rmsnorm(h, gamma1) staged in each workgroup; q|k|v = Wqkv a
//   P2  q staged; h += Wo q
//   P3  b = rmsnorm(h, gamma2) staged; m = silu(Wg b) * (Wu b) (gate/up rows
//       interleaved, so one wave computes both rows of an output)
//   P4  m staged; h += Wdown m
// then logits = Wlm rmsnorm(h, gamma_f).  Each phase splits its table's rows
// over the workgroups in pairs; inside a workgroup the 4 waves take pairs in
// turn.  Every wave streams its rows as in the M = 1 kernel (gemv_m1.hip):
// lane l takes chunk 64 c + l, codes unpacked in registers, integer-digit
// dots against the staged x in LDS, a DPP reduction per row.
//
// Barrier: a monotone counter in the caller's workspace.  The activations
// that cross workgroups are written and read with device-coherent accesses,
// so arriving is: wait for one's own writes to complete, meet the workgroup,
// add 1; waiting is a bounded spin on the counter.  A spin that exceeds its
// bound sets the error word and gives up, so every wave always reaches the
// end of the kernel.
#include "device_common.h"
#include "formats.h"
#include "kernels.h"
#include "staging.h"

namespace mbq {

namespace {

template <int V>
struct ICd {
    static constexpr int value = V;
};
template <int B, int E, class F>
__device__ __forceinline__ void sfor(F&& f) {
    if constexpr (B < E) {
        f(ICd<B>{});
        sfor<B + 1, E>(f);
    }
}

constexpr int kRows = 2;                 // rows per wave step (a gate/up pair)
constexpr uint32_t kSpinLimit = 1u << 22;   // about 0.2 s of 128-cycle sleeps

template <int FMT, int R>
struct PSlot {
    typename Traits<FMT>::Row row[R];
};

// ---- device-coherent activations -------------------------------------------
// h, q and the gated activations cross workgroups (and the 8 XCDs' separate
// L2 caches).  They are written and read with agent-scope atomic accesses,
// which bypass the non-coherent cache levels, so a barrier needs no cache
// write-back or invalidation: only that the writes have completed.
__device__ __forceinline__ float coh_load(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void coh_store(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint4 coh_load16(const float* p) {
    const uint64_t* q = (const uint64_t*)p;
    const uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return make_uint4((uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32));
}

// ---- grid barrier ---------------------------------------------------------
// Two levels: workgroup b arrives on the counter of group b % kBarGroups,
// and the last arrival of each group adds 1 to the global counter, which the
// workgroups wait on.  Atomics on one address are serialized (about 15 ns
// each on MI355X), so one counter for 512 workgroups costs 7.8 us per
// barrier; eight groups cost 2.6 us.  Counters sit 128 bytes apart.
constexpr int kBarGroups = 8;
constexpr int kBarStride = 32;           // uint32 between counters

// Arrive: every thread waits until its own memory operations have completed
// (so its coherent stores are visible device-wide), the workgroup meets, and
// thread 0 arrives.  k = the workgroup's earlier arrivals, G = grid size.
__device__ __forceinline__ void barrier_arrive(uint32_t* ctr, int G, uint32_t k) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __syncthreads();
    if (threadIdx.x == 0) {
        const int ng = G < kBarGroups ? G : kBarGroups;
        const int grp = (int)blockIdx.x % ng;
        const uint32_t members = (uint32_t)(G / ng + (grp < G % ng ? 1 : 0));
        const uint32_t old = __hip_atomic_fetch_add(ctr + kBarStride * (1 + grp), 1u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        if (old == members * (k + 1) - 1)
            __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Wait: thread 0 spins until the global counter reaches target (bounded).
// Once any wait has given up (err bit 0), every later wait returns at once,
// so a broken barrier costs one spin bound, not one per barrier.
__device__ __forceinline__ void barrier_wait(uint32_t* ctr, uint32_t target, uint32_t* err) {
    if (threadIdx.x == 0) {
        uint32_t spins = 0;
        while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
            if (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 1u) break;
            __builtin_amdgcn_s_sleep(1);
            if (++spins > kSpinLimit) {
                atomicOr(err, 1u);
                break;
            }
        }
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __syncthreads();
}

// ---- x into LDS: fp32 row of KS values, optionally RMSNorm-ed -------------
// x is read with coherent loads (it was written by other workgroups).
template <int FMT, int KS, bool NORM>
__device__ __forceinline__ void stage_row(const float* x, const float* gamma, float eps,
                                          uint32_t* xs, float* red) {
    using XP = XPieces<FMT, false>;
    constexpr int NX = KS / 4 / kBlock;
    constexpr int NP = KS / 4;
    uint4 xr[NX], gr[NORM ? NX : 1];
#pragma unroll
    for (int i = 0; i < NX; i++) xr[i] = coh_load16(x + 4 * XP::index(i));
    if constexpr (NORM) {
#pragma unroll
        for (int i = 0; i < NX; i++) gr[i] = XP::load((const uint4*)gamma, i, NP);
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < NX; i++) {
            const float4 v = __builtin_bit_cast(float4, xr[i]);
            ss = fmaf(v.x, v.x, ss);
            ss = fmaf(v.y, v.y, ss);
            ss = fmaf(v.z, v.z, ss);
            ss = fmaf(v.w, v.w, ss);
        }
        const float inv = 1.0f / sqrtf(block_sum(ss, red) / (float)KS + eps);
#pragma unroll
        for (int i = 0; i < NX; i++) {
            const float4 v = __builtin_bit_cast(float4, xr[i]);
            const float4 g = __builtin_bit_cast(float4, gr[i]);
            xr[i] = __builtin_bit_cast(uint4, make_float4(g.x * (v.x * inv), g.y * (v.y * inv),
                                                          g.z * (v.z * inv), g.w * (v.w * inv)));
        }
    }
    XP::template store<NX, true>(xr, 0, NP, xs);
    __syncthreads();
}

// ---- one wave's share of one table ----------------------------------------
// Row pairs of the table are split over the workgroups; pair p of this
// workgroup's range goes to wave p % 4.  A unit is one chunk step of the
// wave's current pair; units are pipelined DD deep.
template <int FMT, int CS>
struct Stream {
    using T = Traits<FMT>;
    static constexpr int K = 64 * CS * T::WPC;
    static constexpr int DD = 4;         // units in flight per wave
    PSlot<FMT, kRows> buf[DD];
    BufPlanes B;
    int64_t N, pair0;   // first pair of this wave
    int np, U;          // pairs of this wave, units

    __device__ __forceinline__ void setup(DevPlanes P_, int64_t N_, int G) {
        B = T::planes(P_, N_, K);
        N = N_;
        const int64_t pairs = N / kRows;
        const int64_t b0 = pairs * blockIdx.x / G, b1 = pairs * (blockIdx.x + 1) / G;
        const int wave = threadIdx.x / kWave;
        const int64_t cnt = b1 - b0;
        np = cnt > wave ? (int)((cnt - wave + kWavesPerBlock - 1) / kWavesPerBlock) : 0;
        pair0 = b0 + wave;
        U = np * CS;
    }
    __device__ __forceinline__ void load(PSlot<FMT, kRows>& s, int u) {
        const int lane = threadIdx.x & (kWave - 1);
        const int uu = U == 0 ? 0 : (u < U ? u : U - 1);
        const int pi = uu / CS, c = uu - pi * CS;
        const int64_t pr = pair0 + (int64_t)pi * kWavesPerBlock;
#pragma unroll
        for (int r = 0; r < kRows; r++) {
            int64_t n = pr * kRows + r;
            n = n < N ? n : N - 1;
            T::load(s.row[r], B, T::row_off(n, K), c * kWave + lane);
        }
    }
    __device__ __forceinline__ void prefetch() {
#pragma unroll
        for (int d = 0; d < DD; d++) load(buf[d], d);
    }
    // EPI: store(row pair index, sum of row 0, sum of row 1), called by every lane
    template <class Epi>
    __device__ __forceinline__ void run(const uint32_t* xs, Epi&& epi) {
        const int lane = threadIdx.x & (kWave - 1);
        float acc[kRows] = {0.f, 0.f};
        for (int u0 = 0; u0 < U; u0 += DD) {
            sfor<0, DD>([&](auto dc) {
                constexpr int d = decltype(dc)::value;
                const int u = u0 + d;
                if (u < U) {
                    const int pi = u / CS, c = u - pi * CS;
                    uint32_t xv[4 * T::F4];
                    read_x<FMT>(xs, c * kWave + lane, xv);
#pragma unroll
                    for (int r = 0; r < kRows; r++) acc[r] += T::dot(buf[d].row[r], xv);
                    if (c == CS - 1) {
                        const float s0 = wave_sum_dpp(acc[0]), s1 = wave_sum_dpp(acc[1]);
                        epi(pair0 + (int64_t)pi * kWavesPerBlock, s0, s1);
                        acc[0] = acc[1] = 0.f;
                    }
                    load(buf[d], u + DD);
                }
            });
        }
    }
};

}  // namespace

template <int FMT_LM>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(1, 1))) void decode_persistent_kernel(
    const DecTable* __restrict__ table, DecTable expect, DecHead head, float eps, float* h,
    float* logits, int64_t vocab, int64_t nqkv, float* qkv, float* mbuf, uint32_t* ctr,
    uint32_t* err, int G) {
    extern __shared__ float4 smem[];
    uint32_t* xs = (uint32_t*)smem;
    __shared__ float red[kWavesPerBlock];
    const int lane = threadIdx.x & (kWave - 1);
    constexpr int D = 4096, F = 12288;
    // the layer table in the workspace must be the one prepared for this model
    if (table->magic != expect.magic || table->n_layers != expect.n_layers ||
        table->tag != expect.tag) {
        if (threadIdx.x == 0 && blockIdx.x == 0) atomicOr(err, 2u);
        return;
    }
    const int n_layers = (int)expect.n_layers;
    const DecLayer* layers = table->layers;
    uint32_t target = 0;                 // global counter after the barriers so far
    uint32_t nbar = 0;                   // this workgroup's arrivals so far
    const uint32_t per_bar = (uint32_t)(G < kBarGroups ? G : kBarGroups);

    for (int l = 0; l < n_layers; l++) {
        const DecLayer L = layers[l];
        // P1: q|k|v = Wqkv rmsnorm(h, gamma1)
        {
            Stream<kQ45, 2> st;
            st.setup(L.qkv, nqkv, G);
            st.prefetch();
            if (l > 0) barrier_wait(ctr, target, err);
            stage_row<kQ45, D, true>(h, L.g1, eps, xs, red);
            st.run(xs, [&](int64_t p, float s0, float s1) {
                if (lane == 0) coh_store(qkv + 2 * p, s0);
                if (lane == 1) coh_store(qkv + 2 * p + 1, s1);
            });
            barrier_arrive(ctr, G, nbar++);
            target += per_bar;
        }
        // P2: h += Wo q
        {
            Stream<kQ45, 2> st;
            st.setup(L.o, D, G);
            st.prefetch();
            barrier_wait(ctr, target, err);
            stage_row<kQ45, D, false>(qkv, nullptr, 0.f, xs, red);
            st.run(xs, [&](int64_t p, float s0, float s1) {
                if (lane == 0) coh_store(h + 2 * p, coh_load(h + 2 * p) + s0);
                if (lane == 1) coh_store(h + 2 * p + 1, coh_load(h + 2 * p + 1) + s1);
            });
            barrier_arrive(ctr, G, nbar++);
            target += per_bar;
        }
        // P3: m = silu(Wg b) * (Wu b), b = rmsnorm(h, gamma2)
        {
            Stream<kQ45, 2> st;
            st.setup(L.gu, 2 * F, G);
            st.prefetch();
            barrier_wait(ctr, target, err);
            stage_row<kQ45, D, true>(h, L.g2, eps, xs, red);
            st.run(xs, [&](int64_t p, float g, float u) {
                if (lane == 0) coh_store(mbuf + p, g / (1.0f + expf(-g)) * u);
            });
            barrier_arrive(ctr, G, nbar++);
            target += per_bar;
        }
        // P4: h += Wdown m
        {
            auto down = [&](auto fc) {
                constexpr int FMT = decltype(fc)::value;
                Stream<FMT, 6> st;
                st.setup(L.dn, D, G);
                st.prefetch();
                barrier_wait(ctr, target, err);
                stage_row<FMT, F, false>(mbuf, nullptr, 0.f, xs, red);
                st.run(xs, [&](int64_t p, float s0, float s1) {
                    if (lane == 0) coh_store(h + 2 * p, coh_load(h + 2 * p) + s0);
                    if (lane == 1) coh_store(h + 2 * p + 1, coh_load(h + 2 * p + 1) + s1);
                });
            };
            if (L.fmt_dn == kQ65)
                down(ICd<kQ65>{});
            else
                down(ICd<kQ45>{});
            barrier_arrive(ctr, G, nbar++);
            target += per_bar;
        }
    }
    // logits = Wlm rmsnorm(h, gamma_f)
    if (vocab > 0) {
        Stream<FMT_LM, 2> st;
        st.setup(head.lm, vocab, G);
        st.prefetch();
        if (n_layers > 0) barrier_wait(ctr, target, err);
        stage_row<FMT_LM, D, true>(h, head.gf, eps, xs, red);
        st.run(xs, [&](int64_t p, float s0, float s1) {
            if (lane == 0) logits[2 * p] = s0;
            if (lane == 1) logits[2 * p + 1] = s1;
        });
    }
}

__global__ void decode_reset_kernel(uint32_t* ctr, uint32_t* err) {
    if (threadIdx.x == 0) {
        *ctr = 0u;
        *err = 0u;
    }
    if (threadIdx.x < kBarGroups) ctr[kBarStride * (1 + threadIdx.x)] = 0u;
}

template <int FMT_LM>
static hipError_t launch_persistent_lm(const DecTable* table, DecTable expect, DecHead head,
                                       float eps, float* h, float* logits, int64_t vocab,
                                       int64_t nqkv, float* qkv, float* mbuf, uint32_t* ctr,
                                       uint32_t* err, hipStream_t stream) {
    auto kern = decode_persistent_kernel<FMT_LM>;
    const size_t lds = (size_t)(12288 / 32) * Stride<kQ65>::DW * 4;   // K = 12288 staged
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    int cus = 0, per_cu = 0;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
        return e;
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)kern, kBlock, lds)) !=
        hipSuccess)
        return e;
    if (per_cu < 1) return hipErrorInvalidConfiguration;
    const int per = per_cu < 2 ? per_cu : 2;
    int G = cus * per;
    hipLaunchKernelGGL(decode_reset_kernel, dim3(1), dim3(64), 0, stream, ctr, err);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    void* args[] = {(void*)&table, (void*)&expect, (void*)&head, (void*)&eps, (void*)&h,
                    (void*)&logits, (void*)&vocab, (void*)&nqkv, (void*)&qkv, (void*)&mbuf,
                    (void*)&ctr, (void*)&err, (void*)&G};
    return hipLaunchCooperativeKernel((const void*)kern, dim3(G), dim3(kBlock), args, (unsigned)lds,
                                      stream);
}

hipError_t launch_decode_persistent(const DecTable* table, DecTable expect, DecHead head,
                                    float eps, float* h, float* logits, int64_t vocab,
                                    int64_t nqkv, float* qkv, float* mbuf, uint32_t* ctr,
                                    uint32_t* err, hipStream_t stream) {
    if (head.fmt_lm == kQ65)
        return launch_persistent_lm<kQ65>(table, expect, head, eps, h, logits, vocab, nqkv, qkv,
                                          mbuf, ctr, err, stream);
    return launch_persistent_lm<kQ45>(table, expect, head, eps, h, logits, vocab, nqkv, qkv, mbuf,
                                      ctr, err, stream);
}

}  // namespace mbq
