// attention.hip -- one new token attending over an fp16 KV cache.
//
// With the conversation loaded, every decode token also reads its keys and
// values ([roofline-holds] "Said before the run": 75.5 MB per token at 512
// positions for the 36-layer model, i.e. 2-byte values, 1024 per position and
// layer for each of K and V).  The reading this library takes (plain scaled
// dot-product attention; the pages name no positional encoding): query head h
// reads key/value head h / G (G query heads per key/value head),
//   s_t = q_h . k_t / sqrt(d),  p_t = exp(s_t - max s) / sum exp(s - max s),
//   out_h = sum_t p_t v_t.
// Like the weight stream it is a read of bytes used once, so it is split the
// way long decode attention is split on GPUs with many compute units: the
// positions are cut into chunks, each workgroup owns one key/value head and
// one chunk and leaves (max, sum of exponentials, weighted sum of values)
// for its G query heads, and a second launch combines the chunks.
//
// Layout: lane 16 p + i of a wave reads 16 bytes (dims 8 i .. 8 i + 7) of
// position p of a group of 4, so a load instruction covers 4 positions' 256
// bytes of one head, whole lines.  Scores are kept in base 2: q is scaled by
// log2(e) / sqrt(d) once, and exp2 is taken of score differences.
#include "device_common.h"
#include "kernels.h"

namespace mbq {

namespace {

typedef float af4 __attribute__((ext_vector_type(4)));
typedef uint32_t au4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

// Sum over the 16 lanes of each row (every lane of the row gets it).
__device__ __forceinline__ float row_sum16(float v) {
    v = dpp_add<0xB1, 0xF>(v);    // quad_perm [1,0,3,2]
    v = dpp_add<0x4E, 0xF>(v);    // quad_perm [2,3,0,1]
    v = dpp_add<0x141, 0xF>(v);   // row_half_mirror
    v = dpp_add<0x140, 0xF>(v);   // row_mirror
    return v;
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_max(float v) {
    // lanes of rows outside ROW_MASK keep their own value (old = v)
    const int s = __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v),
                                              CTRL, ROW_MASK, 0xF, false);
    return fmaxf(v, __builtin_bit_cast(float, s));
}

// Maximum over the 64 lanes with DPP row operations (the pattern of
// wave_sum_dpp); the result is wave-uniform (read from lane 63).
__device__ __forceinline__ float wave_max(float v) {
    v = dpp_max<0xB1, 0xF>(v);    // quad_perm [1,0,3,2]
    v = dpp_max<0x4E, 0xF>(v);    // quad_perm [2,3,0,1]
    v = dpp_max<0x141, 0xF>(v);   // row_half_mirror
    v = dpp_max<0x140, 0xF>(v);   // row_mirror
    v = dpp_max<0x142, 0xA>(v);   // row_bcast:15 into rows 1, 3
    v = dpp_max<0x143, 0xC>(v);   // row_bcast:31 into rows 2, 3
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// The 8 halves of a 16-byte load as floats (exact).
__device__ __forceinline__ void halves(au4 w, float* f) {
#pragma unroll
    for (int e = 0; e < 4; e++) {
        f[2 * e] = h2f(w[e]);
        f[2 * e + 1] = h2f(w[e] >> 16);
    }
}

}  // namespace

// Positions per workgroup: T / P rounded to the nearest multiple of 16 (4
// waves x 4 positions), at least 16 and at most 16 groups of 4 per wave
// (kMaxGroups) so that a wave holds all its keys and values in registers.
// P = 16 chunks per head below 1024 positions, where the call is
// latency-bound and each extra chunk record costs the combine step, and P =
// 32 from 1024 on, where more workgroups stream the cache (µs, 32 on 8
// heads, P = 16 against 32: 12.1 against 10.8 at 2048 positions, 9.3
// either way at 1024; at 4096, 16 chunks per head leave half the compute
// units idle: 17.5 against 14.6).  Rounding to the nearest multiple keeps
// 513 positions (512 cached and the new one) at 17 chunks of 32, 8.3 µs,
// where rounding up gave 11 chunks of 48 and 8.7 µs.  MBQ_ATT_CHUNKS
// overrides P (tuning).
constexpr int kMaxGroups = 16;
int attention_chunk(int64_t T, int n_kv) {
    (void)n_kv;
    int64_t P = T >= 1024 ? 32 : 16;
    if (const char* e = tuning_var("MBQ_ATT_CHUNKS")) P = atoll(e) > 0 ? atoll(e) : P;
    int64_t c = (T + P / 2) / P;                  // T / P to the nearest position
    c = (c + 8) / 16 * 16;                        // to the nearest multiple of 16
    const int cmax = 16 * kMaxGroups;
    return (int)(c < 16 ? 16 : (c > cmax ? cmax : c));
}

size_t attention_workspace_bytes(int64_t T, int n_heads, int n_kv) {
    const int64_t nch = (T + attention_chunk(T, n_kv) - 1) / attention_chunk(T, n_kv);
    return (size_t)n_heads * (size_t)nch * kAttRecord * sizeof(float);
}

// 8 fp32 values -> the 16 bytes of fp16 a cache row holds for them (each
// rounded to nearest even; the order `halves` unpacks).
__device__ __forceinline__ au4 to_halves(const float* __restrict__ src) {
    const af4 a = *(const af4*)src, b = *(const af4*)(src + 4);
    const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    au4 w;
#pragma unroll
    for (int e = 0; e < 4; e++)
        w[e] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f[2 * e]) |
               ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f[2 * e + 1]) << 16);
    return w;
}

// Workgroup (kv head, chunk): the chunk's partial record for each of the G
// query heads of the group, at ws[((kv * nch) + chunk) * G + hl] (records of
// kAttRecord floats: m, l, then d values of o; m and l in base 2).  Wave w
// owns the groups of 4 positions w, w + 4, ...: it issues all their key and
// value loads first, so the chunk costs one memory round trip.
// APPEND: position T - 1 is the new one.  Its key and value come from knew
// and vnew (fp32, rounded to fp16 here exactly as the cache stores them),
// and the lanes that own it write that row of the caches (kw, vw, the same
// arrays as kc, vc); what the cache held in that row before is never used.
// NG: groups of 4 positions per wave the kernel is built for (chunks of up
// to 16 NG positions).
template <int G, bool APPEND, int NG>
__global__ __launch_bounds__(kThreads) void attn_partial_kernel(const float* __restrict__ q,
                                                                const uint16_t* kc,
                                                                const uint16_t* vc,
                                                                int64_t T, int64_t ld, int C,
                                                                float qscale, float* __restrict__ ws,
                                                                const float* __restrict__ knew,
                                                                const float* __restrict__ vnew,
                                                                uint16_t* kw, uint16_t* vw) {
    extern __shared__ __attribute__((aligned(16))) float alds[];
    float* sc = alds;                               // [G][C] scores, then weights
    float* red = alds + G * C;                      // [16][G][d] partial outputs
    float* mls = red + 16 * G * kAttD;              // [G][2] max and sum
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int p = lane >> 4, i = lane & 15;
    const int kv = blockIdx.x, chunk = blockIdx.y, nch = gridDim.y;
    const int64_t t0 = (int64_t)chunk * C;
    const int tn = (int)min((int64_t)C, T - t0);    // >= 1
    const int64_t hoff = (int64_t)kv * kAttD + 8 * i;
    // Chunks of up to 64 positions (NG <= 4 groups per wave) load every group
    // (rows past the chunk clamp to its last position), so the loads carry no
    // branch and the scores wait for q and the keys only; with branches the
    // compiler has to wait for every load first.  Same run, µs, 32 on 8
    // heads, unconditional against branching loads: 8.3 against 8.4 at 512
    // positions, and for the append form 8.3 against 8.8 at 512 cached and
    // 8.7 against 9.6 at 600.
    constexpr bool kAll = NG <= 4;

    // q first, then every key, then every value (positions past the chunk
    // repeat its last one and are masked): load completion is counted in
    // issue order, so the scores wait for q and the keys only, and the
    // values keep arriving while they are computed
    float qv[G][8];
#pragma unroll
    for (int h = 0; h < G; h++) {
        const af4* src = (const af4*)(q + (int64_t)(kv * G + h) * kAttD + 8 * i);
        const af4 a = src[0], b = src[1];
        qv[h][0] = a.x; qv[h][1] = a.y; qv[h][2] = a.z; qv[h][3] = a.w;
        qv[h][4] = b.x; qv[h][5] = b.y; qv[h][6] = b.z; qv[h][7] = b.w;
    }
    au4 kr[NG], vr[NG];
    // The new position (APPEND) comes from knew / vnew.  In the general form
    // its lanes branch to them; with kAll they load the cache row like every
    // other lane (in bounds: the caches hold row T - 1; the value is
    // discarded) and the last chunk patches them once every load is issued,
    // so no wait sits between the loads.
    constexpr bool kBranchNew = APPEND && !kAll;
#pragma unroll
    for (int jg = 0; jg < NG; jg++) {
        const int base = 4 * (wave + kWaves * jg);
        if (kAll || base < tn) {                    // the same in every lane of the wave
            const int64_t row = t0 + min(base + p, tn - 1);
            if (kBranchNew && row == T - 1) {       // only in the last chunk's last group
                kr[jg] = to_halves(knew + hoff);
                if (base + p == tn - 1) *(au4*)(kw + row * ld + hoff) = kr[jg];
            } else {
                kr[jg] = *(const au4*)(kc + row * ld + hoff);
            }
        }
    }
#pragma unroll
    for (int jg = 0; jg < NG; jg++) {
        const int base = 4 * (wave + kWaves * jg);
        if (kAll || base < tn) {
            const int64_t row = t0 + min(base + p, tn - 1);
            if (kBranchNew && row == T - 1) {
                vr[jg] = to_halves(vnew + hoff);
                if (base + p == tn - 1) *(au4*)(vw + row * ld + hoff) = vr[jg];
            } else {
                vr[jg] = *(const au4*)(vc + row * ld + hoff);
            }
        }
    }
    if (APPEND && kAll && t0 + tn == T) {           // the last chunk (uniform)
        const au4 kn = to_halves(knew + hoff), vn = to_halves(vnew + hoff);
#pragma unroll
        for (int jg = 0; jg < NG; jg++) {
            const int base = 4 * (wave + kWaves * jg);
            const int64_t row = t0 + min(base + p, tn - 1);
            if (row == T - 1) {
                kr[jg] = kn;
                vr[jg] = vn;
                if (base + p == tn - 1) {           // one lane per 16 bytes writes the row
                    *(au4*)(kw + row * ld + hoff) = kn;
                    *(au4*)(vw + row * ld + hoff) = vn;
                }
            }
        }
    }
#pragma unroll
    for (int h = 0; h < G; h++)
#pragma unroll
        for (int e = 0; e < 8; e++) qv[h][e] *= qscale;

    // scores; lane i < G of each row stores head i's score
#pragma unroll
    for (int jg = 0; jg < NG; jg++) {
        const int base = 4 * (wave + kWaves * jg);
        if (base >= tn) break;
        float k[8];
        halves(kr[jg], k);
#pragma unroll
        for (int h = 0; h < G; h++) {
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < 8; e++) s = fmaf(qv[h][e], k[e], s);
            s = row_sum16(s);
            if (i == h && base + p < tn) sc[h * C + base + p] = s;
        }
    }
    __syncthreads();

    // per head: max, weights exp2(s - max), their sum
    for (int h = wave; h < G; h += kWaves) {
        float m = -INFINITY;
        for (int t = lane; t < tn; t += kWave) m = fmaxf(m, sc[h * C + t]);
        m = wave_max(m);
        float l = 0.f;
        for (int t = lane; t < tn; t += kWave) {
            const float e = exp2f(sc[h * C + t] - m);
            sc[h * C + t] = e;
            l += e;
        }
        l = wave_sum_dpp(l);
        if (lane == 0) {
            mls[2 * h] = m;
            mls[2 * h + 1] = l;
        }
    }
    __syncthreads();

    // weighted values: lane (p, i) sums its positions' dims 8 i .. 8 i + 7
    float acc[G][8];
#pragma unroll
    for (int h = 0; h < G; h++)
#pragma unroll
        for (int e = 0; e < 8; e++) acc[h][e] = 0.f;
#pragma unroll
    for (int jg = 0; jg < NG; jg++) {
        const int base = 4 * (wave + kWaves * jg);
        if (base >= tn) break;
        const bool ok = base + p < tn;
        const int t = min(base + p, tn - 1);
        float v[8];
        halves(vr[jg], v);
#pragma unroll
        for (int h = 0; h < G; h++) {
            const float w = ok ? sc[h * C + t] : 0.f;
#pragma unroll
            for (int e = 0; e < 8; e++) acc[h][e] = fmaf(w, v[e], acc[h][e]);
        }
    }
    // the 16 (wave, p) partials through LDS, added in a fixed order
    const int slot = wave * 4 + p;
#pragma unroll
    for (int h = 0; h < G; h++) {
        af4* dst = (af4*)(red + (slot * G + h) * kAttD + 8 * i);
        dst[0] = af4{acc[h][0], acc[h][1], acc[h][2], acc[h][3]};
        dst[1] = af4{acc[h][4], acc[h][5], acc[h][6], acc[h][7]};
    }
    __syncthreads();
    float* rec = ws + ((int64_t)(kv * nch + chunk) * G) * kAttRecord;
    for (int o = tid; o < G * kAttD; o += kThreads) {
        const int h = o / kAttD, dd = o % kAttD;
        float s = 0.f;
        for (int r = 0; r < 16; r++) s += red[(r * G + h) * kAttD + dd];
        rec[h * kAttRecord + 2 + dd] = s;
    }
    if (tid < G) {
        rec[tid * kAttRecord] = mls[2 * tid];
        rec[tid * kAttRecord + 1] = mls[2 * tid + 1];
    }
}

// One workgroup per query head, thread = dimension: the chunks' records merged
// in blocks of 128 chunks.  Per block every load goes out at once: thread t
// reads chunk t's maximum and sum, and every thread its dimension of the
// block's value sums.  The block's maximum then updates the running one
// (the sums so far rescaled by 2^(old - new), base 2), thread t leaves chunk
// t's factor 2^(m_t - max) in LDS, and each thread adds its dimension in
// chunk order.  One memory round trip per 128 chunks.
__global__ __launch_bounds__(kAttD) void attn_combine_kernel(const float* __restrict__ ws, int G,
                                                             int nch, float* __restrict__ out) {
    constexpr int NT = kAttD;
    __shared__ float fs[NT];
    __shared__ float red[NT / kWave];
    // Workgroups are dealt to the dies (XCDs) in turn, each with its own L2,
    // and the partial launch's workgroup (kv, chunk) is number kv + n_kv
    // chunk: with n_kv a multiple of 8, every record of head group kv was
    // written on die kv % 8.  Workgroup b takes the query head whose records
    // sit on its own die, b % n_kv's group (same run, µs: 8.31 -> 8.17 at
    // 512 positions, 9.17 -> 9.00 at 1024, 13.32 -> 13.12 at 4096).
    const int n_kv = gridDim.x / G;
    const int h = (blockIdx.x % n_kv) * G + blockIdx.x / n_kv;
    const int t = threadIdx.x, dd = t;
    const int kv = h / G, hl = h % G;
    const float* r0 = ws + ((int64_t)kv * nch * G + hl) * kAttRecord;
    const int64_t stride = (int64_t)G * kAttRecord;

    float Mrun = -INFINITY, L = 0.f, acc = 0.f;
    for (int cb = 0; cb < nch; cb += NT) {
        const int n = min(NT, nch - cb);
        constexpr int BU = 16;                         // loads issued in guarded groups of 16
        float o[NT];
#pragma unroll
        for (int u0 = 0; u0 < NT; u0 += BU) {
            if (u0 < n) {                              // the same in the whole workgroup
#pragma unroll
                for (int u = u0; u < u0 + BU; u++) o[u] = u < n ? r0[(cb + u) * stride + 2 + dd] : 0.f;
            }
        }
        const bool mine = t < n;
        const float* rt = r0 + (mine ? cb + t : cb) * stride;
        const float mt = mine ? rt[0] : -INFINITY;
        const float lt = rt[1];
        float mb = wave_max(mt);
        if ((t & (kWave - 1)) == 0) red[t / kWave] = mb;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < NT / kWave; w++) mb = fmaxf(mb, red[w]);
        const float Mnew = fmaxf(Mrun, mb);
        const float scale = exp2f(Mrun - Mnew);        // 0 on the first block
        const float f = mine ? exp2f(mt - Mnew) : 0.f;
        L = fmaf(L, scale, mine ? lt * f : 0.f);
        acc *= scale;
        Mrun = Mnew;
        fs[t] = f;
        __syncthreads();
#pragma unroll
        for (int u0 = 0; u0 < NT; u0 += BU) {
            if (u0 < n) {
#pragma unroll
                for (int u = u0; u < u0 + BU; u++) acc = fmaf(o[u], fs[u], acc);
            }
        }
        __syncthreads();                               // fs and red are rewritten next
    }
    L = wave_sum_dpp(L);
    if ((t & (kWave - 1)) == 0) red[t / kWave] = L;
    __syncthreads();
    L = red[0];
#pragma unroll
    for (int w = 1; w < NT / kWave; w++) L += red[w];
    out[(int64_t)h * kAttD + dd] = acc / L;
}

template <bool APPEND>
static hipError_t launch_attention(const float* q, const uint16_t* kc, const uint16_t* vc, int64_t T,
                                   int64_t ld, int n_heads, int n_kv, float* out, float* ws,
                                   const float* knew, const float* vnew, uint16_t* kw, uint16_t* vw,
                                   hipStream_t stream) {
    const int G = n_heads / n_kv;
    const int C = attention_chunk(T, n_kv);
    const int nch = (int)((T + C - 1) / C);
    const float qscale = (float)(1.4426950408889634 / 11.313708498984761);   // log2(e) / sqrt(128)
    const size_t lds = ((size_t)G * C + 16 * (size_t)G * kAttD + 2 * (size_t)G) * sizeof(float);
    const dim3 grid((unsigned)n_kv, (unsigned)nch);
    switch (G) {
#define MBQ_ATT_CASE(g)                                                                              \
    case g:                                                                                          \
        if (C <= 32) {                                                                               \
            if (hipError_t e = ensure_lds<attn_partial_kernel<g, APPEND, 2>>(lds)) return e;         \
            hipLaunchKernelGGL((attn_partial_kernel<g, APPEND, 2>), grid, dim3(kThreads), lds,       \
                               stream, q, kc, vc, T, ld, C, qscale, ws, knew, vnew, kw, vw);        \
        } else if (C <= 64) {                                                                        \
            if (hipError_t e = ensure_lds<attn_partial_kernel<g, APPEND, 4>>(lds)) return e;         \
            hipLaunchKernelGGL((attn_partial_kernel<g, APPEND, 4>), grid, dim3(kThreads), lds,       \
                               stream, q, kc, vc, T, ld, C, qscale, ws, knew, vnew, kw, vw);        \
        } else {                                                                                     \
            if (hipError_t e = ensure_lds<attn_partial_kernel<g, APPEND, kMaxGroups>>(lds)) return e; \
            hipLaunchKernelGGL((attn_partial_kernel<g, APPEND, kMaxGroups>), grid, dim3(kThreads),   \
                               lds, stream, q, kc, vc, T, ld, C, qscale, ws, knew, vnew, kw, vw);   \
        }                                                                                            \
        break;
        MBQ_ATT_CASE(1)
        MBQ_ATT_CASE(2)
        MBQ_ATT_CASE(4)
        MBQ_ATT_CASE(8)
#undef MBQ_ATT_CASE
    default: return hipErrorInvalidValue;
    }
    if (hipError_t e = hipGetLastError()) return e;
    hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)n_heads), dim3(kAttD), 0, stream, ws, G,
                       nch, out);
    return hipGetLastError();
}

hipError_t launch_attention_decode(const float* q, const uint16_t* kc, const uint16_t* vc, int64_t T,
                                   int64_t ld, int n_heads, int n_kv, float* out, float* ws,
                                   hipStream_t stream) {
    return launch_attention<false>(q, kc, vc, T, ld, n_heads, n_kv, out, ws, nullptr, nullptr,
                                   nullptr, nullptr, stream);
}

// T cached positions plus the new one (T + 1 in all): the partial launch
// takes the new key and value from knew / vnew and writes them to row T.
hipError_t launch_attention_append(const float* q, const float* knew, const float* vnew,
                                   uint16_t* kc, uint16_t* vc, int64_t T, int64_t ld, int n_heads,
                                   int n_kv, float* out, float* ws, hipStream_t stream) {
    return launch_attention<true>(q, kc, vc, T + 1, ld, n_heads, n_kv, out, ws, knew, vnew, kc, vc,
                                  stream);
}

}  // namespace mbq
