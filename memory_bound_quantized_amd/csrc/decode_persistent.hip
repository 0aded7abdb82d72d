// decode_persistent.hip -- one token through the decoder stack in one launch.
//
// The pages' unbuilt kernel ([one-serial-kernel] "The kernel that was never
// built": the token's work in one kernel, no return to the host between
// steps; [roofline-holds] "Where the time goes": a fixed toll per weight
// kernel, with fusion as the cure).  Weights never depend on activations, so
// the weight stream need not stop at the grid-wide barrier that publishes a
// table's input: each compute wave walks ONE stream of units that runs
// through all tables of the token, and keeps kDD units in flight across
// every barrier ([roofline-holds] "How the breakouts tie out: Little and
// Volkov": bandwidth x latency bytes must stay in flight).
//
// Grid: one workgroup of 16 waves per compute unit, all resident
// (cooperative launch).  Per layer four phases, then the vocabulary:
//   qkv  q|k|v = Wqkv rmsnorm(h, gamma1)
//   o    h' = h + Wo q                  (q stands in for attention's output)
//   gu   m = silu(Wg b) * (Wu b), b = rmsnorm(h', gamma2)   (rows interleaved)
//   dn   h'' = h' + Wdown m
//   lm   logits = Wlm rmsnorm(h, gamma_f)
// Phase p's rows are split into one contiguous block per workgroup (row
// pairs for gu).  A unit is one chunk step of one row (lane l reads chunk
// 64 c + l: a 1 KiB burst per wave, [mountain-runs] section 3); the
// workgroup's units (row-major) are dealt round-robin to its 15 compute
// waves, so at any moment the workgroup reads one contiguous window of the
// table.  Each unit's sum goes to its own LDS slot, and the control wave adds
// a row's chunk steps in order.
//
// Wave 15 is the control wave.  It streams no weights; at each phase
// boundary it applies the finished phase's epilogue (store, residual add or
// silu * up) to the workgroup's rows, writes them through to device-coherent
// memory, waits for those stores only, arrives at the grid barrier, waits for
// every workgroup, and copies the next phase's input vector (and gamma) into
// LDS with direct-to-LDS loads.  The compute waves meanwhile hold their next
// kDD units of weights in flight.  Then all 16 waves stage x (RMSNorm
// included) from LDS into the integer-digit form of formats.h.
//
// Activations that cross workgroups (h after each residual add, q|k|v, m)
// are written once each per token into buffers of their own, with
// device-scope stores, and read with device-scope loads, which the 8 XCDs'
// separate L2 caches cannot serve stale.  The barrier: a workgroup arrives
// on the counter of its group (block % 8), the last of a group on the
// global counter; waiting is a bounded spin, and a spin that gives up sets
// the status word so every wave still reaches the end of the kernel.
#include "device_common.h"
#include "formats.h"
#include "kernels.h"
#include "staging.h"

namespace mbq {

namespace {

constexpr int kPW = 16;                 // waves per workgroup
constexpr int kPT = kPW * kWave;        // threads per workgroup
constexpr int kCW = kPW - 1;            // compute waves; wave kCW is the control wave
constexpr int kDD = 4;                  // units in flight per compute wave (4 measured faster than 5)
constexpr int kD = 4096, kF = 12288;
constexpr int kMaxRowsWG = 1024;        // rows of one phase per workgroup
constexpr uint32_t kSpinLimit = 1u << 22;   // about 0.2 s of 64-cycle sleeps
constexpr int kBarGroups = 8;
constexpr int kBarStride = 32;          // uint32 between counters (128 bytes)

enum Kind : int { kQKV = 0, kO = 1, kGU = 2, kDN = 3, kLM = 4 };

// LDS layout (bytes).  The staged x takes 36 dwords per 32 values (Q45 and
// Q65 alike, staging.h), up to K = 12288.
constexpr int kLdsH = 0;                               // fp32 h being normalised [4096]
constexpr int kLdsX = kLdsH + 4 * kD;                  // fp32 q or m [12288]
constexpr int kLdsG = kLdsX + 4 * kF;                  // fp32 gamma [4096]
constexpr int kLdsS = kLdsG + 4 * kD;                  // staged x
constexpr int kLdsP = kLdsS + (kF / 32) * Stride<kQ65>::DW * 4;   // unit sums [CS][rows]
constexpr int kLdsR = kLdsP + 2 * 4 * kMaxRowsWG;      // block-sum scratch [16]
constexpr int kLdsTotal = kLdsR + 4 * kPW;
static_assert(Stride<kQ45>::DW == Stride<kQ65>::DW, "one staged stride for both formats");

// Raw registers of one unit, in one shape for both formats: a = 16 code
// bytes (Q45 codes, Q65 low bits), qh = Q65 high bits, then the scale bytes
// (Q45: fp16 scale; Q65: two int8 sub-scales) and the Q65 super-scale.
// A Q45 table's high-bit and super-scale planes are zero-size buffer
// resources: those loads return 0 without a memory access, so every unit
// issues the same four loads into the same registers.
struct Raw {
    uint4 a;
    uint2 qh;
    uint32_t sc2, d2;   // the aligned dwords holding the 16-bit scale fields
};
// The 16-bit fields are read as the aligned dword that holds them and picked
// out where they are used (the half is fixed by the lane), so no operation
// on a loaded register sits between the load and its use.
__device__ __forceinline__ Traits<kQ45>::Row as_q45(const Raw& r, int lane) {
    return {r.a, r.sc2 >> (16 * (lane & 1))};
}
__device__ __forceinline__ Traits<kQ65>::Row as_q65(const Raw& r, int lane) {
    return {r.a, r.qh, r.sc2 >> (16 * (lane & 1)), r.d2 >> (16 * ((lane >> 3) & 1))};
}

// What phase p reads and where it goes.
struct PhaseInfo {
    int kind, layer, fmt, N, CS, Q;   // Q: rows that must share a workgroup
    DevPlanes P;
};

// The layer table is written by the host before the launch and only read
// here: reading it through the constant address space lets every access be a
// scalar load, which never waits behind the weight loads in flight.
typedef const DecTable __attribute__((address_space(4)))* CTable;
__device__ __forceinline__ DevPlanes planes_at(const DevPlanes __attribute__((address_space(4)))& q) {
    return DevPlanes{q.p0, q.p1, q.p2, q.p3};
}

struct Ctx {
    CTable t;
    int L, P, nqkv, vocab, G;
    __device__ __forceinline__ static int rows_total(int k, int nqkv, int vocab) {
        return k == kQKV ? nqkv : k == kGU ? 2 * kF : k == kLM ? vocab : kD;
    }
    // This workgroup's rows of a kind of phase, [row_base, row_base + rows):
    // the rows split into G contiguous blocks (row pairs for gate/up).
    __device__ __forceinline__ void rows_of(int k, int& row_base, int& rows) const {
        const int Q = k == kGU ? 2 : 1;
        const int NQ = rows_total(k, nqkv, vocab) / Q;
        const int b = (int)blockIdx.x;
        const int q0 = (int)((uint32_t)(NQ * b) / (uint32_t)G);
        const int q1 = (int)((uint32_t)(NQ * (b + 1)) / (uint32_t)G);
        row_base = Q * q0;
        rows = Q * (q1 - q0);
    }
    __device__ __forceinline__ PhaseInfo info(int p) const {
        PhaseInfo f;
        if (p >= 4 * L) {
            f.kind = kLM;
            f.layer = L;
            f.fmt = t->head.fmt_lm;
            f.N = vocab;
            f.CS = 2;
            f.Q = 1;
            f.P = planes_at(t->head.lm);
            return f;
        }
        f.layer = p >> 2;
        f.kind = p & 3;
        const DecLayer __attribute__((address_space(4)))* ly = t->layers + f.layer;
        f.CS = 2;
        f.Q = 1;
        f.fmt = kQ45;
        if (f.kind == kQKV) {
            f.N = nqkv;
            f.P = planes_at(ly->qkv);
        } else if (f.kind == kO) {
            f.N = kD;
            f.P = planes_at(ly->o);
        } else if (f.kind == kGU) {
            f.N = 2 * kF;
            f.Q = 2;
            f.P = planes_at(ly->gu);
        } else {
            f.N = kD;
            f.CS = 6;
            f.fmt = ly->fmt_dn;
            f.P = planes_at(ly->dn);
        }
        return f;
    }
};

// Device buffers of the token's activations.
struct Bufs {
    float* h_in;        // caller's h: version 0 in, the last version out
    float* hv;          // versions 1 .. 2L, hs floats apart
    float* qkv;         // per layer, qs floats apart
    float* m;           // per layer, ms floats apart
    float* logits;
    int64_t hs, qs, ms;
    __device__ __forceinline__ float* h(int v) const { return v == 0 ? h_in : hv + (int64_t)(v - 1) * hs; }
};

// ---- one compute wave's share of one phase ---------------------------------
// The workgroup's units of a phase (rows x chunk steps, row-major) are dealt
// round-robin: compute wave w takes units w, w + 15, w + 30, ...: U of them,
// the first at row row0 (relative to the workgroup's first row) and chunk
// step cs0.  Upad rounds U up to a multiple of kDD (at least kDD) with units
// that compute nothing, so that the unit stream crosses into the next phase
// with its slots in order: the loads of the next phase's first kDD units are
// issued in the last kDD steps of this one.
struct Span {
    int U, Upad, CS, rows, row_base, row0, cs0;
    BufPlanes B;
    int fmt;
};

__device__ __forceinline__ Span span_of(const Ctx& c, int p, int w) {
    Span s;
    const PhaseInfo f = c.info(p);
    const int k = f.kind;
    s.CS = f.CS;
    s.fmt = f.fmt;
    c.rows_of(k, s.row_base, s.rows);
    const int Uwg = s.rows * f.CS;
    s.U = Uwg > w ? (Uwg - w + kCW - 1) / kCW : 0;
    s.Upad = s.U <= kDD ? kDD : (s.U + kDD - 1) / kDD * kDD;
    s.row0 = f.CS == 6 ? w / 6 : w >> 1;
    s.cs0 = w - s.row0 * f.CS;
    const int K = 2048 * f.CS;
    s.B = f.fmt == kQ65 ? Traits<kQ65>::planes(f.P, f.N, K) : Traits<kQ45>::planes(f.P, f.N, K);
    return s;
}

// Issue the loads of one unit (row relative to the span's base, chunk step
// cs) into r.  A padding unit (real == false) reads outside the table's
// buffer resources, which returns 0 without a memory access; its data is
// never used, and every unit issues the same loads.  Per row a table holds K/2
// code bytes, K/4 high-bit bytes, K/16 scale bytes and K/128 super-scale
// bytes (Q45 and Q65 alike), K = 2048 CS.
__device__ __forceinline__ void load_unit(Raw& r, const Span& s, int row, int cs, bool real) {
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t o3 = (uint32_t)(s.row_base + row) * (uint32_t)(16 * s.CS);
    const uint32_t b = (uint32_t)(cs * kWave + lane);
    // a padding unit reads past every plane (0xF0000000 exceeds any plane's
    // size; the lane offsets are below 2^16, so the sum cannot wrap)
    const uint32_t pad = real ? 0u : 0xF0000000u;
    r.a = bload<uint4, true>(s.B.p0, 16u * b, real ? o3 << 6 : pad);
    r.qh = bload<uint2, true>(s.B.p1, 8u * b, real ? o3 << 5 : pad);
    r.sc2 = bload<uint32_t, true>(s.B.p2, 4u * (b >> 1), real ? o3 << 3 : pad);
    r.d2 = bload<uint32_t, true>(s.B.p3, 4u * (b >> 4), real ? o3 : pad);
}

// The wave's next unit: kCW units on in the workgroup's row-major order.
__device__ __forceinline__ void step(int& row, int& cs, int CS) {
    static_assert(kCW == 15, "strides below are for 15 compute waves");
    cs += CS == 6 ? 3 : 1;           // 15 = 2 * 6 + 3 = 7 * 2 + 1
    row += CS == 6 ? 2 : 7;
    if (cs >= CS) {
        cs -= CS;
        row++;
    }
}

// The first kDD units of a span into the slots.
__device__ __forceinline__ void load_first(Raw (&buf)[kDD], const Span& s) {
    int row = s.row0, cs = s.cs0;
#pragma unroll
    for (int d = 0; d < kDD; d++) {
        load_unit(buf[d], s, row, cs, d < s.U);
        step(row, cs, s.CS);
    }
}

// Where a compute wave is in the current phase.
struct Pos {
    int rc, cc;          // unit being computed (row, chunk step)
    int rl, cl;          // unit being loaded, kDD ahead
};

// Compute unit u of C from slot r; its sum goes to part[cc][row].
__device__ __forceinline__ void compute_unit(const Raw& r, const Span& C, int u, Pos& q,
                                             const uint32_t* xs, float* part) {
    const int lane = threadIdx.x & (kWave - 1);
    if (u < C.U) {
        uint32_t xv[4 * Traits<kQ45>::F4];
        read_x<kQ45>(xs, q.cc * kWave + lane, xv);
        const float v = C.fmt == kQ65 ? Traits<kQ65>::dot(as_q65(r, lane), xv)
                                       : Traits<kQ45>::dot(as_q45(r, lane), xv);
        const float sum = wave_sum_dpp(v);
        if (lane == 0) part[q.cc * C.rows + q.rc] = sum;
        step(q.rc, q.cc, C.CS);
    }
}

// All but the last kDD units of a phase: each slot is refilled from the
// same phase, kDD units ahead.
__device__ __forceinline__ void run_main(Raw (&buf)[kDD], const Span& C, Pos& q,
                                         const uint32_t* xs, float* part) {
    for (int g = 0; g + kDD < C.Upad; g += kDD) {
#pragma unroll
        for (int d = 0; d < kDD; d++) {
            compute_unit(buf[d], C, g + d, q, xs, part);
            load_unit(buf[d], C, q.rl, q.cl, g + d + kDD < C.U);
            step(q.rl, q.cl, C.CS);
        }
    }
}

// The last kDD units of a phase: each slot is refilled with the next phase's
// first units (with padding units after the last phase).
__device__ __forceinline__ void run_tail(Raw (&buf)[kDD], const Span& C, const Span& Nx, bool last,
                                         Pos& q, const uint32_t* xs, float* part) {
    const int g = C.Upad - kDD;
    int rn = Nx.row0, cn = Nx.cs0;
#pragma unroll
    for (int d = 0; d < kDD; d++) {
        compute_unit(buf[d], C, g + d, q, xs, part);
        load_unit(buf[d], Nx, rn, cn, d < Nx.U && !last);
        step(rn, cn, Nx.CS);
    }
}

// ---- workgroup barriers without memory fences ------------------------------
// LDS traffic is ordered by waiting for this wave's LDS operations; nothing
// waits for the weight loads in flight.
__device__ __forceinline__ void wg_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ float block_sum16(float v, float* red) {
    v = wave_sum_dpp(v);
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    if (lane == 0) red[wave] = v;
    wg_barrier();
    float t = red[0];
#pragma unroll
    for (int w = 1; w < kPW; w++) t += red[w];
    wg_barrier();
    return t;
}

// ---- x: fp32 row in LDS -> staged form in LDS (all 1024 threads) ----------
// Each thread stages groups of 8 values (og = tid, tid + 1024, ...), in the
// layout of staging.h; Q45 and Q65 share the digit words and differ only in
// the offset terms of the metadata (one 32-value block times -8, or two
// 16-value blocks times -32), chosen at run time so that one copy of the
// code serves every phase.  With a gamma, x is first replaced by
// gamma * (x * r), r = 1/sqrt(mean(x^2) + eps) ([one-serial-kernel] "One
// thread": the norm as a cooperative reduction).
// Lane exchanges within aligned groups of four lanes by DPP quad
// permutations (no LDS round trip): xor 1 = [1,0,3,2], xor 2 = [2,3,0,1].
template <int CTRL>
__device__ __forceinline__ int quad_swap(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float quad_xor1(float v) {
    return __builtin_bit_cast(float, quad_swap<0xB1>(__builtin_bit_cast(int, v)));
}
__device__ __forceinline__ float quad_xor2(float v) {
    return __builtin_bit_cast(float, quad_swap<0x4E>(__builtin_bit_cast(int, v)));
}

__device__ __forceinline__ void stage_group_rt(const float* v, int og, bool ok, bool q65,
                                               uint32_t* xs) {
    constexpr int DW = Stride<kQ45>::DW;
    const int b = og >> 2, gi = og & 3;
    float amax = 0.f;
#pragma unroll
    for (int k = 0; k < 8; k++) amax = fmaxf(amax, fabsf(v[k]));
    amax = fmaxf(amax, quad_xor1(amax));
    amax = fmaxf(amax, quad_xor2(amax));
    const int e = chunk_exp(amax);
    const float up = pow2f(e);
    int32_t n[8];
#pragma unroll
    for (int k = 0; k < 8; k++) n[k] = round_fixed(v[k], up);
    uint32_t dg[6];
    digit_words(n[0], n[2], n[4], n[6], dg);
    digit_words(n[1], n[3], n[5], n[7], dg + 3);
    int32_t S[3];
#pragma unroll
    for (int p = 0; p < 3; p++) {
        S[p] = p < 2 ? (int32_t)udot4(dg[p], 0x01010101u, udot4(dg[3 + p], 0x01010101u, 0u))
                     : sdot4(dg[2], 0x01010101u, sdot4(dg[5], 0x01010101u, 0));
    }
    int32_t B01[3], B23[3];
#pragma unroll
    for (int p = 0; p < 3; p++) {
        B01[p] = S[p] + quad_swap<0xB1>(S[p]);
        B23[p] = quad_swap<0x4E>(B01[p]);
    }
    if (ok) {
        uint32_t* o = xs + DW * b + 6 * gi;
#pragma unroll
        for (int t = 0; t < 6; t += 2) *(uint2*)(o + t) = make_uint2(dg[t], dg[t + 1]);
        if (gi == 0) {
            uint32_t m[8];
            m[0] = __builtin_bit_cast(uint32_t, pow2f(-e));
#pragma unroll
            for (int p = 0; p < 3; p++) {
                m[1 + p] = q65 ? (uint32_t)(-32 * B01[p]) : (uint32_t)(-8 * (B01[p] + B23[p]));
                m[4 + p] = q65 ? (uint32_t)(-32 * B23[p]) : 0u;
            }
            m[7] = 0u;
            uint32_t* md = xs + DW * b + Traits<kQ45>::META;
            *(uint4*)md = make_uint4(m[0], m[1], m[2], m[3]);
            *(uint4*)(md + 4) = make_uint4(m[4], m[5], m[6], m[7]);
        }
    }
}

__device__ __forceinline__ void stage_lds(const float* raw, int K, const float* gam, float eps,
                                          bool q65, uint32_t* xs, float* red) {
    const int ng = K / 8;
    const int tid = threadIdx.x;
    float inv = 1.f;
    if (gam) {
        float ss = 0.f;
        for (int og = tid; og < ng; og += kPT) {
            const float4 a = *(const float4*)(raw + 8 * og), b = *(const float4*)(raw + 8 * og + 4);
            ss = fmaf(a.x, a.x, ss); ss = fmaf(a.y, a.y, ss); ss = fmaf(a.z, a.z, ss); ss = fmaf(a.w, a.w, ss);
            ss = fmaf(b.x, b.x, ss); ss = fmaf(b.y, b.y, ss); ss = fmaf(b.z, b.z, ss); ss = fmaf(b.w, b.w, ss);
        }
        inv = 1.0f / sqrtf(block_sum16(ss, red) / (float)K + eps);
    }
    // every lane of a wave runs the same rounds (the shuffles need whole waves)
    const int rounds = (ng + kPT - 1) / kPT;
    for (int r = 0; r < rounds; r++) {
        const int og = r * kPT + tid;
        const bool ok = og < ng;
        const int src = ok ? og : 0;
        const float4 a = *(const float4*)(raw + 8 * src), b = *(const float4*)(raw + 8 * src + 4);
        float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        if (gam) {
            const float4 ga = *(const float4*)(gam + 8 * src), gb = *(const float4*)(gam + 8 * src + 4);
            const float g[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
#pragma unroll
            for (int k = 0; k < 8; k++) v[k] = g[k] * (v[k] * inv);
        }
        stage_group_rt(v, og, ok, q65, xs);
    }
}

// ---- control wave: device-coherent stores, barrier, LDS copies -------------
__device__ __forceinline__ void coh_store(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

typedef const void __attribute__((address_space(1)))* gvoid;
typedef void __attribute__((address_space(3)))* lvoid;
// n floats (n % 256 == 0) from global src to LDS dst, 1 KiB per wave
// instruction, straight into LDS.  COH: device-scope loads (sc1).
template <bool COH>
__device__ __forceinline__ void copy_to_lds(const float* src, float* dst, int n) {
    const int lane = threadIdx.x & (kWave - 1);
    for (int i = 0; i < n; i += 256)
        __builtin_amdgcn_global_load_lds((gvoid)(src + i + 4 * lane), (lvoid)(dst + i), 16, 0,
                                         COH ? 16 : 0);
}

// Ordering across the grid without cache maintenance.  Every activation that
// crosses workgroups (h, q|k|v, m) is written with agent-scope atomic stores
// (coh_store) and read with agent-scope loads (copy_to_lds<true>); the
// compiler makes those coherent across the compute dies by writing through
// and reading past each die's L2.  The control wave waits for its own stores
// to complete (s_waitcnt 0) before it arrives, and issues the next phase's
// loads only after the wait has seen every arrival.  Agent-scope release and
// acquire orderings on the counters would add a writeback and an
// invalidation of the die's whole L2 at every boundary: the token took 2.5 ms
// with them against 1.8 ms without, for data that never sits in a
// non-coherent L2 line in the first place.
__device__ __forceinline__ void barrier_arrive(uint32_t* ctr, int G, uint32_t k) {
    if ((threadIdx.x & (kWave - 1)) == 0) {
        const int ng = G < kBarGroups ? G : kBarGroups;
        const int grp = (int)blockIdx.x % ng;
        const uint32_t members = (uint32_t)(G / ng + (grp < G % ng ? 1 : 0));
        const uint32_t old = __hip_atomic_fetch_add(ctr + kBarStride * (1 + grp), 1u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        if (old == members * (k + 1) - 1)
            __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// The wait polls with relaxed loads; the loads of the next phase come after
// it in program order (a compiler barrier keeps them there).  The spin is
// bounded; on timeout it sets bit 0 of err and returns, so every wave still
// ends.
__device__ __forceinline__ void barrier_wait(uint32_t* ctr, uint32_t target, uint32_t* err) {
    if ((threadIdx.x & (kWave - 1)) == 0) {
        uint32_t spins = 0;
        while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
            if (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 1u) break;
            __builtin_amdgcn_s_sleep(1);
            if (++spins > kSpinLimit) {
                __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
        }
    }
    asm volatile("" ::: "memory");
}

struct Lds {
    float* h;
    float* x;
    float* g;
    uint32_t* xs;
    float* part;     // [CS][rows] of the phase being computed
    float* red;
};

// Epilogue of phase f for this workgroup's rows (control wave).  part holds
// one sum per unit, part[cs][row]; a row's chunk steps are added in order.
__device__ __forceinline__ void epilogue(const Ctx& c, const PhaseInfo& f, const Bufs& bf,
                                         const Lds& s) {
    const int lane = threadIdx.x & (kWave - 1);
    int rb, rows;
    c.rows_of(f.kind, rb, rows);
    auto row_sum = [&](int i) {
        float v = s.part[i];
        for (int cs = 1; cs < f.CS; cs++) v += s.part[cs * rows + i];
        return v;
    };
    if (f.kind == kGU) {
        float* m = bf.m + (int64_t)f.layer * bf.ms;
        for (int i = lane; i < rows / 2; i += kWave) {
            const float g = row_sum(2 * i), u = row_sum(2 * i + 1);
            coh_store(m + rb / 2 + i, g / (1.0f + expf(-g)) * u);
        }
    } else {
        for (int i = lane; i < rows; i += kWave) {
            const float v = row_sum(i);
            const int n = rb + i;
            if (f.kind == kQKV) {
                coh_store(bf.qkv + (int64_t)f.layer * bf.qs + n, v);
            } else if (f.kind == kLM) {
                bf.logits[n] = v;
            } else {
                // residual add on the h this layer's norm read (held in LDS)
                const float hn = s.h[n] + v;
                const int ver = 2 * f.layer + (f.kind == kO ? 1 : 2);
                coh_store(bf.h(ver) + n, hn);
                if (f.kind == kDN && f.layer == c.L - 1) bf.h_in[n] = hn;
            }
        }
    }
}

// Input of phase f into LDS (control wave): the fp32 vector, and gamma for
// the norm phases (gamma is issued first; it does not wait for the barrier).
__device__ __forceinline__ void input_gamma(const Ctx& c, const PhaseInfo& f, const Lds& s) {
    if (f.kind == kQKV) copy_to_lds<false>(c.t->layers[f.layer].g1, s.g, kD);
    if (f.kind == kGU) copy_to_lds<false>(c.t->layers[f.layer].g2, s.g, kD);
    if (f.kind == kLM) copy_to_lds<false>(c.t->head.gf, s.g, kD);
}
__device__ __forceinline__ void input_x(const PhaseInfo& f, const Bufs& bf, const Lds& s) {
    if (f.kind == kQKV) copy_to_lds<true>(bf.h(2 * f.layer), s.h, kD);
    if (f.kind == kO) copy_to_lds<true>(bf.qkv + (int64_t)f.layer * bf.qs, s.x, kD);
    if (f.kind == kGU) copy_to_lds<true>(bf.h(2 * f.layer + 1), s.h, kD);
    if (f.kind == kDN) copy_to_lds<true>(bf.m + (int64_t)f.layer * bf.ms, s.x, kF);
    if (f.kind == kLM) copy_to_lds<true>(bf.h(2 * f.layer), s.h, kD);
}

// Stage phase f's x (all waves).
__device__ __forceinline__ void stage_phase(const PhaseInfo& f, float eps, const Lds& s) {
    const bool norm = f.kind == kQKV || f.kind == kGU || f.kind == kLM;
    const float* raw = (f.kind == kO || f.kind == kDN) ? s.x : s.h;
    const int K = f.kind == kDN ? kF : kD;
    stage_lds(raw, K, norm ? s.g : nullptr, eps, f.fmt == kQ65, s.xs, s.red);
}

}  // namespace

__global__ __launch_bounds__(kPT) void decode_persistent_kernel(
    const DecTable* __restrict__ table, DecTable expect, float eps, Bufs bf,
    int nqkv, int vocab, uint32_t* ctr, uint32_t* err, int G) {
    extern __shared__ float4 smem[];
    char* sb = (char*)smem;
    const Lds s{(float*)(sb + kLdsH), (float*)(sb + kLdsX), (float*)(sb + kLdsG),
                (uint32_t*)(sb + kLdsS), (float*)(sb + kLdsP), (float*)(sb + kLdsR)};
    // the layer table in the workspace must be the one prepared for this model
    if (table->magic != expect.magic || table->n_layers != expect.n_layers ||
        table->tag != expect.tag) {
        if (threadIdx.x == 0 && blockIdx.x == 0) atomicOr(err, 2u);
        return;
    }
    Ctx c;
    c.t = (CTable)table;
    c.L = (int)expect.n_layers;
    c.P = 4 * c.L + (vocab > 0 ? 1 : 0);
    c.nqkv = nqkv;
    c.vocab = vocab;
    c.G = G;
    if (c.P == 0) return;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);

    if (wave == kCW) {
        // ------------------------------------------------ control wave
        const uint32_t per_bar = (uint32_t)(G < kBarGroups ? G : kBarGroups);
        PhaseInfo f = c.info(0);
        input_gamma(c, f, s);
        input_x(f, bf, s);
        __builtin_amdgcn_s_waitcnt(0);
        wg_barrier();
        stage_phase(f, eps, s);
        wg_barrier();
        for (int q = 1; q < c.P; q++) {
            wg_barrier();                                  // phase q-1's partials are in LDS
            const PhaseInfo n = c.info(q);
            input_gamma(c, n, s);                          // independent of the barrier
            epilogue(c, f, bf, s);
            __builtin_amdgcn_s_waitcnt(0);                 // own stores and gamma complete
            barrier_arrive(ctr, G, (uint32_t)(q - 1));
            barrier_wait(ctr, per_bar * (uint32_t)q, err);
            input_x(n, bf, s);
            __builtin_amdgcn_s_waitcnt(0);
            wg_barrier();
            stage_phase(n, eps, s);
            wg_barrier();
            f = n;
        }
        wg_barrier();
        epilogue(c, f, bf, s);
        return;
    }

    // ---------------------------------------------------- compute waves
    Raw buf[kDD];
    load_first(buf, span_of(c, 0, wave));
    wg_barrier();                                          // x of phase 0 in LDS
    stage_phase(c.info(0), eps, s);
    wg_barrier();
    for (int p = 0; p < c.P; p++) {
        if (p > 0) {
            wg_barrier();                                  // B1: partials of p-1 written
            wg_barrier();                                  // B2: x of p in LDS
            stage_phase(c.info(p), eps, s);
            wg_barrier();                                  // B3: staged
        }
        const Span C = span_of(c, p, wave);
        Pos q;
        q.rc = q.rl = C.row0;
        q.cc = q.cl = C.cs0;
#pragma unroll
        for (int d = 0; d < kDD; d++) step(q.rl, q.cl, C.CS);
        run_main(buf, C, q, s.xs, s.part);
        const bool last = p + 1 == c.P;
        run_tail(buf, C, span_of(c, last ? p : p + 1, wave), last, q, s.xs, s.part);
    }
    wg_barrier();                                          // partials of the last phase
}

__global__ void decode_reset_kernel(uint32_t* ctr, uint32_t* err) {
    if (threadIdx.x == 0) {
        *ctr = 0u;
        *err = 0u;
    }
    if (threadIdx.x < kBarGroups) ctr[kBarStride * (1 + threadIdx.x)] = 0u;
}

hipError_t launch_decode_persistent(const DecTable* table, DecTable expect,
                                    float eps, float* h, float* logits, int64_t vocab,
                                    int64_t nqkv, const DecodeBuffers& db, uint32_t* ctr,
                                    uint32_t* err, hipStream_t stream) {
    auto kern = decode_persistent_kernel;
    const size_t lds = kLdsTotal;
    hipError_t e = ensure_lds<decode_persistent_kernel>(lds);
    if (e != hipSuccess) return e;
    int dev = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    int cus = 0, per_cu = 0;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
        return e;
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)kern, kPT, lds)) !=
        hipSuccess)
        return e;
    if (per_cu < 1) return hipErrorInvalidConfiguration;
    int G = cus;
    // every phase's unit sums per workgroup must fit in LDS (CS x rows)
    auto fits = [&](int64_t n, int64_t q, int64_t cs) {
        return cs * q * ((n / q + G - 1) / G) <= 2 * kMaxRowsWG;
    };
    if (!fits(vocab, 1, 2) || !fits(nqkv, 1, 2) || !fits(2 * kF, 2, 2) || !fits(kD, 1, 6))
        return hipErrorInvalidConfiguration;
    Bufs bf{h, db.hv, db.qkv, db.m, logits, db.hs, db.qs, db.ms};
    int nq = (int)nqkv, nv = (int)vocab;
    hipLaunchKernelGGL(decode_reset_kernel, dim3(1), dim3(64), 0, stream, ctr, err);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    void* args[] = {(void*)&table, (void*)&expect, (void*)&eps, (void*)&bf,
                    (void*)&nq, (void*)&nv, (void*)&ctr, (void*)&err, (void*)&G};
    return hipLaunchCooperativeKernel((const void*)kern, dim3(G), dim3(kPT), args, (unsigned)lds,
                                      stream);
}

}  // namespace mbq
