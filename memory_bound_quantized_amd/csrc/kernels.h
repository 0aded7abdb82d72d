// kernels.h -- internal launchers of libmbq (not part of the C ABI).
// Every launcher enqueues on `stream` and returns hipGetLastError() after the
// launch.  Arguments have been validated by the C-ABI layer (abi.cpp).
#pragma once
#include <atomic>
#include <cstdlib>

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mbq {

enum Fmt : int { kBF16 = 0, kQ45 = 1, kQ65 = 2, kQ25 = 3 };

// Device planes of one weight matrix (see mbq.h for the layouts).
struct DevPlanes {
    const uint8_t* p0;  // codes
    const uint8_t* p1;  // codes_hi
    const uint8_t* p2;  // scales
    const uint8_t* p3;  // super_scales
};

// Largest K the GEMV kernels stage in LDS (x takes 4.5 bytes per value for the
// quantized formats, 6 for BF16, within the 160 KiB of LDS per workgroup).
constexpr int64_t kMaxK = 32768;
constexpr int64_t kMaxKBF16 = 16384;

// Geometry of the M = 1 GEMV: output rows per wave (4 waves per workgroup).
struct GemvGeom {
    int rows_per_wave;   // 1, 2 or 4
    int groups;          // row groups per wave (K = 4096-class tables; 1 otherwise)
};

// pairs: the silu product's gate/up rows; norm: the RMSNorm prologue.
GemvGeom gemv_m1_default_geom(int fmt, int64_t N, int64_t K, bool pairs = false,
                              bool norm = false);

// Geometry overrides for tuning sweeps (MBQ_GEMV_*, MBQ_SMALLM_*, MBQ_MFMA_*)
// are read at each call only when MBQ_TUNING is set when the library first
// asks; otherwise no environment variable is read.
inline bool tuning_env() {
    static const bool on = getenv("MBQ_TUNING") != nullptr;
    return on;
}
inline const char* tuning_var(const char* name) { return tuning_env() ? getenv(name) : nullptr; }

// Dynamic LDS above 64 KB needs the kernel's attribute raised first; each
// kernel remembers the largest size it was given, so the call is made only
// when a launch needs more than any before it.
template <auto KERN>
hipError_t ensure_lds(size_t lds) {
    static std::atomic<size_t> have{65536};
    if (lds <= have.load(std::memory_order_relaxed)) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute((const void*)KERN,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e == hipSuccess) {
        size_t h = have.load(std::memory_order_relaxed);
        while (h < lds && !have.compare_exchange_weak(h, lds, std::memory_order_relaxed)) {
        }
    }
    return e;
}

// y[n] (+)= W[row(n)] . x for n < N_out.  If gidx != nullptr the output row
// n maps to weight row gidx[n / rpe] * rpe + n % rpe (gathered experts).
// x is fp32 [K], or x staged for fmt (staging.h) when x_staged.
// n_weight_rows: rows of the weight table when it differs from N_out (a
// gather over stacked experts); 0 means N_out.
hipError_t launch_gemv_m1(int fmt, DevPlanes P, int64_t N_out, int64_t K, const void* x,
                          bool x_staged, float* y, int accumulate, const int32_t* gidx,
                          int64_t rpe, GemvGeom geom, hipStream_t stream,
                          int64_t n_weight_rows = 0);

// Fused M = 1 product on fp32 x (Q45/Q65 with K = 4096 or 12288 only, see
// gemv_fused_supported): y = W . rmsnorm(x; gamma, eps) when gamma != nullptr,
// else W . x; silu: W's rows 2i, 2i+1 are gate and up rows and
// y[i] = silu(gate . x) * (up . x) for i < N / 2 (accumulate must be 0).
bool gemv_fused_supported(int fmt, int64_t K);
hipError_t launch_gemv_fused(int fmt, DevPlanes P, int64_t N, int64_t K, const float* x,
                             const float* gamma, float eps, bool silu, float* y, int accumulate,
                             GemvGeom geom, hipStream_t stream);

// Staged x for fmt (staging.h) of M rows of fp32 x: xq[m] = stage(x[m][0:K]),
// rows of xq packed back to back (4*K bytes each).
hipError_t launch_stage_x(int fmt, const float* x, int64_t M, int64_t ldx, int64_t K, void* xq,
                          hipStream_t stream);

// One row: y = RMSNorm(x) (skipped if y == nullptr) and xq = stage(y) for fmt.
hipError_t launch_rmsnorm_xq(const float* x, const float* gamma, float eps, int64_t n, float* y,
                             int fmt, void* xq, hipStream_t stream);

// xq = stage(silu(g) * u) for fmt; n values.
hipError_t launch_silu_mul_xq(const float* g, const float* u, int64_t n, int fmt, void* xq,
                              hipStream_t stream);

// Y[m][n] (+)= W[n] . X[m] for 2 <= M <= 8 (vector units).  X is fp32
// [M][ldx], or staged for fmt (M rows of K) when x_staged.  All M tokens are
// staged in LDS: gemv_smallm_fits tells whether they fit.  Geometry: 1 or 2
// rows per wave, row groups per 16-wave workgroup (gemv_smallm_geom_ok).
bool gemv_smallm_fits(int fmt, int64_t M, int64_t K);
GemvGeom gemv_smallm_default_geom(int fmt, int64_t M, int64_t N);
bool gemv_smallm_geom_ok(int64_t M, GemvGeom g);
hipError_t launch_gemv_smallm(int fmt, DevPlanes P, int64_t N, int64_t K, const void* x,
                              bool x_staged, int64_t M, int64_t ldx, float* y, int64_t ldy,
                              int accumulate, GemvGeom g, hipStream_t stream);

// Matrix-core product for Q45 batches (gemv_mfma.hip; the dispatch sends
// 4 or more tokens).  X comes in the staged tile form: xt_bytes(M, K) bytes
// written by launch_stage_x_mfma.  K % 128 == 0; plane 2 8-byte aligned.
int64_t xt_bytes(int64_t M, int64_t K);
hipError_t launch_stage_x_mfma(const float* x, int64_t M, int64_t ldx, int64_t K, void* xt,
                               hipStream_t stream);
hipError_t launch_gemv_mfma_q45(DevPlanes P, int64_t N, int64_t K, const void* xt, int64_t M,
                                float* y, int64_t ldy, int accumulate, hipStream_t stream);
// The same product on fp32 x [M][ldx] (ldx % 4 == 0, 16-byte aligned rows),
// converted while the slabs are filled, with a power of two per 32-weight
// block and token: no staging launch or buffer.  K % 1024 == 0; passes of
// 16 tokens.
// The K-split form of the staged product (gemv_mfma.hip): the plan (S = 1:
// no split) and its workspace, one counter per output tile then the partial
// tiles; the workspace must be all zero before a call, and every call
// leaves it all zero.
struct SplitPlan {
    int S, RW;
    int64_t gx, gy;
};
SplitPlan mfma_split_plan(int64_t N, int64_t K, int64_t M);
size_t mfma_split_workspace_bytes(int64_t N, int64_t K, int64_t M);
hipError_t launch_gemv_mfma_q45_ws(DevPlanes P, int64_t N, int64_t K, const void* xt, int64_t M, float* y,
                                   int64_t ldy, int accumulate, void* ws, hipStream_t stream);
hipError_t launch_gemv_mfma_q45_f32x(DevPlanes P, int64_t N, int64_t K, const float* x,
                                     int64_t ldx, int64_t M, float* y, int64_t ldy,
                                     int accumulate, hipStream_t stream);

// ---- one decode token in one launch (decode_persistent.hip) --------------
// Device-side description of a decoder layer; the table lives in the
// caller's workspace, written by the prepare call.
struct DecLayer {
    DevPlanes qkv, o, gu, dn;   // gu: gate/up rows interleaved
    const float* g1;
    const float* g2;
    int32_t fmt_dn;
    int32_t pad;
};
struct DecHead {
    DevPlanes lm;
    const float* gf;
    int32_t fmt_lm;
    int32_t pad;
};
struct DecTable {
    uint64_t magic;             // kDecMagic once prepared
    int64_t n_layers;
    uint64_t tag;               // identifies the model the table was written for
    uint64_t pad;
    DecHead head;               // the vocabulary product and the final norm
    DecLayer layers[1];         // n_layers entries
};
constexpr uint64_t kDecMagic = 0x31706564716d6266ull;

// Activation buffers of the one-launch step, each written once per token:
// h versions 1 .. 2L (after each residual add), q|k|v and m per layer.
struct DecodeBuffers {
    float* hv;
    float* qkv;
    float* m;
    int64_t hs, qs, ms;   // floats between consecutive versions / layers
};
// One token in one cooperative launch.  Requires d = dq = 4096 and f = 12288
// when there are layers, Q45 qkv/o/gate-up, Q45 or Q65 down and lm head.
// ctr holds the barrier counters (uint32 index 0: global; 32 (g + 1):
// group g).  ctr and err are zeroed by a small kernel first; err != 0
// afterwards means a barrier spin gave up (1) or the table did not match
// (2).  hipErrorInvalidConfiguration if the device's compute units or the
// model's row counts do not fit.
hipError_t launch_decode_persistent(const DecTable* table, DecTable expect, float eps, float* h,
                                    float* logits, int64_t vocab, int64_t nqkv,
                                    const DecodeBuffers& bufs, uint32_t* ctr, uint32_t* err,
                                    hipStream_t stream);

// y[m][n] = 0 for the K == 0 case (rows of length ldy, first N entries).
hipError_t launch_fill_zero(float* y, int64_t M, int64_t N, int64_t ldy, hipStream_t stream);

hipError_t launch_rmsnorm(const float* x, const float* gamma, float eps, int64_t rows, int64_t n,
                          float* y, hipStream_t stream);
hipError_t launch_layernorm(const float* x, const float* gamma, const float* beta, float eps,
                            int64_t rows, int64_t n, float* y, hipStream_t stream);
hipError_t launch_silu_mul(const float* g, const float* u, int64_t n, float* out,
                           hipStream_t stream);

hipError_t launch_dequant(int fmt, DevPlanes P, int64_t N, int64_t K, float* w_out,
                          hipStream_t stream);
// fp32 w [N][ldw] -> planes of fmt (quantize.hip); the planes are written
// through out's pointers.  K % 32 (Q45, Q25), K % 256 (Q65), K % 8 (BF16).
hipError_t launch_quantize(int fmt, const float* w, int64_t ldw, int64_t N, int64_t K,
                           DevPlanes out, hipStream_t stream);
hipError_t launch_unpack_codes(int fmt, DevPlanes P, int64_t N, int64_t K, uint8_t* out,
                               hipStream_t stream);

// Threads per row and float4s per thread of the single-pass RMSNorm kernels
// (mbq_rmsnorm, mbq_rmsnorm_xq), by the row's n (n % 4 == 0): 256 threads up
// to 1024 values, else 1024 threads with 1, 2, 4 or 8 float4s each (up to
// 32768 values); vec = 0 beyond.  Both kernels take the same geometry, so
// they add the squares in the same order.
struct NormGeom {
    int vec, bt;
};
inline NormGeom norm_geom(int64_t n) {
    const int64_t n4 = n >> 2;
    if (n4 <= 256) return NormGeom{1, 256};
    for (int v = 1; v <= 8; v *= 2)
        if (n4 <= 1024 * v) return NormGeom{v, 1024};
    return NormGeom{0, 256};
}

// One token's attention over an fp16 KV cache (attention.hip): head
// dimension kAttD, n_heads / n_kv in {1, 2, 4, 8}, T >= 1.  The workspace
// holds one record of kAttRecord floats per query head and chunk of
// positions (attention_workspace_bytes).
constexpr int kAttD = 128;
constexpr int kAttRecord = 132;
int attention_chunk(int64_t T, int n_kv);
size_t attention_workspace_bytes(int64_t T, int n_heads, int n_kv);
hipError_t launch_attention_decode(const float* q, const uint16_t* kc, const uint16_t* vc, int64_t T,
                                   int64_t ld, int n_heads, int n_kv, float* out, float* ws,
                                   hipStream_t stream);
// The new token's key and value (fp32, knew / vnew, head g at g * kAttD)
// rounded to fp16 and written to row T of the caches, then attention over
// rows 0 .. T (workspace: attention_workspace_bytes(T + 1, ...)).
hipError_t launch_attention_append(const float* q, const float* knew, const float* vnew,
                                   uint16_t* kc, uint16_t* vc, int64_t T, int64_t ld, int n_heads,
                                   int n_kv, float* out, float* ws, hipStream_t stream);

hipError_t launch_probe_read(const void* buf, size_t bytes, float* sink, hipStream_t stream);
hipError_t launch_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);
hipError_t launch_probe_mixed(const void* distinct, size_t dbytes, const void* shared, size_t sbytes,
                              int mode, int blocks, float* sink, hipStream_t stream);
// Pointer chase over `bytes` of buf: chase_entries(bytes) entries, one per
// 256 bytes (a power of two; 0 if bytes < 256).
uint32_t chase_entries(size_t bytes);
hipError_t launch_chase_init(void* buf, size_t bytes, hipStream_t stream);
hipError_t launch_chase(const void* buf, uint32_t n, int64_t hops, uint32_t* sink,
                        hipStream_t stream);
// Issue-rate loops (kind 0 fp16 matrix, 1 fp32 FMA, 2 int8 dot4); sink holds
// kPeakSinkFloats floats; peak_ops gives the operations one launch executes.
constexpr int kPeakSinkFloats = 2048;
int64_t peak_ops(int kind, int64_t iters);
hipError_t launch_peak(int kind, int64_t iters, float* sink, hipStream_t stream);

}  // namespace mbq
