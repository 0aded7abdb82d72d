// abi.cpp -- the C ABI of libmbq (include/mbq.h): argument validation, the
// host packer/unpacker and dispatch to the HIP launchers.  Nothing is
// enqueued unless every argument check passes.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>
#include <cstddef>

#include "../../include/mbq.h"
#include "kernels.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok() {
    g_err.clear();
    return MBQ_OK;
}

int hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(MBQ_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool fmt_valid(int fmt) { return fmt >= MBQ_FMT_BF16 && fmt <= MBQ_FMT_Q25; }

int64_t block_len(int fmt) {
    switch (fmt) {
    case MBQ_FMT_Q45: return 32;
    case MBQ_FMT_Q65: return 256;
    case MBQ_FMT_Q25: return 32;
    default: return 1;
    }
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
    if (an == 0 || bn == 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + bn && b0 < a0 + an;
}

// Shape checks shared by every entry point taking an mbq_qweight.
int check_weight(const mbq_qweight* W, const char* fn) {
    if (!W) return fail(MBQ_EINVAL, "%s: W is NULL", fn);
    if (!fmt_valid(W->fmt)) return fail(MBQ_EINVAL, "%s: unknown format %d", fn, W->fmt);
    if (W->reserved != 0) return fail(MBQ_EINVAL, "%s: W->reserved must be 0", fn);
    if (W->N < 0 || W->K < 0) return fail(MBQ_EINVAL, "%s: negative shape", fn);
    if (W->N > 0x7FFFFFFF) return fail(MBQ_EUNSUPPORTED, "%s: N >= 2^31", fn);
    if (W->K % block_len(W->fmt))
        return fail(MBQ_EINVAL, "%s: K=%lld is not a multiple of the block length %lld", fn,
                    (long long)W->K, (long long)block_len(W->fmt));
    return MBQ_OK;
}

// Plane pointers and alignment (only when there is data to read).
int check_planes(const mbq_qweight* W, const char* fn) {
    const bool need1 = W->fmt == MBQ_FMT_Q65;
    const bool need2 = W->fmt != MBQ_FMT_BF16;
    const bool need3 = W->fmt == MBQ_FMT_Q65;
    if (!W->codes || (need1 && !W->codes_hi) || (need2 && !W->scales) ||
        (need3 && !W->super_scales))
        return fail(MBQ_EINVAL, "%s: a plane the format needs is NULL", fn);
    if (!aligned(W->codes, 16) || (need1 && !aligned(W->codes_hi, 16)))
        return fail(MBQ_EALIGN, "%s: planes 0 and 1 must be 16-byte aligned", fn);
    if ((need2 && !aligned(W->scales, 4)) || (need3 && !aligned(W->super_scales, 4)))
        return fail(MBQ_EALIGN, "%s: planes 2 and 3 must be 4-byte aligned", fn);
    return MBQ_OK;
}

// An output buffer must not overlap any plane of the weights it is computed
// from (the kernels read the planes while others write the output).
int check_out_vs_planes(const mbq_qweight* W, const void* out, size_t out_bytes, const char* fn) {
    size_t sz[4];
    if (mbq_plane_sizes(W->fmt, W->N, W->K, sz) != MBQ_OK) return fail(MBQ_EINVAL, "%s: bad shape", fn);
    const void* p[4] = {W->codes, W->codes_hi, W->scales, W->super_scales};
    for (int i = 0; i < 4; i++)
        if (p[i] && overlaps(out, out_bytes, p[i], sz[i]))
            return fail(MBQ_EINVAL, "%s: the output overlaps weight plane %d", fn, i);
    return MBQ_OK;
}

// Kernel limits common to the GEMV paths and the device exports.
int check_kernel_shape(const mbq_qweight* W, const char* fn) {
    const int64_t kmax = W->fmt == MBQ_FMT_BF16 ? mbq::kMaxKBF16 : mbq::kMaxK;
    if (W->K > kmax)
        return fail(MBQ_EUNSUPPORTED, "%s: K=%lld exceeds %lld", fn, (long long)W->K,
                    (long long)kmax);
    if (W->fmt == MBQ_FMT_Q25 && W->K % 64)
        return fail(MBQ_EUNSUPPORTED, "%s: Q25 kernels need K %% 64 == 0", fn);
    if (W->fmt == MBQ_FMT_BF16 && W->K % 8)
        return fail(MBQ_EUNSUPPORTED, "%s: BF16 kernels need K %% 8 == 0", fn);
    size_t sz[4];
    mbq_plane_sizes(W->fmt, W->N, W->K, sz);
    for (int p = 0; p < 4; p++)
        if (sz[p] > 0xFFFFFFFFull) return fail(MBQ_EUNSUPPORTED, "%s: a plane of 4 GiB or more", fn);
    return MBQ_OK;
}

// Q45 batches of kMfmaMinM or more tokens run on the matrix cores (staged x
// then takes the tile form), for K % 128 == 0.  The vector units' digit
// arithmetic has M* = (w/16)(R/BW) of about one token on MI355X (measured
// R and BW), the matrix cores' about twelve, so from a few tokens on the
// matrix cores carry the sums at the weight-read rate.  Measured crossover
// (us, staged x, graphs of cold launches): 12288 x 4096 at 3 / 4 / 5 tokens
// 13.9 / 16.0 / 18.6 on the vector units against 13.4 / 13.5 / 13.2 on the
// matrix cores; 4096 x 12288 17.4 / 20.9 / 26.0 against 18.9 / 18.9 / 18.9.
constexpr int64_t kMfmaMinM = 4;
static int64_t mfma_min_m() {
    static const int64_t v = [] {
        const char* e = mbq::tuning_var("MBQ_MFMA_MIN_M");      // tuning: read once
        const int64_t t = e ? atoll(e) : kMfmaMinM;
        return t < 2 ? (int64_t)2 : t;
    }();
    return v;
}
bool mfma_shape(int fmt, int64_t M, int64_t K) {
    return fmt == MBQ_FMT_Q45 && M >= mfma_min_m() && K % 128 == 0;
}
bool xq_tiled(int fmt, int64_t M, int64_t K) { return mfma_shape(fmt, M, K); }

// Values per chunk of staged x (the unit of its fixed-point exponent).
int64_t xq_chunk(int fmt) {
    switch (fmt) {
    case MBQ_FMT_Q45: return 32;
    case MBQ_FMT_Q65: return 32;
    case MBQ_FMT_Q25: return 64;
    default: return 8;
    }
}

mbq::DevPlanes planes_of(const mbq_qweight* W) {
    return mbq::DevPlanes{(const uint8_t*)W->codes, (const uint8_t*)W->codes_hi,
                          (const uint8_t*)W->scales, (const uint8_t*)W->super_scales};
}

// Optional geometry overrides for tuning sweeps (with MBQ_TUNING set):
// MBQ_GEMV_ROWS = 1, 2 or 4 rows per wave; MBQ_GEMV_GROUPS = row groups per
// wave.
bool geom_override(mbq::GemvGeom* g) {
    bool any = false;
    const char* s = mbq::tuning_var("MBQ_GEMV_ROWS");
    int r = 0;
    if (s && sscanf(s, "%d", &r) == 1 && (r == 1 || r == 2 || r == 4)) {
        g->rows_per_wave = r;
        any = true;
    }
    const char* t = mbq::tuning_var("MBQ_GEMV_GROUPS");
    int gg = 0;
    if (t && sscanf(t, "%d", &gg) == 1 && gg >= 1 && gg <= 64) {
        g->groups = gg;
        any = true;
    }
    return any;
}

// Small-batch geometry: defaults, or (with MBQ_TUNING set) MBQ_SMALLM_ROWS
// (1 to 3) and MBQ_SMALLM_GROUPS; an override that does not fit the
// kernel's row-sum buffer is ignored.
mbq::GemvGeom smallm_geom(int fmt, int64_t M, int64_t N) {
    mbq::GemvGeom g = mbq::gemv_smallm_default_geom(fmt, M, N);
    mbq::GemvGeom o = g;
    int v = 0;
    const char* s = mbq::tuning_var("MBQ_SMALLM_ROWS");
    if (s && sscanf(s, "%d", &v) == 1) o.rows_per_wave = v;
    const char* t = mbq::tuning_var("MBQ_SMALLM_GROUPS");
    if (t && sscanf(t, "%d", &v) == 1) o.groups = v;
    return mbq::gemv_smallm_geom_ok(M, o) ? o : g;
}

// ------------------------------------------------------------ host packer

// Bit of the run's 32-bit high-bits word that holds weight r of a Q65 run of
// 16 (mbq.h).  The order lets the device assemble four 6-bit codes in the
// bytes of a dword with at most two shifts, one mask and one and-or.
constexpr int kQ65HighBit[16] = {4, 2, 12, 10, 20, 18, 28, 26, 0, 6, 8, 14, 16, 22, 24, 30};

}  // namespace

extern "C" {

int mbq_version(void) { return 1; }

const char* mbq_status_str(int status) {
    switch (status) {
    case MBQ_OK: return "MBQ_OK";
    case MBQ_EINVAL: return "MBQ_EINVAL: invalid argument";
    case MBQ_EALIGN: return "MBQ_EALIGN: misaligned pointer";
    case MBQ_EUNSUPPORTED: return "MBQ_EUNSUPPORTED: no kernel for this request";
    case MBQ_EHIP: return "MBQ_EHIP: HIP runtime error";
    default: return "unknown status";
    }
}

const char* mbq_last_error(void) { return g_err.c_str(); }

int mbq_format_info(int fmt, double* bits_per_weight, int* block_k) {
    if (!fmt_valid(fmt)) return fail(MBQ_EINVAL, "mbq_format_info: unknown format %d", fmt);
    if (!bits_per_weight || !block_k) return fail(MBQ_EINVAL, "mbq_format_info: NULL output");
    static const double bpw[4] = {16.0, 4.5, 6.5625, 2.5};
    *bits_per_weight = bpw[fmt];
    *block_k = (int)block_len(fmt);
    return ok();
}

int mbq_plane_sizes(int fmt, int64_t N, int64_t K, size_t sizes[4]) {
    if (!sizes) return fail(MBQ_EINVAL, "mbq_plane_sizes: NULL sizes");
    if (!fmt_valid(fmt)) return fail(MBQ_EINVAL, "mbq_plane_sizes: unknown format %d", fmt);
    if (N < 0 || K < 0) return fail(MBQ_EINVAL, "mbq_plane_sizes: negative shape");
    if (K % block_len(fmt)) return fail(MBQ_EINVAL, "mbq_plane_sizes: K not a multiple of the block");
    const size_t nk = (size_t)N * (size_t)K;
    sizes[0] = sizes[1] = sizes[2] = sizes[3] = 0;
    switch (fmt) {
    case MBQ_FMT_BF16: sizes[0] = 2 * nk; break;
    case MBQ_FMT_Q45: sizes[0] = nk / 2; sizes[2] = nk / 16; break;        // 2 B per 32
    case MBQ_FMT_Q65: sizes[0] = nk / 2; sizes[1] = nk / 4; sizes[2] = nk / 16; sizes[3] = nk / 128; break;
    case MBQ_FMT_Q25: sizes[0] = nk / 4; sizes[2] = nk / 16; break;
    }
    return ok();
}

int mbq_pack(int fmt, int64_t N, int64_t K, const void* codes, const void* scales,
             const void* super_scales, void* const planes[4]) {
    size_t sz[4];
    int rc = mbq_plane_sizes(fmt, N, K, sz);
    if (rc) return rc;
    if (!planes || !codes) return fail(MBQ_EINVAL, "mbq_pack: NULL pointer");
    for (int p = 0; p < 4; p++)
        if (sz[p] && !planes[p]) return fail(MBQ_EINVAL, "mbq_pack: plane %d is NULL", p);
    if (fmt != MBQ_FMT_BF16 && sz[2] && !scales) return fail(MBQ_EINVAL, "mbq_pack: NULL scales");
    if (fmt == MBQ_FMT_Q65 && sz[3] && !super_scales)
        return fail(MBQ_EINVAL, "mbq_pack: NULL super_scales");
    const uint8_t* q = (const uint8_t*)codes;
    const size_t nk = (size_t)N * (size_t)K;
    if (fmt == MBQ_FMT_BF16) {
        memcpy(planes[0], codes, sz[0]);
        return ok();
    }
    const int bits = fmt == MBQ_FMT_Q45 ? 4 : fmt == MBQ_FMT_Q65 ? 6 : 2;
    for (size_t i = 0; i < nk; i++)
        if (q[i] >> bits) return fail(MBQ_EINVAL, "mbq_pack: code %u at %zu exceeds %d bits", q[i], i, bits);
    uint8_t* p0 = (uint8_t*)planes[0];
    if (fmt == MBQ_FMT_Q45) {
        for (size_t i = 0; i < nk / 2; i++) p0[i] = (uint8_t)(q[2 * i] | (q[2 * i + 1] << 4));
    } else if (fmt == MBQ_FMT_Q25) {
        for (size_t i = 0; i < nk / 4; i++)
            p0[i] = (uint8_t)(q[4 * i] | (q[4 * i + 1] << 2) | (q[4 * i + 2] << 4) | (q[4 * i + 3] << 6));
    } else {
        // Q65: runs of 16 weights (K % 256 == 0, so runs never span rows);
        // the high bits of a run form one little-endian 32-bit word.
        uint8_t* p1 = (uint8_t*)planes[1];
        for (size_t r = 0; r < nk / 16; r++) {
            const uint8_t* c = q + 16 * r;
            for (int i = 0; i < 8; i++) p0[8 * r + i] = (uint8_t)((c[2 * i] & 15) | ((c[2 * i + 1] & 15) << 4));
            uint32_t w = 0;
            for (int k = 0; k < 16; k++) w |= (uint32_t)(c[k] >> 4) << kQ65HighBit[k];
            for (int j = 0; j < 4; j++) p1[4 * r + j] = (uint8_t)(w >> (8 * j));
        }
    }
    memcpy(planes[2], scales, sz[2]);
    if (fmt == MBQ_FMT_Q65) memcpy(planes[3], super_scales, sz[3]);
    return ok();
}

int mbq_unpack(int fmt, int64_t N, int64_t K, const void* const planes[4], void* codes,
               void* scales, void* super_scales) {
    size_t sz[4];
    int rc = mbq_plane_sizes(fmt, N, K, sz);
    if (rc) return rc;
    if (!planes || !codes) return fail(MBQ_EINVAL, "mbq_unpack: NULL pointer");
    for (int p = 0; p < 4; p++)
        if (sz[p] && !planes[p]) return fail(MBQ_EINVAL, "mbq_unpack: plane %d is NULL", p);
    const size_t nk = (size_t)N * (size_t)K;
    uint8_t* q = (uint8_t*)codes;
    const uint8_t* p0 = (const uint8_t*)planes[0];
    if (fmt == MBQ_FMT_BF16) {
        memcpy(codes, planes[0], sz[0]);
        return ok();
    }
    if ((sz[2] && !scales) || (fmt == MBQ_FMT_Q65 && !super_scales))
        return fail(MBQ_EINVAL, "mbq_unpack: NULL scale output");
    if (fmt == MBQ_FMT_Q45) {
        for (size_t i = 0; i < nk; i++) q[i] = (uint8_t)((p0[i >> 1] >> ((i & 1) * 4)) & 15);
    } else if (fmt == MBQ_FMT_Q25) {
        for (size_t i = 0; i < nk; i++) q[i] = (uint8_t)((p0[i >> 2] >> ((i & 3) * 2)) & 3);
    } else {
        const uint8_t* p1 = (const uint8_t*)planes[1];
        for (size_t r = 0; r < nk / 16; r++) {
            uint8_t* c = q + 16 * r;
            const uint32_t w = (uint32_t)p1[4 * r] | ((uint32_t)p1[4 * r + 1] << 8) |
                               ((uint32_t)p1[4 * r + 2] << 16) | ((uint32_t)p1[4 * r + 3] << 24);
            for (int i = 0; i < 8; i++) {
                c[2 * i] = (uint8_t)(p0[8 * r + i] & 15);
                c[2 * i + 1] = (uint8_t)(p0[8 * r + i] >> 4);
            }
            for (int k = 0; k < 16; k++) c[k] |= (uint8_t)(((w >> kQ65HighBit[k]) & 3) << 4);
        }
    }
    memcpy(scales, planes[2], sz[2]);
    if (fmt == MBQ_FMT_Q65) memcpy(super_scales, planes[3], sz[3]);
    return ok();
}

int mbq_gemv_q(const mbq_qweight* W, const float* x, int64_t M, int64_t ldx, float* y,
               int64_t ldy, int accumulate, void* stream) {
    const char* fn = "mbq_gemv_q";
    int rc = check_weight(W, fn);
    if (rc) return rc;
    if (M < 0) return fail(MBQ_EINVAL, "%s: M < 0", fn);
    if (ldx < W->K || ldy < W->N) return fail(MBQ_EINVAL, "%s: ldx < K or ldy < N", fn);
    if (accumulate != 0 && accumulate != 1) return fail(MBQ_EINVAL, "%s: accumulate must be 0 or 1", fn);
    if (M == 0 || W->N == 0) return ok();
    if (!x || !y) return fail(MBQ_EINVAL, "%s: x or y is NULL", fn);
    if (!aligned(y, 4)) return fail(MBQ_EALIGN, "%s: y must be 4-byte aligned", fn);
    const size_t ybytes = (size_t)((M - 1) * ldy + W->N) * 4;
    hipStream_t s = (hipStream_t)stream;
    if (W->K == 0) {
        if (accumulate) return ok();
        return hip_status(mbq::launch_fill_zero(y, M, W->N, ldy, s), fn);
    }
    if (!aligned(x, 16) || ldx % 4) return fail(MBQ_EALIGN, "%s: x must be 16-byte aligned with ldx %% 4 == 0", fn);
    const size_t xbytes = (size_t)((M - 1) * ldx + W->K) * 4;
    if (overlaps(x, xbytes, y, ybytes)) return fail(MBQ_EINVAL, "%s: x and y overlap", fn);
    if ((rc = check_planes(W, fn))) return rc;
    if ((rc = check_out_vs_planes(W, y, ybytes, fn))) return rc;
    if ((rc = check_kernel_shape(W, fn))) return rc;
    const mbq::DevPlanes P = planes_of(W);
    if (M == 1) {
        mbq::GemvGeom g = mbq::gemv_m1_default_geom(W->fmt, W->N, W->K);
        geom_override(&g);
        return hip_status(mbq::launch_gemv_m1(W->fmt, P, W->N, W->K, x, false, y, accumulate,
                                              nullptr, 1, g, s), fn);
    }
    // Q45 batches on the matrix cores, fp32 x converted in registers by the
    // product
    if (mfma_shape(W->fmt, M, W->K) && aligned(W->scales, 8))
        return hip_status(mbq::launch_gemv_mfma_q45_f32x(P, W->N, W->K, x, ldx, M, y, ldy,
                                                         accumulate, s), fn);
    // 2 <= M: passes of up to 8 tokens on the vector units, as many as the
    // LDS holds staged (a single token always fits: K <= kMaxK)
    int64_t mp = M < 8 ? M : 8;
    while (mp > 1 && !mbq::gemv_smallm_fits(W->fmt, mp, W->K)) mp--;
    for (int64_t m0 = 0; m0 < M; m0 += mp) {
        const int64_t mm = M - m0 < mp ? M - m0 : mp;
        hipError_t e = mm == 1 ? mbq::launch_gemv_m1(W->fmt, P, W->N, W->K, x + m0 * ldx, false,
                                                     y + m0 * ldy, accumulate, nullptr, 1,
                                                     mbq::gemv_m1_default_geom(W->fmt, W->N, W->K), s)
                               : mbq::launch_gemv_smallm(W->fmt, P, W->N, W->K, x + m0 * ldx, false,
                                                         mm, ldx, y + m0 * ldy, ldy, accumulate,
                                                         smallm_geom(W->fmt, mm, W->N), s);
        if (e != hipSuccess) return hip_status(e, fn);
    }
    return ok();
}

int mbq_gemv_q_gather(const mbq_qweight* W_all, int64_t rows_per_expert, const int32_t* idx,
                      int64_t n_sel, const float* x, float* y, void* stream) {
    const char* fn = "mbq_gemv_q_gather";
    int rc = check_weight(W_all, fn);
    if (rc) return rc;
    if (rows_per_expert <= 0 || n_sel < 0) return fail(MBQ_EINVAL, "%s: bad rows_per_expert or n_sel", fn);
    if (W_all->N % rows_per_expert) return fail(MBQ_EINVAL, "%s: N is not a multiple of rows_per_expert", fn);
    if (n_sel == 0) return ok();
    if (!idx || !x || !y) return fail(MBQ_EINVAL, "%s: NULL pointer", fn);
    if (!aligned(idx, 4) || !aligned(y, 4)) return fail(MBQ_EALIGN, "%s: idx and y must be 4-byte aligned", fn);
    const int64_t n_out = n_sel * rows_per_expert;
    hipStream_t s = (hipStream_t)stream;
    if (W_all->K == 0) return hip_status(mbq::launch_fill_zero(y, 1, n_out, n_out, s), fn);
    if (!aligned(x, 16)) return fail(MBQ_EALIGN, "%s: x must be 16-byte aligned", fn);
    if (overlaps(x, (size_t)W_all->K * 4, y, (size_t)n_out * 4)) return fail(MBQ_EINVAL, "%s: x and y overlap", fn);
    if ((rc = check_planes(W_all, fn))) return rc;
    if ((rc = check_out_vs_planes(W_all, y, (size_t)n_out * 4, fn))) return rc;
    if ((rc = check_kernel_shape(W_all, fn))) return rc;
    mbq::GemvGeom g = mbq::gemv_m1_default_geom(W_all->fmt, n_out, W_all->K);
    geom_override(&g);
    return hip_status(mbq::launch_gemv_m1(W_all->fmt, planes_of(W_all), n_out, W_all->K, x, false,
                                          y, 0, idx, rows_per_expert, g, s, W_all->N), fn);
}

int mbq_gemv_fused(const mbq_qweight* W, const float* x, const float* gamma, float eps,
                   int epilogue, float* y, void* stream) {
    const char* fn = "mbq_gemv_fused";
    int rc = check_weight(W, fn);
    if (rc) return rc;
    if (epilogue < MBQ_EPI_STORE || epilogue > MBQ_EPI_SILU_MUL)
        return fail(MBQ_EINVAL, "%s: unknown epilogue %d", fn, epilogue);
    const bool silu = epilogue == MBQ_EPI_SILU_MUL;
    if (silu && W->N % 2) return fail(MBQ_EINVAL, "%s: the silu epilogue needs an even N", fn);
    if (gamma && (!(eps >= 0.f) || eps == __builtin_inff()))
        return fail(MBQ_EINVAL, "%s: eps must be finite and >= 0", fn);
    if (W->N == 0) return ok();
    if (!x || !y) return fail(MBQ_EINVAL, "%s: x or y is NULL", fn);
    if (!aligned(x, 16) || !aligned(y, 4) || (gamma && !aligned(gamma, 16)))
        return fail(MBQ_EALIGN, "%s: x and gamma must be 16-byte aligned, y 4-byte", fn);
    const int64_t n_out = silu ? W->N / 2 : W->N;
    const size_t xb = (size_t)W->K * 4, yb = (size_t)n_out * 4;
    if (overlaps(x, xb, y, yb) || (gamma && overlaps(gamma, xb, y, yb)))
        return fail(MBQ_EINVAL, "%s: y overlaps x or gamma", fn);
    if ((rc = check_planes(W, fn))) return rc;
    if ((rc = check_out_vs_planes(W, y, yb, fn))) return rc;
    if ((rc = check_kernel_shape(W, fn))) return rc;
    hipStream_t s = (hipStream_t)stream;
    mbq::GemvGeom g = mbq::gemv_m1_default_geom(W->fmt, W->N, W->K, silu, gamma != nullptr);
    geom_override(&g);
    if (!gamma && !silu)
        return hip_status(mbq::launch_gemv_m1(W->fmt, planes_of(W), W->N, W->K, x, false, y,
                                              epilogue == MBQ_EPI_ACCUMULATE, nullptr, 1, g, s), fn);
    if (!mbq::gemv_fused_supported(W->fmt, W->K))
        return fail(MBQ_EUNSUPPORTED, "%s: fused kernels exist for Q45/Q65 with K = 4096 or 12288", fn);
    return hip_status(mbq::launch_gemv_fused(W->fmt, planes_of(W), W->N, W->K, x, gamma, eps, silu,
                                             y, epilogue == MBQ_EPI_ACCUMULATE, g, s), fn);
}

// ---------------------------------------------------------- decode step

static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

static int check_decode(const mbq_decode_model* m, const char* fn) {
    if (!m) return fail(MBQ_EINVAL, "%s: model is NULL", fn);
    if (m->n_layers < 0 || m->d <= 0 || m->dq < 0 || m->dkv < 0 || m->f < 0 ||
        (m->n_layers > 0 && m->f == 0) || m->vocab < 0)
        return fail(MBQ_EINVAL, "%s: bad model dimensions", fn);
    if (!(m->eps >= 0.f) || m->eps == __builtin_inff()) return fail(MBQ_EINVAL, "%s: bad eps", fn);
    if (m->n_layers > 0 && !m->layers) return fail(MBQ_EINVAL, "%s: layers is NULL", fn);
    if (!m->gamma_f || !aligned(m->gamma_f, 16)) return fail(MBQ_EALIGN, "%s: gamma_f must be 16-byte aligned", fn);
    auto shape = [&](const mbq_qweight& W, int64_t N, int64_t K, bool fused, const char* what) {
        int rc = check_weight(&W, fn);
        if (rc) return rc;
        if (W.N != N || W.K != K)
            return fail(MBQ_EINVAL, "%s: %s is %lldx%lld, expected %lldx%lld", fn, what,
                        (long long)W.N, (long long)W.K, (long long)N, (long long)K);
        if ((rc = check_planes(&W, fn)) || (rc = check_kernel_shape(&W, fn))) return rc;
        if (fused && !mbq::gemv_fused_supported(W.fmt, W.K))
            return fail(MBQ_EUNSUPPORTED, "%s: %s needs a fused kernel (Q45/Q65, K = 4096 or 12288)", fn, what);
        return MBQ_OK;
    };
    for (int l = 0; l < m->n_layers; l++) {
        const mbq_decode_layer& L = m->layers[l];
        int rc;
        if ((rc = shape(L.qkv, m->dq + 2 * m->dkv, m->d, true, "qkv")) ||
            (rc = shape(L.o, m->d, m->dq, false, "o")) ||
            (rc = shape(L.gate_up, 2 * m->f, m->d, true, "gate_up")) ||
            (rc = shape(L.down, m->d, m->f, false, "down")))
            return rc;
        if (!L.gamma1 || !L.gamma2 || !aligned(L.gamma1, 16) || !aligned(L.gamma2, 16))
            return fail(MBQ_EALIGN, "%s: layer gammas must be 16-byte aligned", fn);
    }
    if (m->vocab > 0) {
        int rc = shape(m->lm_head, m->vocab, m->d, true, "lm_head");
        if (rc) return rc;
    }
    return MBQ_OK;
}

// Workspace of the decode step: [0, 2048) the one-launch step's barrier
// counters (global at 0, group g at 128 (g + 1)) and status word (at 4);
// then q|k|v and the gated activations of each layer (the launch chain uses
// the first layer's), the h versions of the one-launch step (one per
// residual add), and its layer table.
struct DecodeLayout {
    size_t qkv, m, hv, table, total;
    size_t qs, ms, hs;   // bytes between layers / versions
};

static DecodeLayout decode_layout(const mbq_decode_model* m) {
    DecodeLayout L;
    const size_t nl = (size_t)(m->n_layers > 0 ? m->n_layers : 1);
    L.qs = align256((size_t)(m->dq + 2 * m->dkv) * 4);
    L.ms = align256((size_t)m->f * 4);
    L.hs = align256((size_t)m->d * 4);
    L.qkv = 2048;
    L.m = L.qkv + nl * L.qs;
    L.hv = L.m + nl * L.ms;
    L.table = L.hv + 2 * nl * L.hs;
    L.total = L.table + align256(offsetof(mbq::DecTable, layers) + nl * sizeof(mbq::DecLayer));
    return L;
}

int mbq_decode_workspace_bytes(const mbq_decode_model* m, size_t* bytes) {
    const char* fn = "mbq_decode_workspace_bytes";
    if (!m || !bytes) return fail(MBQ_EINVAL, "%s: NULL pointer", fn);
    if (m->n_layers < 0 || m->dq < 0 || m->dkv < 0 || m->f < 0)
        return fail(MBQ_EINVAL, "%s: bad dimensions", fn);
    *bytes = decode_layout(m).total;
    return ok();
}

static int check_workspace(const mbq_decode_model* m, const float* h, const float* logits,
                           const void* workspace, size_t workspace_bytes, const char* fn) {
    const size_t need = decode_layout(m).total;
    if (!h || !aligned(h, 16)) return fail(MBQ_EALIGN, "%s: h must be 16-byte aligned", fn);
    if (m->vocab > 0 && (!logits || !aligned(logits, 4))) return fail(MBQ_EINVAL, "%s: bad logits", fn);
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < need)
        return fail(MBQ_EINVAL, "%s: workspace must be 256-byte aligned and >= %zu bytes", fn, need);
    const size_t hb = (size_t)m->d * 4;
    if (overlaps(h, hb, workspace, need) || (m->vocab > 0 && (overlaps(logits, (size_t)m->vocab * 4, h, hb) ||
                                                               overlaps(logits, (size_t)m->vocab * 4, workspace, need))))
        return fail(MBQ_EINVAL, "%s: h, logits and workspace must not overlap", fn);
    return MBQ_OK;
}

// Attention over per-layer KV caches inside the launch chain: row T of each
// layer's caches takes the new key and value, the attention output (dq
// floats) goes to att, and ws holds the partial records.
struct KvChain {
    void* const* kc;
    void* const* vc;
    int64_t T, ld;
    float* att;
    float* ws;
};

// The launch chain of one token: qkv holds q|k|v (dq + 2 dkv floats) and mm
// the gated activations (f floats) between launches.  Without kv the o
// product reads q (the stand-in); with it, the attention output.
static hipError_t decode_chain(const mbq_decode_model* m, float* h, float* logits, float* qkv,
                               float* mm, hipStream_t s, const KvChain* kv = nullptr) {
    auto geom = [](const mbq_qweight& W, bool pairs = false, bool norm = false) {
        mbq::GemvGeom g = mbq::gemv_m1_default_geom(W.fmt, W.N, W.K, pairs, norm);
        geom_override(&g);
        return g;
    };
    hipError_t e = hipSuccess;
    for (int l = 0; l < m->n_layers && e == hipSuccess; l++) {
        const mbq_decode_layer& L = m->layers[l];
        // a = rmsnorm(h, gamma1); q|k|v = Wqkv a
        e = mbq::launch_gemv_fused(L.qkv.fmt, planes_of(&L.qkv), L.qkv.N, L.qkv.K, h, L.gamma1,
                                   m->eps, false, qkv, 0, geom(L.qkv, false, true), s);
        // att = attention(q, K[0..T], V[0..T]) after K[T] = k, V[T] = v
        const float* o_in = qkv;
        if (kv && e == hipSuccess) {
            e = mbq::launch_attention_append(qkv, qkv + m->dq, qkv + m->dq + m->dkv,
                                             (uint16_t*)kv->kc[l], (uint16_t*)kv->vc[l], kv->T,
                                             kv->ld, (int)(m->dq / mbq::kAttD),
                                             (int)(m->dkv / mbq::kAttD), kv->att, kv->ws, s);
            o_in = kv->att;
        }
        // h += Wo att   (without a cache q stands in for the attention output)
        if (e == hipSuccess)
            e = mbq::launch_gemv_m1(L.o.fmt, planes_of(&L.o), L.o.N, L.o.K, o_in, false, h, 1,
                                    nullptr, 1, geom(L.o), s);
        // b = rmsnorm(h, gamma2); m = silu(Wg b) * (Wu b)
        if (e == hipSuccess)
            e = mbq::launch_gemv_fused(L.gate_up.fmt, planes_of(&L.gate_up), L.gate_up.N,
                                       L.gate_up.K, h, L.gamma2, m->eps, true, mm, 0,
                                       geom(L.gate_up, true), s);
        // h += Wd m
        if (e == hipSuccess)
            e = mbq::launch_gemv_m1(L.down.fmt, planes_of(&L.down), L.down.N, L.down.K, mm, false,
                                    h, 1, nullptr, 1, geom(L.down), s);
    }
    // logits = Wvocab rmsnorm(h, gamma_f)
    if (e == hipSuccess && m->vocab > 0)
        e = mbq::launch_gemv_fused(m->lm_head.fmt, planes_of(&m->lm_head), m->vocab, m->d, h,
                                   m->gamma_f, m->eps, false, logits, 0, geom(m->lm_head, false, true), s);
    return e;
}

int mbq_decode_step(const mbq_decode_model* m, float* h, float* logits, void* workspace,
                    size_t workspace_bytes, void* stream) {
    const char* fn = "mbq_decode_step";
    int rc = check_decode(m, fn);
    if (rc) return rc;
    if ((rc = check_workspace(m, h, logits, workspace, workspace_bytes, fn))) return rc;
    const DecodeLayout lay = decode_layout(m);
    float* qkv = (float*)((char*)workspace + lay.qkv);
    float* mm = (float*)((char*)workspace + lay.m);
    return hip_status(decode_chain(m, h, logits, qkv, mm, (hipStream_t)stream), fn);
}

// ---- the step with attention over KV caches -------------------------------
static int check_attention_shape(int64_t T, int n_heads, int n_kv, int head_dim, const char* fn);

// Workspace: q|k|v, the gated activations, the attention output, then the
// attention's partial records for T + 1 positions.
struct KvLayout {
    size_t qkv, m, att, rec, total;
};

static KvLayout kv_layout(const mbq_decode_model* m, int64_t T) {
    KvLayout L;
    L.qkv = 0;
    L.m = align256((size_t)(m->dq + 2 * m->dkv) * 4);
    L.att = L.m + align256((size_t)m->f * 4);
    L.rec = L.att + align256((size_t)m->dq * 4);
    const int nkv = (int)(m->dkv / mbq::kAttD);
    L.total = L.rec + align256(mbq::attention_workspace_bytes(T + 1, (int)(m->dq / mbq::kAttD),
                                                              nkv > 0 ? nkv : 1));
    return L;
}

static int check_kv_shape(const mbq_decode_model* m, int64_t T, const char* fn) {
    if (m->dq <= 0 || m->dkv <= 0 || m->dq % mbq::kAttD || m->dkv % mbq::kAttD)
        return fail(MBQ_EUNSUPPORTED, "%s: dq and dkv must be positive multiples of the head size %d",
                    fn, mbq::kAttD);
    if (T < 0) return fail(MBQ_EINVAL, "%s: T < 0", fn);
    return check_attention_shape(T + 1, (int)(m->dq / mbq::kAttD), (int)(m->dkv / mbq::kAttD), mbq::kAttD, fn);
}

int mbq_decode_kv_workspace_bytes(const mbq_decode_model* m, int64_t T, size_t* bytes) {
    const char* fn = "mbq_decode_kv_workspace_bytes";
    if (!m || !bytes) return fail(MBQ_EINVAL, "%s: NULL pointer", fn);
    if (m->n_layers < 0 || m->dq < 0 || m->dkv < 0 || m->f < 0)
        return fail(MBQ_EINVAL, "%s: bad dimensions", fn);
    if (int rc = check_kv_shape(m, T, fn)) return rc;
    *bytes = kv_layout(m, T).total;
    return ok();
}

int mbq_decode_step_kv(const mbq_decode_model* m, float* h, float* logits, void* const* k_caches,
                       void* const* v_caches, int64_t T, int64_t ld, void* workspace,
                       size_t workspace_bytes, void* stream) {
    const char* fn = "mbq_decode_step_kv";
    int rc = check_decode(m, fn);
    if (rc) return rc;
    if ((rc = check_kv_shape(m, T, fn))) return rc;
    const KvLayout lay = kv_layout(m, T);
    if (!h || !aligned(h, 16)) return fail(MBQ_EALIGN, "%s: h must be 16-byte aligned", fn);
    if (m->vocab > 0 && (!logits || !aligned(logits, 4))) return fail(MBQ_EINVAL, "%s: bad logits", fn);
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < lay.total)
        return fail(MBQ_EINVAL, "%s: workspace must be 256-byte aligned and >= %zu bytes", fn, lay.total);
    const size_t hb = (size_t)m->d * 4, lb = m->vocab > 0 ? (size_t)m->vocab * 4 : 0;
    if (overlaps(h, hb, workspace, lay.total) || (lb && (overlaps(logits, lb, h, hb) ||
                                                         overlaps(logits, lb, workspace, lay.total))))
        return fail(MBQ_EINVAL, "%s: h, logits and workspace must not overlap", fn);
    if (ld < m->dkv) return fail(MBQ_EINVAL, "%s: ld < dkv", fn);
    if (ld % 8) return fail(MBQ_EALIGN, "%s: ld must be a multiple of 8", fn);
    if (m->n_layers > 0 && (!k_caches || !v_caches)) return fail(MBQ_EINVAL, "%s: cache arrays are NULL", fn);
    const size_t cb = (size_t)(T * ld + m->dkv) * 2;    // rows 0 .. T
    for (int l = 0; l < m->n_layers; l++) {
        const void* kc = k_caches[l];
        const void* vc = v_caches[l];
        if (!kc || !vc) return fail(MBQ_EINVAL, "%s: layer %d's cache is NULL", fn, l);
        if (!aligned(kc, 16) || !aligned(vc, 16))
            return fail(MBQ_EALIGN, "%s: layer %d's caches must be 16-byte aligned", fn, l);
        if (overlaps(kc, cb, vc, cb) || overlaps(kc, cb, workspace, lay.total) ||
            overlaps(vc, cb, workspace, lay.total) || overlaps(kc, cb, h, hb) || overlaps(vc, cb, h, hb) ||
            (lb && (overlaps(kc, cb, logits, lb) || overlaps(vc, cb, logits, lb))))
            return fail(MBQ_EINVAL, "%s: layer %d's caches overlap each other or another buffer", fn, l);
    }
    char* w = (char*)workspace;
    const KvChain kv{k_caches, v_caches, T, ld, (float*)(w + lay.att), (float*)(w + lay.rec)};
    return hip_status(decode_chain(m, h, logits, (float*)(w + lay.qkv), (float*)(w + lay.m),
                                   (hipStream_t)stream, &kv),
                      fn);
}

// ---- the same step without a workspace argument --------------------------
// The activations between launches live in a file-scope device array, one
// copy per GPU, held until the process ends.  Host code never passes the
// array's name to a kernel (it is a host-side stand-in there): each device's
// address comes from hipGetSymbolAddress, taken once per device with that
// device current.
constexpr size_t kScratchBytes = (size_t)1 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::atomic<void*> g_scratch_ptr[kMaxDevices];
static std::mutex g_scratch_mu;

static int scratch_of_current_device(void** out, const char* fn) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, fn);
    if (dev < 0 || dev >= kMaxDevices) return fail(MBQ_EUNSUPPORTED, "%s: device %d beyond %d", fn, dev, kMaxDevices);
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return hip_status(e, fn);
            if (!p) return fail(MBQ_EHIP, "%s: no device address for the scratch array", fn);
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return MBQ_OK;
}

// Identity of a model's device pointers (FNV-1a over every plane and gamma).
static uint64_t decode_tag(const mbq_decode_model* m) {
    uint64_t hsh = 1469598103934665603ull;
    auto mix = [&](const void* p) {
        uint64_t v = (uint64_t)(uintptr_t)p;
        for (int b = 0; b < 8; b++) {
            hsh ^= (v >> (8 * b)) & 0xFF;
            hsh *= 1099511628211ull;
        }
    };
    auto mixw = [&](const mbq_qweight& W) {
        mix(W.codes); mix(W.codes_hi); mix(W.scales); mix(W.super_scales);
    };
    for (int l = 0; l < m->n_layers; l++) {
        const mbq_decode_layer& L = m->layers[l];
        mixw(L.qkv); mixw(L.o); mixw(L.gate_up); mixw(L.down);
        mix(L.gamma1); mix(L.gamma2);
    }
    mix((const void*)(uintptr_t)m->n_layers);
    if (m->vocab > 0) mixw(m->lm_head);
    mix(m->gamma_f);
    mix((const void*)(uintptr_t)m->vocab);
    return hsh;
}

int mbq_decode_prepare(const mbq_decode_model* m, void* workspace, size_t workspace_bytes,
                       void* stream) {
    const char* fn = "mbq_decode_prepare";
    int rc = check_decode(m, fn);
    if (rc) return rc;
    const DecodeLayout lay = decode_layout(m);
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < lay.total)
        return fail(MBQ_EINVAL, "%s: workspace must be 256-byte aligned and >= %zu bytes", fn, lay.total);
    std::vector<uint8_t> host(lay.total - lay.table, 0);
    mbq::DecTable* t = (mbq::DecTable*)host.data();
    t->magic = mbq::kDecMagic;
    t->n_layers = m->n_layers;
    t->tag = decode_tag(m);
    if (m->vocab > 0) {
        t->head.lm = planes_of(&m->lm_head);
        t->head.fmt_lm = m->lm_head.fmt;
    }
    t->head.gf = m->gamma_f;
    for (int l = 0; l < m->n_layers; l++) {
        const mbq_decode_layer& L = m->layers[l];
        mbq::DecLayer& D = t->layers[l];
        D.qkv = planes_of(&L.qkv);
        D.o = planes_of(&L.o);
        D.gu = planes_of(&L.gate_up);
        D.dn = planes_of(&L.down);
        D.g1 = L.gamma1;
        D.g2 = L.gamma2;
        D.fmt_dn = L.down.fmt;
    }
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hipMemcpyAsync((char*)workspace + lay.table, host.data(), host.size(),
                                  hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    return hip_status(e, fn);
}

int mbq_decode_step_persistent(const mbq_decode_model* m, float* h, float* logits, void* workspace,
                               size_t workspace_bytes, void* stream) {
    const char* fn = "mbq_decode_step_persistent";
    int rc = check_decode(m, fn);
    if (rc) return rc;
    if ((rc = check_workspace(m, h, logits, workspace, workspace_bytes, fn))) return rc;
    if (m->d != 4096 || (m->n_layers > 0 && (m->dq != 4096 || m->f != 12288)))
        return fail(MBQ_EUNSUPPORTED, "%s: the one-launch step needs d = dq = 4096 and f = 12288", fn);
    for (int l = 0; l < m->n_layers; l++) {
        const mbq_decode_layer& L = m->layers[l];
        if (L.qkv.fmt != MBQ_FMT_Q45 || L.o.fmt != MBQ_FMT_Q45 || L.gate_up.fmt != MBQ_FMT_Q45 ||
            (L.down.fmt != MBQ_FMT_Q45 && L.down.fmt != MBQ_FMT_Q65))
            return fail(MBQ_EUNSUPPORTED, "%s: layer %d: qkv, o, gate_up must be Q45 and down Q45 or Q65", fn, l);
    }
    if (m->vocab > 0 && m->lm_head.fmt != MBQ_FMT_Q45 && m->lm_head.fmt != MBQ_FMT_Q65)
        return fail(MBQ_EUNSUPPORTED, "%s: lm_head must be Q45 or Q65", fn);
    const DecodeLayout lay = decode_layout(m);
    char* ws = (char*)workspace;
    mbq::DecTable expect;
    memset(&expect, 0, sizeof expect);
    expect.magic = mbq::kDecMagic;
    expect.n_layers = m->n_layers;
    expect.tag = decode_tag(m);
    mbq::DecodeBuffers db{(float*)(ws + lay.hv), (float*)(ws + lay.qkv), (float*)(ws + lay.m),
                          (int64_t)(lay.hs / 4), (int64_t)(lay.qs / 4), (int64_t)(lay.ms / 4)};
    const hipError_t e = mbq::launch_decode_persistent(
        (const mbq::DecTable*)(ws + lay.table), expect, m->eps, h, logits, m->vocab,
        m->dq + 2 * m->dkv, db, (uint32_t*)ws, (uint32_t*)(ws + 4), (hipStream_t)stream);
    if (e == hipErrorInvalidConfiguration)
        return fail(MBQ_EUNSUPPORTED, "%s: the model's row counts or this device's compute-unit count do not fit the one-launch step", fn);
    return hip_status(e, fn);
}

int mbq_decode_step_noalloc(const mbq_decode_model* m, float* h, float* logits, void* stream) {
    const char* fn = "mbq_decode_step_noalloc";
    int rc = check_decode(m, fn);
    if (rc) return rc;
    if (!h || !aligned(h, 16)) return fail(MBQ_EALIGN, "%s: h must be 16-byte aligned", fn);
    if (m->vocab > 0 && (!logits || !aligned(logits, 4))) return fail(MBQ_EINVAL, "%s: bad logits", fn);
    if (m->vocab > 0 && overlaps(logits, (size_t)m->vocab * 4, h, (size_t)m->d * 4))
        return fail(MBQ_EINVAL, "%s: h and logits overlap", fn);
    const size_t qb = align256((size_t)(m->dq + 2 * m->dkv) * 4), mb = align256((size_t)m->f * 4);
    if (qb + mb > kScratchBytes)
        return fail(MBQ_EUNSUPPORTED, "%s: dq + 2 dkv and f need %zu bytes of scratch; the limit is %zu",
                    fn, qb + mb, kScratchBytes);
    void* p = nullptr;
    if ((rc = scratch_of_current_device(&p, fn))) return rc;
    float* qkv = (float*)p;
    float* mm = (float*)((char*)p + qb);
    return hip_status(decode_chain(m, h, logits, qkv, mm, (hipStream_t)stream), fn);
}

int mbq_xq_bytes(int fmt, int64_t M, int64_t K, size_t* bytes) {
    const char* fn = "mbq_xq_bytes";
    if (!fmt_valid(fmt)) return fail(MBQ_EINVAL, "%s: unknown format %d", fn, fmt);
    if (!bytes) return fail(MBQ_EINVAL, "%s: bytes is NULL", fn);
    if (M < 0 || K < 0) return fail(MBQ_EINVAL, "%s: negative shape", fn);
    if (K % xq_chunk(fmt))
        return fail(MBQ_EINVAL, "%s: K=%lld is not a multiple of %lld", fn, (long long)K,
                    (long long)xq_chunk(fmt));
    *bytes = xq_tiled(fmt, M, K) ? (size_t)mbq::xt_bytes(M, K) : (size_t)M * (size_t)K * 4;
    return ok();
}

int mbq_stage_x(int fmt, const float* x, int64_t M, int64_t ldx, int64_t K, void* xq,
                void* stream) {
    const char* fn = "mbq_stage_x";
    size_t xqb = 0;
    int rc = mbq_xq_bytes(fmt, M, K, &xqb);
    if (rc) return fail(rc, "%s: %s", fn, g_err.c_str());
    if (ldx < K) return fail(MBQ_EINVAL, "%s: ldx < K", fn);
    if (M == 0 || K == 0) return ok();
    if (M > 65535) return fail(MBQ_EUNSUPPORTED, "%s: M > 65535", fn);
    if (K > mbq::kMaxK) return fail(MBQ_EUNSUPPORTED, "%s: K > %lld", fn, (long long)mbq::kMaxK);
    if (!x || !xq) return fail(MBQ_EINVAL, "%s: NULL pointer", fn);
    if (!aligned(x, 16) || ldx % 4 || !aligned(xq, 16))
        return fail(MBQ_EALIGN, "%s: x and xq must be 16-byte aligned with ldx %% 4 == 0", fn);
    if (overlaps(x, (size_t)((M - 1) * ldx + K) * 4, xq, xqb))
        return fail(MBQ_EINVAL, "%s: x and xq overlap", fn);
    if (xq_tiled(fmt, M, K))
        return hip_status(mbq::launch_stage_x_mfma(x, M, ldx, K, xq, (hipStream_t)stream), fn);
    return hip_status(mbq::launch_stage_x(fmt, x, M, ldx, K, xq, (hipStream_t)stream), fn);
}

int mbq_gemv_xq(const mbq_qweight* W, const void* xq, int64_t M, float* y, int64_t ldy,
                int accumulate, void* stream) {
    const char* fn = "mbq_gemv_xq";
    int rc = check_weight(W, fn);
    if (rc) return rc;
    if (M < 0) return fail(MBQ_EINVAL, "%s: M < 0", fn);
    if (ldy < W->N) return fail(MBQ_EINVAL, "%s: ldy < N", fn);
    if (accumulate != 0 && accumulate != 1) return fail(MBQ_EINVAL, "%s: accumulate must be 0 or 1", fn);
    if (M == 0 || W->N == 0) return ok();
    if (!xq || !y) return fail(MBQ_EINVAL, "%s: xq or y is NULL", fn);
    if (!aligned(y, 4)) return fail(MBQ_EALIGN, "%s: y must be 4-byte aligned", fn);
    hipStream_t s = (hipStream_t)stream;
    if (W->K == 0) {
        if (accumulate) return ok();
        return hip_status(mbq::launch_fill_zero(y, M, W->N, ldy, s), fn);
    }
    if (!aligned(xq, 16)) return fail(MBQ_EALIGN, "%s: xq must be 16-byte aligned", fn);
    const size_t ybytes = (size_t)((M - 1) * ldy + W->N) * 4;
    const size_t xqb = xq_tiled(W->fmt, M, W->K) ? (size_t)mbq::xt_bytes(M, W->K) : (size_t)(M * W->K) * 4;
    if (overlaps(xq, xqb, y, ybytes)) return fail(MBQ_EINVAL, "%s: xq and y overlap", fn);
    if ((rc = check_planes(W, fn))) return rc;
    if ((rc = check_out_vs_planes(W, y, ybytes, fn))) return rc;
    if ((rc = check_kernel_shape(W, fn))) return rc;
    const mbq::DevPlanes P = planes_of(W);
    if (M == 1) {
        mbq::GemvGeom g = mbq::gemv_m1_default_geom(W->fmt, W->N, W->K);
        geom_override(&g);
        return hip_status(mbq::launch_gemv_m1(W->fmt, P, W->N, W->K, xq, true, y, accumulate,
                                              nullptr, 1, g, s), fn);
    }
    if (xq_tiled(W->fmt, M, W->K)) {
        if (!aligned(W->scales, 8)) return fail(MBQ_EALIGN, "%s: the matrix-core kernel needs 8-byte aligned scales", fn);
        return hip_status(mbq::launch_gemv_mfma_q45(P, W->N, W->K, xq, M, y, ldy, accumulate, s), fn);
    }
    // row form: passes of up to 8 tokens on the vector units
    int64_t mp = M < 8 ? M : 8;
    while (mp > 1 && !mbq::gemv_smallm_fits(W->fmt, mp, W->K)) mp--;
    const uint8_t* xb = (const uint8_t*)xq;
    for (int64_t m0 = 0; m0 < M; m0 += mp) {
        const int64_t mm = M - m0 < mp ? M - m0 : mp;
        const void* xm = xb + m0 * W->K * 4;
        mbq::GemvGeom g1 = mbq::gemv_m1_default_geom(W->fmt, W->N, W->K);
        hipError_t e = mm == 1 ? mbq::launch_gemv_m1(W->fmt, P, W->N, W->K, xm, true, y + m0 * ldy,
                                                     accumulate, nullptr, 1, g1, s)
                               : mbq::launch_gemv_smallm(W->fmt, P, W->N, W->K, xm, true, mm, W->K,
                                                         y + m0 * ldy, ldy, accumulate,
                                                         smallm_geom(W->fmt, mm, W->N), s);
        if (e != hipSuccess) return hip_status(e, fn);
    }
    return ok();
}

int mbq_gemv_xq_workspace_bytes(const mbq_qweight* W, int64_t M, size_t* bytes) {
    const char* fn = "mbq_gemv_xq_workspace_bytes";
    if (!W) return fail(MBQ_EINVAL, "%s: W is NULL", fn);
    if (!bytes) return fail(MBQ_EINVAL, "%s: bytes is NULL", fn);
    if (M < 0 || W->N < 0 || W->K < 0) return fail(MBQ_EINVAL, "%s: negative shape", fn);
    *bytes = mfma_shape(W->fmt, M, W->K) && W->N > 0 && M <= 65535
                 ? mbq::mfma_split_workspace_bytes(W->N, W->K, M) : 0;
    return ok();
}

int mbq_gemv_xq_ws(const mbq_qweight* W, const void* xq, int64_t M, float* y, int64_t ldy,
                   int accumulate, void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "mbq_gemv_xq_ws";
    int rc = check_weight(W, fn);
    if (rc) return rc;
    size_t need = 0;
    if ((rc = mbq_gemv_xq_workspace_bytes(W, M, &need))) return fail(rc, "%s: %s", fn, g_err.c_str());
    if (need == 0) return mbq_gemv_xq(W, xq, M, y, ldy, accumulate, stream);
    if (ldy < W->N) return fail(MBQ_EINVAL, "%s: ldy < N", fn);
    if (accumulate != 0 && accumulate != 1) return fail(MBQ_EINVAL, "%s: accumulate must be 0 or 1", fn);
    if (!xq || !y) return fail(MBQ_EINVAL, "%s: xq or y is NULL", fn);
    if (!workspace) return fail(MBQ_EINVAL, "%s: workspace is NULL", fn);
    if (workspace_bytes < need)
        return fail(MBQ_EINVAL, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, need);
    if (!aligned(y, 4)) return fail(MBQ_EALIGN, "%s: y must be 4-byte aligned", fn);
    if (!aligned(xq, 16) || !aligned(workspace, 256))
        return fail(MBQ_EALIGN, "%s: xq must be 16-byte and workspace 256-byte aligned", fn);
    const size_t ybytes = (size_t)((M - 1) * ldy + W->N) * 4;
    const size_t xqb = (size_t)mbq::xt_bytes(M, W->K);
    if (overlaps(xq, xqb, y, ybytes)) return fail(MBQ_EINVAL, "%s: xq and y overlap", fn);
    if (overlaps(workspace, need, y, ybytes) || overlaps(workspace, need, xq, xqb))
        return fail(MBQ_EINVAL, "%s: the workspace overlaps xq or y", fn);
    if ((rc = check_planes(W, fn))) return rc;
    if ((rc = check_out_vs_planes(W, y, ybytes, fn))) return rc;
    if ((rc = check_out_vs_planes(W, workspace, need, fn))) return rc;
    if ((rc = check_kernel_shape(W, fn))) return rc;
    if (!aligned(W->scales, 8)) return fail(MBQ_EALIGN, "%s: the matrix-core kernel needs 8-byte aligned scales", fn);
    return hip_status(mbq::launch_gemv_mfma_q45_ws(planes_of(W), W->N, W->K, xq, M, y, ldy, accumulate,
                                                   workspace, (hipStream_t)stream), fn);
}

static int check_norm(const float* x, const float* gamma, const float* beta, bool need_beta,
                      float eps, int64_t rows, int64_t n, const float* y, const char* fn) {
    if (rows < 0 || n < 0) return fail(MBQ_EINVAL, "%s: negative shape", fn);
    if (rows > 0x7FFFFFFF) return fail(MBQ_EUNSUPPORTED, "%s: more than 2^31-1 rows", fn);
    if (!(eps >= 0.f) || eps == __builtin_inff()) return fail(MBQ_EINVAL, "%s: eps must be finite and >= 0", fn);
    if (rows == 0 || n == 0) return MBQ_OK;
    if (!x || !gamma || !y || (need_beta && !beta)) return fail(MBQ_EINVAL, "%s: NULL pointer", fn);
    if (!aligned(x, 4) || !aligned(y, 4) || !aligned(gamma, 4) || (need_beta && !aligned(beta, 4)))
        return fail(MBQ_EALIGN, "%s: pointers must be 4-byte aligned", fn);
    const size_t bytes = (size_t)rows * (size_t)n * 4;
    if (x != y && overlaps(x, bytes, y, bytes)) return fail(MBQ_EINVAL, "%s: x and y partially overlap", fn);
    return MBQ_OK;
}

int mbq_rmsnorm(const float* x, const float* gamma, float eps, int64_t rows, int64_t n, float* y,
                void* stream) {
    const char* fn = "mbq_rmsnorm";
    int rc = check_norm(x, gamma, nullptr, false, eps, rows, n, y, fn);
    if (rc) return rc;
    if (rows == 0 || n == 0) return ok();
    return hip_status(mbq::launch_rmsnorm(x, gamma, eps, rows, n, y, (hipStream_t)stream), fn);
}

int mbq_layernorm(const float* x, const float* gamma, const float* beta, float eps, int64_t rows,
                  int64_t n, float* y, void* stream) {
    const char* fn = "mbq_layernorm";
    int rc = check_norm(x, gamma, beta, true, eps, rows, n, y, fn);
    if (rc) return rc;
    if (rows == 0 || n == 0) return ok();
    return hip_status(mbq::launch_layernorm(x, gamma, beta, eps, rows, n, y, (hipStream_t)stream), fn);
}

int mbq_silu_mul(const float* g, const float* u, int64_t n, float* out, void* stream) {
    const char* fn = "mbq_silu_mul";
    if (n < 0) return fail(MBQ_EINVAL, "%s: n < 0", fn);
    if (n == 0) return ok();
    if (!g || !u || !out) return fail(MBQ_EINVAL, "%s: NULL pointer", fn);
    if (!aligned(g, 4) || !aligned(u, 4) || !aligned(out, 4)) return fail(MBQ_EALIGN, "%s: misaligned", fn);
    const size_t b = (size_t)n * 4;
    if ((out != g && overlaps(out, b, g, b)) || (out != u && overlaps(out, b, u, b)))
        return fail(MBQ_EINVAL, "%s: out partially overlaps an input", fn);
    return hip_status(mbq::launch_silu_mul(g, u, n, out, (hipStream_t)stream), fn);
}

// Shape and pointer checks of the producers of staged x.
static int check_xq_out(int fmt, int64_t n, const void* xq, const char* fn) {
    if (!fmt_valid(fmt)) return fail(MBQ_EINVAL, "%s: unknown format %d", fn, fmt);
    if (n % xq_chunk(fmt))
        return fail(MBQ_EINVAL, "%s: n=%lld is not a multiple of %lld", fn, (long long)n,
                    (long long)xq_chunk(fmt));
    if (!xq) return fail(MBQ_EINVAL, "%s: xq is NULL", fn);
    if (!aligned(xq, 16)) return fail(MBQ_EALIGN, "%s: xq must be 16-byte aligned", fn);
    return MBQ_OK;
}

int mbq_rmsnorm_xq(const float* x, const float* gamma, float eps, int64_t n, float* y, int fmt,
                   void* xq, void* stream) {
    const char* fn = "mbq_rmsnorm_xq";
    if (n < 0) return fail(MBQ_EINVAL, "%s: n < 0", fn);
    if (!(eps >= 0.f) || eps == __builtin_inff()) return fail(MBQ_EINVAL, "%s: eps must be finite and >= 0", fn);
    if (n == 0) return ok();
    int rc = check_xq_out(fmt, n, xq, fn);
    if (rc) return rc;
    if (n > 8192) return fail(MBQ_EUNSUPPORTED, "%s: n > 8192", fn);
    if (!x || !gamma) return fail(MBQ_EINVAL, "%s: NULL pointer", fn);
    if (!aligned(x, 16) || !aligned(gamma, 16) || (y && !aligned(y, 16)))
        return fail(MBQ_EALIGN, "%s: x, gamma and y must be 16-byte aligned", fn);
    const size_t b = (size_t)n * 4;
    if (y && x != y && overlaps(x, b, y, b)) return fail(MBQ_EINVAL, "%s: x and y partially overlap", fn);
    if (overlaps(xq, b, x, b) || (y && overlaps(xq, b, y, b)) || overlaps(xq, b, gamma, b))
        return fail(MBQ_EINVAL, "%s: xq overlaps an input or y", fn);
    return hip_status(mbq::launch_rmsnorm_xq(x, gamma, eps, n, y, fmt, xq, (hipStream_t)stream), fn);
}

int mbq_silu_mul_xq(const float* g, const float* u, int64_t n, int fmt, void* xq, void* stream) {
    const char* fn = "mbq_silu_mul_xq";
    if (n < 0) return fail(MBQ_EINVAL, "%s: n < 0", fn);
    if (n == 0) return ok();
    int rc = check_xq_out(fmt, n, xq, fn);
    if (rc) return rc;
    if (n > ((int64_t)1 << 30)) return fail(MBQ_EUNSUPPORTED, "%s: n > 2^30", fn);
    if (!g || !u) return fail(MBQ_EINVAL, "%s: NULL pointer", fn);
    if (!aligned(g, 16) || !aligned(u, 16)) return fail(MBQ_EALIGN, "%s: g and u must be 16-byte aligned", fn);
    const size_t b = (size_t)n * 4;
    if (overlaps(xq, b, g, b) || overlaps(xq, b, u, b)) return fail(MBQ_EINVAL, "%s: xq overlaps an input", fn);
    return hip_status(mbq::launch_silu_mul_xq(g, u, n, fmt, xq, (hipStream_t)stream), fn);
}

int mbq_dequant_f32(const mbq_qweight* W, float* w_out, void* stream) {
    const char* fn = "mbq_dequant_f32";
    int rc = check_weight(W, fn);
    if (rc) return rc;
    if (W->N == 0 || W->K == 0) return ok();
    if (!w_out) return fail(MBQ_EINVAL, "%s: w_out is NULL", fn);
    if (!aligned(w_out, 16)) return fail(MBQ_EALIGN, "%s: w_out must be 16-byte aligned", fn);
    if ((rc = check_planes(W, fn))) return rc;
    if ((rc = check_out_vs_planes(W, w_out, (size_t)(W->N * W->K) * 4, fn))) return rc;
    if ((rc = check_kernel_shape(W, fn))) return rc;
    return hip_status(mbq::launch_dequant(W->fmt, planes_of(W), W->N, W->K, w_out, (hipStream_t)stream), fn);
}

int mbq_unpack_codes(const mbq_qweight* W, uint8_t* codes_out, void* stream) {
    const char* fn = "mbq_unpack_codes";
    int rc = check_weight(W, fn);
    if (rc) return rc;
    if (W->fmt == MBQ_FMT_BF16) return fail(MBQ_EINVAL, "%s: BF16 has no integer codes", fn);
    if (W->N == 0 || W->K == 0) return ok();
    if (!codes_out) return fail(MBQ_EINVAL, "%s: codes_out is NULL", fn);
    if ((rc = check_planes(W, fn))) return rc;
    if ((rc = check_out_vs_planes(W, codes_out, (size_t)(W->N * W->K), fn))) return rc;
    if ((rc = check_kernel_shape(W, fn))) return rc;
    return hip_status(mbq::launch_unpack_codes(W->fmt, planes_of(W), W->N, W->K, codes_out, (hipStream_t)stream), fn);
}

int mbq_quantize(int fmt, const float* w, int64_t N, int64_t K, int64_t ldw, void* const planes[4],
                 void* stream) {
    const char* fn = "mbq_quantize";
    if (!fmt_valid(fmt)) return fail(MBQ_EINVAL, "%s: unknown format %d", fn, fmt);
    if (N < 0 || K < 0) return fail(MBQ_EINVAL, "%s: negative shape", fn);
    if (K % block_len(fmt))
        return fail(MBQ_EINVAL, "%s: K=%lld is not a multiple of the block length %lld", fn,
                    (long long)K, (long long)block_len(fmt));
    if (!planes) return fail(MBQ_EINVAL, "%s: planes is NULL", fn);
    if (N == 0 || K == 0) return ok();
    if (ldw < K) return fail(MBQ_EINVAL, "%s: ldw < K", fn);
    if (fmt == MBQ_FMT_BF16 && K % 8) return fail(MBQ_EUNSUPPORTED, "%s: BF16 needs K %% 8 == 0", fn);
    if (N * (K / 8) > ((int64_t)1 << 39)) return fail(MBQ_EUNSUPPORTED, "%s: N*K above 2^42", fn);
    if (!w) return fail(MBQ_EINVAL, "%s: w is NULL", fn);
    if (!aligned(w, 16) || ldw % 4) return fail(MBQ_EALIGN, "%s: w must be 16-byte aligned with ldw %% 4 == 0", fn);
    size_t sz[4];
    mbq_plane_sizes(fmt, N, K, sz);
    for (int i = 0; i < 4; i++) {
        if (sz[i] && !planes[i]) return fail(MBQ_EINVAL, "%s: a plane the format needs is NULL", fn);
        if (sz[i] && !aligned(planes[i], i < 2 ? 16 : 4))
            return fail(MBQ_EALIGN, "%s: planes 0 and 1 must be 16-byte aligned, 2 and 3 4-byte", fn);
        if (sz[i] && overlaps(w, (size_t)((N - 1) * ldw + K) * 4, planes[i], sz[i]))
            return fail(MBQ_EINVAL, "%s: w and plane %d overlap", fn, i);
        for (int j = 0; j < i; j++)
            if (overlaps(planes[i], sz[i], planes[j], sz[j]))
                return fail(MBQ_EINVAL, "%s: planes %d and %d overlap", fn, j, i);
    }
    const mbq::DevPlanes out{(const uint8_t*)planes[0], (const uint8_t*)planes[1],
                             (const uint8_t*)planes[2], (const uint8_t*)planes[3]};
    return hip_status(mbq::launch_quantize(fmt, w, ldw, N, K, out, (hipStream_t)stream), fn);
}

// Shape checks shared by the two attention entry points.
static int check_attention_shape(int64_t T, int n_heads, int n_kv, int head_dim, const char* fn) {
    if (T < 1) return fail(MBQ_EINVAL, "%s: T must be at least 1 (softmax over no position)", fn);
    if (n_heads < 1 || n_kv < 1 || n_heads % n_kv)
        return fail(MBQ_EINVAL, "%s: n_heads must be a positive multiple of n_kv_heads", fn);
    if (head_dim != mbq::kAttD)
        return fail(MBQ_EUNSUPPORTED, "%s: head_dim %d (kernels for %d only)", fn, head_dim, mbq::kAttD);
    const int G = n_heads / n_kv;
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return fail(MBQ_EUNSUPPORTED, "%s: %d query heads per key/value head (1, 2, 4 or 8)", fn, G);
    if (T > ((int64_t)1 << 26) || n_kv > 65535 || n_heads > 65535)
        return fail(MBQ_EUNSUPPORTED, "%s: T above 2^26 or more than 65535 heads", fn);
    return MBQ_OK;
}

int mbq_attention_workspace_bytes(int64_t T, int n_heads, int n_kv_heads, int head_dim, size_t* bytes) {
    const char* fn = "mbq_attention_workspace_bytes";
    if (!bytes) return fail(MBQ_EINVAL, "%s: bytes is NULL", fn);
    if (int rc = check_attention_shape(T, n_heads, n_kv_heads, head_dim, fn)) return rc;
    *bytes = mbq::attention_workspace_bytes(T, n_heads, n_kv_heads);
    return ok();
}

int mbq_attention_decode(const float* q, const void* k_cache, const void* v_cache, int64_t T,
                         int64_t ld, int n_heads, int n_kv_heads, int head_dim, float* out,
                         void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "mbq_attention_decode";
    if (int rc = check_attention_shape(T, n_heads, n_kv_heads, head_dim, fn)) return rc;
    const int64_t width = (int64_t)n_kv_heads * head_dim;
    if (ld < width) return fail(MBQ_EINVAL, "%s: ld < n_kv_heads * head_dim", fn);
    if (!q || !k_cache || !v_cache || !out || !workspace) return fail(MBQ_EINVAL, "%s: NULL pointer", fn);
    if (!aligned(q, 16) || !aligned(out, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        !aligned(workspace, 16) || ld % 8)
        return fail(MBQ_EALIGN, "%s: buffers must be 16-byte aligned and ld a multiple of 8", fn);
    const size_t need = mbq::attention_workspace_bytes(T, n_heads, n_kv_heads);
    if (workspace_bytes < need)
        return fail(MBQ_EINVAL, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, need);
    const size_t qb = (size_t)n_heads * head_dim * 4, cb = (size_t)((T - 1) * ld + width) * 2;
    if (overlaps(out, qb, q, qb) || overlaps(out, qb, k_cache, cb) || overlaps(out, qb, v_cache, cb) ||
        overlaps(out, qb, workspace, need) || overlaps(workspace, need, q, qb) ||
        overlaps(workspace, need, k_cache, cb) || overlaps(workspace, need, v_cache, cb))
        return fail(MBQ_EINVAL, "%s: out or workspace overlaps another buffer", fn);
    return hip_status(mbq::launch_attention_decode(q, (const uint16_t*)k_cache, (const uint16_t*)v_cache,
                                                   T, ld, n_heads, n_kv_heads, out, (float*)workspace,
                                                   (hipStream_t)stream),
                      fn);
}

int mbq_attention_decode_append(const float* q, const float* k_new, const float* v_new,
                                void* k_cache, void* v_cache, int64_t T, int64_t ld, int n_heads,
                                int n_kv_heads, int head_dim, float* out, void* workspace,
                                size_t workspace_bytes, void* stream) {
    const char* fn = "mbq_attention_decode_append";
    if (T < 0) return fail(MBQ_EINVAL, "%s: T < 0", fn);
    if (int rc = check_attention_shape(T + 1, n_heads, n_kv_heads, head_dim, fn)) return rc;
    const int64_t width = (int64_t)n_kv_heads * head_dim;
    if (ld < width) return fail(MBQ_EINVAL, "%s: ld < n_kv_heads * head_dim", fn);
    if (!q || !k_new || !v_new || !k_cache || !v_cache || !out || !workspace)
        return fail(MBQ_EINVAL, "%s: NULL pointer", fn);
    if (!aligned(q, 16) || !aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(out, 16) ||
        !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(workspace, 16) || ld % 8)
        return fail(MBQ_EALIGN, "%s: buffers must be 16-byte aligned and ld a multiple of 8", fn);
    const size_t need = mbq::attention_workspace_bytes(T + 1, n_heads, n_kv_heads);
    if (workspace_bytes < need)
        return fail(MBQ_EINVAL, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, need);
    const size_t qb = (size_t)n_heads * head_dim * 4, nb = (size_t)width * 4;
    const size_t cb = (size_t)(T * ld + width) * 2;     // rows 0 .. T
    const void* wr[4] = {out, workspace, k_cache, v_cache};
    const size_t wb[4] = {qb, need, cb, cb};
    const void* rd[3] = {q, k_new, v_new};
    const size_t rb[3] = {qb, nb, nb};
    for (int a = 0; a < 4; a++) {
        for (int b = a + 1; b < 4; b++)
            if (overlaps(wr[a], wb[a], wr[b], wb[b]))
                return fail(MBQ_EINVAL, "%s: out, workspace and the caches must not overlap", fn);
        for (int b = 0; b < 3; b++)
            if (overlaps(wr[a], wb[a], rd[b], rb[b]))
                return fail(MBQ_EINVAL, "%s: q, k_new or v_new overlaps a buffer the call writes", fn);
    }
    return hip_status(mbq::launch_attention_append(q, k_new, v_new, (uint16_t*)k_cache,
                                                   (uint16_t*)v_cache, T, ld, n_heads, n_kv_heads,
                                                   out, (float*)workspace, (hipStream_t)stream),
                      fn);
}

int mbq_probe_read(const void* buf, size_t bytes, float* sink, void* stream) {
    const char* fn = "mbq_probe_read";
    if (!buf || !sink) return fail(MBQ_EINVAL, "%s: NULL pointer", fn);
    if (bytes % 16 || !aligned(buf, 16)) return fail(MBQ_EALIGN, "%s: 16-byte granularity", fn);
    return hip_status(mbq::launch_probe_read(buf, bytes, sink, (hipStream_t)stream), fn);
}

int mbq_probe_mixed(const void* distinct, size_t distinct_bytes, const void* shared, size_t shared_bytes,
                    int mode, int blocks, float* sink, void* stream) {
    const char* fn = "mbq_probe_mixed";
    if (mode < 0 || mode > 3) return fail(MBQ_EINVAL, "%s: mode %d", fn, mode);
    if (blocks < 1 || blocks > 4096) return fail(MBQ_EINVAL, "%s: blocks must be 1..4096", fn);
    if (!sink || (mode != 1 && !distinct) || (mode != 0 && !shared))
        return fail(MBQ_EINVAL, "%s: NULL pointer", fn);
    if (distinct_bytes % 1024 || shared_bytes % 1024 || !aligned(distinct, 16) || !aligned(shared, 16))
        return fail(MBQ_EALIGN, "%s: 1 KB granularity, 16-byte aligned buffers", fn);
    return hip_status(mbq::launch_probe_mixed(distinct, distinct_bytes, shared, shared_bytes, mode, blocks,
                                              sink, (hipStream_t)stream),
                      fn);
}

int mbq_probe_copy(void* dst, const void* src, size_t bytes, void* stream) {
    const char* fn = "mbq_probe_copy";
    if (!dst || !src) return fail(MBQ_EINVAL, "%s: NULL pointer", fn);
    if (bytes % 16 || !aligned(dst, 16) || !aligned(src, 16))
        return fail(MBQ_EALIGN, "%s: 16-byte granularity", fn);
    if (overlaps(dst, bytes, src, bytes)) return fail(MBQ_EINVAL, "%s: buffers overlap", fn);
    return hip_status(mbq::launch_probe_copy(dst, src, bytes, (hipStream_t)stream), fn);
}

int mbq_probe_chase_init(void* buf, size_t bytes, uint32_t* entries, void* stream) {
    const char* fn = "mbq_probe_chase_init";
    if (!buf || !entries) return fail(MBQ_EINVAL, "%s: NULL pointer", fn);
    if (bytes < 256) return fail(MBQ_EINVAL, "%s: bytes < 256", fn);
    if (!aligned(buf, 4)) return fail(MBQ_EALIGN, "%s: buf must be 4-byte aligned", fn);
    *entries = mbq::chase_entries(bytes);
    return hip_status(mbq::launch_chase_init(buf, bytes, (hipStream_t)stream), fn);
}

int mbq_probe_chase(const void* buf, uint32_t entries, int64_t hops, uint32_t* sink, void* stream) {
    const char* fn = "mbq_probe_chase";
    if (!buf || !sink) return fail(MBQ_EINVAL, "%s: NULL pointer", fn);
    if (hops < 1) return fail(MBQ_EINVAL, "%s: hops < 1", fn);
    if (entries == 0 || (entries & (entries - 1))) return fail(MBQ_EINVAL, "%s: entries must be a power of two", fn);
    if (!aligned(buf, 4) || !aligned(sink, 4)) return fail(MBQ_EALIGN, "%s: misaligned", fn);
    return hip_status(mbq::launch_chase(buf, entries, hops, sink, (hipStream_t)stream), fn);
}

int mbq_probe_peak(int kind, int64_t iters, float* sink, int64_t* ops, void* stream) {
    const char* fn = "mbq_probe_peak";
    if (kind < MBQ_PEAK_MFMA_F16 || kind > MBQ_PEAK_MFMA_F16_32) return fail(MBQ_EINVAL, "%s: unknown kind %d", fn, kind);
    if (iters < 1 || !sink || !ops) return fail(MBQ_EINVAL, "%s: iters < 1 or NULL pointer", fn);
    if (!aligned(sink, 4)) return fail(MBQ_EALIGN, "%s: sink must be 4-byte aligned", fn);
    *ops = mbq::peak_ops(kind, iters);
    return hip_status(mbq::launch_peak(kind, iters, sink, (hipStream_t)stream), fn);
}

}  // extern "C"
