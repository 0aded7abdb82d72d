/*
 * mbq.h -- C ABI of libmbq: the single-token / small-batch decode step on
 * AMD Instinct MI355X (gfx950).  Block-quantized weights are streamed through
 * matrix-vector products and dequantized in registers; RMSNorm and two-pass
 * LayerNorm reduce rows cooperatively.
 *
 * Sources (web pages, cited by short tag and section):
 *   [one-serial-kernel]  vocodex.ai, "From 22.8 to 42.8 tokens a second
 *                        without touching a matrix multiply"
 *   [mountain-runs]      coderlegion.com S-MoE diary #5, "The Mountain Runs"
 *   [roofline-holds]     research.arkey.ai, "The roofline holds on a second GPU"
 *
 * Conventions for every entry point
 *   - Plain C types only.  Pointers documented as "device" must point to GPU
 *     memory the caller allocated; "host" pointers to CPU memory.  The library
 *     never allocates or frees memory and keeps no state between calls beyond
 *     its loaded code objects and a thread-local error string.
 *   - Device work is enqueued asynchronously on `stream` (a hipStream_t cast
 *     to void*; NULL selects the default stream).  Errors raised while a
 *     kernel runs surface at the caller's next synchronisation.
 *   - Arguments are checked on the host before anything is enqueued.  A
 *     non-zero return means nothing was enqueued, except MBQ_EHIP, which
 *     reports a failed launch.  mbq_last_error() gives the detail.
 *   - Matrices are row-major.  A weight matrix W is N x K (N output rows,
 *     K inputs); its blocks run along K and never span two rows.
 *   - No C++ exception crosses this boundary.
 */
#ifndef MBQ_H
#define MBQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ status */
#define MBQ_OK            0
#define MBQ_EINVAL       (-1) /* null pointer, bad format, bad shape or stride, overlap */
#define MBQ_EALIGN       (-2) /* a pointer lacks the alignment stated below           */
#define MBQ_EUNSUPPORTED (-3) /* valid request this build has no kernel for            */
#define MBQ_EHIP         (-4) /* the HIP runtime reported an error at launch           */

/* ----------------------------------------------------------------- formats
 * Byte budgets per weight follow [roofline-holds] "The Math" (4.5 and 6.5625
 * bits per weight, scales counted) and "The search space" (256 weights in
 * 144 and in 210 bytes); 2- and 4-bit codes are unpacked in registers and
 * never written out unpacked ([mountain-runs] section 3; [roofline-holds]
 * "Hiding, fusing, and keeping the sums busy", Dtypes).  The block structure
 * and bit order are this library's definition of those budgets.
 *
 * Every format is stored as up to four planes, each row-major over rows n:
 *   plane 0 "codes", plane 1 "codes_hi", plane 2 "scales",
 *   plane 3 "super_scales" (unused planes are NULL).
 *
 * MBQ_FMT_BF16  16 bits/weight.  codes: uint16 [N][K], w = float(word << 16).
 * MBQ_FMT_Q45   4.5 bits/weight, blocks of 32.
 *               codes:  uint8 [N][K/2]; weight k is nibble (k & 1) of byte
 *                       k >> 1, low nibble first; q in 0..15
 *               scales: fp16 [N][K/32];  w = s[k >> 5] * (q - 8)
 * MBQ_FMT_Q65   6.5625 bits/weight, sub-blocks of 16, super-blocks of 256.
 *               codes:    uint8 [N][K/2], low 4 bits of q, nibble order as Q45
 *               codes_hi: uint8 [N][K/4], high 2 bits of q.  Each run of 16
 *                         weights g = k >> 4 owns bytes [4g, 4g+4), read as a
 *                         little-endian 32-bit word W; weight r = k & 15 of
 *                         the run keeps its 2 bits at bit pos(r) of W with
 *                         pos = {4, 2, 12, 10, 20, 18, 28, 26,
 *                                0, 6, 8, 14, 16, 22, 24, 30}
 *               scales:       int8 [N][K/16] (signed sub-scale sc)
 *               super_scales: fp16 [N][K/256] (d)
 *               q = lo | hi << 4 in 0..63;  w = d[k >> 8] * sc[k >> 4] * (q - 32)
 * MBQ_FMT_Q25   2.5 bits/weight, blocks of 32.
 *               codes:  uint8 [N][K/4]; weight k is bits 2*(k & 3) of byte k >> 2
 *               scales: fp16 [N][K/32];  w = s[k >> 5] * (q - 2)
 * Every dequantized weight is exactly representable in binary32.
 */
#define MBQ_FMT_BF16 0
#define MBQ_FMT_Q45  1
#define MBQ_FMT_Q65  2
#define MBQ_FMT_Q25  3

/* A weight matrix resident on the device.  All plane pointers are device
 * pointers owned by the caller and must stay valid until the enqueued work
 * has run.  Planes 0 and 1 must be 16-byte aligned, planes 2 and 3 4-byte
 * aligned (MBQ_EALIGN otherwise). */
typedef struct mbq_qweight {
    int32_t fmt;              /* MBQ_FMT_*                                    */
    int32_t reserved;         /* must be 0                                    */
    int64_t N;                /* output rows                                  */
    int64_t K;                /* inputs per row                               */
    const void* codes;        /* plane 0                                      */
    const void* codes_hi;     /* plane 1 (Q65), else NULL                     */
    const void* scales;       /* plane 2 (Q45, Q65, Q25), else NULL           */
    const void* super_scales; /* plane 3 (Q65), else NULL                     */
} mbq_qweight;

/* Bits per weight and block length along K of a format (BF16: 16.0, 1;
 * Q45: 4.5, 32; Q65: 6.5625, 256; Q25: 2.5, 32).  Host only.
 * MBQ_EINVAL for an unknown format or a NULL output. */
int mbq_format_info(int fmt, double* bits_per_weight, int* block_k);

/* Byte size of each of the four planes of an N x K matrix (0 for planes the
 * format does not use).  Their sum is N*K*bits_per_weight/8.  Host only.
 * MBQ_EINVAL for an unknown format, negative sizes or K not a multiple of
 * the block length. */
int mbq_plane_sizes(int fmt, int64_t N, int64_t K, size_t sizes[4]);

/* Host packer ([roofline-holds] "The search space": formats as byte budgets).
 * codes: host, one byte per weight, row-major [N][K] (BF16: uint16 words).
 * scales: host; Q45/Q25 fp16 bit patterns [N][K/32]; Q65 int8 [N][K/16];
 *         NULL for BF16.  super_scales: host fp16 [N][K/256] for Q65, else NULL.
 * planes: host buffers of the sizes mbq_plane_sizes gives (NULL where 0).
 * MBQ_EINVAL if a code does not fit the format's bit width (nothing written
 * is then meaningful), for NULL pointers or a bad shape. */
int mbq_pack(int fmt, int64_t N, int64_t K, const void* codes, const void* scales,
             const void* super_scales, void* const planes[4]);

/* Exact inverse of mbq_pack: planes -> codes (one byte per weight, BF16 uint16
 * words), scales and super_scales as described above.  Host only. */
int mbq_unpack(int fmt, int64_t N, int64_t K, const void* const planes[4],
               void* codes, void* scales, void* super_scales);

/* y[m][n] = sum_k w[n][k] * x[m][k]   (accumulate = 0)
 * y[m][n] += sum_k w[n][k] * x[m][k]  (accumulate = 1, a residual epilogue)
 * for m < M, n < N: the decode-step matrix-vector product
 * ([roofline-holds] "The tensor, the kernel, the token": multiply this tensor
 * by this vector; [mountain-runs] section 3: a wave of lanes owns a row and
 * reads consecutive 16-byte chunks; codes dequantized in registers).
 * W: host pointer to a descriptor of device planes.
 * x: device fp32 [M][ldx], 16-byte aligned, ldx >= K, ldx % 4 == 0.
 * y: device fp32 [M][ldy], 4-byte aligned, ldy >= N; must not overlap x.
 * Arithmetic: weights exact in fp32, fp32 accumulation; the order of the sum
 * is unspecified.  Tokens run on the vector units, up to 8 per launch (as many
 * as fit staged in LDS: all 8 for K = 4096, 2 for K = 12288), each weight
 * read once per launch and unpacked once for all its tokens.  Q45 batches of
 * 4 or more tokens with K % 128 == 0 (and 8-byte aligned scales) run on the
 * matrix cores instead, all tokens in one launch, with x split into fp16
 * high and low parts under a power of two per 32-weight block and token (the
 * relative precision of the vector units' staged x); the same holds through
 * mbq_stage_x + mbq_gemv_xq.
 * MBQ_EUNSUPPORTED for shapes without a kernel (K > 32768, or K > 16384 for
 * BF16; Q25 with K % 64 != 0; BF16 with K % 8 != 0).  M == 0 or N == 0
 * enqueue nothing; K == 0 writes zeros (or leaves y for accumulate = 1). */
int mbq_gemv_q(const mbq_qweight* W, const float* x, int64_t M, int64_t ldx,
               float* y, int64_t ldy, int accumulate, void* stream);

/* Selected experts in one launch ([mountain-runs] section 3: the expert FFN
 * kernels with 2/4-bit codes; section 1: enough workgroups for the job).
 * W_all stacks E experts of rows_per_expert rows each along N
 * (W_all->N = E * rows_per_expert).  idx: device int32 [n_sel] expert ids;
 * ids are not checked on the device and an id outside [0, E) is the caller's
 * error.  x: device fp32 [K], 16-byte aligned.  y: device fp32
 * [n_sel][rows_per_expert]; y[e][r] = sum_k W_all[idx[e]*R + r][k] * x[k].
 * Same format and K limits as mbq_gemv_q with M = 1. */
int mbq_gemv_q_gather(const mbq_qweight* W_all, int64_t rows_per_expert,
                      const int32_t* idx, int64_t n_sel, const float* x,
                      float* y, void* stream);

/* ---------------------------------------------------------- fused products
 * One launch that does the work of several small kernels between weight
 * reads ([roofline-holds] "Hiding, fusing, and keeping the sums busy";
 * "Where the time goes": the norms and adds between the weight kernels).
 *
 * mbq_gemv_fused: M = 1.
 *   gamma == NULL:  a = x;  else a = rmsnorm(x; gamma, eps) (as mbq_rmsnorm),
 *                   computed inside every workgroup of the product.  With
 *                   the store and accumulate epilogues the 1/rms factor
 *                   multiplies each row's sum, W[n] . (gamma x) / rms, which
 *                   is W[n] . a up to rounding (one rounding per output in
 *                   place of one per element of a).
 *   epilogue MBQ_EPI_STORE:      y[n]  = W[n] . a,           n < N
 *            MBQ_EPI_ACCUMULATE: y[n] += W[n] . a            (residual add)
 *            MBQ_EPI_SILU_MUL:   y[i]  = silu(W[2i] . a) * (W[2i+1] . a),
 *                                i < N/2: W holds the gate and up rows of a
 *                                gated feed-forward interleaved (N even).
 * x: device fp32 [K], 16-byte aligned; gamma: device fp32 [K], 16-byte
 * aligned, or NULL; y: device fp32, 4-byte aligned, overlapping neither.
 * With a norm or the silu epilogue only Q45 and Q65 with K = 4096 or 12288
 * have kernels (MBQ_EUNSUPPORTED otherwise); without them every shape of
 * mbq_gemv_q with M = 1 is accepted. */
#define MBQ_EPI_STORE      0
#define MBQ_EPI_ACCUMULATE 1
#define MBQ_EPI_SILU_MUL   2

int mbq_gemv_fused(const mbq_qweight* W, const float* x, const float* gamma, float eps,
                   int epilogue, float* y, void* stream);

/* ----------------------------------------------------------- decode step
 * One token through a stack of decoder layers with attention left out: the
 * weight stream whose rate the pages bound by BW/B ([roofline-holds] "The
 * Math": tokens per second <= memory bandwidth / bytes read per token; "The
 * tensor, the kernel, the token").  Per layer, with a = rmsnorm(h, gamma1),
 * b = rmsnorm(h, gamma2):
 *     q|k|v = Wqkv a;   h += Wo q   (q stands in for the attention output;
 *                                    k and v are computed and not consumed)
 *     h += Wdown (silu(Wgate b) * (Wup b))
 * then logits = Wlm rmsnorm(h, gamma_f).  Four launches per layer: the norms
 * run inside the qkv and gate/up products, silu * up in the gate/up product's
 * epilogue, both residual adds in the o and down products' epilogues.
 *
 * Weights (device planes, caller-owned):
 *   qkv     (dq + 2 dkv) x d: the q rows, then k, then v
 *   o       d x dq
 *   gate_up 2f x d: row 2i is gate row i, row 2i+1 is up row i
 *   down    d x f
 *   lm_head vocab x d
 * qkv, gate_up and lm_head need fused kernels (Q45/Q65, d = 4096 or 12288).
 * gamma1, gamma2, gamma_f: device fp32 [d], 16-byte aligned.
 * h: device fp32 [d], 16-byte aligned, updated in place; logits: device fp32
 * [vocab].  workspace: device, 256-byte aligned, at least
 * mbq_decode_workspace_bytes bytes, not overlapping h or logits; it holds
 * q|k|v and the gated activations (the launch chain uses the first layer's
 * slots; the one-launch step below uses all of them). */
typedef struct mbq_decode_layer {
    mbq_qweight qkv;
    mbq_qweight o;
    mbq_qweight gate_up;
    mbq_qweight down;
    const float* gamma1;
    const float* gamma2;
} mbq_decode_layer;

typedef struct mbq_decode_model {
    int32_t n_layers;
    float eps;
    int64_t d, dq, dkv, f, vocab;
    const mbq_decode_layer* layers;   /* host array of n_layers */
    const float* gamma_f;
    mbq_qweight lm_head;
} mbq_decode_model;

int mbq_decode_workspace_bytes(const mbq_decode_model* model, size_t* bytes);
int mbq_decode_step(const mbq_decode_model* model, float* h, float* logits, void* workspace,
                    size_t workspace_bytes, void* stream);

/* The decode step with attention over per-layer KV caches in place of the
 * stand-in ([roofline-holds] "Said before the run": a token of a loaded
 * conversation also reads every earlier position's keys and values).  Per
 * layer l, with T positions already cached:
 *     q|k|v = Wqkv rmsnorm(h, gamma1)
 *     K_l[T] = fp16(k), V_l[T] = fp16(v)       (nearest even)
 *     att = attention(q, K_l[0 .. T], V_l[0 .. T])   (as mbq_attention_decode,
 *                                                      T + 1 positions)
 *     h += Wo att;  h += Wdown (silu(Wgate b) * (Wup b)), b = rmsnorm(h, gamma2)
 * then logits as in mbq_decode_step.  Six launches per layer: the four of
 * mbq_decode_step and the two of mbq_attention_decode_append between the qkv
 * and o products.  The heads are dq / 128 query heads on dkv / 128
 * key/value heads (head size 128, 1, 2, 4 or 8 query heads per key/value
 * head; MBQ_EUNSUPPORTED otherwise).
 * k_caches, v_caches: host arrays of n_layers device pointers to fp16
 * caches, 16-byte aligned, row t at t * ld elements (ld >= dkv, a multiple
 * of 8), room for at least T + 1 rows; row T of each is written, rows
 * 0 .. T-1 are read.  The caches must not overlap h, logits, the workspace
 * or each other.  workspace: device, 256-byte aligned, at least
 * mbq_decode_kv_workspace_bytes(model, T) bytes (q|k|v, the gated
 * activations, the attention output and its partial records; contents
 * need no initialisation).  h, logits: as for mbq_decode_step.  MBQ_EINVAL
 * for T < 0. */
int mbq_decode_kv_workspace_bytes(const mbq_decode_model* model, int64_t T, size_t* bytes);
int mbq_decode_step_kv(const mbq_decode_model* model, float* h, float* logits,
                       void* const* k_caches, void* const* v_caches, int64_t T, int64_t ld,
                       void* workspace, size_t workspace_bytes, void* stream);

/* mbq_decode_step for callers that cannot allocate device memory (code under
 * HIP graph capture that may not call hipMalloc, tight serving loops,
 * harnesses that forbid allocation): the same launches, kernels and
 * results bit for bit, with no workspace argument.  q|k|v and the gated
 * activations live in a device array inside the library, 1 MiB per GPU,
 * held until the process ends: align256(4 (dq + 2 dkv)) + align256(4 f)
 * must fit in it (MBQ_EUNSUPPORTED otherwise).  Every call on a GPU shares
 * that GPU's array, so calls that overlap on one GPU (two streams, two
 * threads) race; calls on one stream are ordered.  Nothing in the array
 * needs to start at zero: each step writes q|k|v and the activations before
 * it reads them.  h, logits: as for mbq_decode_step.  Allocates nothing. */
int mbq_decode_step_noalloc(const mbq_decode_model* model, float* h, float* logits, void* stream);

/* The same token in ONE launch ([one-serial-kernel] "The kernel that was never
 * built": the token's pieces of work without a return to the host between
 * them; [roofline-holds] "Where the time goes": the per-kernel toll).  Every
 * workgroup stays resident (cooperative launch, one per compute unit); the
 * four steps of a layer and the vocabulary product are phases separated by
 * grid-wide barriers.  Each compute wave walks one stream of weight chunks
 * through all phases and keeps its next chunks in flight across every
 * barrier, so the weight stream does not stop between tables; one control
 * wave per workgroup applies each phase's epilogue, meets the barrier and
 * brings the next input into LDS.  Same arithmetic and the same results
 * within tolerance as mbq_decode_step (the norm is computed inside every
 * workgroup; a row's sum may be split between two waves).
 *
 * mbq_decode_prepare writes the device table of the layers and the
 * vocabulary product into the workspace (a copy and a stream
 * synchronisation; call it once per model and again whenever a descriptor
 * changes).  mbq_decode_step_persistent checks that the workspace holds the
 * table of this model (by an identity of its pointers) and does nothing but
 * set the status word otherwise.  The workspace also holds each layer's
 * q|k|v and gated activations and two versions of h per layer: every
 * activation that crosses workgroups is written once per token.
 * Needs d = dq = 4096, f = 12288, Q45 qkv / o / gate_up, Q45 or Q65 down
 * and lm_head, and row counts that fit the device (MBQ_EUNSUPPORTED).
 * After the step the 32-bit word at byte 4 of the workspace is 0 on success,
 * bit 0 set if a barrier wait gave up (every wave still ends), bit 1 set if
 * the table did not match.  Not for graph capture (cooperative launch). */
int mbq_decode_prepare(const mbq_decode_model* model, void* workspace, size_t workspace_bytes,
                       void* stream);
int mbq_decode_step_persistent(const mbq_decode_model* model, float* h, float* logits,
                               void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------ staged x
 * The quantized products consume x in a "staged" form: per chunk of 32
 * values (64 for Q25) a power-of-two scale 2^-e and the 24-bit integers
 * n = rint(x * 2^e) split into three byte digits, laid out in the order of the
 * format's code vectors, plus the offset terms of each block.  e is chosen so
 * the chunk's largest |x| lies in [2^21, 2^22) (x is rounded to 22 bits
 * relative to its chunk maximum; nothing else is rounded before the fp32
 * sums).  Staging once in the kernel that produces x, instead of in every
 * workgroup of the product, is the fusion of the small kernels between weight
 * reads into their neighbours ([roofline-holds] "Hiding, fusing, and keeping
 * the sums busy").  The form is opaque and format-specific: stage for the
 * format of the matrix that consumes it.  It takes 4 bytes per value
 * (mbq_xq_bytes), rows back to back; for BF16 it is x itself in fp32.
 * For Q45 with M >= 4 tokens and K % 128 == 0 it is the matrix-core tile
 * form instead: per tile of 16 tokens and block of 32 values, each token's
 * block scaled by a power of two (its largest |x| in [2^14, 2^15)) and split
 * into fp16 high and low parts in the MFMA operand order, then the blocks'
 * exponents as bytes (mbq_xq_bytes gives its size).
 */

/* Bytes of staged x for M rows of K values: 4*M*K, or for the Q45 tile form
 * (M >= 4, K % 128 == 0) ceil(M/16) * (K/32 * 2048 + K/128 * 64).
 * Host only.  MBQ_EINVAL for an unknown
 * format or K not a multiple of the chunk (32; Q25 64; BF16 8). */
int mbq_xq_bytes(int fmt, int64_t M, int64_t K, size_t* bytes);

/* xq = staged form of x for fmt.  x: device fp32 [M][ldx], 16-byte aligned,
 * ldx % 4 == 0, ldx >= K.  xq: device, mbq_xq_bytes(fmt, M, K) bytes, 16-byte
 * aligned, not overlapping x.  K <= 32768, M <= 65535 (MBQ_EUNSUPPORTED). */
int mbq_stage_x(int fmt, const float* x, int64_t M, int64_t ldx, int64_t K, void* xq,
                void* stream);

/* mbq_gemv_q with x given in staged form (staged for W->fmt, M rows of K):
 * the same products, sums and limits.  With the row form the result is bit
 * for bit mbq_gemv_q's on the same x.  Q45 in the tile form runs on
 * the matrix cores ([roofline-holds] "The Math": past M* the sums, not the
 * bytes, bound the product): fp16 (q - 8) codes, which are exact, against
 * the fp16 high and low parts of x, fp32 results, each block's scale and
 * 2^-e applied to its fp32 block sum; it needs 8-byte aligned scales.
 * xq: device, 16-byte aligned, must not overlap y. */
int mbq_gemv_xq(const mbq_qweight* W, const void* xq, int64_t M, float* y, int64_t ldy,
                int accumulate, void* stream);

/* Bytes of workspace mbq_gemv_xq_ws takes for W and M tokens: 0 where it
 * does not split (then it is mbq_gemv_xq).  Host only.  MBQ_EINVAL for a
 * NULL W or bytes, or a negative shape. */
int mbq_gemv_xq_workspace_bytes(const mbq_qweight* W, int64_t M, size_t* bytes);

/* mbq_gemv_xq for the matrix-core tile form with K split across workgroups
 * ([roofline-holds] "The Math": the weights are read once whatever the
 * batch; here each compute unit also reads only a share of the batch's x).
 * S workgroups (S = 2 or 4) each cover S times the rows over 1/S of K and
 * write their partial tile into the workspace; the last of them to finish
 * adds the S partials in fixed order, so the result does not depend on
 * timing.  Same sums as mbq_gemv_xq up to the rounding of that split (not
 * bit for bit).  Where mbq_gemv_xq_workspace_bytes is 0 this is mbq_gemv_xq
 * and the workspace is not touched.
 * workspace: device, 256-byte aligned, at least mbq_gemv_xq_workspace_bytes
 * bytes, overlapping none of xq, y and W's planes; it must be all zero before
 * the first call (hipMemset once), and every call leaves it all zero.  Calls
 * that overlap in time on one workspace race.  Other arguments and errors as
 * mbq_gemv_xq; MBQ_EINVAL for a small workspace. */
int mbq_gemv_xq_ws(const mbq_qweight* W, const void* xq, int64_t M, float* y, int64_t ldy,
                   int accumulate, void* workspace, size_t workspace_bytes, void* stream);

/* RMSNorm of one row of n values (as mbq_rmsnorm) that also writes its output
 * in staged form for fmt: the norm before a product, fused with the staging of
 * the product's input.  y: device fp32 [n] or NULL (then only xq is written);
 * y == x allowed.  x, gamma, y 16-byte aligned; n a multiple of the chunk and
 * <= 8192; xq as in mbq_stage_x, overlapping none of x, gamma, y. */
int mbq_rmsnorm_xq(const float* x, const float* gamma, float eps, int64_t n, float* y, int fmt,
                   void* xq, void* stream);

/* xq = staged form for fmt of silu(g) * u (as mbq_silu_mul, same arithmetic):
 * the gated glue fused with the staging of the down product's input.
 * g, u: device fp32 [n], 16-byte aligned; n a multiple of the chunk. */
int mbq_silu_mul_xq(const float* g, const float* u, int64_t n, int fmt, void* xq, void* stream);

/* RMSNorm of each row: y = gamma * x / sqrt(mean(x^2) + eps), one 256-thread
 * workgroup per row ([one-serial-kernel] "One thread": many threads share the
 * row, each sums its part, the parts are combined across the group).
 * x, y: device fp32 [rows][n]; gamma: device fp32 [n]; all 4-byte aligned.
 * y == x (in place) is allowed; any other overlap is MBQ_EINVAL.
 * eps must be finite and >= 0. */
int mbq_rmsnorm(const float* x, const float* gamma, float eps, int64_t rows,
                int64_t n, float* y, void* stream);

/* LayerNorm of each row in two passes, the mean first and then the biased
 * variance of the centred values ([one-serial-kernel] "One thread"):
 * y = (x - mean) / sqrt(var + eps) * gamma + beta.  Same layout, aliasing
 * and eps rules as mbq_rmsnorm; beta: device fp32 [n]. */
int mbq_layernorm(const float* x, const float* gamma, const float* beta, float eps,
                  int64_t rows, int64_t n, float* y, void* stream);

/* out[i] = silu(g[i]) * u[i], silu(t) = t / (1 + exp(-t)): the gated glue
 * between the gate/up and down products of a decode layer ([roofline-holds]
 * "Where the time goes": the small kernels between weight reads).
 * g, u, out: device fp32 [n]; out may equal g or u. */
int mbq_silu_mul(const float* g, const float* u, int64_t n, float* out, void* stream);

/* Device decode exports for bit-exact checks of the in-register unpack.
 * mbq_dequant_f32: w_out device fp32 [N][K] = every dequantized weight.
 * mbq_unpack_codes: codes_out device uint8 [N][K] = every integer code
 * (MBQ_EINVAL for BF16, which has none).  Same format limits as mbq_gemv_q. */
int mbq_dequant_f32(const mbq_qweight* W, float* w_out, void* stream);
int mbq_unpack_codes(const mbq_qweight* W, uint8_t* codes_out, void* stream);

/* One new token's attention over an fp16 KV cache ([roofline-holds] "Said
 * before the run": each token also reads the keys and values of the loaded
 * conversation, 75.5 MB at 512 positions for the 36-layer model, i.e. 2-byte
 * values, 1024 per position and layer for each of K and V).  The pages name
 * no positional encoding or normalisation; the reading here is plain scaled
 * dot-product attention with grouped key/value heads:
 *   query head h (0 <= h < n_heads) reads key/value head g = h / G,
 *   G = n_heads / n_kv_heads;
 *   s_t = q_h . k_{t,g} / sqrt(head_dim);  p_t = exp(s_t - max_t s) / sum;
 *   out_h = sum_t p_t v_{t,g},  t = 0 .. T-1.
 * q: device fp32 [n_heads][head_dim]; k_cache, v_cache: device fp16 bit
 * patterns, position t's row at t * ld elements, head g at g * head_dim
 * within it; out: device fp32 [n_heads][head_dim].  workspace: device,
 * caller-owned, at least mbq_attention_workspace_bytes (partial maxima, sums
 * and value sums per chunk of positions; contents need no initialisation and
 * are meaningless afterwards).  Arithmetic in fp32.  Every pointer 16-byte
 * aligned, ld a multiple of 8 (MBQ_EALIGN).  MBQ_EINVAL for T < 1, ld <
 * n_kv_heads * head_dim, n_heads not a multiple of n_kv_heads, NULL or
 * overlapping buffers, a short workspace; MBQ_EUNSUPPORTED for head_dim !=
 * 128, G not in {1, 2, 4, 8}, T > 2^26. */
int mbq_attention_workspace_bytes(int64_t T, int n_heads, int n_kv_heads, int head_dim, size_t* bytes);
int mbq_attention_decode(const float* q, const void* k_cache, const void* v_cache, int64_t T,
                         int64_t ld, int n_heads, int n_kv_heads, int head_dim, float* out,
                         void* workspace, size_t workspace_bytes, void* stream);

/* mbq_attention_decode for a token whose own key and value are not cached
 * yet (the decode step's order: the new position is stored, then attended
 * to).  k_new, v_new: device fp32 [n_kv_heads][head_dim], 16-byte aligned:
 * they are rounded to fp16 (nearest even) and written to row T of k_cache
 * and v_cache, and the attention covers rows 0 .. T (T + 1 positions; T >= 0
 * cached positions before the call, so the caches need room for T + 1
 * rows).  One fused step: the partial launch takes the new position from
 * k_new / v_new and its owning lanes store the row; whatever row T held
 * before the call is never used.  workspace: at least mbq_attention_workspace_bytes
 * for T + 1 positions.  out, the workspace and the caches' rows 0 .. T must
 * not overlap one another or q, k_new, v_new (MBQ_EINVAL); other arguments
 * and errors as for mbq_attention_decode. */
int mbq_attention_decode_append(const float* q, const float* k_new, const float* v_new,
                                void* k_cache, void* v_cache, int64_t T, int64_t ld, int n_heads,
                                int n_kv_heads, int head_dim, float* out, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Device quantizer: fp32 weights w [N][ldw] (device, 16-byte aligned, ldw a
 * multiple of 4, ldw >= K) -> the planes of format fmt (device pointers in
 * planes[0..3], sizes and alignment as for mbq_qweight; NULL where
 * mbq_plane_sizes gives 0).  The pages fix each format by its byte budget
 * ([roofline-holds] "The Math"; "The search space"); the rule that picks
 * codes and scales is this library's, with every decision in fp32:
 *   Q45, Q25 (blocks of 32): s = half(max|w| / Qmax), Qmax = 7 or 1;
 *       q = clamp(rint(w / s) + off, 0, 2^b - 1), off = 8 or 2 (q = off
 *       where s = 0);
 *   Q65 (super-blocks of 256, sub-blocks of 16): a_j = max_j|w| / 31,
 *       d = half(max_j a_j / 127), sc_j = clamp(rint(a_j / d), -128, 127)
 *       (0 where d = 0), q = clamp(rint(w / (d sc_j)) + 32, 0, 63) (32
 *       where d sc_j = 0);
 *   BF16: round to nearest even.
 * half() rounds to binary16 nearest-even and saturates at 65504; division
 * is correctly rounded fp32, rint rounds half to even.  One pass over w
 * (4 bytes per weight read, bits/8 written).  MBQ_EINVAL for an unknown
 * format, K not a multiple of the block length, NULL or overlapping
 * buffers; MBQ_EALIGN as stated; MBQ_EUNSUPPORTED for BF16 with K % 8 != 0
 * or N*K above 2^42. */
int mbq_quantize(int fmt, const float* w, int64_t N, int64_t K, int64_t ldw, void* const planes[4],
                 void* stream);

/* Measurement kit ([roofline-holds] "The Math" and "How I ran it": measure
 * the ceiling, never quote it; a large in-device copy counts read and write).
 * mbq_probe_read: reads `bytes` (a multiple of 16, buffer 16-byte aligned)
 * and writes one float per workgroup into sink (device, >= 4096 floats).
 * mbq_probe_copy: copies `bytes` (multiple of 16, both 16-byte aligned). */
int mbq_probe_read(const void* buf, size_t bytes, float* sink, void* stream);
int mbq_probe_copy(void* dst, const void* src, size_t bytes, void* stream);

/* Per-compute-unit streams: `blocks` workgroups of 16 waves (one per compute
 * unit); workgroup b reads distinct_bytes of `distinct` from b *
 * distinct_bytes on (the buffer holds blocks * distinct_bytes) and
 * shared_bytes of `shared`, which every workgroup reads (it stays in L2).
 * mode 0: distinct only; 1: shared only; 2: both, each wave interleaving
 * 1 KB of distinct data with its share of shared data; 3: both, waves 0-3
 * on distinct data, 4-15 on shared.  Timing modes 0 and 1 against 2 and 3
 * shows whether a unit's HBM and L2 streams overlap or queue behind each
 * other.  Sizes multiples of 1 KB, buffers 16-byte aligned; sink: device,
 * >= blocks floats.  MBQ_EINVAL for a bad mode or block count. */
int mbq_probe_mixed(const void* distinct, size_t distinct_bytes, const void* shared, size_t shared_bytes,
                    int mode, int blocks, float* sink, void* stream);

/* Memory latency ([roofline-holds] "How the breakouts tie out: Little and
 * Volkov": bytes in flight = bandwidth x latency): a dependent random
 * pointer chase.  mbq_probe_chase_init writes a chain of *entries =
 * the largest power of two <= bytes / 256 entries into buf (device, 4-byte
 * aligned, >= 256 bytes), one entry per 256 bytes, visiting every entry once
 * per cycle in a scattered order.  mbq_probe_chase follows `hops` >= 1 hops
 * of a chain of `entries` entries (the value the init call returned) with one
 * lane, each hop one full memory round trip, starting at the entry *sink
 * holds (device uint32, reduced modulo entries) and leaving the entry it
 * reached in *sink, so consecutive calls walk on into entries no cache holds.
 * Time it with events: latency = time / hops.  MBQ_EINVAL for bytes < 256,
 * hops < 1 or entries not a power of two. */
int mbq_probe_chase_init(void* buf, size_t bytes, uint32_t* entries, void* stream);
int mbq_probe_chase(const void* buf, uint32_t entries, int64_t hops, uint32_t* sink, void* stream);

/* Issue-rate loops for the arithmetic ceilings ([roofline-holds] "The
 * Math": M* = (w/16)(R/BW) needs the measured rate R; "How I ran it": peak
 * loops with no memory traffic).  kind MBQ_PEAK_MFMA_F16 and
 * MBQ_PEAK_MFMA_F16_32: fp16 matrix instructions (16x16x32 and 32x32x16,
 * fp32 accumulate); MBQ_PEAK_FMA_F32: fp32 fused
 * multiply-add on the vector units (the packed two-wide form is not used in
 * this library's code); MBQ_PEAK_DOT4_I8: the 4-way byte dot product the
 * quantized vector kernels use.  Each launch runs `iters` >= 1 rounds on
 * every wave; *ops (host) receives the operations executed (flops: two per
 * multiply-add).  sink: device fp32, >= 2048 floats. */
#define MBQ_PEAK_MFMA_F16 0      /* 16x16x32 instructions */
#define MBQ_PEAK_FMA_F32  1
#define MBQ_PEAK_DOT4_I8  2
#define MBQ_PEAK_MFMA_F16_32 3   /* 32x32x16 instructions */
int mbq_probe_peak(int kind, int64_t iters, float* sink, int64_t* ops, void* stream);

/* Static text for a status code, and the calling thread's last error detail
 * (empty string if none). */
const char* mbq_status_str(int status);
const char* mbq_last_error(void);

/* Library ABI version (this header: 1). */
int mbq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MBQ_H */
