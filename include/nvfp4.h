/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 hot path: block-scaled FP4
 * quantization and the W4A4 matrix product it feeds.
 *
 * Format (ARCQuant article on zizhi168.cn, section 1; abstract of "Replay the
 * Curvature: Accurate and Scalable NVFP4 Quantization for Large Language Model
 * Inference"): each value is an E2M1 code, every 16 consecutive values along K
 * share one E4M3 block scale, and one FP32 scale S covers the whole tensor.
 *
 * Canonical storage of an NVFP4 tensor with `rows` rows and K columns:
 *   codes  : rows x ld_codes bytes; byte j of a row holds code(2j) in its low
 *            nibble and code(2j+1) in its high nibble; a code is
 *            sign (bit 3) | E2M1 magnitude index (bits 2..0; 0,0.5,1,1.5,2,3,4,6)
 *   scales : rows x ld_scales bytes; byte b of a row is the E4M3 scale of
 *            columns [16b, 16b+16)
 *   S      : one float in device memory (so a dynamic scale needs no host sync)
 * The value of an element is e(code) * d(scale) * S.
 *
 * Tiled storage (weights; layout = NVFP4_LAYOUT_TILED), the order in which the
 * decode product reads them, so that each of its loads is one contiguous 1 KiB
 * run. The tensor is cut into items of 16 rows x 512 columns; item (t, u)
 * (rows [16t, 16t+16), columns [512u, 512u+512)) lives at codes + t*ld_codes +
 * u*4096 and scales + t*ld_scales + u*512, with ld_codes = KU*4096,
 * ld_scales = KU*512, KU = ceil(K/512). Inside an item, for p = 0..63 with
 * r = p % 16, g = p / 16:
 *   codes  byte 1024*i + 16*p + j  (i, j < 4 / 16) = byte j of the canonical
 *          codes of row 16t+r starting at column 512u + 128g + 32i;
 *   scales byte 8*p + b  (b < 8) = the block scale of row 16t+r, columns
 *          512u + 128g + 16b .. +16.
 * Rows >= rows and columns >= K are zero codes with zero scales.
 *
 * Quantization rule (the pages fix the format, not the rounding; this is the
 * reading implemented, and the CPU oracle implements the same rule):
 *   S  = amax(tensor) / 2688 (2688 = 6 * 448), or 1 for an all-zero tensor,
 *        or the caller's static scale;
 *   d  = E4M3(amax(block) / (6 S)), round to nearest even, saturating at 448;
 *   q  = x * (1 / (d S)) in FP32 (0 when d S = 0);
 *   code = E2M1(|q|) round to nearest even, saturating at 6, sign bit of x.
 *
 * Conventions for every entry point:
 *  - All buffer pointers are DEVICE pointers unless the name says host.
 *    `stream` is a hipStream_t (NULL = the default stream); every call only
 *    enqueues work on it and returns without synchronizing.
 *  - The caller owns and allocates every buffer, including the workspace
 *    (size from nvfp4_workspace_size). The library never allocates device
 *    memory. The first 8 KiB of every workspace hold counters (the one-launch
 *    quantizers' arrival slots, the decode product's split-K
 *    tile counters): they must be zero before the first call on a workspace;
 *    calls keep them valid, so they never need clearing again. A workspace
 *    must not be used by two calls at the same time.
 *  - Argument errors are detected before anything is enqueued; the call then
 *    returns a status != NVFP4_OK and leaves every output untouched. Launch
 *    failures return NVFP4_ERR_HIP; nvfp4_last_error() gives the HIP text.
 *  - Alignment: codes rows must start on 16-byte boundaries (codes pointer and
 *    ld_codes multiples of 16) and scales rows on 8-byte boundaries (pointer
 *    and ld_scales multiples of 8), else NVFP4_ERR_ALIGN (the ARCQuant article,
 *    section 6.3, asks for 16-byte aligned tensor dimensions). Activation
 *    rows (x, ldx) must be 16-byte aligned; K must be a multiple of 16.
 *  - Inputs must be finite; inputs and outputs must not alias. Calls on one
 *    workspace must be ordered (same stream or synchronized).
 *  - Results are deterministic: the same inputs give bit-identical outputs.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NVFP4_OK = 0,
    NVFP4_ERR_NULL = 1,         /* a required pointer is NULL                        */
    NVFP4_ERR_SHAPE = 2,        /* inconsistent or unsupported sizes                 */
    NVFP4_ERR_ALIGN = 3,        /* pointer or leading dimension misaligned           */
    NVFP4_ERR_DTYPE = 4,        /* unknown dtype code                                */
    NVFP4_ERR_WORKSPACE = 5,    /* workspace missing or smaller than required        */
    NVFP4_ERR_UNSUPPORTED = 6,  /* valid request this build does not implement       */
    NVFP4_ERR_HIP = 7           /* the HIP runtime reported an error                 */
} nvfp4_status;

typedef enum { NVFP4_BF16 = 0, NVFP4_FP32 = 1 } nvfp4_dtype;

typedef enum { NVFP4_LAYOUT_ROWMAJOR = 0, NVFP4_LAYOUT_TILED = 1 } nvfp4_layout;

/* One NVFP4 tensor (rows x K, K % 16 == 0) in the canonical (row-major)
 * layout, or -- for the weight operand of the products only -- the tiled one. */
typedef struct {
    uint8_t *codes;        /* device; row-major: rows x ld_codes bytes       */
    int64_t  ld_codes;     /* row-major: bytes between rows, >= K/2, multiple
                              of 16; tiled: KU*4096 (bytes per 16-row strip) */
    uint8_t *scales;       /* device; row-major: rows x ld_scales bytes      */
    int64_t  ld_scales;    /* row-major: >= K/16, multiple of 8; tiled: KU*512 */
    float   *tensor_scale; /* device, 1 float                                */
    int64_t  rows;
    int64_t  K;
    int32_t  layout;       /* nvfp4_layout                                    */
} nvfp4_tensor;

/* Options of the fused quantizer (ARCQuant article, section 3.2: channel
 * reorder + RMSNorm + main quantization + residual quantization in one kernel). */
typedef struct {
    const void    *gamma;          /* RMSNorm weight, bf16 device [K_in], or NULL = no norm.
                                      y = fl(fl(x*r)*gamma), r = 1/sqrt(mean(x^2)+eps) with
                                      the sum of squares in FP64 and r rounded to FP32   */
    float          eps;            /* RMSNorm epsilon (e.g. 1e-6)                         */
    const int32_t *perm;           /* device [K_in] channel order x'[:, j] = y[:, perm[j]],
                                      or NULL (ARCQuant article, section 3.1: outliers
                                      ranked by calibration absmax come first). Must be a
                                      permutation of [0, K_in); other values are clamped.
                                      16-byte aligned, else NVFP4_ERR_ALIGN (read as
                                      16-byte vectors)                                      */
    int64_t        residue_cols;   /* S: residue of columns [0, S) appended after column
                                      K_in, quantized against the same tensor scale
                                      (ARCQuant section 3.1; ResServe abstract). 0 = none,
                                      S = K_in gives K -> 2K. Multiple of 16.             */
    const float   *static_tensor_scale; /* device float, or NULL = dynamic amax / 2688   */
    const float   *smooth;         /* diagonal smoothing: device FP32 [K_in], or NULL. Input
                                      channel k (before the reorder, after RMSNorm) is
                                      multiplied by smooth[k] in FP32 before quantization;
                                      the caller folds 1/smooth into the weight (abstract of
                                      "OSFP4: Joint Optimization of Diagonal Smoothing and
                                      Block Scales for NVFP4 Quantization"). 16-byte aligned,
                                      else NVFP4_ERR_ALIGN                                   */
} nvfp4_quant_opts;

/* Quantize x (rows x K_in, dtype xt, leading dimension ldx elements) into
 * `out`, which must have rows == rows and K == K_in + opts->residue_cols.
 * opts may be NULL (plain quantization with a dynamic tensor scale). K_in with
 * a permutation is limited to 32768 (a row is staged in LDS). Workspace: nvfp4_workspace_size(0, rows, 0, K_in, S). */
nvfp4_status nvfp4_quantize(const void *x, int xt, int64_t rows, int64_t K_in, int64_t ldx,
                            const nvfp4_quant_opts *opts, const nvfp4_tensor *out,
                            void *ws, size_t ws_bytes, void *stream);

/* W4A4 product y[m][n] = S_a S_w sum_k e(a)d(a) e(w)d(w) over k < K, accumulated
 * in FP32 (ARCQuant article, section 3.1: Y ~ Q(X) Q(W)^T).
 * Exactly one of a_q (pre-quantized activations, M x K) and x (raw activations,
 * dtype xt, leading dimension ldx, quantized inside the call with a dynamic
 * tensor scale) is non-NULL. w is N x K. y is M x N with leading dimension ldy,
 * dtype yt (FP32, or BF16 rounded to nearest even).
 * w may be row-major or tiled (every path reads both); a_q must be row-major.
 * M <= 64 runs as one decode launch that streams the weights once (for
 * M <= 32 a small enough x is quantized inside that launch; otherwise the
 * quantize kernels run first). Larger M quantizes x first and uses the
 * matrix-core tile path.
 * K == 0 gives y = 0. Workspace: nvfp4_workspace_size(1, M, N, K, 0). */
nvfp4_status nvfp4_gemm(const nvfp4_tensor *a_q, const void *x, int xt,
                        int64_t M, int64_t K, int64_t ldx,
                        const nvfp4_tensor *w, void *y, int yt, int64_t ldy,
                        void *ws, size_t ws_bytes, void *stream);

/* nvfp4_gemm without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). Same arguments, kernels and results as nvfp4_gemm.
 * Its workspace is a static device array of NVFP4_NOALLOC_SCRATCH_BYTES, one
 * copy per GPU, held until the process ends; the call allocates nothing. The
 * first call on a device takes the array's address and clears its counters
 * (a fill kernel on `stream`). Every call on one GPU shares that array, so
 * calls that overlap on one GPU (other streams, other threads) race: order
 * them. A product whose workspace (nvfp4_workspace_size(1, M, N, K, 0))
 * exceeds the array returns NVFP4_ERR_WORKSPACE before anything is enqueued,
 * and nvfp4_last_error() says how much it needs. */
#define NVFP4_NOALLOC_SCRATCH_BYTES (32u << 20)
nvfp4_status nvfp4_gemm_noalloc(const nvfp4_tensor *a_q, const void *x, int xt,
                                int64_t M, int64_t K, int64_t ldx,
                                const nvfp4_tensor *w, void *y, int yt, int64_t ldy, void *stream);

/* Residue-compensated product (ARCQuant article, sections 3.1-3.2; ResServe abstract):
 *   X' = perm/RMSNorm(x) per opts, R = X' - deq(Q(X')) on columns [0, S),
 *   Y  = s_aug [Q(X') | Q(R)] [Q(W) | Q(W[:, :S])]^T,  s_aug = S_x S_w,
 * one GEMM over K + S columns in which the weight tail reuses the weight's own
 * first S columns (the same codes and scales; it is never materialized). w must
 * already be in the channel order of opts->perm. S = opts->residue_cols in
 * [0, K]; S = 0 gives the plain product of the normalized/reordered input.
 * a_aug_out (optional, M x (K + S)) receives the quantized X_aug.
 * The decode launches take residue columns when K is a multiple of 32; other
 * K run on the matrix-core tile path at any M.
 * Workspace: nvfp4_workspace_size(2, M, N, K, S). */
nvfp4_status nvfp4_gemm_residue(const void *x, int xt, int64_t M, int64_t K, int64_t ldx,
                                const nvfp4_quant_opts *opts, const nvfp4_tensor *w,
                                void *y, int yt, int64_t ldy, const nvfp4_tensor *a_aug_out,
                                void *ws, size_t ws_bytes, void *stream);

/* ---- MXFP4 (the second block format of the ResServe abstract; the 32-element
 * blocks and E8M0 scales of the MX formats, ARCQuant article, sections 2.2 and
 * 4.2). Each value is an E2M1 code (the same nibbles and packing as above) and
 * every 32 consecutive values along K share one E8M0 byte b, scale 2^(b - 127).
 * There is no tensor scale. Quantization rule (the pages name the format, not
 * its rounding; this is the MX definition): shared exponent e =
 * floor(log2(block amax)) - 2, clamped to [-127, 127] (-127 for an all-zero
 * block); code = E2M1(x * 2^-e) round to nearest even, saturating at 6, sign
 * of x. gfx950's scaled FP4 matrix instructions consume these blocks as they
 * are stored.
 * Canonical storage (layout = NVFP4_LAYOUT_ROWMAJOR): codes rows x ld_codes
 * bytes (ld_codes >= K/2, multiple of 16, 16-byte aligned pointer); scales
 * rows x ld_scales bytes (>= K/32).
 * Tiled storage (weights of the M <= 64 product; layout = NVFP4_LAYOUT_TILED),
 * the order in which that product reads them, so that each of its loads is one
 * contiguous run: items of 16 rows x 512 columns; item (t, u) lives at
 * codes + t*ld_codes + u*4096 and scales + t*ld_scales + u*256, with
 * ld_codes = KU*4096, ld_scales = KU*256, KU = ceil(K/512). Inside an item, for
 * the 128-column step i < 4 and p = 0..63 with r = p % 16, g = p / 16:
 *   codes  byte 1024*i + 16*p + j  (j < 16) = byte j of the canonical codes of
 *          row 16t+r starting at column 512u + 128i + 32g;
 *   scales byte 64*i + p = the E8M0 byte of that 32-column block.
 * Rows >= rows and columns >= K hold zero codes (and zero scale bytes). */
typedef struct {
    uint8_t *codes;  int64_t ld_codes;
    uint8_t *scales; int64_t ld_scales;
    int64_t  rows, K;      /* K % 32 == 0 */
    int32_t  layout;       /* nvfp4_layout; only W of nvfp4_mx_gemm at M <= 64 may be tiled */
} nvfp4_mx_tensor;

/* MXFP4-quantize x (rows x K_in, dtype xt, ldx) into `out` (rows x (K_in + S)).
 * S = residue_cols (multiple of 32, <= K_in): the residue R = x - deq(Q(x)) of
 * columns [0, S), computed in FP32 (exact dequantization, one rounding) and
 * quantized in the same format with its own block scales, is stored after
 * column K_in (the two-stage residue of the ARCQuant article, section 3.1).
 * K_in % 32 == 0. No workspace: every block is independent. */
nvfp4_status nvfp4_mx_quantize(const void *x, int xt, int64_t rows, int64_t K_in, int64_t ldx,
                               int64_t residue_cols, const nvfp4_mx_tensor *out, void *stream);

/* MXFP4 product y = A W^T (ARCQuant article, section 3.1 formula; ResServe
 * abstract for MXFP4 with residue compensation): A is M x (K + S) (its last S
 * columns the quantized residue of its first S), W is N x K; the residue
 * columns meet W's own first S columns (never materialized). FP32 accumulation
 * in the scaled FP4 matrix cores; y dtype yt (FP32 or BF16 round to nearest
 * even), leading dimension ldy. Workspace: nvfp4_workspace_size(4, M, N, K, S)
 * bytes; its first 8 KiB (the counter header the NVFP4 entry points keep) are
 * never written, so one workspace can serve both formats. When the product needs
 * no split-K partials, ws may be NULL. W may be tiled (nvfp4_mx_pack_tiled) when
 * M <= 64; a tiled W at M > 64, or a tiled A, is NVFP4_ERR_UNSUPPORTED. */
nvfp4_status nvfp4_mx_gemm(const nvfp4_mx_tensor *a, const nvfp4_mx_tensor *w, int64_t residue_cols,
                           void *y, int yt, int64_t ldy, void *ws, size_t ws_bytes, void *stream);

/* Decode attention over an NVFP4 KV cache with residue compensation of its
 * activation operands (ResServe abstract: the FP4 base plus FP4-quantized
 * residue of the linear layers, applied to decode attention). The pages give no
 * attention formula; the reading is scaled dot-product attention of one decode
 * query per head, the cache stored like a weight and the two activation operands
 * of the step -- the query and the probabilities -- carrying residue columns as
 * in nvfp4_gemm_residue:
 *   s_h = ([Q(q_h) | Q(R(q_h))] . [K_h | K_h]^T) / sqrt(D)
 *   p_h = softmax(s_h)        FP32: m = max s, e = exp(s - m), p = e / sum(e)
 *   o_h = [Q(p_h) | Q(R(p_h))] . [Vt_h | Vt_h]^T
 * q_h and p_h are each quantized as one tensor (own tensor scale); compensate = 0
 * drops the residue columns (plain W4A4 attention).
 *   q        H x D activations (dtype qt, leading dimension ldq), one row per head
 *   k_cache  row-major NVFP4, H*T rows of D columns: row h*T + t is token t of head h
 *   vt_cache row-major NVFP4, H*D rows of T columns: row h*D + j is dimension j of
 *            head h over the tokens (V transposed, blocks of 16 along the tokens)
 *   out      H x D FP32 (leading dimension ldo)
 * Each cache element meets the sum of the base and residue values of its operand
 * element, (e_q d_q + e_r d_r) e_k d_k, as in the augmented product's definition;
 * sums are FP32 in a fixed order (the output is the same bits on every call).
 * 32 <= D <= 256 with D % 32 == 0, T > 0 with T % 16 == 0, H <= 65535 (else
 * NVFP4_ERR_SHAPE); H == 0 does nothing. Workspace: nvfp4_workspace_size(5, H, D, T, 0)
 * bytes; the scores and softmax statistics go after the 8 KiB counter header,
 * which this call leaves untouched, so the workspace can be shared with the
 * products. */
nvfp4_status nvfp4_decode_attention(const void *q, int qt, int64_t H, int64_t D, int64_t ldq,
                                    const nvfp4_tensor *k_cache, const nvfp4_tensor *vt_cache, int64_t T,
                                    int compensate, float *out, int64_t ldo, void *ws, size_t ws_bytes,
                                    void *stream);

/* Rewrite the row-major weight `src` into the tiled layout `dst` (same rows
 * and K; dst->ld_codes = KU*4096, dst->ld_scales = KU*512; its codes and
 * scales buffers hold ceil(rows/16) strips). The tensor scale is copied.
 * A one-time layout change of static weights: values are not touched. */
nvfp4_status nvfp4_pack_tiled(const nvfp4_tensor *src, const nvfp4_tensor *dst, void *stream);

/* Rewrite the row-major MXFP4 weight `src` into the tiled MX layout `dst` (same
 * rows and K; dst->layout = NVFP4_LAYOUT_TILED, dst->ld_codes = KU*4096,
 * dst->ld_scales = KU*256; its buffers hold ceil(rows/16) strips). A one-time
 * layout change of static weights for the M <= 64 MXFP4 product; values are not
 * touched. Shape or layout errors: NVFP4_ERR_SHAPE; misaligned: NVFP4_ERR_ALIGN. */
nvfp4_status nvfp4_mx_pack_tiled(const nvfp4_mx_tensor *src, const nvfp4_mx_tensor *dst, void *stream);

/* Calibration statistic for the outlier reorder (ARCQuant article, sections 3.1
 * and 6.1): absmax_out[j] = max over rows of |RMSNorm(x)[:, j]| (|x| when
 * gamma == NULL). x is rows x K (dtype xt, ldx); absmax_out is a device float[K].
 * Workspace: nvfp4_workspace_size(3, rows, 0, K, 0). */
nvfp4_status nvfp4_channel_absmax(const void *x, int xt, int64_t rows, int64_t K, int64_t ldx,
                                  const void *gamma, float eps, float *absmax_out,
                                  void *ws, size_t ws_bytes, void *stream);

/* Host helper: perm_host = channels sorted by absmax_host descending, ties by
 * ascending index (host arrays of K elements). */
nvfp4_status nvfp4_perm_from_absmax(const float *absmax_host, int64_t K, int32_t *perm_host);

/* Bytes of workspace an operation needs: op 0 = quantize (M = rows), 1 = gemm,
 * 2 = gemm_residue, 3 = channel_absmax (M = rows), 4 = mx_gemm, 5 = decode_attention
 * (M = H, N = D, K = T). S is the residue
 * column count. */
size_t nvfp4_workspace_size(int op, int64_t M, int64_t N, int64_t K, int64_t S);

const char *nvfp4_status_string(nvfp4_status s);
const char *nvfp4_last_error(void);   /* thread-local text of the last HIP error */
int         nvfp4_version(void);      /* major * 10000 + minor * 100 + patch      */

/* Host-side builds of the kernels' scalar rounding helpers, exported so the
 * rounding logic itself can be checked on a machine without a GPU.
 * nvfp4_host_e4m3_encode: v >= 0 -> E4M3 byte; nvfp4_host_e2m1_encode: q -> 4-bit code. */
int nvfp4_host_e4m3_encode(float v);
int nvfp4_host_e2m1_encode(float q);

#ifdef __cplusplus
}
#endif
#endif /* NVFP4_H */
