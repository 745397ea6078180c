/*
 * pn.h -- C ABI of libpn.so: decode-step GEMV y = W.x over block-quantized weights decoded in
 * registers, on AMD Instinct MI355X (gfx950).
 *
 * Formats:
 *   PN (pn3t, pn4t)  "PN weight format" (PNX-FORMAT-v0), sections "Types", "Block layout",
 *                    "Value", "Reference quantizer", "Validation".
 *   NVFP4 (W4A16)    "Quantisation and profiles", sections "NVFP4" and "The clip search";
 *                    NInfer "tensor formats", section 3.3 (E2M1 and E4M3FN words, validity).
 *   row-scaled E4M3  NInfer "tensor formats", section 3.4 (FP8_E4M3FN_ROW_BF16S);
 *                    "Quantisation and profiles", "The FP8 head".
 *
 * Conventions for every entry point:
 *   - Every pointer argument that names a tensor is a DEVICE pointer, owned by the caller. The
 *     library allocates nothing and keeps no pointer after the call returns.
 *   - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued asynchronously on it;
 *     the call returns after argument checks and kernel launch, not after completion.
 *   - The return value is a status (PN_OK = 0, or a negative PN_ERR_*), decided synchronously from
 *     the arguments and the launch. Per-row verdicts and quantizer statuses are device outputs.
 *   - Nothing falls back silently: a shape, dtype or device this library does not handle is an
 *     error, never a slower path on another device.
 *   - N == 0, nrows == 0 or M == 0 is a no-op that returns PN_OK. K must be a positive whole
 *     number of blocks (80 for pn3t, 64 for pn4t, 16 for NVFP4); otherwise PN_ERR_SHAPE.
 *
 * PN tensor layout: W is N rows of K weights; row n starts at byte n * pn_row_bytes(type, K); a
 * row is K/80 (pn3t) or K/64 (pn4t) consecutive 34-byte blocks. Block b of a row starts at byte
 * 34*b: bytes 0..1 hold d (fp16, little-endian, signed), bytes 2..33 hold eight little-endian u32
 * words. W needs only 2-byte alignment; nothing assumes a word is 4-byte aligned.
 */
#ifndef PN_H
#define PN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ggml type ids of the two PN types ("PN weight format", "Types"). */
enum { PN_TYPE_PN3T = 124, PN_TYPE_PN4T = 125 };

/* Status codes. */
enum {
    PN_OK = 0,
    PN_ERR_TYPE = -1,   /* type is neither PN_TYPE_PN3T nor PN_TYPE_PN4T */
    PN_ERR_SHAPE = -2,  /* K is not a positive whole number of blocks, or a size is negative */
    PN_ERR_TOKENS = -3, /* M (tokens) outside 0..16 (PN GEMV) or 0..4 (NVFP4, row-scaled E4M3) */
    PN_ERR_NULL = -4,   /* a required pointer is NULL */
    PN_ERR_ALIGN = -5,  /* W not 2-byte aligned, x / y / w not 4-byte aligned, bf16 x not 2-byte,
                           NVFP4 codes not 8-byte aligned */
    PN_ERR_HIP = -6,    /* the HIP runtime reported an error (no device, launch failure) */
    PN_ERR_DEVICE = -7, /* the current device is not gfx950 */
    PN_ERR_HADAMARD = -8 /* Hadamard slice size B is not a power of two in 2..16384 dividing K */
};

/* Maximum tokens per GEMV call. */
#define PN_MAX_TOKENS 4        /* NVFP4 and row-scaled E4M3 GEMV */
#define PN_GEMV_MAX_TOKENS 16  /* PN GEMV */
#define PN_GEMV_GROUP_MAX_PARTS 4  /* matrices per pn_gemv_group call */
#define PN_GEMV_HADAMARD_MAX_TOKENS 4  /* PN GEMV with the rotation fused */

/* Bytes of one PN row of K weights: 34*K/80 (pn3t) or 34*K/64 (pn4t); 0 if K is not a positive
 * multiple of the block size or type is unknown. Host-only, no device work. */
int64_t pn_row_bytes(int type, int64_t K);

/* Human-readable name of a status code (static storage). */
const char *pn_status_string(int status);

/* ---- PN validation ("PN weight format", "Validation") --------------------------------------
 * verdict[r] = 1 if row r is valid, 0 if it is invalid: some block's d is an fp16 NaN or infinity,
 * or (pn3t) bit 15 or bit 31 of some word is set. verdict is int32[nrows] on the device. */
int pn_validate_rows(int type, const void *W, int64_t nrows, int64_t K, int32_t *verdict,
                     void *stream);
/* One row (nrows = 1). */
int pn_validate_row(int type, const void *row, int64_t K, int32_t *verdict, void *stream);

/* ---- PN decode ("PN weight format", "Value") -----------------------------------------------
 * out[r*K + k] = fp32(d) * (n - z) for every weight, bit-exact: the product is exact in fp32, IEEE
 * signs apply (code z with a negative d gives -0.0; d = +0 with n < z gives -0.0), fp16 subnormal
 * d are kept. Reserved bits are ignored by the decode (they only make the row invalid). A
 * non-finite d decodes as the IEEE product (NaN or +-inf). out is fp32[nrows, K]. */
int pn_dequantize_rows(int type, const void *W, int64_t nrows, int64_t K, float *out,
                       void *stream);
int pn_dequantize_row(int type, const void *row, int64_t K, float *out, void *stream);

/* ---- PN GEMV -------------------------------------------------------------------------------
 * y[m*N + n] = sum_k w[n, k] * x[m*K + k] for m < M (1 <= M <= 16 tokens), with w the decode above,
 * accumulated in fp32. x is fp32[M, K] row-major, y fp32[M, N] row-major (overwritten).
 * Accuracy ("PN weight format", "Value"): |y - y_ref| <= 1e-5 * sum_k |w_k x_k| per output, y_ref
 * the exact sum, for every finite input whose products and partial sums stay in fp32's normal
 * range. At 1-4 tokens each weight is decoded exactly to the integer n - z, each product with x is
 * exact inside an fp32 fma, and the only roundings are the fp32 sums: eight chains of at most 10
 * terms per lane and block piece, one multiply by d, a 64-lane tree and the in-order sum of at most
 * a few dozen chunk partials per row (under 30 * 2^-24 of sum_k |w x| in the worst case).
 * At 5-16 tokens (the matrix cores) the zero point is taken off each code exactly as well, but
 * each x is carried as an fp16 (hi, lo) pair with one exponent per token and group of blocks (4
 * consecutive blocks where W is staged through LDS, one block where it is read directly): exact to
 * 2^-22 relative or to 2^-32 (pn3t; 2^-34 pn4t) of the largest |x| in its group, whichever is
 * larger, so the bound above holds where every x that meets a nonzero weight is within about 2^14
 * of the largest |x| of its group, or the group's other terms dominate. Rows are not
 * validated here (validate at load); an invalid row gives an unspecified value but no
 * out-of-bounds access. Deterministic: the same inputs and launch give the same bits on every
 * call. */
int pn_gemv(int type, const void *W, int64_t N, int64_t K, const float *x, int64_t M, float *y,
            void *stream);

/* Several PN GEMVs that read the same x (a layer's q, k and v; gate and up):
 * parts[i].y[m*N_i + n] = sum_k w_i[n, k] * x[m*K + k], with the bits of one pn_gemv per part. At
 * 1-4 tokens all parts, of either type, run as one launch where the shapes allow it (else the
 * parts of each type, else one launch per part, in order on the stream). 1 <= count <=
 * PN_GEMV_GROUP_MAX_PARTS (else PN_ERR_SHAPE); every part has its own type, W (N_i rows of K
 * weights) and y, and all share K, x and M (0..16). Argument errors as pn_gemv, for the first part
 * that has one; parts with N = 0 are skipped. The parts' y must not overlap each other or x. */
typedef struct pn_gemv_part {
    int type;       /* PN_TYPE_PN3T or PN_TYPE_PN4T */
    const void *W;  /* N rows of pn_row_bytes(type, K) bytes, 2-byte aligned */
    int64_t N;      /* rows (outputs per token) */
    float *y;       /* fp32[M, N], 4-byte aligned */
} pn_gemv_part;
int pn_gemv_group(const pn_gemv_part *parts, int count, int64_t K, const float *x, int64_t M,
                  void *stream);

/* ---- Hadamard-rotated activations ("PN weight format", "Files that use PN") ----------------
 * The page states that the model rotates the activations that reach the PN weights with a
 * Hadamard transform, done by the engine, and fixes neither its order nor its normalisation.
 * Reading used here: each row of x[M, K] is cut into consecutive slices of B elements (B a power
 * of two, 2 <= B <= 16384, dividing K; otherwise PN_ERR_HADAMARD), and each slice is multiplied by
 * the orthonormal Sylvester-ordered Walsh-Hadamard matrix H_B / sqrt(B),
 * H_B[i][j] = (-1)^popcount(i & j):  x'[m, s*B + i] = sum_j H_B[i][j] x[m, s*B + j] / sqrt(B).
 * Computed in fp32 as log2(B) butterfly stages and one multiply by fp32(1/sqrt B) (exact for even
 * log2 B): |x' - x'_exact| <= (log2(B) + 2) * 2^-24 * sum_j |x[m, s*B + j]| / sqrt(B) per element
 * (up to terms in 2^-48). Deterministic. */

/* out[M, K] = the rotation of x[M, K] (fp32, row-major). K must be a multiple of 4
 * (PN_ERR_SHAPE). out may equal x (in place); otherwise they must not overlap. */
int pn_hadamard_rows(const float *x, int64_t M, int64_t K, int64_t B, float *out, void *stream);

/* y = W x' for M = 1..4 tokens: the rotation of pn_hadamard_rows into a workspace, then pn_gemv
 * on it: the same bits as those two calls made by hand, the rotation's error above adding to the
 * GEMV's; x itself is not modified. The workspace is a buffer per stream (up to 16 streams per
 * device) that the library keeps for the life of the process, grown on its stream
 * (hipMallocAsync, the old one hipFreeAsync'd) when a call needs more than it holds: a call
 * allocates nothing otherwise. Calls on one stream reuse its buffer in stream order; calls on
 * different streams never share one. Past 16 streams on a device, on hipStreamPerThread and under
 * stream capture, a call takes a temporary instead (hipMallocAsync and hipFreeAsync on its stream,
 * which a graph records as nodes of its own). Arguments as pn_gemv, plus B as in
 * pn_hadamard_rows; M outside 0..4 gives PN_ERR_TOKENS, a failed allocation PN_ERR_HIP. */
int pn_gemv_hadamard(int type, const void *W, int64_t N, int64_t K, const float *x, int64_t M,
                     int64_t B, float *y, void *stream);

/* pn_gemv_hadamard without any allocation, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid it). The rotated x goes to a
 * file-scope device array of PN_NOALLOC_MAX_FLOATS floats (1 MiB) that each GPU holds for the life
 * of the process; the rotation overwrites every element the GEMV then reads, so nothing is cleared
 * between calls. Same arguments, errors and bits as pn_gemv_hadamard, plus PN_ERR_SHAPE when
 * M * K exceeds PN_NOALLOC_MAX_FLOATS. Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (on different streams, or from several host threads) race on it, so callers
 * order them. */
#define PN_NOALLOC_MAX_FLOATS 262144
int pn_gemv_hadamard_noalloc(int type, const void *W, int64_t N, int64_t K, const float *x,
                             int64_t M, int64_t B, float *y, void *stream);

/* Several GEMVs that share x, over the rotated x: x rotated once into the workspace of
 * pn_gemv_hadamard (same streams and allocation), then pn_gemv_group on it -- parts[i].y = W_i x'
 * with the bits of pn_hadamard_rows followed by one pn_gemv per part. B as in pn_hadamard_rows,
 * 0 <= M <= 4 (else PN_ERR_TOKENS), parts and errors as pn_gemv_group. */
int pn_gemv_group_hadamard(const pn_gemv_part *parts, int count, int64_t K, const float *x,
                           int64_t M, int64_t B, void *stream);

/* ---- PN reference quantizer ("PN weight format", "Reference quantizer") ---------------------
 * Quantizes fp32 w[nrows, K] (row-major) into PN rows W (nrows * pn_row_bytes bytes), one group of
 * 80 or 64 weights per block: 36 candidate scales s = fp16(sigma * m * amax / z),
 * m = 0.50, 0.52, ..., 1.20, codes clamp(rint(w/s) + z, 0, 2z-1), double-precision squared error,
 * ties to the larger m; an all-zero group, or one whose candidates all round to zero, is the
 * canonical zero group (d = +0, codes z). Every step runs in fp64 in the order stated, so these
 * rules fix every output bit.
 * status (int32[nrows], optional, may be NULL) receives per row the OR of: 1 = a group held a NaN
 * or infinity, 2 = every candidate scale overflowed fp16 (such groups are written as the canonical
 * zero group). */
int pn_quantize_rows(int type, const float *w, int64_t nrows, int64_t K, void *W, int32_t *status,
                     void *stream);

/* ---- NVFP4 W4A16 ---------------------------------------------------------------------------
 * Layout: codes uint8[N, K/2], element k of a row in byte k/2, even k in the low nibble (E2M1
 * words); scales uint8[N, K/16], one E4M3FN word per group of 16 consecutive k; one fp32 global
 * multiplier g (weight_scale_2). A weight is fp32(fp32(e2m1(code) * e4m3(scale)) * g). */

/* verdict[n] = 1 iff every scale word of row n has sign bit 0 and is not NaN (0x7F), and g is
 * finite and > 0. */
int pn_nvfp4_validate_rows(const uint8_t *scales, float g, int64_t N, int64_t K, int32_t *verdict,
                           void *stream);

/* out fp32[N, K], bit-exact decode as above. */
int pn_nvfp4_dequantize_rows(const uint8_t *codes, const uint8_t *scales, float g, int64_t N,
                             int64_t K, float *out, void *stream);

/* y[m*N + n] = sum_k w[n, k] * x[m, k], x bf16[M, K] (raw 16-bit words, row-major), 1 <= M <= 4,
 * fp32 accumulation; same accuracy contract as pn_gemv. codes must be 8-byte aligned (rows of
 * K/2 bytes with K a multiple of 16 keep every row 8-byte aligned), else PN_ERR_ALIGN. */
int pn_gemv_nvfp4(const uint8_t *codes, const uint8_t *scales, float g, int64_t N, int64_t K,
                  const uint16_t *x_bf16, int64_t M, float *y, void *stream);

/* ---- Row-scaled E4M3FN (FP8_E4M3FN_ROW_BF16S) -----------------------------------------------
 * NInfer "tensor formats", section 3.4: codes uint8[N, K] E4M3FN words (section 3.3), row-major;
 * one bfloat16 multiplier word per row, scales uint16[N]; w = binary32(e4m3(c) * bf16(s)).
 * "Quantisation and profiles", "The FP8 head": the output head (248,320 x 5,120) is stored this
 * way, one scale per vocabulary row. */

/* verdict[n] = 1 iff row n is valid: its multiplier has sign bit 0 and is finite (+0 and positive
 * subnormals included), no code is a NaN word (0x7F, 0xFF), and a +0 multiplier has only
 * signed-zero codes (0x00, 0x80). */
int pn_fp8row_validate_rows(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                            int32_t *verdict, void *stream);

/* out fp32[N, K] = binary32(e4m3(code) * bf16(scale)), bit-exact (NaN words decode to NaN). */
int pn_fp8row_dequantize_rows(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                              float *out, void *stream);

/* y[m*N + n] = sum_k w[n, k] * x[m*K + k], x fp32[M, K], y fp32[M, N] (overwritten), 1 <= M <= 4,
 * fp32 accumulation, |y - y_exact| <= 1e-5 * sum_k |w x| for finite inputs. K must be a multiple of
 * 16 (PN_ERR_SHAPE) and codes 16-byte aligned (PN_ERR_ALIGN). Rows are not validated here.
 * Deterministic. */
int pn_gemv_fp8row(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                   const float *x, int64_t M, float *y, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PN_H */
