/*
 * ffn.h -- the chunked feed-forward block of a transformer layer.
 *
 * The English noflash-attention post (ai-navigate-news.com, section "The
 * DIY approach", its list of what worked) names FFN chunking, with a
 * runtime safety check, as its second memory saver next to tiled
 * attention.  Computed here, for every token row i of x:
 *
 *     y_i = W2 gelu(W1 x_i + b1) + b2,
 *     gelu(a) = a/2 (1 + tanh(sqrt(2/pi) (a + 0.044715 a^3)))
 *
 * over chunks of `chunk_rows` rows, so that the N x F hidden activation
 * never exists at once: peak extra memory is chunk_rows x F elements plus
 * the matrix-product workspace (128 MiB; each product runs the first of
 * hipBLASLt's candidate algorithms whose stated workspace fits it).  The
 * two products are hipBLASLt GEMMs (fp32 accumulation) with the bias and
 * GELU (first product) and the output bias (second) applied to the fp32
 * accumulator in hipBLASLt's epilogue; where hipBLASLt offers no algorithm
 * with that epilogue for a shape, the plain product is followed by this
 * library's elementwise kernel.  The hidden activation is rounded to the
 * input type between the products.
 *
 * Layout: row-major, 16-bit (dtype ATTN_F16 or ATTN_BF16 of attn.h):
 * x [N, Dm], w1 [F, Dm], b1 [F], w2 [Dm, F], b2 [Dm], y [N, Dm]; Dm and F
 * multiples of 8; all pointers 16-byte aligned device pointers on the
 * current device; b1 and b2 may be NULL (no bias).  The caller owns every
 * buffer; calls are asynchronous on `stream` (hipStream_t; NULL = the null
 * stream) and allocate their workspace stream-ordered.  Return codes as in
 * attn.h (ATTN_OK, ATTN_EINVAL, ATTN_EUNSUPPORTED, ATTN_ENOMEM, ATTN_EHIP;
 * a failed hipBLASLt call is ATTN_EHIP).
 */
#ifndef FFN_H_
#define FFN_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FFN_GELU_TANH = 0 } ffn_act_t;

/* y = W2 gelu(W1 x + b1) + b2 over chunks of chunk_rows rows (0 = the
 * library's choice: rows whose hidden activation fits 96 MiB, rounded down
 * to a multiple of 1024, at least 1024).  act must be FFN_GELU_TANH.  y
 * must not overlap any input. */
int ffn_chunked(const void* x, const void* w1, const void* b1, const void* w2,
                const void* b2, void* y, int N, int Dm, int F, int act,
                int chunk_rows, int dtype, void* stream);

/* ffn_chunked_check -- host only: ffn_chunked's argument validation. */
int ffn_chunked_check(const void* x, const void* w1, const void* b1,
                      const void* w2, const void* b2, const void* y, int N,
                      int Dm, int F, int act, int chunk_rows, int dtype);

/* Device bytes ffn_chunked allocates for a chunk of chunk_rows rows. */
size_t ffn_workspace_bytes(int chunk_rows, int F, int Dm, int dtype);

/* ffn_verify -- the runtime check of the chunking: evaluates the first
 * R = min(N, 2 * chunk_rows + 1) rows once with the given chunking and once
 * as a single chunk, and writes max |difference| and max |single-chunk
 * result| to the host floats *max_abs_diff and *max_abs_ref.  Synchronises
 * `stream`.  The row-wise block gives the same rows either way up to the
 * rounding of the products; a wrong chunk offset or size shows up as a
 * difference of the order of the result itself.  A NaN or infinity in either
 * evaluation makes *max_abs_diff (and, if in the single-chunk rows,
 * *max_abs_ref) +inf, so a check that also requires both to be finite
 * fails on it. */
int ffn_verify(const void* x, const void* w1, const void* b1, const void* w2,
               const void* b2, int N, int Dm, int F, int act, int chunk_rows,
               int dtype, float* max_abs_diff, float* max_abs_ref, void* stream);

#ifdef __cplusplus
}
#endif

#endif  /* FFN_H_ */
