/*
 * attn.h -- C ABI of the MI355X (gfx950) memory-efficient attention forward
 * and its gradients.
 *
 * The operation is the one the English noflash-attention post
 * (ai-navigate-news.com, section "The DIY approach") tiles over query chunks
 * and, in its online-softmax tier, over key tiles with a running max and
 * running sum: exact softmax attention,
 *
 *     O[b,h,i,:] = sum_{j in J_i} softmax_j(scale * <Q[b,h,i,:], K[b,g(h),j,:]>) V[b,g(h),j,:]
 *     LSE[b,h,i] = ln sum_{j in J_i} exp(scale * <Q[b,h,i,:], K[b,g(h),j,:]>)
 *
 * without ever forming the Nq x Nkv score matrix.  g(h) = h / (Hq / Hkv): the
 * post's flattened GQA groups consecutive query heads on one KV head.  J_i is
 * every key, or with `causal` the keys j <= i (top-left alignment, the
 * semantics of PyTorch's scaled_dot_product_attention is_causal, which is the
 * API the post patches; section "Other areas where this could be useful"),
 * or the keys j <= i + Nkv - Nq (bottom-right alignment, an option of the
 * same API).  An empty J_i gives O = 0 and LSE = -inf.
 *
 * Layout (all tensors): contiguous [batch, heads, seq_len, head_dim], the
 * head dimension fastest -- the layout the ai-manual.ru article's chunked
 * snippet unpacks (section 3).  Q is [B,Hq,Nq,D], K and V are [B,Hkv,Nkv,D],
 * `out` is [B,Hq,Nq,D] in the input dtype, `lse` is float32 [B,Hq,Nq].
 * Inputs are fp16 or bf16; all arithmetic accumulates in fp32.
 *
 * Pointers are device pointers on the current HIP device unless stated.
 * The caller owns every buffer; the library keeps no pointer after return.
 * Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 * stream): results are valid when the stream has reached the call.
 *
 * Errors: every entry point returns ATTN_OK (0) or a negative code.  Argument
 * errors are detected on the host before any HIP call.  There is no fallback
 * path: on error nothing has been launched (ATTN_EINVAL, ATTN_EUNSUPPORTED,
 * ATTN_ENOMEM) or a launch failed (ATTN_EHIP; attn_last_hip_error() gives the
 * hipError_t).
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { ATTN_F16 = 0, ATTN_BF16 = 1 } attn_dtype_t;

/* Kinds of attention mask (attn_fwd_masked). */
enum {
  ATTN_MASK_NONE = 0,
  ATTN_MASK_BOOL = 1, /* bytes: nonzero keeps the key, zero removes it */
  ATTN_MASK_ADD = 2   /* values of the input dtype added to the scaled scores */
};

/* Values of the `causal` argument. */
enum {
  ATTN_CAUSAL_NONE = 0,         /* every key */
  ATTN_CAUSAL_TOP_LEFT = 1,     /* keys j <= i */
  ATTN_CAUSAL_BOTTOM_RIGHT = 2  /* keys j <= i + Nkv - Nq */
};

enum {
  ATTN_OK = 0,
  ATTN_EINVAL = -1,       /* bad argument (shape, pointer, alignment, dtype, scale) */
  ATTN_EUNSUPPORTED = -2, /* the current device is not gfx950 */
  ATTN_ENOMEM = -3,       /* a device workspace could not be allocated */
  ATTN_EHIP = -4,         /* a HIP call or kernel launch failed */
  ATTN_ESCRATCH = -5      /* attn_fwd_noalloc: the plan needs more than its scratch */
};

/* Bytes of the per-device scratch array of attn_fwd_noalloc (64 MiB). */
#define ATTN_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * attn_fwd -- O and LSE of exact softmax attention (definition above).
 *
 * q, k, v : device pointers, fp16/bf16 per `dtype`, 16-byte aligned.
 * out     : device pointer, [B,Hq,Nq,D], same dtype; must not overlap q/k/v.
 * lse     : device pointer to float32 [B,Hq,Nq] (natural log), or NULL to
 *           skip writing it.
 * B, Hq, Hkv, Nq, Nkv : > 0, Hq a multiple of Hkv.
 * D       : 64, 80, 96, 128 or 256 (the tile table is per head
 *           dimension; the extension past the pages' 64/128 follows the
 *           scope's list of further head dimensions; 80 is computed as 96
 *           with zero padding inside the kernel).
 * scale   : finite softmax scale (PyTorch's default is 1/sqrt(D); the
 *           ai-manual.ru snippet divides scores by sqrt(dim)).
 * causal  : ATTN_CAUSAL_NONE (0) = every key, ATTN_CAUSAL_TOP_LEFT (1) =
 *           keys j <= i (PyTorch's is_causal), ATTN_CAUSAL_BOTTOM_RIGHT (2) =
 *           keys j <= i + Nkv - Nq (PyTorch's causal_lower_right bias: the
 *           last query row sees every key, as when new queries follow a
 *           cache of earlier keys).  With Nq > Nkv the first Nq - Nkv rows
 *           of a bottom-right call see no key: their output is 0 and their
 *           LSE -inf.
 * dtype   : ATTN_F16 or ATTN_BF16.
 * stream  : hipStream_t to launch on.
 *
 * GQA head packing: with G = Hq / Hkv > 1 and a query range shorter than
 * the head dimension's tile (decode, short chunks), the G query heads of a
 * KV head are computed as one range of G * Nq rows (the post's "flattened
 * GQA GEMMs", section "The DIY approach"), so each KV head's keys and values
 * are read once for the group.  Results are the same function either way.
 *
 * Query rows are processed in tiles of attn_plan.tile_rows rows.  Where
 * the tiles cannot keep every compute unit busy -- a grid smaller than the
 * device, or, without a mask, the last partial round of a grid that fills it
 * -- those tiles are split over key ranges (split-KV) and the pieces merged
 * by their log-sum-exp, when a cost model finds that the pieces save more
 * than the split costs (for a small causal grid, whose tiles differ in
 * length, often they do not); whole tiles and pieces share one launch,
 * whole tiles first.  Pieces take a workspace of attn_plan.workspace_bytes bytes,
 * stream-ordered on `stream` from the library's pool (attn_workspace_pool);
 * when nothing is split nothing is allocated.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
             int B, int Hq, int Hkv, int Nq, int Nkv, int D,
             float scale, int causal, int dtype, void* stream);

/*
 * attn_fwd_split -- attn_fwd with the split-KV count chosen by the caller.
 * num_splits = 0 plans as attn_fwd does; a positive value splits every
 * query tile into that many key ranges (clamped to the number of key
 * tiles).  Every split count computes the same function; results differ
 * only by fp32 rounding order.
 */
int attn_fwd_split(const void* q, const void* k, const void* v, void* out,
                   float* lse, int B, int Hq, int Hkv, int Nq, int Nkv, int D,
                   float scale, int causal, int dtype, int num_splits,
                   void* stream);

/*
 * attn_fwd_noalloc -- attn_fwd_split that allocates nothing, for callers
 * that cannot call hipMalloc: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Same arguments, plan, kernels
 * and results (bit for bit) as attn_fwd_split with the same num_splits.
 *
 * The split-KV partials go to a file-scope device array of
 * ATTN_NOALLOC_SCRATCH_BYTES (64 MiB) that each GPU the library runs on
 * holds until the process ends; its address is looked up once per device
 * on the first call there.  A shape whose plan needs more (the workspace
 * attn_fwd_plan reports for the same num_splits) returns ATTN_ESCRATCH
 * before anything is launched; e.g. the 17160-token, 24-head video shape
 * needs 59 MiB and fits, the 75600-token one does not.  Shapes that split
 * nothing do not touch the array.
 *
 * Every call on one GPU shares that GPU's array, which keeps the last
 * call's contents (nothing in it needs to start at zero: each call writes
 * every partial it reads).  Calls that may overlap on one GPU -- on
 * different streams, or from different threads without ordering -- race
 * on it and must be serialised by the caller.  Returns as attn_fwd, plus
 * ATTN_ESCRATCH.
 */
int attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out,
                     float* lse, int B, int Hq, int Hkv, int Nq, int Nkv, int D,
                     float scale, int causal, int dtype, int num_splits,
                     void* stream);

/*
 * attn_fwd_check -- the argument validation of attn_fwd, host only: makes no
 * HIP call and dereferences no pointer.  Returns ATTN_OK or ATTN_EINVAL.
 */
int attn_fwd_check(const void* q, const void* k, const void* v, const void* out,
                   const float* lse, int B, int Hq, int Hkv, int Nq, int Nkv,
                   int D, float scale, int causal, int dtype);

/*
 * attn_fwd_strided -- attn_fwd_split on strided tensors, so that a
 * scaled-dot-product-attention front end (the English noflash-attention
 * post, section "From gfx906 to a broader release": the op is routed in
 * under PyTorch's SDPA call) can pass views such as [B,N,H,D] storage
 * transposed to [B,H,N,D] without copying.
 *
 * q_stride, k_stride, v_stride, o_stride: host arrays of 3 element strides
 * for the batch, head and sequence dimensions of Q, K, V and out (logical
 * shapes as in attn_fwd); the head dimension D is contiguous.  NULL means
 * the contiguous layout.  Each stride must be a non-negative multiple of 8;
 * sequence strides must lie in [D, 2^24]; no two elements of `out` may share
 * an address; `out` must not overlap q, k or v, nor `lse` any tensor
 * (ATTN_EINVAL otherwise).  `lse` stays contiguous [B,Hq,Nq].  Everything
 * else (num_splits, workspace, errors) is as for attn_fwd_split.
 */
int attn_fwd_strided(const void* q, const void* k, const void* v, void* out,
                     float* lse, int B, int Hq, int Hkv, int Nq, int Nkv, int D,
                     const long long* q_stride, const long long* k_stride,
                     const long long* v_stride, const long long* o_stride,
                     float scale, int causal, int dtype, int num_splits,
                     void* stream);

/*
 * attn_fwd_strided_check -- the argument validation of attn_fwd_strided,
 * host only (no HIP call, no pointer dereferenced except the stride
 * arrays).  Returns ATTN_OK or ATTN_EINVAL.
 */
int attn_fwd_strided_check(const void* q, const void* k, const void* v,
                           const void* out, const float* lse, int B, int Hq,
                           int Hkv, int Nq, int Nkv, int D,
                           const long long* q_stride,
                           const long long* k_stride,
                           const long long* v_stride,
                           const long long* o_stride, float scale,
                           int causal, int dtype);

/*
 * attn_fwd_masked -- attn_fwd_strided with an attention mask, the semantics
 * of PyTorch's scaled_dot_product_attention attn_mask (the API the post
 * patches; section "Other areas where this could be useful"): for
 * ATTN_MASK_BOOL a zero byte removes key j from row i, for ATTN_MASK_ADD the
 * value (fp16/bf16 per `dtype`) is added to scale * <q_i, k_j> before the
 * softmax (-inf removes the key).  Rows left with no key give O = 0 and
 * LSE = -inf.  A causal mode still applies on top of the mask.
 *
 * mask        : device pointer, element (b, h, i, j) of the [B,Hq,Nq,Nkv] mask
 *               at mask + b*s[0] + h*s[1] + i*s[2] + j elements (keys
 *               contiguous; strides may be 0 to broadcast), 8-byte aligned.
 * mask_type   : ATTN_MASK_BOOL or ATTN_MASK_ADD (ATTN_MASK_NONE ignores the
 *               mask and behaves as attn_fwd_strided).
 * mask_stride : 3 element strides (batch, query head, query row), each a
 *               non-negative multiple of 4.
 * The mask must not overlap `out` or `lse`.  Masked calls use the 32-row
 * query tiles.  Returns as attn_fwd.
 */
int attn_fwd_masked(const void* q, const void* k, const void* v, void* out,
                    float* lse, int B, int Hq, int Hkv, int Nq, int Nkv, int D,
                    const long long* q_stride, const long long* k_stride,
                    const long long* v_stride, const long long* o_stride,
                    const void* mask, int mask_type, const long long* mask_stride,
                    float scale, int causal, int dtype, int num_splits,
                    void* stream);

/* attn_fwd_masked_check -- host only: attn_fwd_masked's validation. */
int attn_fwd_masked_check(const void* q, const void* k, const void* v,
                          const void* out, const float* lse, int B, int Hq,
                          int Hkv, int Nq, int Nkv, int D,
                          const long long* q_stride, const long long* k_stride,
                          const long long* v_stride, const long long* o_stride,
                          const void* mask, int mask_type,
                          const long long* mask_stride, float scale,
                          int causal, int dtype);

/*
 * attn_fwd_dv -- attn_fwd_masked with value and output rows of Dv elements
 * while Q and K rows keep D.  Nothing in the definition above ties the width
 * of V to that of Q and K: the scores use D, and each output column is the
 * softmax-weighted sum of one V column (PyTorch's
 * scaled_dot_product_attention, the API the post patches, takes such V;
 * section "Other areas where this could be useful").  Supported: Dv == D
 * for every D above (the call is then attn_fwd_masked's), and the pair
 * D = 192, Dv = 128 (multi-head latent attention at prefill).
 *
 * V is [B,Hkv,Nkv,Dv] and `out` [B,Hq,Nq,Dv]; v_stride and o_stride are
 * their element strides (sequence strides in [Dv, 2^24]; NULL =
 * contiguous).  mask, mask_type and mask_stride are as for
 * attn_fwd_masked (ATTN_MASK_NONE, with NULL mask and mask_stride, for no
 * mask).  Split calls allocate fp32 partials of Dv columns.  Returns as
 * attn_fwd; an unsupported (D, Dv) pair is ATTN_EINVAL.
 */
int attn_fwd_dv(const void* q, const void* k, const void* v, void* out,
                float* lse, int B, int Hq, int Hkv, int Nq, int Nkv, int D,
                int Dv, const long long* q_stride, const long long* k_stride,
                const long long* v_stride, const long long* o_stride,
                const void* mask, int mask_type, const long long* mask_stride,
                float scale, int causal, int dtype, int num_splits,
                void* stream);

/* attn_fwd_dv_check -- host only: attn_fwd_dv's validation. */
int attn_fwd_dv_check(const void* q, const void* k, const void* v,
                      const void* out, const float* lse, int B, int Hq, int Hkv,
                      int Nq, int Nkv, int D, int Dv,
                      const long long* q_stride, const long long* k_stride,
                      const long long* v_stride, const long long* o_stride,
                      const void* mask, int mask_type,
                      const long long* mask_stride, float scale, int causal,
                      int dtype);

/*
 * attn_fwd_fp8 -- the forward on 8-bit inputs: q, k, v hold OCP FP8 E4M3
 * bytes (torch.float8_e4m3fn) whose values are byte * q_descale (resp.
 * k_descale, v_descale), one positive finite factor per tensor.  The
 * pages fix no 8-bit format; this computes O and LSE of the definition
 * above on those values, with `out` [B,Hq,Nq,D] in out_dtype (ATTN_BF16 or
 * ATTN_F16) and lse as for attn_fwd.  Both products run on the gfx950
 * 8-bit matrix instruction; the probabilities are rounded to E4M3 for
 * P V (relative error up to 2^-4 per probability, 2^-10 absolute below
 * 2^-6).  Supported: D = 128, contiguous [B,H,N,D] tensors, no mask;
 * causal modes and num_splits as for attn_fwd_split.  Each call allocates
 * (stream-ordered) a transposed copy of V, B*Hkv*128*ceil(Nkv/64)*64 bytes,
 * plus the split partials.  Returns as attn_fwd.
 */
int attn_fwd_fp8(const void* q, const void* k, const void* v, void* out,
                 float* lse, int B, int Hq, int Hkv, int Nq, int Nkv, int D,
                 float q_descale, float k_descale, float v_descale, float scale,
                 int causal, int out_dtype, int num_splits, void* stream);

/* attn_fwd_fp8_check -- host only: attn_fwd_fp8's validation. */
int attn_fwd_fp8_check(const void* q, const void* k, const void* v,
                       const void* out, const float* lse, int B, int Hq,
                       int Hkv, int Nq, int Nkv, int D, float q_descale,
                       float k_descale, float v_descale, float scale,
                       int causal, int out_dtype);

/*
 * attn_plan -- how attn_fwd_split covers a shape (see attn_fwd_plan).
 * Output rows are numbered (b * Hq + h) * Nq + i, 0 <= r < B*Hq*Nq.
 */
typedef struct attn_plan {
  int tile_rows;          /* query rows per workgroup tile */
  int num_splits;         /* key-range pieces per split tile; 1 = no split */
  long long split_rows;   /* rows [B*Hq*Nq - split_rows, B*Hq*Nq) are merged
                             from pieces (0 when num_splits == 1) */
  size_t workspace_bytes; /* device bytes allocated per call: fp32 partial
                             outputs [num_splits, split_rows, D] and LSE
                             [num_splits, split_rows] */
} attn_plan;

/*
 * attn_fwd_plan -- host only: fills *plan with what attn_fwd_split (same
 * num_splits; 0 = as attn_fwd) does for this shape on a device with
 * `num_cus` compute units (256 on MI355X; <= 0 means 256).  D = 192 stands
 * for attn_fwd_dv's (192, 128) pair (partials of 128 columns).  Returns
 * ATTN_OK, or ATTN_EINVAL for invalid shapes, a negative num_splits or a
 * NULL plan.
 */
int attn_fwd_plan(int B, int Hq, int Hkv, int Nq, int Nkv, int D, int causal,
                  int dtype, int num_splits, int num_cus, attn_plan* plan);

/*
 * attn_fwd_num_splits -- host only: attn_fwd_plan(..., 0, num_cus)'s
 * num_splits, the split-KV count attn_fwd uses for the tiles it splits
 * (D = 192: attn_fwd_dv's (192, 128) pair).  Returns >= 1, or ATTN_EINVAL
 * for invalid shapes.
 */
int attn_fwd_num_splits(int B, int Hq, int Hkv, int Nq, int Nkv, int D,
                        int causal, int dtype, int num_cus);

/*
 * attn_fwd_workspace_bytes -- host only (no HIP call): the device bytes
 * attn_fwd allocates for this shape on an MI355X (256 compute units): the
 * fp32 partial outputs and partial LSE of the rows its plan splits over key
 * ranges, attn_plan.workspace_bytes of attn_fwd_plan(..., 0, 256, ...).
 * 0 when nothing is split, and for invalid arguments (a non-positive size,
 * an unsupported D, or causal outside 0..2).  The dtype does not change the
 * plan; the number of KV heads does only through GQA head packing (see
 * attn_fwd), so this returns the largest workspace over every Hkv that
 * divides Hq, a bound a caller can size a buffer by.  D = 192 stands for
 * attn_fwd_dv's (192, 128) pair.  For one Hkv, or a device with another
 * compute-unit count, use attn_fwd_plan.
 */
size_t attn_fwd_workspace_bytes(int B, int Hq, int Nq, int Nkv, int D,
                                int causal);

/*
 * attn_bwd -- gradients of attn_fwd's O with respect to Q, K and V.
 *
 * The post keeps training possible through its tiled forward (first tier,
 * section "The DIY approach": the chunked attention stays differentiable).
 * With P[i,j] = exp(scale <Q_i, K_j> - LSE_i) over J_i (0 elsewhere) and dO
 * the gradient arriving at O:
 *
 *     dV_j = sum_i P[i,j] dO_i,        dP[i,j] = <dO_i, V_j>,
 *     Delta_i = <dO_i, O_i>,           dS[i,j] = P[i,j] (dP[i,j] - Delta_i),
 *     dQ_i = scale sum_j dS[i,j] K_j,  dK_j = scale sum_i dS[i,j] Q_i,
 *
 * where the sums for dK and dV of a KV head run over every query head of its
 * group.  The probabilities are recomputed tile by tile from `lse`; nothing
 * of size Nq x Nkv is stored.
 *
 * q, k, v  : the forward's inputs (contiguous [B,H,N,D], fp16/bf16).
 * out, lse : the forward's outputs for these inputs (attn_fwd with the same
 *            scale and causal flag; `lse` must not be NULL).
 * dout     : [B,Hq,Nq,D], same dtype: the gradient at `out`.
 * dq       : [B,Hq,Nq,D]; dk, dv: [B,Hkv,Nkv,D]; same dtype, written
 *            completely (no accumulation into their previous contents);
 *            must not overlap each other or any input.
 * All pointers 16-byte aligned; D in {64, 80, 96, 128, 256}; Hq a multiple
 * of Hkv.
 * Allocates its workspace stream-ordered on `stream` from the library's
 * pool (attn_workspace_pool) and frees it there: Delta and the base-2 LSE
 * (float32 [B,Hq,Nq] each), fp32 dK/dV partials when the query heads of a
 * GQA group are split over workgroups, and fp32 dQ partials when the dQ
 * grid (without a causal mask) ends in a partial round of workgroups whose
 * key ranges are split -- all O(N * D).  dQ runs
 * on a second stream of the library's, forked from `stream` after Delta and
 * joined back before the call returns (except at D = 128); the caller sees
 * ordinary stream order on `stream`.  Returns ATTN_OK, ATTN_EINVAL,
 * ATTN_EUNSUPPORTED, ATTN_ENOMEM or ATTN_EHIP.  Results are deterministic
 * (no atomics).
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* out,
             const void* dout, const float* lse, void* dq, void* dk, void* dv,
             int B, int Hq, int Hkv, int Nq, int Nkv, int D, float scale,
             int causal, int dtype, void* stream);

/*
 * attn_bwd_masked -- attn_bwd for a forward computed with an attention mask
 * (attn_fwd_masked with the same mask, mask_type and mask_stride, whose
 * conditions apply): the mask enters the recomputed probabilities and is
 * not differentiated.  Rows the mask (or a causal mode) leaves with no key
 * get zero gradients.
 */
int attn_bwd_masked(const void* q, const void* k, const void* v, const void* out,
                    const void* dout, const float* lse, void* dq, void* dk, void* dv,
                    int B, int Hq, int Hkv, int Nq, int Nkv, int D,
                    const void* mask, int mask_type, const long long* mask_stride,
                    float scale, int causal, int dtype, void* stream);

/* attn_bwd_masked_check -- host only: attn_bwd_masked's validation. */
int attn_bwd_masked_check(const void* q, const void* k, const void* v,
                          const void* out, const void* dout, const float* lse,
                          const void* dq, const void* dk, const void* dv, int B,
                          int Hq, int Hkv, int Nq, int Nkv, int D,
                          const void* mask, int mask_type,
                          const long long* mask_stride, float scale,
                          int causal, int dtype);

/*
 * attn_bwd_dv -- gradients of attn_fwd_dv: attn_bwd_masked with V, out, dout
 * and dv of Dv-element rows ([B,Hkv,Nkv,Dv] and [B,Hq,Nq,Dv], contiguous)
 * while Q, K, dq, dk keep D.  The derivative is the same as attn_bwd's:
 * dV = P^T dO and dP = dO V^T run over Dv columns, dQ and dK over D.
 * Supported: Dv == D for every D above, and D = 192 with Dv = 128.  mask,
 * mask_type and mask_stride as for attn_bwd_masked (ATTN_MASK_NONE, NULL,
 * NULL for none).  Returns as attn_bwd; an unsupported pair is ATTN_EINVAL.
 */
int attn_bwd_dv(const void* q, const void* k, const void* v, const void* out,
                const void* dout, const float* lse, void* dq, void* dk, void* dv,
                int B, int Hq, int Hkv, int Nq, int Nkv, int D, int Dv,
                const void* mask, int mask_type, const long long* mask_stride,
                float scale, int causal, int dtype, void* stream);

/* attn_bwd_dv_check -- host only: attn_bwd_dv's validation. */
int attn_bwd_dv_check(const void* q, const void* k, const void* v,
                      const void* out, const void* dout, const float* lse,
                      const void* dq, const void* dk, const void* dv, int B,
                      int Hq, int Hkv, int Nq, int Nkv, int D, int Dv,
                      const void* mask, int mask_type,
                      const long long* mask_stride, float scale, int causal,
                      int dtype);

/*
 * attn_bwd_check -- host only: attn_bwd's argument validation; makes no HIP
 * call and dereferences no pointer.  Returns ATTN_OK or ATTN_EINVAL.
 */
int attn_bwd_check(const void* q, const void* k, const void* v, const void* out,
                   const void* dout, const float* lse, const void* dq,
                   const void* dk, const void* dv, int B, int Hq, int Hkv,
                   int Nq, int Nkv, int D, float scale, int causal, int dtype);

/* attn_strerror -- static description of a return code (never NULL). */
const char* attn_strerror(int code);

/* attn_last_hip_error -- the hipError_t behind the calling thread's last
 * ATTN_EHIP / ATTN_ENOMEM / ATTN_EUNSUPPORTED, 0 if none. */
int attn_last_hip_error(void);

/*
 * attn_workspace_pool -- the memory pool that serves the library's
 * stream-ordered workspace on the current device (split-KV partials of
 * attn_fwd and its variants, the gradients' Delta rows and head-split
 * partials, the FP8 path's transposed V, the FFN's hidden chunks).
 *
 * The library creates one pool per device on first use and allocates from
 * it with hipMallocFromPoolAsync on the caller's stream.  The pool's release
 * threshold is the maximum: memory it has handed out stays mapped between
 * calls, so a call after a stream or device synchronisation does not map its
 * workspace again (with a threshold of 0 that cost ~0.4 ms on a 62 MB
 * workspace).  The memory is therefore held until the process ends.
 *
 * pool : out, the hipMemPool_t (as void*).  The library owns it: callers may
 *        read its attributes (e.g. hipMemPoolAttrUsedMemHigh for the peak
 *        workspace) or release idle memory with hipMemPoolTrimTo, and must
 *        not destroy it.
 * Returns ATTN_OK; ATTN_EINVAL if pool is NULL; ATTN_EHIP if the device
 * query or the pool's creation fails (attn_last_hip_error).
 */
int attn_workspace_pool(void** pool);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
