/*
 * attn.h -- C ABI of libattn.so: fused scaled dot-product attention (forward,
 * log-sum-exp, backward, weights, single-row decode, multi-head wrapper) for
 * AMD Instinct MI355X (gfx950).
 *
 * Operation (per batch entry b and head, for every query row i):
 *
 *     out[b,h,i,:] = sum_j w_ij * v[b,h,j,:],
 *     w_ij = exp(s_ij - m_i) / sum_{j' allowed} exp(s_ij' - m_i),
 *     s_ij = scale * <q[b,h,i,:], k[b,h,j,:]>,  m_i = max over allowed j of s_ij,
 *
 * i.e. Attention(Q, K, V) = softmax(Q K^T / sqrt(d_k)) V as defined in
 * "Attention Is All You Need" (overview on azimuth.plus, section "The idea:
 * every word queries every word"; notebook chapter on antoniofranca.me,
 * section "Multi-Head Self-Attention"; cuijiawei.cn, section "The core idea:
 * scaled dot-product attention"), with the caller supplying the scale
 * (normally 1/sqrt(d_k): aiany.app explainer, Step 5 "Scale: divide by 8").
 * Heads are independent (multi-head layout [B, h, T, d] of the cuijiawei.cn
 * MultiHeadAttention snippet).  Weights for disallowed keys are exactly 0:
 *
 *   ATTN_MASK_CAUSAL: key j is allowed for query row i only if j <= i
 *     (notebook chapter, "Masked Attention in the Decoder", the e_tj cases),
 *     applied literally (top-left aligned) also when Tq != Tk.
 *   ATTN_MASK_KEYPAD: key j of batch entry b is allowed only if j < L_b,
 *     L_b = key_lens[b] clamped to [0, Tk] (the generic masked_fill(mask == 0,
 *     -inf) of the cuijiawei.cn snippet with a per-sequence length mask).
 *   Both bits may be set: the allowed set is the intersection.
 *   A query row with no allowed key (L_b = 0, or Tk = 0) gets an all-zero output.
 *
 * Layout: all tensors dense, row-major, no strides:
 *   q   [B, h, Tq, d_k]     k [B, h, Tk, d_k]     v [B, h, Tk, d_v]
 *   out [B, h, Tq, d_v]     key_lens int32 [B] (device memory), or NULL
 * Offsets are computed in 64-bit arithmetic.
 *
 * Ownership: every pointer is caller-owned device memory (HIP / PyTorch
 * allocations); the library allocates nothing and keeps no per-call state.
 *
 * Asynchrony: the work is enqueued on `stream` (0 = the null stream) and the
 * call returns without synchronising.  key_lens is read by the kernel, so its
 * values are never validated on the host; they are clamped to [0, Tk].
 * Every pointer of a call must be memory of the device `stream` belongs to
 * (the null stream: the current device); the library does not look the
 * pointers' device up, so a mismatch is the caller's error (the Python
 * wrapper checks it).
 *
 * Errors: 0 on success.  Argument errors return a negative ATTN_ERR_* code
 * before any HIP call is made (nothing is launched); a failed launch returns
 * ATTN_ERR_HIP and the hipError_t is kept per thread (attn_last_hip_error).
 * The library never prints and never aborts.
 *
 * Empty work: B, h or Tq equal to 0 is a valid no-op (pointers unused).
 * Tk = 0 is valid: every output row is written as zeros (k, v unused).
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* bits of mask_kind (bitwise OR) */
enum {
  ATTN_MASK_NONE = 0,
  ATTN_MASK_CAUSAL = 1,
  ATTN_MASK_KEYPAD = 2
};

/* status codes */
enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = -1,        /* a pointer that must be non-NULL is NULL */
  ATTN_ERR_SHAPE = -2,       /* negative dimension, or d_k != d_v */
  ATTN_ERR_HEADDIM = -3,     /* head size not supported (supported: 64, 128) */
  ATTN_ERR_MASK = -4,        /* unknown mask bits, or KEYPAD with key_lens == NULL */
  ATTN_ERR_ALIAS = -5,       /* an output buffer (or workspace) overlaps an input, another
                                output or, under key padding, key_lens[0 .. B) */
  ATTN_ERR_ALIGN = -6,       /* a bf16/fp32 tensor not 16-byte aligned; key_lens, lse or delta
                                not 4-byte aligned */
  ATTN_ERR_SCALE = -7,       /* scale is NaN or infinite */
  ATTN_ERR_TOO_LARGE = -8,   /* more than 2^31-1 work-groups, or one head's rows of a tensor
                                exceed 4 GiB (T * d * element size >= 2^32) */
  ATTN_ERR_WORKSPACE = -9,   /* workspace NULL or smaller than the *_workspace_bytes() figure */
  ATTN_ERR_HIP = -100        /* the kernel launch failed; see attn_last_hip_error() */
};

/*
 * attn_fwd: bfloat16 q, k, v and out; fp32 accumulation and fp32 softmax
 * state; the probabilities are rounded to bfloat16 (round-to-nearest-even)
 * before the probability-value product, and the output is rounded once to
 * bfloat16 (round-to-nearest-even).
 *   q, k, v, out : device pointers, bfloat16 elements, layout above
 *   B, h         : batch entries and heads (>= 0)
 *   Tq, Tk       : query and key/value lengths (>= 0)
 *   d_k, d_v     : head sizes; must be equal, 64 or 128
 *   scale        : finite score multiplier (any sign; 0 gives uniform weights)
 *   mask_kind    : OR of ATTN_MASK_* bits
 *   key_lens     : device int32 [B] when ATTN_MASK_KEYPAD is set, else ignored
 *   stream       : HIP stream the kernel is enqueued on
 */
int attn_fwd(const void* q, const void* k, const void* v, void* out,
             int B, int h, int Tq, int Tk, int d_k, int d_v, float scale,
             int mask_kind, const int32_t* key_lens, hipStream_t stream);

/*
 * attn_fwd_f32: identical parameter list and semantics with fp32 q, k, v and
 * out; every product, sum and the softmax are computed in fp32 (no bfloat16
 * rounding anywhere).
 */
int attn_fwd_f32(const void* q, const void* k, const void* v, void* out,
                 int B, int h, int Tq, int Tk, int d_k, int d_v, float scale,
                 int mask_kind, const int32_t* key_lens, hipStream_t stream);

/*
 * attn_fwd_lse: attn_fwd (bfloat16, same arguments and semantics) that also
 * writes the log-sum-exp of every query row's scaled, allowed scores,
 *
 *     lse[b,h,i] = ln sum_{j allowed} exp(s_ij)     (natural log, fp32),
 *
 * -inf for a row with no allowed key.  It is the normaliser of the row
 * softmax (the row sum of exp in the stable softmax of the azimuth.plus
 * overview, "The idea: every word queries every word") kept in log form:
 * w_ij = exp(s_ij - lse_i), which is what attn_bwd recomputes the weights
 * from.  The value is the normaliser the kernel actually divided by (its sum
 * of the bfloat16-rounded probabilities).
 *   lse : device fp32 [B, h, Tq], 4-byte aligned, caller-owned, must not
 *         overlap q, k, v or out; NULL is ATTN_ERR_NULL unless the work is empty.
 */
int attn_fwd_lse(const void* q, const void* k, const void* v, void* out, float* lse,
                 int B, int h, int Tq, int Tk, int d_k, int d_v, float scale,
                 int mask_kind, const int32_t* key_lens, hipStream_t stream);

/*
 * attn_bwd: gradients of out = attention(q, k, v) (the operation above, same
 * scale and mask) with respect to q, k and v, given the gradient dout of a
 * loss with respect to out.  Training through the formula is what the pages
 * describe (aiany.app explainer, Step 11: every weight matrix is nudged by
 * back-propagating a cross-entropy loss).  With w the weights and
 * D_i = <dout_i, out_i>, the chain rule through out = w v and the row softmax:
 *
 *     dv_j = sum_i w_ij dout_i
 *     dp_ij = <dout_i, v_j>,   ds_ij = w_ij (dp_ij - D_i)
 *     dq_i = scale sum_j ds_ij k_j,   dk_j = scale sum_i ds_ij q_i
 *
 * Keys that no query row may see (past L_b, or beyond every row under the
 * causal mask) get zero dk and dv; rows with no allowed key get zero dq.
 *   q, k, v, out, dout : bfloat16 inputs, layout above; out and lse are what
 *                        attn_fwd_lse returned for these q, k, v, scale, mask
 *   lse                : fp32 [B, h, Tq] from attn_fwd_lse
 *   delta              : fp32 [2, B, h, Tq] caller-owned workspace: the first
 *                        kernel writes D_i (from the bfloat16 out and dout)
 *                        and lse_i * log2(e) (+inf for an empty row) there,
 *                        the second reads them; no initialisation needed
 *   dq, dk, dv         : bfloat16 outputs shaped like q, k, v (fp32
 *                        accumulation, one rounding each)
 *   other arguments    : as for attn_fwd; d_k = d_v in {64, 128}
 * Two kernels are enqueued on `stream`: the first writes delta and dq, the
 * second reads delta and writes dk, dv.  Outputs may not overlap any input
 * or each other (ATTN_ERR_ALIAS).  Empty work: B or h = 0, or Tq = Tk = 0,
 * is a no-op; Tq = 0 with Tk > 0 writes zero dk, dv (q, out, dout, lse,
 * delta, dq unused); Tk = 0 with Tq > 0 writes zero dq, D = 0 and
 * lse * log2(e) = +inf into delta (k, v, dk, dv unused).
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
             const float* lse, float* delta, void* dq, void* dk, void* dv,
             int B, int h, int Tq, int Tk, int d_k, int d_v, float scale,
             int mask_kind, const int32_t* key_lens, hipStream_t stream);

/*
 * attn_fwd_weights: attn_fwd_lse, then the attention weights themselves,
 *
 *     weights[b,h,i,j] = w_ij = exp(s_ij - lse[b,h,i])   (0 where j is not allowed),
 *
 * written in full as fp32 [B, h, Tq, Tk] -- the second result of the pages'
 * attention() (aiany.app explainer, Step 6: the matrix A = softmax(S) whose
 * rows sum to 1; the cuijiawei.cn snippet returns output and weights), for
 * inspection such as attention heat maps.  The scores are recomputed from q
 * and k; the normaliser is the forward's own, so each row of weights sums to
 * 1 within the bfloat16 rounding of the forward's probabilities (2^-9).
 *   lse     : fp32 [B, h, Tq] (required; as attn_fwd_lse)
 *   weights : fp32 [B, h, Tq, Tk], 16-byte aligned, overlapping no other tensor
 *   other arguments as for attn_fwd (bfloat16 q, k, v, out).
 * Two kernels are enqueued on `stream` (the forward, then the weights).  Rows
 * with no allowed key get all-zero weights.  B, h or Tq = 0 is a no-op;
 * Tk = 0 writes zero outputs and -inf lse (weights unused).
 */
int attn_fwd_weights(const void* q, const void* k, const void* v, void* out, float* lse,
                     float* weights, int B, int h, int Tq, int Tk, int d_k, int d_v,
                     float scale, int mask_kind, const int32_t* key_lens, hipStream_t stream);

/*
 * attn_decode: the operation above for one query row per (b, head) -- the
 * generation loop of the pages, where the decoder emits one token at a time
 * and the newest position attends every cached key (muhitai.com, "What Is
 * Masked Attention?"; notebook chapter, "Masked Attention in the Decoder":
 * the newest row of the causal mask allows all earlier keys).  bfloat16 q, k,
 * v and out; fp32 scores, weights and sums (no bfloat16 rounding before the
 * weighted sum); the output is rounded once to bfloat16.
 *   q, out      : [B, h, 1, d] (i.e. [B, h, d]) bfloat16
 *   k, v        : [B, h, Tk, d] bfloat16, the key/value cache
 *   mask_kind   : ATTN_MASK_NONE or ATTN_MASK_KEYPAD (per-sequence cache
 *                 lengths key_lens[b], clamped to [0, Tk]); ATTN_MASK_CAUSAL is
 *                 rejected (ATTN_ERR_MASK): under the top-left causal reading
 *                 of attn_fwd a single row 0 would see key 0 only, while the
 *                 newest decode position sees the whole valid cache
 *   workspace   : caller-owned device memory of at least
 *                 attn_decode_workspace_bytes(B, h, Tk, d) bytes, 16-byte
 *                 aligned, not overlapping any tensor; it holds the per-split
 *                 partial results between the two kernels and needs no
 *                 initialisation.  Calls that share a workspace must not
 *                 overlap in time (same stream, or synchronised).
 *   other arguments as for attn_fwd; d_k = d_v in {64, 128}.
 * Two kernels are enqueued on `stream`: a split kernel (one work-group per
 * (b, head, chunk of keys)) and a merge kernel.  A row with no valid key
 * (L_b = 0 or Tk = 0) gets zeros.  B or h = 0 is a no-op.
 */
int attn_decode(const void* q, const void* k, const void* v, void* out,
                int B, int h, int Tk, int d_k, int d_v, float scale,
                int mask_kind, const int32_t* key_lens,
                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace attn_decode needs for (B, h, Tk, d); 0 for invalid sizes. */
size_t attn_decode_workspace_bytes(int B, int h, int Tk, int d);

/*
 * attn_decode_static: attn_decode without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  The per-split partials go
 * to a static device array of the library, ATTN_DECODE_STATIC_SCRATCH_BYTES
 * bytes on each GPU the library runs on, held until the process ends; its
 * address is looked up once per device (on the first call with that device
 * current).  The call allocates nothing.
 *   Arguments, results and errors as attn_decode; in addition
 *   ATTN_ERR_WORKSPACE when attn_decode_workspace_bytes(B, h, Tk, d) exceeds
 *   ATTN_DECODE_STATIC_SCRATCH_BYTES (returned before any HIP call), and
 *   ATTN_ERR_HIP (hipErrorInvalidDevice) when `stream` belongs to another
 *   device than the current one.
 * Every call on one GPU uses that GPU's one array, so calls that overlap in
 * time on one GPU (different streams, not synchronised) race and give wrong
 * results; calls in order on one stream are safe.  Nothing in the array needs
 * to start at zero: the split kernel writes every partial the merge reads.
 */
#define ATTN_DECODE_STATIC_SCRATCH_BYTES ((size_t)16 << 20)
int attn_decode_static(const void* q, const void* k, const void* v, void* out,
                       int B, int h, int Tk, int d_k, int d_v, float scale,
                       int mask_kind, const int32_t* key_lens, hipStream_t stream);

/*
 * attn_mha_fwd: multi-head attention forward,
 *
 *     MultiHead = Concat(head_1, ..., head_h) W^O,
 *     head_i = Attention(Xq W_i^Q, Xk W_i^K, Xv W_i^V)
 *
 * ("Attention Is All You Need" notebook chapter, "Multi-Head Self-Attention";
 * cuijiawei.cn, the MultiHeadAttention snippet: head i is columns i*d .. i*d+d-1
 * of each projection, d = d_model / h), with Attention() the operation of
 * attn_fwd (same scale, mask_kind and key_lens meaning).  No bias terms (the
 * formula has none).  Self-attention passes the same pointer for xq, xk, xv.
 *   xq      : bf16 [B, Tq, d_model];  xk, xv : bf16 [B, Tk, d_model]
 *   wq, wk, wv : bf16 [d_model, d_model] (row vector times matrix: x W)
 *   wo      : bf16 [d_model, d_model]
 *   y       : bf16 [B, Tq, d_model]
 *   h       : heads; d_model / h must be 64 or 128
 *   workspace : caller-owned device memory of at least
 *             attn_mha_workspace_bytes(B, Tq, Tk, d_model) bytes, 256-byte
 *             aligned, overlapping no tensor; no initialisation needed; calls
 *             that share it must not overlap in time
 * The projections are this library's GEMM kernel (bf16 operands, fp32
 * accumulation, bf16 results: the projected Q, K, V and the merged heads are
 * rounded to bf16); the attention reads the projections in place.  All work is
 * enqueued on `stream`; nothing is allocated.
 * Errors as attn_fwd, plus ATTN_ERR_WORKSPACE, and ATTN_ERR_TOO_LARGE when
 * B * max(Tq, Tk) exceeds 2^31 - 1 rows.  B or Tq = 0 is a no-op; Tk = 0 gives
 * y = 0.
 */
int attn_mha_fwd(const void* xq, const void* xk, const void* xv,
                 const void* wq, const void* wk, const void* wv, const void* wo, void* y,
                 int B, int Tq, int Tk, int d_model, int h, float scale,
                 int mask_kind, const int32_t* key_lens,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace attn_mha_fwd needs for (B, Tq, Tk, d_model); 0 for invalid sizes. */
size_t attn_mha_workspace_bytes(int B, int Tq, int Tk, int d_model);

/* Static description of a status code (never NULL). */
const char* attn_status_str(int status);

/* The hipError_t of the last failed launch on the calling thread (0 if none). */
int attn_last_hip_error(void);

/* Library version string, e.g. "attn 0.1.0 gfx950". */
const char* attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
