/*
 * sdpa.h — C ABI of the MI355X (gfx950) scaled dot-product attention library.
 *
 * The operation is Eq. (1) of the page 《精读 Attention Is All You Need：原始
 * Transformer 论文》 (section "缩放点积注意力：点积为什么要缩放"):
 *
 *     Attention(Q, K, V) = softmax(Q Kᵀ · scale) V,   scale = 1/√d_k by default,
 *
 * applied independently to each of B·h (batch, head) pairs, as the multi-head
 * section of the same page runs h heads in parallel.  The three uses the pages
 * list (《Attention Is All You Need：注意力就是你所需要的一切》 §3.2.3) are all
 * this one call:
 *   - encoder self-attention:            n == m, mask_kind = SDPA_MASK_NONE;
 *   - decoder (masked) self-attention:   n == m, mask_kind = SDPA_MASK_CAUSAL
 *                                        (query i sees keys j <= i, inclusive);
 *   - encoder–decoder attention:         queries from the decoder (n), keys and
 *                                        values from the encoder (m), n != m allowed.
 * Illegal logits are set to −∞ before the softmax, so their weights are exactly
 * zero (same §3.2.3).  A query row that has no legal key returns the zero vector.
 *
 * Names: n = number of queries, m = number of keys/values, as in the page
 * 《企业官网建设流程全解析》 §2.2 (Q is n×d_k, K is m×d_k, V is m×d_v).
 */
#ifndef SDPA_H
#define SDPA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Only the entry points below are exported from libsdpa.so. */
#define SDPA_API __attribute__((visibility("default")))

/* Status codes returned by every entry point.  No exception crosses the ABI. */
#define SDPA_OK               0
#define SDPA_ERR_NULL        -1 /* a required pointer is NULL                        */
#define SDPA_ERR_SHAPE       -2 /* a dimension < 1, or an element count overflows   */
#define SDPA_ERR_UNSUPPORTED -3 /* d_k / d_v, dtype or option not supported here    */
#define SDPA_ERR_ALIGN       -4 /* a pointer is not 16-byte aligned                  */
#define SDPA_ERR_MASK        -5 /* unknown mask_kind, causal with n != m, bad window */
#define SDPA_ERR_DTYPE       -6 /* unknown dtype                                     */
#define SDPA_ERR_LAUNCH      -7 /* the HIP runtime refused this call's kernel launch */
#define SDPA_ERR_SCALE       -8 /* scale (or keep_scale) not finite, or not > 0     */
#define SDPA_ERR_ALIAS       -9 /* out overlaps q, k, v or key_lens                   */
#define SDPA_ERR_WORKSPACE  -10 /* workspace smaller than its *_workspace_bytes size */
#define SDPA_ERR_SCRATCH    -11 /* a call needs more than the library's static scratch */

/* Size of the library's static device scratch (per GPU), used by
 * sdpa_forward_ex_noalloc in place of a caller's workspace. */
#define SDPA_NOALLOC_SCRATCH_BYTES (8u << 20)

/* Element types (input and output share one type). */
#define SDPA_F32  0 /* fp32 in, fp32 arithmetic, fp32 out                          */
#define SDPA_BF16 1 /* bf16 in, fp32 accumulate and softmax, bf16 out (RNE)        */

/* Mask kinds. */
#define SDPA_MASK_NONE   0
#define SDPA_MASK_CAUSAL 1 /* inclusive: query i sees keys j <= i; needs n == m    */

/* Window alignment (sdpa_forward_window). */
#define SDPA_ALIGN_TOP_LEFT     0 /* query i is at key position i                  */
#define SDPA_ALIGN_BOTTOM_RIGHT 1 /* query i is at key position i + L - n          */

/*
 * sdpa_forward — one fused forward pass over all B·h heads.
 *
 * q        device pointer, [B, h, n, d_k], contiguous row-major, element type `dtype`.
 * k        device pointer, [B, h, m, d_k], contiguous.
 * v        device pointer, [B, h, m, d_v], contiguous.
 * out      device pointer, [B, h, n, d_v], contiguous; written completely (rows
 *          with no legal key are written as zeros).  Must not overlap q, k, v, key_lens.
 * B, h     batch size and number of heads (>= 1).
 * n, m     number of queries and of keys/values per head (>= 1).  One head's
 *          rows of any of the four tensors must span less than 2^31 bytes
 *          (n·d·size and m·d·size; the kernels use 32-bit offsets within a
 *          head), else SDPA_ERR_SHAPE.
 * d_k, d_v query/key and value widths: d_k == d_v == 64 for both dtypes; for
 *          SDPA_BF16 also d_k == d_v == 16, 32, 128 or 512, and d_v == 64 with
 *          d_k == 16 or 32 (the model variants of 《精读 Attention Is All
 *          You Need：原始 Transformer 论文》 Table 3, rows (A), (B) and (C)).
 *          Other pairs: SDPA_ERR_UNSUPPORTED.
 * scale    multiplier of the dot products; pass 1/sqrt(d_k) for Eq. (1).  Must
 *          be finite and > 0 (scale = 1 runs the unscaled dot-product form).
 * mask_kind SDPA_MASK_NONE or SDPA_MASK_CAUSAL.
 * key_lens NULL for no key padding, else a DEVICE pointer to int32[B]: key j of
 *          batch element b is legal only if j < clamp(key_lens[b], 0, m).  It
 *          applies to every head of b and to keys only; query rows are never
 *          masked.  K and V rows at j >= key_lens[b] are never read and may
 *          hold anything (also NaN).  Causally hidden keys are read and must be
 *          finite.
 * dtype    SDPA_F32 or SDPA_BF16.
 * stream   a hipStream_t (as void*; NULL = the default stream).
 *
 * All device pointers must be 16-byte aligned.  The call is asynchronous on
 * `stream`: it validates the arguments on the host (before any HIP call),
 * enqueues one kernel, and returns.  It allocates nothing, keeps no pointer
 * after returning, holds no mutable global state and is thread-safe.  The
 * caller owns every buffer.  Returns SDPA_OK or a negative status.  Before
 * launching, every entry point clears the thread's pending HIP error (left by
 * earlier, unrelated calls that no one collected), so SDPA_ERR_LAUNCH always
 * means that this call's own launch was refused.
 */
SDPA_API int sdpa_forward(const void* q, const void* k, const void* v, void* out,
                 int32_t B, int32_t h, int32_t n, int32_t m, int32_t d_k, int32_t d_v,
                 float scale, int32_t mask_kind, const int32_t* key_lens,
                 int32_t dtype, void* stream);

/*
 * sdpa_forward_window — restricted attention: each query sees only a window of
 * keys around its own position.
 *
 * The pages propose restricting self-attention to a neighbourhood of size r
 * around each output position for long sequences (《精读 Attention Is All You
 * Need：原始 Transformer 论文》 Table 1 and the discussion after it;
 * 《Attention Is All You Need：注意力就是你所需要的一切》 §4).  Here query row i
 * has the aligned position
 *     c_i = i                 (align = SDPA_ALIGN_TOP_LEFT), or
 *     c_i = i + L_b - n       (align = SDPA_ALIGN_BOTTOM_RIGHT: the n queries are
 *                              the last n positions of the L_b keys, as in a
 *                              decoder step against its cached keys),
 * where L_b = clamp(key_lens[b], 0, m), or m without key_lens.  Key j is legal
 * for query i iff
 *     j < L_b,  j >= c_i - window_left (if window_left >= 0),
 *     and j <= c_i + window_right (if window_right >= 0);
 * window_left / window_right = -1 leave that side unbounded.  A neighbourhood
 * of size r centred on the query is window_left = window_right = r/2 (rounded
 * down).  sdpa_forward's SDPA_MASK_CAUSAL is the window (-1, 0), top-left;
 * SDPA_MASK_NONE is (-1, -1).  Any n and m are allowed.  A query with no
 * legal key returns the zero vector.
 *
 * Every other argument, the layout, ownership, execution and error behaviour
 * are those of sdpa_forward.  Additional errors: SDPA_ERR_MASK if a window
 * side is < -1 or align is not one of the two SDPA_ALIGN_* values.  Keys
 * outside a query's window but below L_b may be read (with weight exactly
 * zero) and must be finite.
 */
SDPA_API int sdpa_forward_window(const void* q, const void* k, const void* v, void* out,
                 int32_t B, int32_t h, int32_t n, int32_t m, int32_t d_k, int32_t d_v,
                 float scale, int32_t window_left, int32_t window_right, int32_t align,
                 const int32_t* key_lens, int32_t dtype, void* stream);

/*
 * The multi-head attention sublayer (bf16), the pages' MultiHead
 * (《精读 Attention Is All You Need：原始 Transformer 论文》 multi-head section;
 * 《Attention Is All You Need：注意力就是你所需要的一切》 §3.2.2):
 *
 *     out = Concat(head_1, …, head_h) W^O,
 *     head_i = Attention(x_q W_i^Q, x_kv W_i^K, x_kv W_i^V),
 *
 * with Attention as in sdpa_forward_window (scale, key window, key_lens).
 * Self-attention passes the same tensor as x_q and x_kv; encoder–decoder
 * attention passes the decoder states as x_q and the encoder output as x_kv.
 * The pages' projections carry no bias, and neither do these.
 *
 * x_q      device, [B, n, d_model] bf16, contiguous.
 * x_kv     device, [B, m, d_model] bf16, contiguous (may equal x_q).
 * w_q, w_k device, [h·d_k, d_model] bf16: row i·d_k + j is column j of W_i^Q
 *          (resp. W_i^K), i.e. the [out features, in features] layout.
 * w_v      device, [h·d_v, d_model] bf16, row i·d_v + j = column j of W_i^V.
 * w_o      device, [d_model, h·d_v] bf16: the transpose of W^O.
 * out      device, [B, n, d_model] bf16, written completely; must not overlap
 *          any input, weight or the workspace.
 * d_k, d_v d_k = d_v = 32, 64 or 128 with h·d_k a multiple of 64 (the model
 *          variants' head widths); d_model a multiple of 64; dtype SDPA_BF16
 *          (other values: SDPA_ERR_UNSUPPORTED, or SDPA_ERR_DTYPE if unknown).
 * workspace, workspace_bytes
 *          device scratch of at least sdpa_mha_workspace_bytes(...) bytes,
 *          16-byte aligned, owned by the caller; it receives the projected
 *          Q, K, V and the attention output.  Too small: SDPA_ERR_WORKSPACE.
 * Every tensor (and the workspace) must stay below 2^31 bytes (else
 * SDPA_ERR_SHAPE).  All other arguments and rules as in sdpa_forward_window.
 * Enqueues three kernels on `stream` (projections, attention, output
 * projection) and returns; allocates nothing.
 */
SDPA_API size_t sdpa_mha_workspace_bytes(int32_t B, int32_t n, int32_t m, int32_t h, int32_t d_k,
                                         int32_t d_v);
SDPA_API int sdpa_mha_forward(const void* x_q, const void* x_kv, const void* w_q, const void* w_k,
                              const void* w_v, const void* w_o, void* out, int32_t B, int32_t n,
                              int32_t m, int32_t d_model, int32_t h, int32_t d_k, int32_t d_v,
                              float scale, int32_t window_left, int32_t window_right,
                              int32_t align, const int32_t* key_lens, int32_t dtype,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * sdpa_forward_lse — sdpa_forward_window that also returns, for every query
 * row, the natural log of its softmax denominator:
 *
 *     lse[b, h, i] = ln Σ_j exp(scale · q_i · k_j)   over the legal keys j,
 *
 * and −∞ for a row with no legal key.  The weights of Eq. (1) are then
 * exp(scale · q_i · k_j − lse_i), which is how sdpa_backward recomputes them
 * without storing the n × m weight matrix.
 *
 * lse      device, float [B, h, n], contiguous, 4-byte aligned, written
 *          completely; must not overlap any other argument.
 * dtype    SDPA_BF16 or SDPA_F32 (the fp32 kernels form it from their fp32
 *          running sum, to a few fp32 ulps of |lse|).
 * Everything else as in sdpa_forward_window; `out` is bitwise the same as
 * sdpa_forward_window's.
 */
SDPA_API int sdpa_forward_lse(const void* q, const void* k, const void* v, void* out, float* lse,
                              int32_t B, int32_t h, int32_t n, int32_t m, int32_t d_k, int32_t d_v,
                              float scale, int32_t window_left, int32_t window_right,
                              int32_t align, const int32_t* key_lens, int32_t dtype, void* stream);

/*
 * sdpa_forward_ex — sdpa_forward_window with an optional log-sum-exp output
 * and an optional workspace.
 *
 * lse        NULL, or as in sdpa_forward_lse (either dtype).
 * workspace  NULL, or device scratch of workspace_bytes >= the size
 *            sdpa_forward_workspace_bytes gives, 16-byte aligned, owned by the
 *            caller, overlapping no other argument.  With it, decoder steps
 *            against long key caches (bf16, d = 64, n <= 16, any B·h) split
 *            each head's keys into pieces on separate workgroups (1024 keys,
 *            or down to 256 with fewer heads, towards 1024 pieces in all;
 *            only when that gives at least two pieces per head) and merge the
 *            partial softmaxes in a second launch,
 *            which keeps the CUs busy when there are few heads (one sequence
 *            decoding alone) or when cache lengths differ.  The
 *            output then differs from the workspace-free call by rounding only
 *            (the fp32 partial sums are added in another order); each path is
 *            deterministic.  A workspace smaller than needed: SDPA_ERR_WORKSPACE.
 * Everything else as in sdpa_forward_window.
 *
 * sdpa_forward_workspace_bytes returns the workspace such a call would use,
 * and 0 when it would use none (then any workspace argument is ignored).
 */
SDPA_API size_t sdpa_forward_workspace_bytes(int32_t B, int32_t h, int32_t n, int32_t m, int32_t d_k,
                                             int32_t d_v, int32_t dtype);
SDPA_API int sdpa_forward_ex(const void* q, const void* k, const void* v, void* out, float* lse,
                             int32_t B, int32_t h, int32_t n, int32_t m, int32_t d_k, int32_t d_v,
                             float scale, int32_t window_left, int32_t window_right, int32_t align,
                             const int32_t* key_lens, int32_t dtype, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * sdpa_forward_strided — sdpa_forward_ex on tensors laid out at any element
 * strides, e.g. the token-major [B, len, h, d] layout in which the multi-head
 * section of 《精读 Attention Is All You Need：原始 Transformer 论文》 writes
 * Concat(head_1, …, head_h) (row i of every head side by side), read and
 * written in place without a transpose.
 *
 * strides   NULL (then this is sdpa_forward_ex on the packed [B, h, len, d]
 *           layout), or a HOST array of 12 int64 element strides: batch, head
 *           and row stride of q, then of k, v and out, in that order.  Element
 *           (b, head, i, j) of a tensor is at base + b·batch + head·head_stride
 *           + i·row + j: the last dimension is contiguous.  Rules:
 *             * batch and head strides >= 0 (0 shares one tensor across that
 *               dimension, e.g. one K/V head for all query heads);
 *             * row stride >= the row width (d_k or d_v): rows never overlap;
 *             * every stride times the element size is a multiple of 16;
 *             * one head's rows span less than 2^31 bytes, and 64 rows at its
 *               row stride do too;
 *             * the output's (batch, head, row) rows are pairwise disjoint;
 *           else SDPA_ERR_SHAPE, SDPA_ERR_ALIGN or SDPA_ERR_ALIAS.  out, lse
 *           and the workspace must not overlap the span of any input, judged
 *           from the first to the last element each layout reaches
 *           (SDPA_ERR_ALIAS).
 * Everything else, lse and workspace included, as in sdpa_forward_ex; lse
 * stays packed [B, h, n].  Every forward kernel takes the strides, so the
 * arithmetic, and the result, is that of the packed call on the same values.
 */
SDPA_API int sdpa_forward_strided(const void* q, const void* k, const void* v, void* out, float* lse,
                                  int32_t B, int32_t h, int32_t n, int32_t m, int32_t d_k,
                                  int32_t d_v, float scale, int32_t window_left,
                                  int32_t window_right, int32_t align, const int32_t* key_lens,
                                  int32_t dtype, const int64_t* strides, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * sdpa_forward_ex_noalloc — sdpa_forward_ex for callers that cannot allocate
 * device memory (code under HIP graph capture, tight decoder-step serving
 * loops, harnesses that forbid hipMalloc): the same call and the same kernels,
 * but the split-key workspace is the library's own static device array of
 * SDPA_NOALLOC_SCRATCH_BYTES, one per GPU, held until the process ends.
 *
 * Arguments as in sdpa_forward_ex, without workspace and workspace_bytes.
 * When sdpa_forward_workspace_bytes(...) is 0 the call uses no scratch and is
 * sdpa_forward_ex with workspace = NULL.  When it exceeds
 * SDPA_NOALLOC_SCRATCH_BYTES the call returns SDPA_ERR_SCRATCH before any HIP
 * call and launches nothing.  The output is bitwise that of sdpa_forward_ex
 * with a workspace.
 *
 * Allocates nothing and calls no allocating routine.  The first call on a
 * device looks up that device's copy of the array (hipGetSymbolAddress, on
 * the calling thread's current device); make that first call outside graph
 * capture.  Every call on one GPU shares its array and leaves its contents
 * there (no call needs it zeroed: each call's merge launch reads only what its
 * own split launch wrote): calls that may overlap on one GPU (other streams,
 * other host threads) race on it and must be serialised by the caller, e.g.
 * by issuing them on one stream.  A runtime error in the lookup returns
 * SDPA_ERR_LAUNCH.
 */
SDPA_API int sdpa_forward_ex_noalloc(const void* q, const void* k, const void* v, void* out, float* lse,
                                     int32_t B, int32_t h, int32_t n, int32_t m, int32_t d_k,
                                     int32_t d_v, float scale, int32_t window_left,
                                     int32_t window_right, int32_t align, const int32_t* key_lens,
                                     int32_t dtype, void* stream);

/*
 * sdpa_backward — the gradient of Eq. (1) (bf16 or fp32).  The pages train the model
 * through attention but print only the forward pass; by the chain rule, for
 * any loss with output gradient dO:
 *
 *     dV = Pᵀ dO,  dP = dO Vᵀ,  dS = P ∘ (dP − D) with D_i = dO_i · O_i,
 *     dQ = scale · dS K,  dK = scale · dSᵀ Q,
 *
 * where P = exp(scale · Q Kᵀ − lse) row-wise over the legal keys (masked
 * connections get no gradient; a row with no legal key passes none back).
 *
 * q, k, v   the forward inputs, as in sdpa_forward_window.
 * out       the forward output O, [B, h, n, d_v].
 * dout      dO, [B, h, n, d_v], of the inputs' dtype.
 * lse       the forward pass's lse (sdpa_forward_lse), float [B, h, n].
 * dq        device, [B, h, n, d_k] of the inputs' dtype, written completely.
 * dk, dv    device, [B, h, m, d_k] and [B, h, m, d_v] of the inputs' dtype, written completely
 *           (rows of keys at or past key_lens[b] are zero).
 * scale, window_left, window_right, align, key_lens
 *           exactly as given to the forward pass.
 * workspace, workspace_bytes
 *           device scratch of at least sdpa_backward_workspace_bytes(B, h, n)
 *           bytes, 16-byte aligned, owned by the caller (it receives D and
 *           lse · log2 e per row).  Too small: SDPA_ERR_WORKSPACE.
 * dtype     SDPA_BF16 (P and dS rounded to bf16 for their products, as in
 *           the forward pass) or SDPA_F32 (fp32 throughout).
 * d_k, d_v  bf16: d_k == d_v == 32, 64 or 128; fp32: d_k == d_v == 64 (other
 *           pairs: SDPA_ERR_UNSUPPORTED).
 * The outputs and the workspace must not overlap each other or any input
 * (SDPA_ERR_ALIAS).  All tensors 16-byte aligned, lse and key_lens 4-byte
 * aligned.  Enqueues two kernels on `stream` (dQ, then dK and dV) and
 * returns; allocates nothing; uses no atomics, so the result is bitwise
 * reproducible.  Other errors as in sdpa_forward_window.
 */
SDPA_API size_t sdpa_backward_workspace_bytes(int32_t B, int32_t h, int32_t n);
SDPA_API int sdpa_backward(const void* q, const void* k, const void* v, const void* out,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv,
                           int32_t B, int32_t h, int32_t n, int32_t m, int32_t d_k, int32_t d_v,
                           float scale, int32_t window_left, int32_t window_right, int32_t align,
                           const int32_t* key_lens, int32_t dtype, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * Attention dropout (training).  The pages train with dropout (《Attention Is
 * All You Need：注意力就是你所需要的一切》 §5.4, citing the dropout paper [33])
 * and tune an attention dropout for parsing (same page, §6.3) without placing
 * it; here it acts on the weights after the softmax of Eq. (1):
 *
 *     O = (P ∘ Z) V · keep_scale,    P = softmax(scale · Q Kᵀ) over the legal keys,
 *
 * with Z the caller's keep mask (draw Z_ij = 1 with probability 1 − p and
 * pass keep_scale = 1/(1 − p) for the usual unbiased form).  The softmax is
 * unchanged: its normaliser, and lse, count every legal key, kept or not.
 *
 * sdpa_forward_dropout: arguments as in sdpa_forward_window, plus
 * lse        optional (NULL or float [B, h, n], as in sdpa_forward_lse).
 * keep_mask  device, uint32 [B, h, n, ⌈m/32⌉], 4-byte aligned, read only: bit
 *            (j mod 32) of word ⌊j/32⌋ of row (b, head, i) is 1 to keep
 *            weight (i, j).  Bits of illegal keys and past m are ignored.
 * keep_scale finite and > 0 (else SDPA_ERR_SCALE).
 * dtype SDPA_BF16 and d_k == d_v ∈ {32, 64, 128} only (else SDPA_ERR_UNSUPPORTED).  out
 * and lse must not overlap the mask or the inputs (SDPA_ERR_ALIAS).
 *
 * sdpa_backward_dropout: the gradient of that forward pass for the same mask
 * and factor (dV = (P ∘ Z)ᵀ dO · keep_scale, dP = (dO Vᵀ) ∘ Z · keep_scale,
 * then as in sdpa_backward, whose other arguments it takes unchanged; `out`
 * and `lse` are the dropout forward's).  Widths and dtype as for the forward;
 * the outputs and workspace must not overlap the mask either.
 */
SDPA_API int sdpa_forward_dropout(const void* q, const void* k, const void* v, void* out, float* lse,
                                  int32_t B, int32_t h, int32_t n, int32_t m, int32_t d_k, int32_t d_v,
                                  float scale, int32_t window_left, int32_t window_right, int32_t align,
                                  const int32_t* key_lens, const uint32_t* keep_mask, float keep_scale,
                                  int32_t dtype, void* stream);
SDPA_API int sdpa_backward_dropout(const void* q, const void* k, const void* v, const void* out,
                                   const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                   int32_t B, int32_t h, int32_t n, int32_t m, int32_t d_k, int32_t d_v,
                                   float scale, int32_t window_left, int32_t window_right, int32_t align,
                                   const int32_t* key_lens, const uint32_t* keep_mask, float keep_scale,
                                   int32_t dtype, void* workspace, size_t workspace_bytes, void* stream);

/* Static text for a status code (never NULL). */
SDPA_API const char* sdpa_strerror(int status);

/* Library version: major*10000 + minor*100 + patch. */
SDPA_API int sdpa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SDPA_H */
