/*
 * fa2mi - exact FlashAttention-2 style attention for AMD Instinct MI355X
 * (gfx950), plus the PSA pack/merge rearrangements around it.
 *
 * C ABI. Every pointer argument is a DEVICE pointer owned by the caller
 * unless stated otherwise; the library never allocates, frees or keeps device
 * memory and holds no state between calls. Every call only validates its
 * arguments and enqueues its kernel(s) on `stream` (a hipStream_t; NULL means
 * the default stream), then returns: results are ready once the caller
 * synchronises that stream.
 *
 * Layout (vision-rs flash_attn2.rs, module doc): attention tensors are flat
 * [BH, N, HEAD_DIM] row-major and contiguous, BH = batch * heads; the caller
 * reshapes [B, H, N, D] tensors to that layout. Query-side tensors (q, o, d_o,
 * dq) are [bh, n_q, head_dim]; key-side tensors (k, v, dk, dv) are
 * [bh, n_k, head_dim]; lse and delta are [bh, n_q] float32. Query and key
 * lengths may differ (same page, "Forward": separate query and key lengths).
 *
 * Element types: all non-float32 tensors of one call share `dt`; accumulation
 * is always float32; outputs are rounded to `dt` with round-to-nearest-even.
 * lse and delta are always float32. LSE is in natural-log units.
 *
 * Supported: head_dim in {32, 64, 128} (other head dims up to 128 through
 * fa2_pad_cols, below); non-causal attention without mask, dropout or bias
 * (the pages describe none).
 *
 * Errors (checked on the host before anything is enqueued; nothing is enqueued
 * when a call fails):
 *   FA2_ERR_INVALID_ARG  a NULL pointer, a pointer not 16-byte aligned, a size
 *                        <= 0, one head's rows larger than 2 GiB
 *                        (n * head_dim * element size; for the PSA calls,
 *                        h * w * key_dim above 2^31 - 1 elements), a softmax
 *                        scale that is not positive and finite, or an
 *                        unknown dtype;
 *   FA2_ERR_UNSUPPORTED  a head_dim / key_dim outside {32, 64, 128};
 *   FA2_ERR_LAUNCH       the HIP runtime refused the launch.
 * fa2_last_error() returns a message for the calling thread's last failure.
 * Faults inside a kernel surface at the caller's next synchronisation.
 * Outputs must not alias inputs. Calls on one stream run in order; calls on
 * different streams writing the same buffers race.
 */
#ifndef FA2MI_H
#define FA2MI_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA2_OK = 0,
    FA2_ERR_INVALID_ARG = 1,
    FA2_ERR_UNSUPPORTED = 2,
    FA2_ERR_LAUNCH = 3
} fa2_status;

typedef enum { FA2_F32 = 0, FA2_F16 = 1, FA2_BF16 = 2 } fa2_dtype;

/* Version of this ABI (bumped on any signature change). */
int32_t fa2_abi_version(void);

/* Short fixed description of a status code. */
const char *fa2_status_str(fa2_status s);

/* Detail message of the calling thread's most recent failed call ("" if none). */
const char *fa2_last_error(void);

/*
 * Forward (vision-rs flash_attn2.rs, "Forward"; vyre-libs
 * flash_attention_2.rs, the tiled builder): for every head b and query row i,
 *   O[b,i,:]  = sum_j softmax_j(scale * q_i . k_j) v_j
 *   lse[b,i]  = log(sum_j exp(scale * q_i . k_j))      (natural log)
 * computed with the online-softmax recurrence over key tiles, so the
 * n_q x n_k score matrix never reaches memory.
 * In: q [bh,n_q,head_dim], k and v [bh,n_k,head_dim] (dt). Out: o
 * [bh,n_q,head_dim] (dt), lse [bh,n_q] (float32), both fully overwritten.
 * `scale` is the softmax scale (usually 1/sqrt(head_dim)); it must be > 0.
 */
fa2_status fa2_fwd(fa2_dtype dt, const void *q, const void *k, const void *v, void *o, float *lse,
                   int64_t bh, int64_t n_q, int64_t n_k, int32_t head_dim, float scale,
                   void *stream);

/*
 * Key-split forward ("flash-decoding"): the same O and lse as fa2_fwd, for
 * shapes with few query rows per head (decoding, short prompts against a
 * long cache), where one workgroup per head and query block would leave most
 * of the device idle. The key rows of each head are cut into consecutive
 * ranges; pass 1 runs the forward's online-softmax recurrence (vision-rs
 * flash_attn2.rs, "Forward") over each range separately, pass 2 merges the
 * ranges by the log-sum-exp rule: with L_s = log sum_{j in range s} e^{s_ij}
 * and O_s the range's softmax output,
 *   lse = log sum_s e^{L_s},   O = sum_s e^{L_s - lse} O_s,
 * which equals the single-range result exactly up to rounding (the same
 * merge joins sequence shards across devices).
 *
 * fa2_fwd_splitkv_plan reports, for num_splits (0: chosen from the sizes,
 * >0: requested; clamped to one range per 64 keys), the number of ranges
 * used (*splits_used) and the workspace the call needs in bytes
 * (*workspace_bytes = splits * bh * n_q * (head_dim + 1) * 4, or 0 when one
 * range is used). Host-only; splits_used and workspace_bytes are host
 * pointers; enqueues nothing.
 *
 * fa2_fwd_splitkv: arguments as fa2_fwd, plus `workspace`, a caller-owned
 * device buffer of `workspace_bytes` bytes (16-byte aligned; may be NULL
 * when the plan needs none), and num_splits as above. The workspace holds
 * float32 partial results between the two passes; its contents on return
 * are unspecified, and two calls in flight must not share one. Enqueues two
 * kernels (one when a single range is used, which is fa2_fwd itself).
 * FA2_ERR_INVALID_ARG also for num_splits < 0 and for a workspace smaller
 * than the plan's size.
 */
fa2_status fa2_fwd_splitkv_plan(fa2_dtype dt, int64_t bh, int64_t n_q, int64_t n_k, int32_t head_dim,
                                int32_t num_splits, int32_t *splits_used, int64_t *workspace_bytes);
fa2_status fa2_fwd_splitkv(fa2_dtype dt, const void *q, const void *k, const void *v, void *o, float *lse,
                           void *workspace, int64_t workspace_bytes,
                           int64_t bh, int64_t n_q, int64_t n_k, int32_t head_dim, float scale,
                           int32_t num_splits, void *stream);

/*
 * Allocation-free key-split forward, for callers that cannot allocate device
 * memory (code under HIP graph capture, serving loops that forbid
 * allocation). Same arguments and results as fa2_fwd_splitkv without the
 * workspace: the float32 partials live in a static device array of
 * fa2_fwd_splitkv_noalloc_max_bytes() bytes (32 MiB) that the library holds
 * on every device it runs on until the process ends. Calls nothing that
 * allocates. The partials are fully written before they are read, so the
 * array needs no clearing and its contents between calls do not matter.
 * All calls on one device share that array: calls that overlap in time on
 * one device (different streams, or different host threads) race and give
 * wrong results; order them on one stream. `stream` must belong to the
 * current device (NULL: the current device's default stream).
 * FA2_ERR_INVALID_ARG, before anything is enqueued, when the plan's
 * partials (splits * bh * n_q * (head_dim + 1) * 4 bytes, as
 * fa2_fwd_splitkv_plan reports) exceed the array, or for a stream of another
 * device; otherwise errors as fa2_fwd_splitkv.
 */
int64_t fa2_fwd_splitkv_noalloc_max_bytes(void);
fa2_status fa2_fwd_splitkv_noalloc(fa2_dtype dt, const void *q, const void *k, const void *v, void *o, float *lse,
                                   int64_t bh, int64_t n_q, int64_t n_k, int32_t head_dim, float scale,
                                   int32_t num_splits, void *stream);

/*
 * Backward pre-pass (vision-rs flash_attn2.rs, "Backward - dQ": the per-row
 * term rowsum(O * dO)): delta[b,i] = sum_d o[b,i,d] * d_o[b,i,d] in float32.
 * In: o, d_o [bh,n_q,head_dim] (dt). Out: delta [bh,n_q] float32, fully
 * overwritten. Must run before fa2_bwd_dq / fa2_bwd_dkdv, which read delta.
 */
fa2_status fa2_bwd_delta(fa2_dtype dt, const void *o, const void *d_o, float *delta,
                         int64_t bh, int64_t n_q, int32_t head_dim, void *stream);

/*
 * Backward, query side (vision-rs flash_attn2.rs, "Backward - dQ"): with
 * p_ij = exp(scale * q_i . k_j - lse_i) recomputed from the saved lse,
 *   dS_ij = p_ij * (d_o_i . v_j - delta_i),   dq_i = scale * sum_j dS_ij k_j.
 * In: q, d_o [bh,n_q,head_dim]; k, v [bh,n_k,head_dim] (dt); lse, delta
 * [bh,n_q] float32 from fa2_fwd and fa2_bwd_delta. Out: dq [bh,n_q,head_dim]
 * (dt), fully overwritten (no zero-initialisation needed).
 */
fa2_status fa2_bwd_dq(fa2_dtype dt, const void *q, const void *k, const void *v, const void *d_o,
                      const float *lse, const float *delta, void *dq,
                      int64_t bh, int64_t n_q, int64_t n_k, int32_t head_dim, float scale,
                      void *stream);

/*
 * Backward, key side (vision-rs flash_attn2.rs, "Backward - dK / dV"): with
 * p_ij and dS_ij as above,
 *   dv_j = sum_i p_ij d_o_i,   dk_j = scale * sum_i dS_ij q_i.
 * Inputs as for fa2_bwd_dq. Out: dk, dv [bh,n_k,head_dim] (dt), fully
 * overwritten. Deterministic: no atomics.
 */
fa2_status fa2_bwd_dkdv(fa2_dtype dt, const void *q, const void *k, const void *v, const void *d_o,
                        const float *lse, const float *delta, void *dk, void *dv,
                        int64_t bh, int64_t n_q, int64_t n_k, int32_t head_dim, float scale,
                        void *stream);

/*
 * Column pad / crop for head dims the attention kernels do not take
 * (vyre-libs flash_attention_2.rs tests run head dims 4, 7, 8 and 16):
 *   dst[r][c] = src[r][c]  for c < min(d_src, d_dst),   0 for d_src <= c < d_dst,
 * over row-major src [rows, d_src] and dst [rows, d_dst] (dt elements; bit
 * copy). Widening q, k and v of any head_dim <= 128 with zero columns to the
 * next supported size (32, 64, 128) leaves every score q . k unchanged and
 * only adds output columns equal to zero, so fa2_fwd / fa2_bwd_* on the padded
 * copies (with the ORIGINAL head_dim's softmax scale) followed by a crop back
 * to d_src columns give O, lse, dq, dk and dv of the original problem. The
 * Python binding's attention_fwd / attention_bwd do exactly that.
 * FA2_ERR_INVALID_ARG for sizes <= 0, NULL or misaligned pointers.
 */
fa2_status fa2_pad_cols(fa2_dtype dt, const void *src, void *dst, int64_t rows, int32_t d_src, int32_t d_dst,
                        void *stream);

/*
 * PSA pack (vision_rs psa.rs, "psa_pack_qkv"): qkv is the NCHW output of the
 * block's qkv convolution, [batch, num_heads*4*key_dim, h, w]; per head its
 * channels are Q, K, V_lo, V_hi, key_dim each. Writes
 *   packed[s][b*num_heads + hd][n][d] = qkv[b][hd*4*key_dim + s*key_dim + d][n]
 * for sections s = 0 Q, 1 K, 2 V_lo, 3 V_hi and pixel n < h*w: packed is
 * [4, batch*num_heads, h*w, key_dim], so each section is a ready [BH, N, D]
 * operand for fa2_fwd (Q, K, V_lo or V_hi). Bit-exact copy. dt is F16, BF16
 * or F32; key_dim in {32, 64, 128}.
 */
fa2_status psa_pack_qkv(fa2_dtype dt, const void *qkv, void *packed,
                        int32_t batch, int32_t num_heads, int32_t key_dim, int32_t h, int32_t w,
                        void *stream);

/*
 * PSA merge (vision_rs psa.rs, "psa_merge_attn_nchw"): o_lo and o_hi are the
 * attention outputs for V_lo and V_hi, [batch*num_heads, h*w, key_dim];
 * writes out NCHW [batch, num_heads*2*key_dim, h, w] with
 *   out[b][hd*2*key_dim + d][n]           = o_lo[b*num_heads + hd][n][d]
 *   out[b][hd*2*key_dim + key_dim + d][n] = o_hi[b*num_heads + hd][n][d].
 * Bit-exact copy.
 */
fa2_status psa_merge_attn(fa2_dtype dt, const void *o_lo, const void *o_hi, void *out,
                          int32_t batch, int32_t num_heads, int32_t key_dim, int32_t h, int32_t w,
                          void *stream);

/*
 * Fused PSA attention forward (vision_rs psa.rs: module doc, "psa_pack_qkv",
 * "psa_merge_attn_nchw" and "FlashAttn2PsaRuntimeOp"): the result of
 * psa_pack_qkv, fa2_fwd on (Q, K, V_lo), fa2_fwd on (Q, K, V_hi) and
 * psa_merge_attn, with scale 1/sqrt(key_dim) as that runtime op fixes it,
 * in one kernel: Q, K and V are read straight from the NCHW qkv activation
 * [batch, num_heads*4*key_dim, h, w] and the output is written straight to
 * NCHW out [batch, num_heads*2*key_dim, h, w]. The two value halves share
 * one probability matrix, so attention runs once with value width
 * 2*key_dim. lse, if not NULL, receives the [batch*num_heads, h*w] float32
 * natural-log LSE (the same for both halves). dt is F16 or BF16 and key_dim
 * 32 or 64 (others: FA2_ERR_UNSUPPORTED); lse must be 4-byte aligned.
 */
fa2_status psa_attn_fused(fa2_dtype dt, const void *qkv, void *out, float *lse,
                          int32_t batch, int32_t num_heads, int32_t key_dim, int32_t h, int32_t w,
                          void *stream);

/*
 * Fused backward of the PSA attention block (vision_rs psa.rs, the block's
 * backward hooks psa_merge_attn_backward -> psa_fa2_backward for V_lo and
 * V_hi -> psa_pack_qkv_backward; vision-rs flash_attn2.rs "Backward - dQ",
 * "Backward - dK / dV"). Given qkv, the block output `out` and its `lse`
 * from psa_attn_fused, and d_out (the gradient of out, NCHW like out), writes
 * d_qkv [batch, num_heads*4*key_dim, h, w], the gradient with respect to
 * qkv: its Q, K, V_lo and V_hi channels, fully overwritten. With
 * p_ij = exp(scale q_i.k_j - lse_i), scale = 1/sqrt(key_dim), and v, d_out
 * the 2*key_dim value channels of a head:
 *   delta_i = sum_c out_ic d_out_ic,   dS_ij = p_ij (d_out_i.v_j - delta_i),
 *   dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i,
 *   dv_j = sum_i p_ij d_out_i
 * (the sum of the two value halves' gradients of the pages' V-split, since
 * both halves share p). `delta` is a caller-owned float32 [batch*num_heads,
 * h*w] buffer (4-byte aligned) that receives delta. Three kernels, no
 * atomics, deterministic. dt F16 or BF16; key_dim 32 with h*w <= 512, or
 * key_dim 64 with h*w <= 128, else FA2_ERR_UNSUPPORTED (psa_block_backward's
 * composition covers the rest).
 * A V-extraction gradient is added afterwards with psa_extract_v_backward.
 */
fa2_status psa_attn_fused_backward(fa2_dtype dt, const void *qkv, const void *out, const float *lse,
                                   const void *d_out, void *d_qkv, float *delta,
                                   int32_t batch, int32_t num_heads, int32_t key_dim, int32_t h, int32_t w,
                                   void *stream);

/*
 * Backward of psa_merge_attn (vision_rs psa.rs, "psa_merge_attn_backward"):
 * d_out is the gradient of the merged NCHW output, [batch,
 * num_heads*2*key_dim, h, w]; writes the gradients of the two attention
 * outputs, [batch*num_heads, h*w, key_dim] each:
 *   d_o_lo[b*num_heads + hd][n][d] = d_out[b][hd*2*key_dim + d][n]
 *   d_o_hi[b*num_heads + hd][n][d] = d_out[b][hd*2*key_dim + key_dim + d][n].
 * Bit-exact copy (the inverse permutation of psa_merge_attn); every element
 * of d_o_lo and d_o_hi is written. dt is F16, BF16 or F32.
 */
fa2_status psa_merge_attn_backward(fa2_dtype dt, const void *d_out, void *d_o_lo, void *d_o_hi,
                                   int32_t batch, int32_t num_heads, int32_t key_dim, int32_t h, int32_t w,
                                   void *stream);

/*
 * Backward of psa_pack_qkv (vision_rs psa.rs, "psa_pack_qkv_backward"):
 * d_packed is the gradient of the packed buffer, [4, batch*num_heads, h*w,
 * key_dim] (sections dQ, dK, dV_lo, dV_hi); writes the NCHW gradient of the
 * qkv activation [batch, num_heads*4*key_dim, h, w]:
 *   d_qkv[b][hd*4*key_dim + s*key_dim + d][n] = d_packed[s][b*num_heads + hd][n][d]
 *                                               (+ d_qk_extra[s][...][n][d] for s < 2).
 * d_qk_extra, if not NULL, is a second [2, batch*num_heads, h*w, key_dim]
 * pair (dQ, dK) added to sections 0 and 1: the V-split block runs attention
 * twice on the same Q and K, and the page's combined backward adds both
 * calls' dQ and dK atomically; here the second call's pair is passed
 * separately and added in fp32 before rounding. Without it the result is a
 * bit-exact copy (the inverse permutation of psa_pack_qkv). d_qkv is
 * overwritten entirely (the page accumulates with atomics because
 * psa_extract_v_backward also adds into the V channels; here that call
 * follows this one on the stream and adds). dt is F16, BF16 or F32.
 */
fa2_status psa_pack_qkv_backward(fa2_dtype dt, const void *d_packed, const void *d_qk_extra, void *d_qkv,
                                 int32_t batch, int32_t num_heads, int32_t key_dim, int32_t h, int32_t w,
                                 void *stream);

/*
 * PSA V extraction (vision_rs psa.rs, "psa_extract_v_nchw"): copies the V
 * channels of the qkv activation [batch, num_heads*4*key_dim, h, w] into v
 * NCHW [batch, num_heads*2*key_dim, h, w]:
 *   v[b][hd*2*key_dim + d][n] = qkv[b][hd*4*key_dim + 2*key_dim + d][n],
 * d < 2*key_dim (V_lo then V_hi). Bit-exact copy.
 */
fa2_status psa_extract_v_nchw(fa2_dtype dt, const void *qkv, void *v,
                              int32_t batch, int32_t num_heads, int32_t key_dim, int32_t h, int32_t w,
                              void *stream);

/*
 * Backward of psa_extract_v_nchw (vision_rs psa.rs, "psa_extract_v_backward"):
 * ADDS the gradient d_v [batch, num_heads*2*key_dim, h, w] into the V
 * channels of d_qkv [batch, num_heads*4*key_dim, h, w] (fp32 add, one
 * rounding); the Q and K channels are not touched. The page accumulates
 * with atomics because psa_pack_qkv_backward writes the same channels; here
 * the two are ordered on the stream instead: call psa_pack_qkv_backward
 * (which overwrites d_qkv) first, then this.
 */
fa2_status psa_extract_v_backward(fa2_dtype dt, const void *d_v, void *d_qkv,
                                  int32_t batch, int32_t num_heads, int32_t key_dim, int32_t h, int32_t w,
                                  void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FA2MI_H */
