/*
 * libswasink -- hybrid sliding-window attention forward for AMD Instinct MI355X (gfx950).
 *
 * The operator (MiMo-V2-Flash Technical Report digest, section 2.2.2 "Learnable
 * Attention Sink Bias"; MiMo-V2 blog, section 2.2): for query row i of head h with
 * key set J(i) = the last `window` positions of its own sequence up to and
 * including i (digest, section 2.2.1: window of 128 tokens),
 *
 *     a_j = scale * <q_i, k_j>,  m = max(max_j a_j, sink_h),
 *     Z   = exp(sink_h - m) + sum_j exp(a_j - m),
 *     o_i = sum_j exp(a_j - m) v_j / Z,      lse_i = m + ln Z.
 *
 * The sink is a learnable per-head scalar that only enters the softmax
 * denominator (a virtual key with no value); it is compared with the scaled
 * logits.  Global-attention layers (digest, section 2.2: one GA layer per five SWA
 * layers) are the same operator with an unbounded window and no sink.  GQA
 * (ICML 2026 keynote write-up, section 02): query head h reads KV head
 * h / (num_q_heads / num_kv_heads).
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers, row-major and contiguous, owned by
 *    the caller.  The library allocates nothing and keeps no state across calls.
 *  - The tensors read or written with 16-byte vector accesses (q, k, v, k_new, v_new,
 *    the caches, prev_k, prev_v, out, dout, dq, dk, dv, the backward workspace and
 *    swa_rope's x) must be 16-byte aligned, as every torch or hipMalloc allocation is;
 *    a misaligned one is refused with SWA_ERR_UNSUPPORTED.  Index, length, score and
 *    fp32 per-row arrays need only their element alignment.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Every
 *    call only enqueues work on `stream` and returns without synchronising.
 *  - Arguments are validated on the host before anything is launched.  On error
 *    a negative swa_status is returned, nothing is launched, and
 *    swa_last_error() (thread-local) describes the problem.  SWA_ERR_HIP reports
 *    a failed launch with the HIP runtime's message.  No C++ exception crosses
 *    this interface.
 *  - dtype selects the element type of q, k, v, caches and out: SWA_DTYPE_F32
 *    (fp32) or SWA_DTYPE_BF16 (bfloat16).  Arithmetic is fp32 in both cases
 *    (bf16 inputs feed bf16 matrix cores with fp32 accumulation; softmax
 *    weights are rounded to bf16 before the weighted sum of values).  sinks and
 *    lse are always fp32; out is written in dtype, rounded to nearest even.
 *  - head_dim must be 64 or 128; num_q_heads must be a multiple of num_kv_heads.
 *  - scale <= 0 selects 1/sqrt(head_dim).
 *  - lse may be NULL (not written).  It holds the natural-log normaliser of each
 *    row, sink included.
 */
#ifndef SWASINK_H
#define SWASINK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SWA_OK = 0,
  SWA_ERR_NULL = -1,        /* a required pointer is NULL */
  SWA_ERR_SHAPE = -2,       /* a size is out of range or inconsistent */
  SWA_ERR_DTYPE = -3,       /* unknown dtype */
  SWA_ERR_UNSUPPORTED = -4, /* valid request this library does not implement */
  SWA_ERR_HIP = -5          /* the HIP runtime reported an error */
} swa_status;

typedef enum { SWA_DTYPE_F32 = 0, SWA_DTYPE_BF16 = 1 } swa_dtype;

#define SWASINK_ABI_VERSION 12

#if defined(__GNUC__) || defined(__clang__)
#define SWASINK_API __attribute__((visibility("default")))
#else
#define SWASINK_API
#endif

/*
 * Causal GQA sliding-window attention with a per-head sink over packed
 * variable-length sequences (technical report digest, sections 2.2.1-2.2.2).
 *
 *  q          [total_tokens, num_q_heads, head_dim]   dtype
 *  k, v       [total_tokens, num_kv_heads, head_dim]  dtype
 *  sinks      [num_q_heads] fp32: the learnable sink logit of each query head
 *  cu_seqlens [num_seqs + 1] int32: sequence s holds tokens cu_seqlens[s] ..
 *             cu_seqlens[s+1]-1; must rise from 0 to total_tokens (not checked on
 *             the device; a violating array gives unspecified output, never an
 *             out-of-bounds access).  No attention crosses a sequence boundary.
 *  max_seqlen upper bound on any sequence length (1 .. total_tokens); only
 *             validated, the kernels derive their tiling from total_tokens.
 *  window     >= 1: row i attends keys max(seq_start, i-window+1) .. i.
 *  out        [total_tokens, num_q_heads, head_dim]   dtype
 *  lse        [total_tokens, num_q_heads] fp32, or NULL
 * total_tokens == 0 is accepted once the sizes validate: nothing is launched, read or
 * written, and the data pointers may then be NULL.
 */
SWASINK_API int swa_sink_prefill(const void* q, const void* k, const void* v, const float* sinks,
                     const int32_t* cu_seqlens, int32_t num_seqs, int32_t total_tokens,
                     int32_t max_seqlen, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, int32_t window, float scale, swa_dtype dtype,
                     void* out, float* lse, void* stream);

/*
 * Global causal attention: the same operator with an unbounded window and no
 * sink (the GA layers of the hybrid block, technical report digest, section 2.2).
 * Arguments as for swa_sink_prefill without sinks and window.
 */
SWASINK_API int ga_causal_prefill(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                      int32_t num_seqs, int32_t total_tokens, int32_t max_seqlen,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float scale,
                      swa_dtype dtype, void* out, float* lse, void* stream);

/*
 * swa_sink_prefill (or, with NULL sinks and an unbounded window, the GA layer) with K
 * and V as one-byte E4M3 codes: the FP8 (E4M3) KV format of the MiMo-V2 blog, section
 * 6, with the same bit layout and per-tensor scales as swa_sink_decode_fp8kv.  The
 * value of a key / value element is its code's value times k_scale / v_scale.  Q, sinks,
 * out and lse keep their types; every other argument, the masking and the outputs are
 * those of swa_sink_prefill.
 *
 *  k, v             [total_tokens, num_kv_heads, head_dim] uint8 E4M3 codes
 *  k_scale, v_scale host fp32, finite and > 0 (SWA_ERR_SHAPE otherwise)
 *  sinks            [num_q_heads] fp32, or NULL for no sink (GA: window = INT32_MAX)
 * The K/V bytes halve against bf16; at window 128 they are 1/9 of the prefill's bytes.
 */
SWASINK_API int swa_sink_prefill_fp8kv(const void* q, const uint8_t* k, const uint8_t* v, float k_scale,
                           float v_scale, const float* sinks, const int32_t* cu_seqlens,
                           int32_t num_seqs, int32_t total_tokens, int32_t max_seqlen,
                           int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t window, float scale, swa_dtype dtype, void* out, float* lse,
                           void* stream);

/*
 * Decode / MTP verify against a window-slot ring buffer per (sequence, KV head).
 * T query tokens per sequence (the current token and T-1 drafts, verified in one
 * pass: technical report digest, section 2.3) attend the cached window plus the
 * new tokens, causal among themselves.
 *
 *  q            [batch, T, num_q_heads, head_dim]   dtype
 *  k_new, v_new [batch, T, num_kv_heads, head_dim]  dtype: the T new tokens, NOT in
 *               the ring (committing accepted tokens is the caller's job)
 *  k_cache, v_cache [batch, num_kv_heads, window, head_dim] dtype, read only
 *  ring_head    [batch] int32: physical slot of the OLDEST cached token (logical
 *               slot 0); logical slot l lives at physical (ring_head + l) mod window.
 *               Values outside [0, window) are reduced modulo window.
 *  sinks        [num_q_heads] fp32
 *  out          [batch, T, num_q_heads, head_dim] dtype
 *  lse          [batch, T, num_q_heads] fp32, or NULL
 * Query t sees logical slots t+1 .. window-1 and new tokens 0 .. t, i.e. exactly
 * `window` keys; logical slot 0 is never read.  Requires 1 <= T < window.
 * batch == 0 is accepted once the sizes validate: nothing is launched, read or written,
 * and the data pointers may then be NULL.
 */
SWASINK_API int swa_sink_decode(const void* q, const void* k_new, const void* v_new, const void* k_cache,
                    const void* v_cache, const int32_t* ring_head, const float* sinks,
                    int32_t batch, int32_t T, int32_t num_q_heads, int32_t num_kv_heads,
                    int32_t head_dim, int32_t window, float scale, swa_dtype dtype, void* out,
                    float* lse, void* stream);

/*
 * swa_sink_decode against an FP8 ring: the caches hold one-byte E4M3 codes (the
 * FP8 (E4M3) format of the MiMo-V2 blog, section 6, used for the KV cache as in the
 * MiMo-V3 / HySparse2 report's FP8-cache sizes; bit layout: sign, 4 exponent bits
 * with bias 7, 3 mantissa bits, subnormals, no infinities, S.1111.111 = NaN).  The
 * value of a cache element is its code's value times k_scale (K) or v_scale (V),
 * one fp32 scale per tensor.  Every other argument, the masking and the outputs
 * are those of swa_sink_decode; the T new tokens keep `dtype`.
 *
 *  k_cache, v_cache [batch, num_kv_heads, window, head_dim] uint8 E4M3 codes, read only
 *  k_scale, v_scale host fp32, finite and > 0 (SWA_ERR_SHAPE otherwise)
 * The ring bytes halve against a bf16 ring; decode is bound by them.
 */
SWASINK_API int swa_sink_decode_fp8kv(const void* q, const void* k_new, const void* v_new,
                    const uint8_t* k_cache, const uint8_t* v_cache, float k_scale, float v_scale,
                    const int32_t* ring_head, const float* sinks, int32_t batch, int32_t T,
                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t window,
                    float scale, swa_dtype dtype, void* out, float* lse, void* stream);

/*
 * Gradients of swa_sink_prefill's output: given dout = dL/dO, returns dL/dq, dL/dk,
 * dL/dv and dL/dsinks, where the sink is the learnable per-head scalar of the
 * technical report digest, section 2.2.2 (the ICML keynote's Q&A, section 06, names
 * its training stability as critical).  With p_ij the forward weights and
 * p_s(i) = exp(sink - lse_i) the sink's: delta_i = dout_i . O_i,
 * da_ij = p_ij (dout_i . v_j - delta_i), dq_i = scale sum_j da_ij k_j,
 * dk_j = scale sum_i da_ij q_i, dv_j = sum_i p_ij dout_i (dk, dv summed over the
 * query heads of each KV head), dsink_h = -sum_i p_s(i) delta_i.  The LSE output is
 * not differentiated.  Since O_i = sum_j p_ij v_j (the sink carries no value),
 * delta_i = sum_j p_ij (dout_i . v_j): the matrix-core path (bf16, head_dim 128,
 * query heads per KV head a multiple of 8, window <= 128) forms it that way from the
 * weights it recomputes and does not read `out`; the other shapes take it from `out`.
 *
 *  q, k, v, sinks, cu_seqlens, num_seqs, total_tokens, max_seqlen, heads, head_dim,
 *  window, scale, dtype: as swa_sink_prefill; sinks may be NULL (no sink, e.g. a GA
 *  layer with window >= the longest sequence), and then dsinks must be NULL too.
 *  out   [total_tokens, num_q_heads, head_dim] dtype: the forward output (required;
 *        read only where delta is taken from it, see above)
 *  lse   [total_tokens, num_q_heads] fp32: the forward log-sum-exp (required)
 *  dout  like out
 *  dq    like q;  dk, dv like k, v;  dsinks [num_q_heads] fp32 (written, not added to)
 *  workspace  device memory of at least swa_sink_prefill_backward_workspace(...) bytes,
 *             owned by the caller, overwritten; calls sharing one workspace must not
 *             overlap.  The library allocates nothing.
 * Deterministic (no atomics).  total_tokens == 0 writes zeros to dsinks (if given) and
 * reads nothing: the other pointers and the workspace may then be NULL.
 */
SWASINK_API int swa_sink_prefill_backward(const void* q, const void* k, const void* v,
                    const float* sinks, const int32_t* cu_seqlens, int32_t num_seqs,
                    int32_t total_tokens, int32_t max_seqlen, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t window, float scale,
                    swa_dtype dtype, const void* out, const float* lse, const void* dout,
                    void* dq, void* dk, void* dv, float* dsinks, void* workspace,
                    int64_t workspace_bytes, void* stream);

/* Bytes of workspace swa_sink_prefill_backward needs (-1 for invalid sizes). */
SWASINK_API int64_t swa_sink_prefill_backward_workspace(int32_t total_tokens, int32_t num_q_heads);

/*
 * swa_sink_prefill_backward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight training loops, harnesses that forbid hipMalloc): the same
 * kernels and results, with the workspace taken from a scratch array the library owns
 * (16 MiB per GPU, a static device array, held until the process ends) instead of an
 * argument.  It calls no allocating routine.  Arguments, layouts, outputs and errors are
 * those of swa_sink_prefill_backward without workspace and workspace_bytes; in
 * addition, total_tokens * num_q_heads must not exceed 2,097,152 (the array holds the
 * 2 x total_tokens x num_q_heads fp32 delta and sink terms), else SWA_ERR_UNSUPPORTED.
 * Every call on one GPU shares that GPU's array, which keeps the last call's contents
 * (nothing in it must start at zero): calls that overlap on one GPU -- on different
 * streams, or from different threads -- race and give unspecified gradients.  Calls
 * ordered on one stream are safe.
 */
SWASINK_API int swa_sink_prefill_backward_noalloc(const void* q, const void* k, const void* v,
                    const float* sinks, const int32_t* cu_seqlens, int32_t num_seqs,
                    int32_t total_tokens, int32_t max_seqlen, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t window, float scale,
                    swa_dtype dtype, const void* out, const float* lse, const void* dout,
                    void* dq, void* dk, void* dv, float* dsinks, void* stream);

/*
 * Rotary position embedding (RoPE), in place.  Bases: 10,000 in SWA layers, 640,000
 * in GA layers and 5,000,000 for GA after the 256K extension (technical report digest,
 * section 3.1); positions keep increasing as the window slides (ICML keynote write-up,
 * section 06).  Rotate-half pairing: for i < head_dim/2, angle = position *
 * rope_base^(-2i/head_dim),
 *   y[i] = x[i] cos - x[i + D/2] sin,   y[i + D/2] = x[i + D/2] cos + x[i] sin,
 * the angle formed and reduced in fp64, the rotation in fp32, rounded to dtype.
 *
 *  x          [rows, heads, head_dim] dtype, rotated in place (e.g. the q or k of a
 *             prefill: rows = tokens)
 *  positions  [rows] int32 device array: position of each row (any int32 value)
 *  rope_base  host fp32, finite and >= 0; 0 leaves x unchanged (nothing is launched)
 * rows == 0 is accepted (x and positions may then be NULL).
 */
SWASINK_API int swa_rope(void* x, const int32_t* positions, int32_t rows, int32_t heads,
                    int32_t head_dim, float rope_base, swa_dtype dtype, void* stream);

/*
 * swa_sink_decode with the rotary embedding applied inside the kernel: q and k_new
 * arrive unrotated, new token t of sequence b sits at position positions[b] + t, and
 * both are rotated (as swa_rope would, rounded to dtype) before attending.  The ring
 * holds keys already rotated at their own positions (swa_ring_append_rope writes
 * them so).  Every other argument and the outputs are those of swa_sink_decode.
 *
 *  positions  [batch] int32 device array: position of new token 0 of each sequence
 *  rope_base  host fp32, finite and >= 0; 0 means no rotation (swa_sink_decode)
 */
SWASINK_API int swa_sink_decode_rope(const void* q, const void* k_new, const void* v_new,
                    const void* k_cache, const void* v_cache, const int32_t* ring_head,
                    const int32_t* positions, const float* sinks, int32_t batch, int32_t T,
                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t window,
                    float scale, float rope_base, swa_dtype dtype, void* out, float* lse,
                    void* stream);

/*
 * swa_sink_decode_rope against an FP8 ring (RoPE: technical report digest, section
 * 3.1; FP8 (E4M3) KV cache: MiMo-V2 blog, section 6, and the MiMo-V3 / HySparse2
 * report): q and k_new arrive unrotated and are
 * rotated in the kernel as in swa_sink_decode_rope; the caches hold E4M3 codes with
 * per-tensor scales as in swa_sink_decode_fp8kv (keys rotated at their own positions
 * before they were encoded: swa_ring_append_fp8kv writes them so).
 *
 *  k_cache, v_cache [batch, num_kv_heads, window, head_dim] uint8 E4M3 codes, read only
 *  k_scale, v_scale host fp32, finite and > 0 (SWA_ERR_SHAPE otherwise)
 *  positions, rope_base as for swa_sink_decode_rope (rope_base 0: swa_sink_decode_fp8kv)
 */
SWASINK_API int swa_sink_decode_rope_fp8kv(const void* q, const void* k_new, const void* v_new,
                    const uint8_t* k_cache, const uint8_t* v_cache, float k_scale, float v_scale,
                    const int32_t* ring_head, const int32_t* positions, const float* sinks,
                    int32_t batch, int32_t T, int32_t num_q_heads, int32_t num_kv_heads,
                    int32_t head_dim, int32_t window, float scale, float rope_base,
                    swa_dtype dtype, void* out, float* lse, void* stream);

/*
 * Commit the accepted tokens of a decode / MTP-verify step to the ring (the drafts the
 * verification rejected never enter it).  For each sequence b, with n = n_accept[b]
 * clamped to [0, T] and h = ring_head[b] reduced modulo window: accepted token t < n
 * is written to physical slot (h + t) mod window (evicting the n oldest), its key
 * rotated at position positions[b] + t (as swa_rope, rounded to dtype) and its value
 * copied; then ring_head[b] = (h + n) mod window.  Other slots are untouched.
 *
 *  k_new, v_new  [batch, T, num_kv_heads, head_dim] dtype: the step's new tokens,
 *                keys unrotated
 *  n_accept      [batch] int32 device array
 *  positions     [batch] int32 device array (position of new token 0); may be NULL
 *                when rope_base == 0 (keys copied as given)
 *  k_cache, v_cache [batch, num_kv_heads, window, head_dim] dtype, updated in place
 *  ring_head     [batch] int32 device array, updated in place
 *  rope_base     host fp32, finite and >= 0; 0 copies the keys unrotated
 * Requires 1 <= T < window.  batch == 0 is accepted (pointers may then be NULL).
 * Calls that touch the same sequences must not overlap.
 */
SWASINK_API int swa_ring_append_rope(const void* k_new, const void* v_new, const int32_t* n_accept,
                    const int32_t* positions, void* k_cache, void* v_cache, int32_t* ring_head,
                    int32_t batch, int32_t T, int32_t num_kv_heads, int32_t head_dim,
                    int32_t window, float rope_base, swa_dtype dtype, void* stream);

/*
 * One MTP step in one call (MTP verification: technical report digest, section 2.3;
 * RoPE: section 3.1): the previous step's accepted tokens are committed to the ring,
 * then the T new tokens are verified against the ring so updated.  The results -- out,
 * lse, the caches and the new head -- are those of swa_ring_append_rope(prev_k, prev_v,
 * prev_accept, prev_positions, k_cache, v_cache, head, prev_T) followed by
 * swa_sink_decode_rope(q, k_new, v_new, k_cache, v_cache, head, positions), where head
 * starts as a copy of ring_head, with one difference: ring_head is only read, and the
 * head after the commit is written to ring_head_out (so the next step passes
 * ring_head_out as its ring_head and this step's k_new / v_new / positions as its
 * prev_k / prev_v / prev_positions).
 *
 *  prev_k, prev_v   [batch, prev_T, num_kv_heads, head_dim] dtype: the previous step's
 *                   new tokens, keys unrotated
 *  prev_accept      [batch] int32 device array: tokens of the previous step to commit,
 *                   clamped to [0, prev_T] (0 for the first step of a sequence)
 *  prev_positions   [batch] int32 device array: position of the previous step's token
 *                   0; may be NULL when rope_base == 0
 *  prev_T           1 <= prev_T < window
 *  k_cache, v_cache [batch, num_kv_heads, window, head_dim] dtype, updated in place
 *  ring_head        [batch] int32 device array, read only
 *  ring_head_out    [batch] int32 device array, written; must not be ring_head
 * Every other argument is as for swa_sink_decode_rope.  With bf16, head_dim 128,
 * window 128, num_q_heads / num_kv_heads a multiple of 8, T <= 4, prev_T <= 4 and
 * rope_base > 0 the step is one kernel launch (the verify reads the committed tokens'
 * rows from prev_k / prev_v); otherwise it runs as the copy of the head and the two
 * calls above, in order on the stream.  prev_k / prev_v must not overlap the caches.
 * batch == 0 is accepted once the sizes validate (pointers may then be NULL).  Calls
 * that touch the same sequences must not overlap.
 */
SWASINK_API int swa_sink_decode_rope_commit(const void* q, const void* k_new, const void* v_new,
                    const int32_t* positions, const void* prev_k, const void* prev_v,
                    const int32_t* prev_accept, const int32_t* prev_positions, int32_t prev_T,
                    void* k_cache, void* v_cache, const int32_t* ring_head, int32_t* ring_head_out,
                    const float* sinks, int32_t batch, int32_t T, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t window, float scale,
                    float rope_base, swa_dtype dtype, void* out, float* lse, void* stream);

/*
 * swa_sink_decode_rope_commit against an FP8 ring: the results are those of
 * swa_ring_append_fp8kv(prev_k, prev_v, prev_accept, prev_positions, k_cache, v_cache,
 * k_scale, v_scale, head, prev_T) followed by swa_sink_decode_rope_fp8kv(q, k_new, v_new,
 * k_cache, v_cache, k_scale, v_scale, head, positions), head starting as a copy of
 * ring_head and the advanced head written to ring_head_out (ring_head is only read).
 *
 *  k_cache, v_cache [batch, num_kv_heads, window, head_dim] uint8 E4M3 codes, updated in
 *                   place (the committed tokens' codes as swa_ring_append_fp8kv writes them)
 *  k_scale, v_scale host fp32, finite and > 0 (SWA_ERR_SHAPE otherwise)
 * Every other argument, the one-launch shapes and the three-launch fallback are as for
 * swa_sink_decode_rope_commit.
 */
SWASINK_API int swa_sink_decode_rope_commit_fp8kv(const void* q, const void* k_new, const void* v_new,
                    const int32_t* positions, const void* prev_k, const void* prev_v,
                    const int32_t* prev_accept, const int32_t* prev_positions, int32_t prev_T,
                    uint8_t* k_cache, uint8_t* v_cache, float k_scale, float v_scale,
                    const int32_t* ring_head, int32_t* ring_head_out, const float* sinks,
                    int32_t batch, int32_t T, int32_t num_q_heads, int32_t num_kv_heads,
                    int32_t head_dim, int32_t window, float scale, float rope_base,
                    swa_dtype dtype, void* out, float* lse, void* stream);

/*
 * swa_ring_append_rope into an FP8 ring (the E4M3 caches swa_sink_decode_fp8kv
 * reads: the FP8 (E4M3) format of the MiMo-V2 blog, section 6, for the KV cache whose
 * FP8 sizes the MiMo-V3 / HySparse2 report quotes; the pages give no rounding, so the
 * one below is the usual one of a rounding conversion, with saturation as FP8 caches
 * are commonly filled): the same slots, head update, clamping and rotation, but each committed
 * element x -- the rotated key rounded to dtype, or the value as given -- is stored as
 * the E4M3 code of x / k_scale (keys) or x / v_scale (values): the exact quotient
 * rounded once to the nearest E4M3 value, ties to the even mantissa, finite
 * magnitudes beyond 448 saturating to 448 (codes 0x7E / 0xFE), zero keeping its sign,
 * and an x that is not finite stored as the NaN code of its sign (0x7F / 0xFF).
 * Rotating a non-finite key gives an unspecified code.
 *
 *  k_cache, v_cache [batch, num_kv_heads, window, head_dim] uint8 E4M3 codes, updated
 *                   in place
 *  k_scale, v_scale host fp32, finite and > 0 (SWA_ERR_SHAPE otherwise)
 * Everything else is as for swa_ring_append_rope.
 */
SWASINK_API int swa_ring_append_fp8kv(const void* k_new, const void* v_new, const int32_t* n_accept,
                    const int32_t* positions, uint8_t* k_cache, uint8_t* v_cache, float k_scale,
                    float v_scale, int32_t* ring_head, int32_t batch, int32_t T,
                    int32_t num_kv_heads, int32_t head_dim, int32_t window, float rope_base,
                    swa_dtype dtype, void* stream);

/*
 * Token selection for sparse attention with a forced recent window (the HySparse2
 * selection of the MiMo-V3 / HySparse2 report: top k tokens by the full-attention
 * layer's scores, 1024 there, plus the most recent 128 always kept).  For each
 * (sequence b, KV head g) row, the candidates are the positions older than the recent
 * window, j < lengths[b] - recent; the min(k, #candidates) with the largest scores are
 * chosen, equal scores going to the lower position, NaN ranking below every number.
 * Exact and deterministic.
 *
 *  scores   [batch, num_kv_heads, max_len] fp32 (position j of sequence b at [b, g, j])
 *  lengths  [batch] int32 device array, clamped to [0, max_len]
 *  indices  [batch, num_kv_heads, k] int32: chosen positions in increasing order, -1 past
 *           the count
 *  counts   [batch, num_kv_heads] int32
 * Requires k >= 0, recent >= 1, max_len >= 1.  batch == 0 is accepted (pointers may then
 * be NULL).
 */
SWASINK_API int swa_topk_select(const float* scores, const int32_t* lengths, int32_t batch,
                    int32_t num_kv_heads, int32_t max_len, int32_t k, int32_t recent,
                    int32_t* indices, int32_t* counts, void* stream);

/*
 * Sparse decode: one query token per sequence -- the newest, at position
 * lengths[b] - 1 -- attends its KV head's selected positions indices[b, g, :counts[b, g]]
 * plus the recent window max(0, L - recent) .. L - 1, with the sink in the denominator
 * when sinks is given (the operator of swa_sink_prefill on that key set).
 *
 *  q            [batch, num_q_heads, head_dim] dtype
 *  k_cache, v_cache [batch, num_kv_heads, max_len, head_dim] dtype (the full-attention
 *               layer's cache, shared with the sparse layers)
 *  lengths      [batch] int32, clamped to [1, max_len]
 *  indices, counts  as written by swa_topk_select (the listed positions must be distinct
 *               and older than the recent window; out-of-range entries are clamped into the
 *               sequence, never read out of bounds); counts clamped to [0, k]
 *  sinks        [num_q_heads] fp32, or NULL (no sink)
 *  out          [batch, num_q_heads, head_dim] dtype;  lse [batch, num_q_heads] fp32 or NULL
 * Requires recent >= 1 and k + recent <= 8192.  batch == 0 is accepted.
 */
SWASINK_API int swa_sparse_decode(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* lengths, const int32_t* indices, const int32_t* counts,
                    const float* sinks, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                    int32_t head_dim, int32_t max_len, int32_t k, int32_t recent, float scale,
                    swa_dtype dtype, void* out, float* lse, void* stream);

/*
 * MTP verify in a sparse layer: the newest T tokens of each sequence are the queries
 * (positions p_t = L - T + t, t < T, with L = lengths[b]; their K/V already in the
 * caches).  Query t attends its own most recent window max(0, p_t - recent + 1) .. p_t
 * and the selected positions (indices[b, g, :counts[b, g]]) below that window: a
 * selected position inside the window is counted once, as part of it (reading of the
 * HySparse2 selection for drafts; with T = 1 this is swa_sparse_decode).  The selection
 * must be increasing, as swa_topk_select writes it.
 *
 *  q     [batch, T, num_q_heads, head_dim] dtype
 *  out   [batch, T, num_q_heads, head_dim] dtype
 *  lse   [batch, T, num_q_heads] fp32, or NULL
 *  T     1 <= T <= max_len; k + recent + T - 1 <= 8192
 * Lengths below T are taken as T.  Every other argument is as for swa_sparse_decode; the
 * matrix-core kernel takes T <= 2 (bf16, head_dim 128, groups of 8k heads), other shapes
 * the vector kernel.
 */
SWASINK_API int swa_sparse_decode_mtp(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* lengths, const int32_t* indices, const int32_t* counts,
                    const float* sinks, int32_t batch, int32_t T, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t max_len, int32_t k,
                    int32_t recent, float scale, swa_dtype dtype, void* out, float* lse,
                    void* stream);

/*
 * swa_sparse_decode_mtp over an FP8 cache: k_cache and v_cache hold E4M3 codes, element
 * value = code value * k_scale (K) or v_scale (V), as the FP8 ring of swa_sink_decode_fp8kv
 * (MiMo-V2-Flash report, FP8 KV cache; HySparse2 selection over it).  The codes are decoded
 * exactly and scaled in fp32, so the result is swa_sparse_decode_mtp's on the dequantised
 * cache up to fp32 rounding.
 *
 *  k_cache, v_cache [batch, num_kv_heads, max_len, head_dim] uint8 E4M3 codes
 *  k_scale, v_scale finite, > 0
 * Every other argument is as for swa_sparse_decode_mtp (T = 1 is the single-token step;
 * the matrix-core kernel takes the same shapes).
 */
SWASINK_API int swa_sparse_decode_fp8kv(const void* q, const uint8_t* k_cache, const uint8_t* v_cache,
                    float k_scale, float v_scale, const int32_t* lengths, const int32_t* indices,
                    const int32_t* counts, const float* sinks, int32_t batch, int32_t T,
                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t max_len,
                    int32_t k, int32_t recent, float scale, swa_dtype dtype, void* out, float* lse,
                    void* stream);

/* Message for the last non-OK return on the calling thread ("" if none). */
SWASINK_API const char* swa_last_error(void);

/* SWASINK_ABI_VERSION of the built library. */
SWASINK_API int32_t swa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SWASINK_H */
