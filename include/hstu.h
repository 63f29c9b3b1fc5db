/*
 * hstu.h -- C ABI of the HSTU jagged causal attention forward for AMD MI355X
 * (gfx950).
 *
 * Operation (Ascend HSTU blog "都是生成式推荐，为什么昇腾这么快？", §1: the
 * formula HSTU(Q,K,V) = (mask/n) * silu(Q K^T / alpha^-1) V and its five-step
 * PyTorch definition; §3.2: causal mask generated inside the operator, diagonal
 * blocks lower-triangular, blocks above the diagonal skipped; §4.2: jagged
 * values + offsets input):
 *
 *   for every sequence i (tokens off[i] .. off[i+1]-1), head h, local row r:
 *     out[off[i]+r][h][:] = (1/n) * sum_{c=0..r} silu(alpha * <q[off[i]+r][h], k[off[i]+c][h]>)
 *                                                * v[off[i]+c][h][:]
 *   silu(x) = x / (1 + e^-x)   (HSTU paper translation "行动胜于言语…", §3: phi_2 = SiLU)
 *
 * Sequences never attend to each other; the mask keeps c <= r (diagonal
 * included) and multiplies after SiLU, so masked terms are exactly zero.
 *
 * Layouts (all device pointers, caller-owned):
 *   q, k, v, out : row-major (T, heads, d) of one element type, T = off[num_seqs];
 *                  the row of token t, head h starts at element (t*heads + h)*d.
 *                  16-byte aligned.  out must not overlap q, k, v or the offsets.
 *   seq_offsets  : int32[num_seqs + 1], off[0] = 0, non-decreasing.  Lives on the
 *                  device; the host never reads it.  Empty sequences are allowed.
 *   alpha, n     : float32 scalars; alpha multiplies the scores before SiLU, n
 *                  divides the result.  n must be finite and non-zero, alpha finite.
 *
 * Element types: bfloat16 and float16 run on the matrix cores with float32
 * accumulation, the SiLU in float32 and the weights rounded to the input type
 * (nearest even) before the second product; float32 runs both products in
 * float32.  out has the same element type as q/k/v, rounded to nearest even.
 * Supported head sizes: d = 64 and d = 128; heads >= 1; num_seqs >= 0 (0 is a
 * no-op).
 *
 * Streams and memory: every device operation is enqueued on `stream` (0 = the
 * null stream); no call synchronises the host except hstu_validate_offsets and
 * hstu_profile_read.  The library owns a small grow-only scratch area per
 * (device, stream): a work list of 12 bytes per sequence plus a header.  It is
 * allocated on the first call that needs more; later calls with no more
 * sequences allocate nothing.  Two calls on the same stream are ordered by the
 * stream; calls on different streams use different scratch areas.  Host
 * threads may call on one stream concurrently: the library serialises the
 * enqueueing of calls per (device, stream).  A call is
 * one kernel for batches of up to 256 sequences and 2048 (sequence, head)
 * pairs (the attention kernel ranks the sequences itself), two kernels
 * otherwise (a work-list kernel, then the attention kernel); the first call on
 * a new scratch area always takes the two-kernel form.
 *
 * Graph capture: a call made while `stream` is being captured into a HIP
 * graph (hipStreamIsCapturing) is recorded with a scratch area of its own,
 * allocated during the capture (the calling thread switches to relaxed
 * capture mode for that allocation) and kept until the process ends, since
 * the graph holds its address; its first recorded kernel zeroes that area's
 * queue counters, so every replay starts from the same state whatever ran
 * before it.  Captured calls share nothing with eager calls or with each
 * other; replaying one graph on two streams at once races on its area.
 * Under capture, HSTU_VALIDATE and the kernel timers are ignored.
 *
 * Errors: argument checks happen on the host before anything is enqueued; a
 * failed check returns a negative status and leaves the stream untouched.  A
 * failed HIP call returns HSTU_ERR_HIP and its hipError_t is kept for
 * hstu_last_hip_error() (per thread).  Malformed device offsets (off[0] != 0 or
 * decreasing) are not detected by the forward call itself: sequences with a
 * negative length are treated as empty, and what is computed for the rest is
 * unspecified; hstu_validate_offsets checks them synchronously.
 */
#ifndef HSTU_H_
#define HSTU_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

typedef enum {
    HSTU_OK = 0,
    HSTU_ERR_INVALID_ARG = -1, /* null pointer, negative count, bad scalar, misaligned */
    HSTU_ERR_UNSUPPORTED = -2, /* d or dtype not supported, or no gfx950 device */
    HSTU_ERR_HIP = -3,         /* a HIP runtime call failed (see hstu_last_hip_error) */
    HSTU_ERR_NO_MEMORY = -4,   /* the scratch area could not be grown */
    HSTU_ERR_BAD_OFFSETS = -5, /* hstu_validate_offsets found malformed offsets */
    HSTU_ERR_SCRATCH_LIMIT = -6 /* hstu_attn_fwd_noalloc: the work list does not fit */
} hstu_status_t;

typedef enum { HSTU_BF16 = 0, HSTU_FP16 = 1, HSTU_FP32 = 2 } hstu_dtype_t;

/* The forward pass with the element type given by `dtype`.  The first eleven
 * parameters are the call's data; see the file comment for their meaning. */
hstu_status_t hstu_attn_fwd(const void* q, const void* k, const void* v,
                            const int32_t* seq_offsets, int32_t num_seqs, int32_t heads,
                            int32_t d, float alpha, float n, void* out, hipStream_t stream,
                            hstu_dtype_t dtype);

/* The same call with the element type fixed by the name. */
hstu_status_t hstu_attn_fwd_bf16(const void* q, const void* k, const void* v,
                                 const int32_t* seq_offsets, int32_t num_seqs, int32_t heads,
                                 int32_t d, float alpha, float n, void* out, hipStream_t stream);
hstu_status_t hstu_attn_fwd_fp16(const void* q, const void* k, const void* v,
                                 const int32_t* seq_offsets, int32_t num_seqs, int32_t heads,
                                 int32_t d, float alpha, float n, void* out, hipStream_t stream);
hstu_status_t hstu_attn_fwd_fp32(const void* q, const void* k, const void* v,
                                 const int32_t* seq_offsets, int32_t num_seqs, int32_t heads,
                                 int32_t d, float alpha, float n, void* out, hipStream_t stream);

/* The forward pass under the target-aware mask of M-FALCON inference (HSTU
 * paper translation "行动胜于言语…", §3.4 and Appendix H: candidates appended
 * after a user history are scored in one pass; each candidate attends to the
 * whole history and to itself, never to the other candidates, Fig. 11).
 *
 *   num_targets : device int32[num_seqs]; the last t_i tokens of sequence i are
 *                 candidates (t_i is clamped to [0, s_i], s_i the length).  With
 *                 h_i = s_i - t_i, local row r keeps key c iff c <= r and
 *                 (c < h_i or c == r).  Rows r < h_i (the history) see the plain
 *                 causal mask; t_i = 0 gives hstu_attn_fwd exactly.
 *
 * All other parameters, layouts, element types and errors are those of
 * hstu_attn_fwd; num_targets is caller-owned, read on the device only, and
 * must be non-null and 4-byte aligned when num_seqs > 0 (else
 * HSTU_ERR_INVALID_ARG). */
hstu_status_t hstu_attn_fwd_targets(const void* q, const void* k, const void* v,
                                    const int32_t* seq_offsets, const int32_t* num_targets,
                                    int32_t num_seqs, int32_t heads, int32_t d, float alpha,
                                    float n, void* out, hipStream_t stream, hstu_dtype_t dtype);

/* The later micro-batches of M-FALCON: candidates scored against a cached
 * history (HSTU paper translation, Appendix H: K and V of the history are
 * cached across micro-batches and requests; a micro-batch computes q, k, v
 * for its candidates only).  For request i with h_i cached history rows and
 * t_i candidates, candidate j (global row cand_offsets[i] + j) gets
 *
 *   out[j] = (1/n) * ( sum_{c < h_i} silu(alpha <q[j], k_cache[hist_offsets[i] + c]>)
 *                                     * v_cache[hist_offsets[i] + c]
 *                      + silu(alpha <q[j], k[j]>) * v[j] )
 *
 * i.e. the target-aware mask over history + candidates, computed for the
 * candidate rows only.
 *
 *   q, k, v, out     : the candidates, (T_cand, heads, d), T_cand = cand_offsets[num_seqs];
 *                      layout, alignment and aliasing as in hstu_attn_fwd.
 *   cand_offsets     : device int32[num_seqs + 1], as seq_offsets of hstu_attn_fwd.
 *   k_cache, v_cache : the cached history K and V, (T_hist, heads, d), same element
 *                      type, 16-byte aligned, T_hist = hist_offsets[num_seqs];
 *                      read only; out must not overlap them.  Both may be NULL
 *                      when there is no history (T_hist = 0): then no cache row
 *                      is read and every history counts as empty, whatever
 *                      hist_offsets holds.
 *   hist_offsets     : device int32[num_seqs + 1], off[0] = 0, non-decreasing (an
 *                      empty history is allowed: candidates then see themselves only).
 *
 * Element types, streams, scratch and errors as in hstu_attn_fwd;
 * hist_offsets must be non-null when num_seqs > 0, and the two cache pointers
 * both null or both non-null (else HSTU_ERR_INVALID_ARG).  Malformed history offsets are not detected
 * (hstu_validate_offsets checks them). */
hstu_status_t hstu_attn_fwd_cached(const void* q, const void* k, const void* v,
                                   const int32_t* cand_offsets, const void* k_cache,
                                   const void* v_cache, const int32_t* hist_offsets,
                                   int32_t num_seqs, int32_t heads, int32_t d, float alpha,
                                   float n, void* out, hipStream_t stream, hstu_dtype_t dtype);

/* The forward on the dense padded layout of the Ascend HSTU blog's PyTorch
 * definition (§1: Q, K, V of shape (b, heads, s, d); §4.1 describes this
 * padded layout before replacing it by the jagged one): q, k, v, out are
 * row-major (batch, heads, seq_len, d), element (b, h, r, e) at
 * ((b * heads + h) * seq_len + r) * d + e, and every one of the seq_len
 * positions of every batch entry is a token (the causal mask runs over all of
 * them; padding, if any, is computed like any other row).  No offsets are
 * passed: the library writes i * seq_len into its scratch area once per
 * (stream, batch, seq_len).  batch * seq_len < 2^31.  Element types, scalars,
 * alignment, aliasing, streams and errors as in hstu_attn_fwd. */
hstu_status_t hstu_attn_fwd_dense(const void* q, const void* k, const void* v, int32_t batch,
                                  int32_t heads, int32_t seq_len, int32_t d, float alpha, float n,
                                  void* out, hipStream_t stream, hstu_dtype_t dtype);

/* The layer around the attention (HSTU paper translation, §3: f1 and f2 are
 * one linear layer each, phi_1 is SiLU, Norm is layer normalisation, layers
 * are joined by residual connections; §3.3: phi_1(f_1(.)) is one fused
 * operator, and so are the layer norm and the output MLP).  bfloat16 /
 * float16 (HSTU_FP32 returns HSTU_ERR_UNSUPPORTED); d_model and heads * d each
 * 128, 256 or 512.  All pointers are device pointers, 16-byte aligned,
 * caller-owned; outputs overlap no input.  fp32 accumulation; outputs rounded
 * to nearest even.
 *
 * hstu_layer_in_proj: per token t (num_tokens = T),
 *   [u | v | q | k] = silu(w1 x_t + b1)
 *   x : (T, d_model);  w1 : (4 heads d, d_model) row-major (one output feature
 *   per row);  b1 : float32 [4 heads d].  Output feature j of part p (p = 0..3
 *   for u, v, q, k) is row p * heads * d + j of w1; each part is written as
 *   (T, heads, d) (feature j = h * d + e), the layout hstu_attn_fwd reads. */
hstu_status_t hstu_layer_in_proj(const void* x, const void* w1, const float* b1,
                                 int64_t num_tokens, int32_t d_model, int32_t heads, int32_t d,
                                 void* u, void* v, void* q, void* k, hipStream_t stream,
                                 hstu_dtype_t dtype);

/* hstu_layer_out_proj: per token t,
 *   y_t = x_t + w2 (LN(a_t) * u_t) + b2,
 *   LN(a) = (a - mean(a)) / sqrt(var(a) + eps) * gamma + beta  over the heads * d
 *   features of the token (biased variance);
 *   attn (a), u : (T, heads, d);  x, y : (T, d_model);  w2 : (d_model, heads d)
 *   row-major;  gamma, beta : float32 [heads d];  b2 : float32 [d_model];
 *   eps >= 0 and finite.  No dropout (inference). */
hstu_status_t hstu_layer_out_proj(const void* attn, const void* u, const void* x,
                                  const float* gamma, const float* beta, float eps,
                                  const void* w2, const float* b2, int64_t num_tokens,
                                  int32_t d_model, int32_t heads, int32_t d, void* y,
                                  hipStream_t stream, hstu_dtype_t dtype);

/* Causal forward with the relative attention bias rab_{p,t} (HSTU paper
 * translation, §3: a bias merging relative position and time is added to the
 * scores before phi_2 = SiLU; Appendix G: the bias is built inside the
 * attention operator from its parameters instead of being read as a
 * tensor).  The page's equation is lost; this call takes the reading
 *
 *   out[r] = (1/n) * sum_{c <= r} silu(alpha <q[r], k[c]> + rab(r, c)) * v[c]
 *   rab(r, c) = pos_bias[r - c] + time_bias[min(floor(log2(ts[r] - ts[c] + 1)), num_time - 1)]
 *
 * per sequence and head, r and c local rows, ts the sequence's timestamps;
 * pos_bias[j] counts as 0 for j >= num_pos, and a negative gap (a key later
 * than its query) takes bucket num_time - 1.  The tables are shared by all
 * heads.
 *
 *   q, k, v, out, seq_offsets : as in hstu_attn_fwd (jagged layout).
 *   timestamps   : device int32[T], T = seq_offsets[num_seqs], one per token, 4-byte
 *                  aligned; within one sequence every gap ts[r] - ts[c] must lie
 *                  in (-2^31 + 1, 2^31 - 1) (for example non-decreasing
 *                  timestamps spanning less than 2^31 - 1).
 *   pos_bias     : device float[num_pos], 1 <= num_pos <= 2^28, 4-byte aligned.
 *   time_bias    : device float[num_time], 1 <= num_time <= 32, 4-byte aligned.
 * All three are caller-owned and read only.  alpha must be non-zero with a
 * finite float reciprocal (the kernels add rab / alpha to the raw score).
 * Null or misaligned pointers (with num_seqs > 0), table sizes out of range or
 * such an alpha give HSTU_ERR_INVALID_ARG before anything is enqueued.  Element types, streams, scratch and errors as
 * in hstu_attn_fwd. */
hstu_status_t hstu_attn_fwd_rab(const void* q, const void* k, const void* v,
                                const int32_t* seq_offsets, const int32_t* timestamps,
                                const float* pos_bias, int32_t num_pos, const float* time_bias,
                                int32_t num_time, int32_t num_seqs, int32_t heads, int32_t d,
                                float alpha, float n, void* out, hipStream_t stream,
                                hstu_dtype_t dtype);

/* hstu_attn_fwd_rab under the target-aware mask of hstu_attn_fwd_targets
 * (HSTU paper translation, §3.4: M-FALCON adjusts the attention mask and
 * rab_{p,t} together so that every candidate of a micro-batch runs the same
 * operations).  The page gives no formula; this call takes the reading that a
 * candidate row sits at the position right after the history, hist = s - t,
 * and keeps its own timestamp:
 *
 *   out[r] = (1/n) * sum over the keys c that row r sees of
 *            silu(alpha <q[r], k[c]> + rab_t(r, c)) * v[c]
 *   rab_t(r, c) = rab(r, c)                                   for r < hist
 *               = pos_bias[hist - c] + time term of (r, c)    for r >= hist, c < hist
 *               = pos_bias[0] + time_bias[0]                  for r >= hist, c = r
 *
 * with rab's time term as in hstu_attn_fwd_rab.  A candidate's output thus
 * equals the last row of hstu_attn_fwd_rab over the history followed by that
 * candidate alone, whatever the other candidates are.
 *
 *   num_targets : as in hstu_attn_fwd_targets (device int32[num_seqs],
 *                 clamped to [0, length]).
 *   the rest    : as in hstu_attn_fwd_rab.
 * Errors as in hstu_attn_fwd_rab; a null or misaligned num_targets (with
 * num_seqs > 0) also gives HSTU_ERR_INVALID_ARG. */
hstu_status_t hstu_attn_fwd_rab_targets(const void* q, const void* k, const void* v,
                                        const int32_t* seq_offsets, const int32_t* num_targets,
                                        const int32_t* timestamps, const float* pos_bias,
                                        int32_t num_pos, const float* time_bias,
                                        int32_t num_time, int32_t num_seqs, int32_t heads,
                                        int32_t d, float alpha, float n, void* out,
                                        hipStream_t stream, hstu_dtype_t dtype);

/* hstu_attn_fwd_cached with the relative attention bias (HSTU paper
 * translation, §3.4: M-FALCON adjusts rab_{p,t} with the mask; Appendix H:
 * the history's K and V come from a cache).  Read as in
 * hstu_attn_fwd_rab_targets, with the history taken from the cache: a
 * candidate sits at the position right after its request's h_i cached rows
 * and keeps its own timestamp.  Candidate j of request i (global row
 * cand_offsets[i] + j, history rows hist_offsets[i] + c) gets
 *
 *   out[j] = (1/n) * ( sum_{c < h_i} silu(alpha <q[j], k_cache[.. + c]> + rab_c(j, c))
 *                                     * v_cache[.. + c]
 *                      + silu(alpha <q[j], k[j]> + pos_bias[0] + time_bias[0]) * v[j] )
 *   rab_c(j, c) = pos_bias[h_i - c] (0 past the table)
 *               + time_bias[min(floor(log2(timestamps[j] - hist_timestamps[.. + c] + 1)),
 *                               num_time - 1)]   (a negative gap: the last entry)
 *
 * so a candidate's output equals the last row of hstu_attn_fwd_rab over its
 * history followed by that candidate alone.
 *
 *   q, k, v, out, cand_offsets, k_cache, v_cache, hist_offsets :
 *                     as in hstu_attn_fwd_cached.
 *   timestamps      : device int32[T_cand], the candidates' timestamps, 4-byte aligned.
 *   hist_timestamps : device int32[T_hist], the cached rows' timestamps (the
 *                     layout of k_cache), 4-byte aligned; ignored (may be
 *                     NULL) when the caches are NULL.
 *   pos_bias, num_pos, time_bias, num_time : as in hstu_attn_fwd_rab.
 *
 * Element types, streams, scratch and errors as in hstu_attn_fwd_cached and
 * hstu_attn_fwd_rab; a null or misaligned hist_timestamps with non-null
 * caches (num_seqs > 0) also gives HSTU_ERR_INVALID_ARG. */
hstu_status_t hstu_attn_fwd_rab_cached(const void* q, const void* k, const void* v,
                                       const int32_t* cand_offsets, const void* k_cache,
                                       const void* v_cache, const int32_t* hist_offsets,
                                       const int32_t* timestamps,
                                       const int32_t* hist_timestamps, const float* pos_bias,
                                       int32_t num_pos, const float* time_bias,
                                       int32_t num_time, int32_t num_seqs, int32_t heads,
                                       int32_t d, float alpha, float n, void* out,
                                       hipStream_t stream, hstu_dtype_t dtype);

/* Backward: gradients of hstu_attn_fwd (or, with num_targets, of
 * hstu_attn_fwd_targets) with respect to q, k and v, for the upstream
 * gradient dout = dLoss/dout.  The attention is recomputed block by block and
 * nothing of size T x T is stored (HSTU paper translation, Appendix G); the
 * gradients are the derivative of the forward definition.  Per sequence,
 * head and kept (row r, key c) pair, with x = alpha <q_r, k_c>:
 *
 *   dv_c += silu(x) / n * dout_r
 *   g     = (alpha / n) * silu'(x) * <dout_r, v_c>,  silu'(x) = sig(x) (1 + x (1 - sig(x)))
 *   dq_r += g * k_c,   dk_c += g * q_r
 *
 *   q, k, v, dout  : (T, heads, d) inputs as for the forward; dout has their type.
 *   dq, dk, dv     : (T, heads, d) outputs of the same type, fully written
 *                    (rounded to nearest even from fp32 accumulation); 16-byte
 *                    aligned, none overlapping another or any input.
 *   num_targets    : as for hstu_attn_fwd_targets (device int32[num_seqs]).
 *
 * Element types: bfloat16 and float16 on the matrix cores with float32
 * accumulation, P = silu(x) and the score gradient rounded to the input type
 * before their products (as the forward rounds its weights); float32 runs
 * every product in float32.
 * A call is two kernels (dk/dv, then dq; plus the work-list kernel on a new
 * scratch area or for more than 256 sequences).  Streams, scratch and errors
 * as for hstu_attn_fwd. */
hstu_status_t hstu_attn_bwd(const void* q, const void* k, const void* v, const void* dout,
                            const int32_t* seq_offsets, int32_t num_seqs, int32_t heads,
                            int32_t d, float alpha, float n, void* dq, void* dk, void* dv,
                            hipStream_t stream, hstu_dtype_t dtype);
hstu_status_t hstu_attn_bwd_targets(const void* q, const void* k, const void* v,
                                    const void* dout, const int32_t* seq_offsets,
                                    const int32_t* num_targets, int32_t num_seqs, int32_t heads,
                                    int32_t d, float alpha, float n, void* dq, void* dk,
                                    void* dv, hipStream_t stream, hstu_dtype_t dtype);

/* Backward of hstu_attn_fwd_rab: dq, dk, dv as in hstu_attn_bwd, for the
 * biased scores x = alpha <q_r, k_c> + rab(r, c), plus the gradients of the
 * two bias tables (HSTU paper translation, Appendix G: the backward recomputes
 * the attention and the relative bias and accumulates the bias gradients on
 * chip).  Per kept pair, with dx = silu'(x) <dout_r, v_c> / n:
 *
 *   dq_r += alpha dx k_c,  dk_c += alpha dx q_r,  dv_c += silu(x) / n dout_r
 *   d_pos_bias[r - c] += dx   (r - c < num_pos)
 *   d_time_bias[min(floor(log2(ts[r] - ts[c] + 1)), num_time - 1)] += dx
 *
 * summed over all sequences and heads.
 *
 *   q, k, v, dout, dq, dk, dv, seq_offsets : as in hstu_attn_bwd.
 *   timestamps, pos_bias, time_bias        : as in hstu_attn_fwd_rab, but
 *                                            1 <= num_pos <= 2^18.
 *   d_pos_bias   : device float[num_pos], overwritten, 4-byte aligned.
 *   d_time_bias  : device float[num_time], overwritten, 4-byte aligned.
 *
 * bfloat16 and float16 on the matrix cores as in hstu_attn_bwd; float32 runs
 * every product in float32 and reads the bias per element from global memory
 * (the reference-precision path, not a fast one).  The table gradients are
 * sums taken with float atomics: not bitwise reproducible across calls (dq,
 * dk, dv are).  The call also uses 64 * (num_pos + 32)
 * floats of library scratch.  A call is four kernels (zeroing the partials,
 * dk/dv, dq with the table sums, the partials' reduction; plus the work-list
 * kernel as in hstu_attn_bwd).  Other conventions and errors as in
 * hstu_attn_fwd_rab and hstu_attn_bwd. */
hstu_status_t hstu_attn_bwd_rab(const void* q, const void* k, const void* v, const void* dout,
                                const int32_t* seq_offsets, const int32_t* timestamps,
                                const float* pos_bias, int32_t num_pos, const float* time_bias,
                                int32_t num_time, int32_t num_seqs, int32_t heads, int32_t d,
                                float alpha, float n, void* dq, void* dk, void* dv,
                                float* d_pos_bias, float* d_time_bias, hipStream_t stream,
                                hstu_dtype_t dtype);

/* Backward of hstu_attn_fwd_rab_targets (HSTU paper translation, §3.4:
 * M-FALCON changes the mask and rab_{p,t} together; Appendix G: the bias
 * gradients are accumulated on chip): hstu_attn_bwd_rab's gradients for the
 * target-aware mask and its bias reading.  A kept pair's score gradient goes
 * to the position entry of the distance its bias used: r - c for a history
 * row, hist - c for a candidate row and a history key, 0 for a candidate and
 * itself (hist = s - t); the time bucket is the pair's real one.  So each
 * candidate's share equals the last row's share of hstu_attn_bwd_rab over the
 * history followed by that candidate alone.
 *
 *   num_targets : as in hstu_attn_fwd_targets (device int32[num_seqs],
 *                 clamped to [0, length]).
 *   the rest    : as in hstu_attn_bwd_rab.
 * Errors as in hstu_attn_bwd_rab; a null or misaligned num_targets (with
 * num_seqs > 0) also gives HSTU_ERR_INVALID_ARG. */
hstu_status_t hstu_attn_bwd_rab_targets(const void* q, const void* k, const void* v,
                                        const void* dout, const int32_t* seq_offsets,
                                        const int32_t* num_targets, const int32_t* timestamps,
                                        const float* pos_bias, int32_t num_pos,
                                        const float* time_bias, int32_t num_time,
                                        int32_t num_seqs, int32_t heads, int32_t d, float alpha,
                                        float n, void* dq, void* dk, void* dv, float* d_pos_bias,
                                        float* d_time_bias, hipStream_t stream,
                                        hstu_dtype_t dtype);

/* The backward on the dense (batch, heads, seq_len, d) layout of
 * hstu_attn_fwd_dense (causal mask over all seq_len positions); q, k, v, dout,
 * dq, dk, dv all have that layout.  Other conventions as in hstu_attn_bwd. */
hstu_status_t hstu_attn_bwd_dense(const void* q, const void* k, const void* v, const void* dout,
                                  int32_t batch, int32_t heads, int32_t seq_len, int32_t d,
                                  float alpha, float n, void* dq, void* dk, void* dv,
                                  hipStream_t stream, hstu_dtype_t dtype);

/* Checks device offsets synchronously: off[0] == 0 and non-decreasing.  Writes
 * T = off[num_seqs] to *total (may be NULL).  Returns HSTU_OK or
 * HSTU_ERR_BAD_OFFSETS; synchronises `stream`. */
hstu_status_t hstu_validate_offsets(const int32_t* seq_offsets, int32_t num_seqs,
                                    int64_t* total, hipStream_t stream);

/* Bytes of the fixed device array behind hstu_attn_fwd_noalloc (one per GPU). */
#define HSTU_NOALLOC_SCRATCH_BYTES (1u << 20)

/* The forward of hstu_attn_fwd (causal mask, jagged layout, same arguments,
 * same result bit for bit), for callers that cannot allocate: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  It
 * calls no allocating routine: its work list lives in a fixed device array of
 * HSTU_NOALLOC_SCRATCH_BYTES per GPU, which the library holds until the
 * process ends, instead of the per-stream scratch area; it is never timed by
 * hstu_profile_* (timing creates events).  A batch whose work list does not
 * fit, about (8 + 4 heads) bytes per sequence plus 5 KB, returns
 * HSTU_ERR_SCRATCH_LIMIT before anything is enqueued.  Every call on one GPU
 * shares that GPU's array and leaves its contents there: calls that overlap
 * on one GPU (on two streams, or a graph replay beside another call) race on
 * it and may give wrong results; calls ordered on one stream are safe, since
 * each call zeroes the array's queue counters itself (with one extra one-wave
 * kernel for batches of up to 256 sequences and 2048 (sequence, head) pairs;
 * larger batches' work-list kernel does it). */
hstu_status_t hstu_attn_fwd_noalloc(const void* q, const void* k, const void* v,
                                    const int32_t* seq_offsets, int32_t num_seqs, int32_t heads,
                                    int32_t d, float alpha, float n, void* out,
                                    hipStream_t stream, hstu_dtype_t dtype);

/* Human-readable name of a status. */
const char* hstu_status_string(hstu_status_t status);

/* The hipError_t (as int) of the last failed HIP call on this thread. */
int hstu_last_hip_error(void);

/* Frees every scratch area the library holds on the current device.  Must not
 * race with calls in flight on that device (synchronise first). */
void hstu_release_workspace(void);

/* ---- kernel timing (for benchmarks) -------------------------------------- */

/* Per-kernel time accumulated over calls made while profiling was on. */
typedef struct {
    int64_t calls;        /* forward calls timed */
    double sched_ms;      /* total time of the work-list kernel (0 for one-kernel calls) */
    double attn_ms;       /* total time of the attention kernel */
    int64_t dropped;      /* calls not timed because the event ring was full */
    double attn_min_ms;   /* shortest attention-kernel time of one call (0 if none) */
    double attn_median_ms;/* median attention-kernel time of one call (0 if none) */
    double clock_mhz;     /* shader clock during the last timed forward call, averaged over
                           * its workgroups (each reads the shader-clock counter and the
                           * 100 MHz counter at its start and end); 0 if none */
} hstu_kernel_times_t;

/* on != 0: from now on each forward call records start and stop events on
 * the dispatch of each of its kernels. */
hstu_status_t hstu_profile_enable(int on);

/* Waits for the recorded events, adds their durations to *out and, if reset,
 * clears the accumulated totals.  Reads the clock record of the last timed
 * forward call back from the device (a synchronous copy). */
hstu_status_t hstu_profile_read(hstu_kernel_times_t* out, int reset);

#ifdef __cplusplus
}
#endif

#endif /* HSTU_H_ */
