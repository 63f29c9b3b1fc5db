/*
 * hstu_oracle.c -- plain fp64 CPU oracle for the HSTU jagged causal attention
 * forward.  TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may call it; the library path never does, and
 * this file shares no code, header or constant with it.
 *
 * What it computes (the plain definition, evaluated row by row):
 *
 *   for sequence i with tokens [off[i], off[i+1]), head h, local row r:
 *     out[off[i]+r, h, :] = (1/n) * sum_{c=0..r} silu(alpha * <q_r, k_c>) * v_c
 *
 * Sources, by page and section:
 *   - Ascend HSTU blog ("都是生成式推荐，为什么昇腾这么快？"), §1: the formula
 *     HSTU(Q,K,V) = (mask/n) * silu(QK^T / alpha^-1) V and the five-step
 *     PyTorch definition (matmul, *= alpha, silu, *= mask/n, matmul).
 *   - same page, §3.1-§3.2: the mask is the decoder-only causal mask; the
 *     diagonal block gets a lower-triangular mask, so position c <= r is kept
 *     (diagonal included).
 *   - same page, §4.2: jagged tensors, values (total, heads, d) plus offsets;
 *     each segment is an independent sample, so no cross-sequence terms.
 *   - HSTU paper translation ("行动胜于言语…"), §3: phi_2 is SiLU.
 *
 * Target-aware mask (the M-FALCON mask), for the *_targets entry points:
 *   - HSTU paper translation, §3.4 and Appendix H (Algorithm 1 and Fig. 11):
 *     a sequence is n history tokens followed by b_m candidate tokens; the
 *     causal lower-triangular mask is kept and, in addition, entries (i, j)
 *     with i, j >= n and i != j are masked, so a candidate sees the history
 *     and itself only.  Per sequence the caller gives the candidate count t;
 *     history length = s - t.  The mask stays multiplicative 0/1 after SiLU
 *     (the -inf of the pseudo-code is for softmax models).
 *
 * Cached history (the later micro-batches of M-FALCON), for the *_cached
 * entry points:
 *   - HSTU paper translation, Appendix H (the encoder-level cache and
 *     Algorithm 1's loop over micro-batches): K and V of the n history tokens
 *     are kept from an earlier pass; a micro-batch then computes Q, K, V for
 *     its b_m candidates only and attends, under the mask above, to the cached
 *     history plus itself.  Written out, candidate j of request i gets
 *       (1/n) * ( sum_{c < h_i} silu(alpha <q_j, kc_c>) vc_c
 *                 + silu(alpha <q_j, k_j>) v_j ),
 *     kc, vc the cached history rows of request i, h_i their count.
 *
 * Backward (the *_bwd entry points): the pages say only that the attention is
 * recomputed in the backward pass instead of storing the h x N x N attention
 * tensor (HSTU paper translation, Appendix G).  The gradients here are the
 * derivative of the forward definition above, written out per (row r, key c)
 * pair that the mask keeps, with x = alpha <q_r, k_c> and dO the gradient of
 * the loss with respect to out:
 *   dv_c += silu(x) / n * dO_r
 *   g     = (alpha / n) * silu'(x) * <dO_r, v_c>,  silu'(x) = sig(x) (1 + x (1 - sig(x)))
 *   dq_r += g * k_c,   dk_c += g * q_r
 *
 * Layer surroundings (the *_layer_* entry points): HSTU paper translation,
 * §3 (f1 and f2 are one linear layer each, f_i(X) = W_i X + b_i; phi_1 is
 * SiLU; Norm is layer normalisation; the layers are joined by residual
 * connections; the attention output is used as Norm(A(X)V(X)) * U(X), fed to
 * f2) and §3.3 (phi_1(f_1(.)) is one fused operator, and so are the layer
 * norm, the optional dropout and the output MLP).  Written out per token t:
 *   [u | v | q | k] = silu(W1 x_t + b1)       (W1: 4*heads*d rows of d_model)
 *   y_t = x_t + W2 (LN(a_t) * u_t) + b2        (W2: d_model rows of heads*d)
 *   LN(a) = (a - mean(a)) / sqrt(var(a) + eps) * gamma + beta   (over heads*d,
 *           biased variance)
 * Readings: the split order U, V, Q, K and each part's (heads, d) layout; no
 * dropout (inference); the residual adds x.
 *
 * Relative attention bias (the *_rab entry points): HSTU paper translation,
 * §3 (the spatial aggregation adds rab_{p,t}, a relative attention bias that
 * merges position p and time t, before phi_2 = SiLU; the equation itself is
 * lost from the page) and Appendix G (the bias is built from its parameters
 * inside the attention operator rather than read as a tensor).  Reading: per
 * (row r, key c <= r) of a sequence with token timestamps ts,
 *   rab(r, c) = wpos[r - c] + wtime[min(floor(log2(ts_r - ts_c + 1)), ntime - 1)]
 * with wpos[j] = 0 for j >= npos and a negative gap in the last time bucket,
 * added after alpha: out[r] = (1/n) sum_{c <= r} silu(alpha <q_r, k_c> + rab(r, c)) v_c.
 * Under the target-aware mask (the *_rab_targets entry points; HSTU paper
 * translation §3.4: M-FALCON adjusts the mask and rab_{p,t} so that every
 * candidate of a micro-batch runs the same operations) a candidate row takes
 * the position right after the history: distance hist - c to a history key
 * c, and 0 to itself; the time term keeps the real timestamps.
 * Its gradients (the *_bwd_rab entry points, also under the target-aware
 * mask) differentiate that definition: per kept pair, dx = silu'(x) <dO_r,
 * v_c> / n with x the biased score; dq_r += alpha dx k_c, dk_c += alpha dx
 * q_r, dv_c += silu(x) / n dO_r, and dx is added to the position entry of the
 * distance the pair's bias used (r - c, or a candidate's hist - c and 0; only
 * below npos) and to the pair's time bucket (the tables' gradients, summed
 * over sequences and heads).
 * With the cached history (the *_rab_cached entry points) a candidate takes
 * the same positions as under the target-aware mask, right after its
 * request's h cached keys: distance h - c to cached key c, 0 to itself, and
 * the time terms of the real gaps (candidate timestamp minus the cached
 * key's; zero to itself).
 *
 * Readings taken where the pages are silent (each listed in the design notes):
 *   - alpha multiplies the scores before SiLU; n is a caller-given scalar;
 *   - the mask multiplies after SiLU (0/1), so masked terms are exactly 0;
 *   - inputs are the already-rounded stored values, widened exactly to fp64;
 *     alpha and n are the fp64 images of the float32 values the GPU call gets.
 *
 * Element types of q/k/v: 0 = bfloat16 bits (uint16), 1 = IEEE binary16
 * (uint16 bits), 2 = float32.  Output is always fp64.
 *
 * ORACLE_PLANT (compile-time, default 0) plants one deliberate mistake so the
 * test suite can show that its pins catch it; the built library used for
 * parity is always compiled with ORACLE_PLANT=0.
 */
#include <math.h>
#include <stdlib.h>
#include <stdint.h>
#include <string.h>

#ifndef ORACLE_PLANT
#define ORACLE_PLANT 0
#endif

/* ---- exact widening of the stored element types ------------------------- */

static double widen_bf16(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double widen_fp16(uint16_t h) {
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int mant = h & 0x3ff;
    double mag;
    if (expo == 0) {
        mag = ldexp((double)mant, -24); /* subnormal: mant * 2^-24 */
    } else if (expo == 31) {
        mag = mant ? NAN : INFINITY;
    } else {
        mag = ldexp((double)(mant | 0x400), expo - 25); /* (1.mant) * 2^(e-15) */
    }
    return sign ? -mag : mag;
}

static double load_elem(const void* base, int dtype, int64_t idx) {
    switch (dtype) {
    case 0: return widen_bf16(((const uint16_t*)base)[idx]);
    case 1: return widen_fp16(((const uint16_t*)base)[idx]);
    default: return (double)((const float*)base)[idx];
    }
}

/* ---- the pointwise nonlinearity ------------------------------------------ */

/* silu(x) = x * sigmoid(x), with the sigmoid written in the form that never
 * forms exp of a large positive number. */
static double silu(double x) {
#if ORACLE_PLANT == 2
    x = -x; /* planted: sign error inside the nonlinearity */
#endif
    if (x >= 0.0) return x / (1.0 + exp(-x));
    double e = exp(x);
    return x * e / (1.0 + e);
}

/* ---- one output row -------------------------------------------------------- */

/* Computes the d outputs of (sequence start `s0`, local row r, head h) into
 * acc[0..d).  Widening q, k and v per element keeps memory small; the cost is
 * irrelevant for an oracle. */
/* `hist` is the sequence's history length: keys c >= hist (candidates) count
 * only for c == r.  hist = sequence length gives the plain causal mask. */
static void one_row(const void* q, const void* k, const void* v, int dtype,
                    int64_t s0, int64_t r, int64_t hist, int heads, int d, int h,
                    double alpha, double n, double* qrow, double* acc) {
    const int64_t row_stride = (int64_t)heads * d;
    for (int e = 0; e < d; ++e) {
        qrow[e] = load_elem(q, dtype, (s0 + r) * row_stride + (int64_t)h * d + e);
        acc[e] = 0.0;
    }
    int64_t c_end = r; /* inclusive: the causal mask keeps the diagonal */
#if ORACLE_PLANT == 1
    c_end = r - 1; /* planted: diagonal dropped */
#endif
    int64_t c_begin = 0;
#if ORACLE_PLANT == 5
    c_begin = -s0; /* planted: attends back across the sequence boundary */
#endif
    for (int64_t c = c_begin; c <= c_end; ++c) {
        /* a candidate key is seen by its own row only */
#if ORACLE_PLANT == 7
        (void)hist; /* planted: candidates see each other */
#elif ORACLE_PLANT == 8
        if (c >= hist && r >= hist) continue; /* planted: candidate misses itself */
#else
        if (c >= hist && c != r) continue;
#endif
        int64_t krow = s0 + c;
#if ORACLE_PLANT == 4
        /* planted: transposed score operand, <q_c, k_r> instead of <q_r, k_c> */
        double dot = 0.0;
        for (int e = 0; e < d; ++e)
            dot += load_elem(q, dtype, krow * row_stride + (int64_t)h * d + e) *
                   load_elem(k, dtype, (s0 + r) * row_stride + (int64_t)h * d + e);
#else
        double dot = 0.0;
        for (int e = 0; e < d; ++e)
            dot += qrow[e] * load_elem(k, dtype, krow * row_stride + (int64_t)h * d + e);
#endif
#if ORACLE_PLANT == 3
        double w = alpha * silu(dot); /* planted: alpha applied after SiLU */
#else
        double w = silu(alpha * dot);
#endif
        for (int e = 0; e < d; ++e)
            acc[e] += w * load_elem(v, dtype, krow * row_stride + (int64_t)h * d + e);
    }
    double inv_n = 1.0 / n;
#if ORACLE_PLANT == 6
    inv_n = 1.0; /* planted: normaliser dropped */
#endif
    for (int e = 0; e < d; ++e) acc[e] *= inv_n;
}

/* One candidate row against a cached history: history rows [hs0, hs0 + hlen)
 * of kc/vc, the candidate at global row `row` of q/k/v.  Result in acc[0..d). */
static void cached_row(const void* q, const void* k, const void* v, const void* kc,
                       const void* vc, int dtype, int64_t row, int64_t hs0, int64_t hlen,
                       int heads, int d, int h, double alpha, double n, double* qrow,
                       double* acc) {
    const int64_t row_stride = (int64_t)heads * d;
    const int64_t hoff = (int64_t)h * d;
    for (int e = 0; e < d; ++e) {
        qrow[e] = load_elem(q, dtype, row * row_stride + hoff + e);
        acc[e] = 0.0;
    }
    int64_t c_end = hlen;
#if ORACLE_PLANT == 9
    c_end = hlen - 1; /* planted: last history key missed */
#endif
    for (int64_t c = 0; c < c_end; ++c) {
        double dot = 0.0;
        for (int e = 0; e < d; ++e)
            dot += qrow[e] * load_elem(kc, dtype, (hs0 + c) * row_stride + hoff + e);
        double w = silu(alpha * dot);
        for (int e = 0; e < d; ++e)
            acc[e] += w * load_elem(vc, dtype, (hs0 + c) * row_stride + hoff + e);
    }
    /* the candidate's own key and value */
    double dot = 0.0;
    for (int e = 0; e < d; ++e) dot += qrow[e] * load_elem(k, dtype, row * row_stride + hoff + e);
    double w = silu(alpha * dot);
#if ORACLE_PLANT == 10
    w = 0.0; /* planted: candidate misses itself */
#endif
    for (int e = 0; e < d; ++e) acc[e] += w * load_elem(v, dtype, row * row_stride + hoff + e);
    for (int e = 0; e < d; ++e) acc[e] /= n;
}

/* ---- entry points ---------------------------------------------------------- */

/* Full output: out is fp64 (T, heads, d), T = off[num_seqs].  ntgt is null
 * (plain causal mask) or the candidate count of each sequence (clamped to
 * [0, length]).  Returns 0, or -1 on malformed offsets (off[0] != 0 or
 * decreasing).  d <= 1024. */
int hstu_oracle_fwd_targets(const void* q, const void* k, const void* v, int dtype,
                            const int32_t* off, const int32_t* ntgt, int num_seqs, int heads,
                            int d, double alpha, double n, double* out) {
    if (num_seqs < 0 || heads < 1 || d < 1 || d > 1024) return -1;
    if (num_seqs > 0 && off[0] != 0) return -1;
    for (int i = 0; i < num_seqs; ++i)
        if (off[i + 1] < off[i]) return -1;
    const int64_t row_stride = (int64_t)heads * d;
    const int64_t items = (int64_t)num_seqs * heads;
#pragma omp parallel
    {
        double qrow[1024], acc[1024];
#pragma omp for schedule(dynamic, 1)
        for (int64_t it = 0; it < items; ++it) {
            int i = (int)(it / heads), h = (int)(it % heads);
            int64_t s0 = off[i], len = (int64_t)off[i + 1] - off[i];
            int64_t t = ntgt ? ntgt[i] : 0;
            if (t < 0) t = 0;
            if (t > len) t = len;
            for (int64_t r = 0; r < len; ++r) {
                one_row(q, k, v, dtype, s0, r, len - t, heads, d, h, alpha, n, qrow, acc);
                double* o = out + (s0 + r) * row_stride + (int64_t)h * d;
                for (int e = 0; e < d; ++e) o[e] = acc[e];
            }
        }
    }
    return 0;
}

int hstu_oracle_fwd(const void* q, const void* k, const void* v, int dtype,
                    const int32_t* off, int num_seqs, int heads, int d,
                    double alpha, double n, double* out) {
    return hstu_oracle_fwd_targets(q, k, v, dtype, off, 0, num_seqs, heads, d, alpha, n, out);
}

/* Sampled rows: for m = 0..count-1, out_rows[m, 0..d) is the output at global
 * token tok[m] and head hd[m].  The token's sequence is found by a binary
 * search over the offsets.  ntgt as for hstu_oracle_fwd_targets.  Returns 0,
 * or -1 on a token or head out of range. */
int hstu_oracle_rows_targets(const void* q, const void* k, const void* v, int dtype,
                             const int32_t* off, const int32_t* ntgt, int num_seqs, int heads,
                             int d, double alpha, double n, const int64_t* tok,
                             const int32_t* hd, int64_t count, double* out_rows) {
    if (num_seqs < 1 || heads < 1 || d < 1 || d > 1024) return -1;
    int64_t T = off[num_seqs];
    for (int64_t m = 0; m < count; ++m)
        if (tok[m] < 0 || tok[m] >= T || hd[m] < 0 || hd[m] >= heads) return -1;
#pragma omp parallel
    {
        double qrow[1024];
#pragma omp for schedule(dynamic, 4)
        for (int64_t m = 0; m < count; ++m) {
            /* largest i with off[i] <= tok, among non-empty sequences */
            int lo = 0, hi = num_seqs - 1;
            while (lo < hi) {
                int mid = (lo + hi + 1) / 2;
                if (off[mid] <= tok[m]) lo = mid; else hi = mid - 1;
            }
            int64_t s0 = off[lo], len = (int64_t)off[lo + 1] - off[lo];
            int64_t t = ntgt ? ntgt[lo] : 0;
            if (t < 0) t = 0;
            if (t > len) t = len;
            one_row(q, k, v, dtype, s0, tok[m] - s0, len - t, heads, d, hd[m], alpha, n, qrow,
                    out_rows + m * (int64_t)d);
        }
    }
    return 0;
}

int hstu_oracle_rows(const void* q, const void* k, const void* v, int dtype,
                     const int32_t* off, int num_seqs, int heads, int d,
                     double alpha, double n, const int64_t* tok, const int32_t* hd,
                     int64_t count, double* out_rows) {
    return hstu_oracle_rows_targets(q, k, v, dtype, off, 0, num_seqs, heads, d, alpha, n, tok,
                                    hd, count, out_rows);
}

/* ---- backward ------------------------------------------------------------- */

static double dsilu(double x) {
    double sg = x >= 0.0 ? 1.0 / (1.0 + exp(-x)) : exp(x) / (1.0 + exp(x));
#if ORACLE_PLANT == 11
    return sg; /* planted: the sigmoid taken for the derivative of silu */
#else
    return sg * (1.0 + x * (1.0 - sg));
#endif
}

/* Does row r of a sequence with history length hist see key c? */
static int sees(int64_t r, int64_t c, int64_t hist) {
    return c <= r && (c < hist || c == r);
}

/* The gradient terms of one (row r, key c) pair of sequence start s0, head h:
 * adds to the d-element rows dq_r (if non-null), dk_c and dv_c (if non-null). */
static void pair_grads(const void* q, const void* k, const void* v, const void* dout, int dtype,
                       int64_t s0, int64_t r, int64_t c, int heads, int d, int h, double alpha,
                       double n, double* dq_r, double* dk_c, double* dv_c) {
    const int64_t rs = (int64_t)heads * d, ho = (int64_t)h * d;
    const int64_t qr = (s0 + r) * rs + ho, kc = (s0 + c) * rs + ho;
    double dot = 0.0, dov = 0.0;
    for (int e = 0; e < d; ++e) {
        dot += load_elem(q, dtype, qr + e) * load_elem(k, dtype, kc + e);
        dov += load_elem(dout, dtype, qr + e) * load_elem(v, dtype, kc + e);
    }
    const double x = alpha * dot;
    double chain = alpha;
#if ORACLE_PLANT == 13
    chain = 1.0; /* planted: alpha dropped from the chain rule */
#endif
    const double g = chain / n * dsilu(x) * dov;
    const double w = silu(x) / n;
    for (int e = 0; e < d; ++e) {
        if (dq_r) dq_r[e] += g * load_elem(k, dtype, kc + e);
        if (dk_c) {
#if ORACLE_PLANT == 12
            dk_c[e] += g * load_elem(k, dtype, qr + e); /* planted: k for q */
#else
            dk_c[e] += g * load_elem(q, dtype, qr + e);
#endif
        }
        if (dv_c) dv_c[e] += w * load_elem(dout, dtype, qr + e);
    }
}

/* Gradients of the forward (causal, or target-aware when ntgt is non-null)
 * with respect to q, k and v for upstream gradient dout (same storage type as
 * q); dq, dk, dv are fp64 (T, heads, d) and are overwritten.  Returns 0, or -1
 * on malformed offsets.  Each (sequence, head) pair writes only its own rows. */
int hstu_oracle_bwd(const void* q, const void* k, const void* v, const void* dout, int dtype,
                    const int32_t* off, const int32_t* ntgt, int num_seqs, int heads, int d,
                    double alpha, double n, double* dq, double* dk, double* dv) {
    if (num_seqs < 0 || heads < 1 || d < 1) return -1;
    if (num_seqs > 0 && off[0] != 0) return -1;
    for (int i = 0; i < num_seqs; ++i)
        if (off[i + 1] < off[i]) return -1;
    const int64_t rs = (int64_t)heads * d;
    const int64_t T = num_seqs > 0 ? off[num_seqs] : 0;
    memset(dq, 0, sizeof(double) * T * rs);
    memset(dk, 0, sizeof(double) * T * rs);
    memset(dv, 0, sizeof(double) * T * rs);
    const int64_t items = (int64_t)num_seqs * heads;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t it = 0; it < items; ++it) {
        int i = (int)(it / heads), h = (int)(it % heads);
        int64_t s0 = off[i], len = (int64_t)off[i + 1] - off[i];
        int64_t t = ntgt ? ntgt[i] : 0;
        if (t < 0) t = 0;
        if (t > len) t = len;
        for (int64_t r = 0; r < len; ++r)
            for (int64_t c = 0; c < len; ++c) {
                double* dq_r = dq + (s0 + r) * rs + (int64_t)h * d;
                double* dk_c = dk + (s0 + c) * rs + (int64_t)h * d;
                double* dv_c = dv + (s0 + c) * rs + (int64_t)h * d;
#if ORACLE_PLANT == 14
                if (c > r) { /* planted: the key gradients also take keys above the diagonal */
                    pair_grads(q, k, v, dout, dtype, s0, r, c, heads, d, h, alpha, n, 0, dk_c,
                               dv_c);
                    continue;
                }
#endif
                if (sees(r, c, len - t))
                    pair_grads(q, k, v, dout, dtype, s0, r, c, heads, d, h, alpha, n, dq_r, dk_c,
                               dv_c);
            }
    }
    return 0;
}

/* Sampled gradient rows: kind 0 = dq at query token tok[m], 1 = dk and 2 = dv
 * at key token tok[m], head hd[m]; out_rows[m, 0..d).  Returns 0, or -1 on
 * bad arguments.  d <= 1024. */
int hstu_oracle_bwd_rows(const void* q, const void* k, const void* v, const void* dout,
                         int dtype, const int32_t* off, const int32_t* ntgt, int num_seqs,
                         int heads, int d, double alpha, double n, int kind, const int64_t* tok,
                         const int32_t* hd, int64_t count, double* out_rows) {
    if (num_seqs < 1 || heads < 1 || d < 1 || d > 1024 || kind < 0 || kind > 2) return -1;
    int64_t T = off[num_seqs];
    for (int64_t m = 0; m < count; ++m)
        if (tok[m] < 0 || tok[m] >= T || hd[m] < 0 || hd[m] >= heads) return -1;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t m = 0; m < count; ++m) {
        int lo = 0, hi = num_seqs - 1;   /* largest i with off[i] <= tok */
        while (lo < hi) {
            int mid = (lo + hi + 1) / 2;
            if (off[mid] <= tok[m]) lo = mid; else hi = mid - 1;
        }
        int64_t s0 = off[lo], len = (int64_t)off[lo + 1] - off[lo];
        int64_t t = ntgt ? ntgt[lo] : 0;
        if (t < 0) t = 0;
        if (t > len) t = len;
        const int64_t x = tok[m] - s0;
        double acc[1024], other[1024];
        for (int e = 0; e < d; ++e) acc[e] = other[e] = 0.0;
        if (kind == 0) {
            for (int64_t c = 0; c < len; ++c)
                if (sees(x, c, len - t))
                    pair_grads(q, k, v, dout, dtype, s0, x, c, heads, d, hd[m], alpha, n, acc, 0,
                               0);
        } else {
            for (int64_t r = 0; r < len; ++r)
                if (sees(r, x, len - t))
                    pair_grads(q, k, v, dout, dtype, s0, r, x, heads, d, hd[m], alpha, n, 0,
                               kind == 1 ? acc : other, kind == 2 ? acc : other);
        }
        for (int e = 0; e < d; ++e) out_rows[m * (int64_t)d + e] = acc[e];
    }
    return 0;
}

/* ---- layer surroundings ---------------------------------------------------- */

/* Input projection: x (T, d_model) and w1 (4*heads*d, d_model) in the storage
 * type; b1 fp64 [4*heads*d].  Writes u, v, q, k, each fp64 (T, heads, d).
 * Returns 0, or -1 on bad sizes. */
int hstu_oracle_layer_in(const void* x, const void* w1, const double* b1, int dtype, int64_t T,
                         int dm, int heads, int d, double* u, double* v, double* q, double* k) {
    if (T < 0 || dm < 1 || heads < 1 || d < 1) return -1;
    const int64_t hd = (int64_t)heads * d, n_out = 4 * hd;
    double* part[4] = {u, v, q, k};
#if ORACLE_PLANT == 15
    part[0] = v; /* planted: U and V swapped */
    part[1] = u;
#endif
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t c = 0; c < n_out; ++c) {
            double z = b1[c];
            for (int e = 0; e < dm; ++e)
                z += load_elem(x, dtype, t * dm + e) * load_elem(w1, dtype, c * dm + e);
            part[c / hd][t * hd + c % hd] = silu(z);
        }
    return 0;
}

/* Output projection: attn, u (T, heads, d) and x (T, d_model), w2 (d_model,
 * heads*d) in the storage type; gamma, beta fp64 [heads*d], b2 fp64
 * [d_model].  Writes y fp64 (T, d_model).  Returns 0, or -1 on bad sizes. */
int hstu_oracle_layer_out(const void* attn, const void* u, const void* x, const double* gamma,
                          const double* beta, double eps, const void* w2, const double* b2,
                          int dtype, int64_t T, int dm, int heads, int d, double* y) {
    if (T < 0 || dm < 1 || heads < 1 || d < 1 || heads * d > 4096) return -1;
    const int64_t hd = (int64_t)heads * d;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        double z[4096];
        double mean = 0.0, var = 0.0;
        for (int64_t c = 0; c < hd; ++c) mean += load_elem(attn, dtype, t * hd + c);
        mean /= (double)hd;
        for (int64_t c = 0; c < hd; ++c) {
            const double a = load_elem(attn, dtype, t * hd + c) - mean;
            var += a * a;
        }
#if ORACLE_PLANT == 16
        var /= (double)(hd - 1); /* planted: unbiased variance */
#else
        var /= (double)hd;
#endif
        const double rstd = 1.0 / sqrt(var + eps);
        for (int64_t c = 0; c < hd; ++c) {
            const double ln = (load_elem(attn, dtype, t * hd + c) - mean) * rstd * gamma[c] + beta[c];
            z[c] = ln * load_elem(u, dtype, t * hd + c);
        }
        for (int o = 0; o < dm; ++o) {
            double acc = b2[o];
#if ORACLE_PLANT != 17
            acc += load_elem(x, dtype, t * dm + o); /* (planted 17: residual dropped) */
#endif
            for (int64_t c = 0; c < hd; ++c) acc += z[c] * load_elem(w2, dtype, (int64_t)o * hd + c);
            y[t * dm + o] = acc;
        }
    }
    return 0;
}

static int offsets_ok(const int32_t* off, int num_seqs) {
    if (num_seqs > 0 && off[0] != 0) return 0;
    for (int i = 0; i < num_seqs; ++i)
        if (off[i + 1] < off[i]) return 0;
    return 1;
}

/* Cached-history form: q, k, v, out are the candidates (Tc, heads, d) with
 * offsets coff; kc, vc the cached history (Th, heads, d) with offsets hoff;
 * request i has coff[i+1]-coff[i] candidates and hoff[i+1]-hoff[i] history
 * rows.  out is fp64.  Returns 0, or -1 on malformed offsets.  d <= 1024. */
int hstu_oracle_fwd_cached(const void* q, const void* k, const void* v, const void* kc,
                           const void* vc, int dtype, const int32_t* coff, const int32_t* hoff,
                           int num_seqs, int heads, int d, double alpha, double n, double* out) {
    if (num_seqs < 0 || heads < 1 || d < 1 || d > 1024) return -1;
    if (!offsets_ok(coff, num_seqs) || !offsets_ok(hoff, num_seqs)) return -1;
    const int64_t row_stride = (int64_t)heads * d;
    const int64_t items = (int64_t)num_seqs * heads;
#pragma omp parallel
    {
        double qrow[1024], acc[1024];
#pragma omp for schedule(dynamic, 1)
        for (int64_t it = 0; it < items; ++it) {
            int i = (int)(it / heads), h = (int)(it % heads);
            for (int64_t row = coff[i]; row < coff[i + 1]; ++row) {
                cached_row(q, k, v, kc, vc, dtype, row, hoff[i], (int64_t)hoff[i + 1] - hoff[i],
                           heads, d, h, alpha, n, qrow, acc);
                double* o = out + row * row_stride + (int64_t)h * d;
                for (int e = 0; e < d; ++e) o[e] = acc[e];
            }
        }
    }
    return 0;
}

/* Sampled rows of the cached-history form: out_rows[m, 0..d) is candidate
 * row tok[m] (global index into q), head hd[m].  Returns 0, or -1 on a token
 * or head out of range or malformed offsets. */
int hstu_oracle_rows_cached(const void* q, const void* k, const void* v, const void* kc,
                            const void* vc, int dtype, const int32_t* coff, const int32_t* hoff,
                            int num_seqs, int heads, int d, double alpha, double n,
                            const int64_t* tok, const int32_t* hd, int64_t count,
                            double* out_rows) {
    if (num_seqs < 1 || heads < 1 || d < 1 || d > 1024) return -1;
    if (!offsets_ok(coff, num_seqs) || !offsets_ok(hoff, num_seqs)) return -1;
    int64_t T = coff[num_seqs];
    for (int64_t m = 0; m < count; ++m)
        if (tok[m] < 0 || tok[m] >= T || hd[m] < 0 || hd[m] >= heads) return -1;
#pragma omp parallel
    {
        double qrow[1024];
#pragma omp for schedule(dynamic, 4)
        for (int64_t m = 0; m < count; ++m) {
            int lo = 0, hi = num_seqs - 1;   /* largest i with coff[i] <= tok */
            while (lo < hi) {
                int mid = (lo + hi + 1) / 2;
                if (coff[mid] <= tok[m]) lo = mid; else hi = mid - 1;
            }
            cached_row(q, k, v, kc, vc, dtype, tok[m], hoff[lo],
                       (int64_t)hoff[lo + 1] - hoff[lo], heads, d, hd[m], alpha, n, qrow,
                       out_rows + m * (int64_t)d);
        }
    }
    return 0;
}

/* ---- relative attention bias ----------------------------------------------- */

/* Time bucket of the gap between a query token's timestamp and a key token's:
 * floor(log2(gap + 1)) for gap >= 0, at most ntime - 1; a negative gap (a key
 * later than the query) falls in the last bucket.  Integer arithmetic only. */
static int time_bucket(int64_t gap, int ntime) {
    if (gap < 0) return ntime - 1;
    int b = 0;
#if ORACLE_PLANT == 20
    while (b < 62 && (gap >> (b + 1)) != 0) ++b; /* planted: log2(gap), not log2(gap + 1) */
#else
    while (b < 62 && ((gap + 1) >> (b + 1)) != 0) ++b;
#endif
    return b < ntime - 1 ? b : ntime - 1;
}

/* rab(r, c) for local query row r and key c <= r of one sequence whose token
 * timestamps are ts[0..s): a position term, wpos[r - c] (zero for distances
 * of npos and beyond), plus a time term, wtime[bucket(ts[r] - ts[c])].
 * Under the target-aware mask (history length hist < s), a candidate row
 * r >= hist takes the position it would have right after the history:
 * distance hist - c to a history key, 0 to itself. */
static int64_t rab_dist(int64_t r, int64_t c, int64_t hist) {
    return r >= hist ? (c == r ? 0 : hist - c) : r - c;
}

static double rab_value_hist(int64_t r, int64_t c, int64_t hist, const int32_t* ts,
                             const double* wpos, int npos, const double* wtime, int ntime) {
    int64_t dist = rab_dist(r, c, hist);
#if ORACLE_PLANT == 24
    if (r >= hist) dist = r - c; /* planted: candidates keep their own positions */
#endif
#if ORACLE_PLANT == 19
    dist = dist + 1; /* planted: relative position off by one */
#endif
    double p = dist < npos ? wpos[dist] : 0.0;
    return p + wtime[time_bucket((int64_t)ts[r] - (int64_t)ts[c], ntime)];
}

/* One output row under the causal mask with the relative attention bias added
 * to the scaled score before SiLU:
 *   out[r] = (1/n) sum_{c <= r} silu(alpha <q_r, k_c> + rab(r, c)) v_c
 * ts points at the sequence's first token's timestamp. */
static void rab_row(const void* q, const void* k, const void* v, int dtype, int64_t s0,
                    int64_t r, int64_t hist, const int32_t* ts, const double* wpos, int npos,
                    const double* wtime, int ntime, int heads, int d, int h, double alpha,
                    double n, double* qrow, double* acc) {
    const int64_t row_stride = (int64_t)heads * d;
    for (int e = 0; e < d; ++e) {
        qrow[e] = load_elem(q, dtype, (s0 + r) * row_stride + (int64_t)h * d + e);
        acc[e] = 0.0;
    }
    for (int64_t c = 0; c <= r; ++c) {
        if (c >= hist && c != r) continue; /* a candidate key is seen by its own row only */
        const int64_t krow = s0 + c;
        double dot = 0.0;
        for (int e = 0; e < d; ++e)
            dot += qrow[e] * load_elem(k, dtype, krow * row_stride + (int64_t)h * d + e);
        const double bias = rab_value_hist(r, c, hist, ts, wpos, npos, wtime, ntime);
#if ORACLE_PLANT == 18
        const double w = silu(alpha * (dot + bias)); /* planted: bias scaled by alpha */
#elif ORACLE_PLANT == 21
        const double w = silu(alpha * dot) + bias; /* planted: bias added after SiLU */
#else
        const double w = silu(alpha * dot + bias);
#endif
        for (int e = 0; e < d; ++e)
            acc[e] += w * load_elem(v, dtype, krow * row_stride + (int64_t)h * d + e);
    }
    for (int e = 0; e < d; ++e) acc[e] /= n;
}

/* Causal forward with the relative attention bias.  ts: int32 timestamp of
 * every token (T entries, the jagged layout of q); wpos[npos], wtime[ntime]:
 * the bias tables, shared by all heads (fp64 images of the values the GPU
 * call gets).  out is fp64 (T, heads, d).  Returns 0, or -1 on malformed
 * offsets or sizes (npos >= 1, 1 <= ntime <= 32, d <= 1024). */
int hstu_oracle_fwd_rab_targets(const void* q, const void* k, const void* v, int dtype,
                                const int32_t* off, const int32_t* ntgt, const int32_t* ts,
                                const double* wpos, int npos, const double* wtime, int ntime,
                                int num_seqs, int heads, int d, double alpha, double n,
                                double* out) {
    if (num_seqs < 0 || heads < 1 || d < 1 || d > 1024) return -1;
    if (npos < 1 || ntime < 1 || ntime > 32 || !offsets_ok(off, num_seqs)) return -1;
    const int64_t row_stride = (int64_t)heads * d;
    const int64_t items = (int64_t)num_seqs * heads;
#pragma omp parallel
    {
        double qrow[1024], acc[1024];
#pragma omp for schedule(dynamic, 1)
        for (int64_t it = 0; it < items; ++it) {
            int i = (int)(it / heads), h = (int)(it % heads);
            int64_t s0 = off[i], len = (int64_t)off[i + 1] - off[i];
            int64_t t = ntgt ? ntgt[i] : 0;
            if (t < 0) t = 0;
            if (t > len) t = len;
            const int64_t hist = ntgt ? len - t : INT64_MAX;
            for (int64_t r = 0; r < len; ++r) {
                rab_row(q, k, v, dtype, s0, r, hist, ts + s0, wpos, npos, wtime, ntime, heads, d,
                        h, alpha, n, qrow, acc);
                double* o = out + (s0 + r) * row_stride + (int64_t)h * d;
                for (int e = 0; e < d; ++e) o[e] = acc[e];
            }
        }
    }
    return 0;
}

int hstu_oracle_fwd_rab(const void* q, const void* k, const void* v, int dtype,
                        const int32_t* off, const int32_t* ts, const double* wpos, int npos,
                        const double* wtime, int ntime, int num_seqs, int heads, int d,
                        double alpha, double n, double* out) {
    return hstu_oracle_fwd_rab_targets(q, k, v, dtype, off, 0, ts, wpos, npos, wtime, ntime,
                                       num_seqs, heads, d, alpha, n, out);
}

/* Sampled rows of the same: out_rows[m, 0..d) at global token tok[m], head
 * hd[m].  ntgt as for hstu_oracle_fwd_rab_targets (null: causal).  Returns 0,
 * or -1 on a token or head out of range. */
int hstu_oracle_rows_rab_targets(const void* q, const void* k, const void* v, int dtype,
                                 const int32_t* off, const int32_t* ntgt, const int32_t* ts,
                                 const double* wpos, int npos, const double* wtime, int ntime,
                                 int num_seqs, int heads, int d, double alpha, double n,
                                 const int64_t* tok, const int32_t* hd, int64_t count,
                                 double* out_rows) {
    if (num_seqs < 1 || heads < 1 || d < 1 || d > 1024) return -1;
    if (npos < 1 || ntime < 1 || ntime > 32 || !offsets_ok(off, num_seqs)) return -1;
    int64_t T = off[num_seqs];
    for (int64_t m = 0; m < count; ++m)
        if (tok[m] < 0 || tok[m] >= T || hd[m] < 0 || hd[m] >= heads) return -1;
#pragma omp parallel
    {
        double qrow[1024];
#pragma omp for schedule(dynamic, 4)
        for (int64_t m = 0; m < count; ++m) {
            int lo = 0, hi = num_seqs - 1;   /* largest i with off[i] <= tok */
            while (lo < hi) {
                int mid = (lo + hi + 1) / 2;
                if (off[mid] <= tok[m]) lo = mid; else hi = mid - 1;
            }
            const int64_t s0 = off[lo], len = (int64_t)off[lo + 1] - off[lo];
            int64_t t = ntgt ? ntgt[lo] : 0;
            if (t < 0) t = 0;
            if (t > len) t = len;
            const int64_t hist = ntgt ? len - t : INT64_MAX;
            rab_row(q, k, v, dtype, s0, tok[m] - s0, hist, ts + s0, wpos, npos, wtime, ntime,
                    heads, d, hd[m], alpha, n, qrow, out_rows + m * (int64_t)d);
        }
    }
    return 0;
}

int hstu_oracle_rows_rab(const void* q, const void* k, const void* v, int dtype,
                         const int32_t* off, const int32_t* ts, const double* wpos, int npos,
                         const double* wtime, int ntime, int num_seqs, int heads, int d,
                         double alpha, double n, const int64_t* tok, const int32_t* hd,
                         int64_t count, double* out_rows) {
    return hstu_oracle_rows_rab_targets(q, k, v, dtype, off, 0, ts, wpos, npos, wtime, ntime,
                                        num_seqs, heads, d, alpha, n, tok, hd, count, out_rows);
}

/* One candidate row of the cached-history form (hstu_oracle_fwd_cached) with
 * the relative attention bias: the candidate sits right after its request's
 * history of hlen cached keys, so, as under the target-aware mask, its bias
 * to history key c is wpos[hlen - c] plus the time term of ts_cand - ts_hist[c],
 * and to its own key wpos[0] plus the time term of a zero gap.
 *   out[row] = (1/n) (sum_{c < hlen} silu(alpha <q, kc_c> + rab(c)) vc_c
 *                     + silu(alpha <q, k_row> + rab(self)) v_row)
 * ts_c: the candidate's timestamp; hts: the history's timestamps. */
static void rab_cached_row(const void* q, const void* k, const void* v, const void* kc,
                           const void* vc, int dtype, int64_t row, int64_t hs0, int64_t hlen,
                           int32_t ts_c, const int32_t* hts, const double* wpos, int npos,
                           const double* wtime, int ntime, int heads, int d, int h,
                           double alpha, double n, double* qrow, double* acc) {
    const int64_t row_stride = (int64_t)heads * d;
    const int64_t hoff = (int64_t)h * d;
    for (int e = 0; e < d; ++e) {
        qrow[e] = load_elem(q, dtype, row * row_stride + hoff + e);
        acc[e] = 0.0;
    }
    for (int64_t c = 0; c < hlen; ++c) {
        double dot = 0.0;
        for (int e = 0; e < d; ++e)
            dot += qrow[e] * load_elem(kc, dtype, (hs0 + c) * row_stride + hoff + e);
        int64_t dist = hlen - c;
#if ORACLE_PLANT == 26
        dist = hlen + (row & 3) - c; /* planted: candidates spread over positions */
#endif
        int64_t gap = (int64_t)ts_c - (int64_t)hts[hs0 + c];
#if ORACLE_PLANT == 27
        gap = -gap; /* planted: time gap taken the other way */
#endif
        const double bias = (dist < npos ? wpos[dist] : 0.0) + wtime[time_bucket(gap, ntime)];
        const double w = silu(alpha * dot + bias);
        for (int e = 0; e < d; ++e)
            acc[e] += w * load_elem(vc, dtype, (hs0 + c) * row_stride + hoff + e);
    }
    double dot = 0.0;
    for (int e = 0; e < d; ++e) dot += qrow[e] * load_elem(k, dtype, row * row_stride + hoff + e);
    const double w = silu(alpha * dot + wpos[0] + wtime[time_bucket(0, ntime)]);
    for (int e = 0; e < d; ++e) acc[e] += w * load_elem(v, dtype, row * row_stride + hoff + e);
    for (int e = 0; e < d; ++e) acc[e] /= n;
}

/* The cached-history form with the relative attention bias: as
 * hstu_oracle_fwd_cached, plus ts (int32 per candidate token, the jagged
 * layout of q), hts (int32 per cached history token, the layout of kc) and
 * the bias tables wpos[npos], wtime[ntime].  out is fp64 (T, heads, d).
 * Returns 0, or -1 on malformed offsets or sizes. */
int hstu_oracle_fwd_rab_cached(const void* q, const void* k, const void* v, const void* kc,
                               const void* vc, int dtype, const int32_t* coff,
                               const int32_t* hoff, const int32_t* ts, const int32_t* hts,
                               const double* wpos, int npos, const double* wtime, int ntime,
                               int num_seqs, int heads, int d, double alpha, double n,
                               double* out) {
    if (num_seqs < 0 || heads < 1 || d < 1 || d > 1024) return -1;
    if (npos < 1 || ntime < 1 || ntime > 32) return -1;
    if (!offsets_ok(coff, num_seqs) || !offsets_ok(hoff, num_seqs)) return -1;
    const int64_t row_stride = (int64_t)heads * d;
    const int64_t items = (int64_t)num_seqs * heads;
#pragma omp parallel
    {
        double qrow[1024], acc[1024];
#pragma omp for schedule(dynamic, 1)
        for (int64_t it = 0; it < items; ++it) {
            const int i = (int)(it / heads), h = (int)(it % heads);
            for (int64_t row = coff[i]; row < coff[i + 1]; ++row) {
                rab_cached_row(q, k, v, kc, vc, dtype, row, hoff[i],
                               (int64_t)hoff[i + 1] - hoff[i], ts[row], hts, wpos, npos, wtime,
                               ntime, heads, d, h, alpha, n, qrow, acc);
                double* o = out + row * row_stride + (int64_t)h * d;
                for (int e = 0; e < d; ++e) o[e] = acc[e];
            }
        }
    }
    return 0;
}

/* Sampled rows of the same: out_rows[m, 0..d) is candidate row tok[m], head
 * hd[m].  Returns 0, or -1 on bad arguments. */
int hstu_oracle_rows_rab_cached(const void* q, const void* k, const void* v, const void* kc,
                                const void* vc, int dtype, const int32_t* coff,
                                const int32_t* hoff, const int32_t* ts, const int32_t* hts,
                                const double* wpos, int npos, const double* wtime, int ntime,
                                int num_seqs, int heads, int d, double alpha, double n,
                                const int64_t* tok, const int32_t* hd, int64_t count,
                                double* out_rows) {
    if (num_seqs < 1 || heads < 1 || d < 1 || d > 1024) return -1;
    if (npos < 1 || ntime < 1 || ntime > 32) return -1;
    if (!offsets_ok(coff, num_seqs) || !offsets_ok(hoff, num_seqs)) return -1;
    const int64_t T = coff[num_seqs];
    for (int64_t m = 0; m < count; ++m)
        if (tok[m] < 0 || tok[m] >= T || hd[m] < 0 || hd[m] >= heads) return -1;
#pragma omp parallel
    {
        double qrow[1024];
#pragma omp for schedule(dynamic, 4)
        for (int64_t m = 0; m < count; ++m) {
            int lo = 0, hi = num_seqs - 1;   /* largest i with coff[i] <= tok */
            while (lo < hi) {
                int mid = (lo + hi + 1) / 2;
                if (coff[mid] <= tok[m]) lo = mid; else hi = mid - 1;
            }
            rab_cached_row(q, k, v, kc, vc, dtype, tok[m], hoff[lo],
                           (int64_t)hoff[lo + 1] - hoff[lo], ts[tok[m]], hts, wpos, npos, wtime,
                           ntime, heads, d, hd[m], alpha, n, qrow, out_rows + m * (int64_t)d);
        }
    }
    return 0;
}

/* Gradient terms of one kept pair (r, c) of a sequence with the relative
 * attention bias: x = alpha <q_r, k_c> + rab(r, c) (with the candidate
 * positions of history length hist; INT64_MAX: causal); returns dx = dLoss/dx
 * and adds to dq_r, dk_c, dv_c (each d elements, any may be null). */
static double rab_pair_grads(const void* q, const void* k, const void* v, const void* dout,
                             int dtype, int64_t s0, int64_t r, int64_t c, int64_t hist,
                             const int32_t* ts,
                             const double* wpos, int npos, const double* wtime, int ntime,
                             int heads, int d, int h, double alpha, double n, double* dq_r,
                             double* dk_c, double* dv_c) {
    const int64_t rs = (int64_t)heads * d, ho = (int64_t)h * d;
    const int64_t qr = (s0 + r) * rs + ho, kc = (s0 + c) * rs + ho;
    double dot = 0.0, dov = 0.0;
    for (int e = 0; e < d; ++e) {
        dot += load_elem(q, dtype, qr + e) * load_elem(k, dtype, kc + e);
        dov += load_elem(dout, dtype, qr + e) * load_elem(v, dtype, kc + e);
    }
    const double x = alpha * dot + rab_value_hist(r, c, hist, ts, wpos, npos, wtime, ntime);
    const double dx = dsilu(x) * dov / n;
    const double w = silu(x) / n;
    for (int e = 0; e < d; ++e) {
        if (dq_r) dq_r[e] += alpha * dx * load_elem(k, dtype, kc + e);
        if (dk_c) dk_c[e] += alpha * dx * load_elem(q, dtype, qr + e);
        if (dv_c) dv_c[e] += w * load_elem(dout, dtype, qr + e);
    }
#if ORACLE_PLANT == 22
    return alpha * dx; /* planted: the bias gradient scaled by alpha */
#else
    return dx;
#endif
}

/* Gradients of hstu_oracle_fwd_rab_targets (ntgt null: of hstu_oracle_fwd_rab)
 * for upstream gradient dout: dq, dk, dv fp64 (T, heads, d), and the tables'
 * gradients dwpos[npos], dwtime[ntime] (summed over sequences and heads), all
 * overwritten.  Each kept pair's dx goes to the position entry of the
 * distance its bias used (a candidate's distance hist - c to a history key, 0
 * to itself) and to its time bucket.  The table sums are taken per
 * (sequence, head) pair and then added in pair order, so the result does not
 * depend on the thread count.  Returns 0, or -1 on bad arguments. */
int hstu_oracle_bwd_rab_targets(const void* q, const void* k, const void* v, const void* dout,
                                int dtype, const int32_t* off, const int32_t* ntgt,
                                const int32_t* ts, const double* wpos, int npos,
                                const double* wtime, int ntime, int num_seqs, int heads, int d,
                                double alpha, double n, double* dq, double* dk, double* dv,
                                double* dwpos, double* dwtime) {
    if (num_seqs < 0 || heads < 1 || d < 1) return -1;
    if (npos < 1 || ntime < 1 || ntime > 32 || !offsets_ok(off, num_seqs)) return -1;
    const int64_t rs = (int64_t)heads * d;
    const int64_t T = num_seqs > 0 ? off[num_seqs] : 0;
    const int64_t items = (int64_t)num_seqs * heads;
    const int64_t nt = (int64_t)npos + ntime;
    double* part = (double*)calloc((size_t)(items > 0 ? items : 1) * (size_t)nt, sizeof(double));
    if (!part) return -1;
    memset(dq, 0, sizeof(double) * T * rs);
    memset(dk, 0, sizeof(double) * T * rs);
    memset(dv, 0, sizeof(double) * T * rs);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t it = 0; it < items; ++it) {
        const int i = (int)(it / heads), h = (int)(it % heads);
        const int64_t s0 = off[i], len = (int64_t)off[i + 1] - off[i];
        int64_t t = ntgt ? ntgt[i] : 0;
        if (t < 0) t = 0;
        if (t > len) t = len;
        const int64_t hist = ntgt ? len - t : INT64_MAX;
        double* pp = part + it * nt;
        for (int64_t r = 0; r < len; ++r)
            for (int64_t c = 0; c <= r; ++c) {
                if (!sees(r, c, hist)) continue;
                const double dx = rab_pair_grads(
                        q, k, v, dout, dtype, s0, r, c, hist, ts + s0, wpos, npos, wtime, ntime,
                        heads, d, h, alpha, n, dq + (s0 + r) * rs + (int64_t)h * d,
                        dk + (s0 + c) * rs + (int64_t)h * d, dv + (s0 + c) * rs + (int64_t)h * d);
                int64_t dist = rab_dist(r, c, hist);
#if ORACLE_PLANT == 23
                dist = dist + 1; /* planted: position gradient one distance off */
#endif
#if ORACLE_PLANT == 25
                dist = r - c; /* planted: candidates' position gradient at their own distance */
#endif
                if (dist < npos) pp[dist] += dx;
                pp[npos + time_bucket((int64_t)ts[s0 + r] - (int64_t)ts[s0 + c], ntime)] += dx;
            }
    }
    for (int64_t j = 0; j < nt; ++j) {
        double acc = 0.0;
        for (int64_t it = 0; it < items; ++it) acc += part[it * nt + j];
        if (j < npos) dwpos[j] = acc; else dwtime[j - npos] = acc;
    }
    free(part);
    return 0;
}

int hstu_oracle_bwd_rab(const void* q, const void* k, const void* v, const void* dout, int dtype,
                        const int32_t* off, const int32_t* ts, const double* wpos, int npos,
                        const double* wtime, int ntime, int num_seqs, int heads, int d,
                        double alpha, double n, double* dq, double* dk, double* dv,
                        double* dwpos, double* dwtime) {
    return hstu_oracle_bwd_rab_targets(q, k, v, dout, dtype, off, 0, ts, wpos, npos, wtime,
                                       ntime, num_seqs, heads, d, alpha, n, dq, dk, dv, dwpos,
                                       dwtime);
}

/* Sampled gradient rows of the same: kind 0 = dq at query token tok[m], 1 =
 * dk and 2 = dv at key token tok[m], head hd[m]; out_rows[m, 0..d).  ntgt as
 * for hstu_oracle_bwd_rab_targets.  Returns 0, or -1 on bad arguments. */
int hstu_oracle_bwd_rab_rows_targets(const void* q, const void* k, const void* v,
                                     const void* dout, int dtype, const int32_t* off,
                                     const int32_t* ntgt, const int32_t* ts, const double* wpos,
                                     int npos, const double* wtime, int ntime, int num_seqs,
                                     int heads, int d, double alpha, double n, int kind,
                                     const int64_t* tok, const int32_t* hd, int64_t count,
                                     double* out_rows) {
    if (num_seqs < 1 || heads < 1 || d < 1 || kind < 0 || kind > 2) return -1;
    if (npos < 1 || ntime < 1 || ntime > 32 || !offsets_ok(off, num_seqs)) return -1;
    const int64_t T = off[num_seqs];
    for (int64_t m = 0; m < count; ++m)
        if (tok[m] < 0 || tok[m] >= T || hd[m] < 0 || hd[m] >= heads) return -1;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t m = 0; m < count; ++m) {
        int lo = 0, hi = num_seqs - 1;   /* largest i with off[i] <= tok */
        while (lo < hi) {
            int mid = (lo + hi + 1) / 2;
            if (off[mid] <= tok[m]) lo = mid; else hi = mid - 1;
        }
        const int64_t s0 = off[lo], len = (int64_t)off[lo + 1] - off[lo], x = tok[m] - s0;
        int64_t t = ntgt ? ntgt[lo] : 0;
        if (t < 0) t = 0;
        if (t > len) t = len;
        const int64_t hist = ntgt ? len - t : INT64_MAX;
        double* o = out_rows + m * (int64_t)d;
        for (int e = 0; e < d; ++e) o[e] = 0.0;
        if (kind == 0) {
            for (int64_t c = 0; c <= x; ++c)
                if (sees(x, c, hist))
                    rab_pair_grads(q, k, v, dout, dtype, s0, x, c, hist, ts + s0, wpos, npos,
                                   wtime, ntime, heads, d, hd[m], alpha, n, o, 0, 0);
        } else {
            for (int64_t r = x; r < len; ++r)
                if (sees(r, x, hist))
                    rab_pair_grads(q, k, v, dout, dtype, s0, r, x, hist, ts + s0, wpos, npos,
                                   wtime, ntime, heads, d, hd[m], alpha, n, 0,
                                   kind == 1 ? o : 0, kind == 2 ? o : 0);
        }
    }
    return 0;
}

int hstu_oracle_bwd_rab_rows(const void* q, const void* k, const void* v, const void* dout,
                             int dtype, const int32_t* off, const int32_t* ts, const double* wpos,
                             int npos, const double* wtime, int ntime, int num_seqs, int heads,
                             int d, double alpha, double n, int kind, const int64_t* tok,
                             const int32_t* hd, int64_t count, double* out_rows) {
    return hstu_oracle_bwd_rab_rows_targets(q, k, v, dout, dtype, off, 0, ts, wpos, npos, wtime,
                                            ntime, num_seqs, heads, d, alpha, n, kind, tok, hd,
                                            count, out_rows);
}

/* Number of threads an OpenMP parallel region here uses (for reporting). */
int hstu_oracle_threads(void) {
    int t = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            t = omp_get_num_threads();
#endif
        }
    }
    return t;
}
