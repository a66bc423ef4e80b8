/*
 * gdn_oracle.c -- plain, sequential fp64 CPU oracle for the gated-delta-rule
 * token mixer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call
 * this file; only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header or constant with the HIP
 * library.
 *
 * Every routine is the literal definition of the operation, evaluated one token
 * at a time in IEEE double precision with libm.  There is no chunking, no
 * blocking and no reordering beyond what the definition states, so each line
 * can be checked against the mathematics by eye.
 *
 * Sources (cited by page title and section; the pages carry no equations for
 * the rule itself, the equation below is the one the method is specified by):
 *   - "Agnes-3.0-Flash" model card (ModelScope), Architecture table, row
 *     "Delta-rule layers": 16 key heads / 48 value heads, head dim 128, causal
 *     conv of kernel 4 in front, gated RMS-norm after, recurrent state in fp32.
 *   - "Agnes-3.0-Flash Deep Dive: A 33B Hybrid-Attention Multimodal Model",
 *     section "Attention Layer Details" (the same head geometry, conv, norm
 *     and fp32 state), and its explanatory paragraph on the Gated Delta Rule
 *     (after "Feed-Forward and Positional Encoding"): the delta rule erases
 *     before it writes, and a forget gate decays the state.
 *   - Update rule:  S_t = S_{t-1} * a_t (I - b_t k_t k_t^T) + b_t v_t k_t^T,
 *                   o_t = scale * S_t q_t,  a_t = exp(g_t).
 *     S is dv x dk (row index = value channel), so S k is a dv-vector.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   value head h reads key/query head h / (Hv/Hk) (contiguous groups);
 *   conv: y_t = sum_i w[c][i] x_{t-3+i}, w[c][3] is the current token, history
 *   before a sequence start comes from that sequence's conv state (oldest
 *   first) or zeros; SiLU on every channel; L2 as y / sqrt(sum y^2 + eps) on
 *   each q and k head; gated norm as (o / rms(o)) * w * silu(z).
 *
 * Parity pins: every exported routine here is pinned by the CPU tests against
 * invariants, closed forms, a brute-force unrolled form, an independent chunked
 * (WY) formulation, and library routines (torch conv1d / rms_norm in fp64).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARG (-1)
#define ORACLE_ERR_NOMEM (-2)

int oracle_abi_version(void) { return 1; }

/* ---------------------------------------------------------------------------
 * Round a double to the nearest bfloat16 value, ties to even.
 * bfloat16 has an 8-bit significand (7 stored + hidden), exponent range of
 * binary32 (normal down to 2^-126, subnormal spacing 2^-133), max finite
 * (2 - 2^-7) * 2^127.  Written from that definition with frexp/ldexp/nearbyint
 * (nearbyint rounds half to even in the default rounding mode).
 * ------------------------------------------------------------------------- */
static double round_to_bf16(double x)
{
    if (!isfinite(x) || x == 0.0) return x;
    double ax = fabs(x);
    double r;
    if (ax < ldexp(1.0, -126)) {
        /* subnormal range: fixed spacing 2^-133 */
        r = ldexp(nearbyint(ldexp(ax, 133)), -133);
    } else {
        int e;
        double m = frexp(ax, &e);              /* ax = m * 2^e, m in [0.5, 1) */
        r = ldexp(nearbyint(ldexp(m, 8)), e - 8);
        double maxf = ldexp(2.0 - ldexp(1.0, -7), 127);
        if (r > maxf) r = INFINITY;
    }
    return x < 0 ? -r : r;
}

double oracle_round_bf16(double x) { return round_to_bf16(x); }

void oracle_round_bf16_array(const double* x, double* y, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) y[i] = round_to_bf16(x[i]);
}

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }
static double silu(double x) { return x * sigmoid(x); }

/* Sequence bounds: explicit cu_seqlens, or n_seqs equal pieces of T_total. */
static int seq_bounds(const int32_t* cu, int32_t n_seqs, int32_t T_total, int32_t n,
                      int64_t* start, int64_t* end)
{
    if (cu) {
        *start = cu[n];
        *end = cu[n + 1];
    } else {
        if (n_seqs <= 0 || T_total % n_seqs) return ORACLE_ERR_ARG;
        int64_t len = T_total / n_seqs;
        *start = (int64_t)n * len;
        *end = *start + len;
    }
    if (*start < 0 || *end < *start || *end > T_total) return ORACLE_ERR_ARG;
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------------
 * One token of the rule on one value head, in place on S (dv x dk, row-major):
 *   a = exp(g);  S <- a S;  p = S k;  u = beta (v - p);  S <- S + u k^T;
 *   o = scale * S q.
 * Expanding: S_new = a S (I - beta k k^T) + beta v k^T, i.e. decay first, the
 * erase uses the decayed state, and the output reads the updated state.
 * ------------------------------------------------------------------------- */
static void rule_step(double* S, const double* kk, const double* qq, const double* vv,
                      double g, double beta, double* o_out, int32_t dk, int32_t dv,
                      double scale)
{
    double a = exp(g);
    for (int64_t i = 0; i < (int64_t)dv * dk; ++i) S[i] *= a;
    for (int32_t i = 0; i < dv; ++i) {
        double* row = S + (int64_t)i * dk;
        double p = 0.0;
        for (int32_t j = 0; j < dk; ++j) p += row[j] * kk[j];
        double u = beta * (vv[i] - p);
        for (int32_t j = 0; j < dk; ++j) row[j] += u * kk[j];
    }
    if (o_out) {
        for (int32_t i = 0; i < dv; ++i) {
            const double* row = S + (int64_t)i * dk;
            double acc = 0.0;
            for (int32_t j = 0; j < dk; ++j) acc += row[j] * qq[j];
            o_out[i] = scale * acc;
        }
    }
}

/* ---------------------------------------------------------------------------
 * Sequential recurrence over packed sequences.
 *   q, k : [T_total, Hk, dk]      v : [T_total, Hv, dv]
 *   g, beta : [T_total, Hv]       o : [T_total, Hv, dv]
 *   h0 (nullable -> zeros), hT (nullable) : [n_seqs, Hv, dv, dk]
 *   cu_seqlens : [n_seqs + 1] (nullable -> n_seqs equal lengths)
 * Parallel over independent (sequence, value head) pairs only.
 * ------------------------------------------------------------------------- */
int oracle_gdn_recurrence(const double* q, const double* k, const double* v,
                          const double* g, const double* beta,
                          const double* h0, double* o, double* hT,
                          const int32_t* cu_seqlens, int32_t n_seqs, int32_t T_total,
                          int32_t Hk, int32_t Hv, int32_t dk, int32_t dv,
                          double scale, int32_t n_threads)
{
    if (!q || !k || !v || !g || !beta || !o) return ORACLE_ERR_ARG;
    if (n_seqs < 0 || T_total < 0 || Hk <= 0 || Hv <= 0 || Hv % Hk || dk <= 0 || dv <= 0)
        return ORACLE_ERR_ARG;
    for (int32_t n = 0; n < n_seqs; ++n) {
        int64_t s0, s1;
        if (seq_bounds(cu_seqlens, n_seqs, T_total, n, &s0, &s1)) return ORACLE_ERR_ARG;
    }
    const int32_t group = Hv / Hk;
    const int64_t units = (int64_t)n_seqs * Hv;
    int err = ORACLE_OK;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int64_t unit = 0; unit < units; ++unit) {
        const int32_t n = (int32_t)(unit / Hv);
        const int32_t h = (int32_t)(unit % Hv);
        const int32_t kh = h / group;
        int64_t s0, s1;
        seq_bounds(cu_seqlens, n_seqs, T_total, n, &s0, &s1);
        const int64_t ssz = (int64_t)dv * dk;
        double* S = (double*)malloc(sizeof(double) * ssz);
        if (!S) { err = ORACLE_ERR_NOMEM; continue; }
        if (h0) memcpy(S, h0 + ((int64_t)n * Hv + h) * ssz, sizeof(double) * ssz);
        else memset(S, 0, sizeof(double) * ssz);
        for (int64_t t = s0; t < s1; ++t) {
            rule_step(S, k + (t * Hk + kh) * dk, q + (t * Hk + kh) * dk,
                      v + (t * Hv + h) * dv, g[t * Hv + h], beta[t * Hv + h],
                      o + (t * Hv + h) * dv, dk, dv, scale);
        }
        if (hT) memcpy(hT + ((int64_t)n * Hv + h) * ssz, S, sizeof(double) * ssz);
        free(S);
    }
    return err;
}

/* ---------------------------------------------------------------------------
 * Backward of the recurrence: the derivatives of the loss
 *   L = sum(d_o * o) + sum(dhT * hT)
 * with respect to q, k, v, g, beta and h0, by the chain rule through the
 * operations of rule_step taken in reverse order.  Forward, per token:
 *   a = e^g;  Sh = a S_prev;  p = Sh k;  u = beta (v - p);  S = Sh + u k^T;
 *   o = scale S q.
 * Backward, with D = dL/dS (from dhT, or zero, after the last token):
 *   D  += scale d_o q^T           dq += scale S^T d_o
 *   du  = D k                     dk += D^T u
 *   dv  = beta du                 dbeta = (v - p) . du
 *   dp  = -beta du
 *   dSh = D + dp k^T              dk += Sh^T dp
 *   dg  = a (S_prev : dSh)        D   = a dSh      (dL/dS_prev)
 * and dh0 is the D left after the first token.  dq and dk of a key head sum
 * over the value heads that share it.  Every forward state is kept (one per
 * token), so this is for small sizes.  Layouts as oracle_gdn_recurrence;
 * d_o like o, dhT and dh0 like the states (dhT, dh0 nullable).
 * ------------------------------------------------------------------------- */
int oracle_gdn_backward(const double* q, const double* k, const double* v, const double* g,
                        const double* beta, const double* h0, const double* d_o,
                        const double* dhT, const int32_t* cu_seqlens, int32_t n_seqs,
                        int32_t T_total, int32_t Hk, int32_t Hv, int32_t dk, int32_t dv,
                        double scale, double* dq, double* dkey, double* dval, double* dg,
                        double* dbeta, double* dh0, int32_t n_threads)
{
    if (!q || !k || !v || !g || !beta || !d_o || !dq || !dkey || !dval || !dg || !dbeta)
        return ORACLE_ERR_ARG;
    if (n_seqs < 0 || T_total < 0 || Hk <= 0 || Hv <= 0 || Hv % Hk || dk <= 0 || dv <= 0)
        return ORACLE_ERR_ARG;
    for (int32_t n = 0; n < n_seqs; ++n) {
        int64_t s0, s1;
        if (seq_bounds(cu_seqlens, n_seqs, T_total, n, &s0, &s1)) return ORACLE_ERR_ARG;
    }
    const int32_t group = Hv / Hk;
    const int64_t ssz = (int64_t)dv * dk;
    const int64_t units = (int64_t)n_seqs * Hk;      /* (sequence, key head): owns dq, dk rows */
    int err = ORACLE_OK;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int64_t unit = 0; unit < units; ++unit) {
        const int32_t n = (int32_t)(unit / Hk);
        const int32_t kh = (int32_t)(unit % Hk);
        int64_t s0, s1;
        seq_bounds(cu_seqlens, n_seqs, T_total, n, &s0, &s1);
        const int64_t len = s1 - s0;
        for (int64_t t = s0; t < s1; ++t) {
            memset(dq + (t * Hk + kh) * dk, 0, sizeof(double) * dk);
            memset(dkey + (t * Hk + kh) * dk, 0, sizeof(double) * dk);
        }
        double* Sall = (double*)malloc(sizeof(double) * ssz * (len + 1));
        double* D = (double*)malloc(sizeof(double) * ssz);
        double* dSh = (double*)malloc(sizeof(double) * ssz);
        double* work = (double*)malloc(sizeof(double) * 3 * dv);
        if (!Sall || !D || !dSh || !work) {
            free(Sall); free(D); free(dSh); free(work);
            err = ORACLE_ERR_NOMEM;
            continue;
        }
        double* p = work;
        double* u = work + dv;
        double* du = work + 2 * dv;
        for (int32_t j = 0; j < group; ++j) {
            const int32_t h = kh * group + j;
            /* forward, every state kept: Sall[i] = state before token s0 + i */
            if (h0) memcpy(Sall, h0 + ((int64_t)n * Hv + h) * ssz, sizeof(double) * ssz);
            else memset(Sall, 0, sizeof(double) * ssz);
            for (int64_t i = 0; i < len; ++i) {
                const int64_t t = s0 + i;
                memcpy(Sall + (i + 1) * ssz, Sall + i * ssz, sizeof(double) * ssz);
                rule_step(Sall + (i + 1) * ssz, k + (t * Hk + kh) * dk, q + (t * Hk + kh) * dk,
                          v + (t * Hv + h) * dv, g[t * Hv + h], beta[t * Hv + h], NULL, dk, dv,
                          scale);
            }
            /* backward */
            if (dhT) memcpy(D, dhT + ((int64_t)n * Hv + h) * ssz, sizeof(double) * ssz);
            else memset(D, 0, sizeof(double) * ssz);
            for (int64_t i = len - 1; i >= 0; --i) {
                const int64_t t = s0 + i;
                const double* Sp = Sall + i * ssz;          /* S_prev */
                const double* S = Sall + (i + 1) * ssz;     /* S after the token */
                const double* kk = k + (t * Hk + kh) * dk;
                const double* qq = q + (t * Hk + kh) * dk;
                const double* vv = v + (t * Hv + h) * dv;
                const double* dout = d_o + (t * Hv + h) * dv;
                double* dqt = dq + (t * Hk + kh) * dk;
                double* dkt = dkey + (t * Hk + kh) * dk;
                const double a = exp(g[t * Hv + h]);
                const double b = beta[t * Hv + h];
                /* o = scale S q */
                for (int32_t r = 0; r < dv; ++r)
                    for (int32_t c = 0; c < dk; ++c) D[(int64_t)r * dk + c] += scale * dout[r] * qq[c];
                for (int32_t c = 0; c < dk; ++c) {
                    double acc = 0.0;
                    for (int32_t r = 0; r < dv; ++r) acc += S[(int64_t)r * dk + c] * dout[r];
                    dqt[c] += scale * acc;
                }
                /* p and u of the forward step (Sh = a S_prev) */
                for (int32_t r = 0; r < dv; ++r) {
                    double acc = 0.0;
                    for (int32_t c = 0; c < dk; ++c) acc += a * Sp[(int64_t)r * dk + c] * kk[c];
                    p[r] = acc;
                    u[r] = b * (vv[r] - acc);
                }
                /* S = Sh + u k^T */
                for (int32_t r = 0; r < dv; ++r) {
                    double acc = 0.0;
                    for (int32_t c = 0; c < dk; ++c) acc += D[(int64_t)r * dk + c] * kk[c];
                    du[r] = acc;
                }
                for (int32_t c = 0; c < dk; ++c) {
                    double acc = 0.0;
                    for (int32_t r = 0; r < dv; ++r) acc += D[(int64_t)r * dk + c] * u[r];
                    dkt[c] += acc;
                }
                /* u = beta (v - p) */
                double db = 0.0;
                for (int32_t r = 0; r < dv; ++r) {
                    dval[(t * Hv + h) * dv + r] = b * du[r];
                    db += (vv[r] - p[r]) * du[r];
                }
                dbeta[t * Hv + h] = db;
                /* p = Sh k, with dp = -beta du */
                for (int32_t r = 0; r < dv; ++r) {
                    const double dp = -b * du[r];
                    for (int32_t c = 0; c < dk; ++c)
                        dSh[(int64_t)r * dk + c] = D[(int64_t)r * dk + c] + dp * kk[c];
                }
                for (int32_t c = 0; c < dk; ++c) {
                    double acc = 0.0;
                    for (int32_t r = 0; r < dv; ++r) acc += a * Sp[(int64_t)r * dk + c] * (-b * du[r]);
                    dkt[c] += acc;
                }
                /* Sh = a S_prev, a = e^g */
                double da = 0.0;
                for (int64_t e = 0; e < ssz; ++e) da += Sp[e] * dSh[e];
                dg[t * Hv + h] = a * da;
                for (int64_t e = 0; e < ssz; ++e) D[e] = a * dSh[e];
            }
            if (dh0) memcpy(dh0 + ((int64_t)n * Hv + h) * ssz, D, sizeof(double) * ssz);
        }
        free(Sall); free(D); free(dSh); free(work);
    }
    return err;
}

/* ---------------------------------------------------------------------------
 * Decode: one token per sequence, state updated in place.
 *   q, k : [N, Hk, dk]  v : [N, Hv, dv]  g, beta : [N, Hv]  o : [N, Hv, dv]
 *   state : [n_slots, Hv, dv, dk]; sequence n uses slot state_slot[n]
 *   (state_slot nullable -> slot n).
 * ------------------------------------------------------------------------- */
int oracle_gdn_decode(const double* q, const double* k, const double* v,
                      const double* g, const double* beta, double* state,
                      const int32_t* state_slot, int32_t n_slots, double* o,
                      int32_t N, int32_t Hk, int32_t Hv, int32_t dk, int32_t dv,
                      double scale, int32_t n_threads)
{
    if (!q || !k || !v || !g || !beta || !state || !o) return ORACLE_ERR_ARG;
    if (N < 0 || Hk <= 0 || Hv <= 0 || Hv % Hk || dk <= 0 || dv <= 0) return ORACLE_ERR_ARG;
    for (int32_t n = 0; n < N; ++n) {
        int32_t slot = state_slot ? state_slot[n] : n;
        if (slot < 0 || slot >= n_slots) return ORACLE_ERR_ARG;
    }
    const int32_t group = Hv / Hk;
    const int64_t ssz = (int64_t)dv * dk;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(static)
#endif
    for (int64_t unit = 0; unit < (int64_t)N * Hv; ++unit) {
        const int32_t n = (int32_t)(unit / Hv);
        const int32_t h = (int32_t)(unit % Hv);
        const int32_t kh = h / group;
        const int32_t slot = state_slot ? state_slot[n] : n;
        rule_step(state + ((int64_t)slot * Hv + h) * ssz,
                  k + ((int64_t)n * Hk + kh) * dk, q + ((int64_t)n * Hk + kh) * dk,
                  v + ((int64_t)n * Hv + h) * dv, g[(int64_t)n * Hv + h],
                  beta[(int64_t)n * Hv + h], o + ((int64_t)n * Hv + h) * dv, dk, dv,
                  scale);
    }
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------------
 * Causal depthwise conv (kernel 4) + SiLU + per-head L2 of the q/k channels.
 *   x : [T_total, C]  w : [C, 4] (w[c][3] multiplies the current token)
 *   bias : [C] nullable
 *   conv_state_in : [n_seqs, C, 3] nullable (zeros), oldest first: it holds
 *                   the three inputs that precede the sequence.
 *   y : [T_total, C]
 *   conv_state_out : [n_seqs, C, 3] nullable: the last three inputs of the
 *                   sequence's history (state_in followed by the sequence).
 *   Channels [0, n_l2_heads * head_dim) are L2-normalised per head of
 *   head_dim channels: y <- y / sqrt(sum y^2 + eps).
 *   stage_bf16 != 0 rounds every y to bf16 (the stored dtype); 0 keeps fp64.
 * ------------------------------------------------------------------------- */
int oracle_conv1d(const double* x, const double* w, const double* bias,
                  const double* conv_state_in, double* y, double* conv_state_out,
                  const int32_t* cu_seqlens, int32_t n_seqs, int32_t T_total, int32_t C,
                  int32_t n_l2_heads, int32_t head_dim, double l2_eps, int32_t stage_bf16,
                  int32_t n_threads)
{
    const int K = 4;
    if (!x || !w || !y || n_seqs < 0 || T_total < 0 || C <= 0 || n_l2_heads < 0 ||
        head_dim <= 0 || (int64_t)n_l2_heads * head_dim > C)
        return ORACLE_ERR_ARG;
    for (int32_t n = 0; n < n_seqs; ++n) {
        int64_t s0, s1;
        if (seq_bounds(cu_seqlens, n_seqs, T_total, n, &s0, &s1)) return ORACLE_ERR_ARG;
    }
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int32_t n = 0; n < n_seqs; ++n) {
        int64_t s0, s1;
        seq_bounds(cu_seqlens, n_seqs, T_total, n, &s0, &s1);
        const int64_t len = s1 - s0;
        /* conv + bias + SiLU on every channel */
        for (int64_t t = s0; t < s1; ++t) {
            for (int32_t c = 0; c < C; ++c) {
                double acc = 0.0;
                for (int i = 0; i < K; ++i) {
                    int64_t pos = t - (K - 1) + i;   /* absolute position */
                    double xv;
                    if (pos >= s0) xv = x[pos * C + c];
                    else {
                        int64_t back = s0 - pos;     /* 1..3 steps before the start */
                        xv = conv_state_in
                                 ? conv_state_in[((int64_t)n * C + c) * (K - 1) + (K - 1) - back]
                                 : 0.0;
                    }
                    acc += w[(int64_t)c * K + i] * xv;
                }
                if (bias) acc += bias[c];
                y[t * C + c] = silu(acc);
            }
            /* L2 over each q/k head */
            for (int32_t hh = 0; hh < n_l2_heads; ++hh) {
                double* yh = y + t * C + (int64_t)hh * head_dim;
                double ss = 0.0;
                for (int32_t j = 0; j < head_dim; ++j) ss += yh[j] * yh[j];
                double inv = 1.0 / sqrt(ss + l2_eps);
                for (int32_t j = 0; j < head_dim; ++j) yh[j] *= inv;
            }
            if (stage_bf16)
                for (int32_t c = 0; c < C; ++c) y[t * C + c] = round_to_bf16(y[t * C + c]);
        }
        /* new conv state: last K-1 entries of (state_in ++ x[s0:s1]) */
        if (conv_state_out) {
            for (int32_t c = 0; c < C; ++c) {
                double hist[3];
                for (int i = 0; i < K - 1; ++i) {
                    /* position relative to sequence end: len-3+i */
                    int64_t rel = len - (K - 1) + i;
                    if (rel >= 0) hist[i] = x[(s0 + rel) * C + c];
                    else {
                        int64_t back = -rel; /* 1..3 steps before the start */
                        hist[i] = conv_state_in
                                      ? conv_state_in[((int64_t)n * C + c) * (K - 1) + (K - 1) - back]
                                      : 0.0;
                    }
                }
                for (int i = 0; i < K - 1; ++i)
                    conv_state_out[((int64_t)n * C + c) * (K - 1) + i] = hist[i];
            }
        }
    }
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------------
 * Gated RMSNorm per (row, value head):
 *   r = sqrt(mean_i o_i^2 + eps);  out_i = (o_i / r) * w_i * z_i * sigmoid(z_i)
 *   o, z, out : [rows, Hv, dv]   w : [dv] shared by all heads.
 *   stage_bf16 != 0 rounds out to bf16.
 * ------------------------------------------------------------------------- */
int oracle_gated_rmsnorm(const double* o, const double* z, const double* w, double* out,
                         int64_t rows, int32_t Hv, int32_t dv, double eps, int32_t stage_bf16,
                         int32_t n_threads)
{
    if (!o || !z || !w || !out || rows < 0 || Hv <= 0 || dv <= 0) return ORACLE_ERR_ARG;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(static)
#endif
    for (int64_t r = 0; r < rows * Hv; ++r) {
        const double* oo = o + r * dv;
        const double* zz = z + r * dv;
        double* dst = out + r * dv;
        double ss = 0.0;
        for (int32_t i = 0; i < dv; ++i) ss += oo[i] * oo[i];
        double rms = sqrt(ss / dv + eps);
        for (int32_t i = 0; i < dv; ++i) {
            double val = (oo[i] / rms) * w[i] * silu(zz[i]);
            dst[i] = stage_bf16 ? round_to_bf16(val) : val;
        }
    }
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------------
 * Gate preparation from per-head projections.  The pages name a forget gate
 * (the explanatory paragraph on the Gated Delta Rule in the Deep Dive article)
 * but not its parametrisation; the reading taken here is a learned per-head
 * decay rate A_h = exp(A_log[h]) times a data-dependent step
 * softplus(a + dt_bias[h]):
 *     g[t][h]    = -exp(A_log[h]) * softplus(a[t][h] + dt_bias[h])
 *     beta[t][h] = sigmoid(b[t][h])
 * so the decay exp(g) = (1 + e^{a + dt_bias})^{-A_h} lies in (0, 1].
 *   a, b : [T, Hv] with row strides a_stride, b_stride (elements)
 *   A_log, dt_bias : [Hv];  g, beta : [T, Hv] contiguous.
 * softplus(x) = log(1 + e^x), evaluated as max(x, 0) + log1p(e^{-|x|}).
 * ------------------------------------------------------------------------- */
static double softplus(double x) { return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x))); }

int oracle_gate_prep(const double* a, int64_t a_stride, const double* b, int64_t b_stride,
                     const double* A_log, const double* dt_bias, double* g, double* beta,
                     int64_t T, int32_t Hv)
{
    if (!a || !b || !A_log || !dt_bias || !g || !beta || T < 0 || Hv <= 0 ||
        a_stride < Hv || b_stride < Hv)
        return ORACLE_ERR_ARG;
    for (int64_t t = 0; t < T; ++t)
        for (int32_t h = 0; h < Hv; ++h) {
            g[t * Hv + h] = -exp(A_log[h]) * softplus(a[t * a_stride + h] + dt_bias[h]);
            beta[t * Hv + h] = sigmoid(b[t * b_stride + h]);
        }
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------------
 * Varlen chunk map (integer bookkeeping of the chunked prefill), from its
 * definition:
 *   chunk_off[n] sum over m < n of ceil(len_m / C)
 *   tab[c]       (sequence, first token, token count) of chunk c, chunks of
 *                C tokens restarting at every sequence start
 * Plain loops.  (The order in which a kernel schedules the sequences is a
 * performance choice, not part of the result, and is not defined here.)
 * ------------------------------------------------------------------------- */
int oracle_chunk_map(const int32_t* cu, int32_t n_seqs, int32_t C, int32_t* chunk_off,
                     int32_t* tab)
{
    if (!cu || n_seqs < 0 || C <= 0) return ORACLE_ERR_ARG;
    int32_t c = 0;
    for (int32_t n = 0; n < n_seqs; ++n) {
        chunk_off[n] = c;
        for (int32_t t = cu[n]; t < cu[n + 1]; t += C) {
            tab[3 * c + 0] = n;
            tab[3 * c + 1] = t;
            tab[3 * c + 2] = (cu[n + 1] - t < C) ? cu[n + 1] - t : C;
            ++c;
        }
    }
    chunk_off[n_seqs] = c;
    return ORACLE_OK;
}
