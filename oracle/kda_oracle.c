/*
 * KDA fp64 reference oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may load
 * or call this library.  The product path (the HIP library and its Python
 * binding) never does; it shares no code, header, table or helper with it.
 *
 * What it computes: the Kimi Delta Attention (KDA) token mixer as the plain
 * sequential token-by-token recurrence, in IEEE double precision, one
 * (batch, head) sequence at a time.  Sources, by page and section:
 *
 *  - "3T models are no longer magic" (affta.cn/jrzx/86753.html), section
 *    "Gate 1: KDA makes it computable": the per-token order of work is
 *    control signals -> forget the old state -> corrective write scaled by
 *    the update strength -> read the *new* state -> output gate.  The forget
 *    gate is channel-wise (each state direction decays at its own rate), the
 *    per-step retention has a floor of about 0.67 %, the write uses the delta
 *    rule (read the state with the current key, compare with the new value,
 *    write the correction), and the output gate filters the read-out channel
 *    by channel.
 *  - The algebraic form of that description: with D_t = Diag(alpha_t),
 *        S_t = (I - beta_t k_t k_t^T) D_t S_{t-1} + beta_t k_t v_t^T,
 *        o_t = S_t^T q_t,   y_t = o_t (.) sigmoid(z_t),
 *    where S is a d_k x d_v matrix whose rows are indexed by key channels.
 *
 * Readings taken where the pages are silent (each is listed in the design doc):
 *  - log alpha is clamped to [ln 0.0067, 0] when `clamp` is non-zero
 *    (the retention floor, and retention never above 1);
 *  - the gate is the logistic sigmoid of the given logits, no normalisation
 *    of o before it;
 *  - q and k arrive already normalised/scaled unless `qk_norm` is set; with
 *    it, every token's k is divided by its L2 norm and q by its L2 norm times
 *    sqrt(d_k) (the normalisation and query scale of the inputs the kernel is
 *    specified on, done inside; page "3T models are no longer magic", section
 *    "FlashKDA", puts Q and K normalisation into the preparation step);
 *  - with `logits` set, log_alpha holds forget-gate logits x and
 *    log alpha = logsigmoid(x) = -log(1 + e^-x), the parameterisation of the
 *    inputs the kernel is specified on; the floor clamp follows as usual;
 *  - a NULL initial state means zeros.
 *
 * Inputs are read as the exact bit patterns the GPU receives (fp32 or bf16)
 * and widened exactly to double.  No blocking, chunking or reordering: the
 * loop below is the definition.  Further down: the segment summary (the affine
 * map a run of tokens applies to its incoming state) and the gradients of the
 * forward (the same token steps taken backwards, reverse mode).
 *
 * Layouts (row-major, contiguous):
 *   q, k, log_alpha: [B, T, H, Dk]    v, gate, out: [B, T, H, Dv]
 *   beta: [B, T, H]                   states: [B, H, Dk, Dv]
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_F32 0
#define ORC_BF16 1

/* Retention floor: per-step alpha >= 0.0067, so log alpha >= ln 0.0067. */
static const double ORC_LOG_ALPHA_MIN = -5.005647752585217; /* log(0.0067) */

/* log(sigmoid(x)) without overflow: -log1p(e^-x) for x >= 0, x - log1p(e^x) below. */
static double orc_logsigmoid(double x) {
    return x >= 0.0 ? -log1p(exp(-x)) : x - log1p(exp(x));
}

/* Divide x (n entries) by max(||x||_2, 1e-12) * extra. */
static void orc_unit(double *x, int64_t n, double extra) {
    double ss = 0.0;
    for (int64_t c = 0; c < n; ++c) ss += x[c] * x[c];
    double nrm = sqrt(ss);
    if (nrm < 1e-12) nrm = 1e-12;
    for (int64_t c = 0; c < n; ++c) x[c] /= nrm * extra;
}

/* Widen element i of a float32 or bfloat16 array to double (exact). */
static double orc_load(const void *p, int dtype, int64_t i) {
    if (dtype == ORC_F32) return (double)((const float *)p)[i];
    uint32_t w = ((uint32_t)((const uint16_t *)p)[i]) << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/*
 * Run the recurrence for one (b, h) sequence over tokens [0, T).
 * S is d_k x d_v, updated in place.  Scratch r/u/o have d_v entries.
 */
static void orc_sequence(int64_t b, int64_t h, int64_t T, int64_t H, int64_t Dk,
                         int64_t Dv, int dtype, const void *q, const void *k,
                         const void *v, const void *la, const void *beta,
                         const void *gate, double *S, double *out, int clamp,
                         int qk_norm, int logits,
                         double *kv, double *qv, double *r, double *u, double *o) {
    for (int64_t t = 0; t < T; ++t) {
        const int64_t tok = (b * T + t) * H + h; /* index of (b, t, h) */
        const double bt = orc_load(beta, dtype, tok);
        for (int64_t c = 0; c < Dk; ++c) {
            kv[c] = orc_load(k, dtype, tok * Dk + c);
            qv[c] = orc_load(q, dtype, tok * Dk + c);
        }
        if (qk_norm) { /* unit key; query of norm 1/sqrt(d_k) */
            orc_unit(kv, Dk, 1.0);
            orc_unit(qv, Dk, sqrt((double)Dk));
        }
        /* forget: S <- Diag(alpha_t) S, alpha_t = exp(log alpha_t) per key channel */
        for (int64_t c = 0; c < Dk; ++c) {
            double l = orc_load(la, dtype, tok * Dk + c);
            if (logits) l = orc_logsigmoid(l); /* forget-gate logit -> log alpha */
            if (clamp) {
                if (l < ORC_LOG_ALPHA_MIN) l = ORC_LOG_ALPHA_MIN;
                if (l > 0.0) l = 0.0;
            }
            const double a = exp(l);
            double *row = S + c * Dv;
            for (int64_t j = 0; j < Dv; ++j) row[j] *= a;
        }
        /* delta rule: read the decayed state with the key, r = S^T k */
        for (int64_t j = 0; j < Dv; ++j) r[j] = 0.0;
        for (int64_t c = 0; c < Dk; ++c) {
            const double *row = S + c * Dv;
            for (int64_t j = 0; j < Dv; ++j) r[j] += row[j] * kv[c];
        }
        /* compare with the new value, scale by the update strength */
        for (int64_t j = 0; j < Dv; ++j)
            u[j] = bt * (orc_load(v, dtype, tok * Dv + j) - r[j]);
        /* corrective write: S <- S + k u^T */
        for (int64_t c = 0; c < Dk; ++c) {
            double *row = S + c * Dv;
            for (int64_t j = 0; j < Dv; ++j) row[j] += kv[c] * u[j];
        }
        /* read the new state with the query, o = S^T q */
        for (int64_t j = 0; j < Dv; ++j) o[j] = 0.0;
        for (int64_t c = 0; c < Dk; ++c) {
            const double *row = S + c * Dv;
            for (int64_t j = 0; j < Dv; ++j) o[j] += row[j] * qv[c];
        }
        /* output gate: y = o * sigmoid(z), channel by channel */
        for (int64_t j = 0; j < Dv; ++j) {
            const double z = orc_load(gate, dtype, tok * Dv + j);
            out[tok * Dv + j] = o[j] / (1.0 + exp(-z));
        }
    }
}

/* Number of OpenMP threads a call with nthreads <= 0 would use. */
int kda_oracle_default_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Full forward over [B, T, H].  init_state may be NULL (zeros); final_state
 * may be NULL (not returned) and may alias init_state.  out is [B, T, H, Dv].
 * Returns 0, or -1 on bad sizes / dtype, -2 on allocation failure.
 */
int kda_oracle_fwd_ex(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                      int dtype, const void *q, const void *k, const void *v,
                      const void *log_alpha, const void *beta, const void *gate,
                      const double *init_state, double *out, double *final_state,
                      int clamp, int qk_norm, int logits, int nthreads) {
    if (B < 0 || T < 0 || H < 0 || Dk <= 0 || Dv <= 0) return -1;
    if (dtype != ORC_F32 && dtype != ORC_BF16) return -1;
    const int64_t units = B * H;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t unit = 0; unit < units; ++unit) {
        const int64_t b = unit / H, h = unit % H;
        double *S = (double *)malloc(sizeof(double) * (size_t)(Dk * Dv));
        double *scratch = (double *)malloc(sizeof(double) * (size_t)(2 * Dk + 3 * Dv));
        if (!S || !scratch) {
            free(S);
            free(scratch);
#ifdef _OPENMP
#pragma omp atomic write
#endif
            failed = 1;
            continue;
        }
        const int64_t soff = unit * Dk * Dv;
        if (init_state)
            memcpy(S, init_state + soff, sizeof(double) * (size_t)(Dk * Dv));
        else
            memset(S, 0, sizeof(double) * (size_t)(Dk * Dv));
        double *kv = scratch, *qv = kv + Dk, *r = qv + Dk, *u = r + Dv, *o = u + Dv;
        orc_sequence(b, h, T, H, Dk, Dv, dtype, q, k, v, log_alpha, beta, gate, S,
                     out, clamp, qk_norm, logits, kv, qv, r, u, o);
        if (final_state) memcpy(final_state + soff, S, sizeof(double) * (size_t)(Dk * Dv));
        free(S);
        free(scratch);
    }
    return failed ? -2 : 0;
}

int kda_oracle_fwd(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                   int dtype, const void *q, const void *k, const void *v,
                   const void *log_alpha, const void *beta, const void *gate,
                   const double *init_state, double *out, double *final_state,
                   int clamp, int nthreads) {
    return kda_oracle_fwd_ex(B, T, H, Dk, Dv, dtype, q, k, v, log_alpha, beta, gate,
                             init_state, out, final_state, clamp, 0, 0, nthreads);
}

/*
 * One recurrent decode step for every (b, h): the same per-token update as
 * above with T = 1.  q, k, log_alpha: [B, H, Dk]; v, gate, out: [B, H, Dv];
 * beta: [B, H]; state: [B, H, Dk, Dv], read and written in place.
 */
int kda_oracle_decode(int64_t B, int64_t H, int64_t Dk, int64_t Dv, int dtype,
                      const void *q, const void *k, const void *v,
                      const void *log_alpha, const void *beta, const void *gate,
                      double *state, double *out, int clamp, int qk_norm, int logits,
                      int nthreads) {
    if (!state) return -1;
    return kda_oracle_fwd_ex(B, 1, H, Dk, Dv, dtype, q, k, v, log_alpha, beta, gate,
                             state, out, state, clamp, qk_norm, logits, nthreads);
}

/*
 * Segment summary.  Page "3T models are no longer magic", section "KDA context
 * parallelism", and page "Kimi K3 report walk-through", section "KDA Context
 * Parallelism": a run of tokens is summarised by how it transforms the state it
 * receives and by the state it produces from a zero start.  Because every token
 * maps S to A_t S + beta_t k_t v_t^T with A_t = (I - beta_t k_t k_t^T) Diag(alpha_t),
 * a whole run maps S_0 to M S_0 + b:
 *   M = A_T ... A_1                (d_k x d_k, latest token on the left),
 *   b = the state the run reaches from S_0 = 0 (d_k x d_v).
 * Both are built here token by token in double precision: M by applying each
 * A_t to the identity, b by the plain recurrence (the same steps as the forward
 * above, without the query read and the gate).
 * k, log_alpha: [B, T, H, Dk]; v: [B, T, H, Dv]; beta: [B, T, H];
 * M: [B, H, Dk, Dk]; b: [B, H, Dk, Dv].  Returns 0, -1 on bad sizes, -2 on
 * allocation failure.
 */

/* X <- (I - bt k k^T) Diag(a) X (+ bt k v^T when v is given); X has n columns. */
static void orc_transition(double *X, int64_t Dk, int64_t n, const double *kv,
                           const double *a, double bt, const double *vv, double *r) {
    for (int64_t c = 0; c < Dk; ++c)
        for (int64_t j = 0; j < n; ++j) X[c * n + j] *= a[c];
    for (int64_t j = 0; j < n; ++j) r[j] = 0.0;
    for (int64_t c = 0; c < Dk; ++c)
        for (int64_t j = 0; j < n; ++j) r[j] += X[c * n + j] * kv[c];
    for (int64_t j = 0; j < n; ++j) r[j] = (vv ? bt * vv[j] : 0.0) - bt * r[j];
    for (int64_t c = 0; c < Dk; ++c)
        for (int64_t j = 0; j < n; ++j) X[c * n + j] += kv[c] * r[j];
}

int kda_oracle_summary(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                       int dtype, const void *k, const void *v,
                       const void *log_alpha, const void *beta, double *M,
                       double *bstate, int clamp, int qk_norm, int logits, int nthreads) {
    if (B < 0 || T < 0 || H < 0 || Dk <= 0 || Dv <= 0 || !M || !bstate) return -1;
    if (dtype != ORC_F32 && dtype != ORC_BF16) return -1;
    const int64_t units = B * H;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t unit = 0; unit < units; ++unit) {
        const int64_t b = unit / H, h = unit % H;
        const int64_t nmax = Dk > Dv ? Dk : Dv;
        double *scratch = (double *)malloc(sizeof(double) * (size_t)(2 * Dk + Dv + nmax));
        if (!scratch) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            failed = 1;
            continue;
        }
        double *kk = scratch, *a = kk + Dk, *vv = a + Dk, *r = vv + Dv;
        double *Mu = M + unit * Dk * Dk, *bu = bstate + unit * Dk * Dv;
        for (int64_t i = 0; i < Dk; ++i)
            for (int64_t j = 0; j < Dk; ++j) Mu[i * Dk + j] = (i == j) ? 1.0 : 0.0;
        memset(bu, 0, sizeof(double) * (size_t)(Dk * Dv));
        for (int64_t t = 0; t < T; ++t) {
            const int64_t tok = (b * T + t) * H + h;
            const double bt = orc_load(beta, dtype, tok);
            for (int64_t c = 0; c < Dk; ++c) {
                kk[c] = orc_load(k, dtype, tok * Dk + c);
                const double x = orc_load(log_alpha, dtype, tok * Dk + c);
                const double l = logits ? orc_logsigmoid(x) : x;
                /* retention floor and retention <= 1, as in the forward */
                a[c] = exp(clamp ? fmin(fmax(l, ORC_LOG_ALPHA_MIN), 0.0) : l);
            }
            if (qk_norm) orc_unit(kk, Dk, 1.0);
            for (int64_t j = 0; j < Dv; ++j) vv[j] = orc_load(v, dtype, tok * Dv + j);
            orc_transition(Mu, Dk, Dk, kk, a, bt, NULL, r);
            orc_transition(bu, Dk, Dv, kk, a, bt, vv, r);
        }
        free(scratch);
    }
    return failed ? -2 : 0;
}

/*
 * Gradients of the forward above (reverse mode, the steps of the recurrence taken
 * backwards).  For the scalar loss L = sum(dy * y) + sum(dS_T * S_T), given dy
 * [B, T, H, Dv] and dS_T [B, H, Dk, Dv] (or NULL: zero), returns dL/dq, dL/dk
 * [B, T, H, Dk], dL/dv, dL/dgate [B, T, H, Dv], dL/dbeta [B, T, H], dL/dlog_alpha
 * [B, T, H, Dk] and dL/dS_0 [B, H, Dk, Dv], all in double.  Per token, forward:
 *   S^ = Diag(e^l) S_{t-1};  r = S^T k;  u = beta (v - r);  S_t = S^ + k u^T;
 *   o = S_t^T q;  y = o * sigmoid(z),
 * so, backwards from G = dL/dS_t:
 *   do = dy * sigmoid(z);  dz = dy * o * sigmoid(z) (1 - sigmoid(z));
 *   dq = S_t do;  G += q do^T;
 *   dk = G u;  du = G^T k;  dbeta = du . (v - r);  dv = beta du;  dr = -beta du;
 *   dS^ = G + k dr^T;  dk += S^ dr;
 *   dl_c = sum_j S^[c, j] dS^[c, j];  dS_{t-1} = Diag(e^l) dS^.
 * The clamp of log alpha passes the gradient where it leaves the value unchanged
 * (ln 0.0067 <= x <= 0) and stops it where it clips.  Every state S_t of a sequence
 * is kept (T * Dk * Dv doubles per (b, h)): meant for small cases.
 * Returns 0, -1 on bad sizes, -2 on allocation failure.
 */
/*
 * With qk_norm / logits the forward reads raw q, k and forget logits as the forward
 * oracle does (k / |k|, q / (|q| sqrt(Dk)), log alpha = logsigmoid(x), then the
 * clamp), and the gradients are taken with respect to those raw inputs: per token,
 *   unit vector e = x / n (n = max(|x|, 1e-12)), x^ = x / (n s):
 *     dx = (dx^ - e (e . dx^)) / (n s)    (n > 1e-12; below it x^ = x / (1e-12 s) is
 *     linear and dx = dx^ / (1e-12 s)),  s = sqrt(Dk) for q, 1 for k;
 *   dlogit = dlog_alpha * sigmoid(-x)  (d logsigmoid(x) / dx), zero where the clamp
 *     of logsigmoid(x) is active.
 */
static void orc_unit_back(const double *raw, double *g, int64_t n, double extra) {
    double ss = 0.0, dot = 0.0;
    for (int64_t c = 0; c < n; ++c) ss += raw[c] * raw[c];
    const double nrm = sqrt(ss);
    if (nrm < 1e-12) {
        for (int64_t c = 0; c < n; ++c) g[c] /= 1e-12 * extra;
        return;
    }
    for (int64_t c = 0; c < n; ++c) dot += raw[c] / nrm * g[c];
    for (int64_t c = 0; c < n; ++c) g[c] = (g[c] - raw[c] / nrm * dot) / (nrm * extra);
}

int kda_oracle_bwd_ex(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv, int dtype,
                      const void *q, const void *k, const void *v, const void *log_alpha,
                      const void *beta, const void *gate, const double *init_state,
                      const double *dy, const double *dST, double *dq, double *dk, double *dv,
                      double *dla, double *dbeta, double *dgate, double *dS0, int clamp,
                      int qk_norm, int logits, int nthreads) {
    if (B < 0 || T < 0 || H < 0 || Dk <= 0 || Dv <= 0) return -1;
    if (dtype != ORC_F32 && dtype != ORC_BF16) return -1;
    const int64_t units = B * H, SZ = Dk * Dv;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t unit = 0; unit < units; ++unit) {
        const int64_t b = unit / H, h = unit % H;
        /* states S_0 .. S_T, then per-token scratch */
        double *Sall = (double *)malloc(sizeof(double) * (size_t)((T + 1) * SZ));
        double *G = (double *)malloc(sizeof(double) * (size_t)SZ);
        double *Sh = (double *)malloc(sizeof(double) * (size_t)SZ);
        double *w = (double *)malloc(sizeof(double) * (size_t)(6 * Dk + 6 * Dv));
        if (!Sall || !G || !Sh || !w) {
            free(Sall); free(G); free(Sh); free(w);
#ifdef _OPENMP
#pragma omp atomic write
#endif
            failed = 1;
            continue;
        }
        double *kk = w, *qv = kk + Dk, *a = qv + Dk, *xg = a + Dk;  /* xg: raw log alpha */
        double *r = xg + Dk, *u = r + Dv, *o = u + Dv, *dov = o + Dv, *duv = dov + Dv, *drv = duv + Dv;
        double *kraw = drv + Dv, *qraw = kraw + Dk;  /* raw q and k of the token (qk_norm) */
        if (init_state)
            memcpy(Sall, init_state + unit * SZ, sizeof(double) * (size_t)SZ);
        else
            memset(Sall, 0, sizeof(double) * (size_t)SZ);
        /* forward, keeping every state */
        for (int64_t t = 0; t < T; ++t) {
            const int64_t tok = (b * T + t) * H + h;
            const double bt = orc_load(beta, dtype, tok);
            const double *Sp = Sall + t * SZ;
            double *Sn = Sall + (t + 1) * SZ;
            for (int64_t c = 0; c < Dk; ++c) {
                kk[c] = orc_load(k, dtype, tok * Dk + c);
                const double x = orc_load(log_alpha, dtype, tok * Dk + c);
                const double l = logits ? orc_logsigmoid(x) : x;
                a[c] = exp(clamp ? fmin(fmax(l, ORC_LOG_ALPHA_MIN), 0.0) : l);
            }
            if (qk_norm) { /* the unit key the forward uses */
                orc_unit(kk, Dk, 1.0);
            }
            for (int64_t c = 0; c < Dk; ++c)
                for (int64_t j = 0; j < Dv; ++j) Sn[c * Dv + j] = a[c] * Sp[c * Dv + j];
            for (int64_t j = 0; j < Dv; ++j) {
                double acc = 0.0;
                for (int64_t c = 0; c < Dk; ++c) acc += Sn[c * Dv + j] * kk[c];
                u[j] = bt * orc_load(v, dtype, tok * Dv + j) - bt * acc;
            }
            for (int64_t c = 0; c < Dk; ++c)
                for (int64_t j = 0; j < Dv; ++j) Sn[c * Dv + j] += kk[c] * u[j];
        }
        /* backwards */
        if (dST)
            memcpy(G, dST + unit * SZ, sizeof(double) * (size_t)SZ);
        else
            memset(G, 0, sizeof(double) * (size_t)SZ);
        for (int64_t t = T - 1; t >= 0; --t) {
            const int64_t tok = (b * T + t) * H + h;
            const double bt = orc_load(beta, dtype, tok);
            const double *Sp = Sall + t * SZ, *St = Sall + (t + 1) * SZ;
            for (int64_t c = 0; c < Dk; ++c) {
                kk[c] = kraw[c] = orc_load(k, dtype, tok * Dk + c);
                qv[c] = qraw[c] = orc_load(q, dtype, tok * Dk + c);
                xg[c] = orc_load(log_alpha, dtype, tok * Dk + c);
                const double l = logits ? orc_logsigmoid(xg[c]) : xg[c];
                a[c] = exp(clamp ? fmin(fmax(l, ORC_LOG_ALPHA_MIN), 0.0) : l);
            }
            if (qk_norm) {
                orc_unit(kk, Dk, 1.0);
                orc_unit(qv, Dk, sqrt((double)Dk));
            }
            /* recompute S^ = Diag(a) S_{t-1}, r = S^T k, u = beta (v - r), o = S_t^T q */
            for (int64_t c = 0; c < Dk; ++c)
                for (int64_t j = 0; j < Dv; ++j) Sh[c * Dv + j] = a[c] * Sp[c * Dv + j];
            for (int64_t j = 0; j < Dv; ++j) {
                double rr = 0.0, oo = 0.0;
                for (int64_t c = 0; c < Dk; ++c) {
                    rr += Sh[c * Dv + j] * kk[c];
                    oo += St[c * Dv + j] * qv[c];
                }
                r[j] = rr;
                o[j] = oo;
                u[j] = bt * orc_load(v, dtype, tok * Dv + j) - bt * rr;
            }
            /* output gate and the query read */
            for (int64_t j = 0; j < Dv; ++j) {
                const double z = orc_load(gate, dtype, tok * Dv + j);
                const double sg = 1.0 / (exp(-z) + 1.0);
                const double g_y = dy[tok * Dv + j];
                dov[j] = g_y * sg;
                dgate[tok * Dv + j] = g_y * o[j] * sg * (1.0 - sg);
            }
            for (int64_t c = 0; c < Dk; ++c) {
                double acc = 0.0;
                for (int64_t j = 0; j < Dv; ++j) acc += St[c * Dv + j] * dov[j];
                dq[tok * Dk + c] = acc;
            }
            for (int64_t c = 0; c < Dk; ++c)
                for (int64_t j = 0; j < Dv; ++j) G[c * Dv + j] += qv[c] * dov[j];
            /* the corrective write S_t = S^ + k u^T */
            double dbt = 0.0;
            for (int64_t j = 0; j < Dv; ++j) {
                double acc = 0.0;
                for (int64_t c = 0; c < Dk; ++c) acc += G[c * Dv + j] * kk[c];
                duv[j] = acc;
                dbt += acc * orc_load(v, dtype, tok * Dv + j) - acc * r[j];
                dv[tok * Dv + j] = bt * acc;
                drv[j] = -bt * acc;
            }
            dbeta[tok] = dbt;
            for (int64_t c = 0; c < Dk; ++c) {
                double acc = 0.0;
                for (int64_t j = 0; j < Dv; ++j) acc += G[c * Dv + j] * u[j] + Sh[c * Dv + j] * drv[j];
                dk[tok * Dk + c] = acc;
            }
            /* the key read r = S^T k adds k dr^T to dS^; then the decay */
            for (int64_t c = 0; c < Dk; ++c) {
                double dl = 0.0;
                for (int64_t j = 0; j < Dv; ++j) {
                    const double dsh = G[c * Dv + j] + kk[c] * drv[j];
                    dl += Sh[c * Dv + j] * dsh;
                    G[c * Dv + j] = a[c] * dsh;
                }
                const double l = logits ? orc_logsigmoid(xg[c]) : xg[c];
                const int pass = !clamp || (l >= ORC_LOG_ALPHA_MIN && l <= 0.0);
                /* d logsigmoid(x) / dx = sigmoid(-x) */
                dla[tok * Dk + c] = pass ? (logits ? dl / (1.0 + exp(xg[c])) : dl) : 0.0;
            }
            if (qk_norm) { /* back through the per-token normalisation to the raw q and k */
                orc_unit_back(qraw, dq + tok * Dk, Dk, sqrt((double)Dk));
                orc_unit_back(kraw, dk + tok * Dk, Dk, 1.0);
            }
        }
        memcpy(dS0 + unit * SZ, G, sizeof(double) * (size_t)SZ);
        free(Sall); free(G); free(Sh); free(w);
    }
    return failed ? -2 : 0;
}

int kda_oracle_bwd(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv, int dtype,
                   const void *q, const void *k, const void *v, const void *log_alpha,
                   const void *beta, const void *gate, const double *init_state,
                   const double *dy, const double *dST, double *dq, double *dk, double *dv,
                   double *dla, double *dbeta, double *dgate, double *dS0, int clamp,
                   int nthreads) {
    return kda_oracle_bwd_ex(B, T, H, Dk, Dv, dtype, q, k, v, log_alpha, beta, gate, init_state, dy,
                             dST, dq, dk, dv, dla, dbeta, dgate, dS0, clamp, 0, 0, nthreads);
}
