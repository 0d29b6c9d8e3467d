/*
 * gla_oracle.c -- plain, slow CPU oracle for the causal gated-linear-attention
 * forward pass, in double precision.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or load
 * this file or the library built from it: only the tests, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * helper with the HIP implementation.
 *
 * What it computes, per (batch b, head h), token by token, with no chunking:
 *
 *   S_{-1} = S0 (or zero)                            d_k x d_v state
 *   for t = 0 .. L-1:
 *       q~ = phi(q_t),  k~ = phi(k_t)                 phi = identity or elu(x)+1
 *       a  = exp(g_t)                                 per key dim / scalar / 1
 *       S_t[i][j] = a_i * S_{t-1}[i][j] + k~_i * v_t[j]
 *       o_t[j]    = sum_i q~_i * S_t[i][j]
 *
 * Sources (the pages, by title and section):
 *  - "Attention is recurrent", section "Linear attention": with the softmax
 *    removed the history collapses into one fixed-size state; the output of token
 *    n is a function of the previous state and token n's q, k, v, and the state is
 *    carried from step to step.  Section "Gated linear attention": the state
 *    forgets through a gate alpha_n applied before the new write.
 *  - "Gated Linear Attention", section "GLA / Recurrent Form": the gate
 *    G_t = alpha_t 1^T, i.e. the update Diag(alpha_t) S_{t-1} + (outer product of
 *    key and value), and the Mamba2 special case G_t = gamma_t 1 1^T with a scalar
 *    gamma_t in (0,1) (also in "Motivation").
 *  - "Transformers are RNNs" notes, feature-map paragraph: similarity written as
 *    phi(Q_i)^T phi(K_j); the elu(x)+1 choice of phi.
 *
 * Readings taken where the pages are silent or garbled:
 *  - orientation: S is d_k x d_v, the write is k v^T, the gate scales key rows and
 *    the read-out is o_t = S_t^T q_t (the first page's row-vector k^T v form);
 *  - the read-out is inclusive: o_t uses S_t, which already holds token t's write;
 *  - alpha_0 also decays the initial state S0;
 *  - no normaliser and no 1/sqrt(d) scaling inside the operation;
 *  - gates are passed as natural-log values g = log(alpha) <= 0.
 *
 * Layouts: contiguous [B][H][L][d] for q, k, v, o; g is [B][H][L][d_k] (key-dim
 * mode) or [B][H][L] (scalar mode) or unused; s0 / s_out are [B][H][d_k][d_v].
 *
 * Normalised form (gla_oracle_forward_norm): the "Transformers are RNNs" notes
 * divide the kernel-weighted sum of values by the sum of the same weights, both
 * written with the feature map, numerator over denominator.  Carried as a second,
 * vector-valued state:
 *
 *       z_t = a (*) z_{t-1} + k~                          d_k vector, z_{-1} = z0 (or 0)
 *       o_t[j] = (sum_i q~_i S_t[i][j]) / (sum_i q~_i z_t[i])
 *
 * Reading taken: with a gate, z decays with the same gate as S (it is the state of
 * a value that is 1 in every token); the notes have no gate.  No epsilon is added
 * to the denominator.  z0 / z_out are [B][H][d_k].
 *
 * Delta rule (gla_oracle_delta): "Attention is recurrent", section "Delta attention".
 * Before writing, the state is asked what it already predicts for the key, and only
 * the error is written, scaled by the write strength beta_n:
 *
 *       u_t = beta_t (v_t - S_{t-1}^T k_t)                d_v
 *       S_t = S_{t-1} + k_t u_t^T,     o_t = S_t^T q_t
 *
 * Readings taken: the read-out is inclusive as above; beta is one scalar per token
 * and head, passed as is; no gate, no feature map and no key normalisation inside
 * (callers scale keys); S_{-1} = s0 or zero (the page assumes zero).  beta is
 * [B][H][L].
 *
 * Outer-product gate (gla_oracle_forward_outer): "Gated Linear Attention", section
 * "GLA / Recurrent Form", names the low-rank parameterisation G_t = alpha_t beta_t^T
 * of the general gate G_t (.) S_{t-1}: the state decays along both dimensions,
 *
 *       S_t[i][j] = alpha_t[i] * beta_t[j] * S_{t-1}[i][j] + k~_i * v_t[j]
 *
 * with alpha_t = exp(g_t) per key dimension and beta_t = exp(gv_t) per value
 * dimension (natural-log gates, gv [B][H][L][d_v]).  Read-out as above.
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_GATE_NONE = 0, ORACLE_GATE_KEYDIM = 1, ORACLE_GATE_SCALAR = 2, ORACLE_GATE_OUTER = 3 };
enum { ORACLE_PHI_IDENTITY = 0, ORACLE_PHI_ELU1 = 1 };

/* elu(x) + 1 with elu's alpha = 1: x + 1 for x > 0, exp(x) otherwise. */
static double feature(double x, int phi)
{
    if (phi == ORACLE_PHI_IDENTITY) return x;
    return x > 0.0 ? x + 1.0 : exp(x);
}

typedef struct {
    const double *q, *k, *v, *g, *gv, *s0, *z0, *beta;
    double *o, *s_out, *z_out;
    int norm, delta;
    long B, H, L, dk, dv;
    int gate_mode, phi;
    long next_head;          /* shared work counter, guarded by lock */
    pthread_mutex_t lock;
} job_t;

static void run_head(const job_t *jb, long head, double *S, double *qf, double *kf, double *a,
                     double *z, double *bv)
{
    const long L = jb->L, dk = jb->dk, dv = jb->dv;
    const double *q = jb->q + head * L * dk;
    const double *k = jb->k + head * L * dk;
    const double *v = jb->v + head * L * dv;
    double *o = jb->o + head * L * dv;

    if (jb->s0) memcpy(S, jb->s0 + head * dk * dv, sizeof(double) * dk * dv);
    else memset(S, 0, sizeof(double) * dk * dv);
    if (jb->z0) memcpy(z, jb->z0 + head * dk, sizeof(double) * dk);
    else memset(z, 0, sizeof(double) * dk);

    for (long t = 0; jb->delta && t < L; ++t) {
        /* delta rule: write the prediction error of the key, scaled by beta */
        const double bt = jb->beta[head * L + t];
        for (long j = 0; j < dv; ++j) {
            double pred = 0.0;
            for (long i = 0; i < dk; ++i) pred += k[t * dk + i] * S[i * dv + j];
            z[j] = bt * (v[t * dv + j] - pred);     /* z holds u_t here (d_v <= its size) */
        }
        for (long i = 0; i < dk; ++i)
            for (long j = 0; j < dv; ++j) S[i * dv + j] += k[t * dk + i] * z[j];
        for (long j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (long i = 0; i < dk; ++i) acc += q[t * dk + i] * S[i * dv + j];
            o[t * dv + j] = acc;
        }
    }
    for (long t = 0; !jb->delta && t < L; ++t) {
        for (long i = 0; i < dk; ++i) {
            qf[i] = feature(q[t * dk + i], jb->phi);
            kf[i] = feature(k[t * dk + i], jb->phi);
        }
        for (long i = 0; i < dk; ++i) {
            if (jb->gate_mode == ORACLE_GATE_KEYDIM || jb->gate_mode == ORACLE_GATE_OUTER)
                a[i] = exp(jb->g[(head * L + t) * dk + i]);
            else if (jb->gate_mode == ORACLE_GATE_SCALAR) a[i] = exp(jb->g[head * L + t]);
            else a[i] = 1.0;
        }
        for (long j = 0; j < dv; ++j)        /* value-dimension gate: outer-product mode only */
            bv[j] = jb->gate_mode == ORACLE_GATE_OUTER ? exp(jb->gv[(head * L + t) * dv + j]) : 1.0;
        /* state update: decay the key rows (and value columns), then add k~ v^T */
        for (long i = 0; i < dk; ++i)
            for (long j = 0; j < dv; ++j)
                S[i * dv + j] = a[i] * bv[j] * S[i * dv + j] + kf[i] * v[t * dv + j];
        /* normaliser state: the same decay, the feature-mapped key added */
        double den = 1.0;
        if (jb->norm) {
            den = 0.0;
            for (long i = 0; i < dk; ++i) {
                z[i] = a[i] * z[i] + kf[i];
                den += qf[i] * z[i];
            }
        }
        /* read-out from the updated state: o_t = S_t^T q~ (normalised: / q~ . z_t) */
        for (long j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (long i = 0; i < dk; ++i) acc += qf[i] * S[i * dv + j];
            o[t * dv + j] = jb->norm ? acc / den : acc;
        }
    }
    if (jb->s_out) memcpy(jb->s_out + head * dk * dv, S, sizeof(double) * dk * dv);
    if (jb->z_out) memcpy(jb->z_out + head * dk, z, sizeof(double) * dk);
}

static void *worker(void *arg)
{
    job_t *jb = (job_t *)arg;
    double *S = (double *)malloc(sizeof(double) * jb->dk * jb->dv);
    double *qf = (double *)malloc(sizeof(double) * jb->dk);
    double *kf = (double *)malloc(sizeof(double) * jb->dk);
    double *a = (double *)malloc(sizeof(double) * jb->dk);
    double *z = (double *)malloc(sizeof(double) * (jb->dk > jb->dv ? jb->dk : jb->dv));
    double *bv = (double *)malloc(sizeof(double) * jb->dv);
    if (S && qf && kf && a && z && bv) {     /* on allocation failure take no head */
        for (;;) {
            pthread_mutex_lock(&jb->lock);
            long head = jb->next_head++;
            pthread_mutex_unlock(&jb->lock);
            if (head >= jb->B * jb->H) break;
            run_head(jb, head, S, qf, kf, a, z, bv);
        }
    }
    free(S); free(qf); free(kf); free(a); free(z); free(bv);
    return NULL;
}

static int forward(const double *q, const double *k, const double *v, const double *g,
                   const double *gv, int gate_mode, int phi, const double *s0, const double *z0,
                   double *o, double *s_out, double *z_out, int norm, const double *beta, long B,
                   long H, long L, long dk, long dv, int nthreads)
{
    if (!q || !k || !v || !o || B < 0 || H < 0 || L < 0 || dk <= 0 || dv <= 0) return -1;
    if (gate_mode != ORACLE_GATE_NONE && gate_mode != ORACLE_GATE_KEYDIM &&
        gate_mode != ORACLE_GATE_SCALAR && gate_mode != ORACLE_GATE_OUTER) return -1;
    if (gate_mode != ORACLE_GATE_NONE && !g) return -1;
    if (gate_mode == ORACLE_GATE_OUTER && (!gv || norm)) return -1;
    if (phi != ORACLE_PHI_IDENTITY && phi != ORACLE_PHI_ELU1) return -1;

    job_t jb;
    jb.q = q; jb.k = k; jb.v = v; jb.g = g; jb.gv = gv; jb.s0 = s0; jb.o = o; jb.s_out = s_out;
    jb.z0 = z0; jb.z_out = z_out; jb.norm = norm;
    jb.beta = beta; jb.delta = beta != NULL;
    jb.B = B; jb.H = H; jb.L = L; jb.dk = dk; jb.dv = dv;
    jb.gate_mode = gate_mode; jb.phi = phi; jb.next_head = 0;
    pthread_mutex_init(&jb.lock, NULL);

    long heads = B * H;
    if (nthreads <= 0) nthreads = 1;
    if (nthreads > heads) nthreads = heads > 0 ? (int)heads : 1;
    /* The heads form a shared work queue: whichever threads start drain all of it,
     * and if none can be started the calling thread does the whole job. */
    pthread_t *th = nthreads > 1 ? (pthread_t *)malloc(sizeof(pthread_t) * nthreads) : NULL;
    int started = 0;
    for (int t = 0; th && t < nthreads; ++t) {
        if (pthread_create(&th[t], NULL, worker, &jb) != 0) break;
        ++started;
    }
    if (started == 0) worker(&jb);
    for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
    free(th);
    pthread_mutex_destroy(&jb.lock);
    /* a worker that failed took no head: if none succeeded, heads are left over */
    if (jb.next_head < B * H) return -2;
    return 0;
}

/*
 * Forward pass over all (b, h).  Returns 0 on success, -1 on bad arguments,
 * -2 if scratch memory could not be allocated.  nthreads <= 0 means 1.
 */
int gla_oracle_forward(const double *q, const double *k, const double *v, const double *g,
                       int gate_mode, int phi, const double *s0, double *o, double *s_out,
                       long B, long H, long L, long dk, long dv, int nthreads)
{
    if (gate_mode == ORACLE_GATE_OUTER) return -1;
    return forward(q, k, v, g, NULL, gate_mode, phi, s0, NULL, o, s_out, NULL, 0, NULL, B, H, L, dk, dv,
                   nthreads);
}

/* The normalised form (see the header): as gla_oracle_forward, plus the normaliser
 * state z0 (nullable: zero) and z_out (nullable). */
int gla_oracle_forward_norm(const double *q, const double *k, const double *v, const double *g,
                            int gate_mode, int phi, const double *s0, const double *z0,
                            double *o, double *s_out, double *z_out, long B, long H, long L,
                            long dk, long dv, int nthreads)
{
    return forward(q, k, v, g, NULL, gate_mode, phi, s0, z0, o, s_out, z_out, 1, NULL, B, H, L, dk, dv,
                   nthreads);
}

/* The delta rule (see the header): beta [B][H][L] required; s0 nullable (zero). */
int gla_oracle_delta(const double *q, const double *k, const double *v, const double *beta,
                     const double *s0, double *o, double *s_out, long B, long H, long L, long dk,
                     long dv, int nthreads)
{
    if (!beta) return -1;
    return forward(q, k, v, NULL, NULL, ORACLE_GATE_NONE, ORACLE_PHI_IDENTITY, s0, NULL, o, s_out, NULL, 0,
                   beta, B, H, L, dk, dv, nthreads);
}

/* The outer-product gate (see the header): g [B][H][L][d_k] and gv [B][H][L][d_v]
 * natural-log gates, both required; s0 nullable (zero). */
int gla_oracle_forward_outer(const double *q, const double *k, const double *v, const double *g,
                             const double *gv, int phi, const double *s0, double *o, double *s_out,
                             long B, long H, long L, long dk, long dv, int nthreads)
{
    return forward(q, k, v, g, gv, ORACLE_GATE_OUTER, phi, s0, NULL, o, s_out, NULL, 0, NULL, B, H, L,
                   dk, dv, nthreads);
}
