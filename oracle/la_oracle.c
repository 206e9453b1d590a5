/*
 * la_oracle.c -- plain fp64 CPU oracle for Transformer-based linear attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header, table or helper with
 * the HIP library.
 *
 * What it computes (sources are the pages about the paper "Transformer Based
 * Linear Attention with Optimized GPU Kernel Implementation"):
 *
 *   - sciencestack.ai page, TL;DR: LA is a forward/backward formulation with a
 *     normalisation scheme, O(N D^2) time and O(N D) memory, with analytical
 *     gradients for the LA head.
 *   - same page, Figure 1 caption: the kernel evaluates a "linear term"; the
 *     reading adopted here is that the similarity of a query and a key is a
 *     constant term plus a linear term, sim(q, k) = 1 + q.k (the first two
 *     Taylor terms of the exponential used by softmax attention).
 *   - cloud.baidu.com article (section 2, matrix-product reordering and the
 *     state-update pseudocode): computing K^T V (D x D) first and then
 *     Q (K^T V) gives O(N D^2), and causally the state is grown token by token
 *     with the outer product k_t v_t^T.
 *
 * Definition (per head, rows of the [B,H,N,D] tensors, J(i) = all j for the
 * non-causal case and j <= i for the causal case):
 *
 *     w_ij  = 1 + q_i . k_j                     (j in J(i))
 *     den_i = sum_j w_ij
 *     o_i   = (sum_j w_ij v_j) / den_i
 *
 * Backward, for the scalar loss L = sum_i g_i . o_i (g = dO):
 *
 *     a_i = g_i / den_i,   c_i = a_i . o_i
 *     dq_i = sum_{j in J(i)} (a_i . v_j - c_i) k_j
 *     dk_j = sum_{i : j in J(i)} (a_i . v_j - c_i) q_i
 *     dv_j = sum_{i : j in J(i)} w_ij a_i
 *
 * Two independent evaluations are provided:
 *   *_direct : the O(N^2 D) definition written out, pair by pair.
 *   *_state  : the method's reordering, O(N D^2): non-causal sums the state
 *              S = sum_j k_j v_j^T, z = sum_j k_j, u = sum_j v_j, n = N once;
 *              causal grows (S, z, u, n) one token at a time.  The backward
 *              uses the matching states of the gradient (R = sum q a^T,
 *              r = sum c q, t = sum a), summed over the visible queries.
 *
 * Carried state (a sequence processed in pieces; the state-update pseudocode
 * of the cloud.baidu.com article grows one running state, so a piece can start
 * from the state its predecessors left): the *_carry entry points take a
 * record [S (D x D) | z (D) | u (D)] standing for n0 tokens outside the call
 * whose keys every row of the call sees (causal: the tokens before it;
 * non-causal: the rest of the sequence), and return the record of those
 * tokens plus the call's own.  Their backward takes the matching gradient
 * record [R | r | t] of the rows outside the call that see the call's keys
 * (causal: the rows after it; non-causal: the other rows) and returns it
 * plus the call's own rows' record.  With empty carries they are exactly the
 * *_state evaluations.
 *
 * Where the pages are silent (no epsilon in the denominator, no scaling of
 * q.k, identity feature map, causal mask includes the diagonal) the plainest
 * reading is taken; the denominator is divided as is (IEEE semantics).
 *
 * All arrays are fp64, layout [B,H,N,D] contiguous (den: [B,H,N]).
 * Heads are independent, so the only parallelism is one OpenMP thread per
 * head; inside a head everything runs in the order written.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* constant term + linear term of the similarity */
static double sim(const double *q, const double *k, int64_t D)
{
    double dot = 0.0;
    for (int64_t d = 0; d < D; ++d)
        dot += q[d] * k[d];
    return 1.0 + dot;
}

static double dotv(const double *x, const double *y, int64_t D)
{
    double s = 0.0;
    for (int64_t d = 0; d < D; ++d)
        s += x[d] * y[d];
    return s;
}

/* number of keys visible to query i */
static int64_t visible(int64_t i, int64_t N, int causal)
{
    return causal ? i + 1 : N;
}

int la_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------- direct */

static void head_forward_direct(const double *q, const double *k,
                                const double *v, double *o, double *den,
                                int64_t N, int64_t D, int causal)
{
    for (int64_t i = 0; i < N; ++i) {
        double *oi = o + i * D;
        double deni = 0.0;
        for (int64_t e = 0; e < D; ++e)
            oi[e] = 0.0;
        for (int64_t j = 0; j < visible(i, N, causal); ++j) {
            double w = sim(q + i * D, k + j * D, D);
            deni += w;
            for (int64_t e = 0; e < D; ++e)
                oi[e] += w * v[j * D + e];
        }
        for (int64_t e = 0; e < D; ++e)
            oi[e] /= deni;
        if (den)
            den[i] = deni;
    }
}

void la_oracle_forward_direct(const double *Q, const double *K,
                              const double *V, double *O, double *den,
                              int64_t B, int64_t H, int64_t N, int64_t D,
                              int causal)
{
    int64_t heads = B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t h = 0; h < heads; ++h) {
        int64_t off = h * N * D;
        head_forward_direct(Q + off, K + off, V + off, O + off,
                            den ? den + h * N : NULL, N, D, causal);
    }
}

static void head_backward_direct(const double *q, const double *k,
                                 const double *v, const double *g,
                                 double *dq, double *dk, double *dv,
                                 int64_t N, int64_t D, int causal)
{
    double *o = (double *)malloc(sizeof(double) * (size_t)(N * D));
    double *den = (double *)malloc(sizeof(double) * (size_t)N);
    double *a = (double *)malloc(sizeof(double) * (size_t)D);
    head_forward_direct(q, k, v, o, den, N, D, causal);
    memset(dq, 0, sizeof(double) * (size_t)(N * D));
    memset(dk, 0, sizeof(double) * (size_t)(N * D));
    memset(dv, 0, sizeof(double) * (size_t)(N * D));
    for (int64_t i = 0; i < N; ++i) {
        for (int64_t e = 0; e < D; ++e)
            a[e] = g[i * D + e] / den[i];
        double c = dotv(a, o + i * D, D);
        for (int64_t j = 0; j < visible(i, N, causal); ++j) {
            double m = dotv(a, v + j * D, D) - c;   /* dL/d(q_i . k_j) */
            double w = sim(q + i * D, k + j * D, D);
            for (int64_t d = 0; d < D; ++d) {
                dq[i * D + d] += m * k[j * D + d];
                dk[j * D + d] += m * q[i * D + d];
                dv[j * D + d] += w * a[d];
            }
        }
    }
    free(a);
    free(den);
    free(o);
}

void la_oracle_backward_direct(const double *Q, const double *K,
                               const double *V, const double *dO, double *dQ,
                               double *dK, double *dV, int64_t B, int64_t H,
                               int64_t N, int64_t D, int causal)
{
    int64_t heads = B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t h = 0; h < heads; ++h) {
        int64_t off = h * N * D;
        head_backward_direct(Q + off, K + off, V + off, dO + off, dQ + off,
                             dK + off, dV + off, N, D, causal);
    }
}

/* ----------------------------------------------------------------- state */

/* S += k v^T, z += k, u += v */
static void state_add(double *S, double *z, double *u, const double *k,
                      const double *v, int64_t D)
{
    for (int64_t d = 0; d < D; ++d) {
        for (int64_t e = 0; e < D; ++e)
            S[d * D + e] += k[d] * v[e];
        z[d] += k[d];
        u[d] += v[d];
    }
}

/* den = n + q.z ; o = (u + S^T q) / den */
static double state_apply(const double *S, const double *z, const double *u,
                          double n, const double *q, double *o, int64_t D)
{
    double den = n + dotv(q, z, D);
    for (int64_t e = 0; e < D; ++e) {
        double num = u[e];
        for (int64_t d = 0; d < D; ++d)
            num += q[d] * S[d * D + e];
        o[e] = num / den;
    }
    return den;
}

/* record [S | z | u] <-> separate arrays (NULL record = zero state) */
static void record_load(const double *rec, double *S, double *z, double *u,
                        int64_t D)
{
    if (!rec)
        return;
    memcpy(S, rec, sizeof(double) * (size_t)(D * D));
    memcpy(z, rec + D * D, sizeof(double) * (size_t)D);
    memcpy(u, rec + D * D + D, sizeof(double) * (size_t)D);
}

static void record_store(double *rec, const double *S, const double *z,
                         const double *u, int64_t D)
{
    if (!rec)
        return;
    memcpy(rec, S, sizeof(double) * (size_t)(D * D));
    memcpy(rec + D * D, z, sizeof(double) * (size_t)D);
    memcpy(rec + D * D + D, u, sizeof(double) * (size_t)D);
}

/* The state starts from rec_in (n0 tokens), or zero; rec_out gets the final
 * state. */
static void head_forward_state(const double *q, const double *k,
                               const double *v, double *o, double *den,
                               int64_t N, int64_t D, int causal,
                               const double *rec_in, double n0,
                               double *rec_out)
{
    double *S = (double *)calloc((size_t)(D * D), sizeof(double));
    double *z = (double *)calloc((size_t)D, sizeof(double));
    double *u = (double *)calloc((size_t)D, sizeof(double));
    record_load(rec_in, S, z, u, D);
    if (!causal) {
        for (int64_t j = 0; j < N; ++j)
            state_add(S, z, u, k + j * D, v + j * D, D);
        for (int64_t i = 0; i < N; ++i) {
            double di = state_apply(S, z, u, n0 + (double)N, q + i * D,
                                    o + i * D, D);
            if (den)
                den[i] = di;
        }
    } else {
        for (int64_t i = 0; i < N; ++i) {
            state_add(S, z, u, k + i * D, v + i * D, D);
            double di = state_apply(S, z, u, n0 + (double)(i + 1), q + i * D,
                                    o + i * D, D);
            if (den)
                den[i] = di;
        }
    }
    record_store(rec_out, S, z, u, D);
    free(u);
    free(z);
    free(S);
}

void la_oracle_forward_state(const double *Q, const double *K,
                             const double *V, double *O, double *den,
                             int64_t B, int64_t H, int64_t N, int64_t D,
                             int causal)
{
    int64_t heads = B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t h = 0; h < heads; ++h) {
        int64_t off = h * N * D;
        head_forward_state(Q + off, K + off, V + off, O + off,
                           den ? den + h * N : NULL, N, D, causal, NULL, 0.0,
                           NULL);
    }
}

/* records: [B,H,D*D+2D]; rec_in may be NULL (zero state) */
void la_oracle_forward_carry(const double *Q, const double *K,
                             const double *V, double *O, double *den,
                             const double *rec_in, double n0, double *rec_out,
                             int64_t B, int64_t H, int64_t N, int64_t D,
                             int causal)
{
    int64_t heads = B * H, PS = D * D + 2 * D;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t h = 0; h < heads; ++h) {
        int64_t off = h * N * D;
        head_forward_state(Q + off, K + off, V + off, O + off,
                           den ? den + h * N : NULL, N, D, causal,
                           rec_in ? rec_in + h * PS : NULL, n0,
                           rec_out + h * PS);
    }
}

/*
 * Query-side gradient for one row, given the state (S, z, u, n) visible to it:
 *   den = n + q.z, a = g / den, y = S a, o = (u + S^T q) / den, c = a.o,
 *   dq = y - c z.   Returns c; writes a and dq.
 */
static double state_grad_query(const double *S, const double *z,
                               const double *u, double n, const double *q,
                               const double *g, double *a, double *dq,
                               double *o_tmp, int64_t D)
{
    double den = state_apply(S, z, u, n, q, o_tmp, D);
    for (int64_t e = 0; e < D; ++e)
        a[e] = g[e] / den;
    double c = dotv(a, o_tmp, D);
    for (int64_t d = 0; d < D; ++d) {
        double y = 0.0;
        for (int64_t e = 0; e < D; ++e)
            y += S[d * D + e] * a[e];
        dq[d] = y - c * z[d];
    }
    return c;
}

/* R += q a^T, r += c q, t += a */
static void grad_state_add(double *R, double *r, double *t, const double *q,
                           const double *a, double c, int64_t D)
{
    for (int64_t d = 0; d < D; ++d) {
        for (int64_t e = 0; e < D; ++e)
            R[d * D + e] += q[d] * a[e];
        r[d] += c * q[d];
        t[d] += a[d];
    }
}

/* dk = R v - r ; dv = t + R^T k */
static void grad_state_apply(const double *R, const double *r,
                             const double *t, const double *k,
                             const double *v, double *dk, double *dv,
                             int64_t D)
{
    for (int64_t d = 0; d < D; ++d) {
        double s = 0.0;
        for (int64_t e = 0; e < D; ++e)
            s += R[d * D + e] * v[e];
        dk[d] = s - r[d];
    }
    for (int64_t e = 0; e < D; ++e) {
        double s = t[e];
        for (int64_t d = 0; d < D; ++d)
            s += R[d * D + e] * k[d];
        dv[e] = s;
    }
}

/* The forward state starts from rec_in (n0 tokens), the gradient state from
 * grec_in; grec_out gets the final gradient state. */
static void head_backward_state(const double *q, const double *k,
                                const double *v, const double *g, double *dq,
                                double *dk, double *dv, int64_t N, int64_t D,
                                int causal, const double *rec_in, double n0,
                                const double *grec_in, double *grec_out)
{
    size_t DD = (size_t)(D * D);
    double *S = (double *)calloc(DD, sizeof(double));
    double *z = (double *)calloc((size_t)D, sizeof(double));
    double *u = (double *)calloc((size_t)D, sizeof(double));
    double *R = (double *)calloc(DD, sizeof(double));
    double *r = (double *)calloc((size_t)D, sizeof(double));
    double *t = (double *)calloc((size_t)D, sizeof(double));
    double *otmp = (double *)malloc(sizeof(double) * (size_t)D);
    double *A = (double *)malloc(sizeof(double) * (size_t)(N * D));
    double *C = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    record_load(rec_in, S, z, u, D);
    record_load(grec_in, R, r, t, D);

    if (!causal) {
        for (int64_t j = 0; j < N; ++j)
            state_add(S, z, u, k + j * D, v + j * D, D);
        for (int64_t i = 0; i < N; ++i)
            C[i] = state_grad_query(S, z, u, n0 + (double)N, q + i * D,
                                    g + i * D, A + i * D, dq + i * D, otmp, D);
        for (int64_t i = 0; i < N; ++i)
            grad_state_add(R, r, t, q + i * D, A + i * D, C[i], D);
        for (int64_t j = 0; j < N; ++j)
            grad_state_apply(R, r, t, k + j * D, v + j * D, dk + j * D,
                             dv + j * D, D);
    } else {
        /* forward sweep: prefix states (including token i) feed dq_i */
        for (int64_t i = 0; i < N; ++i) {
            state_add(S, z, u, k + i * D, v + i * D, D);
            C[i] = state_grad_query(S, z, u, n0 + (double)(i + 1), q + i * D,
                                    g + i * D, A + i * D, dq + i * D, otmp, D);
        }
        /* reverse sweep: suffix states (queries i >= j) feed dk_j, dv_j */
        for (int64_t j = N - 1; j >= 0; --j) {
            grad_state_add(R, r, t, q + j * D, A + j * D, C[j], D);
            grad_state_apply(R, r, t, k + j * D, v + j * D, dk + j * D,
                             dv + j * D, D);
        }
    }
    record_store(grec_out, R, r, t, D);
    free(C);
    free(A);
    free(otmp);
    free(t);
    free(r);
    free(R);
    free(u);
    free(z);
    free(S);
}

void la_oracle_backward_state(const double *Q, const double *K,
                              const double *V, const double *dO, double *dQ,
                              double *dK, double *dV, int64_t B, int64_t H,
                              int64_t N, int64_t D, int causal)
{
    int64_t heads = B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t h = 0; h < heads; ++h) {
        int64_t off = h * N * D;
        head_backward_state(Q + off, K + off, V + off, dO + off, dQ + off,
                            dK + off, dV + off, N, D, causal, NULL, 0.0, NULL,
                            NULL);
    }
}

/* records: [B,H,D*D+2D]; rec_in and grec_in may be NULL (zero state) */
void la_oracle_backward_carry(const double *Q, const double *K,
                              const double *V, const double *dO, double *dQ,
                              double *dK, double *dV, const double *rec_in,
                              double n0, const double *grec_in,
                              double *grec_out, int64_t B, int64_t H,
                              int64_t N, int64_t D, int causal)
{
    int64_t heads = B * H, PS = D * D + 2 * D;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t h = 0; h < heads; ++h) {
        int64_t off = h * N * D;
        head_backward_state(Q + off, K + off, V + off, dO + off, dQ + off,
                            dK + off, dV + off, N, D, causal,
                            rec_in ? rec_in + h * PS : NULL, n0,
                            grec_in ? grec_in + h * PS : NULL,
                            grec_out + h * PS);
    }
}
