/*
 * oracle.c -- plain, slow CPU reference of the conventional SSM decode recurrences.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the bench's CPU-baseline leg load
 * this library; the decode library never calls it and shares no code, header or table with it.
 *
 * What it computes is the definition that ReplaySSM must reproduce: the pages state that the
 * replayed outputs equal those of conventional decoding except for floating-point differences
 * (fagnersouza.tech post "ReplaySSM: o ganho aparece na carga concorrente...", section
 * "Cuidados e limites"), and that conventional decoding reads and rewrites the whole state on
 * every token (same post, lede; ia.goatify.app article, paragraph "ReplaySSM cambia qué se
 * almacena").
 *
 * Arithmetic: fp64 on fp32 inputs, plain loops in the order of the definition, built with
 * -O2 -ffp-contract=off and no fast-math. OpenMP only spreads independent (batch, head) pairs over
 * threads; it does not change any result.
 */
#include <math.h>
#include <stddef.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

/*
 * One conventional Mamba-2 decode token for every (b, h) pair.
 *
 * Discretisation (the plain Mamba-2 reading of "decay, add an outer product, output"):
 *     a       = exp(dt[b,h] * A[h])
 *     S[p][n] = a * S[p][n] + (dt[b,h] * x[b,h,p]) * Bm[b,g,n]
 *     y[p]    = sum_n S[p][n] * C[b,g,n] + D[h] * x[b,h,p]          (post-update state)
 * with g = h / (nh / ng).
 *
 * Layouts (row-major, last index fastest): x [nb,nh,P], Bm and C [nb,ng,N], dt [nb,nh],
 * A and D [nh], state [nb,nh,P,N] (fp64, updated in place), y [nb,nh,P] (fp64, written).
 */
void orc_m2_step(int nb, int nh, int ng, int P, int N,
                 const float *A, const float *D,
                 const float *x, const float *Bm, const float *C, const float *dt,
                 double *state, double *y)
{
    const int hpg = nh / ng;
    const long pairs = (long)nb * nh;
#pragma omp parallel for schedule(static)
    for (long bh = 0; bh < pairs; ++bh) {
        const long b = bh / nh;
        const int h = (int)(bh % nh);
        const int g = h / hpg;
        const double dtv = (double)dt[bh];
        const double a = exp(dtv * (double)A[h]);
        const float *xv = x + bh * P;
        const float *Bv = Bm + (b * ng + g) * N;
        const float *Cv = C + (b * ng + g) * N;
        double *S = state + bh * (long)P * N;
        for (int p = 0; p < P; ++p) {
            const double coef = dtv * (double)xv[p];
            double acc = 0.0;
            for (int n = 0; n < N; ++n) {
                const double s = a * S[(long)p * N + n] + coef * (double)Bv[n];
                S[(long)p * N + n] = s;
                acc += s * (double)Cv[n];
            }
            y[bh * P + p] = acc + (double)D[h] * (double)xv[p];
        }
    }
}

/*
 * One conventional Gated DeltaNet decode token for every (b, h) pair. The state S is d_v x d_k
 * (row i is an output channel), so the rank-1 correction multiplies from the right:
 *     S   <- alpha * S (I - beta k k^T) + beta v k^T
 *          = alpha * (S - beta (S k) k^T) + beta v k^T
 *     o    = S q                                                     (post-update state)
 * Layouts: q, k [nb,nh,dk], v [nb,nh,dv], beta and alpha [nb,nh], state [nb,nh,dv,dk] fp64 in
 * place, o [nb,nh,dv] fp64.
 */
void orc_gdn_step(int nb, int nh, int dk, int dv,
                  const float *q, const float *k, const float *v,
                  const float *beta, const float *alpha,
                  double *state, double *o)
{
    const long pairs = (long)nb * nh;
#pragma omp parallel for schedule(static)
    for (long bh = 0; bh < pairs; ++bh) {
        const double be = (double)beta[bh];
        const double al = (double)alpha[bh];
        const float *qv = q + bh * dk;
        const float *kv = k + bh * dk;
        const float *vv = v + bh * dv;
        double *S = state + bh * (long)dv * dk;
        for (int i = 0; i < dv; ++i) {
            double *row = S + (long)i * dk;
            double sk = 0.0;
            for (int j = 0; j < dk; ++j) sk += row[j] * (double)kv[j];
            double acc = 0.0;
            for (int j = 0; j < dk; ++j) {
                const double s = al * (row[j] - be * sk * (double)kv[j])
                               + be * (double)vv[i] * (double)kv[j];
                row[j] = s;
                acc += s * (double)qv[j];
            }
            o[bh * dv + i] = acc;
        }
    }
}

/*
 * The same conventional Mamba-2 token evaluated in fp32: the state is fp32, every operation is
 * rounded to fp32 in the order of the definition above (exp by the C library's expf, the output
 * sum accumulated over n in increasing order, no contraction). This is conventional decoding as
 * an fp32 implementation runs it; the pages fix the state precision at FP32 (fagnersouza.tech
 * post, section "O que muda para quem desenvolve"), and the outputs of the method are to equal
 * conventional decoding up to floating-point differences (same post, "Cuidados e limites"). It
 * gives the size of those differences on given inputs; it is not what the GPU path is checked
 * against. Layouts as orc_m2_step; state [nb,nh,P,N] fp32 in place, y [nb,nh,P] fp32.
 */
void orc_m2_step_f32(int nb, int nh, int ng, int P, int N,
                     const float *A, const float *D,
                     const float *x, const float *Bm, const float *C, const float *dt,
                     float *state, float *y)
{
    const int hpg = nh / ng;
    const long pairs = (long)nb * nh;
#pragma omp parallel for schedule(static)
    for (long bh = 0; bh < pairs; ++bh) {
        const long b = bh / nh;
        const int h = (int)(bh % nh);
        const int g = h / hpg;
        const float dtv = dt[bh];
        const float a = expf(dtv * A[h]);
        const float *xv = x + bh * P;
        const float *Bv = Bm + (b * ng + g) * N;
        const float *Cv = C + (b * ng + g) * N;
        float *S = state + bh * (long)P * N;
        for (int p = 0; p < P; ++p) {
            const float coef = dtv * xv[p];
            float acc = 0.0f;
            for (int n = 0; n < N; ++n) {
                const float s = a * S[(long)p * N + n] + coef * Bv[n];
                S[(long)p * N + n] = s;
                acc += s * Cv[n];
            }
            y[bh * P + p] = acc + D[h] * xv[p];
        }
    }
}

/*
 * Conditioning of one Gated DeltaNet token, for rounding-error bounds. M [nb,nh,dv,dk] (fp64, in
 * place) bounds, entry by entry, the absolute values of the terms the update sums: with
 * s_i = sum_l M[i][l] |k_l|,
 *     M[i][j] <- alpha (M[i][j] + beta s_i |k_j|) + beta |v_i| |k_j|
 * (the three terms of alpha (S - beta (S k) k^T) + beta v k^T), starting from |S_0|; and
 *     kappa[i] = sum_j M[i][j] |q_j|
 * bounds the terms of the output o = S q. A rounding error of relative size e on any term moves
 * o_i by at most e kappa_i. Layouts as orc_gdn_step; kappa [nb,nh,dv].
 */
void orc_gdn_kappa_step(int nb, int nh, int dk, int dv,
                        const float *q, const float *k, const float *v,
                        const float *beta, const float *alpha,
                        double *M, double *kappa)
{
    const long pairs = (long)nb * nh;
#pragma omp parallel for schedule(static)
    for (long bh = 0; bh < pairs; ++bh) {
        const double be = (double)beta[bh];
        const double al = (double)alpha[bh];
        const float *qv = q + bh * dk;
        const float *kv = k + bh * dk;
        const float *vv = v + bh * dv;
        double *Mt = M + bh * (long)dv * dk;
        for (int i = 0; i < dv; ++i) {
            double *row = Mt + (long)i * dk;
            double s = 0.0;
            for (int j = 0; j < dk; ++j) s += row[j] * fabs((double)kv[j]);
            double acc = 0.0;
            for (int j = 0; j < dk; ++j) {
                const double kj = fabs((double)kv[j]);
                const double m = al * (row[j] + be * s * kj) + be * fabs((double)vv[i]) * kj;
                row[j] = m;
                acc += m * fabs((double)qv[j]);
            }
            kappa[bh * dv + i] = acc;
        }
    }
}

/*
 * One conventional Kimi Delta Attention decode token for every (b, h) pair. The pages name Kimi
 * Delta Attention as the third SSM layer type of the hybrids ReplaySSM targets (news.hamidun.com
 * item "NVIDIA présente ReplaySSM : accélérer le décodage des modèles hybrides Mamba et GDN",
 * section "Pourquoi les hybrides sont devenus la norme") but give no formula. Read here as the
 * delta rule of Gated DeltaNet with the scalar forget gate replaced by one gate per key channel
 * (a vector a in (0, 1]^dk applied before the rank-1 correction); with S d_v x d_k as for Gated
 * DeltaNet (row i is an output channel):
 *     S   <- S diag(a) (I - beta k k^T) + beta v k^T
 *          = S' - beta (S' k) k^T + beta v k^T,       S' = S diag(a)  (column j scaled by a_j)
 *     o    = S q                                                     (post-update state)
 * With a_j = alpha for every j this is the Gated DeltaNet step above.
 * Layouts: q, k, a [nb,nh,dk], v [nb,nh,dv], beta [nb,nh], state [nb,nh,dv,dk] fp64 in place,
 * o [nb,nh,dv] fp64.
 */
void orc_kda_step(int nb, int nh, int dk, int dv,
                  const float *q, const float *k, const float *v,
                  const float *beta, const float *a,
                  double *state, double *o)
{
    const long pairs = (long)nb * nh;
#pragma omp parallel for schedule(static)
    for (long bh = 0; bh < pairs; ++bh) {
        const double be = (double)beta[bh];
        const float *qv = q + bh * dk;
        const float *kv = k + bh * dk;
        const float *av = a + bh * dk;
        const float *vv = v + bh * dv;
        double *S = state + bh * (long)dv * dk;
        for (int i = 0; i < dv; ++i) {
            double *row = S + (long)i * dk;
            for (int j = 0; j < dk; ++j) row[j] = row[j] * (double)av[j];
            double sk = 0.0;
            for (int j = 0; j < dk; ++j) sk += row[j] * (double)kv[j];
            double acc = 0.0;
            for (int j = 0; j < dk; ++j) {
                const double s = row[j] - be * sk * (double)kv[j] + be * (double)vv[i] * (double)kv[j];
                row[j] = s;
                acc += s * (double)qv[j];
            }
            o[bh * dv + i] = acc;
        }
    }
}

/*
 * Conditioning of one Kimi Delta Attention token (as orc_gdn_kappa_step): M bounds the absolute
 * values of the terms the update sums, with s_i = sum_l a_l M[i][l] |k_l|,
 *     M[i][j] <- a_j M[i][j] + beta s_i |k_j| + beta |v_i| |k_j|,
 * starting from |S_0|, and kappa[i] = sum_j M[i][j] |q_j|. Layouts as orc_kda_step.
 */
void orc_kda_kappa_step(int nb, int nh, int dk, int dv,
                        const float *q, const float *k, const float *v,
                        const float *beta, const float *a,
                        double *M, double *kappa)
{
    const long pairs = (long)nb * nh;
#pragma omp parallel for schedule(static)
    for (long bh = 0; bh < pairs; ++bh) {
        const double be = (double)beta[bh];
        const float *qv = q + bh * dk;
        const float *kv = k + bh * dk;
        const float *av = a + bh * dk;
        const float *vv = v + bh * dv;
        double *Mt = M + bh * (long)dv * dk;
        for (int i = 0; i < dv; ++i) {
            double *row = Mt + (long)i * dk;
            double s = 0.0;
            for (int j = 0; j < dk; ++j) s += (double)av[j] * row[j] * fabs((double)kv[j]);
            double acc = 0.0;
            for (int j = 0; j < dk; ++j) {
                const double kj = fabs((double)kv[j]);
                const double m = (double)av[j] * row[j] + be * s * kj + be * fabs((double)vv[i]) * kj;
                row[j] = m;
                acc += m * fabs((double)qv[j]);
            }
            kappa[bh * dv + i] = acc;
        }
    }
}
