/*
 * CPU oracle for the Mamba-2 SSD layer scan -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library.  The product path (the HIP library) never calls it
 * and shares no code, header or table with it.
 *
 * What it computes is the plain definition of the layer, token by token, in
 * float64 ("Accelerating Mamba-2 with High-Performance Forward Pass Kernels in
 * NVIDIA CUDA Tile", section "Mamba-2 architecture"; the same update is the
 * decode step of "Optimizing Nemotron v3 Super in TensorRT-LLM", section 6.1
 * "The SSU Math"):
 *
 *     h_t = exp(A_h * dt_t) * h_{t-1} + dt_t * x_t (outer) B_t      (P x N)
 *     y_t = h_t C_t + D_h * x_t                                      (P)
 *
 * The output uses the updated state h_t (the diagonal of the causal mask is
 * included).  Optionally (the layer interface around the scan, "Optimizing
 * Nemotron v3 Super in TensorRT-LLM", sections 6.1 and 6.3): the step is
 * preprocessed per token, dt <- dt + dt_bias_h and then, if requested,
 * dt <- softplus(dt) = log(1 + e^dt) for dt <= 20 (left as is above 20); and
 * the output is gated, y_t <- y_t * silu(z_t) with silu(z) = z / (1 + e^-z),
 * after the D term.  The gate does not touch the state.  Head h reads B and C of group h / (H / G).  The state of head h
 * is stored [P][N] (N contiguous).  The chunked SSD form the GPU path uses is
 * an algebraic rearrangement of exactly this recurrence, so the recurrence is
 * the reference.
 *
 * Rows p of one (b, h) never interact, so the unit of work is one (b, h, p)
 * row: an N-vector of state carried over all T tokens.  Rows are handed out
 * to a pool of POSIX threads through an atomic counter.
 *
 * Inputs are float32 arrays (bf16 inputs arrive exactly upcast); the state,
 * every product and every sum are float64, and exp is the host libm exp.
 */
#define _GNU_SOURCE
#include <math.h>
#include <pthread.h>
#include <sched.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

typedef struct {
    const float *x, *dt, *A, *B, *C, *D;
    const float *dt_bias;   /* [H] or NULL */
    int softplus;           /* nonzero: softplus on dt (+ bias), identity above 20 */
    const float *z;         /* [Bt,T,H,P] gate or NULL */
    const double *init;     /* [npairs][P][N] or NULL */
    double *y;              /* [npairs][T][P] or NULL */
    double *fin;            /* [npairs][P][N] or NULL */
    int64_t Bt, T, H, P, N, G;
    const int64_t *pairs;   /* flattened b*H + h, npairs entries, or NULL = all */
    int64_t npairs;
    int64_t nunits;         /* npairs * P */
    int64_t next;           /* work counter */
} fwd_job;

static void run_row(const fwd_job *j, int64_t unit, double *s)
{
    const int64_t pi = unit / j->P, p = unit % j->P;
    const int64_t bh = j->pairs ? j->pairs[pi] : pi;
    const int64_t b = bh / j->H, h = bh % j->H;
    const int64_t hpg = j->H / j->G, g = h / hpg;
    const int64_t T = j->T, H = j->H, P = j->P, N = j->N, G = j->G;
    const double A = (double)j->A[h], D = (double)j->D[h];

    if (j->init)
        for (int64_t n = 0; n < N; ++n) s[n] = j->init[(pi * P + p) * N + n];
    else
        for (int64_t n = 0; n < N; ++n) s[n] = 0.0;

    for (int64_t t = 0; t < T; ++t) {
        const int64_t bt = b * T + t;
        double dt = (double)j->dt[bt * H + h];
        if (j->dt_bias) dt += (double)j->dt_bias[h];
        if (j->softplus && dt <= 20.0) dt = log1p(exp(dt));
        const double xv = (double)j->x[(bt * H + h) * P + p];
        const float *Bv = j->B + (bt * G + g) * N;
        const float *Cv = j->C + (bt * G + g) * N;
        const double alpha = exp(A * dt);
        const double u = dt * xv;
        double acc = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            const double v = alpha * s[n] + u * (double)Bv[n];
            s[n] = v;
            acc += (double)Cv[n] * v;
        }
        double yv = acc + D * xv;
        if (j->z) {
            const double zv = (double)j->z[(bt * H + h) * P + p];
            yv *= zv / (1.0 + exp(-zv));
        }
        if (j->y) j->y[(pi * T + t) * P + p] = yv;
    }
    if (j->fin)
        for (int64_t n = 0; n < N; ++n) j->fin[(pi * P + p) * N + n] = s[n];
}

static void *worker(void *arg)
{
    fwd_job *j = (fwd_job *)arg;
    double *s = (double *)malloc(sizeof(double) * (size_t)j->N);
    if (!s) return NULL;
    for (;;) {
        int64_t u = __atomic_fetch_add(&j->next, 1, __ATOMIC_RELAXED);
        if (u >= j->nunits) break;
        run_row(j, u, s);
    }
    free(s);
    return NULL;
}

/* Number of host threads this process may run on (affinity mask). */
int ssd_oracle_host_threads(void)
{
    cpu_set_t set;
    if (sched_getaffinity(0, sizeof(set), &set) == 0) {
        int c = CPU_COUNT(&set);
        if (c > 0) return c;
    }
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}

/*
 * Token-by-token forward over the (b, h) pairs listed in `pairs` (b*H + h;
 * NULL = all Bt*H pairs in order).  x [Bt,T,H,P], dt [Bt,T,H], A [H],
 * B and C [Bt,T,G,N], D [H]; init [npairs,P,N] (NULL = zeros); outputs
 * y [npairs,T,P] and fin [npairs,P,N] (either may be NULL).  init may alias
 * fin.  dt_bias [H] (NULL = none), softplus (0/1) and the gate z [Bt,T,H,P]
 * (NULL = none) are the optional layer interface described above.  Returns
 * the number of threads used, or a negative value on a bad argument.
 */
int ssd_oracle_fwd_gated(const float *x, const float *dt, const float *A, const float *B,
                         const float *C, const float *D, const float *dt_bias, int softplus,
                         const float *z, const double *init, int64_t Bt, int64_t T, int64_t H,
                         int64_t P, int64_t N, int64_t G, const int64_t *pairs, int64_t npairs,
                         double *y, double *fin, int nthreads)
{
    if (!x || !dt || !A || !B || !C || !D) return -1;
    if (Bt < 1 || T < 0 || H < 1 || P < 1 || N < 1 || G < 1 || H % G) return -2;
    if (!pairs) npairs = Bt * H;
    for (int64_t i = 0; pairs && i < npairs; ++i)
        if (pairs[i] < 0 || pairs[i] >= Bt * H) return -3;

    fwd_job j = {x, dt, A, B, C, D, dt_bias, softplus, z, init, y, fin, Bt, T, H, P, N, G,
                 pairs, npairs, npairs * P, 0};
    if (nthreads <= 0) nthreads = ssd_oracle_host_threads();
    if (nthreads > j.nunits) nthreads = (int)(j.nunits > 0 ? j.nunits : 1);

    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!th) return -4;
    int started = 0;
    for (int i = 1; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, worker, &j) != 0) break;
        ++started;
    }
    worker(&j);
    for (int i = 1; i <= started; ++i) pthread_join(th[i], NULL);
    free(th);
    return started + 1;
}

/* The plain recurrence: no dt preprocessing, no gate. */
int ssd_oracle_fwd(const float *x, const float *dt, const float *A, const float *B,
                   const float *C, const float *D, const double *init,
                   int64_t Bt, int64_t T, int64_t H, int64_t P, int64_t N, int64_t G,
                   const int64_t *pairs, int64_t npairs, double *y, double *fin,
                   int nthreads)
{
    return ssd_oracle_fwd_gated(x, dt, A, B, C, D, NULL, 0, NULL, init, Bt, T, H, P, N, G,
                                pairs, npairs, y, fin, nthreads);
}

/*
 * One recurrent decode step ("Optimizing Nemotron v3 Super in TensorRT-LLM",
 * section 6.1): the forward body for a single token, with the state read from
 * and written back to `state` [npairs,P,N].  x_t [Bt,H,P], dt_t [Bt,H],
 * B_t and C_t [Bt,G,N]; y_t [npairs,P].
 */
int ssd_oracle_decode(double *state, const float *x_t, const float *dt_t, const float *B_t,
                      const float *C_t, const float *A, const float *D,
                      int64_t Bt, int64_t H, int64_t P, int64_t N, int64_t G,
                      const int64_t *pairs, int64_t npairs, double *y_t, int nthreads)
{
    if (!state) return -1;
    return ssd_oracle_fwd(x_t, dt_t, A, B_t, C_t, D, state, Bt, 1, H, P, N, G, pairs, npairs,
                          y_t, state, nthreads);
}

/* The decode step with the optional dt preprocessing and gate z_t [Bt,H,P]. */
int ssd_oracle_decode_gated(double *state, const float *x_t, const float *dt_t,
                            const float *B_t, const float *C_t, const float *A, const float *D,
                            const float *dt_bias, int softplus, const float *z_t, int64_t Bt,
                            int64_t H, int64_t P, int64_t N, int64_t G, const int64_t *pairs,
                            int64_t npairs, double *y_t, int nthreads)
{
    if (!state) return -1;
    return ssd_oracle_fwd_gated(x_t, dt_t, A, B_t, C_t, D, dt_bias, softplus, z_t, state, Bt, 1,
                                H, P, N, G, pairs, npairs, y_t, state, nthreads);
}

/*
 * The backward of the plain forward: the exact adjoint of the recurrence,
 * token by token in float64.  With g_t = dL/dh_t (P x N), starting from
 * g = dL/d(final state) and walking t = T .. 1:
 *
 *     g_t    = (g from later tokens) + dy_t (outer) C_t
 *     dC_t  += h_t^T dy_t                 (summed over the heads of the group)
 *     dx_t   = D dy_t + dt_t g_t B_t
 *     dB_t  += dt_t g_t^T x_t             (summed over the heads of the group)
 *     ddt_t  = x_t^T g_t B_t + A a_t <g_t, h_{t-1}>,   a_t = exp(A dt_t)
 *     dA    += dt_t a_t <g_t, h_{t-1}>     (summed over batch and tokens)
 *     dD    += dy_t . x_t                  (summed over batch and tokens)
 *     g_{t-1} = a_t g_t,   and finally dL/d(init state) = g_0.
 *
 * This is the chain rule applied to the recurrence of the header comment
 * (the "mamba3" kernel card, section "Backward", gives the chunked order of the
 * same adjoint: a reverse scan of the state adjoint between chunk-parallel
 * passes).  Rows p of a head do not interact, so each row's forward states
 * are stored (T + 1 vectors of N) and walked back.  The unit of work is one
 * (b, g): all rows of all heads of group g in batch row b, in head and row
 * order, so the sums over heads and rows are taken in a fixed order; dA and
 * dD are summed over b in order at the end.
 */
typedef struct {
    const float *x, *dt, *A, *B, *C, *D, *dy, *dfin;
    const double *init;      /* [Bt*H][P][N] or NULL */
    double *dx, *ddt, *dB, *dC, *dinit, *dA_part, *dD_part;   /* part: [Bt*H] */
    int64_t Bt, T, H, P, N, G;
    int64_t next;
} bwd_job;

static void bwd_unit(const bwd_job *j, int64_t unit, double *S, double *gr)
{
    const int64_t b = unit / j->G, g = unit % j->G;
    const int64_t T = j->T, H = j->H, P = j->P, N = j->N, G = j->G, hpg = H / G;
    for (int64_t h = g * hpg; h < (g + 1) * hpg; ++h) {
        const int64_t bh = b * H + h;
        const double A = (double)j->A[h], D = (double)j->D[h];
        double dA = 0.0, dD = 0.0;
        for (int64_t p = 0; p < P; ++p) {
            /* forward: S[t] = state row after t tokens */
            for (int64_t n = 0; n < N; ++n)
                S[n] = j->init ? j->init[(bh * P + p) * N + n] : 0.0;
            for (int64_t t = 0; t < T; ++t) {
                const int64_t bt = b * T + t;
                const double dt = (double)j->dt[bt * H + h];
                const double a = exp(A * dt), u = dt * (double)j->x[(bt * H + h) * P + p];
                const float *Bv = j->B + (bt * G + g) * N;
                for (int64_t n = 0; n < N; ++n)
                    S[(t + 1) * N + n] = a * S[t * N + n] + u * (double)Bv[n];
            }
            /* backward */
            for (int64_t n = 0; n < N; ++n)
                gr[n] = j->dfin ? (double)j->dfin[(bh * P + p) * N + n] : 0.0;
            for (int64_t t = T - 1; t >= 0; --t) {
                const int64_t bt = b * T + t;
                const double dt = (double)j->dt[bt * H + h];
                const double a = exp(A * dt);
                const double xv = (double)j->x[(bt * H + h) * P + p];
                const double dyv = (double)j->dy[(bt * H + h) * P + p];
                const float *Bv = j->B + (bt * G + g) * N;
                const float *Cv = j->C + (bt * G + g) * N;
                double *dBt = j->dB + (bt * G + g) * N;
                double *dCt = j->dC + (bt * G + g) * N;
                double gB = 0.0, sh = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    gr[n] += dyv * (double)Cv[n];
                    dCt[n] += S[(t + 1) * N + n] * dyv;
                    gB += gr[n] * (double)Bv[n];
                    dBt[n] += dt * xv * gr[n];
                    sh += gr[n] * S[t * N + n];
                }
                j->dx[(bt * H + h) * P + p] = D * dyv + dt * gB;
                j->ddt[bt * H + h] += xv * gB + A * a * sh;
                dA += dt * a * sh;
                dD += dyv * xv;
                for (int64_t n = 0; n < N; ++n) gr[n] *= a;
            }
            if (j->dinit)
                for (int64_t n = 0; n < N; ++n) j->dinit[(bh * P + p) * N + n] = gr[n];
        }
        j->dA_part[bh] = dA;
        j->dD_part[bh] = dD;
    }
}

static void *bwd_worker(void *arg)
{
    bwd_job *j = (bwd_job *)arg;
    double *S = (double *)malloc(sizeof(double) * (size_t)((j->T + 1) * j->N));
    double *gr = (double *)malloc(sizeof(double) * (size_t)j->N);
    if (S && gr) {
        for (;;) {
            int64_t u = __atomic_fetch_add(&j->next, 1, __ATOMIC_RELAXED);
            if (u >= j->Bt * j->G) break;
            bwd_unit(j, u, S, gr);
        }
    }
    free(S);
    free(gr);
    return NULL;
}

/*
 * Gradients of L = sum(dy . y) + sum(dfin . final) for the plain forward.
 * Inputs as ssd_oracle_fwd plus dy [Bt,T,H,P] and dfin [Bt,H,P,N] (NULL = 0);
 * init [Bt*H,P,N] float64 or NULL.  Outputs (float64, all written): dx
 * [Bt,T,H,P], ddt [Bt,T,H], dB and dC [Bt,T,G,N], dA and dD [H], and dinit
 * [Bt,H,P,N] (may be NULL).  Returns the number of threads used, or a
 * negative value on a bad argument or allocation failure.
 */
int ssd_oracle_bwd(const float *x, const float *dt, const float *A, const float *B,
                   const float *C, const float *D, const double *init, const float *dy,
                   const float *dfin, int64_t Bt, int64_t T, int64_t H, int64_t P, int64_t N,
                   int64_t G, double *dx, double *ddt, double *dB, double *dC, double *dA,
                   double *dD, double *dinit, int nthreads)
{
    if (!x || !dt || !A || !B || !C || !D || !dy || !dx || !ddt || !dB || !dC || !dA || !dD)
        return -1;
    if (Bt < 1 || T < 0 || H < 1 || P < 1 || N < 1 || G < 1 || H % G) return -2;
    double *part = (double *)calloc((size_t)(2 * Bt * H), sizeof(double));
    if (!part) return -4;
    memset(ddt, 0, sizeof(double) * (size_t)(Bt * T * H));
    memset(dB, 0, sizeof(double) * (size_t)(Bt * T * G * N));
    memset(dC, 0, sizeof(double) * (size_t)(Bt * T * G * N));
    bwd_job j = {x, dt, A, B, C, D, dy, dfin, init, dx, ddt, dB, dC, dinit, part,
                 part + Bt * H, Bt, T, H, P, N, G, 0};
    if (nthreads <= 0) nthreads = ssd_oracle_host_threads();
    if (nthreads > Bt * G) nthreads = (int)(Bt * G);
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!th) {
        free(part);
        return -4;
    }
    int started = 0;
    for (int i = 1; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, bwd_worker, &j) != 0) break;
        ++started;
    }
    bwd_worker(&j);
    for (int i = 1; i <= started; ++i) pthread_join(th[i], NULL);
    free(th);
    for (int64_t h = 0; h < H; ++h) {
        double a = 0.0, d = 0.0;
        for (int64_t b = 0; b < Bt; ++b) {
            a += part[b * H + h];
            d += part[Bt * H + b * H + h];
        }
        dA[h] = a;
        dD[h] = d;
    }
    free(part);
    return started + 1;
}

