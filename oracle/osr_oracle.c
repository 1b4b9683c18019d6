/*
 * osr_oracle.c -- fp64 CPU oracle for the Orthogonal State Recurrence (OSR).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the correctness reference that the
 * GPU path is compared against.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it.  It shares no code, header, table
 * or helper with the HIP library, and the HIP library never calls it.
 *
 * What it computes (source: "Lattice: Learning to Efficiently Compress the
 * Memory", Karami, Pascanu, Mirrokni, arXiv 2504.05646):
 *
 *   State S holds m slots s_1..s_m, each a vector in R^d (stored row-major,
 *   row = slot, as the implementation appendix lays out S as M x D).
 *
 *   The sequence is cut into chunks of C tokens (section "Parallel and
 *   Hardware Efficient Form").  At every chunk start each slot is projected
 *   onto the unit sphere (section "Stabilizing Memory Updates via
 *   Normalization": the feasible set is the unit sphere and the update is
 *   derived assuming unit slots).  The projected chunk-start state is S_{t'}.
 *   For each token t of the chunk, in the pages' notation:
 *
 *     h_t      = phi(S_{t'}) k_t - v_t   (decoding objective, e_t)
 *              = -v_t                    (similarity objective)
 *              = v_t                     (encoding layer)
 *                                         (eq. OSR and the table of (h_t, c_t)
 *                                          in the general-form appendix)
 *     h~_t     = S_{t'}^T h_t            (per slot: s_{t',i} . h_t)
 *     c_{t,i}  = k_{t,i}                 (decoding, similarity)
 *              = h~_{t,i} - k_{t,i}      (encoding layer: the per-slot error
 *                                         e_t = phi(S)^T v_t - k_t of
 *                                         eq. encoding_stateNorm_loss, the
 *                                         coefficient of eq. encoding_recurrence)
 *     |ds_i|^2 = (gamma_i c_i)^2 (|h_t|^2 - h~_{t,i}^2), clamped at 0
 *                                         (norm of the orthogonal update,
 *                                          appendix paragraph "Computing beta")
 *     beta_i   = (mu_t^2 + |ds_i|^2)^(-1/2)
 *                                         (eq. normalized_recurrence with the
 *                                          forget gate of eq. dacay_recurrence)
 *     k^_t     = gamma_t (.) beta_t (.) c_t          (eq. recurrence_detailed)
 *     G^_t     = mu_t beta_t + h~_t (.) k^_t         (eq. recurrence_linear2)
 *     s_{t,i}  = G^_{t,i} s_{t-1,i} - k^_{t,i} h_t   (eq. recurrence_linear2)
 *     y_t      = S_t q_t = sum_i q_{t,i} s_{t,i}     (memory read-out)
 *
 *   With C = 1 the chunk-start state is the current state, so each step is the
 *   exact normalised OSR step s_i <- (mu s_i - gamma_i c_i P(s_i) h)/|...|.
 *
 *   The pages derive two chunk linearisations.  The one above (the default,
 *   eq. recurrence_linear2) puts the projection term on the running slot.
 *   The first one (eq. recurrence_linear1) keeps only mu beta on the running
 *   slot and takes the projection term at the chunk-start slot z_i:
 *     s_{t,i}  = mu_t beta_i s_{t-1,i} + h~_{t,i} k^_{t,i} z_i - k^_{t,i} h_t
 *   (the same step when C = 1).
 *   The returned state is projected onto the unit sphere once more.
 *
 * Readings where the pages are silent or disagree (each is listed in the
 * design notes): gamma may be one value per token or one per token and slot;
 * the first term under the square root of beta is mu^2 (the chunk listing's
 * eta^2 is read as a typo); the norm term subtracts h~^2 (the appendix prints
 * a plus sign, the listing a minus with a clamp); no epsilon is added to slot
 * norms because every slot is projected to norm 1 first; the gradient carries
 * no factor 2; a slot of norm zero in the initial state is an error.
 *
 * Arithmetic is IEEE double throughout, no fast-math.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORACLE_OK 0
#define ORACLE_ERR_NULL (-1)
#define ORACLE_ERR_SHAPE (-2)
#define ORACLE_ERR_ZERO_SLOT (-6)
#define ORACLE_ERR_NOMEM (-7)

#define ORACLE_MODE_DEC 0
#define ORACLE_MODE_SIM 1
#define ORACLE_MODE_ENC 2

#define ORACLE_LIN2 0 /* eq. recurrence_linear2 (default) */
#define ORACLE_LIN1 1 /* eq. recurrence_linear1 */

typedef struct {
    int32_t B, T, H, m, d;
    int32_t gamma_per_slot; /* 1: gamma is [B,T,H,m]; 0: gamma is [B,T,H] */
    int32_t mode;           /* ORACLE_MODE_DEC, ORACLE_MODE_SIM or ORACLE_MODE_ENC */
    int32_t chunk_size;     /* C >= 1, T % C == 0 */
    int32_t linearisation;  /* ORACLE_LIN2 or ORACLE_LIN1 */
} oracle_osr_problem;

typedef struct {
    const oracle_osr_problem* p;
    const double *q, *k, *v, *gamma, *mu, *state_in;
    double *state_out, *y;
    int next;            /* next (b,h) index to take, guarded by lock */
    int status;          /* first error seen */
    pthread_mutex_t lock;
} oracle_job;

/* Project every slot (row) of S onto the unit sphere. */
static int project_slots(double* S, int m, int d) {
    for (int i = 0; i < m; ++i) {
        double sq = 0.0;
        for (int j = 0; j < d; ++j) sq += S[(size_t)i * d + j] * S[(size_t)i * d + j];
        if (!(sq > 0.0)) return ORACLE_ERR_ZERO_SLOT;
        double n = sqrt(sq);
        for (int j = 0; j < d; ++j) S[(size_t)i * d + j] /= n;
    }
    return ORACLE_OK;
}

/* Run the whole sequence of one (batch b, head hd) pair. */
static int run_sequence(const oracle_job* job, int b, int hd, double* work) {
    const oracle_osr_problem* p = job->p;
    const int T = p->T, H = p->H, m = p->m, d = p->d, C = p->chunk_size;
    double* S = work;                      /* running state S_t      m*d */
    double* Z = S + (size_t)m * d;         /* chunk-start state S_t' m*d */
    double* h = Z + (size_t)m * d;         /* h_t                     d  */
    double* htil = h + d;                  /* h~_t                    m  */
    double* khat = htil + m;               /* k^_t                    m  */
    double* Ghat = khat + m;               /* G^_t                    m  */

    memcpy(S, job->state_in + ((size_t)b * H + hd) * m * d, sizeof(double) * (size_t)m * d);

    for (int t0 = 0; t0 < T; t0 += C) {
        int rc = project_slots(S, m, d);
        if (rc != ORACLE_OK) return rc;
        memcpy(Z, S, sizeof(double) * (size_t)m * d);

        for (int t = t0; t < t0 + C; ++t) {
            const size_t bth = ((size_t)b * T + t) * H + hd;   /* [B,T,H] index */
            const double* kt = job->k + bth * m;
            const double* qt = job->q + bth * m;
            const double* vt = job->v + bth * d;
            const double* gt = job->gamma + (p->gamma_per_slot ? bth * m : bth);
            const double mu = job->mu[bth];
            double* yt = job->y + bth * d;

            /* h_t: the decoding error phi(S_t') k_t - v_t, -v_t, or v_t. */
            for (int j = 0; j < d; ++j) {
                double acc = 0.0;
                if (p->mode == ORACLE_MODE_DEC)
                    for (int i = 0; i < m; ++i) acc += kt[i] * Z[(size_t)i * d + j];
                h[j] = p->mode == ORACLE_MODE_ENC ? vt[j] : acc - vt[j];
            }
            double hsq = 0.0;
            for (int j = 0; j < d; ++j) hsq += h[j] * h[j];

            for (int i = 0; i < m; ++i) {
                double dot = 0.0;
                for (int j = 0; j < d; ++j) dot += Z[(size_t)i * d + j] * h[j];
                htil[i] = dot;
                const double g = p->gamma_per_slot ? gt[i] : gt[0];
                /* coefficient c_i: k_i, or the encoding error s_i . v - k_i */
                const double ci = p->mode == ORACLE_MODE_ENC ? dot - kt[i] : kt[i];
                const double wi = g * ci;                    /* writing intensity */
                double dsq = wi * wi * (hsq - dot * dot);    /* |ds_i|^2 */
                if (dsq < 0.0) dsq = 0.0;
                const double beta = 1.0 / sqrt(mu * mu + dsq);
                khat[i] = g * beta * ci;
                /* gate on the running slot: mu beta (eq. recurrence_linear1), or
                   mu beta plus the projection term (eq. recurrence_linear2) */
                Ghat[i] = p->linearisation == ORACLE_LIN1 ? mu * beta : mu * beta + htil[i] * khat[i];
            }

            if (p->linearisation == ORACLE_LIN1) {
                /* the projection term is taken at the chunk-start slot z_i */
                for (int i = 0; i < m; ++i)
                    for (int j = 0; j < d; ++j)
                        S[(size_t)i * d + j] = Ghat[i] * S[(size_t)i * d + j] + htil[i] * khat[i] * Z[(size_t)i * d + j]
                                               - khat[i] * h[j];
            } else {
                for (int i = 0; i < m; ++i)
                    for (int j = 0; j < d; ++j)
                        S[(size_t)i * d + j] = Ghat[i] * S[(size_t)i * d + j] - khat[i] * h[j];
            }

            for (int j = 0; j < d; ++j) {
                double acc = 0.0;
                for (int i = 0; i < m; ++i) acc += qt[i] * S[(size_t)i * d + j];
                yt[j] = acc;
            }
        }
    }
    int rc = project_slots(S, m, d);
    if (rc != ORACLE_OK) return rc;
    memcpy(job->state_out + ((size_t)b * H + hd) * m * d, S, sizeof(double) * (size_t)m * d);
    return ORACLE_OK;
}

static void* worker(void* arg) {
    oracle_job* job = (oracle_job*)arg;
    const oracle_osr_problem* p = job->p;
    const size_t wsz = 2 * (size_t)p->m * p->d + p->d + 3 * (size_t)p->m;
    double* work = (double*)malloc(sizeof(double) * wsz);
    if (!work) {
        pthread_mutex_lock(&job->lock);
        if (job->status == ORACLE_OK) job->status = ORACLE_ERR_NOMEM;
        pthread_mutex_unlock(&job->lock);
        return NULL;
    }
    for (;;) {
        pthread_mutex_lock(&job->lock);
        int idx = job->next++;
        int stop = job->status != ORACLE_OK;
        pthread_mutex_unlock(&job->lock);
        if (stop || idx >= p->B * p->H) break;
        int rc = run_sequence(job, idx / p->H, idx % p->H, work);
        if (rc != ORACLE_OK) {
            pthread_mutex_lock(&job->lock);
            if (job->status == ORACLE_OK) job->status = rc;
            pthread_mutex_unlock(&job->lock);
        }
    }
    free(work);
    return NULL;
}

int oracle_osr_hardware_threads(void) {
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}

/*
 * Forward pass over all (b,h) pairs.  Layouts (all contiguous, double):
 *   q, k, gamma  [B,T,H,m]   (gamma [B,T,H] when gamma_per_slot == 0)
 *   v, y         [B,T,H,d]
 *   mu           [B,T,H]
 *   state_in/out [B,H,m,d]   row = slot
 * nthreads <= 0 uses every online CPU.  Returns the number of threads used
 * through *threads_used (may be NULL).  Returns 0 or a negative status.
 */
int oracle_osr_forward(const oracle_osr_problem* p, const double* q, const double* k,
                       const double* v, const double* gamma, const double* mu,
                       const double* state_in, double* state_out, double* y,
                       int nthreads, int* threads_used) {
    if (!p || !q || !k || !v || !gamma || !mu || !state_in || !state_out || !y)
        return ORACLE_ERR_NULL;
    if (p->B <= 0 || p->T <= 0 || p->H <= 0 || p->m <= 0 || p->d <= 0 || p->chunk_size <= 0 ||
        p->T % p->chunk_size != 0 ||
        (p->mode != ORACLE_MODE_DEC && p->mode != ORACLE_MODE_SIM && p->mode != ORACLE_MODE_ENC) ||
        (p->linearisation != ORACLE_LIN2 && p->linearisation != ORACLE_LIN1))
        return ORACLE_ERR_SHAPE;

    oracle_job job;
    job.p = p;
    job.q = q; job.k = k; job.v = v; job.gamma = gamma; job.mu = mu;
    job.state_in = state_in; job.state_out = state_out; job.y = y;
    job.next = 0;
    job.status = ORACLE_OK;
    pthread_mutex_init(&job.lock, NULL);

    int n = nthreads > 0 ? nthreads : oracle_osr_hardware_threads();
    if (n > p->B * p->H) n = p->B * p->H;
    if (threads_used) *threads_used = n;

    if (n == 1) {
        worker(&job);
    } else {
        pthread_t* tids = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)n);
        if (!tids) { pthread_mutex_destroy(&job.lock); return ORACLE_ERR_NOMEM; }
        int started = 0;
        for (; started < n; ++started)
            if (pthread_create(&tids[started], NULL, worker, &job) != 0) break;
        if (started == 0) worker(&job);
        for (int i = 0; i < started; ++i) pthread_join(tids[i], NULL);
        free(tids);
    }
    pthread_mutex_destroy(&job.lock);
    return job.status;
}
