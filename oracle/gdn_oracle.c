/*
 * gdn_oracle.c -- plain fp64 CPU reference for the Gated DeltaNet token mixer.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the oracle that the GPU library is checked
 * against. Only the tests, the smoke check and the benchmark's CPU-baseline leg may load
 * it. It shares no source, header or build step with the HIP library.
 *
 * What it computes (sources: the pages on Qwen3-Next):
 *
 *  - The gated delta rule, one token at a time. Page "Qwen3-Next -- How a running memory
 *    and a searchable history cooperate", section "Correcting a memory instead of adding
 *    to it": the old state is first shrunk by the decay alpha, then corrected toward the
 *    target with write strength beta along the current key. For a matrix state S
 *    (d_v x d_k), key k, value v:
 *        S_t = alpha_t * S_{t-1} * (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *    which equals alpha*S + beta*(v - alpha*S k) k^T (the form coded below).
 *  - The read-out o_t = scale * S_t q_t, taken after the update, as in the token loop of
 *    page "Qwen3-Next 80B-A3B -- The Evolving Transformer", section
 *    "01 . GatedDeltaNet(config)".
 *  - Head sharing: 16 QK heads serve 32 V heads (model card "Qwen3-Next", section "Model
 *    Overview"); V head h reads QK head h / (h_v / h_qk), the repeat-interleave convention
 *    of the GQA code in section "02 . GatedAttention(config)" of the Evolving Transformer
 *    page.
 *  - The per-channel form of the code panel in section "01 . GatedDeltaNet(config)" of the
 *    Evolving Transformer page: one decay per value channel, and the correction measured
 *    against the state before the decay:
 *        S_t = diag(alpha_t) S_{t-1} + beta_t (v_t - S_{t-1} k_t) k_t^T
 *    (alpha_t a vector of d_v decays; o_t = scale * S_t q_t as above).
 *  - The front end: a short causal depthwise convolution over the projected q|k|v
 *    channels, SiLU, L2 normalisation of each q and k head and a scale on q (the
 *    GatedDeltaNet section names a short 1-D convolution for local context and normalises
 *    the keys; kernel size, channels and the q normalisation follow the layer shape of
 *    the workload).
 *  - The epilogue after the mixer: an RMS norm over each V head's d_v read-out channels
 *    with the zero-centred scale (1 + w_i) (page "Qwen3-Next 80B-A3B", the architecture
 *    knowledge-base page, table "Architecture", row "Norm type": zero-centred RMSNorm),
 *    then an elementwise output gate from a second projection z (the GatedDeltaNet section
 *    of the Evolving Transformer page: a gate decides how much of the recurrent read-out
 *    reaches the output). The pages give no formula: the norm is taken over one head at a
 *    time, the gate is applied after the norm, and the gate function is sigmoid (a
 *    fraction between 0 and 1) or, on request, SiLU.
 *
 * Plain loops, fp64, no blocking or reordering beyond the definitions above. Threads only
 * split independent (sequence, V head) chains or tokens.
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -pthread gdn_oracle.c -o libgdn_oracle.so -lm
 * (no fast-math: the point is a result that can be trusted).
 */
#include <math.h>
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------------------ */
/* One chain: one sequence, one V head.                                                  */
/* ------------------------------------------------------------------------------------ */

/*
 * Runs the token loop for T tokens of one (sequence, V head) chain.
 *   q, k     : token t at q + t*qk_stride, d_k entries each
 *   v        : token t at v + t*v_stride, d_v entries each
 *   g, beta  : token t at g[t*gb_stride], beta[t*gb_stride]; alpha_t = exp(g_t)
 *   S        : d_v x d_k row-major, in: state before the first token, out: after the last
 *   o        : token t at o + t*o_stride, d_v entries (may be NULL)
 *   traj     : NULL, or T * d_v * d_k doubles receiving the state after each token
 *   u        : scratch of d_v doubles
 */
void gdn_ref_chain(int T, int d_k, int d_v,
                   const double* q, ptrdiff_t qk_stride_q,
                   const double* k, ptrdiff_t qk_stride_k,
                   const double* v, ptrdiff_t v_stride,
                   const double* g, const double* beta, ptrdiff_t gb_stride,
                   double scale, double* S, double* o, ptrdiff_t o_stride,
                   double* traj, double* u)
{
    for (int t = 0; t < T; ++t) {
        const double* qt = q + (ptrdiff_t)t * qk_stride_q;
        const double* kt = k + (ptrdiff_t)t * qk_stride_k;
        const double* vt = v + (ptrdiff_t)t * v_stride;
        const double a = exp(g[(ptrdiff_t)t * gb_stride]);
        const double b = beta[(ptrdiff_t)t * gb_stride];

        /* u = S k : what the state currently returns for this key */
        for (int i = 0; i < d_v; ++i) {
            double s = 0.0;
            for (int j = 0; j < d_k; ++j) s += S[(ptrdiff_t)i * d_k + j] * kt[j];
            u[i] = s;
        }
        /* S <- a*S + b*(v - a*u) k^T : decay first, then correct the decayed memory */
        for (int i = 0; i < d_v; ++i) {
            const double c = b * (vt[i] - a * u[i]);
            for (int j = 0; j < d_k; ++j)
                S[(ptrdiff_t)i * d_k + j] = a * S[(ptrdiff_t)i * d_k + j] + c * kt[j];
        }
        /* o = scale * S q, read after the update */
        if (o) {
            double* ot = o + (ptrdiff_t)t * o_stride;
            for (int i = 0; i < d_v; ++i) {
                double s = 0.0;
                for (int j = 0; j < d_k; ++j) s += S[(ptrdiff_t)i * d_k + j] * qt[j];
                ot[i] = scale * s;
            }
        }
        if (traj) memcpy(traj + (ptrdiff_t)t * d_v * d_k, S, sizeof(double) * (size_t)d_v * d_k);
    }
}

/*
 * The per-channel form for T tokens of one chain: as gdn_ref_chain, with g holding d_v
 * log-decays per token (token t at g + t*g_stride, one per value channel i) and the
 * correction taken from the state before the decay.
 */
void gdn_ref_chain_channel(int T, int d_k, int d_v,
                           const double* q, ptrdiff_t qk_stride_q,
                           const double* k, ptrdiff_t qk_stride_k,
                           const double* v, ptrdiff_t v_stride,
                           const double* g, ptrdiff_t g_stride,
                           const double* beta, ptrdiff_t b_stride,
                           double scale, double* S, double* o, ptrdiff_t o_stride,
                           double* traj, double* u)
{
    for (int t = 0; t < T; ++t) {
        const double* qt = q + (ptrdiff_t)t * qk_stride_q;
        const double* kt = k + (ptrdiff_t)t * qk_stride_k;
        const double* vt = v + (ptrdiff_t)t * v_stride;
        const double* gt = g + (ptrdiff_t)t * g_stride;
        const double b = beta[(ptrdiff_t)t * b_stride];

        /* u = S k, from the state before this token's decay */
        for (int i = 0; i < d_v; ++i) {
            const double* Si = S + (ptrdiff_t)i * d_k;
            double acc = 0.0;
            for (int j = 0; j < d_k; ++j) acc += Si[j] * kt[j];
            u[i] = acc;
        }
        /* row i: S_i <- alpha_i S_i + b (v_i - u_i) k^T */
        for (int i = 0; i < d_v; ++i) {
            double* Si = S + (ptrdiff_t)i * d_k;
            const double ai = exp(gt[i]);
            const double ci = b * (vt[i] - u[i]);
            for (int j = 0; j < d_k; ++j) Si[j] = ai * Si[j] + ci * kt[j];
        }
        /* read-out after the update */
        if (o) {
            double* ot = o + (ptrdiff_t)t * o_stride;
            for (int i = 0; i < d_v; ++i) {
                const double* Si = S + (ptrdiff_t)i * d_k;
                double acc = 0.0;
                for (int j = 0; j < d_k; ++j) acc += Si[j] * qt[j];
                ot[i] = scale * acc;
            }
        }
        if (traj) memcpy(traj + (ptrdiff_t)t * d_v * d_k, S, sizeof(double) * (size_t)d_v * d_k);
    }
}

/* ------------------------------------------------------------------------------------ */
/* Packed variable-length batch.                                                         */
/* ------------------------------------------------------------------------------------ */

typedef struct {
    const double *q, *k, *v, *g, *beta;
    const int64_t* cu;
    int num_seqs, h_qk, h_v, d_k, d_v;
    double scale;
    const double* s0;
    double* s_final;
    double* o;
    double* traj;
    int channel;            /* 1: per-channel form, g is [T][h_v][d_v] */
    int next;               /* next chain index, taken under the lock */
    pthread_mutex_t lock;
} batch_job;

static void run_chain(batch_job* J, int chain, double* S, double* u)
{
    const int n = chain / J->h_v, h = chain % J->h_v;
    const int j = h / (J->h_v / J->h_qk);
    const int64_t t0 = J->cu[n], T = J->cu[n + 1] - J->cu[n];
    const size_t sz = (size_t)J->d_v * J->d_k;
    if (J->s0) memcpy(S, J->s0 + ((size_t)n * J->h_v + h) * sz, sizeof(double) * sz);
    else memset(S, 0, sizeof(double) * sz);
    const ptrdiff_t qk_stride = (ptrdiff_t)J->h_qk * J->d_k;
    const ptrdiff_t v_stride = (ptrdiff_t)J->h_v * J->d_v;
    /* trajectory layout [h_v][T_total][d_v][d_k]: the chain's states are consecutive */
    double* traj = J->traj ? J->traj + ((size_t)h * J->cu[J->num_seqs] + (size_t)t0) * sz : NULL;
    if (J->channel)
        gdn_ref_chain_channel((int)T, J->d_k, J->d_v,
                              J->q + t0 * qk_stride + (ptrdiff_t)j * J->d_k, qk_stride,
                              J->k + t0 * qk_stride + (ptrdiff_t)j * J->d_k, qk_stride,
                              J->v + t0 * v_stride + (ptrdiff_t)h * J->d_v, v_stride,
                              J->g + t0 * v_stride + (ptrdiff_t)h * J->d_v, v_stride,
                              J->beta + t0 * J->h_v + h, J->h_v,
                              J->scale, S,
                              J->o ? J->o + t0 * v_stride + (ptrdiff_t)h * J->d_v : NULL, v_stride,
                              traj, u);
    else
        gdn_ref_chain((int)T, J->d_k, J->d_v,
                      J->q + t0 * qk_stride + (ptrdiff_t)j * J->d_k, qk_stride,
                      J->k + t0 * qk_stride + (ptrdiff_t)j * J->d_k, qk_stride,
                      J->v + t0 * v_stride + (ptrdiff_t)h * J->d_v, v_stride,
                      J->g + t0 * J->h_v + h, J->beta + t0 * J->h_v + h, J->h_v,
                      J->scale, S,
                      J->o ? J->o + t0 * v_stride + (ptrdiff_t)h * J->d_v : NULL, v_stride,
                      traj, u);
    if (J->s_final) memcpy(J->s_final + ((size_t)n * J->h_v + h) * sz, S, sizeof(double) * sz);
}

static void* batch_worker(void* arg)
{
    batch_job* J = (batch_job*)arg;
    const size_t sz = (size_t)J->d_v * J->d_k;
    double* S = (double*)malloc(sizeof(double) * sz);
    double* u = (double*)malloc(sizeof(double) * (size_t)J->d_v);
    const int n_chains = J->num_seqs * J->h_v;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        const int c = J->next++;
        pthread_mutex_unlock(&J->lock);
        if (c >= n_chains) break;
        run_chain(J, c, S, u);
    }
    free(S);
    free(u);
    return NULL;
}

/*
 * Gated delta rule over a packed batch (gdn_ref_recurrence below; the shared driver).
 *   q, k  [T][h_qk][d_k];  v [T][h_v][d_v];  g, beta [T][h_v];  cu_seqlens [N+1]
 *   initial_state [N][h_v][d_v][d_k] or NULL (zeros); final_state same shape or NULL
 *   o [T][h_v][d_v] or NULL
 *   traj: NULL, or [h_v][T][d_v][d_k] receiving the state after every token (small cases)
 * Returns 0, or -1 on a bad argument.
 */
static int run_batch(const double* q, const double* k, const double* v,
                     const double* g, const double* beta,
                     const int64_t* cu_seqlens, int num_seqs,
                     int h_qk, int h_v, int d_k, int d_v, double scale,
                     const double* initial_state, double* final_state,
                     double* o, double* traj, int n_threads, int channel)
{
    if (num_seqs < 0 || h_qk <= 0 || h_v <= 0 || d_k <= 0 || d_v <= 0) return -1;
    if (h_v % h_qk != 0) return -1;
    if (num_seqs == 0) return 0;
    batch_job J;
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.cu = cu_seqlens;
    J.num_seqs = num_seqs; J.h_qk = h_qk; J.h_v = h_v; J.d_k = d_k; J.d_v = d_v;
    J.scale = scale; J.s0 = initial_state; J.s_final = final_state; J.o = o; J.traj = traj;
    J.channel = channel;
    J.next = 0;
    pthread_mutex_init(&J.lock, NULL);
    if (n_threads < 1) n_threads = 1;
    if (n_threads > num_seqs * h_v) n_threads = num_seqs * h_v;
    if (n_threads == 1) {
        batch_worker(&J);
    } else {
        pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)n_threads);
        for (int i = 0; i < n_threads; ++i) pthread_create(&th[i], NULL, batch_worker, &J);
        for (int i = 0; i < n_threads; ++i) pthread_join(th[i], NULL);
        free(th);
    }
    pthread_mutex_destroy(&J.lock);
    return 0;
}

int gdn_ref_recurrence(const double* q, const double* k, const double* v,
                       const double* g, const double* beta,
                       const int64_t* cu_seqlens, int num_seqs,
                       int h_qk, int h_v, int d_k, int d_v, double scale,
                       const double* initial_state, double* final_state,
                       double* o, double* traj, int n_threads)
{
    return run_batch(q, k, v, g, beta, cu_seqlens, num_seqs, h_qk, h_v, d_k, d_v, scale,
                     initial_state, final_state, o, traj, n_threads, 0);
}

/*
 * The per-channel form over a packed batch: as gdn_ref_recurrence, with g [T][h_v][d_v]
 * (one log-decay per value channel) and beta [T][h_v].
 */
int gdn_ref_recurrence_channel(const double* q, const double* k, const double* v,
                               const double* g, const double* beta,
                               const int64_t* cu_seqlens, int num_seqs,
                               int h_qk, int h_v, int d_k, int d_v, double scale,
                               const double* initial_state, double* final_state,
                               double* o, double* traj, int n_threads)
{
    return run_batch(q, k, v, g, beta, cu_seqlens, num_seqs, h_qk, h_v, d_k, d_v, scale,
                     initial_state, final_state, o, traj, n_threads, 1);
}

/* ------------------------------------------------------------------------------------ */
/* Front end: causal depthwise conv, SiLU, per-head L2 norm of q and k, scale on q.      */
/* ------------------------------------------------------------------------------------ */

typedef struct {
    const double* x;        /* [T][C] */
    const double* w;        /* [C][K], tap K-1 multiplies the current token */
    int K;
    const int64_t* cu;
    int num_seqs, h_qk, h_v, d_k, d_v;
    double q_scale, eps;
    double *q, *k, *v;      /* [T][h_qk][d_k], [T][h_qk][d_k], [T][h_v][d_v] */
    int n_threads, tid;
} fe_job;

static void fe_token(const fe_job* J, int64_t t, int64_t start, double* z)
{
    const int C = 2 * J->h_qk * J->d_k + J->h_v * J->d_v;
    for (int c = 0; c < C; ++c) {
        double y = 0.0;
        for (int i = 0; i < J->K; ++i) {
            const int64_t src = t - (J->K - 1) + i;      /* zero history before the start */
            if (src >= start) y += J->w[(ptrdiff_t)c * J->K + i] * J->x[src * C + c];
        }
        z[c] = y / (1.0 + exp(-y));                     /* SiLU */
    }
    const int nq = J->h_qk * J->d_k;
    for (int hh = 0; hh < J->h_qk; ++hh) {
        for (int part = 0; part < 2; ++part) {          /* 0: q head, 1: k head */
            const double* zz = z + part * nq + (ptrdiff_t)hh * J->d_k;
            double ss = 0.0;
            for (int e = 0; e < J->d_k; ++e) ss += zz[e] * zz[e];
            double nrm = sqrt(ss);
            if (nrm < J->eps) nrm = J->eps;
            double* out = (part == 0 ? J->q : J->k) + (t * J->h_qk + hh) * (ptrdiff_t)J->d_k;
            const double f = (part == 0 ? J->q_scale : 1.0) / nrm;
            for (int e = 0; e < J->d_k; ++e) out[e] = zz[e] * f;
        }
    }
    const int nv = J->h_v * J->d_v;
    for (int e = 0; e < nv; ++e) J->v[t * (ptrdiff_t)nv + e] = z[2 * nq + e];
}

static void* fe_worker(void* arg)
{
    const fe_job* J = (const fe_job*)arg;
    const int C = 2 * J->h_qk * J->d_k + J->h_v * J->d_v;
    double* z = (double*)malloc(sizeof(double) * (size_t)C);
    int64_t idx = 0;
    for (int n = 0; n < J->num_seqs; ++n)
        for (int64_t t = J->cu[n]; t < J->cu[n + 1]; ++t, ++idx)
            if (idx % J->n_threads == J->tid) fe_token(J, t, J->cu[n], z);
    free(z);
    return NULL;
}

int gdn_ref_conv_prep(const double* mixed, const double* conv_weight, int conv_kernel,
                      const int64_t* cu_seqlens, int num_seqs,
                      int h_qk, int h_v, int d_k, int d_v, double q_scale, double eps,
                      double* q, double* k, double* v, int n_threads)
{
    if (conv_kernel <= 0 || num_seqs < 0 || h_qk <= 0 || h_v <= 0 || d_k <= 0 || d_v <= 0) return -1;
    if (n_threads < 1) n_threads = 1;
    fe_job* jobs = (fe_job*)malloc(sizeof(fe_job) * (size_t)n_threads);
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)n_threads);
    for (int i = 0; i < n_threads; ++i) {
        fe_job J = {mixed, conv_weight, conv_kernel, cu_seqlens, num_seqs, h_qk, h_v, d_k, d_v,
                    q_scale, eps, q, k, v, n_threads, i};
        jobs[i] = J;
    }
    if (n_threads == 1) fe_worker(&jobs[0]);
    else {
        for (int i = 0; i < n_threads; ++i) pthread_create(&th[i], NULL, fe_worker, &jobs[i]);
        for (int i = 0; i < n_threads; ++i) pthread_join(th[i], NULL);
    }
    free(th);
    free(jobs);
    return 0;
}


/* ------------------------------------------------------------------------------------ */
/* Output epilogue: per-head RMS norm with zero-centred scale, then the output gate.     */
/* ------------------------------------------------------------------------------------ */

/*
 * For each of rows * h_v vectors x = o[r][h][0 .. d_v-1] (and the gate input z at the same
 * place):
 *     ms    = (1/d_v) * sum_i x_i^2
 *     y_i   = x_i / sqrt(ms + eps) * (1 + weight[i])
 *     out_i = y_i * sigmoid(z_i)          (gate == 0)
 *     out_i = y_i * z_i * sigmoid(z_i)    (gate == 1, SiLU)
 * weight has d_v entries, shared by all heads. Returns 0, or -1 for an unknown gate.
 */
int gdn_ref_gated_rmsnorm(const double* o, const double* z, const double* weight,
                          int64_t rows, int h_v, int d_v, double eps, int gate, double* out)
{
    if (gate != 0 && gate != 1) return -1;
    for (int64_t r = 0; r < rows; ++r) {
        for (int h = 0; h < h_v; ++h) {
            const size_t base = ((size_t)r * h_v + h) * d_v;
            double ms = 0.0;
            for (int i = 0; i < d_v; ++i) ms += o[base + i] * o[base + i];
            ms /= d_v;
            const double inv_rms = 1.0 / sqrt(ms + eps);
            for (int i = 0; i < d_v; ++i) {
                const double y = o[base + i] * inv_rms * (1.0 + weight[i]);
                const double zi = z[base + i];
                const double sig = 1.0 / (1.0 + exp(-zi));
                out[base + i] = y * (gate == 0 ? sig : zi * sig);
            }
        }
    }
    return 0;
}
