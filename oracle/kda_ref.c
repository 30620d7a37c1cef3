/*
 * Plain fp64 CPU oracle for the Kimi Delta Attention (KDA) forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously correct
 * definition that the GPU path is checked against.  Only the test suite,
 * the smoke check and the CPU-baseline leg of the benchmark may load it; the
 * GPU library never links, includes or calls anything here, and nothing here
 * comes from the GPU library.
 *
 * What it computes (token by token, no chunking, no reordering):
 *
 *   For every chain (sequence n, head h) and every token t of that sequence:
 *     x_t   = exp(A_log[h]) * (g_t + dt_bias[h, :])          K-vector
 *             (FlashKDA input-tensor page, "Gating Parameters and
 *              Constraints": A_log is applied per head, dt_bias is [H,K];
 *              lower_bound page, FAQ "How does lower_bound interact with
 *              dt_bias": the bias is added before the sigmoid)
 *     a_t   = lower_bound * sigmoid(x_t)                      natural-log decay
 *             (lower_bound page, "Conversion to the Gate Scale Factor":
 *              the bound scales the activated gate; the GPU carries the same
 *              value in log2 units, which does not change exp(a_t))
 *     beta_t = sigmoid(beta_logit_t)
 *             (input-tensor page, "Gating Tensors and Output Buffer")
 *     S <- diag(exp(a_t)) S                                   decay first
 *     S <- S + beta_t k_t (v_t - S^T k_t)^T                   delta write
 *     o_t = scale * S^T q_t                                   read after write
 *
 *   S is K x V and starts at initial_state[n,h]^T (stored [V,K], input-tensor
 *   page, "Initial and Final States") or zero; final_state[n,h] = S^T.
 *   Sequences are batch rows, or the segments [cu[n], cu[n+1]) of a packed
 *   batch of one row (input-tensor page, "Variable-Length Mode").
 *
 * All arithmetic is IEEE double.  bf16 inputs are widened exactly.  The
 * chains are independent, so threads take whole chains; each chain's result
 * does not depend on the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_STATE_NONE = 0, ORACLE_STATE_BF16 = 1, ORACLE_STATE_FP32 = 2 };

static double bf16_bits_to_double(uint16_t bits)
{
    uint32_t word = (uint32_t)bits << 16; /* bf16 is the top half of an fp32 */
    float f;
    memcpy(&f, &word, sizeof f);
    return (double)f;
}

/* Logistic function 1/(1+e^-x), written so that neither branch overflows. */
static double logistic(double x)
{
    if (x >= 0.0) {
        double e = exp(-x);
        return 1.0 / (1.0 + e);
    }
    double e = exp(x);
    return e / (1.0 + e);
}

typedef struct {
    const uint16_t *q, *k, *v, *g, *beta;
    double scale;
    const float *A_log;   /* [H] or NULL (then exp(A_log) is taken as 1) */
    const float *dt_bias; /* [H,K] or NULL (then the bias is 0) */
    double lower_bound;
    const void *init;     /* [N,H,V,K] or NULL */
    int init_dtype;
    const int64_t *cu;    /* [N+1] host int64, or NULL for batch mode */
    int64_t T, H, K, V;
    const int64_t *chains;      /* n_chains pairs (n, h) */
    const int64_t *out_offsets; /* first output row of each chain */
    int64_t n_chains;
    double *out;   /* [sum of chain lengths, V] */
    double *final; /* [n_chains, V, K] or NULL */
    int64_t next;  /* work counter, taken with an atomic add */
    int64_t done;  /* chains finished */
} oracle_job;

static void run_chain(const oracle_job *job, int64_t c, double *S, double *alpha,
                      double *pred)
{
    const int64_t n = job->chains[2 * c], h = job->chains[2 * c + 1];
    const int64_t H = job->H, K = job->K, V = job->V;
    int64_t t_begin, t_end, row0;
    if (job->cu) {
        t_begin = job->cu[n];
        t_end = job->cu[n + 1];
        row0 = 0;
    } else {
        t_begin = 0;
        t_end = job->T;
        row0 = n * job->T;
    }

    /* S[kk*V + vv] holds S[kk][vv]; the stored state is its transpose. */
    for (int64_t kk = 0; kk < K; ++kk)
        for (int64_t vv = 0; vv < V; ++vv) {
            double s = 0.0;
            if (job->init) {
                int64_t idx = ((n * H + h) * V + vv) * K + kk;
                if (job->init_dtype == ORACLE_STATE_BF16)
                    s = bf16_bits_to_double(((const uint16_t *)job->init)[idx]);
                else
                    s = (double)((const float *)job->init)[idx];
            }
            S[kk * V + vv] = s;
        }

    const double head_mult = job->A_log ? exp((double)job->A_log[h]) : 1.0;
    double *out_rows = job->out + job->out_offsets[c] * V;

    for (int64_t t = t_begin; t < t_end; ++t) {
        const int64_t tok = (row0 + t) * H + h; /* token index in [B*T, H] */
        const uint16_t *qt = job->q + tok * K;
        const uint16_t *kt = job->k + tok * K;
        const uint16_t *vt = job->v + tok * V;
        const uint16_t *gt = job->g + tok * K;

        for (int64_t kk = 0; kk < K; ++kk) {
            double bias = job->dt_bias ? (double)job->dt_bias[h * K + kk] : 0.0;
            double x = head_mult * (bf16_bits_to_double(gt[kk]) + bias);
            alpha[kk] = exp(job->lower_bound * logistic(x));
        }
        const double b = logistic(bf16_bits_to_double(job->beta[tok]));

        /* decay */
        for (int64_t kk = 0; kk < K; ++kk)
            for (int64_t vv = 0; vv < V; ++vv)
                S[kk * V + vv] *= alpha[kk];

        /* prediction S^T k with the decayed state, then the delta write */
        for (int64_t vv = 0; vv < V; ++vv) {
            double acc = 0.0;
            for (int64_t kk = 0; kk < K; ++kk)
                acc += S[kk * V + vv] * bf16_bits_to_double(kt[kk]);
            pred[vv] = acc;
        }
        for (int64_t kk = 0; kk < K; ++kk) {
            double bk = b * bf16_bits_to_double(kt[kk]);
            for (int64_t vv = 0; vv < V; ++vv)
                S[kk * V + vv] += bk * (bf16_bits_to_double(vt[vv]) - pred[vv]);
        }

        /* read-out with the updated state */
        double *o = out_rows + (t - t_begin) * V;
        for (int64_t vv = 0; vv < V; ++vv) {
            double acc = 0.0;
            for (int64_t kk = 0; kk < K; ++kk)
                acc += S[kk * V + vv] * bf16_bits_to_double(qt[kk]);
            o[vv] = job->scale * acc;
        }
    }

    if (job->final) {
        double *f = job->final + c * V * K;
        for (int64_t vv = 0; vv < V; ++vv)
            for (int64_t kk = 0; kk < K; ++kk)
                f[vv * K + kk] = S[kk * V + vv];
    }
}

static void *worker(void *arg)
{
    oracle_job *job = (oracle_job *)arg;
    double *S = malloc(sizeof(double) * (size_t)(job->K * job->V));
    double *alpha = malloc(sizeof(double) * (size_t)job->K);
    double *pred = malloc(sizeof(double) * (size_t)job->V);
    if (!S || !alpha || !pred) {
        free(S);
        free(alpha);
        free(pred);
        return (void *)1;
    }
    for (;;) {
        int64_t c = __atomic_fetch_add(&job->next, 1, __ATOMIC_RELAXED);
        if (c >= job->n_chains)
            break;
        run_chain(job, c, S, alpha, pred);
        __atomic_fetch_add(&job->done, 1, __ATOMIC_RELAXED);
    }
    free(S);
    free(alpha);
    free(pred);
    return NULL;
}

/*
 * Run the recurrence for the listed chains.
 *
 *   q, k, g     bf16 bit patterns, [B,T,H,K] (B = 1 when cu is given)
 *   v           bf16 bit patterns, [B,T,H,V]
 *   beta        bf16 bit patterns, [B,T,H] (logits)
 *   A_log       fp32 [H] or NULL;   dt_bias fp32 [H,K] or NULL
 *   init        [N,H,V,K] of init_dtype (1 = bf16 bits, 2 = fp32) or NULL
 *   cu          host int64 [N+1] or NULL
 *   chains      n_chains pairs (sequence n, head h)
 *   out_offsets first output row of each chain in `out`
 *   out         fp64 [total rows, V], rows of each chain contiguous
 *   final       fp64 [n_chains, V, K] or NULL
 *
 * Returns 0 when every listed chain was computed, non-zero otherwise (no
 * thread could start, or every thread failed to allocate its work arrays).
 */
int kda_oracle_chains(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                      const uint16_t *g, const uint16_t *beta, double scale,
                      const float *A_log, const float *dt_bias, double lower_bound,
                      const void *init, int init_dtype, const int64_t *cu,
                      int64_t T, int64_t H, int64_t K, int64_t V,
                      const int64_t *chains, const int64_t *out_offsets,
                      int64_t n_chains, double *out, double *final, int n_threads)
{
    oracle_job job = {q,        k,     v,     g,     beta,    scale, A_log, dt_bias,
                      lower_bound, init, init_dtype, cu, T, H, K, V, chains,
                      out_offsets, n_chains, out, final, 0, 0};
    if (init == NULL)
        job.init_dtype = ORACLE_STATE_NONE;
    if (n_threads < 1)
        n_threads = 1;
    if ((int64_t)n_threads > n_chains)
        n_threads = n_chains > 0 ? (int)n_chains : 1;

    pthread_t *tids = malloc(sizeof(pthread_t) * (size_t)n_threads);
    if (!tids)
        return 1;
    int started = 0;
    for (int i = 0; i < n_threads; ++i) {
        if (pthread_create(&tids[i], NULL, worker, &job) != 0)
            break;
        ++started;
    }
    for (int i = 0; i < started; ++i)
        pthread_join(tids[i], NULL);
    free(tids);
    return job.done == n_chains ? 0 : 1;
}
