/*
 * ssd_oracle.c -- plain, slow, fp64 CPU oracle for the scalar-decay multi-head
 * SSM forward pass (Mamba-2 "SSD").
 *
 * TEST INFRASTRUCTURE ONLY.  This library exists to check the GPU path.  Only
 * the test suite, the package smoke check and the CPU-baseline leg of the
 * benchmark load it.  It shares no code, header, table or helper with the HIP
 * library, and the HIP library never calls it.
 *
 * It computes the literal per-timestep recurrence, with no chunking, no
 * blocking and no reordering beyond what the definition states:
 *
 *   Delta_t = softplus(dt_t)             (or dt_t itself when softplus is off)
 *   a_t     = exp(Delta_t * A_h)
 *   h_t     = a_t * h_{t-1} + Delta_t * B_t * x_t^T     (state, stored [P][N])
 *   y_t     = C_t^T h_t + D_h * x_t
 *
 * Sources (the pages' text):
 *   - recurrence and output with a scalar decay a_t:
 *       "Mamba 2 -- Transformers are SSMs" paper story (ai.tomabc.com),
 *       section 3.1 (scalar-A simplification);
 *   - one independent state and decay per head:
 *       same page, section 5.1 (multi-head architecture);
 *   - a_t = exp(Delta_t A) (zero-order-hold decay):
 *       "SSM 家族全景图（下）：Mamba-2 与 Jamba" (scwacadex), closing question
 *       on state decay; and the Transformer->Mamba page (answer.freetools.me),
 *       "连续到离散：零阶保持";
 *   - the D skip term y = C h + D x:
 *       answer.freetools.me page, continuous SSM equations;
 *   - packed sequences: setting A_t = 0 at a sequence boundary stops the state
 *       crossing it: "Transformers与SSMs的隐藏联系" (jsqmd.com), section 4.2.
 *
 * Readings taken where the pages are silent:
 *   - softplus(z) = log(1 + e^z), evaluated as max(z,0) + log1p(exp(-|z|));
 *   - the initial state is h_{-1}, so it is decayed by a_0 at t = 0;
 *   - head h uses B/C group g = floor(h * G / H) (H divisible by G);
 *   - a boundary is a position t > 0 with seq_idx[t] != seq_idx[t-1]; there the
 *     carried state is *replaced* by zero (a select, not a multiply by 0), so a
 *     NaN or Inf can never cross it.  t = 0 is never a boundary, so the initial
 *     state flows into the first segment only.
 *
 * Parallelism: OpenMP over independent (batch, head, state-row p) units.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int64_t batch, seqlen, nheads, headdim, dstate, ngroups; /* b, T, H, P, N, G */
    int32_t dt_softplus;              /* 1: Delta = softplus(dt); 0: Delta = dt */
    const double *x;                  /* [b,T,H,P] */
    const double *dt;                 /* [b,T,H] */
    const double *A;                  /* [H] */
    const double *B;                  /* [b,T,G,N] */
    const double *C;                  /* [b,T,G,N] */
    const double *D;                  /* [H] or NULL (no skip term) */
    const double *initial_states;     /* [b,H,P,N] or NULL (zeros) */
    const int32_t *seq_idx;           /* [T] or NULL; requires batch == 1 */
    int64_t nseq;                     /* number of segment ids when seq_idx != NULL */
    const uint8_t *unit_mask;         /* [b*H] or NULL: compute only (b,h) with mask != 0 */
    int64_t chunk;                    /* > 0: chunk length used by the two options below */
    int32_t chunk_local;              /* 1: the state restarts from zero at each chunk start */
    double *y;                        /* [b,T,H,P] out (rows of skipped units untouched) */
    double *final_states;             /* [b,H,P,N], or [nseq,H,P,N] with seq_idx; NULL to skip */
    double *chunk_end_states;         /* [b,nc,H,P,N] state after each chunk's last token; NULL to skip */
} ssd_oracle_args;

enum { ORACLE_OK = 0, ORACLE_BAD_ARGS = -1, ORACLE_NO_MEMORY = -2 };

static double softplus(double z)
{
    /* log(1 + e^z) without overflow for large |z| */
    return (z > 0.0 ? z : 0.0) + log1p(exp(-fabs(z)));
}

int ssd_oracle_abi_version(void) { return 1; }

int ssd_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* The forward recurrence.  See the file header for the definition. */
int ssd_oracle_forward(const ssd_oracle_args *a)
{
    if (!a || !a->x || !a->dt || !a->A || !a->B || !a->C || !a->y) return ORACLE_BAD_ARGS;
    const int64_t Bt = a->batch, T = a->seqlen, H = a->nheads, P = a->headdim;
    const int64_t N = a->dstate, G = a->ngroups;
    if (Bt < 1 || T < 1 || H < 1 || P < 1 || N < 1 || G < 1 || H % G != 0) return ORACLE_BAD_ARGS;
    if (a->seq_idx && (Bt != 1 || a->nseq < 1)) return ORACLE_BAD_ARGS;
    if ((a->chunk_local || a->chunk_end_states) && a->chunk < 1) return ORACLE_BAD_ARGS;
    const int64_t Q = a->chunk > 0 ? a->chunk : T;
    const int64_t nc = (T + Q - 1) / Q;
    const int64_t units = Bt * H * P;
    int status = ORACLE_OK;

#pragma omp parallel
    {
        double *hrow = (double *)malloc((size_t)N * sizeof(double));
        if (!hrow) {
#pragma omp atomic write
            status = ORACLE_NO_MEMORY;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t u = 0; u < units; ++u) {
            if (!hrow) continue;
            const int64_t p = u % P;
            const int64_t h = (u / P) % H;
            const int64_t b = u / (P * H);
            if (a->unit_mask && !a->unit_mask[b * H + h]) continue;
            const int64_t g = h * G / H;
            const double Ah = a->A[h];
            const double Dh = a->D ? a->D[h] : 0.0;

            /* h_{-1}: the initial state row (or zero) */
            for (int64_t n = 0; n < N; ++n)
                hrow[n] = a->initial_states ? a->initial_states[((b * H + h) * P + p) * N + n] : 0.0;

            for (int64_t t = 0; t < T; ++t) {
                const int64_t bt = b * T + t;
                const double z = a->dt[bt * H + h];
                const double delta = a->dt_softplus ? softplus(z) : z;
                const double decay = exp(delta * Ah);
                const double xv = a->x[(bt * H + h) * P + p];
                const double *Bv = a->B + (bt * G + g) * N;
                const double *Cv = a->C + (bt * G + g) * N;

                /* carry: replaced by zero at a packed-sequence boundary, and at a
                 * chunk start in chunk-local mode */
                int keep = 1;
                if (a->seq_idx && t > 0 && a->seq_idx[t] != a->seq_idx[t - 1]) keep = 0;
                if (a->chunk_local && t % Q == 0) keep = 0;

                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    const double carried = keep ? decay * hrow[n] : 0.0;
                    hrow[n] = carried + delta * Bv[n] * xv;
                    acc += Cv[n] * hrow[n];
                }
                a->y[(bt * H + h) * P + p] = acc + Dh * xv;

                if (a->chunk_end_states && (t % Q == Q - 1 || t == T - 1)) {
                    double *dst = a->chunk_end_states + (((b * nc + t / Q) * H + h) * P + p) * N;
                    memcpy(dst, hrow, (size_t)N * sizeof(double));
                }
                if (a->final_states && a->seq_idx) {
                    if (t == T - 1 || a->seq_idx[t + 1] != a->seq_idx[t]) {
                        const int64_t s = a->seq_idx[t];
                        if (s >= 0 && s < a->nseq)
                            memcpy(a->final_states + ((s * H + h) * P + p) * N, hrow,
                                   (size_t)N * sizeof(double));
                    }
                }
            }
            if (a->final_states && !a->seq_idx)
                memcpy(a->final_states + ((b * H + h) * P + p) * N, hrow, (size_t)N * sizeof(double));
        }
        free(hrow);
    }
    return status;
}

/*
 * Per-token step size and within-chunk cumulative log-decay.
 *
 *   Delta_t = softplus(dt_t) (or dt_t);  l_t = Delta_t * A_h = log a_t;
 *   cs[c][i] = sum_{k=cQ}^{cQ+i} l_k        (inclusive, restarting every chunk)
 *
 * so exp(cs_t - cs_s) = a_{s+1} ... a_t is the decay mask entry between two
 * tokens of one chunk ("Mamba 2 -- Transformers are SSMs" paper story,
 * section 3.2, the mask L as a product of a's).  With packed sequences the sum
 * also restarts at every segment boundary inside a chunk, so cs_t is the log of
 * the decay from the later of the chunk start and t's segment start through t;
 * the decay across a boundary is zero and is never formed from cs.  Positions
 * past the end of the sequence (t >= T in the last chunk) get Delta = 0 and
 * l = 0, so cs keeps its last value there.  Outputs are laid out [b][H][nc][Q].
 */
int ssd_oracle_chunk_cumsum(int64_t batch, int64_t T, int64_t H, int64_t Q, int32_t dt_softplus,
                            const double *dt, const double *A, const int32_t *seq_idx,
                            double *delta_out, double *cs_out)
{
    if (batch < 1 || T < 1 || H < 1 || Q < 1 || !dt || !A || !delta_out || !cs_out) return ORACLE_BAD_ARGS;
    if (seq_idx && batch != 1) return ORACLE_BAD_ARGS;
    const int64_t nc = (T + Q - 1) / Q;
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t h = 0; h < H; ++h)
            for (int64_t c = 0; c < nc; ++c) {
                double run = 0.0;
                for (int64_t i = 0; i < Q; ++i) {
                    const int64_t t = c * Q + i;
                    double delta = 0.0;
                    if (t < T) {
                        const double z = dt[(b * T + t) * H + h];
                        delta = dt_softplus ? softplus(z) : z;
                        if (seq_idx && t > 0 && seq_idx[t] != seq_idx[t - 1]) run = 0.0;
                    }
                    run += delta * A[h];
                    const int64_t o = ((b * H + h) * nc + c) * Q + i;
                    delta_out[o] = delta;
                    cs_out[o] = run;
                }
            }
    return ORACLE_OK;
}

/*
 * Reverse-mode derivative of the forward recurrence above (no chunking): the
 * gradients of L = sum y * dy + sum final_states * dfinal with respect to every
 * input.  The pages give no backward equations, so this is the chain rule
 * applied to the recurrence of ssd_oracle_forward, step by step in reverse:
 *
 *   g_t   = dL/dh_t = C_t dy_t^T  (+ dfinal at a sequence's last token)
 *                     + [carry into t+1] a_{t+1} g_{t+1}
 *   dx_t  = Delta_t g_t B_t + D dy_t          dB_t += Delta_t g_t^T x_t
 *   dC_t += h_t^T dy_t                        dDelta_t = x_t . (g_t B_t) + A dl_t
 *   dl_t  = [carry into t] a_t <g_t, h_{t-1}> (l_t = Delta_t A = log a_t)
 *   dA   += Delta_t dl_t                      dD += dy_t . x_t
 *   ddt_t = dDelta_t * sigmoid(dt_t)  (softplus' = sigmoid; or dDelta_t for raw dt)
 *   dinit = a_0 g_0
 *
 * dB and dC sum over the heads of a group, dA and dD over batch rows and time.
 * The forward states h_t of one (b, h, p) row are kept (T x N doubles), so the
 * derivative needs no identity beyond the chain rule.  Partial sums are reduced
 * in a fixed order, so results do not depend on the thread count.
 */
typedef struct {
    ssd_oracle_args f;       /* forward problem (its y / final_states / chunk fields are ignored) */
    const double *dy;        /* [b,T,H,P] */
    const double *dfinal;    /* [b,H,P,N], or [nseq,H,P,N] with seq_idx; NULL = zero */
    double *dx;              /* [b,T,H,P] */
    double *ddt;             /* [b,T,H] */
    double *dA;              /* [H] */
    double *dB, *dC;         /* [b,T,G,N] */
    double *dD;              /* [H] (may be NULL) */
    double *dinit;           /* [b,H,P,N] (may be NULL) */
} ssd_oracle_bwd_args;

int ssd_oracle_backward(const ssd_oracle_bwd_args *ba)
{
    if (!ba) return ORACLE_BAD_ARGS;
    const ssd_oracle_args *a = &ba->f;
    if (!a->x || !a->dt || !a->A || !a->B || !a->C || !ba->dy) return ORACLE_BAD_ARGS;
    if (!ba->dx || !ba->ddt || !ba->dA || !ba->dB || !ba->dC) return ORACLE_BAD_ARGS;
    const int64_t Bt = a->batch, T = a->seqlen, H = a->nheads, P = a->headdim;
    const int64_t N = a->dstate, G = a->ngroups;
    if (Bt < 1 || T < 1 || H < 1 || P < 1 || N < 1 || G < 1 || H % G != 0) return ORACLE_BAD_ARGS;
    if (a->seq_idx && (Bt != 1 || a->nseq < 1)) return ORACLE_BAD_ARGS;
    const int64_t units = Bt * H;
    /* per-(b,h) partial sums, reduced in a fixed order afterwards */
    double *pdB = (double *)calloc((size_t)(units * T * N), sizeof(double));
    double *pdC = (double *)calloc((size_t)(units * T * N), sizeof(double));
    double *pdA = (double *)calloc((size_t)units, sizeof(double));
    double *pdD = (double *)calloc((size_t)units, sizeof(double));
    if (!pdB || !pdC || !pdA || !pdD) {
        free(pdB); free(pdC); free(pdA); free(pdD);
        return ORACLE_NO_MEMORY;
    }
    int status = ORACLE_OK;

#pragma omp parallel
    {
        double *hs = (double *)malloc((size_t)(T * N) * sizeof(double));  /* h_t of one row */
        double *g = (double *)malloc((size_t)N * sizeof(double));
        double *dDelta = (double *)malloc((size_t)T * sizeof(double));
        double *dl = (double *)malloc((size_t)T * sizeof(double));
        if (!hs || !g || !dDelta || !dl) {
#pragma omp atomic write
            status = ORACLE_NO_MEMORY;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t u = 0; u < units; ++u) {
            if (!hs || !g || !dDelta || !dl) continue;
            const int64_t h = u % H, b = u / H, g_ = h * G / H;
            const double Ah = a->A[h], Dh = a->D ? a->D[h] : 0.0;
            double *uB = pdB + u * T * N, *uC = pdC + u * T * N;
            for (int64_t t = 0; t < T; ++t) dDelta[t] = dl[t] = 0.0;
            for (int64_t p = 0; p < P; ++p) {
                /* forward sweep of this row, keeping every h_t */
                for (int64_t t = 0; t < T; ++t) {
                    const int64_t bt = b * T + t;
                    const double z = a->dt[bt * H + h];
                    const double delta = a->dt_softplus ? softplus(z) : z;
                    const double decay = exp(delta * Ah);
                    const int keep = !(a->seq_idx && t > 0 && a->seq_idx[t] != a->seq_idx[t - 1]);
                    const double xv = a->x[(bt * H + h) * P + p];
                    const double *Bv = a->B + (bt * G + g_) * N;
                    for (int64_t n = 0; n < N; ++n) {
                        const double prev = t == 0 ? (a->initial_states ? a->initial_states[((b * H + h) * P + p) * N + n] : 0.0)
                                                   : hs[(t - 1) * N + n];
                        hs[t * N + n] = (keep ? decay * prev : 0.0) + delta * Bv[n] * xv;
                    }
                }
                /* reverse sweep */
                for (int64_t n = 0; n < N; ++n) g[n] = 0.0;
                for (int64_t t = T - 1; t >= 0; --t) {
                    const int64_t bt = b * T + t;
                    const double z = a->dt[bt * H + h];
                    const double delta = a->dt_softplus ? softplus(z) : z;
                    const double decay = exp(delta * Ah);
                    const int keep = !(a->seq_idx && t > 0 && a->seq_idx[t] != a->seq_idx[t - 1]);
                    const double xv = a->x[(bt * H + h) * P + p];
                    const double dyv = ba->dy[(bt * H + h) * P + p];
                    const double *Bv = a->B + (bt * G + g_) * N;
                    const double *Cv = a->C + (bt * G + g_) * N;
                    /* dfinal enters at the last token of the row (or of each segment) */
                    if (ba->dfinal) {
                        int64_t row = -1;
                        if (!a->seq_idx) {
                            if (t == T - 1) row = b;
                        } else if (t == T - 1 || a->seq_idx[t + 1] != a->seq_idx[t]) {
                            row = a->seq_idx[t];
                            if (row < 0 || row >= a->nseq) row = -1;
                        }
                        if (row >= 0)
                            for (int64_t n = 0; n < N; ++n) g[n] += ba->dfinal[((row * H + h) * P + p) * N + n];
                    }
                    for (int64_t n = 0; n < N; ++n) g[n] += Cv[n] * dyv;
                    double gB = 0.0;
                    for (int64_t n = 0; n < N; ++n) {
                        gB += g[n] * Bv[n];
                        uC[t * N + n] += hs[t * N + n] * dyv;
                        uB[t * N + n] += delta * xv * g[n];
                    }
                    ba->dx[(bt * H + h) * P + p] = delta * gB + Dh * dyv;
                    dDelta[t] += xv * gB;
                    pdD[u] += dyv * xv;
                    if (keep) {
                        double gh = 0.0;
                        for (int64_t n = 0; n < N; ++n) {
                            const double prev = t == 0 ? (a->initial_states ? a->initial_states[((b * H + h) * P + p) * N + n] : 0.0)
                                                       : hs[(t - 1) * N + n];
                            gh += g[n] * prev;
                        }
                        dl[t] += decay * gh;
                        for (int64_t n = 0; n < N; ++n) g[n] *= decay;
                    } else {
                        for (int64_t n = 0; n < N; ++n) g[n] = 0.0;
                    }
                }
                if (ba->dinit)
                    for (int64_t n = 0; n < N; ++n) ba->dinit[((b * H + h) * P + p) * N + n] = g[n];
            }
            for (int64_t t = 0; t < T; ++t) {
                const int64_t bt = b * T + t;
                const double z = a->dt[bt * H + h];
                const double delta = a->dt_softplus ? softplus(z) : z;
                const double dd = dDelta[t] + Ah * dl[t];
                const double sig = z >= 0.0 ? 1.0 / (1.0 + exp(-z)) : exp(z) / (1.0 + exp(z));
                ba->ddt[bt * H + h] = a->dt_softplus ? dd * sig : dd;
                pdA[u] += delta * dl[t];
            }
        }
        free(hs); free(g); free(dDelta); free(dl);
    }
    if (status == ORACLE_OK) {
        for (int64_t h = 0; h < H; ++h) {
            double sa = 0.0, sd = 0.0;
            for (int64_t b = 0; b < Bt; ++b) {
                sa += pdA[b * H + h];
                sd += pdD[b * H + h];
            }
            ba->dA[h] = sa;
            if (ba->dD) ba->dD[h] = sd;
        }
        for (int64_t b = 0; b < Bt; ++b)
            for (int64_t t = 0; t < T; ++t)
                for (int64_t g_ = 0; g_ < G; ++g_)
                    for (int64_t n = 0; n < N; ++n) {
                        double sb = 0.0, sc = 0.0;
                        for (int64_t h = g_ * (H / G); h < (g_ + 1) * (H / G); ++h) {
                            sb += pdB[((b * H + h) * T + t) * N + n];
                            sc += pdC[((b * H + h) * T + t) * N + n];
                        }
                        ba->dB[((b * T + t) * G + g_) * N + n] = sb;
                        ba->dC[((b * T + t) * G + g_) * N + n] = sc;
                    }
    }
    free(pdB); free(pdC); free(pdA); free(pdD);
    return status;
}
