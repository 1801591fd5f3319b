/*
 * la_oracle.c -- plain, slow, obviously correct CPU oracle for chunked linear attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and its Python
 * binding) may include, link, load or call this file.  Only the test-suite, the smoke check
 * and the CPU-baseline leg of the benchmark use it.  It shares no code, header, table or
 * constant with the GPU kernels.
 *
 * Everything is evaluated token by token in IEEE double precision, straight from the
 * definition of causal linear attention as a fixed-size state recurrence (the review page
 * "ZeCO: Zero Communication Overhead Sequence Parallelism for Linear Attention", fields
 * pith_extraction.supporting_citations[0] (Katharopoulos et al.: linear attention is a
 * fixed-size state recurrence) and [1] (Yang et al.: the gated, GLA-style recurrence whose
 * state S in R^{dk x dv} ZeCO passes between devices, pith_extraction.core_discovery)):
 *
 *     S_0 = s_in,   S_t = diag(a_t) S_{t-1} + k_t v_t^T,   o_t = S_t^T q_t,   s_out = S_L.
 *
 * There is no chunking, blocking or reordering here: one token at a time, one state column at
 * a time.  The per-token decay a_t in R^{dk} is, by mode:
 *     NONE : a_t = 1
 *     HEAD : a_t = exp(lambda_h)                       (one log-decay per head, lambda_h <= 0)
 *     GATE : a_t = sigmoid(g_t)^(1 / gate_norm)         (per token and key dimension)
 * GATE is evaluated directly as a power of the sigmoid, not in log space.
 *
 * Inputs q, k, v, decay are float arrays (bf16 and fp32 inputs are exactly representable in
 * float); every product and sum below is done in double.  Outputs are double.
 *
 * Segments: a sequence of L tokens may be cut into nseg equal segments that are treated as
 * independent sequences; segment 0 starts from s_in, the others from zero.  With nseg = 1 this
 * is the one-pass recurrence.  The linear-decomposition identity of the same page
 * (pith_extraction.key_machinery) is what makes the segmented form recombinable; the helpers
 * orc_cumdecay / orc_state_scan / orc_state_correct write that recombination out literally.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_NONE = 0, ORC_HEAD = 1, ORC_GATE = 2 };

/* Per-token, per-key-dimension decay a_t[d] of the recurrence, by mode. */
static double orc_decay(int mode, const float* decay, double gate_norm, int64_t h,
                        int64_t bh, int64_t L, int64_t t, int dk, int d) {
    if (mode == ORC_HEAD) return exp((double)decay[h]);
    if (mode == ORC_GATE) {
        double g = (double)decay[(bh * L + t) * (int64_t)dk + d];
        double sig = 1.0 / (1.0 + exp(-g));
        return pow(sig, 1.0 / gate_norm);
    }
    return 1.0;
}

typedef struct {
    int64_t B, H, L;
    int dk, dv, nseg, mode, cblk;
    double gate_norm;
    const float *q, *k, *v, *decay;
    const double* s_in;
    double *o, *s_out;
    int64_t nitems;
    int64_t next; /* work counter, guarded by mu */
    pthread_mutex_t mu;
} rec_job;

/* One work item = one (b, h, segment, block of state columns).  The recurrence is separable
 * per column of S: column c only ever reads v_t[c] and writes o_t[c]. */
static void rec_item(rec_job* J, int64_t item, double* S, double* a) {
    const int dk = J->dk, dv = J->dv;
    const int64_t ncb = (dv + J->cblk - 1) / J->cblk;
    const int64_t cb = item % ncb;
    const int64_t seg = (item / ncb) % J->nseg;
    const int64_t bh = item / (ncb * J->nseg);
    const int64_t h = bh % J->H;
    const int c0 = (int)(cb * J->cblk);
    const int nc = (c0 + J->cblk <= dv) ? J->cblk : dv - c0;
    const int64_t Ls = J->L / J->nseg;
    const int64_t t0 = seg * Ls, t1 = t0 + Ls;

    for (int d = 0; d < dk; d++)
        for (int c = 0; c < nc; c++)
            S[d * nc + c] = (seg == 0 && J->s_in) ? J->s_in[(bh * dk + d) * dv + c0 + c] : 0.0;

    for (int64_t t = t0; t < t1; t++) {
        const float* qt = J->q + (bh * J->L + t) * dk;
        const float* kt = J->k + (bh * J->L + t) * dk;
        const float* vt = J->v + (bh * J->L + t) * dv + c0;
        double* ot = J->o + (bh * J->L + t) * dv + c0;
        for (int d = 0; d < dk; d++) a[d] = orc_decay(J->mode, J->decay, J->gate_norm, h, bh, J->L, t, dk, d);
        /* S_t = diag(a_t) S_{t-1} + k_t v_t^T */
        for (int d = 0; d < dk; d++) {
            const double ad = a[d], kd = (double)kt[d];
            for (int c = 0; c < nc; c++) S[d * nc + c] = ad * S[d * nc + c] + kd * (double)vt[c];
        }
        /* o_t = S_t^T q_t */
        for (int c = 0; c < nc; c++) ot[c] = 0.0;
        for (int d = 0; d < dk; d++) {
            const double qd = (double)qt[d];
            for (int c = 0; c < nc; c++) ot[c] += qd * S[d * nc + c];
        }
    }
    if (J->s_out)
        for (int d = 0; d < dk; d++)
            for (int c = 0; c < nc; c++)
                J->s_out[((bh * J->nseg + seg) * dk + d) * dv + c0 + c] = S[d * nc + c];
}

static void* rec_worker(void* arg) {
    rec_job* J = (rec_job*)arg;
    double* S = (double*)malloc(sizeof(double) * (size_t)J->dk * J->cblk);
    double* a = (double*)malloc(sizeof(double) * (size_t)J->dk);
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int64_t it = J->next++;
        pthread_mutex_unlock(&J->mu);
        if (it >= J->nitems) break;
        rec_item(J, it, S, a);
    }
    free(S);
    free(a);
    return NULL;
}

/*
 * Token-by-token recurrence.  q, k: [B,H,L,dk]; v: [B,H,L,dv]; decay: NULL (NONE), [H] log-decay
 * (HEAD) or [B,H,L,dk] raw gate g (GATE); s_in: [B,H,dk,dv] or NULL (zero); o: [B,H,L,dv];
 * s_out: [B,H,nseg,dk,dv] or NULL.  Returns 0, or -1 on a bad argument.
 */
int orc_recurrence(int64_t B, int64_t H, int64_t L, int dk, int dv, int nseg,
                   const float* q, const float* k, const float* v, int mode, const float* decay,
                   double gate_norm, const double* s_in, double* o, double* s_out, int nthreads) {
    if (B < 0 || H < 0 || L < 0 || dk <= 0 || dv <= 0 || nseg <= 0 || L % nseg) return -1;
    if (mode != ORC_NONE && mode != ORC_HEAD && mode != ORC_GATE) return -1;
    if (mode != ORC_NONE && !decay) return -1;
    if (mode == ORC_GATE && !(gate_norm > 0)) return -1;
    rec_job J;
    memset(&J, 0, sizeof J);
    J.B = B; J.H = H; J.L = L; J.dk = dk; J.dv = dv; J.nseg = nseg; J.mode = mode;
    J.cblk = 16; J.gate_norm = gate_norm;
    J.q = q; J.k = k; J.v = v; J.decay = decay; J.s_in = s_in; J.o = o; J.s_out = s_out;
    J.nitems = B * H * nseg * ((dv + J.cblk - 1) / J.cblk);
    J.next = 0;
    pthread_mutex_init(&J.mu, NULL);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    int started = 0;
    for (int i = 1; i < nthreads; i++)
        if (pthread_create(&th[started], NULL, rec_worker, &J) == 0) started++;
    rec_worker(&J);
    for (int i = 0; i < started; i++) pthread_join(th[i], NULL);
    pthread_mutex_destroy(&J.mu);
    return 0;
}

/*
 * Cumulative decay inside each segment: cum[b,h,t,d] = prod_{s = segment start .. t} a_s[d]
 * (inclusive), and total[b,h,p,d] = the product over the whole segment p.  This is the
 * "cumulative decay" that the decomposition identity applies to an incoming state.  Either
 * output may be NULL.
 */
int orc_cumdecay(int64_t B, int64_t H, int64_t L, int dk, int nseg, int mode, const float* decay,
                 double gate_norm, double* cum, double* total) {
    if (B < 0 || H < 0 || L < 0 || dk <= 0 || nseg <= 0 || L % nseg) return -1;
    if (mode != ORC_NONE && !decay) return -1;
    const int64_t Ls = L / nseg;
    for (int64_t bh = 0; bh < B * H; bh++) {
        const int64_t h = bh % H;
        for (int64_t p = 0; p < nseg; p++) {
            for (int d = 0; d < dk; d++) {
                double run = 1.0;
                for (int64_t t = p * Ls; t < (p + 1) * Ls; t++) {
                    run *= orc_decay(mode, decay, gate_norm, h, bh, L, t, dk, d);
                    if (cum) cum[(bh * L + t) * dk + d] = run;
                }
                if (total) total[(bh * nseg + p) * dk + d] = run;
            }
        }
    }
    return 0;
}

/*
 * Inclusive state scan over P segments, one (b,h) at a time, p in order:
 *     out[p] = diag(seg_decay[p]) out[p-1] + seg_states[p],   out[-1] = 0.
 * This is the receive-update-forward rule of All-Scan written as a plain sequential loop
 * (page "ZeCO ...", pith_extraction.key_machinery; the accumulated state is what moves on, as
 * referee_report.major_comments[3] says it must).  seg_states, out: [B,H,P,dk,dv];
 * seg_decay: [B,H,P,dk].  out may equal seg_states.
 */
int orc_state_scan(int64_t B, int64_t H, int P, int dk, int dv, const double* seg_states,
                   const double* seg_decay, double* out) {
    if (B < 0 || H < 0 || P <= 0 || dk <= 0 || dv <= 0) return -1;
    const int64_t SZ = (int64_t)dk * dv;
    for (int64_t bh = 0; bh < B * H; bh++) {
        for (int p = 0; p < P; p++) {
            const double* x = seg_states + (bh * P + p) * SZ;
            const double* lam = seg_decay + (bh * P + p) * dk;
            double* y = out + (bh * P + p) * SZ;
            const double* yprev = (p > 0) ? out + (bh * P + p - 1) * SZ : NULL;
            for (int d = 0; d < dk; d++)
                for (int c = 0; c < dv; c++)
                    y[d * dv + c] = (yprev ? lam[d] * yprev[d * dv + c] : 0.0) + x[d * dv + c];
        }
    }
    return 0;
}

/*
 * Output correction for an incoming state, token by token:
 *     o_t += sum_d q_t[d] * cum_t[d] * s_recv[p][d, :]     for every token t of segment p >= seg_begin,
 * where s_recv for segment p is s_recv[b,h,p - seg_begin].  q: [B,H,L,dk] float; cum: [B,H,L,dk];
 * s_recv: [B,H,nseg - seg_begin,dk,dv]; o: [B,H,L,dv] updated in place.
 */
int orc_state_correct(int64_t B, int64_t H, int64_t L, int dk, int dv, int nseg, int seg_begin,
                      const float* q, const double* cum, const double* s_recv, double* o) {
    if (B < 0 || H < 0 || L < 0 || dk <= 0 || dv <= 0 || nseg <= 0 || L % nseg) return -1;
    if (seg_begin < 0 || seg_begin > nseg) return -1;
    const int64_t Ls = L / nseg;
    const int np = nseg - seg_begin;
    for (int64_t bh = 0; bh < B * H; bh++) {
        for (int p = seg_begin; p < nseg; p++) {
            const double* S = s_recv + ((bh * np) + (p - seg_begin)) * (int64_t)dk * dv;
            for (int64_t t = p * Ls; t < (p + 1) * Ls; t++) {
                const float* qt = q + (bh * L + t) * dk;
                const double* ct = cum + (bh * L + t) * dk;
                double* ot = o + (bh * L + t) * dv;
                for (int d = 0; d < dk; d++) {
                    const double w = (double)qt[d] * ct[d];
                    for (int c = 0; c < dv; c++) ot[c] += w * S[d * dv + c];
                }
            }
        }
    }
    return 0;
}

/*
 * Reverse-mode derivative of the same recurrence, token by token in double (the backward pass the
 * review page lists as a consequence of the forward design, pith_extraction.forward_implications).
 * For a loss whose gradients with respect to o and to each segment's final state are given
 * (d_o: [B,H,L,dv]; ds_out: [B,H,nseg,dk,dv] or NULL for zero), the chain rule applied to
 *     S_t = diag(a_t) S_{t-1} + k_t v_t^T,   o_t = S_t^T q_t
 * gives, with G_t the total derivative with respect to S_t (walked from the segment's end):
 *     G_last = ds_out + q_last d_o_last^T,   G_{t-1} = diag(a_t) G_t + q_{t-1} d_o_{t-1}^T,
 *     dq_t = S_t d_o_t,   dk_t = G_t v_t,   dv_t = G_t^T k_t,
 *     da_t[d] = sum_c G_t[d,c] S_{t-1}[d,c],   ds_in = diag(a_first) G_first.
 * The state trajectory S_t of the segment is kept whole (no recomputation).  The decay parameter's
 * derivative follows from da by the chain rule of its own definition:
 *     HEAD: a = exp(lambda_h)            -> d lambda_h = sum over b, t, d of da_t[d] a_t[d]
 *     GATE: a = sigmoid(g)^(1/gate_norm) -> dg_t[d] = da_t[d] a_t[d] (1 - sigmoid(g_t[d])) / gate_norm
 * Outputs (all double): dq, dk [B,H,L,dk]; dv [B,H,L,dv]; ddecay: [H] (HEAD), [B,H,L,dk] (GATE) or
 * NULL (NONE, or not wanted); ds_in: [B,H,nseg,dk,dv] (the derivative with respect to each
 * segment's initial state, s_in for segment 0 and zero for the others) or NULL.
 * Returns 0, -1 on a bad argument, -2 if a trajectory buffer cannot be allocated.
 */
typedef struct {
    int64_t B, H, L;
    int dk, dv, nseg, mode;
    double gate_norm;
    const float *q, *k, *v, *decay, *d_o;
    const double *s_in, *ds_out;
    double *dq, *dk_out, *dv_out, *ddecay, *ds_in;
    double* head_part; /* one partial d lambda_h per item (HEAD) */
    int64_t nitems, next;
    int failed;
    pthread_mutex_t mu;
} bwd_job;

static int bwd_item(bwd_job* J, int64_t item, double* traj, double* G, double* a_all) {
    const int dk = J->dk, dv = J->dv;
    const int64_t SZ = (int64_t)dk * dv;
    const int64_t seg = item % J->nseg, bh = item / J->nseg, h = bh % J->H;
    const int64_t Ls = J->L / J->nseg, t0 = seg * Ls;
    /* forward: traj[i] = S after i tokens of the segment (traj[0] = initial state) */
    for (int64_t e = 0; e < SZ; e++) traj[e] = (seg == 0 && J->s_in) ? J->s_in[bh * SZ + e] : 0.0;
    for (int64_t i = 0; i < Ls; i++) {
        const int64_t t = t0 + i;
        const float* kt = J->k + (bh * J->L + t) * dk;
        const float* vt = J->v + (bh * J->L + t) * dv;
        double* a = a_all + i * dk;
        for (int d = 0; d < dk; d++) a[d] = orc_decay(J->mode, J->decay, J->gate_norm, h, bh, J->L, t, dk, d);
        const double* Sp = traj + i * SZ;
        double* Sn = traj + (i + 1) * SZ;
        for (int d = 0; d < dk; d++)
            for (int c = 0; c < dv; c++) Sn[d * dv + c] = a[d] * Sp[d * dv + c] + (double)kt[d] * (double)vt[c];
    }
    /* backward */
    for (int64_t e = 0; e < SZ; e++) G[e] = J->ds_out ? J->ds_out[(bh * J->nseg + seg) * SZ + e] : 0.0;
    double head_acc = 0.0;
    for (int64_t i = Ls - 1; i >= 0; i--) {
        const int64_t t = t0 + i, row = bh * J->L + t;
        const float* qt = J->q + row * dk;
        const float* kt = J->k + row * dk;
        const float* vt = J->v + row * dv;
        const float* dot = J->d_o + row * dv;
        const double* St = traj + (i + 1) * SZ;
        const double* Sp = traj + i * SZ;
        const double* a = a_all + i * dk;
        for (int d = 0; d < dk; d++)
            for (int c = 0; c < dv; c++) G[d * dv + c] += (double)qt[d] * (double)dot[c];
        for (int d = 0; d < dk; d++) {
            double sq = 0.0, sk = 0.0, da = 0.0;
            for (int c = 0; c < dv; c++) {
                sq += St[d * dv + c] * (double)dot[c];
                sk += G[d * dv + c] * (double)vt[c];
                da += G[d * dv + c] * Sp[d * dv + c];
            }
            J->dq[row * dk + d] = sq;
            J->dk_out[row * dk + d] = sk;
            if (J->mode == ORC_HEAD) head_acc += da * a[d];
            if (J->mode == ORC_GATE && J->ddecay) {
                const double g = (double)J->decay[row * dk + d];
                const double sig = 1.0 / (1.0 + exp(-g));
                J->ddecay[row * dk + d] = da * a[d] * (1.0 - sig) / J->gate_norm;
            }
        }
        for (int c = 0; c < dv; c++) {
            double s = 0.0;
            for (int d = 0; d < dk; d++) s += G[d * dv + c] * (double)kt[d];
            J->dv_out[row * dv + c] = s;
        }
        for (int d = 0; d < dk; d++)
            for (int c = 0; c < dv; c++) G[d * dv + c] *= a[d];
    }
    if (J->ds_in)
        for (int64_t e = 0; e < SZ; e++) J->ds_in[(bh * J->nseg + seg) * SZ + e] = G[e];
    J->head_part[item] = head_acc;
    return 0;
}

static void* bwd_worker(void* arg) {
    bwd_job* J = (bwd_job*)arg;
    const int64_t Ls = J->L / J->nseg, SZ = (int64_t)J->dk * J->dv;
    double* traj = (double*)malloc(sizeof(double) * (size_t)((Ls + 1) * SZ));
    double* G = (double*)malloc(sizeof(double) * (size_t)SZ);
    double* a = (double*)malloc(sizeof(double) * (size_t)(Ls * J->dk + 1));
    if (!traj || !G || !a) {
        pthread_mutex_lock(&J->mu);
        J->failed = 1;
        pthread_mutex_unlock(&J->mu);
    } else {
        for (;;) {
            pthread_mutex_lock(&J->mu);
            int64_t it = J->next++;
            pthread_mutex_unlock(&J->mu);
            if (it >= J->nitems) break;
            bwd_item(J, it, traj, G, a);
        }
    }
    free(traj);
    free(G);
    free(a);
    return NULL;
}

int orc_recurrence_bwd(int64_t B, int64_t H, int64_t L, int dk, int dv, int nseg,
                       const float* q, const float* k, const float* v, int mode, const float* decay,
                       double gate_norm, const double* s_in, const float* d_o, const double* ds_out,
                       double* dq, double* dk_out, double* dv_out, double* ddecay, double* ds_in,
                       int nthreads) {
    if (B < 0 || H < 0 || L < 0 || dk <= 0 || dv <= 0 || nseg <= 0 || L % nseg) return -1;
    if (mode != ORC_NONE && mode != ORC_HEAD && mode != ORC_GATE) return -1;
    if (mode != ORC_NONE && !decay) return -1;
    if (mode == ORC_GATE && !(gate_norm > 0)) return -1;
    if (!q || !k || !v || !d_o || !dq || !dk_out || !dv_out) return -1;
    bwd_job J;
    memset(&J, 0, sizeof J);
    J.B = B; J.H = H; J.L = L; J.dk = dk; J.dv = dv; J.nseg = nseg; J.mode = mode;
    J.gate_norm = gate_norm;
    J.q = q; J.k = k; J.v = v; J.decay = decay; J.d_o = d_o; J.s_in = s_in; J.ds_out = ds_out;
    J.dq = dq; J.dk_out = dk_out; J.dv_out = dv_out; J.ddecay = ddecay; J.ds_in = ds_in;
    J.nitems = B * H * nseg;
    J.head_part = (double*)calloc((size_t)(J.nitems + 1), sizeof(double));
    if (!J.head_part) return -2;
    pthread_mutex_init(&J.mu, NULL);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > J.nitems) nthreads = J.nitems > 0 ? (int)J.nitems : 1;
    pthread_t th[256];
    int started = 0;
    for (int i = 1; i < nthreads; i++)
        if (pthread_create(&th[started], NULL, bwd_worker, &J) == 0) started++;
    bwd_worker(&J);
    for (int i = 0; i < started; i++) pthread_join(th[i], NULL);
    pthread_mutex_destroy(&J.mu);
    if (mode == ORC_HEAD && ddecay) {
        for (int64_t h = 0; h < H; h++) ddecay[h] = 0.0;
        for (int64_t it = 0; it < J.nitems; it++) ddecay[(it / nseg) % H] += J.head_part[it];
    }
    free(J.head_part);
    return J.failed ? -2 : 0;
}
