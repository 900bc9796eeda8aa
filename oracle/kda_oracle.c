/*
 * kda_oracle.c -- plain fp64, token-by-token CPU oracle for the Kimi Delta
 * Attention (KDA) layer.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check
 * and the CPU-baseline leg of the benchmark call it; the GPU library never
 * does, and the two share no code.
 *
 * What it computes, per sequence n and head h, one token t at a time (all in
 * double precision; inputs are read exactly and widened to double):
 *
 *   1. short causal depthwise convolution of width W over every q, k and v
 *      channel, the window being the W-1 previous raw inputs (taken from the
 *      conv state, oldest first) and the current raw input; tap W-1 multiplies
 *      the current token; no bias.  SiLU on the result.  The conv state keeps
 *      the raw (pre-convolution) inputs.
 *      [vLLM blog "A Preview of Production-Scale Kimi K3 Support on vLLM",
 *       section "The Hardest Part: Prefix Caching for KDA": each KDA layer keeps
 *       a short convolution state beside its recurrent state; section "KDA
 *       prefill and decode": the causal convolution sits in front of the
 *       recurrence.]
 *   2. q and k are L2-normalised: x / sqrt(sum x^2 + l2_eps); no query scale.
 *   3. the state decays per key channel: S[i][:] *= exp(g[i]).
 *   4. delta rule on the decayed state:
 *        u = beta * (v - S^T k);  S += k u^T
 *      i.e. S_t = (I - beta k k^T) Diag(exp g) S_{t-1} + beta k v^T.
 *   5. readout of the updated state: o = S^T q.
 *   6. gated RMSNorm over the value dimension:
 *        y = o / sqrt(mean(o^2) + rms_eps) * norm_w * sigmoid(z)
 *      [same blog, section "KDA prefill and decode": the fused decode performs
 *       the short convolution, state update, output gate and normalisation
 *       together; agentlenshq "vLLM Kimi K3 Support", section "Fused Kernels and
 *       Metadata Optimization": the fused decode covers convolution, recurrent
 *       update and RMSNorm.]
 *   7. checkpoints: after token t, if ckpt_interval > 0 and the absolute
 *      position start_pos + t + 1 is a multiple of ckpt_interval, or t is the
 *      sequence's last token, the pair (S, conv state) is written to the
 *      sequence's next checkpoint slot.
 *      [vLLM blog, "The Hardest Part": resuming needs the state at the exact
 *       prefix boundary; agentlenshq, "Agentic Cache Retention Policies":
 *       interval-based retention checkpoints at fixed intervals and at prompt
 *       boundaries.]
 *   8. optional bf16 state storage (state_round != 0): wherever the state is
 *      stored -- every checkpoint and the sequence end -- it is rounded to the
 *      nearest bf16 value (ties to even) and the run continues from the
 *      rounded state; the readout of step 5 uses the state before rounding.
 *      [vLLM recipe "moonshotai/Kimi-K3", section "AMD MI355X: disaggregated
 *       prefill and decode": the worker command keeps the Mamba-style (KDA)
 *       state cache in bfloat16.]
 *
 * Steps 3-5 are the gated delta rule with a per-channel decay,
 * S_t = (I - beta_t k_t k_t^T) Diag(exp g_t) S_{t-1} + beta_t k_t v_t^T and
 * o_t = S_t^T q_t.  The pages describe the layer's parts but print no
 * equation; the SiLU-before-L2-norm order, the unit query scale, the logistic
 * output gate and the conv tap order are the plainest readings of them.
 *
 * Layouts (row-major, T = total tokens, N = sequences):
 *   q, k, g [T][H][dk]; v, z, out [T][H][dv]; beta [T][H]
 *   conv_w [H][2dk+dv][W]  (channels: q, then k, then v)
 *   norm_w [dv]
 *   S  [N][H][dk][dv]        in: initial state, out: final state
 *   X  [N][H][2dk+dv][W-1]   in: initial conv state, out: final
 *   ckpt_S [K][H][dk][dv], ckpt_X [K][H][2dk+dv][W-1]; sequence n's j-th
 *   checkpoint goes to slot ckpt_base[n] + j.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Number of checkpoints a sequence of len tokens starting at absolute
 * position start writes: the multiples of interval strictly inside
 * (start, start+len), plus the sequence end (counted once). */
int64_t kda_oracle_num_checkpoints(int64_t start, int64_t len, int64_t interval)
{
    if (interval <= 0 || len <= 0) return 0;
    int64_t end = start + len;
    /* multiples p of interval with start < p < end */
    int64_t first = (start / interval + 1) * interval;
    int64_t count = 0;
    for (int64_t p = first; p < end; p += interval) count++;
    return count + 1;
}

/* Nearest bf16 value of x (8 significant bits, ties to even; bf16 subnormals
 * are multiples of 2^-133). */
static double round_bf16(double x)
{
    if (x == 0.0 || !isfinite(x)) return x;
    int e;
    (void)frexp(x, &e);               /* x = m 2^e with 0.5 <= |m| < 1 */
    int qe = e - 8;                   /* weight of the last kept bit */
    if (qe < -133) qe = -133;
    return ldexp(nearbyint(ldexp(x, -qe)), qe);
}

static void round_state(double* Sh, int64_t n)
{
    for (int64_t i = 0; i < n; i++) Sh[i] = round_bf16(Sh[i]);
}

static double silu(double y) { return y / (1.0 + exp(-y)); }
static double sigmoid(double y) { return 1.0 / (1.0 + exp(-y)); }

static void run_chain(int n, int h, int H, int dk, int dv, int W,
                      double l2_eps, double rms_eps,
                      int64_t t0, int64_t L, int64_t start,
                      const double* q, const double* k, const double* v, const double* z,
                      const double* g, const double* beta,
                      const double* conv_w, const double* norm_w,
                      double* S, double* X,
                      int64_t interval, int64_t ckpt_slot0,
                      double* ckpt_S, double* ckpt_X, int state_round, double* out)
{
    const int C = 2 * dk + dv;
    const int Wm = W - 1;
    double* a = (double*)malloc(sizeof(double) * C);   /* post-conv, post-SiLU */
    double* u = (double*)malloc(sizeof(double) * dv);
    double* o = (double*)malloc(sizeof(double) * dv);
    double* Sh = S + ((int64_t)n * H + h) * dk * dv;   /* this chain's state */
    double* Xh = X + ((int64_t)n * H + h) * C * Wm;    /* this chain's conv state */
    const double* wh = conv_w + (int64_t)h * C * W;
    int64_t ck = 0;

    for (int64_t t = 0; t < L; t++) {
        const int64_t tok = t0 + t;
        const double* qt = q + (tok * H + h) * dk;
        const double* kt = k + (tok * H + h) * dk;
        const double* vt = v + (tok * H + h) * dv;
        const double* zt = z + (tok * H + h) * dv;
        const double* gt = g + (tok * H + h) * dk;
        const double bt = beta[tok * H + h];

        /* 1. causal depthwise conv over [q | k | v] channels, then SiLU */
        for (int c = 0; c < C; c++) {
            double x = c < dk ? qt[c] : (c < 2 * dk ? kt[c - dk] : vt[c - 2 * dk]);
            double* xs = Xh + (int64_t)c * Wm;
            const double* w = wh + (int64_t)c * W;
            double y = w[W - 1] * x;
            for (int m = 0; m < Wm; m++) y += w[m] * xs[m];
            a[c] = silu(y);
            for (int m = 0; m + 1 < Wm; m++) xs[m] = xs[m + 1];
            if (Wm > 0) xs[Wm - 1] = x;
        }
        /* 2. L2-normalise q and k */
        double sq = 0.0, sk = 0.0;
        for (int i = 0; i < dk; i++) { sq += a[i] * a[i]; sk += a[dk + i] * a[dk + i]; }
        const double rq = 1.0 / sqrt(sq + l2_eps), rk = 1.0 / sqrt(sk + l2_eps);
        double* qh = a;            /* normalised in place */
        double* kh = a + dk;
        const double* vh = a + 2 * dk;
        for (int i = 0; i < dk; i++) { qh[i] *= rq; kh[i] *= rk; }

        /* 3. per-key-channel decay of the state rows */
        for (int i = 0; i < dk; i++) {
            const double e = exp(gt[i]);
            double* row = Sh + (int64_t)i * dv;
            for (int j = 0; j < dv; j++) row[j] *= e;
        }
        /* 4. delta rule: u = beta (v - S^T k); S += k u^T */
        for (int j = 0; j < dv; j++) {
            double p = 0.0;
            for (int i = 0; i < dk; i++) p += Sh[(int64_t)i * dv + j] * kh[i];
            u[j] = bt * (vh[j] - p);
        }
        for (int i = 0; i < dk; i++) {
            double* row = Sh + (int64_t)i * dv;
            for (int j = 0; j < dv; j++) row[j] += kh[i] * u[j];
        }
        /* 5. readout of the updated state */
        for (int j = 0; j < dv; j++) {
            double s = 0.0;
            for (int i = 0; i < dk; i++) s += Sh[(int64_t)i * dv + j] * qh[i];
            o[j] = s;
        }
        /* 6. gated RMSNorm over dv */
        double ms = 0.0;
        for (int j = 0; j < dv; j++) ms += o[j] * o[j];
        ms /= (double)dv;
        const double r = 1.0 / sqrt(ms + rms_eps);
        double* yt = out + (tok * H + h) * dv;
        for (int j = 0; j < dv; j++) yt[j] = o[j] * r * norm_w[j] * sigmoid(zt[j]);

        /* 7. checkpoints */
        if (interval > 0) {
            const int64_t pos = start + t + 1;
            if (pos % interval == 0 || t == L - 1) {
                const int64_t slot = ckpt_slot0 + ck++;
                if (state_round) round_state(Sh, (int64_t)dk * dv);
                memcpy(ckpt_S + (slot * H + h) * dk * dv, Sh, sizeof(double) * dk * dv);
                if (Wm > 0)
                    memcpy(ckpt_X + (slot * H + h) * C * Wm, Xh, sizeof(double) * C * Wm);
            }
        }
    }
    /* 8. the final state is stored too */
    if (state_round) round_state(Sh, (int64_t)dk * dv);
    free(a); free(u); free(o);
}

/* Runs the recurrence over num_seqs packed sequences.  Returns 0 on success,
 * a negative value on invalid arguments.  state_round != 0 selects bf16 state
 * storage (step 8). */
int kda_oracle_run(int H, int dk, int dv, int W, double l2_eps, double rms_eps,
                   int num_seqs, const int64_t* cu_seqlens, const int64_t* start_pos,
                   const double* q, const double* k, const double* v, const double* z,
                   const double* g, const double* beta,
                   const double* conv_w, const double* norm_w,
                   double* S, double* X,
                   int64_t ckpt_interval, const int64_t* ckpt_base,
                   double* ckpt_S, double* ckpt_X, int state_round,
                   double* out, int num_threads)
{
    if (H <= 0 || dk <= 0 || dv <= 0 || W <= 0 || num_seqs < 0) return -1;
    if (ckpt_interval > 0 && (!ckpt_base || !ckpt_S || !ckpt_X)) return -2;
    const int64_t pairs = (int64_t)num_seqs * H;
#ifdef _OPENMP
    if (num_threads > 0) omp_set_num_threads(num_threads);
#else
    (void)num_threads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t p = 0; p < pairs; p++) {
        const int n = (int)(p / H), h = (int)(p % H);
        const int64_t t0 = cu_seqlens[n], L = cu_seqlens[n + 1] - cu_seqlens[n];
        const int64_t start = start_pos ? start_pos[n] : 0;
        run_chain(n, h, H, dk, dv, W, l2_eps, rms_eps, t0, L, start,
                  q, k, v, z, g, beta, conv_w, norm_w, S, X,
                  ckpt_interval, ckpt_base ? ckpt_base[n] : 0, ckpt_S, ckpt_X, state_round, out);
    }
    return 0;
}

/* round_bf16 over an array (exposed for its pin against a library conversion) */
void kda_oracle_round_bf16(const double* x, double* y, int64_t n)
{
    for (int64_t i = 0; i < n; i++) y[i] = round_bf16(x[i]);
}

int kda_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
