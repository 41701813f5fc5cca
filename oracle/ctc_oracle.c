/*
 * Packed CTC loss and gradient — float64 CPU ORACLE.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain reference that the HIP path is checked
 * against.  Only the tests, the smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no code, header, table or helper with the HIP library, and the product path never
 * calls it.
 *
 * Source of the method: the NVIDIA-NeMo/Speech pull request page "feat(asr): native CTC loss kernel
 * over sequence-packed log probabilities" (cited below as [PR]).  Its Triton file holds the module
 * description, the public function `packed_ctc_loss`, the autograd function and the two kernels
 * `_alpha_kernel` and `_beta_grad_kernel`; its `ctc.py` diff holds the reductions of
 * `forward_packed`.  The method computes the exact CTC negative log-likelihood of each utterance
 * and its gradient; only rounding differs between implementations, so this oracle evaluates the
 * same recursion in float64, in the order the kernels take it:
 *
 *   1. per utterance b: first row r = cu_seqlens[b], T = lengths[b] frames, U = target_lengths[b]
 *      labels, S = 2U + 1 extended states; state s is the blank for even s and the label
 *      targets[b][(s-1)/2] for odd s  ([PR] `_extended_labels`);
 *   2. T = 0: no rows; the loss is 0 without labels, +inf with labels  ([PR] `_alpha_kernel`);
 *   3. alpha[0] holds the first blank and the first label, everything else is -inf; each later
 *      frame takes the log-sum-exp of stay / advance-by-one / skip-by-two, the skip allowed only
 *      into a label state s >= 3 whose label differs from the label two states back (ids compared
 *      as ids: a target equal to the blank id is an ordinary label), plus the frame's log prob at
 *      the state's class  ([PR] `_alpha_kernel`, `_logsumexp3`);
 *   4. nll = -logsumexp(alpha[T-1][S-1], alpha[T-1][S-2])  ([PR] `_alpha_kernel`);
 *   5. beta mirrors alpha from the last frame, emission included  ([PR] `_beta_grad_kernel`);
 *   6. the gradient weight is the upstream scale, forced to 0 under zero_infinity when the loss is
 *      infinite; the posterior of state s at frame t is exp(alpha + beta - lp + nll), formed only
 *      when the weight is non-zero  ([PR] `_beta_grad_kernel`);
 *   7. gradient row = weight * (exp(lp) - posterior summed per class); rows owned by no utterance
 *      are zero  ([PR] `_PackedCTCLoss.backward`, `_beta_grad_kernel`);
 *   8. zero_infinity turns an infinite loss into 0  ([PR] `_PackedCTCLoss.forward`);
 *   9. reductions: sum of losses; mean = mean over utterances of loss / max(U, 1)
 *      ([PR] `ctc.py` `forward_packed`).
 *
 * Readings where the page leaves a step open (each is listed with its reason in the design notes):
 *   - an infeasible utterance with a non-zero weight (no zero_infinity) gets NaN in every column of
 *     its rows (the page's kernel would give NaN only at the blank and label columns; the padded
 *     library reference gives NaN everywhere);
 *   - the loss of a zero-frame utterance without labels is +0.0;
 *   - a NaN log prob at a column the recursion reads (the blank or one of the utterance's labels) in
 *     any of its rows makes the loss NaN, whether or not an alignment exists, and zero_infinity
 *     leaves it (the loss is not infinite); its rows are then NaN in every column under a non-zero
 *     weight.  A NaN at any other column leaves the loss alone and shows only in that column of
 *     the gradient row.  (The page does not treat NaN inputs; torch's float64 ctc_loss gives the
 *     same results wherever the NaN lies on a state some alignment can pass through.)
 *   - a zero gradient weight gives zero rows, whatever the log probs hold.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARG 1
#define ORACLE_ERR_ALLOC 2

enum { RED_NONE = 0, RED_SUM = 1, RED_MEAN = 2 };

/* -inf-safe log-sum-exp of three terms: the peak, and if the peak is -inf the result is -inf. */
static double logsumexp3(double a, double b, double c) {
    double peak = fmax(fmax(a, b), c);
    if (peak == -INFINITY) return -INFINITY;
    return peak + log(exp(a - peak) + exp(b - peak) + exp(c - peak));
}

/* class of extended state s */
static int64_t ext_label(const int64_t* tgt, int64_t s, int64_t blank) {
    return (s % 2 == 0) ? blank : tgt[(s - 1) / 2];
}

/*
 * One utterance: alpha, beta, nll.  lp points at the utterance's first row, row stride D.
 * alpha, beta: (T, S) caller-provided work arrays.  Returns nll (+inf if no alignment exists).
 */
static double utterance_alpha_beta(const double* lp, int64_t D, int64_t T, const int64_t* tgt, int64_t U,
                                   int64_t blank, double* alpha, double* beta) {
    const int64_t S = 2 * U + 1;
    if (T == 0) return U == 0 ? 0.0 : INFINITY;
    /* step 3: the first frame */
    for (int64_t s = 0; s < S; ++s) alpha[s] = -INFINITY;
    alpha[0] = lp[ext_label(tgt, 0, blank)];
    if (S > 1) alpha[1] = lp[ext_label(tgt, 1, blank)];
    for (int64_t t = 1; t < T; ++t) {
        const double* prev = alpha + (t - 1) * S;
        double* cur = alpha + t * S;
        const double* row = lp + t * D;
        for (int64_t s = 0; s < S; ++s) {
            const int64_t l = ext_label(tgt, s, blank);
            double stay = prev[s];
            double advance = s >= 1 ? prev[s - 1] : -INFINITY;
            double skip = -INFINITY;
            if (s % 2 == 1 && s >= 2 && l != ext_label(tgt, s - 2, blank)) skip = prev[s - 2];
            cur[s] = logsumexp3(stay, advance, skip) + row[l];
        }
    }
    /* step 4 */
    const double* last = alpha + (T - 1) * S;
    double nll = -logsumexp3(last[S - 1], S >= 2 ? last[S - 2] : -INFINITY, -INFINITY);
    /* step 5: beta from the last frame */
    double* bl = beta + (T - 1) * S;
    for (int64_t s = 0; s < S; ++s) bl[s] = -INFINITY;
    bl[S - 1] = lp[(T - 1) * D + ext_label(tgt, S - 1, blank)];
    if (S >= 2) bl[S - 2] = lp[(T - 1) * D + ext_label(tgt, S - 2, blank)];
    for (int64_t t = T - 2; t >= 0; --t) {
        const double* next = beta + (t + 1) * S;
        double* cur = beta + t * S;
        const double* row = lp + t * D;
        for (int64_t s = 0; s < S; ++s) {
            const int64_t l = ext_label(tgt, s, blank);
            double stay = next[s];
            double advance = s + 1 < S ? next[s + 1] : -INFINITY;
            double skip = -INFINITY;
            if (s % 2 == 1 && s + 2 < S && l != ext_label(tgt, s + 2, blank)) skip = next[s + 2];
            cur[s] = logsumexp3(stay, advance, skip) + row[l];
        }
    }
    return nll;
}

/*
 * Posteriors of one utterance, for the invariant tests: gamma (T, S) = exp(alpha + beta - lp + nll),
 * and gamma_norm (T, S) = the same quantity normalised per frame, softmax over s of
 * (alpha + beta - lp).  The two agree for a feasible utterance; both are left at 0 (gamma) / NaN
 * when the utterance is infeasible.  alpha_out / beta_out may be NULL.  Returns nll.
 */
double ctc_oracle_posteriors(const double* lp, int64_t D, int64_t T, const int64_t* tgt, int64_t U, int64_t blank,
                             double* gamma, double* gamma_norm, double* alpha_out, double* beta_out) {
    const int64_t S = 2 * U + 1;
    if (T <= 0) return U == 0 ? 0.0 : INFINITY;
    double* alpha = (double*)malloc(sizeof(double) * T * S);
    double* beta = (double*)malloc(sizeof(double) * T * S);
    if (!alpha || !beta) { free(alpha); free(beta); return NAN; }
    double nll = utterance_alpha_beta(lp, D, T, tgt, U, blank, alpha, beta);
    for (int64_t t = 0; t < T; ++t) {
        double peak = -INFINITY;
        for (int64_t s = 0; s < S; ++s) {
            double x = alpha[t * S + s] + beta[t * S + s] - lp[t * D + ext_label(tgt, s, blank)];
            if (gamma) gamma[t * S + s] = isinf(nll) ? 0.0 : exp(x + nll);
            if (x > peak) peak = x;
        }
        double z = 0.0;
        for (int64_t s = 0; s < S; ++s) {
            double x = alpha[t * S + s] + beta[t * S + s] - lp[t * D + ext_label(tgt, s, blank)];
            z += (peak == -INFINITY) ? 0.0 : exp(x - peak);
        }
        for (int64_t s = 0; s < S; ++s) {
            double x = alpha[t * S + s] + beta[t * S + s] - lp[t * D + ext_label(tgt, s, blank)];
            if (gamma_norm) gamma_norm[t * S + s] = (peak == -INFINITY) ? NAN : exp(x - peak) / z;
        }
    }
    if (alpha_out) memcpy(alpha_out, alpha, sizeof(double) * T * S);
    if (beta_out) memcpy(beta_out, beta, sizeof(double) * T * S);
    free(alpha);
    free(beta);
    return nll;
}

/*
 * The whole packed batch.
 *   lp            (T_total, D) float64 log probabilities (bf16/f16 inputs upcast exactly)
 *   cu, len       (B+1,), (B,) int64: utterance b owns rows [cu[b], cu[b] + len[b])
 *   targets       (B, W) int64, target_lengths (B,) int64
 *   grad_scale    (B,) upstream scale per utterance, or NULL for 1
 *   nll_out       (B,) raw negative log-likelihood (+inf when infeasible), may be NULL
 *   loss_out      (B,) loss after zero_infinity, may be NULL
 *   reduced_out   scalar for sum/mean, may be NULL
 *   grad          (T_total, D) gradient with the reduction's weights, may be NULL; fully written
 * Returns 0, or ORACLE_ERR_ARG for inputs outside the method's domain (negative lengths, rows
 * outside the buffer, a target length beyond the width, a class id outside [0, D)).
 */
int ctc_oracle(const double* lp, int64_t T_total, int64_t D, const int64_t* cu, const int64_t* len, int64_t B,
               const int64_t* targets, int64_t W, const int64_t* target_lengths, int64_t blank, int zero_infinity,
               int reduction, const double* grad_scale, double* nll_out, double* loss_out, double* reduced_out,
               double* grad, int nthreads) {
    if (D <= 0 || blank < 0 || blank >= D || B < 0 || T_total < 0) return ORACLE_ERR_ARG;
    if (reduction < RED_NONE || reduction > RED_MEAN) return ORACLE_ERR_ARG;
    for (int64_t b = 0; b < B; ++b) {
        if (len[b] < 0 || cu[b] < 0 || cu[b] + len[b] > T_total) return ORACLE_ERR_ARG;
        if (target_lengths[b] < 0 || target_lengths[b] > W) return ORACLE_ERR_ARG;
        for (int64_t j = 0; j < target_lengths[b]; ++j)
            if (targets[b * W + j] < 0 || targets[b * W + j] >= D) return ORACLE_ERR_ARG;
    }
    double* nll = (double*)malloc(sizeof(double) * (B > 0 ? B : 1));
    int64_t* order = (int64_t*)malloc(sizeof(int64_t) * (B > 0 ? B : 1));
    if (!nll || !order) { free(nll); free(order); return ORACLE_ERR_ALLOC; }
    if (grad) memset(grad, 0, sizeof(double) * T_total * D); /* rows owned by no utterance stay 0 */

    /* longest work first, so the parallel loop balances */
    for (int64_t b = 0; b < B; ++b) order[b] = b;
    for (int64_t i = 1; i < B; ++i) {
        int64_t k = order[i], j = i - 1;
        double ck = (double)len[k] * (2 * target_lengths[k] + 1);
        while (j >= 0 && (double)len[order[j]] * (2 * target_lengths[order[j]] + 1) < ck) { order[j + 1] = order[j]; --j; }
        order[j + 1] = k;
    }
    int failed = 0;
#ifdef _OPENMP
    /* a thread count for this call only (0: the runtime's default); it does not change later calls */
    const int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
#endif
    for (int64_t i = 0; i < B; ++i) {
        const int64_t b = order[i];
        const int64_t T = len[b], U = target_lengths[b], S = 2 * U + 1, r = cu[b];
        const int64_t* tgt = targets + b * W;
        double* alpha = T > 0 ? (double*)malloc(sizeof(double) * T * S) : NULL;
        double* beta = T > 0 ? (double*)malloc(sizeof(double) * T * S) : NULL;
        if (T > 0 && (!alpha || !beta)) { free(alpha); free(beta); failed = 1; continue; }
        const double* ulp = lp + r * D;
        double n = utterance_alpha_beta(ulp, D, T, tgt, U, blank, alpha, beta);
        /* reading: a NaN at the blank or a label column of an owned row makes the loss NaN */
        for (int64_t t = 0; t < T && !isnan(n); ++t)
            for (int64_t s = 0; s < S; ++s)
                if (isnan(ulp[t * D + ext_label(tgt, s, blank)])) { n = NAN; break; }
        nll[b] = n;
        if (grad && T > 0) {
            /* step 6: the gradient weight of this utterance */
            double w = grad_scale ? grad_scale[b] : 1.0;
            if (reduction == RED_MEAN) w /= (double)B * (double)(U > 1 ? U : 1);
            if (zero_infinity && isinf(n)) w = 0.0;
            for (int64_t t = 0; t < T; ++t) {
                const double* row = ulp + t * D;
                double* g = grad + (r + t) * D;
                if (w == 0.0) continue; /* reading: a zero weight gives zero rows (left as cleared) */
                for (int64_t c = 0; c < D; ++c) g[c] = w * exp(row[c]);
                if (isinf(n) || isnan(n)) { /* readings: no alignment, or a NaN the recursion reads */
                    for (int64_t c = 0; c < D; ++c) g[c] = NAN;
                    continue;
                }
                for (int64_t s = 0; s < S; ++s) {
                    const int64_t l = ext_label(tgt, s, blank);
                    double post = exp(alpha[t * S + s] + beta[t * S + s] - row[l] + n);
                    g[l] -= w * post;
                }
            }
        }
        free(alpha);
        free(beta);
    }
    if (failed) { free(nll); free(order); return ORACLE_ERR_ALLOC; }
    /* step 8 and 9 */
    double total = 0.0;
    for (int64_t b = 0; b < B; ++b) {
        double l = (zero_infinity && isinf(nll[b])) ? 0.0 : nll[b];
        if (nll_out) nll_out[b] = nll[b];
        if (loss_out) loss_out[b] = l;
        if (reduction == RED_MEAN) {
            int64_t U = target_lengths[b];
            total += l / (double)(U > 1 ? U : 1);
        } else {
            total += l;
        }
    }
    if (reduced_out) *reduced_out = (reduction == RED_MEAN) ? (B > 0 ? total / (double)B : NAN) : total;
    free(nll);
    free(order);
    return ORACLE_OK;
}

int ctc_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
