/*
 * Dense log-space HMM forward on MI355X (gfx950), in the same library as the packed CTC loss
 * (libpacked_ctc.so).
 *
 * Source of the method: the POPCORNBENCH page "HMM forward, Kimi-K2.6 l2_p50" (its problem
 * statement: the PyTorch HMM module with parameters log_init, log_trans, log_emit, and its forward).
 * The CTC alpha recursion of packed_ctc.h is the banded special case of this recursion.
 */
#ifndef HMM_FORWARD_H
#define HMM_FORWARD_H

#include <stddef.h>
#include <stdint.h>

#include "packed_ctc.h" /* error codes PCTC_*, packed_ctc_last_error */

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Log-likelihood of each observation sequence under an HMM ([HMM page] problem statement: the
 * module normalises its log weights by their log-sum-exp, then runs the log-space forward).
 *
 *   log_pi = log_init - logsumexp(log_init)                         (S,)
 *   log_A[i, :] = log_trans[i, :] - logsumexp(log_trans[i, :])      (S, S), row i = from state i
 *   log_B[s, :] = log_emit[s, :] - logsumexp(log_emit[s, :])        (S, O), row s = emissions of s
 *   alpha_0 = log_pi + log_B[:, o_0];  alpha_t[j] = logsumexp_i(alpha_{t-1}[i] + log_A[i, j]) + log_B[j, o_t]
 *   log_lik_out[b] = logsumexp_j alpha_{T-1}[j]    (natural log, float32; -inf if no path has mass)
 *
 * log_init, log_trans, log_emit: device float32, row-major, read only.  observations: device
 * (B, T) row-major, int32 (observations_i64 = 0) or int64 (1), symbols in [0, O) (a symbol outside
 * is a precondition violation: it is clamped so that every access stays in bounds, and that
 * sequence's result is unspecified).  log_lik_out: device (B,) float32, fully written.
 * Limits: 1 <= S <= 64, O >= 1, S * O <= 16384 (PCTC_ERR_LIMIT); T >= 1 when B > 0
 * (PCTC_ERR_SHAPE); B = 0 writes nothing.  Arithmetic in float32 (base-2 log space).
 * Asynchronous on `stream`; allocates nothing.  Returns PCTC_OK or an error code with a message in
 * packed_ctc_last_error().
 */
int hmm_forward_loglik(const float* log_init, const float* log_trans, const float* log_emit, const void* observations,
                       int observations_i64, int64_t B, int64_t T, int64_t S, int64_t O, float* log_lik_out,
                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HMM_FORWARD_H */
