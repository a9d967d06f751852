// Adaptive draft depth (host arithmetic): the running per-draft acceptance estimate and the
// depth that maximises expected tokens per unit time at the measured pass times ("Decode is
// memory-bound ...", sections "Speculative decoding" (the expected tokens per pass tau and
// the speedup with a drafter cost) and "Two things the math says to do" (adapt the depth to
// the acceptance, and keep measuring it)).
#include <math.h>

#include "vq_internal.h"

namespace {

// Expected tokens per pass with k drafts at per-draft acceptance a.
double tau(double a, int k) {
    if (a == 1.0) return (double)(k + 1);
    return (1.0 - pow(a, (double)(k + 1))) / (1.0 - a);
}

}  // namespace

extern "C" {

int vq_depth_observe(vq_depth_stats* st, const int32_t* n_accepted, const int32_t* n_drafted, int32_t W,
                     double decay) {
    vq::clear_error();
    if (!st) return vq::fail(VQ_ERR_ARG, "NULL statistics");
    if (W < 0) return vq::fail(VQ_ERR_ARG, "W %d < 0", W);
    if (!(decay > 0.0 && decay <= 1.0)) return vq::fail(VQ_ERR_ARG, "decay must be in (0, 1]");
    if (W == 0) return VQ_OK;
    if (!n_accepted || !n_drafted) return vq::fail(VQ_ERR_ARG, "NULL window arrays");
    for (int32_t w = 0; w < W; ++w)
        if (n_drafted[w] < 0 || n_accepted[w] < 0 || n_accepted[w] > n_drafted[w])
            return vq::fail(VQ_ERR_ARG, "window %d: n_accepted %d outside [0, n_drafted %d]", w, n_accepted[w],
                            n_drafted[w]);
    double acc = st->accepted, rej = st->rejected;
    for (int32_t w = 0; w < W; ++w) {
        acc = decay * acc + (double)n_accepted[w];
        rej = decay * rej + (n_accepted[w] < n_drafted[w] ? 1.0 : 0.0);
    }
    st->accepted = acc;
    st->rejected = rej;
    return VQ_OK;
}

int vq_depth_choose(const vq_depth_stats* st, double alpha_prior, double prior_weight, const double* t_pass,
                    int32_t k_max, double t_draft, int32_t* k_out, double* alpha_out, double* rate_out) {
    vq::clear_error();
    if (!st || !t_pass || !k_out) return vq::fail(VQ_ERR_ARG, "NULL argument");
    if (k_max < 0 || k_max > VQ_MAX_K - 1) return vq::fail(VQ_ERR_ARG, "k_max %d outside 0..%d", k_max, VQ_MAX_K - 1);
    if (!(alpha_prior >= 0.0 && alpha_prior <= 1.0)) return vq::fail(VQ_ERR_ARG, "alpha_prior outside [0, 1]");
    if (!(prior_weight >= 0.0) || !isfinite(prior_weight)) return vq::fail(VQ_ERR_ARG, "prior_weight must be >= 0");
    if (!(t_draft >= 0.0) || !isfinite(t_draft)) return vq::fail(VQ_ERR_ARG, "t_draft must be finite and >= 0");
    for (int k = 0; k <= k_max; ++k)
        if (!(t_pass[k] > 0.0) || !isfinite(t_pass[k]))
            return vq::fail(VQ_ERR_ARG, "t_pass[%d] must be finite and > 0", k);
    if (!(st->accepted >= 0.0) || !(st->rejected >= 0.0)) return vq::fail(VQ_ERR_ARG, "negative statistics");
    const double n = st->accepted + st->rejected + prior_weight;
    if (!(n > 0.0)) return vq::fail(VQ_ERR_ARG, "no acceptance evidence and no prior weight");
    const double a = (st->accepted + prior_weight * alpha_prior) / n;
    int best = 0;
    double best_rate = tau(a, 0) / t_pass[0];
    for (int k = 1; k <= k_max; ++k) {
        const double r = tau(a, k) / (t_pass[k] + (double)k * t_draft);
        if (r > best_rate) {
            best = k;
            best_rate = r;
        }
    }
    *k_out = best;
    if (alpha_out) *alpha_out = a;
    if (rate_out) *rate_out = best_rate;
    return VQ_OK;
}

}  // extern "C"
