// Draft-cap policy from the measured verify-cost curve (host code, no GPU).
//
// "mlx-dspark" wiki summary, "Key techniques" (hardware-aware
// auto-calibration) and "Design decisions" (calibrate once, cache on disk);
// "mlx-dspark 0.7.0", "Tuning" (--max-draft auto) and "The Apple-Silicon
// speedup ceiling": a round that drafts c tokens commits 1 + sum_{i=1..c}
// alpha^i tokens in expectation (alpha = per-position acceptance) and costs
// one verify pass at width c + 1 plus the drafter's work, so the cap to use
// is the c with the most expected tokens per unit time; when no c beats
// plain decoding (c = 0), speculation parks and only an occasional probe
// round keeps the acceptance estimate alive.
#include <math.h>

#include "../../include/dspk.h"

namespace {

// Expected committed tokens of a round that drafts c tokens: sum_{i=0..c} alpha^i.
double expected_tokens(int c, double alpha) {
    double e = 0.0, a = 1.0;
    for (int i = 0; i <= c; ++i) {
        e += a;
        a *= alpha;
    }
    return e;
}

bool valid_curve(const double *verify_us, const double *draft_us, int32_t n) {
    if (verify_us == nullptr || n < 1 || n > DSPK_MAX_ROWS) return false;
    for (int i = 0; i < n; ++i) {
        if (!(verify_us[i] > 0.0) || !isfinite(verify_us[i])) return false;
        if (draft_us != nullptr && (!(draft_us[i] >= 0.0) || !isfinite(draft_us[i]))) return false;
    }
    return true;
}

}  // namespace

extern "C" {

int32_t dspk_choose_cap(const double *verify_us, const double *draft_us, int32_t n, double alpha,
                        double *tokens_per_us) {
    if (!valid_curve(verify_us, draft_us, n) || !(alpha >= 0.0 && alpha <= 1.0)) return DSPK_EINVAL;
    // Verify cost of width c + 1: the least measured cost at that width or
    // wider, since a narrower pass can always run as a wider one with padding
    // rows (so noise cannot make a longer cap look cheaper than a shorter one).
    double envelope[DSPK_MAX_ROWS];
    envelope[n - 1] = verify_us[n - 1];
    for (int c = n - 2; c >= 0; --c) envelope[c] = fmin(verify_us[c], envelope[c + 1]);
    int best = 0;
    double best_rate = 0.0;
    for (int c = 0; c < n; ++c) {
        const double cost = envelope[c] + (c > 0 && draft_us != nullptr ? draft_us[c] : 0.0);
        const double rate = expected_tokens(c, alpha) / cost;
        if (c == 0 || rate > best_rate) {   // ties keep the smaller cap
            best = c;
            best_rate = rate;
        }
    }
    if (tokens_per_us != nullptr) *tokens_per_us = best_rate;
    return best;
}

int dspk_cap_init(dspk_cap_controller *ctl, const double *verify_us, const double *draft_us, int32_t n,
                  double decay, double prior_alpha, int32_t probe_every, int32_t probe_cap) {
    if (ctl == nullptr || !valid_curve(verify_us, draft_us, n)) return DSPK_EINVAL;
    if (!(decay > 0.0 && decay <= 1.0) || !(prior_alpha >= 0.0 && prior_alpha <= 1.0)) return DSPK_EINVAL;
    if (probe_every < 1 || probe_cap < 1 || probe_cap >= n) return DSPK_EINVAL;
    for (int i = 0; i < DSPK_MAX_ROWS; ++i) {
        ctl->verify_us[i] = i < n ? verify_us[i] : 0.0;
        ctl->draft_us[i] = (i < n && draft_us != nullptr) ? draft_us[i] : 0.0;
    }
    ctl->n = n;
    ctl->decay = decay;
    // the prior counts as one position's worth of evidence
    ctl->hits = prior_alpha;
    ctl->trials = 1.0;
    ctl->probe_every = probe_every;
    ctl->probe_cap = probe_cap;
    ctl->parked_rounds = 0;
    return DSPK_OK;
}

double dspk_cap_alpha(const dspk_cap_controller *ctl) {
    if (ctl == nullptr || !(ctl->trials > 0.0)) return 0.0;
    return ctl->hits / ctl->trials;
}

int dspk_cap_observe(dspk_cap_controller *ctl, int32_t drafted, int32_t accepted) {
    if (ctl == nullptr || drafted < 0 || accepted < 0 || accepted > drafted) return DSPK_EINVAL;
    if (drafted == 0) return DSPK_OK;   // a parked round says nothing about acceptance
    // positions tested: the accepted ones plus the first reject, if any
    const double trials = accepted + (accepted < drafted ? 1 : 0);
    ctl->hits = ctl->decay * ctl->hits + accepted;
    ctl->trials = ctl->decay * ctl->trials + trials;
    return DSPK_OK;
}

int32_t dspk_cap_next(dspk_cap_controller *ctl) {
    if (ctl == nullptr) return DSPK_EINVAL;
    const int32_t cap = dspk_choose_cap(ctl->verify_us, ctl->draft_us, ctl->n, dspk_cap_alpha(ctl), nullptr);
    if (cap > 0) {
        ctl->parked_rounds = 0;
        return cap;
    }
    // parked: plain steps, and every probe_every-th round a short probe
    ctl->parked_rounds += 1;
    if (ctl->parked_rounds >= ctl->probe_every) {
        ctl->parked_rounds = 0;
        return ctl->probe_cap;
    }
    return 0;
}

}  // extern "C"
