"""Adaptive verify width: a plain reference of the controller.  Test infrastructure: only
tests, the smoke check and the bench's CPU baseline may use it.

lucebox-hub PR "feat(qwen4exp): MTP speculative decoding", section "What": by default the
width is adaptive, up to seven drafts, chosen from the acceptance seen at each draft depth
and a per-request fit of the cycle's cost; width 1 is MTP off.  The page gives no
formulas; the reading taken here:
  * alpha[j] (j = 0..6): exponential moving average (weight ``decay``) of "draft j+1 was
    accepted", updated only by cycles that decided draft j+1: drafts 1..j accepted and
    draft j+1 accepted (an accepted EOS draft included) or rejected.  A block that ended
    at an unusable target row, or a full accept (no draft j+1 beyond k), decides nothing
    at its stopping depth; an EOS correction after a rejection is a rejection;
  * w[j]: how recently depth j was decided -- every request-cycle multiplies all w by
    (1 - decay) and adds 1 at each depth it decided;
  * exploration: a depth decided too rarely to be current (w[j] < 1/2) is estimated by
    the depth before it, a[j] = a[j-1] (a[0] = alpha[0]); acceptance seldom rises with
    depth, so this is an optimistic estimate for depths the current width never reaches,
    and a rise in acceptance at the shallow depths makes the controller try deeper drafts,
    which then measure their own rate;
  * expected tokens of a cycle with k drafts: E(k) = 1 + sum_{i=1..k} prod_{j<i} a[j]
    (every accepted draft is a token, and the correction or bonus adds one);
  * cycle cost c(k) = c0 + c1 k, fitted by least squares to the measured cycle times with
    exponentially decaying weights; with fewer than two distinct widths observed the slope
    is a prior fraction of the intercept; a negative slope is taken as 0;
  * k* = argmax over 1 <= k <= k_max of E(k) / c(k), the smallest k on ties (widths the
    fit prices at <= 0 are skipped; if all are, k* = 1).
"""
from __future__ import annotations

import numpy as np

ACC_ALL_ACCEPTED = 0x01
ACC_EOS = 0x02
ACC_ROW_INVALID = 0x08
ACC_EOS_DRAFT = 0x80
STALE_WEIGHT = 0.5      # depths with w[j] below this take the estimate of depth j - 1


class WidthController:
    def __init__(self, k_max: int = 7, decay: float = 0.1, alpha0: float = 0.8, slope_prior: float = 0.1):
        assert 1 <= k_max <= 7 and 0.0 < decay <= 1.0 and 0.0 <= alpha0 <= 1.0 and slope_prior >= 0.0
        self.k_max, self.decay, self.slope_prior = k_max, decay, slope_prior
        self.alpha = [alpha0] * 7
        self.weight = [0.0] * 7
        self.sw = self.sk = self.skk = self.st = self.skt = 0.0
        self.verifier_passes = self.cycles = self.drafted = self.accepted = 0
        self.depth_hist = [0] * 8

    def observe(self, k: int, n_accept, flags, seconds: float) -> None:
        """One verify pass of len(n_accept) requests, each with k drafts; the pass took
        ``seconds`` (<= 0: no timing)."""
        self.verifier_passes += 1
        for a, f in zip(n_accept, flags):
            a, f = int(a), int(f)
            self.cycles += 1
            self.drafted += k
            self.accepted += a
            self.depth_hist[a] += 1
            self.weight = [(1.0 - self.decay) * x for x in self.weight]
            accepted = a + 1 if (a < k and f & ACC_EOS_DRAFT) else a   # an accepted EOS draft
            for j in range(accepted):                                 # drafts 1..accepted
                self.alpha[j] += self.decay * (1.0 - self.alpha[j])
                self.weight[j] += 1.0
            if accepted == a and a < k and not (f & (ACC_ROW_INVALID | ACC_ALL_ACCEPTED)):
                self.alpha[a] += self.decay * (0.0 - self.alpha[a])   # draft a+1 was rejected
                self.weight[a] += 1.0
        if seconds > 0.0:
            g = 1.0 - self.decay
            self.sw = g * self.sw + 1.0
            self.sk = g * self.sk + k
            self.skk = g * self.skk + k * k
            self.st = g * self.st + seconds
            self.skt = g * self.skt + k * seconds

    def cost_params(self):
        if self.sw <= 0.0:
            return 1.0, self.slope_prior
        den = self.sw * self.skk - self.sk * self.sk
        if den > 1e-9 * self.sw * self.sw:
            c1 = (self.sw * self.skt - self.sk * self.st) / den
            c1 = max(c1, 0.0)
            c0 = (self.st - c1 * self.sk) / self.sw
        else:
            kbar = self.sk / self.sw
            c0 = (self.st / self.sw) / (1.0 + self.slope_prior * kbar)
            c1 = self.slope_prior * c0
        return c0, c1

    def cost(self, k: int) -> float:
        c0, c1 = self.cost_params()
        return c0 + c1 * k

    def estimates(self):
        """Per-depth acceptance used for E(k): alpha[j], or the estimate of depth j - 1
        where depth j is not current."""
        est = [self.alpha[0]]
        for j in range(1, 7):
            est.append(self.alpha[j] if self.weight[j] >= STALE_WEIGHT else est[j - 1])
        return est

    def expected_tokens(self, k: int) -> float:
        e, run = 1.0, 1.0
        est = self.estimates()
        for j in range(k):
            run *= est[j]
            e += run
        return e

    def choose(self) -> int:
        best, best_k = -np.inf, 1
        for k in range(1, self.k_max + 1):
            c = self.cost(k)
            if not c > 0.0:
                continue                           # an inconsistent fit: skip widths it prices at <= 0
            v = self.expected_tokens(k) / c
            if v > best:
                best, best_k = v, k
        return best_k
