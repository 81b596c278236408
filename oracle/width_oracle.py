"""Adaptive verify width: a plain reference of the controller.  Test infrastructure: only
tests, the smoke check and the bench's CPU baseline may use it.

lucebox-hub PR "feat(qwen4exp): MTP speculative decoding", section "What": by default the
width is adaptive, up to seven drafts, chosen from the acceptance seen at each draft depth
and a per-request fit of the cycle's cost; width 1 is MTP off.  The page gives no
formulas; the reading taken here:
  * alpha[j] (j = 0..k_max-1): exponential moving average of "draft j+1 was accepted",
    updated only by cycles that reached draft j+1 (drafts 1..j accepted, j+1 drafted);
  * expected tokens of a cycle with k drafts: E(k) = 1 + sum_{i=1..k} prod_{j<i} alpha[j]
    (every accepted draft is a token, and the correction or bonus adds one);
  * cycle cost c(k) = c0 + c1 k, fitted by least squares to the measured cycle times with
    exponentially decaying weights; with fewer than two distinct widths observed the slope
    is a prior fraction of the intercept; a negative slope is taken as 0;
  * k* = argmax over 1 <= k <= k_max of E(k) / c(k), the smallest k on ties (widths the
    fit prices at <= 0 are skipped; if all are, k* = 1).
Outcomes that say nothing about the stopping draft (the block ended with EOS, or a target
row was unusable) update the depths before it only.
"""
from __future__ import annotations

import numpy as np

ACC_ALL_ACCEPTED = 0x01
ACC_EOS = 0x02
ACC_ROW_INVALID = 0x08


class WidthController:
    def __init__(self, k_max: int = 7, decay: float = 0.1, alpha0: float = 0.8, slope_prior: float = 0.1):
        assert 1 <= k_max <= 7 and 0.0 < decay <= 1.0 and 0.0 <= alpha0 <= 1.0 and slope_prior >= 0.0
        self.k_max, self.decay, self.slope_prior = k_max, decay, slope_prior
        self.alpha = [alpha0] * 7
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
            for j in range(a):                      # drafts 1..a were accepted
                self.alpha[j] += self.decay * (1.0 - self.alpha[j])
            if a < k and not (f & (ACC_EOS | ACC_ROW_INVALID | ACC_ALL_ACCEPTED)):
                self.alpha[a] += self.decay * (0.0 - self.alpha[a])   # draft a+1 was rejected
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

    def expected_tokens(self, k: int) -> float:
        e, run = 1.0, 1.0
        for j in range(k):
            run *= self.alpha[j]
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
