"""Pins of the oracle's near-tie flags: which decisions the logit tolerance delta can turn.

The comparison excuses a decision of the GPU only where the oracle flags it, so each rule
is pinned against something other than its own code:
  * the tolerance of each score is the table below, written out per temperature (the
    literal reading: a top-2 or ratio-test margin within one logit tolerance, in the
    score's own units), checked at margins of (1 - 1e-3) and (1 + 1e-3) times it, at
    T = 0, 0.5, 1 and 2, for delta = 2e-2 (bf16, 4-bit) and 1e-4 (fp32);
  * for the residual pick, the shift of ln p(x) a logit tolerance can cause is measured on
    perturbed logits, and the flag is compared with a brute force over every extreme
    perturbation of ln p and ln q on small vocabularies;
  * planted mistakes (delta in place of delta/T, a residual shift ten times too wide, a
    ratio margin in logit units, a flagger that flags everything) each break a pin.
"""
import itertools

import numpy as np
import pytest
from scipy.special import logsumexp

from oracle import mtp_oracle as O

SEED, CYCLE = 4321, 9
# the tolerance of each kind of score, per temperature, for a logit tolerance delta
TOL_GUMBEL = {0.0: 1.0, 0.5: 2.0, 1.0: 1.0, 2.0: 0.5}   # x delta: argmax of z/T + Gumbel
TOL_RATIO = {0.5: 2.0, 1.0: 1.0, 2.0: 0.5}               # x delta: |ln u + ln q - ln p|
DELTAS = (2e-2, 1e-4)
REL = 1e-3


def _identity_head(n):
    """W = I: the logits of hidden row h are h itself, exactly."""
    return np.eye(n, dtype=np.float64)


def _scores_with_gap(n, top, second, gap, rng):
    """A score row whose best id is `top` and second-best `second`, gap apart; the other
    scores at least 3 below."""
    s = rng.uniform(-6.0, 2.0, size=n) - 3.0
    s[top] = 5.0
    s[second] = 5.0 - gap
    return s


# ----------------------------------------------------------------------------------
# argmax and Gumbel-max picks
# ----------------------------------------------------------------------------------
def _draft_cases(delta, T):
    """(gap, expected flag) pairs for one temperature."""
    tol = TOL_GUMBEL[T] * delta
    cases = [(tol * (1 - REL), True), (tol * (1 + REL), False), (0.0, True), (3 * tol, False)]
    if T == 0.5:
        cases.append((1.5 * delta, True))     # between delta and delta/T
    if T == 2.0:
        cases.append((0.75 * delta, False))   # between delta/T and delta
    return cases


def pin_draft_gaps():
    rng = np.random.default_rng(0)
    n = 12
    for delta in DELTAS:
        for T in TOL_GUMBEL:
            cases = _draft_cases(delta, T)
            B = len(cases)
            S = np.stack([_scores_with_gap(n, 3 + b % 5, 9 - b % 3, g, rng) for b, (g, _) in enumerate(cases)])
            if T > 0:
                # logits whose z/T + Gumbel are the scores
                G = O.gumbel_noise(SEED, O.STREAM_DRAFT, 2, np.arange(B), CYCLE, n)
                H = T * (S - G)
            else:
                H = S
            r = O.draft_rows(_identity_head(n), n, H, T, SEED, 2, CYCLE, delta)
            assert list(r["token"]) == [3 + b % 5 for b in range(B)], (delta, T, r["token"])
            want = np.array([f for _, f in cases])
            assert np.array_equal(r["near_tie"], want), (delta, T, [g for g, _ in cases], r["near_tie"], r["margin"])


def pin_verify_gaps():
    """Verify rows: the argmax of z is flagged at a gap of delta whatever T; the sample
    (stream 2, or the trunk's own position-keyed sample) at delta/T."""
    rng = np.random.default_rng(1)
    n, K1 = 10, 2
    for delta in DELTAS:
        for T in TOL_GUMBEL:
            cases = _draft_cases(delta, T)
            B = len(cases)
            for exact in (False, True):
                if exact and T == 0:
                    continue
                pos = rng.integers(0, 1000, size=B)
                # row 0 of request b: argmax gap in logit units; row 1: sample gap in score units
                zy = np.stack([_scores_with_gap(n, 2, 7, delta * (1 - REL) if b % 2 == 0 else delta * (1 + REL), rng)
                               for b in range(B)])
                S = np.stack([_scores_with_gap(n, 4, 8, g, rng) for g, _ in cases])
                if T > 0:
                    if exact:
                        G = np.stack([O.trunk_noise(SEED, b, int(pos[b]) + 1, n) for b in range(B)])
                    else:
                        G = O.gumbel_noise(SEED, O.STREAM_RESAMPLE, 1, np.arange(B), CYCLE, n)
                    zs = T * (S - G)
                else:
                    zs = S
                H = np.stack([zy, zs], axis=1)
                r = O.verify_rows(_identity_head(n), H, np.zeros((B, 1), np.int64), T, SEED, CYCLE, delta,
                                  positions=pos if exact else None)
                want_y = np.array([b % 2 == 0 for b in range(B)])
                assert np.array_equal(r["y_near_tie"][:, 0], want_y), (delta, T, exact, r["y_margin"][:, 0])
                assert np.array_equal(r["sample"][:, 1], np.full(B, 4)), (delta, T, exact)
                want_s = np.array([f for _, f in cases])
                assert np.array_equal(r["s_near_tie"][:, 1], want_s), (delta, T, exact, r["s_margin"][:, 1])


def test_draft_gap_boundaries():
    pin_draft_gaps()


def test_verify_gap_boundaries():
    pin_verify_gaps()


# ----------------------------------------------------------------------------------
# the ratio test, through the acceptance step
# ----------------------------------------------------------------------------------
def _softmax_logit_for(lp_target, others):
    """Logit a for which softmax([a] + others)[0] has log-probability lp_target."""
    s = logsumexp(others)
    return lp_target + s - np.log1p(-np.exp(lp_target))


def pin_ratio_margins():
    """One request per margin: draft t = 1 at row 0 with ln q(t) = -ln 3; ln p(t) chosen so
    that ln u + ln q(t) - ln p(t) is the margin.  Row 0's residual and row 1's bonus have
    one dominant id, so the ratio test is the only decision near a tie."""
    V, t = 4, 1
    for delta in DELTAS:
        for T in TOL_RATIO:
            tol = TOL_RATIO[T] * delta
            margins = [s * tol * f for s in (-1, 1) for f in (1 - REL, 1 + REL)] + [0.0, 4 * tol, -4 * tol]
            want = [abs(m) <= tol * (1 + REL / 2) for m in margins]
            if T == 0.5:
                margins += [1.5 * delta, -1.5 * delta]
                want += [True, True]
            if T == 2.0:
                margins += [0.75 * delta, -0.75 * delta]
                want += [False, False]
            B = len(margins)
            u = O.uniform_accept(O.philox_words(SEED, O.STREAM_ACCEPT, 0, np.arange(B), CYCLE, 0))
            zv = np.zeros((B, 2, V))
            zd = np.zeros((B, 1, V))
            for b, m in enumerate(margins):
                lq_t = -np.log(3.0)
                lp_t = np.log(u[b]) + lq_t - m
                # verify row 0: id 2 holds almost all of p (and none of q): a clear residual pick
                others = np.array([0.0, 40.0, 0.0])
                a = _softmax_logit_for(lp_t, others)
                zv[b, 0] = T * np.array([0.0, a, 40.0, 0.0])
                zd[b, 0] = T * np.array([0.0, 0.0, -40.0, 0.0])
                zv[b, 1] = T * np.array([0.0, 0.0, 0.0, 60.0])     # the bonus row: id 3
            drafts = np.full((B, 1), t)
            acc = O.accept(drafts, zd, zv, V, T, SEED, CYCLE, -1, delta)
            got = acc["tie_row"] == 0
            assert np.array_equal(got, np.array(want)), (delta, T, margins, got)
            # away from the boundary the decision is the exact comparison u*q <= p
            for b, m in enumerate(margins):
                if abs(m) > 2 * tol:
                    assert acc["n_accept"][b] == (1 if m < 0 else 0), (delta, T, m)


def test_ratio_margin_boundaries():
    pin_ratio_margins()


# ----------------------------------------------------------------------------------
# the residual pick
# ----------------------------------------------------------------------------------
@pytest.mark.parametrize("T", [0.5, 1.0, 2.0])
def test_logit_tolerance_moves_log_probabilities_by_at_most_twice_delta_over_t(T):
    """Logits each moved by at most delta move ln p(x) = z_x/T - lse(z/T) by at most
    2 delta/T, and that bound is reached (the residual flag's shift)."""
    delta = 2e-2
    rng = np.random.default_rng(7)
    eps = O.residual_logprob_shift(delta, T)
    worst = 0.0
    for _ in range(300):
        z = rng.standard_normal(50) * 2
        dz = rng.choice([-delta, delta], size=50) * rng.uniform(0.5, 1.0, size=50)
        lp = z / T - logsumexp(z / T)
        lp2 = (z + dz) / T - logsumexp((z + dz) / T)
        worst = max(worst, float(np.abs(lp2 - lp).max()))
    assert worst <= eps + 1e-12
    # a small p(x) whose logit drops while every other logit rises
    z = np.zeros(5000)
    z[0] = -5.0
    dz = np.full(5000, delta)
    dz[0] = -delta
    lp = z / T - logsumexp(z / T)
    lp2 = (z + dz) / T - logsumexp((z + dz) / T)
    assert abs(lp2[0] - lp[0]) >= 0.999 * eps
    assert abs(lp2[0] - lp[0]) <= eps + 1e-12


def _brute_force_flip(lp, lq, G, pick, eps):
    """Does some move of every ln p(x), ln q(x) by at most eps change the residual pick (or
    empty the residual)?  The score of x grows with ln p(x) and falls with ln q(x), so the
    extreme moves are the corners: every sign pattern is tried."""
    V = lp.size
    p, q = np.exp(lp), np.exp(lq)
    for signs in itertools.product((-1.0, 1.0), repeat=2 * V):
        a = np.array(signs[:V]) * eps
        b = np.array(signs[V:]) * eps
        r = np.maximum(0.0, p * np.exp(a) - q * np.exp(b))
        if not (r > 0).any():
            return True
        with np.errstate(divide="ignore"):
            s = np.log(r) + G
        if int(np.argmax(s)) != pick:
            return True
    return False


def _random_residual_case(rng, V):
    p = rng.dirichlet(np.full(V, 0.7))
    q = rng.dirichlet(np.full(V, 0.7))
    kind = rng.integers(0, 4)
    if kind == 1:                      # some ids outside the draft vocabulary
        q[rng.integers(0, V)] = 0.0
        q /= q.sum()
    elif kind == 2:                    # an id whose p and q nearly agree
        x = rng.integers(0, V)
        q[x] = p[x] * np.exp(rng.uniform(-0.1, 0.1))
    elif kind == 3:                    # p with a zero
        p[rng.integers(0, V)] = 0.0
        p /= p.sum()
    with np.errstate(divide="ignore"):
        return np.log(p), np.log(q)


@pytest.mark.parametrize("V", [3, 4])
def test_residual_flag_equals_brute_force_over_extreme_moves(V):
    rng = np.random.default_rng(100 + V)
    n_flag = n_clear = 0
    for _ in range(1500):
        lp, lq = _random_residual_case(rng, V)
        ln_r = O.residual_log_weights(lp, lq)
        if not (ln_r > -np.inf).any():
            continue
        G = -np.log(-np.log(rng.uniform(1e-9, 1.0, size=V)))
        pick = int(np.argmax(ln_r + G))
        delta, T = rng.choice([2e-2, 1e-3, 0.1]), rng.choice([0.5, 1.0, 2.0])
        eps = 2 * delta / T
        want = _brute_force_flip(lp, lq, G, pick, eps)
        got = bool(O.residual_near_tie(lp[None], lq[None], G[None], np.array([pick]), delta, T)[0])
        assert got == want, (lp, lq, G, pick, eps)
        n_flag += want
        n_clear += not want
    assert n_flag > 50 and n_clear > 50


def test_residual_flag_is_not_limited_to_the_runner_up():
    """A third id whose p and q nearly agree has almost no residual now, but a small move
    can give it a large one: the pick is flagged although the runner-up is far behind."""
    delta, T = 2e-2, 1.0
    lp = np.log(np.array([0.30, 0.05, 0.65]))
    lq = np.log(np.array([0.05, 0.04, 0.91]))
    lq[2] = lp[2] + 0.001                      # r(2) = 0, but up to ~0.05 after a move
    G = np.array([0.0, 0.0, 2.0])
    ln_r = O.residual_log_weights(lp, lq)
    pick = int(np.argmax(ln_r + G))
    assert pick == 0 and ln_r[0] + G[0] - (ln_r[1] + G[1]) > 1.0
    assert O.residual_near_tie(lp[None], lq[None], G[None], np.array([pick]), delta, T)[0]
    assert _brute_force_flip(lp, lq, G, pick, O.residual_logprob_shift(delta, T))
    # the same case with id 2 clearly over-drafted is clear
    lq[2] = lp[2] + 1.0
    assert not O.residual_near_tie(lp[None], lq[None], G[None], np.array([pick]), delta, T)[0]


def test_empty_residual_flagged_when_a_move_can_give_it_mass():
    delta, T = 2e-2, 1.0
    lp = np.log(np.array([0.5, 0.5]))
    assert O.empty_residual_near_tie(lp[None], lp[None], delta, T)[0]           # p = q
    lq = np.log(np.array([0.5 * np.exp(0.2), 0.5 * np.exp(0.2)]))              # q above p by 0.2 everywhere
    assert not O.empty_residual_near_tie(lp[None], lq[None], delta, T)[0]


def pin_residual_boundary():
    """Through the acceptance step: ids outside the draft vocabulary (q = 0) have r = p, so
    each score may move by eps = 2 delta/T and the pick is flagged at a gap of 4 delta/T."""
    V, nd = 6, 2
    for delta in DELTAS:
        for T in (0.5, 1.0, 2.0):
            tol = 4 * delta / T
            gaps = [tol * (1 - REL), tol * (1 + REL), 0.5 * tol, 2 * tol]
            want = [True, False, True, False]
            B = len(gaps)
            G = O.gumbel_noise(SEED, O.STREAM_RESAMPLE, 0, np.arange(B), CYCLE, V)
            zv = np.zeros((B, 2, V))
            zd = np.zeros((B, 1, nd))
            for b, gap in enumerate(gaps):
                # residual scores ln p(x) + G(x) for ids 2..5 (q = 0 there); id 0 has p = 0
                s = np.array([-np.inf, -30.0, 1.0, 1.0 - gap, -6.0, -7.0])
                lp = s - G[b]
                lp[0] = -np.inf
                lp -= logsumexp(lp)
                zv[b, 0] = T * lp
                zv[b, 1] = T * np.array([0.0, 0.0, 0.0, 0.0, 0.0, 60.0])
                zd[b, 0] = T * np.log(np.array([0.5, 0.5]))
            drafts = np.zeros((B, 1), np.int64)           # p(0) = 0: always rejected
            acc = O.accept(drafts, zd, zv, nd, T, SEED, CYCLE, -1, delta)
            assert np.all(acc["n_accept"] == 0) and np.all(acc["tokens"][:, 0] == 2), acc["tokens"]
            got = acc["tie_row"] == 0
            assert np.array_equal(got, np.array(want)), (delta, T, gaps, got)


def test_residual_pick_boundary_through_acceptance():
    pin_residual_boundary()


# ----------------------------------------------------------------------------------
# planted mistakes in the flagger break the pins
# ----------------------------------------------------------------------------------
def test_planted_delta_in_place_of_delta_over_t_is_caught(monkeypatch):
    monkeypatch.setattr(O, "score_tolerance", lambda delta, T: delta)
    with pytest.raises(AssertionError):
        pin_draft_gaps()
    with pytest.raises(AssertionError):
        pin_verify_gaps()


def test_planted_ratio_margin_in_logit_units_is_caught(monkeypatch):
    real = O.ratio_near_tie
    monkeypatch.setattr(O, "ratio_near_tie", lambda m, delta, T: real(m, delta * T, T))
    with pytest.raises(AssertionError):
        pin_ratio_margins()


def test_planted_wide_residual_shift_is_caught(monkeypatch):
    real = O.residual_logprob_shift
    monkeypatch.setattr(O, "residual_logprob_shift", lambda delta, T: 10 * real(delta, T))
    with pytest.raises(AssertionError):
        pin_residual_boundary()


def test_planted_residual_shift_without_the_normaliser_is_caught(monkeypatch):
    monkeypatch.setattr(O, "residual_logprob_shift", lambda delta, T: delta / T)
    with pytest.raises(AssertionError):
        pin_residual_boundary()


def test_planted_flag_everything_is_caught(monkeypatch):
    monkeypatch.setattr(O, "gap_near_tie", lambda gap, tol: np.ones(np.shape(gap), dtype=bool))
    with pytest.raises(AssertionError):
        pin_draft_gaps()
    monkeypatch.undo()
    monkeypatch.setattr(O, "ratio_near_tie", lambda m, delta, T: np.ones(np.shape(m), dtype=bool))
    with pytest.raises(AssertionError):
        pin_ratio_margins()
    monkeypatch.undo()
    monkeypatch.setattr(O, "residual_near_tie", lambda lp, lq, G, pick, delta, T: np.ones(len(pick), dtype=bool))
    with pytest.raises(AssertionError):
        pin_residual_boundary()


def test_rows_holding_plus_inf_take_their_lowest_plus_inf_id_without_a_flag():
    """Sanitised +inf ids are all exactly 0: the argmax among them is the lowest id by an
    exact rule (no finite logit, so nothing the tolerance can move), while a finite row
    with the same two best values tied is flagged."""
    n = 6
    h = np.array([[0.5, 3.0, -1.0, 3.0, 0.0, 2.0]])
    W_inf = _identity_head(n)
    W_inf[1, 0] = W_inf[3, 0] = np.inf          # logits 1 and 3 are +inf
    for W, flagged in ((W_inf, False), (_identity_head(n), True)):
        r = O.draft_rows(W, n, h, 0.0, SEED, 0, CYCLE, 2e-2)
        assert list(r["token"]) == [1] and list(r["near_tie"]) == [flagged]
        v = O.verify_rows(W, h[:, None, :], np.zeros((1, 0), np.int64), 0.0, SEED, CYCLE, 2e-2)
        assert list(v["argmax"][:, 0]) == [1] and list(v["y_near_tie"][:, 0]) == [flagged]
