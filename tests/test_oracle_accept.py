"""Pins of the oracle's acceptance / residual / EOS logic.

  * closed form: one speculative step emits exactly p (hand-set dyadic p, q; exact
    count of accepting uniforms on the 2^-24 grid; residual weights vs max(0, p - q));
  * Monte Carlo chi-square: every emitted position follows the target row's p, and two
    planted mistakes (no residual; argmax drafts under ratio acceptance) are caught;
  * rejection, EOS and an unusable target row at every position;
  * special cases: q = p accepts every draft; T -> 0+ equals greedy; q(t) = 0 < p(t)
    accepts, p(t) = 0 rejects; determinism of seeded sampling.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy import stats

import synth
from oracle import mtp_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))
GRID = 1 << 24


def _log(p):
    with np.errstate(divide="ignore"):
        return np.log(np.asarray(p, dtype=np.float64))


def _accept_count(lp_t, lq_t):
    """Number of u = j * 2^-24 (j = 1..2^24) that the oracle's ratio test accepts."""
    def acc(j):
        return bool(O.accept_test(np.array(lp_t), np.array(lq_t), np.array(j * 2.0 ** -24)))
    if not acc(1):
        return 0
    lo, hi = 1, GRID
    if acc(hi):
        return GRID
    while hi - lo > 1:               # the test is monotone in u
        mid = (lo + hi) // 2
        if acc(mid):
            lo = mid
        else:
            hi = mid
    return lo


def _emission_law(p, q):
    lp, lq = _log(p), _log(q)
    V = len(p)
    acc = [Fraction(_accept_count(lp[t], lq[t]), GRID) if q[t] > 0 else Fraction(0) for t in range(V)]
    ln_r = O.residual_log_weights(lp, lq)
    r = np.exp(ln_r)
    reject_mass = sum(Fraction(q[t]) * (1 - acc[t]) for t in range(V))
    law = []
    for x in range(V):
        e = Fraction(q[x]) * acc[x]
        if reject_mass > 0:
            if r.sum() > 0:
                e += reject_mass * Fraction(float(r[x] / r.sum()))
            else:
                e += reject_mass * Fraction(p[x])        # empty residual: draw from p
        law.append(e)
    return law, acc, r


CASES = json.load(open(os.path.join(HERE, "golden", "closed_form_cases.json")))["cases"]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_one_step_emits_exactly_p(case):
    p, q = CASES[case]["p"], CASES[case]["q"]
    law, acc, r = _emission_law(p, q)
    for x in range(len(p)):
        assert abs(float(law[x]) - p[x]) <= 1e-6, (x, float(law[x]), p[x])
    for t in range(len(p)):
        if q[t] > 0:
            assert abs(float(acc[t]) - min(1.0, p[t] / q[t])) <= 2.0 ** -20
    want_r = np.maximum(0.0, np.asarray(p) - np.asarray(q))
    assert np.allclose(r, want_r, rtol=1e-12, atol=0)


def test_planted_mistakes_break_the_closed_form(monkeypatch):
    p, q = CASES[0]["p"], CASES[0]["q"]
    # mistake 1: resample from p instead of the residual
    monkeypatch.setattr(O, "residual_log_weights", lambda lp, lq: lp)
    law, _, _ = _emission_law(p, q)
    assert max(abs(float(law[x]) - p[x]) for x in range(8)) > 0.01
    monkeypatch.undo()
    # mistake 2: residual max(0, q - p) (operands swapped)
    real = O.residual_log_weights
    monkeypatch.setattr(O, "residual_log_weights", lambda lp, lq: real(lq, lp))
    law, _, _ = _emission_law(p, q)
    assert max(abs(float(law[x]) - p[x]) for x in range(8)) > 0.01
    monkeypatch.undo()
    # mistake 3: ratio test with the inequality reversed (q * u >= p)
    monkeypatch.setattr(O, "accept_test",
                        lambda lp, lq, u: (np.asarray(lp) > -np.inf) & (np.log(u) + lq >= lp))
    law, _, _ = _emission_law(p, q)
    assert max(abs(float(law[x]) - p[x]) for x in range(8)) > 0.01


# ---------------------------------------------------------------------------------
# Monte Carlo: identity head, fixed per-row logits
# ---------------------------------------------------------------------------------
V_MC, ND_MC, K_MC = 16, 8, 3


def _mc_rows(seed=21):
    rng = np.random.default_rng(seed)
    h_v = rng.standard_normal((K_MC + 1, V_MC)) * 1.2
    h_d = rng.standard_normal((K_MC, V_MC)) * 1.2
    h_d[:, :ND_MC] += 0.6 * h_v[:K_MC, :ND_MC]     # partly agreeing draft, as an MTP head would
    return h_v, h_d


def _run_mc(n, drafts_fn=None, cycle_id=0):
    W = O.head_weights_f64(synth.identity_head(V_MC))
    h_v, h_d = _mc_rows()
    Hv = np.broadcast_to(h_v, (n, K_MC + 1, V_MC)).copy()
    Hd = np.broadcast_to(h_d, (n, K_MC, V_MC)).copy()
    drafts = None if drafts_fn is None else drafts_fn(h_d, n)
    out = O.cycle(W, ND_MC, Hd, Hv, 1.0, 1234, cycle_id, -1, 1e-4, drafts=drafts)
    return out, h_v, h_d


def _softmax(z):
    e = np.exp(z - z.max())
    return e / e.sum()


def _position_pvalues(acc, h_v):
    pvals = []
    for i in range(K_MC + 1):
        reach = acc["n_accept"] >= i
        tok = acc["tokens"][reach, i]
        p = _softmax(h_v[i])
        counts = np.bincount(tok, minlength=V_MC)
        pvals.append(stats.chisquare(counts, counts.sum() * p).pvalue)
    return pvals


@pytest.mark.slow
def test_monte_carlo_every_position_follows_p():
    n = 200_000
    out, h_v, h_d = _run_mc(n)
    acc = out["accept"]
    # invariants
    assert np.all((acc["n_accept"] >= 0) & (acc["n_accept"] <= K_MC))
    assert np.array_equal(acc["n_emit"], acc["n_accept"] + 1)
    for i in range(K_MC):
        m = acc["n_accept"] > i
        assert np.array_equal(acc["tokens"][m, i], out["drafts"][m, i])
    pv = _position_pvalues(acc, h_v)
    assert min(pv) >= 1e-4 / (K_MC + 1), pv
    # acceptance rate at row i -> sum_x min(p_i, q_i)
    for i in range(K_MC):
        p = _softmax(h_v[i])
        q = np.zeros(V_MC)
        q[:ND_MC] = _softmax(h_d[i][:ND_MC])
        reach = acc["n_accept"] >= i
        rate = np.mean(acc["n_accept"][reach] > i)
        want = np.minimum(p, q).sum()
        assert abs(rate - want) < 5 * np.sqrt(want * (1 - want) / reach.sum()) + 1e-3


@pytest.mark.slow
def test_monte_carlo_negative_controls(monkeypatch):
    n = 100_000
    # no residual: resample from p at the first rejection
    monkeypatch.setattr(O, "residual_log_weights", lambda lp, lq: lp)
    out, h_v, _ = _run_mc(n)
    assert min(_position_pvalues(out["accept"], h_v)) < 1e-6
    monkeypatch.undo()
    # drafts are the argmax of q, but ratio acceptance assumes they are samples of q
    out, h_v, _ = _run_mc(n, drafts_fn=lambda h_d, m: np.broadcast_to(
        np.argmax(h_d[:, :ND_MC], axis=1), (m, K_MC)).copy())
    assert min(_position_pvalues(out["accept"], h_v)) < 1e-6


# ---------------------------------------------------------------------------------
# rejection / EOS / invalid rows at every position
# ---------------------------------------------------------------------------------
def _planted_logits(rng, K1, V, tops):
    z = rng.standard_normal((1, K1, V))
    for i, t in enumerate(tops):
        z[0, i, t] = 20.0
    return z


@pytest.mark.parametrize("j", range(8))
def test_greedy_rejection_at_every_position(j):
    rng = np.random.default_rng(j)
    k, V = 7, 40
    y = rng.integers(0, V, size=k + 1)
    zv = _planted_logits(rng, k + 1, V, y)
    drafts = y[:k].copy()[None, :]
    if j < k:
        drafts[0, j] = (y[j] + 1) % V
    r = O.accept(drafts, None, zv, V, 0.0, 0, 0, -1, 1e-4)
    assert r["n_accept"][0] == j and r["n_emit"][0] == j + 1
    assert list(r["tokens"][0, :j + 1]) == list(y[:j + 1])
    assert np.all(r["tokens"][0, j + 1:] == -1)
    assert bool(r["flags"][0] & O.ACC_ALL_ACCEPTED) == (j == k)


@pytest.mark.parametrize("j", range(7))
@pytest.mark.parametrize("as_correction", [False, True])
def test_greedy_eos_at_every_position(j, as_correction):
    rng = np.random.default_rng(100 + j)
    k, V, eos = 7, 40, 2
    y = rng.integers(3, V, size=k + 1)
    y[j] = eos
    zv = _planted_logits(rng, k + 1, V, y)
    drafts = y[:k].copy()[None, :]
    if as_correction:
        drafts[0, j] = 7 if y[j] != 7 else 8
    drafts[0, j + 1:] = eos                 # later drafts must never be emitted
    r = O.accept(drafts, None, zv, V, 0.0, 0, 0, eos, 1e-4)
    assert r["n_accept"][0] == j and r["n_emit"][0] == j + 1
    assert list(r["tokens"][0, :j + 1]) == list(y[:j]) + [eos]
    assert np.all(r["tokens"][0, j + 1:] == -1)
    assert r["flags"][0] & O.ACC_EOS


def _peaked(V, top, scale=40.0):
    z = np.full(V, -scale)
    z[top] = scale
    return z


@pytest.mark.parametrize("j", range(4))
def test_sampled_rejection_and_eos_at_every_position(j):
    k, V, nd, eos = 3, 12, 8, 2
    drafts = np.array([[4, 5, 6]])
    zd = np.stack([_peaked(nd, t) for t in drafts[0]])[None]
    zv = np.stack([_peaked(V, t) for t in list(drafts[0]) + [9]])[None]
    if j < k:
        zv[0, j] = _peaked(V, 10)         # p_j(draft) ~ 0: rejected, residual ~ one-hot on 10
    n = 64
    r = O.accept(np.repeat(drafts, n, 0), np.repeat(zd, n, 0), np.repeat(zv, n, 0), nd, 1.0,
                 77, 0, eos, 1e-4)
    assert np.all(r["n_accept"] == j)
    want_last = 10 if j < k else 9
    assert np.all(r["tokens"][:, j] == want_last)
    # EOS drafted and accepted at position j ends the block there
    if j < k:
        d2 = drafts.copy()
        d2[0, j] = eos
        zd2 = zd.copy()
        zd2[0, j] = _peaked(nd, eos)
        zv2 = np.stack([_peaked(V, t) for t in list(d2[0]) + [9]])[None]
        r2 = O.accept(np.repeat(d2, n, 0), np.repeat(zd2, n, 0), np.repeat(zv2, n, 0), nd, 1.0,
                      77, 0, eos, 1e-4)
        assert np.all(r2["n_accept"] == j) and np.all(r2["n_emit"] == j + 1)
        assert np.all(r2["tokens"][:, j] == eos) and np.all(r2["flags"] & O.ACC_EOS)


@pytest.mark.parametrize("T", [0.0, 1.0])
@pytest.mark.parametrize("j", range(4))
def test_invalid_target_row_stops_before_it(T, j):
    k, V, nd = 3, 12, 8
    drafts = np.array([[1, 2, 3]])
    zv = np.stack([_peaked(V, t) for t in [1, 2, 3, 4]])[None]
    zd = np.stack([_peaked(nd, t) for t in [1, 2, 3]])[None]
    zv[0, j] = np.nan
    r = O.accept(drafts, zd, zv, nd, T, 5, 0, -1, 1e-4)
    assert r["n_accept"][0] == j and r["n_emit"][0] == j
    assert r["flags"][0] & O.ACC_ROW_INVALID
    assert list(r["tokens"][0, :j]) == [1, 2, 3][:j] and np.all(r["tokens"][0, j:] == -1)


def test_all_minus_inf_draft_row_is_rejected_and_resampled_from_p():
    k, V, nd = 1, 6, 4
    zd = np.full((1, 1, nd), -np.inf)
    zv = np.log(np.array([[[0.5, 0.5, 0, 0, 0, 0], [1, 0, 0, 0, 0, 0]]]) + 0.0)
    n = 4000
    r = O.accept(np.full((n, 1), -1), np.repeat(zd, n, 0), np.repeat(zv, n, 0), nd, 1.0, 3, 0, -1, 1e-4,
                 b_ids=np.arange(n))
    assert np.all(r["n_accept"] == 0) and np.all(r["flags"] & O.ACC_DRAFT_INVALID)
    c = np.bincount(r["tokens"][:, 0], minlength=V)
    assert c[2:].sum() == 0 and stats.binomtest(int(c[0]), n, 0.5).pvalue > 1e-4


def test_q_zero_accepts_and_p_zero_rejects():
    V, nd = 8, 4
    zv = np.log(np.array([[[0.1, 0.2, 0.3, 0.0, 0.1, 0.3, 0.0, 0.0], [1, 0, 0, 0, 0, 0, 0, 0]]]) + 0.0)
    zd = np.log(np.array([[[0.25, 0.25, 0.25, 0.25]]]))
    n = 500
    # draft 5 lies outside the draft vocabulary: q(5) = 0 < p(5) -> always accepted
    r = O.accept(np.full((n, 1), 5), np.repeat(zd, n, 0), np.repeat(zv, n, 0), nd, 1.0, 1, 0, -1, 1e-4,
                 b_ids=np.arange(n))
    assert np.all(r["n_accept"] == 1)
    # draft 3: p(3) = 0 -> always rejected, even though q(3) > 0
    r = O.accept(np.full((n, 1), 3), np.repeat(zd, n, 0), np.repeat(zv, n, 0), nd, 1.0, 1, 0, -1, 1e-4,
                 b_ids=np.arange(n))
    assert np.all(r["n_accept"] == 0) and np.all(r["tokens"][:, 0] != 3)


def test_draft_equal_target_accepts_every_draft():
    # n_draft = V and the draft hidden equals the verify hidden: q = p, so u*q <= p always
    rng = np.random.default_rng(8)
    V, d, k, B = 64, 16, 3, 200
    W = rng.standard_normal((V, d))
    hv = rng.standard_normal((B, k + 1, d))
    hd = hv[:, :k].copy()
    out = O.cycle(W, V, hd, hv, 1.0, 99, 0, -1, 1e-4)
    assert np.all(out["accept"]["n_accept"] == k)
    assert np.all(out["accept"]["flags"] & O.ACC_ALL_ACCEPTED)


def test_small_temperature_equals_greedy():
    rng = np.random.default_rng(9)
    V, k, B = 32, 3, 50
    W = np.eye(V)
    # logits on a grid with gaps >= 1: at T = 1e-3 every softmax is one-hot to fp64 precision
    hv = rng.permutation(np.tile(np.arange(V, dtype=float), (B * (k + 1), 1)).T).T.reshape(B, k + 1, V)
    hd = hv[:, :k].copy()
    hd[:, 1] = rng.permutation(np.tile(np.arange(V, dtype=float), (B, 1)).T).T
    g = O.cycle(W, V, hd, hv, 0.0, 0, 0, -1, 1e-4)["accept"]
    s = O.cycle(W, V, hd, hv, 1e-3, 5, 0, -1, 1e-4)["accept"]
    assert np.array_equal(g["tokens"], s["tokens"]) and np.array_equal(g["n_accept"], s["n_accept"])


def test_seeded_sampling_is_deterministic_and_cycle_keyed():
    rng = np.random.default_rng(10)
    head = synth.make_head(rng, 512, 32, "f32")
    hv, hd = synth.make_hidden(rng, 4, 3, 32)
    W = O.head_weights_f64(head)
    a = O.cycle(W, 128, hd.astype(float), hv.astype(float), 1.0, 1234, 0, 2, 1e-4)
    b = O.cycle(W, 128, hd.astype(float), hv.astype(float), 1.0, 1234, 0, 2, 1e-4)
    c = O.cycle(W, 128, hd.astype(float), hv.astype(float), 1.0, 1234, 1, 2, 1e-4)
    assert np.array_equal(a["drafts"], b["drafts"]) and np.array_equal(a["accept"]["tokens"], b["accept"]["tokens"])
    assert not np.array_equal(a["drafts"], c["drafts"])
