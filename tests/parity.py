"""Comparison rules between the HIP path and the oracle.

Integer results (token ids, accept counts, flags, committed bytes) must match bit for bit,
except where the oracle flags the decision as a near tie (its near-tie rules: a top-2 or
ratio-test margin within the logit tolerance delta in the score's units, or a residual pick
that moves of ln p and ln q within 2 delta/T can change).  Such decisions are counted, and
everything downstream of a flagged decision in the same request is excluded.  Floating
results are compared within delta.

What the flags excuse is bounded independently of the flagger: every comparison asserts
that at least one request was compared exactly, and that the excluded requests do not
exceed a high quantile of their count under a model of the margins that does not use the
oracle's flags (flag_budget).
"""
import numpy as np
from scipy.stats import norm, poisson

NEG_INF = -np.inf


def close(a, b, tol):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_ninf = (a == NEG_INF) & (b == NEG_INF)
    both_pinf = (a == np.inf) & (b == np.inf)
    both_nan = np.isnan(a) & np.isnan(b)
    with np.errstate(invalid="ignore"):
        diff = np.abs(a - b)
    return both_ninf | both_pinf | both_nan | (diff <= tol)


def gauss_top2_within(N: int, sigma: float, tol: float) -> float:
    """P(top-1 minus top-2 <= tol) for N iid N(0, sigma^2) logits: the joint density of the
    two largest, N(N-1) phi(y) Phi(y)^(N-2) phi(x) for x > y, integrated over x in (y, y+tol]."""
    if N < 2 or sigma <= 0:
        return 0.0
    t = tol / sigma
    y = np.linspace(-4.0, 12.0, 16001)
    dens = np.exp(np.log(N) + np.log(N - 1) + (N - 2) * norm.logcdf(y) + norm.logpdf(y))
    return float(min(1.0, np.trapezoid(dens * (norm.cdf(y + t) - norm.cdf(y)), y)))


def runner_up_within(z, tol: float) -> float:
    """The same model given the row's largest logit: the other N-1 logits iid normal (their
    own mean and standard deviation) below it, so P(runner-up >= top - tol) =
    1 - (Phi(a - t) / Phi(a))^(N-1), a and t the top and tol in units of that deviation.
    Averaged over rows of N iid normals it is gauss_top2_within; a row whose top was
    planted far above the rest gets almost no chance of a tie.  A row holding +inf takes its
    lowest +inf id by an exact rule: no tie the tolerance can turn."""
    z = np.asarray(z, dtype=np.float64)
    if np.isposinf(z).any():
        return 0.0
    f = np.sort(z[np.isfinite(z)])
    if f.size < 2:
        return 0.0
    top, rest = f[-1], f[:-1]
    sd = rest.std()
    if sd <= 0:
        return 1.0 if top - rest.max() <= tol else 0.0
    a = (top - rest.mean()) / sd
    t = tol / sd
    return float(-np.expm1(rest.size * (norm.logcdf(a - t) - norm.logcdf(a))))


def flag_budget(o, T: float, delta: float, rule: str = "ratio", drafts_supplied: bool = False,
                lattice: float = 0.0) -> float:
    """Expected number of requests with a flagged decision, from a model of the margins that
    does not look at the oracle's flags or top-2 gaps:
      * argmax of logits (greedy drafts, verify argmax, greedy bonus): runner_up_within the
        tolerance (lattice: logits on a grid of that spacing, where a gap is 0 or at least
        one step, so the tolerance counts as one step);
      * argmax of z/T + Gumbel (sampled drafts, the trunk's sample, bonus draws): the gap of
        the two best Gumbel-max scores is at most 1 - exp(-delta/T) likely to be within
        delta/T (for weights w, P(gap > e) = sum_x w_x e^-e / (w_x e^-e + W - w_x) >= e^-e);
      * the ratio test: -ln u is exponential with density at most 1, so |ln u + c| <= delta/T
        has probability at most 1 - exp(-2 delta/T);
      * the residual pick, whose scores may each move by 2 delta/T: 1 - exp(-8 delta/T)
        (twice the q << p value, two scores each moving by 2 delta/T);
    Decisions count up to the row where the oracle's request stopped."""
    acc = o["accept"]
    n_acc = np.asarray(acc["n_accept"])
    stop = np.asarray(acc["stop_kind"])
    B = n_acc.shape[0]
    k = o["drafts"].shape[1]
    zv = o["verify"]["logits"]
    exact = T > 0 and rule == "exact"
    ratio = T > 0 and rule == "ratio"
    tg = 1.0 - np.exp(-delta / T) if T > 0 else 0.0
    tr = 1.0 - np.exp(-2 * delta / T) if T > 0 else 0.0
    tres = 1.0 - np.exp(-8 * delta / T) if T > 0 else 0.0
    tol = max(delta, lattice)
    mu = 0.0
    for b in range(B):
        a = int(n_acc[b])
        ps = []
        for i in range(min(a + 1, k)):
            if not drafts_supplied:
                zd = o["draft"][i]["logits"][b]
                ps.append(tg if ratio and np.isfinite(zd).any() else runner_up_within(zd, tol))
            if exact:
                ps.append(tg)
            elif ratio:
                ps.append(tr)
            else:
                ps.append(runner_up_within(zv[b, i], tol))
        if stop[b] == 0 and ratio:
            ps.append(tres)
        if stop[b] == 2:
            ps.append(tg if T > 0 else runner_up_within(zv[b, k], tol))
        mu += 1.0 - float(np.prod([1.0 - p for p in ps]))
    return mu


def excluded_bound(mu: float) -> int:
    """Excluded requests allowed for an expected count mu: the 1 - 1e-6 quantile of a Poisson
    count with that mean (a sum of independent Bernoulli counts is no more spread out)."""
    return int(poisson.ppf(1.0 - 1e-6, max(mu, 1e-9)))


def check_draft_slot(gd_tok, gd_stats, od, T, delta, slot, tag=""):
    """One draft slot: tokens (unless flagged), max within delta, lse within delta / T_eff."""
    Te = T if T > 0 else 1.0
    tok = gd_tok[:, slot]
    flagged = od["near_tie"]
    bad = (tok != od["token"]) & ~flagged
    assert not bad.any(), f"{tag} draft slot {slot}: ids {tok[bad]} vs oracle {od['token'][bad]}"
    assert close(gd_stats["max"][:, slot], od["max"], delta).all(), f"{tag} draft max"
    assert close(gd_stats["lse"][:, slot], od["lse"], delta / Te).all(), f"{tag} draft lse"
    return int(flagged.sum()), int(((tok != od["token"]) & flagged).sum())


def check_verify(g, vr, drafts_equal, T, delta, tag=""):
    Te = T if T > 0 else 1.0
    vs = g["vstats"]
    y_flag = vr["y_near_tie"]
    bad = (vs["argmax"] != vr["argmax"]) & ~y_flag
    assert not bad.any(), f"{tag} verify argmax {vs['argmax'][bad]} vs {vr['argmax'][bad]}"
    if T > 0:
        s_flag = vr["s_near_tie"]
        bad = (vs["sample"] != vr["sample"]) & ~s_flag
        assert not bad.any(), f"{tag} verify sample {vs['sample'][bad]} vs {vr['sample'][bad]}"
    assert close(vs["max"], vr["max"], delta).all(), f"{tag} verify max"
    assert close(vs["lse"], vr["lse"], delta / Te).all(), f"{tag} verify lse"
    zt = close(vs["z_tok"], vr["z_tok"], delta)
    assert zt[drafts_equal].all(), f"{tag} verify z at drafted id"
    assert np.array_equal(vs["flags"].astype(np.uint32), vr["flags"]), f"{tag} verify row flags"
    if T > 0 and "logits" in g:
        z = np.asarray(vr["logits"])
        assert close(g["logits"], z, delta).all(), f"{tag} verify logits max err " \
            f"{np.nanmax(np.abs(np.where(np.isfinite(z), g['logits'] - z, 0)))}"
    return int(y_flag.sum())


def check_accept(g, acc, drafts_equal_rows, tag=""):
    """Exact comparison on requests whose drafts agree and whose path has no flagged decision."""
    clean = (acc["tie_row"] < 0) & drafts_equal_rows
    for key, gk in (("tokens", "tokens"), ("n_accept", "n_accept"), ("n_emit", "n_emit")):
        a = np.asarray(g[gk])[clean]
        b = np.asarray(acc[key])[clean]
        assert np.array_equal(a, b), f"{tag} accept {key}: {a} vs {b}"
    assert np.array_equal(g["flags"][clean], acc["flags"][clean].astype(np.uint32)), f"{tag} accept flags"
    return int((~clean).sum())


def check_cycle(g, o, T, delta, tag="", rule="ratio", drafts_supplied=False, lattice=0.0, bound=True,
                certain_ties=0, min_clean=1):
    """Whole cycle: drafts per slot, verify rows, acceptance; then the bound on what the
    near-tie flags excused (unless ``bound`` is False: a caller that sums several cycles
    checks the total with check_excluded).  ``certain_ties``: requests whose path holds an
    exact tie planted by the test, added to the budget."""
    k = g["drafts"].shape[1]
    flagged = 0
    for i in range(k):
        f, _ = check_draft_slot(g["drafts"], g["dstats"], o["draft"][i], T, delta, i, tag)
        flagged += f
    drafts_equal = g["drafts"] == o["drafts"]
    # the acceptance of a request reads its drafts up to the row where it stopped
    a_stop = np.minimum(np.asarray(o["accept"]["n_accept"]), k - 1)
    rows_equal = (drafts_equal | (np.arange(k)[None, :] > a_stop[:, None])).all(axis=1)
    deq = np.concatenate([drafts_equal, np.ones((drafts_equal.shape[0], 1), bool)], axis=1)
    flagged += check_verify(g, o["verify"], deq, T, delta, tag)
    excluded = check_accept(g, o["accept"], rows_equal, tag)
    res = dict(flagged=flagged, excluded=excluded, requests=int(rows_equal.shape[0]),
               budget=flag_budget(o, T, delta, rule, drafts_supplied, lattice) + certain_ties)
    if bound:
        check_excluded(res, tag, min_clean)
    return res


def add_results(total, r):
    """Running sums of check_cycle results over cycles."""
    if total is None:
        return dict(r)
    return {key: total[key] + r[key] for key in total}


def check_excluded(res, tag="", min_clean=1):
    """At least ``min_clean`` requests compared exactly, and no more excluded than the
    budget allows."""
    clean = res["requests"] - res["excluded"]
    lim = excluded_bound(res["budget"])
    print(f"{tag}: {res['excluded']} of {res['requests']} requests excused by near ties "
          f"(expected at most {res['budget']:.2f}, allowed {lim})", flush=True)
    assert clean >= min_clean, f"{tag}: only {clean} requests compared exactly"
    assert res["excluded"] <= lim, f"{tag}: {res['excluded']} excluded, budget {res['budget']:.2f} allows {lim}"
