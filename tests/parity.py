"""Comparison rules between the HIP path and the oracle.

Integer results (token ids, accept counts, flags, committed bytes) must match bit for bit,
except where the oracle flags the decision as a near tie: a top-2 margin, or a ratio-test
margin |ln(u q) - ln p|, within the logit tolerance delta (delta / T in log-probability
units).  Such decisions are counted, and everything downstream of a flagged decision in
the same request is excluded.  Floating results are compared within delta.
"""
import numpy as np

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
    y_flag = vr["y_margin"] <= delta
    bad = (vs["argmax"] != vr["argmax"]) & ~y_flag
    assert not bad.any(), f"{tag} verify argmax {vs['argmax'][bad]} vs {vr['argmax'][bad]}"
    if T > 0:
        s_flag = vr["s_margin"] <= delta / T
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


def check_cycle(g, o, T, delta, tag=""):
    """Whole cycle: drafts per slot, verify rows, acceptance."""
    k = g["drafts"].shape[1]
    flagged = 0
    for i in range(k):
        f, _ = check_draft_slot(g["drafts"], g["dstats"], o["draft"][i], T, delta, i, tag)
        flagged += f
    drafts_equal = g["drafts"] == o["drafts"]
    rows_equal = drafts_equal.all(axis=1)
    deq = np.concatenate([drafts_equal, np.ones((drafts_equal.shape[0], 1), bool)], axis=1)
    flagged += check_verify(g, o["verify"], deq, T, delta, tag)
    excluded = check_accept(g, o["accept"], rows_equal, tag)
    return dict(flagged=flagged, excluded=excluded)
