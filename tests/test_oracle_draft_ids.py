"""The draft vocabulary as an id list (lucebox-hub PR "feat(qwen4exp): MTP speculative
decoding", section "What": the draft head covers control/special tokens plus the lowest
ids).  Pins of the oracle's id-mapped draft head and acceptance:
  * the prefix list 0..n-1 reproduces the default draft vocabulary exactly;
  * gathering the rows equals masking the full vocabulary to the list (argmax, and
    Gumbel-max with noise keyed by the vocabulary id);
  * ratio acceptance with a non-prefix list still emits p at every position (Monte Carlo),
    and the acceptance rate is sum_x min(p, q) with q supported on the list.
"""
import numpy as np
import pytest
from scipy import stats

import synth
from oracle import mtp_oracle as O

V, D = 64, 32


def _setup(seed=0):
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((V, D))
    ids = np.sort(np.concatenate([np.arange(20), [40, 51, 63]]))   # lowest ids + a few specials
    return rng, W, ids


@pytest.mark.parametrize("T", [0.0, 0.8])
def test_prefix_list_is_the_default_vocabulary(T):
    rng, W, _ = _setup()
    h = rng.standard_normal((5, D))
    a = O.draft_rows(W, 24, h, T, 7, 2, 3, 1e-9)
    b = O.draft_rows(W, 24, h, T, 7, 2, 3, 1e-9, ids=np.arange(24))
    for key in ("token", "max", "lse", "z_tok", "logits"):
        assert np.array_equal(a[key], b[key]), key


@pytest.mark.parametrize("T", [0.0, 0.5, 1.0])
def test_gathered_rows_equal_the_masked_vocabulary(T):
    rng, W, ids = _setup(1)
    h = rng.standard_normal((400, D)) * 0.7
    out = O.draft_rows(W, ids.size, h, T, 11, 1, 5, 1e-9, ids=ids)
    z = h @ W.T
    mask = np.full(V, -np.inf)
    mask[ids] = 0.0
    if T > 0:
        G = O.gumbel_noise(11, O.STREAM_DRAFT, 1, np.arange(400), 5, V)   # noise for every id
        want = np.argmax(z / T + G + mask, axis=1)
    else:
        want = np.argmax(z + mask, axis=1)
    clear = out["margin"] > 1e-9
    assert np.array_equal(out["token"][clear], want[clear])
    assert np.all(np.isin(out["token"], ids))
    assert np.allclose(out["logits"], z[:, ids])


def test_sampled_draft_follows_q_on_the_list():
    _, W, ids = _setup(2)
    W = np.eye(V, D)
    h = np.zeros((20000, D))
    h[:, :D] = np.linspace(-1.0, 1.0, D)                           # the same logits for every request
    out = O.draft_rows(W, ids.size, h, 1.0, 3, 0, 0, 1e-9, ids=ids)
    z = h[0] @ W.T
    q = np.exp(z[ids]) / np.exp(z[ids]).sum()
    counts = np.array([(out["token"] == x).sum() for x in ids])
    assert counts.sum() == 20000
    assert stats.chisquare(counts, 20000 * q).pvalue > 1e-4


@pytest.mark.slow
def test_ratio_acceptance_with_an_id_list_emits_p():
    V_, K, n = 16, 3, 120_000
    rng = np.random.default_rng(21)
    ids = np.array([0, 1, 2, 5, 9, 12, 15])
    h_v = rng.standard_normal((K + 1, V_)) * 1.2
    h_d = rng.standard_normal((K, V_)) * 1.2
    h_d[:, ids] += 0.6 * h_v[:K, ids]
    W = O.head_weights_f64(synth.identity_head(V_))
    Hv = np.broadcast_to(h_v, (n, K + 1, V_)).copy()
    Hd = np.broadcast_to(h_d, (n, K, V_)).copy()
    out = O.cycle(W, ids.size, Hd, Hv, 1.0, 99, 0, -1, 1e-4, draft_ids=ids)
    acc = out["accept"]
    assert np.all(np.isin(out["drafts"], ids))
    sm = lambda z: np.exp(z - z.max()) / np.exp(z - z.max()).sum()
    pv = []
    for i in range(K + 1):
        reach = acc["n_accept"] >= i
        c = np.bincount(acc["tokens"][reach, i], minlength=V_)
        pv.append(stats.chisquare(c, c.sum() * sm(h_v[i])).pvalue)
    assert min(pv) >= 1e-4 / (K + 1), pv
    for i in range(K):
        p = sm(h_v[i])
        q = np.zeros(V_)
        q[ids] = sm(h_d[i][ids])
        reach = acc["n_accept"] >= i
        rate = np.mean(acc["n_accept"][reach] > i)
        want = np.minimum(p, q).sum()
        assert abs(rate - want) < 5 * np.sqrt(want * (1 - want) / reach.sum()) + 1e-3
    # the same drafts with q taken on the prefix 0..6 (the wrong rows) break the law
    bad = O.accept(out["drafts"], np.stack([r["logits"] for r in out["draft"]], 1), out["verify"]["logits"],
                   ids.size, 1.0, 99, 0, -1, 1e-4)
    pvb = []
    for i in range(K + 1):
        reach = bad["n_accept"] >= i
        c = np.bincount(bad["tokens"][reach, i], minlength=V_)
        pvb.append(stats.chisquare(c, c.sum() * sm(h_v[i])).pvalue)
    assert min(pvb) < 1e-6
