"""End-to-end pins of the oracle on a tiny recurrent trunk.

Greedy speculative decoding must emit exactly the tokens of ordinary argmax decoding
(lucebox-hub PR "feat(qwen4exp): MTP speculative decoding", section "Exactness"), so must
sampled decoding with exact-match acceptance against ordinary sampled decoding under the
same seed (same PR, "Exactness" and "Notes"; the trunk's draws are keyed by position), and
after every commit the live recurrent state, the KV rows and kv_len must equal those of
ordinary decoding after the same number of tokens (DS4Server issue "Add Qwen3.8 Flash
Next native MTP speculation", section "Completion requirements": rejected rows leave every
cache and recurrent component identical to ordinary decoding).  Also: the commit itself,
brute force, for every acceptance depth with guard bytes.
"""
import numpy as np
import pytest

from oracle import mtp_oracle as O
from toy_trunk import ToyTrunk

MAX_ROWS = 512


def ordinary_greedy(tt: ToyTrunk, t0: int, n: int):
    S = tt.zero_state()
    t = t0
    out, states, kv = [], [], []
    for _ in range(n):
        S = tt.step(S, t)
        kv.append(tt.kv_row(t))
        y = int(np.argmax(tt.W @ tt.hidden(S, t)))
        out.append(y)
        states.append(tt.state_bytes(S))
        t = y
    return out, states, kv


def ordinary_sampled(tt: ToyTrunk, t0: int, n: int, T: float, seed: int):
    """Decoding without speculation at temperature T: the token at position p is the
    trunk's own draw at p."""
    S = tt.zero_state()
    t = t0
    out, states, kv = [], [], []
    for pos in range(n):
        S = tt.step(S, t)
        kv.append(tt.kv_row(t))
        y, _ = O.trunk_sample(tt.W @ tt.hidden(S, t), T, seed, 0, pos)
        out.append(y)
        states.append(tt.state_bytes(S))
        t = y
    return out, states, kv


def _kv_bytes(row: np.ndarray) -> np.ndarray:
    return np.frombuffer(row.tobytes(), dtype=np.uint8)


def speculative_greedy(tt: ToyTrunk, t0: int, n: int, k: int, n_draft: int, forced=None,
                       T: float = 0.0, seed: int = 0):
    """Drive draft -> verify -> accept -> commit with the oracle; yield per-cycle snapshots.
    T > 0: exact-match acceptance against the trunk's position-keyed draws."""
    W = tt.W
    S = tt.zero_state()
    row_bytes = tt.kv_dim * 8
    kv = np.zeros((1, 1, 2, MAX_ROWS, row_bytes), dtype=np.uint8)
    kv_len = np.zeros(1, dtype=np.int32)
    emitted = []
    cycles = []
    cont = None
    c = 0
    while len(emitted) < n:
        # k chained drafts from the drafter's own copy of the state
        Sd, tok, drafts = S, t0, []
        for i in range(k):
            Sd = tt.step(Sd, tok)
            h = tt.hidden(Sd, tok, drafter=True)
            d = int(O.draft_rows(W, n_draft, h[None], 0.0, 0, i, c, 1e-9)["token"][0])
            drafts.append(d)
            tok = d
        if forced is not None:
            # first mismatch forced at depth a: drafts = true continuation up to a, then a wrong id
            a_force = forced[c % len(forced)]
            if cont is None:
                cont = ordinary_greedy(tt, 0, n + k + 2)[0]
            base = len(emitted)
            truth = cont[base:base + k]
            drafts = list(truth)
            if a_force < k:
                drafts[a_force] = (truth[a_force] + 1) % n_draft
        # verify the k+1 rows, snapshot after each row, append their KV rows
        Sv, toks, snaps, hv = S, [t0] + drafts, [], []
        for i, tk in enumerate(toks):
            Sv = tt.step(Sv, tk)
            snaps.append(tt.state_bytes(Sv))
            hv.append(tt.hidden(Sv, tk))
            r = _kv_bytes(tt.kv_row(tk))
            kv[0, 0, 0, kv_len[0] + i] = r
            kv[0, 0, 1, kv_len[0] + i] = r[::-1]
        if T > 0:
            # verify row 0 predicts the token at position len(emitted)
            vr = O.verify_rows(W, np.array(hv)[None], np.array([drafts]), T, seed, c, 1e-9,
                               positions=[len(emitted)])
            acc = O.accept(np.array([drafts]), None, vr["logits"], n_draft, T, seed, c, -1, 1e-9,
                           rule=O.RULE_EXACT, target=vr)
        else:
            zv = (np.array(hv) @ W.T)[None]
            acc = O.accept(np.array([drafts]), None, zv, n_draft, 0.0, 0, c, -1, 1e-9)
        live, kv, kv_len = O.commit(np.array([snaps]), np.zeros((1, snaps[0].size), np.uint8), kv, kv_len,
                                    acc["n_accept"], k)
        S = np.frombuffer(live[0].tobytes(), dtype=np.float64).reshape(S.shape).copy()
        m = int(acc["n_emit"][0])
        emitted += [int(v) for v in acc["tokens"][0, :m]]
        t0 = emitted[-1]
        cycles.append(dict(n_accept=int(acc["n_accept"][0]), live=live[0].copy(), kv=kv.copy(),
                           kv_len=int(kv_len[0]), n_emitted=len(emitted)))
        c += 1
    return emitted[:n], cycles


def _check_state(tt, cycles, states, kv_rows):
    for cy in cycles:
        n = cy["n_emitted"]
        if n > len(states):
            break
        assert np.array_equal(cy["live"], states[n - 1])
        assert cy["kv_len"] == n
        for r in range(n):
            assert np.array_equal(cy["kv"][0, 0, 0, r], _kv_bytes(kv_rows[r]))
            assert np.array_equal(cy["kv"][0, 0, 1, r], _kv_bytes(kv_rows[r])[::-1])
        assert not cy["kv"][0, 0, :, n:].any()


@pytest.mark.parametrize("k", [1, 2, 3, 5, 7])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_greedy_speculation_equals_ordinary_decoding(k, seed):
    tt = ToyTrunk(seed)
    n = 200
    want, states, kv_rows = ordinary_greedy(tt, 0, n + 8)
    got, cycles = speculative_greedy(tt, 0, n, k, n_draft=tt.V)
    assert got == want[:n]
    _check_state(tt, cycles, states, kv_rows)
    # the drafter is imperfect, so several acceptance depths occur
    assert len({cy["n_accept"] for cy in cycles}) >= min(k + 1, 2)


@pytest.mark.parametrize("k", [3, 7])
def test_every_acceptance_depth_commits_ordinary_state(k):
    tt = ToyTrunk(5)
    n = 120
    want, states, kv_rows = ordinary_greedy(tt, 0, n + k + 8)
    got, cycles = speculative_greedy(tt, 0, n, k, n_draft=tt.V, forced=list(range(k + 1)))
    assert got == want[:n]
    assert {cy["n_accept"] for cy in cycles} == set(range(k + 1))
    _check_state(tt, cycles, states, kv_rows)


def test_truncated_draft_vocabulary_keeps_output_exact():
    # drafts can only come from the first 10 ids; output still equals ordinary decoding
    tt = ToyTrunk(3)
    want, states, kv_rows = ordinary_greedy(tt, 0, 160)
    got, cycles = speculative_greedy(tt, 0, 150, 4, n_draft=10)
    assert got == want[:150]
    _check_state(tt, cycles, states, kv_rows)


@pytest.mark.parametrize("a", range(8))
def test_commit_brute_force_with_guards(a):
    rng = np.random.default_rng(a)
    B, k, S, L, R, rb = 3, 7, 40, 2, 20, 6
    snaps = rng.integers(0, 256, size=(B, k + 1, S), dtype=np.uint8)
    live = rng.integers(0, 256, size=(B, S), dtype=np.uint8)
    kv_len = np.array([0, 5, R - k - 1], dtype=np.int32)
    kv = rng.integers(1, 256, size=(B, L, 2, R, rb), dtype=np.uint8)   # no zero bytes anywhere
    n_acc = np.array([a, (a + 3) % (k + 1), k - a % (k + 1)])
    new_live, new_kv, new_len = O.commit(snaps, live, kv, kv_len, n_acc, k)
    for b in range(B):
        ab = int(n_acc[b])
        for j in range(S):
            assert new_live[b, j] == snaps[b, ab, j]
        assert new_len[b] == kv_len[b] + ab + 1
        for layer in range(L):
            for kvh in range(2):
                for r in range(R):
                    rejected = kv_len[b] + ab + 1 <= r <= kv_len[b] + k
                    for j in range(rb):
                        want = 0 if rejected else kv[b, layer, kvh, r, j]
                        assert new_kv[b, layer, kvh, r, j] == want
    # inputs untouched
    assert kv.all()


def test_commit_clips_to_the_cache():
    k = 3
    snaps = np.arange(2 * 4 * 2, dtype=np.uint8).reshape(2, 4, 2)
    kv = np.ones((2, 1, 2, 6, 1), dtype=np.uint8)
    # request 0: kv_len + k + 1 > max_rows; request 1: n_accept out of range (clamped to k)
    live, nkv, nlen = O.commit(snaps, np.zeros((2, 2), np.uint8), kv, np.array([4, 1], np.int32),
                               np.array([0, 99]), k)
    assert list(nlen) == [5, 5]
    assert np.array_equal(live[1], snaps[1, 3])
    assert nkv[0, 0, 0, :, 0].tolist() == [1, 1, 1, 1, 1, 0]
    assert nkv[1].all()


def test_planted_off_by_one_commit_is_caught(monkeypatch):
    # committing snapshot a+1 (the row of the rejected draft) must break state equality
    real = O.commit

    def off_by_one(snaps, live, kv, kv_len, n_acc, k):
        return real(snaps, live, kv, kv_len, np.minimum(np.asarray(n_acc) + 1, k), k)
    monkeypatch.setattr(O, "commit", off_by_one)
    tt = ToyTrunk(5)
    want, states, kv_rows = ordinary_greedy(tt, 0, 80)
    got, cycles = speculative_greedy(tt, 0, 60, 3, n_draft=tt.V, forced=[0, 1, 2, 3])
    with pytest.raises(AssertionError):
        assert got == want[:60]
        _check_state(tt, cycles, states, kv_rows)


def test_planted_wrong_row_in_exact_match_is_caught(monkeypatch):
    # comparing draft d_{i+1} with y_{i+1} instead of y_i must change the output
    real = O.accept

    def shifted(drafts, zd, zv, *a, **kw):
        zv2 = np.concatenate([zv[:, 1:], zv[:, -1:]], axis=1)
        return real(drafts, zd, zv2, *a, **kw)
    monkeypatch.setattr(O, "accept", shifted)
    tt = ToyTrunk(1)
    want, _, _ = ordinary_greedy(tt, 0, 100)
    got, _ = speculative_greedy(tt, 0, 100, 3, n_draft=tt.V)
    assert got != want[:100]


@pytest.mark.parametrize("k", [1, 3, 7])
@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("T", [0.7, 1.0])
def test_exact_match_sampling_equals_ordinary_sampling(k, seed, T):
    tt = ToyTrunk(seed)
    n = 150
    want, states, kv_rows = ordinary_sampled(tt, 0, n + 8, T, 1234 + seed)
    got, cycles = speculative_greedy(tt, 0, n, k, n_draft=tt.V, T=T, seed=1234 + seed)
    assert got == want[:n]
    _check_state(tt, cycles, states, kv_rows)
    # sampling departs from the argmax path, and drafts are both kept and rejected
    assert got != ordinary_greedy(tt, 0, n)[0]
    assert len({cy["n_accept"] for cy in cycles}) >= 2


def test_planted_cycle_keyed_trunk_draw_is_caught(monkeypatch):
    # the trunk's draw keyed by (cycle, row) instead of position: no longer the output
    # of ordinary sampling
    calls = {"n": 0}
    real = O.trunk_noise

    def by_call(seed, b, position, n):
        calls["n"] += 1
        return real(seed, b, position + 7 * calls["n"], n)
    monkeypatch.setattr(O, "trunk_noise", by_call)
    tt = ToyTrunk(2)
    got, _ = speculative_greedy(tt, 0, 60, 3, n_draft=tt.V, T=1.0, seed=5)
    calls["n"] = 0
    monkeypatch.setattr(O, "trunk_noise", real)
    want, _, _ = ordinary_sampled(tt, 0, 60, 1.0, 5)
    assert got != want
