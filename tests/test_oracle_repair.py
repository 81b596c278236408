"""Capture-commit against an ordinary-forward repair fallback.

DS4Server issue "Add Qwen3.8 Flash Next native MTP speculation": "Implementation" asks to
capture the verification rows' recurrent (gated-delta) state, commit only accepted rows,
and keep a correct ordinary-forward repair fallback; "Verification" asks to compare the two
at logit, token and complete cache-state level; "Completion requirements": both correct.
llama.cpp PR #28104, the "store" commit: a replay that verifies its tokens again can loop
forever on a backend whose logits depend on the batch shape; replayed tokens are accepted
as they are and only the continuation is taken at the final position.

Here, on the toy trunk with short-convolution rows in its state: both paths emit ordinary
decoding's tokens, leave byte-identical state, KV and length after every cycle, and give
identical logits for the next position; a repair that re-verifies stalls under batch-shape
dependent logits while the one that does not always makes progress.
"""
import numpy as np
import pytest

from repair_paths import ordinary, speculative
from toy_trunk import ToyTrunkConv


def _same_cycles(a, b):
    assert len(a) == len(b)
    for x, y in zip(a, b):
        assert x["n_accept"] == y["n_accept"] and x["n_emitted"] == y["n_emitted"]
        assert np.array_equal(x["live"], y["live"])                 # state incl. conv rows, bytewise
        assert x["kv_len"] == y["kv_len"]
        assert np.array_equal(x["kv"], y["kv"])                     # KV rows and the zeroed tail
        assert np.array_equal(x["next_logits"], y["next_logits"])   # logit level


@pytest.mark.parametrize("k", [1, 3, 7])
@pytest.mark.parametrize("T", [0.0, 1.0])
def test_capture_commit_equals_repair_and_ordinary_decoding(k, T):
    tt = ToyTrunkConv(3)
    n = 120
    want, states, logits = ordinary(tt, 0, n + k + 2, T, seed=42)
    got_c, cyc_c, _ = speculative(tt, 0, n, k, "capture", T, seed=42)
    got_r, cyc_r, _ = speculative(tt, 0, n, k, "repair", T, seed=42)
    assert got_c == want[:n] and got_r == want[:n]                  # token level
    _same_cycles(cyc_c, cyc_r)
    for cy in cyc_c:                                                # = ordinary decoding's state
        m = cy["n_emitted"]
        if m <= len(states):
            assert np.array_equal(cy["live"], states[m - 1])
            assert np.array_equal(cy["next_logits"], logits[m]) if m < len(logits) else True
    assert len({cy["n_accept"] for cy in cyc_c}) >= 2


def test_conv_rows_are_part_of_the_rollback():
    # committing only the matrix part of the snapshot (stale conv rows) breaks equality
    from oracle import mtp_oracle as O
    tt = ToyTrunkConv(4)

    def matrices_only(snaps, live, kv, kv_len, n_acc, k):
        new_live, kv2, len2 = O.commit(snaps, live, kv, kv_len, n_acc, k)
        cut = tt.ns * 8
        new_live[:, cut:] = snaps[:, k, cut:]                       # conv rows of the last row instead
        return new_live, kv2, len2
    want, _, _ = ordinary(tt, 0, 80)
    got, _, _ = speculative(tt, 0, 60, 3, "capture", commit=matrices_only)
    assert got != want[:60]


def _batch_shape_noise(seed):
    rng = np.random.default_rng(seed)
    offs = {w: rng.standard_normal(64) * 0.6 for w in range(1, 9)}
    return lambda z, width: z + offs[width][:z.size]


def test_reverifying_replay_livelocks_and_the_plain_replay_does_not():
    tt = ToyTrunkConv(6)
    pert = _batch_shape_noise(1)
    got, cyc, ncyc = speculative(tt, 0, 150, 4, "repair", perturb=pert, reverify=False, max_cycles=400)
    assert len(got) == 150                                          # progress every cycle
    assert all(c["n_accept"] >= 0 for c in cyc)
    _, cyc_rv, _ = speculative(tt, 0, 150, 4, "repair", perturb=pert, reverify=True, max_cycles=400)
    stalls = sum(c["n_accept"] < 0 for c in cyc_rv)
    assert stalls > 0
    # a stalled cycle restores and repeats the same position: the same cycle repeats forever
    first = next(i for i, c in enumerate(cyc_rv) if c["n_accept"] < 0)
    assert all(c["n_accept"] < 0 and c["n_emitted"] == cyc_rv[first]["n_emitted"] for c in cyc_rv[first:])
