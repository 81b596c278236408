"""Adaptive verify width (lucebox-hub PR "feat(qwen4exp): MTP speculative decoding",
section "What": the width adapts, up to seven drafts, from per-depth acceptance and a
per-request cycle-cost fit).  The oracle's controller is pinned to closed forms and
special cases; the library's native controller (mtp_width_*, host code, no GPU) must
agree with it on random observation streams."""
import ctypes
import os

import numpy as np
import pytest

import speculative_decoding_head_amd as mtp
from oracle.width_oracle import ACC_ALL_ACCEPTED, ACC_EOS, ACC_EOS_DRAFT, ACC_ROW_INVALID, WidthController as OW


def _native_ok():
    return os.path.exists(mtp.LIB_PATH)


# ---- oracle pins ------------------------------------------------------------------
@pytest.mark.parametrize("a", [0.0, 0.3, 0.75, 0.99])
def test_expected_tokens_closed_form(a):
    w = OW(alpha0=a)
    for k in range(0, 8):
        want = 1.0 + (k if a == 1.0 else a * (1 - a ** k) / (1 - a))
        assert abs(w.expected_tokens(k) - want) < 1e-12


def test_always_accepting_drafts_pick_by_cost_shape():
    # alpha = 1: E(k) = k + 1, so E/c = (k+1)/(c0 + c1 k) rises with k iff c0 > c1
    for c0, c1, want in ((1.0, 0.2, 7), (1.0, 0.9, 7), (0.3, 1.0, 1)):
        w = OW(alpha0=1.0)
        for k in (2, 5, 2, 5):
            w.observe(k, [k], [ACC_ALL_ACCEPTED], c0 + c1 * k)
        assert abs(w.cost(0) - c0) < 1e-9 and abs(w.cost(1) - (c0 + c1)) < 1e-9
        assert w.choose() == want


def test_never_accepting_drafts_pick_one():
    w = OW(alpha0=0.0)
    assert w.choose() == 1
    w = OW(alpha0=0.9)
    for _ in range(200):
        w.observe(4, [0, 0], [0, 0], 0.0)
    assert w.alpha[0] < 1e-8 and w.choose() == 1


def test_free_drafts_pick_the_maximum():
    w = OW(k_max=5, alpha0=0.2, slope_prior=0.0)   # c1 = 0: every draft is free
    assert w.choose() == 5


def test_cost_fit_recovers_a_linear_cost():
    w = OW(decay=0.2)
    for i in range(40):
        k = 1 + i % 7
        w.observe(k, [0], [0], 2.0 + 0.3 * k)
    c0, c1 = w.cost_params()
    assert abs(c0 - 2.0) < 1e-9 and abs(c1 - 0.3) < 1e-9


def test_single_width_uses_the_prior_slope():
    w = OW(slope_prior=0.25)
    for _ in range(10):
        w.observe(3, [1], [0], 1.75)
    c0, c1 = w.cost_params()
    assert abs(c1 - 0.25 * c0) < 1e-12 and abs(w.cost(3) - 1.75) < 1e-12


def test_acceptance_ema_tracks_per_depth_rates():
    rng = np.random.default_rng(0)
    p = [0.9, 0.7, 0.5, 0.3, 0.2, 0.1, 0.05]
    w = OW(decay=0.01, alpha0=0.5)
    for _ in range(20000):
        a = 0
        while a < 7 and rng.random() < p[a]:
            a += 1
        w.observe(7, [a], [ACC_ALL_ACCEPTED if a == 7 else 0], 0.0)
    for j in range(5):
        assert abs(w.alpha[j] - p[j]) < 0.08, (j, w.alpha[j])


def test_stopping_depth_by_how_the_block_ended():
    # an unusable target row decides nothing at its depth
    w = OW(alpha0=0.5, decay=0.5)
    w.observe(4, [2], [ACC_ROW_INVALID], 0.0)
    assert w.alpha[:4] == [0.75, 0.75, 0.5, 0.5] and w.weight[:4] == [1.0, 1.0, 0.0, 0.0]
    # a rejection at draft 3, with or without an EOS correction after it
    for f in (0, ACC_EOS):
        w = OW(alpha0=0.5, decay=0.5)
        w.observe(4, [2], [f], 0.0)
        assert w.alpha[:4] == [0.75, 0.75, 0.25, 0.5] and w.weight[:4] == [1.0, 1.0, 1.0, 0.0]
    # draft 3 was an EOS and was accepted: the block ends there, draft 3 counts as accepted
    w = OW(alpha0=0.5, decay=0.5)
    w.observe(4, [2], [ACC_EOS | ACC_EOS_DRAFT], 0.0)
    assert w.alpha[:4] == [0.75, 0.75, 0.75, 0.5] and w.weight[:4] == [1.0, 1.0, 1.0, 0.0]
    # recency decays for every depth at each request-cycle
    w.observe(4, [0], [0], 0.0)
    assert w.weight[:4] == [1.5, 0.5, 0.5, 0.0]


def test_depths_not_decided_recently_take_the_shallower_estimate():
    # only k = 1 cycles: deeper depths are never decided, so E(k) is the geometric series of
    # alpha[0]; once depth 1 and 2 are decided they use their own rates
    w = OW(alpha0=0.2, decay=0.25)
    for _ in range(30):
        w.observe(1, [1], [ACC_ALL_ACCEPTED], 0.0)
    a = w.alpha[0]
    assert a > 0.99 and w.alpha[1] == 0.2
    for k in range(8):
        assert abs(w.expected_tokens(k) - sum(a ** i for i in range(k + 1))) < 1e-12
    w.observe(3, [1], [0], 0.0)                   # depth 1 decided (rejected); depth 2 still not
    a0, a1 = w.alpha[0], w.alpha[1]
    assert abs(w.expected_tokens(3) - (1 + a0 + a0 * a1 + a0 * a1 * a1)) < 1e-12
    # a depth decided long ago is stale again
    for _ in range(10):
        w.observe(1, [1], [ACC_ALL_ACCEPTED], 0.0)
    assert w.weight[1] < 0.5 and w.estimates()[1] == w.alpha[0]


def _run_step_law(ctl, phases, c0=144e-6, c1=57.5e-6, seed=0):
    """Drive a controller through phases (cycles, per-draft acceptance) with a planted
    geometric acceptance law and a linear cycle cost; return the width chosen each cycle."""
    rng = np.random.default_rng(seed)
    ks = []
    for n, p in phases:
        for _ in range(n):
            k = ctl.choose()
            a = 0
            while a < k and rng.random() < p:
                a += 1
            ctl.observe(k, [a], [ACC_ALL_ACCEPTED if a == k else 0], c0 + c1 * k)
            ks.append(k)
    return ks


def _step_pin(make):
    """Acceptance 0.3, then 0.98, then 0.3 again: the width climbs to seven drafts within 80
    cycles of the rise and falls back to at most two within 80 cycles of the drop."""
    ks = _run_step_law(make(), [(300, 0.3), (300, 0.98), (300, 0.3)])
    assert max(ks[200:300]) <= 2, ks[200:300]
    assert 7 in ks[300:380], ks[300:380]
    assert np.mean(np.array(ks[400:600]) >= 6) > 0.8, ks[400:600]
    assert max(ks[680:900]) <= 2, ks[680:900]


def test_width_climbs_to_seven_and_back_on_a_step_in_acceptance():
    _step_pin(lambda: OW(decay=0.1, alpha0=0.8, slope_prior=0.1))


def test_a_controller_without_exploration_is_caught():
    class Frozen(OW):
        def estimates(self):
            return list(self.alpha)        # stale depths keep their old values
    with pytest.raises(AssertionError):
        _step_pin(lambda: Frozen(decay=0.1, alpha0=0.8, slope_prior=0.1))


@pytest.mark.skipif(not _native_ok(), reason="libmtp.so not built")
def test_native_width_climbs_to_seven_and_back():
    _step_pin(lambda: mtp.WidthController(decay=0.1, alpha0=0.8, slope_prior=0.1))


def test_a_planted_off_by_one_depth_is_caught():
    # counting the rejected draft as accepted must break the per-depth rates
    class Bad(OW):
        def observe(self, k, n_accept, flags, seconds):
            super().observe(k, [min(int(a) + 1, k) for a in n_accept], flags, seconds)
    rng = np.random.default_rng(1)
    good, bad = OW(decay=0.01), Bad(decay=0.01)
    for _ in range(5000):
        a = int(rng.integers(0, 3))
        good.observe(7, [a], [0], 0.0)
        bad.observe(7, [a], [0], 0.0)
    assert abs(good.alpha[0] - bad.alpha[0]) > 0.2


# ---- the native controller against the oracle ------------------------------------
@pytest.mark.skipif(not _native_ok(), reason="libmtp.so not built")
@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_native_controller_matches_the_oracle(seed):
    rng = np.random.default_rng(seed)
    k_max = int(rng.integers(1, 8))
    args = dict(k_max=k_max, decay=float(rng.uniform(0.02, 0.5)), alpha0=float(rng.uniform(0, 1)),
                slope_prior=float(rng.uniform(0, 0.5)))
    o, n = OW(**args), mtp.WidthController(**args)
    for step in range(300):
        k = o.choose() if step % 3 else int(rng.integers(1, k_max + 1))
        assert n.choose() == o.choose()
        B = int(rng.integers(1, 17))
        acc = rng.integers(0, k + 1, size=B).astype(np.int32)
        fl = np.zeros(B, np.uint32)
        fl[acc == k] |= ACC_ALL_ACCEPTED
        fl[rng.random(B) < 0.05] |= ACC_EOS
        fl[(rng.random(B) < 0.05) & (acc < k)] |= ACC_EOS | ACC_EOS_DRAFT
        fl[rng.random(B) < 0.02] |= ACC_ROW_INVALID
        secs = float(rng.uniform(2e-4, 9e-4)) if rng.random() < 0.8 else 0.0
        o.observe(k, acc, fl, secs)
        n.observe(k, acc, fl, secs)
        assert np.allclose(n.alpha, o.alpha, rtol=0, atol=1e-12)
        assert np.allclose(n.weight, o.weight, rtol=0, atol=1e-12)
        for kk in range(8):
            assert abs(n.expected_tokens(kk) - o.expected_tokens(kk)) < 1e-12
            assert abs(n.cost(kk) - o.cost(kk)) <= 1e-12 * max(1.0, abs(o.cost(kk)))
    c = n.counters
    assert (c["verifier_passes"], c["cycles"], c["drafted"], c["accepted"], c["depth_hist"]) == \
        (o.verifier_passes, o.cycles, o.drafted, o.accepted, o.depth_hist)


@pytest.mark.skipif(not _native_ok(), reason="libmtp.so not built")
def test_native_controller_rejects_bad_arguments():
    lib = mtp.load_library()
    c = mtp.mtp._WidthCtl()
    assert lib.mtp_width_init(None, 7, 0.1, 0.8, 0.1) == -1
    for args, want in (((0, 0.1, 0.8, 0.1), -2), ((8, 0.1, 0.8, 0.1), -2), ((7, 0.0, 0.8, 0.1), -4),
                       ((7, 1.5, 0.8, 0.1), -4), ((7, 0.1, 1.2, 0.1), -4), ((7, 0.1, 0.8, -1.0), -4)):
        assert lib.mtp_width_init(ctypes.byref(c), *args) == want
    assert lib.mtp_width_init(ctypes.byref(c), 7, 0.1, 0.8, 0.1) == 0
    acc = np.array([1, 5], np.int32)
    fl = np.zeros(2, np.uint32)
    assert lib.mtp_width_observe(ctypes.byref(c), 3, 2, acc.ctypes.data, fl.ctypes.data, 1e-3) == -4
    assert lib.mtp_width_observe(ctypes.byref(c), 0, 2, acc.ctypes.data, fl.ctypes.data, 1e-3) == -2
    assert lib.mtp_width_observe(ctypes.byref(c), 5, 2, None, fl.ctypes.data, 1e-3) == -1
    assert c.cycles == 0 and c.verifier_passes == 0           # nothing was counted
    assert ctypes.sizeof(mtp.mtp._WidthCtl) == 4 + 4 + 8 + 8 + 56 + 56 + 40 + 32 + 64
