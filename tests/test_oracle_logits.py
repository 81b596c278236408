"""Pins of the oracle's weight decoding, logits, sanitising, argmax and row statistics.

Pinned against exact integer arithmetic on exactly representable inputs, hand-built
4-bit bytes, library routines (scipy's logsumexp), and hand-written expectations.
"""
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import logsumexp

import synth
from oracle import mtp_oracle as O


def _exact_head(rng, V, d):
    # W = m / 256 with |m| <= 127: exact in bf16 (<= 7 significant bits after the leading one)
    m = rng.integers(-127, 128, size=(V, d))
    w = (m / 256.0).astype(np.float32)
    return m, synth.Head("bf16", V, d, synth.bf16_bits(w))


def test_bf16_decode_and_logits_are_exact_on_representable_inputs():
    rng = np.random.default_rng(3)
    V, d = 37, 96
    m, head = _exact_head(rng, V, d)
    h_int = rng.integers(-3, 4, size=(5, d))
    h_bits = synth.bf16_bits(h_int.astype(np.float32))
    W = O.head_weights_f64(head)
    assert np.array_equal(W * 256, m)
    z = O.logits_f64(W, O.hidden_f64(h_bits, "bf16"))
    for r in range(5):
        for x in range(V):
            want = Fraction(int(sum(int(m[x, j]) * int(h_int[r, j]) for j in range(d))), 256)
            assert Fraction(z[r, x]) == want


def test_q4a32_decode_from_hand_built_bytes():
    # one row, d = 64 (two groups); q[j] = j % 16; group 0: scale 2^-4, min -8 * 2^-4 -> w = (q-8)/16
    # group 1: scale 2^-2, min 1.0 -> w = q/4 + 1
    d = 64
    q = [j % 16 for j in range(d)]
    nib = bytes((q[2 * i] | (q[2 * i + 1] << 4)) for i in range(d // 2))
    bf16 = {0.0625: 0x3D80, -0.5: 0xBF00, 0.25: 0x3E80, 1.0: 0x3F80}
    head = synth.Head("q4a32", 1, d, np.frombuffer(nib, dtype=np.uint8).reshape(1, d // 2),
                      scale=np.array([[bf16[0.0625], bf16[0.25]]], dtype=np.uint16),
                      minv=np.array([[bf16[-0.5], bf16[1.0]]], dtype=np.uint16))
    W = O.head_weights_f64(head)[0]
    want = [(q[j] - 8) / 16 for j in range(32)] + [q[j] / 4 + 1 for j in range(32, 64)]
    assert list(W) == want


def test_q4a32_packer_round_trip_within_half_step():
    rng = np.random.default_rng(11)
    w = (rng.standard_normal((50, 256)) * 0.02).astype(np.float32)
    nib, sc, mn = synth.pack_q4a32(w)
    W = O.head_weights_f64(synth.Head("q4a32", 50, 256, nib, sc, mn))
    step = np.repeat(O.bf16_to_f64(sc), 32, axis=1)
    # bf16 rounding of min/scale moves the grid slightly: allow half a step plus that shift
    err = np.abs(W - w)
    assert np.all(err <= 0.5 * step + 16 * step * 2.0 ** -8 + np.abs(w) * 2.0 ** -8 + 1e-12)


def test_sanitize_rules():
    inf, nan = np.inf, np.nan
    z = np.array([
        [1.0, 2.0, 3.0],          # finite
        [nan, 2.0, -inf],         # NaN -> -inf
        [inf, 5.0, inf],          # +inf row -> uniform over +inf ids
        [nan, -inf, -inf],        # invalid
        [-inf, inf, nan],         # +inf with NaN
    ])
    s, f = O.sanitize(z)
    assert np.array_equal(s[0], [1.0, 2.0, 3.0]) and f[0] == 0
    assert np.array_equal(s[1], [-inf, 2.0, -inf]) and f[1] == O.ROW_NONFINITE
    assert np.array_equal(s[2], [0.0, -inf, 0.0]) and f[2] == O.ROW_NONFINITE | O.ROW_POSINF
    assert np.all(s[3] == -inf) and f[3] == O.ROW_NONFINITE | O.ROW_INVALID
    assert np.array_equal(s[4], [-inf, 0.0, -inf]) and f[4] == O.ROW_NONFINITE | O.ROW_POSINF


def test_argmax_lowest_id_on_exact_ties_and_invalid_rows():
    z = np.array([[1.0, 3.0, 3.0, 2.0], [-np.inf] * 4, [5.0, 5.0, 5.0, 5.0]])
    assert list(O.argmax_lowest_f32(z)) == [1, -1, 0]
    # values that differ in fp64 but round to the same fp32 tie -> lowest id
    a = 1.0
    b = 1.0 + 2.0 ** -40
    assert O.argmax_lowest_f32(np.array([[0.0, a, b]]))[0] == 1
    assert O.top2_gap(np.array([[0.0, 3.0, 1.0]]))[0] == 2.0
    assert O.top2_gap(np.array([[0.0, -np.inf, -np.inf]]))[0] == np.inf


def test_logsumexp_matches_library_and_handles_minus_inf():
    rng = np.random.default_rng(2)
    s = rng.standard_normal((6, 1000)) * 30
    s[1, ::3] = -np.inf
    assert np.allclose(O.logsumexp_rows(s), logsumexp(s, axis=-1), rtol=0, atol=1e-12)
    assert O.logsumexp_rows(np.full((1, 5), -np.inf))[0] == -np.inf


def test_draft_rows_uses_only_the_first_n_draft_rows():
    rng = np.random.default_rng(4)
    V, d, nd = 300, 16, 100
    W = rng.standard_normal((V, d))
    h = rng.standard_normal((3, d))
    W[150] = h[0] * 50            # a huge logit outside the draft vocabulary
    r = O.draft_rows(W, nd, h, 0.0, 0, 0, 0, 1e-4)
    z = h @ W[:nd].T
    assert list(r["token"]) == list(np.argmax(z, axis=1))
    assert np.allclose(r["lse"], logsumexp(z, axis=1))
    assert np.all(r["token"] < nd)


def test_verify_rows_stats_and_drafted_logit():
    rng = np.random.default_rng(5)
    V, d = 64, 8
    W = rng.standard_normal((V, d))
    hv = rng.standard_normal((2, 3, d))
    drafts = np.array([[3, 60], [-1, 7]])
    T = 0.7
    r = O.verify_rows(W, hv, drafts, T, 9, 0, 1e-4)
    z = hv @ W.T
    assert np.array_equal(r["argmax"], np.argmax(z, axis=-1))
    assert np.allclose(r["lse"], logsumexp(z / T, axis=-1))
    assert r["z_tok"][0, 0] == z[0, 0, 3] and r["z_tok"][0, 1] == z[0, 1, 60]
    assert r["z_tok"][1, 0] == -np.inf and r["z_tok"][1, 1] == z[1, 1, 7]
    assert np.all(r["z_tok"][:, 2] == -np.inf)
    # the sample is the Gumbel-max pick on stream 2 at each row
    for b in range(2):
        for i in range(3):
            G = O.gumbel_noise(9, 2, i, b, 0, V)
            assert r["sample"][b, i] == np.argmax(z[b, i] / T + G)


@pytest.mark.parametrize("wtype", ["f32", "bf16", "q4a32"])
def test_synth_heads_decode_near_their_source(wtype):
    rng = np.random.default_rng(0)
    head = synth.make_head(rng, 64, 64, wtype, keep_source=True)
    W = O.head_weights_f64(head)
    src = head.source if head.source is not None else head.w
    tol = {"f32": 0, "bf16": 2.0 ** -8 * 0.1, "q4a32": 0.03}[wtype]
    assert np.max(np.abs(W - src)) <= tol
