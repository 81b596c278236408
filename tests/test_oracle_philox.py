"""Pins of the oracle's counter-based generator (Philox4x32-10) and uniform/Gumbel maps.

The oracle's Philox is written from the SC'11 paper.  It is pinned here against an
independent implementation (rocRAND's engine, through its public API, compiled for and
run on the CPU), plus the exact uniform maps and the Gumbel-max theorem.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest
from scipy import stats

from oracle import mtp_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_ref(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
        pytest.skip("hipcc / rocRAND headers not available")
    exe = str(tmp_path_factory.mktemp("rr") / "philox_ref")
    subprocess.run([hipcc, "-O1", "-x", "hip", "--offload-arch=gfx950", "-I/opt/rocm/include",
                    os.path.join(HERE, "philox_rocrand_ref.cpp"), "-o", exe],
                   check=True, capture_output=True, timeout=300)

    def run(triples):
        inp = "".join(f"{s} {u} {o}\n" for s, u, o in triples)
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True, timeout=60)
        return np.array([[int(v) for v in line.split()] for line in out.stdout.strip().splitlines()],
                        dtype=np.uint64)
    return run


def test_philox_matches_rocrand_on_random_counters_and_keys(rocrand_ref):
    rng = np.random.default_rng(7)
    triples = []
    for _ in range(300):
        seed = int(rng.integers(0, 2**63)) | (int(rng.integers(0, 2)) << 63)
        sub = int(rng.integers(0, 2**63))
        off = int(rng.integers(0, 2**40)) * 4       # word-aligned: four words of one counter
        triples.append((seed, sub, off))
    triples += [(0, 0, 0), (2**64 - 1, 2**64 - 1, (2**64 - 4)), (1234, 5, 8)]
    ref = rocrand_ref(triples)
    for (seed, sub, off), want in zip(triples, ref):
        c = off // 4
        got = O.philox4x32_10(c & 0xFFFFFFFF, c >> 32, sub & 0xFFFFFFFF, sub >> 32,
                              seed & 0xFFFFFFFF, seed >> 32)
        assert [int(v) for v in got] == [int(v) for v in want]


def test_philox_words_select_word_by_low_bits(rocrand_ref):
    # element x of (stream, row, b, cycle) = word x & 3 of counter (x >> 2, stream<<8|row, b, cycle)
    seed, stream, row, b, cyc = 0x0123456789ABCDEF, 2, 5, 77, 3
    xs = np.arange(40)
    got = O.philox_words(seed, stream, row, b, cyc, xs)
    sub = b | (cyc << 32)
    triples = [(seed, sub, 4 * ((x >> 2) | (((stream << 8) | row) << 32))) for x in xs[::4]]
    ref = rocrand_ref(triples).reshape(-1)
    assert np.array_equal(got.astype(np.uint64), ref)


def test_uniform_maps_are_exact_and_in_range():
    w = np.array([0, 1, 255, 256, 2**31, 2**32 - 1], dtype=np.uint64)
    ua = O.uniform_accept(w)
    ug = O.uniform_gumbel(w)
    assert ua[0] == 2.0 ** -24 and ua[-1] == 1.0
    assert ug[0] == 2.0 ** -24 and ug[-1] == 1.0 - 2.0 ** -24
    assert np.all(ua > 0) and np.all(ua <= 1) and np.all(ug > 0) and np.all(ug < 1)
    # every value is an fp32 number
    assert np.array_equal(ua.astype(np.float32).astype(np.float64), ua)
    assert np.array_equal(ug.astype(np.float32).astype(np.float64), ug)
    # monotone in the word
    ws = np.sort(np.random.default_rng(1).integers(0, 2**32, 1000).astype(np.uint64))
    assert np.all(np.diff(O.uniform_accept(ws)) >= 0)


def test_words_are_uniform_and_streams_differ():
    xs = np.arange(1 << 16)
    w = O.philox_words(99, 0, 0, 0, 0, xs)
    counts = np.bincount((w >> 24).astype(np.int64), minlength=256)
    assert stats.chisquare(counts).pvalue > 1e-4
    for other in [(1, 0, 0, 0), (0, 1, 0, 0), (0, 0, 1, 0), (0, 0, 0, 1)]:
        w2 = O.philox_words(99, *other, xs[:64])
        assert not np.array_equal(w[:64], w2)
    # same inputs, same words (deterministic)
    assert np.array_equal(w[:64], O.philox_words(99, 0, 0, 0, 0, xs[:64]))


def test_gumbel_max_samples_the_softmax():
    # Gumbel-max theorem: argmax(log w + G) ~ w / sum(w); one request id per draw
    logits = np.log(np.array([0.5, 0.25, 0.125, 0.0625, 0.0625]))
    n = 40000
    G = O.gumbel_noise(5, O.STREAM_RESAMPLE, 0, np.arange(n), 0, logits.size)
    pick = O.argmax_lowest_f32(logits[None, :] + G)
    counts = np.bincount(pick, minlength=logits.size)
    p = stats.chisquare(counts, n * np.exp(logits)).pvalue
    assert p > 1e-4
    # a planted mistake in the noise (ln u instead of -ln(-ln u)) is caught
    u = O.uniform_gumbel(O.philox_words(5, 2, 0, np.arange(n)[:, None], 0, np.arange(logits.size)))
    bad = O.argmax_lowest_f32(logits[None, :] + np.log(u))
    assert stats.chisquare(np.bincount(bad, minlength=logits.size), n * np.exp(logits)).pvalue < 1e-6


def test_trunk_draw_is_keyed_by_position_and_samples_the_softmax():
    # the trunk's own draw (stream 3): one word per (request, position); over positions it
    # samples softmax(z/T) (Gumbel-max), and it does not depend on anything but the position
    T = 0.8
    z = np.array([1.0, 0.4, 0.0, -0.3, -2.0])
    n = 30000
    picks = np.array([O.trunk_sample(z, T, 77, 3, pos)[0] for pos in range(n)])
    p = np.exp(z / T) / np.exp(z / T).sum()
    assert stats.chisquare(np.bincount(picks, minlength=z.size), n * p).pvalue > 1e-4
    # counter layout (x >> 2, 3 << 8, request, position)
    w = O.philox_words(77, 3, 0, 3, 1234, np.arange(z.size))
    u = O.uniform_gumbel(w)
    assert np.array_equal(O.trunk_noise(77, 3, 1234, z.size), -np.log(-np.log(u)))
    assert O.trunk_sample(z, T, 77, 3, 1234)[0] == int(O.argmax_lowest_f32(z / T - np.log(-np.log(u))))
    # another request or position gives other draws; the draft and resample streams differ
    assert not np.array_equal(O.trunk_noise(77, 3, 1234, 8), O.trunk_noise(77, 4, 1234, 8))
    assert not np.array_equal(O.trunk_noise(77, 3, 1234, 8), O.trunk_noise(77, 3, 1235, 8))
    assert not np.array_equal(O.trunk_noise(77, 3, 1234, 8), O.gumbel_noise(77, O.STREAM_RESAMPLE, 0, 3, 1234, 8))
