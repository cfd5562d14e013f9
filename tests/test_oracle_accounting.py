"""Pins for the oracle's waste accounting against the interview post's simulation (CPU only)."""
import json
import os
from fractions import Fraction

import numpy as np

from oracle.accounting import class_block_size, paged_footprint, tail_waste, waste_report
from synth import skewed_lengths

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _mixture_support(g):
    """Every length of the mix repeated in proportion to its probability (exact weights)."""
    weights = [Fraction(p).limit_denominator(100) / (hi - lo) for p, lo, hi in g["mix"]]
    den = 1
    for w in weights:
        den = den * w.denominator // np.gcd(den, w.denominator)
    lengths = []
    for (p, lo, hi), w in zip(g["mix"], weights):
        lengths.append(np.repeat(np.arange(lo, hi), int(w * den)))
    return np.concatenate(lengths)


def test_closed_form_expectation_of_the_mix():
    """E[len] = 663.5 and E[tail waste] = 7.5 at B = 16, computed by hand from the mix."""
    g = json.load(open(os.path.join(GOLDEN, "waste_simulation.json")))
    support = _mixture_support(g)
    assert abs(support.mean() - 663.5) < 1e-9
    cont, paged, gain = waste_report(support, g["max_len"], g["block_size"])
    assert abs(cont - (1 - 663.5 / 4096)) < 1e-12
    assert abs(paged - 7.5 / 671.0) < 1e-12
    assert abs(gain - 4096 / 671.0) < 1e-12


def test_seeded_run_and_the_printed_run_fall_in_the_same_band():
    """Sampling bands from 300 seeded runs of N = 1000 contain both our run and the page's."""
    g = json.load(open(os.path.join(GOLDEN, "waste_simulation.json")))
    runs = np.array([waste_report(skewed_lengths(np.random.default_rng(s), g["num_requests"]),
                                  g["max_len"], g["block_size"]) for s in range(300)])
    lo = np.percentile(runs, 0.5, axis=0)
    hi = np.percentile(runs, 99.5, axis=0)
    printed = g["printed"]
    page = np.array([printed["contiguous_waste_pct"] / 100, printed["paged_waste_pct"] / 100,
                     printed["concurrency_gain"]])
    tol = np.array([0.0005, 0.0005, 0.05])  # the page rounds to one decimal
    assert ((page + tol >= lo) & (page - tol <= hi)).all(), (lo, hi, page)
    ours = np.array(waste_report(skewed_lengths(np.random.default_rng(1000), 1000), 4096, 16))
    assert ((ours >= lo) & (ours <= hi)).all()
    # and the bands sit around the closed form
    assert lo[0] < 1 - 663.5 / 4096 < hi[0] and lo[2] < 4096 / 671 < hi[2]


def test_33_token_request_figures():
    """31 slots wasted at B = 32: 31/64 of the allocation (48%) and 31/33 of the tokens (94%)."""
    g = json.load(open(os.path.join(GOLDEN, "block_size_tradeoff.json")))["cases"][0]
    w = tail_waste(g["request_tokens"], g["block_size"])
    assert w == g["wasted_tokens"]
    assert round(100 * w / 64) == 48 and round(100 * w / 33) == 94
    assert tail_waste(33, 16) == 15


def test_paged_waste_is_below_one_block_per_request():
    rng = np.random.default_rng(0)
    L = skewed_lengths(rng, 5000)
    for B in (16, 32):
        w = np.array([tail_waste(x, B) for x in L])
        assert w.min() >= 0 and w.max() <= B - 1


def test_length_class_footprint_hand_example():
    """33, 100 and 5000 tokens with the class threshold at 1024: 3 and 7 blocks of 16
    (15 and 12 slots wasted), 157 blocks of 32 (24 wasted)."""
    L = [33, 100, 5000]
    Bs = [class_block_size(x, 1024) for x in L]
    assert Bs == [16, 16, 32]
    assert paged_footprint(L, Bs) == (48 + 112 + 5024, 15 + 12 + 24, 3 + 7 + 157)
    assert paged_footprint(L, [16] * 3) == (48 + 112 + 5008, 15 + 12 + 8, 3 + 7 + 313)
    assert paged_footprint(L, [32] * 3) == (64 + 128 + 5024, 31 + 28 + 24, 2 + 4 + 157)
    assert class_block_size(1023, 1024) == 16 and class_block_size(1024, 1024) == 32


def test_length_class_expectation_of_the_doubled_mix():
    """Doubled mix (70% U{64..1023}, 25% U{1024..4095}, 5% U{4096..8191}), threshold 1024.
    By hand: each range spans whole periods of 16 and 32, so the mean tail waste is
    (B - 1) / 2 within a range: 7.5 at 16, 15.5 at 32, and 0.7 * 7.5 + 0.3 * 15.5 = 9.9
    with the class choice.  Mean table entries = (E[len] + E[waste]) / B per range, with
    range means 543.5, 2559.5, 6143.5: 83.4375 at 16, 41.96875 at 32, and
    0.7 * 551 / 16 + 0.25 * 2575 / 32 + 0.05 * 6159 / 32 = 53.846875 by class."""
    ranges = [(Fraction(7, 10), 64, 1024), (Fraction(1, 4), 1024, 4096), (Fraction(1, 20), 4096, 8192)]

    def expect(choose):
        waste = entries = Fraction(0)
        for p, lo, hi in ranges:
            Ls = list(range(lo, hi))
            _, w, e = paged_footprint(Ls, [choose(x) for x in Ls])
            waste += p * Fraction(w, len(Ls))
            entries += p * Fraction(e, len(Ls))
        return waste, entries

    assert expect(lambda x: 16) == (Fraction(15, 2), Fraction(834375, 10000))
    assert expect(lambda x: 32) == (Fraction(31, 2), Fraction(4196875, 100000))
    assert expect(lambda x: class_block_size(x, 1024)) == (Fraction(99, 10), Fraction(53846875, 1000000))
