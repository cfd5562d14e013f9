"""Pins for the oracle's waste accounting against the interview post's simulation (CPU only)."""
import json
import os
from fractions import Fraction

import numpy as np

from oracle.accounting import tail_waste, waste_report
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
