"""The staggering scheduler's draft-length rule: the oracle against closed forms
and an independent route to the expectation, planted mistakes, and the
library's host policy (vc_sched_*) against the oracle, exactly (no GPU)."""
import ctypes
import itertools
import os

import numpy as np
import pytest

from oracle import sched as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "compressed_kv_draft_amd", "libvc.so")


def expected_by_outcomes(a, k):
    """The same expectation from the distribution of the accepted count n:
    P(n) = a^n (1 - a) for n < k, a^k for n = k; a round emits n + 1 tokens."""
    return sum((n + 1) * (a ** n) * (1 - a) for n in range(k)) + (k + 1) * a ** k


def pin_sched(accept_rate, expected_tokens, choose_k):
    # the estimate: one prior match and one prior mismatch
    assert accept_rate(0, 0) == 0.5 and accept_rate(30, 0) == 31 / 32 and accept_rate(0, 10) == 1 / 12
    # closed forms of the expectation, and the distribution route
    for k in (0, 1, 5, 32):
        assert expected_tokens(1.0, k) == k + 1 and expected_tokens(0.0, k) == 1.0
    assert expected_tokens(0.5, 1) == 1.5
    for a, k in itertools.product((0.1, 0.5, 0.9, 0.99), (1, 2, 7, 32)):
        assert abs(expected_tokens(a, k) - expected_by_outcomes(a, k)) <= 1e-12 * (k + 1), (a, k)
    # near-certain acceptance and verification dearer than a draft step:
    # (k+1)/(k t_d + t_r) grows with k, so the longest round wins
    assert choose_k(10 ** 9, 0, 1.0, 0.0, 20.0, 1, 40) == 40
    # ... but with a draft step dearer than verification it shrinks: the shortest wins
    assert choose_k(10 ** 9, 0, 5.0, 0.0, 1.0, 1, 40) == 1
    # hopeless drafts, unstaggered: the shortest round
    assert choose_k(0, 10 ** 9, 1.0, 0.0, 20.0, 1, 40) == 1
    # poor drafts (a = 0.1), staggered beside 10 draft steps' worth of the
    # other group's work: drafting up to that length is free and still adds
    # expected tokens, so k = 10, and no more
    assert choose_k(0, 8, 1.0, 10.0, 20.0, 1, 40) == 10
    assert choose_k(0, 8, 1.0, 10.5, 20.0, 1, 40) == 10
    # bounds are respected
    assert choose_k(0, 8, 1.0, 10.0, 20.0, 12, 40) == 12
    assert choose_k(10 ** 9, 0, 1.0, 0.0, 20.0, 1, 8) == 8
    # an interior optimum, checked against a hand computation: a = 0.5 (no
    # history), t_d = 1, t_r = 2: k=1: 1.5/3 = .5, k=2: 1.75/4 = .4375 -> 1;
    # a = 31/32 (30 accepted): tokens grow nearly linearly until a^k decays
    assert choose_k(0, 0, 1.0, 0.0, 2.0, 1, 8) == 1
    rates = [S.expected_tokens(31 / 32, k) / (k + 2.0) for k in range(1, 65)]
    assert choose_k(30, 0, 1.0, 0.0, 2.0, 1, 64) == 1 + int(np.argmax(rates))
    # ties go to the shorter round: at a = 1e-18 every round emits 1.0 token
    # in fp64 and every k up to the overlap costs the same
    assert choose_k(0, 10 ** 18, 1.0, 8.0, 1.0, 1, 40) == 1


def test_sched_oracle_pins():
    pin_sched(S.accept_rate, S.expected_tokens, S.choose_k)


def test_sched_pins_catch_planted_mistakes():
    def no_bonus(a, k):                   # forgets the verifier's token
        return S.expected_tokens(a, k) - 1.0

    def no_prior(acc, rej):               # raw ratio
        return acc / max(acc + rej, 1)

    def ties_long(acc, rej, td, to, tr, lo, hi):
        a = S.accept_rate(acc, rej)
        r = {k: S.expected_tokens(a, k) / S.round_time(k, td, to, tr) for k in range(lo, hi + 1)}
        b = max(r.values())
        return max(k for k, v in r.items() if v == b)

    def summed_time(acc, rej, td, to, tr, lo, hi):   # no overlap: k t_d + t_o + t_r
        a = S.accept_rate(acc, rej)
        r = {k: S.expected_tokens(a, k) / (k * td + to + tr) for k in range(lo, hi + 1)}
        b = max(r.values())
        return min(k for k, v in r.items() if v == b)

    def choose_with(rate=S.accept_rate, tokens=S.expected_tokens):
        def f(acc, rej, td, to, tr, lo, hi):
            a = rate(acc, rej)
            r = {k: tokens(a, k) / S.round_time(k, td, to, tr) for k in range(lo, hi + 1)}
            b = max(r.values())
            return min(k for k, v in r.items() if v == b)
        return f

    for name, args in {
        "no_bonus": (S.accept_rate, no_bonus, choose_with(tokens=no_bonus)),
        "no_prior": (no_prior, S.expected_tokens, choose_with(rate=no_prior)),
        "ties_long": (S.accept_rate, S.expected_tokens, ties_long),
        "summed_time": (S.accept_rate, S.expected_tokens, summed_time),
    }.items():
        with pytest.raises(AssertionError):
            pin_sched(*args)
        print("caught", name)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libvc.so is not built (run __graft_entry__.build())")
    L = ctypes.CDLL(LIB)
    L.vc_sched_accept_rate.restype = ctypes.c_double
    L.vc_sched_accept_rate.argtypes = [ctypes.c_longlong, ctypes.c_longlong]
    L.vc_sched_expected_tokens.restype = ctypes.c_double
    L.vc_sched_expected_tokens.argtypes = [ctypes.c_double, ctypes.c_int]
    L.vc_sched_choose_k.restype = ctypes.c_int
    L.vc_sched_choose_k.argtypes = [ctypes.c_longlong, ctypes.c_longlong, ctypes.c_double, ctypes.c_double,
                                    ctypes.c_double, ctypes.c_int, ctypes.c_int]
    return L


def test_library_policy_equals_oracle(lib):
    """Same fp64 operations in the same order: every decision is identical."""
    rng = np.random.default_rng(3)
    for acc, rej in [(0, 0), (5, 1), (300, 2), (31, 9), (10 ** 6, 3), (0, 50)]:
        assert lib.vc_sched_accept_rate(acc, rej) == S.accept_rate(acc, rej)
    for a in (0.0, 0.3, 0.97, 1.0):
        for k in (0, 1, 17, 64):
            assert lib.vc_sched_expected_tokens(a, k) == S.expected_tokens(a, k)
    n = 0
    for _ in range(3000):
        acc = int(rng.integers(0, 2000))
        rej = int(rng.integers(0, 60))
        td = float(rng.uniform(0.01, 5.0))
        to = float(rng.choice([0.0, rng.uniform(0.0, 200.0)]))
        tr = float(rng.uniform(0.0, 100.0))
        lo = int(rng.integers(1, 20))
        hi = int(rng.integers(lo, 65))
        got = lib.vc_sched_choose_k(acc, rej, td, to, tr, lo, hi)
        assert got == S.choose_k(acc, rej, td, to, tr, lo, hi), (acc, rej, td, to, tr, lo, hi)
        n += got != lo
    assert n > 500   # the grid reaches interior and upper optima, not only k_min


def test_library_policy_rejects_bad_input(lib):
    f = lib.vc_sched_choose_k
    assert f(-1, 0, 1.0, 0.0, 1.0, 1, 8) == -1
    assert f(0, 0, 0.0, 0.0, 1.0, 1, 8) == -1
    assert f(0, 0, 1.0, -1.0, 1.0, 1, 8) == -1
    assert f(0, 0, 1.0, 0.0, float("nan"), 1, 8) == -1
    assert f(0, 0, 1.0, 0.0, float("inf"), 1, 8) == -1
    assert f(0, 0, 1.0, 0.0, 1.0, 0, 8) == -1 and f(0, 0, 1.0, 0.0, 1.0, 9, 8) == -1
    assert f(0, 0, 1.0, 0.0, 1.0, 1, 65) == -1
    assert np.isnan(lib.vc_sched_expected_tokens(1.5, 3)) and np.isnan(lib.vc_sched_accept_rate(-1, 0))
