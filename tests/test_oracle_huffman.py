"""Pins for the oracle's Huffman construction and canonical code.

* optimality: on alphabets of <= 7 symbols the Huffman cost sum(f * len)
  equals the minimum over every length vector that satisfies Kraft's
  inequality (brute force);
* validity: Kraft equality for >= 2 coded symbols, prefix-freeness by a
  pairwise check, and codes consecutive within each length (canonical form);
* the Shannon bound H <= mean length < H + 1 on the synthetic workloads.
"""
import itertools
import math

import numpy as np
import pytest

from oracle import codec
import workloads


def _cost(freq, lengths):
    return sum(int(f) * int(L) for f, L in zip(freq, lengths))


@pytest.mark.parametrize("n", [2, 3, 4, 5, 6, 7])
def test_huffman_is_optimal_brute_force(n):
    rng = np.random.default_rng(100 + n)
    for trial in range(6 if n == 7 else 12):
        freq = list(rng.integers(1, 50, size=n))
        if trial % 3 == 0:
            freq = list(rng.integers(1, 4, size=n))        # many ties
        freq16 = freq + [0] * (16 - n)
        L = codec.huffman_code_lengths(freq16)
        assert all(L[s] == 0 for s in range(n, 16))
        best = None
        for cand in itertools.product(range(1, n), repeat=n):
            if sum(2.0 ** -c for c in cand) <= 1.0 + 1e-12:
                cst = _cost(freq, cand)
                best = cst if best is None or cst < best else best
        assert _cost(freq, L[:n]) == best


def _kraft(lengths):
    from fractions import Fraction
    return sum(Fraction(1, 2 ** int(L)) for L in lengths if L)


def test_kraft_equality_and_prefix_free():
    rng = np.random.default_rng(7)
    for trial in range(200):
        n = int(rng.integers(2, 17))
        freq = np.zeros(16, dtype=np.int64)
        syms = rng.choice(16, size=n, replace=False)
        freq[syms] = rng.integers(1, 10 ** int(rng.integers(1, 8)), size=n)
        L = codec.huffman_code_lengths(freq)
        assert _kraft(L) == 1
        assert max(L) <= 15
        codes = codec.canonical_codes(L)
        words = [format(int(codes[s]), f"0{int(L[s])}b") for s in range(16) if L[s]]
        assert all(len(wd) == int(L[s]) for wd, s in zip(words, [s for s in range(16) if L[s]]))
        for a, b in itertools.permutations(words, 2):
            assert not b.startswith(a)


def test_canonical_codes_consecutive_within_length():
    L = np.array([3, 2, 3, 3, 4, 4, 2, 0, 0, 0, 0, 0, 0, 0, 0, 0])
    assert _kraft(L) == 1
    codes = codec.canonical_codes(L)
    # ordered by (length, symbol): 1,6 (len 2); 0,2,3 (len 3); 4,5 (len 4)
    assert [int(codes[s]) for s in (1, 6)] == [0b00, 0b01]
    assert [int(codes[s]) for s in (0, 2, 3)] == [0b100, 0b101, 0b110]
    assert [int(codes[s]) for s in (4, 5)] == [0b1110, 0b1111]


def test_degenerate_alphabets():
    assert list(codec.huffman_code_lengths([0] * 16)) == [0] * 16
    one = [0] * 16
    one[5] = 99
    L = codec.huffman_code_lengths(one)
    assert L[5] == 1 and sum(L) == 1
    two = [0] * 16
    two[3], two[9] = 1, 1000
    L = codec.huffman_code_lengths(two)
    assert L[3] == 1 and L[9] == 1


def test_worst_case_depth_is_15():
    # Fibonacci-like weights force the deepest tree: 16 symbols -> max length 15
    fib = [1, 1]
    while len(fib) < 16:
        fib.append(fib[-1] + fib[-2])
    L = codec.huffman_code_lengths(fib)
    assert max(L) == 15
    assert _kraft(L) == 1


def _entropy(freq):
    f = np.asarray([x for x in freq if x > 0], dtype=np.float64)
    p = f / f.sum()
    return float(-(p * np.log2(p)).sum())


@pytest.mark.parametrize("wl", ["small", "layer2", "layer4", "stack5"])
def test_shannon_bound_on_workloads(wl):
    if wl == "small":
        w, _ = workloads.small_matrix()
    elif wl == "layer2":
        w = workloads.layer_weight(2, 0, 0, shape=(1024, 4096))
    elif wl == "layer4":
        w = workloads.layer_weight(4, 0, 2, shape=(512, 14336))
    else:
        w = workloads.layer_weight(5, 3, 1, shape=(1024, 4096))
    c = codec.encode(w)
    H = _entropy(c.freq)
    mean_len = _cost(c.freq, c.lengths) / c.freq.sum()
    assert H <= mean_len < H + 1
    # the page's "about 2.6 bits" of exponent information (plausibility band)
    assert 2.3 < H < 3.2
