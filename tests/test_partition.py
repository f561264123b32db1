"""Host-side checks of the balanced partition's share bounds.

The decode kernel's balanced mode gives workgroup w of G the pages
[floor(w T / G), floor((w + 1) T / G)) of the batch's T pages, computing the
floor with one IEEE double division.  These tests check, on the CPU with the
same double arithmetic, that this equals the exact integer quotient over the
range the library accepts (at most 65535 sequences of at most 2^24 pages, so
T < 2^40, and G <= 512 workgroups: two per compute unit where the kernel
splits channels), and that the shares tile [0, T) with no
empty share when G <= T.
"""
import math
import random

import pytest

T_MAX = 65535 * (1 << 24)


def share_start_double(w, T, G):
    return math.floor(float(w * T) / float(G))


EDGE_T = [1, 2, 3, 63, 64, 255, 256, 257, 4095, 16384, 32768, 1 << 31, (1 << 31) + 1, (1 << 35) - 1,
          T_MAX - 1, T_MAX, 65535 * 2048, 999983 * 1021]


@pytest.mark.parametrize("T", EDGE_T)
def test_double_floor_matches_integer_quotient(T):
    for G in list(range(1, 65)) + [127, 128, 129, 200, 255, 256, 257, 384, 511, 512]:
        if G > T:
            continue
        for w in range(G + 1):
            assert share_start_double(w, T, G) == (w * T) // G, (w, T, G)


def test_double_floor_random():
    rng = random.Random(0)
    for _ in range(20000):
        T = rng.randrange(1, T_MAX + 1)
        G = rng.randrange(1, 513)
        if G > T:
            continue
        w = rng.randrange(0, G + 1)
        assert share_start_double(w, T, G) == (w * T) // G


@pytest.mark.parametrize("T,G", [(1, 1), (5, 5), (7, 3), (16384, 256), (300, 256), (T_MAX, 256), (16384, 512), (513, 512),
                                 (T_MAX, 512), (T_MAX - 1, 511)])
def test_shares_tile_the_pages(T, G):
    bounds = [share_start_double(w, T, G) for w in range(G + 1)]
    assert bounds[0] == 0 and bounds[-1] == T
    assert all(bounds[i + 1] - bounds[i] >= 1 for i in range(G))
