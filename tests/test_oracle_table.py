"""Pins for the oracle's suppression-table builder (OSC page §3.1, Algorithm 1; §2.2 clustering density).

find_consistent_outlier is only named on the page; the oracle's reading (event:
max |x| > alpha * mean |x| of the group; candidate: most frequent event channel;
kept when it is the event channel on >= rho of the calibration tokens) is
pinned here by hand-built cases and by its provable properties: planted
persistent channels are recovered, and raising alpha never adds a protected
channel (the page's §5.2 direction).
"""
import numpy as np

import oracle
import synth
from synth import to_bf16_bits


def test_hand_built_group():
    G, R = 32, 10
    x = np.ones((R, 2 * G), np.float32)
    # group 0: channel 7 is 10x on 6 of 10 rows (event: 10 > 5 * mean); channel 3 on 2 rows
    x[:6, 7] = 10.0
    x[6:8, 3] = 10.0
    # group 1: channel 2 is 5.1x on 9 rows: mean = (31 + 5.1)/32 = 1.128..., 5.1 < 5 * 1.128 -> no event
    x[:9, G + 2] = 5.1
    L, hits, events = oracle.build_table(to_bf16_bits(x), G, alpha=5.0, rho=0.35)
    assert L.tolist() == [7, -1]
    assert hits.tolist() == [6, 0] and events.tolist() == [8, 0]
    # with rho above 0.6 the 6/10 channel is no longer persistent enough
    L2, _, _ = oracle.build_table(to_bf16_bits(x), G, alpha=5.0, rho=0.61)
    assert L2.tolist() == [-1, -1]


def test_offset_zero_is_a_valid_entry():
    """Algorithm 1's `j_star if j_star else -1` would drop channel 0; the reading keeps it."""
    x = np.ones((4, 32), np.float32)
    x[:, 0] = 50.0
    L, _, _ = oracle.build_table(to_bf16_bits(x), 32)
    assert L.tolist() == [0]


def test_ties_take_lowest_index():
    x = np.ones((4, 32), np.float32)
    x[:2, 9] = 50.0
    x[2:, 4] = 50.0
    x[:, 20] = 0.5
    L, hits, events = oracle.build_table(to_bf16_bits(x), 32)
    assert L.tolist() == [4] and hits.tolist() == [2] and events.tolist() == [4]


def test_recovers_planted_channels_qkv():
    w = synth.qkv(S=16)
    L, hits, events = oracle.build_table(w.calib, 32)
    expect = synth.planted_table(w.plant, w.H, 32)
    np.testing.assert_array_equal(L, expect)
    assert (L >= 0).sum() == 90


def test_recovers_planted_channels_ffn_and_down():
    for w in (synth.ffn_up(S=16), synth.ffn_down(S=16)):
        L, _, _ = oracle.build_table(w.calib, 32)
        np.testing.assert_array_equal(L, synth.planted_table(w.plant, w.H, 32))


def test_alpha_monotone():
    w = synth.ffn_down(S=16)
    prev = None
    for alpha in (2.0, 3.0, 4.0, 5.0, 6.0, 8.0, 12.0):
        L, _, _ = oracle.build_table(w.calib, 32, alpha=alpha)
        prot = set(np.nonzero(L >= 0)[0].tolist())
        if prev is not None:
            assert prot <= prev
        prev = prot


def test_in_row_ties_and_the_alpha_boundary_m1():
    """Hand-built groups (tests/calib_cases.py, values exact in bf16 and fp64): two or three channels
    sharing the row's max |x| give the event to the lowest of them; a max exactly equal to alpha times
    the group mean is not an event, one just above it is.  Taking the last arg-max, or testing with
    '>=', fails here."""
    import calib_cases as cc
    R = 64
    L, hits, events = oracle.build_table(to_bf16_bits(cc.calibration_rows(R)), cc.G, cc.ALPHA, cc.RHO)
    np.testing.assert_array_equal(L, cc.expected(1))
    np.testing.assert_array_equal(events, cc.expected_events(R))
    np.testing.assert_array_equal(hits, cc.expected_events(R))  # one channel takes every event


def test_in_row_ties_and_the_alpha_boundary_m2():
    """The same groups with two entries per group: the two largest |x| taken lower channel first among
    equals (a three-way tie keeps the two lowest), each an event only strictly above alpha * mean."""
    import calib_cases as cc
    R = 64
    L, hits, events = oracle.build_table_multi(to_bf16_bits(cc.calibration_rows(R)), cc.G, 2, cc.ALPHA, cc.RHO)
    np.testing.assert_array_equal(L, cc.expected(2))
    np.testing.assert_array_equal(events, cc.expected_events(R))
    # every listed channel is the event channel on all R rows
    np.testing.assert_array_equal(hits[L >= 0], R)
