"""Host logic of the block executor (w4a4_outlier_split_amd/block.py) that needs no GPU: the §2.2
clustering-density average and §2.3's per-module rule, against the oracle's independent C
implementation and hand values."""
import numpy as np
import pytest

import oracle

blk = pytest.importorskip("w4a4_outlier_split_amd.block", reason="libosc.so not built")


def test_mean_density_matches_the_oracle():
    rng = np.random.default_rng(0)
    for m in (1, 2, 3):
        K = 64
        events = rng.integers(0, 50, K).astype(np.int32)
        events[::7] = 0
        hits = np.minimum(rng.integers(0, 60, (K, m)), events[:, None]).astype(np.int32)
        assert blk.mean_density(hits, events) == pytest.approx(oracle.mean_density(hits, events), abs=1e-15)


def test_rule_boundary():
    assert blk.DENSITY_THRESHOLD == 0.35
    # a density of exactly 35 % keeps the OSC path (§2.3: below 35 % falls back)
    hits = np.array([35, 7], np.int32)
    events = np.array([100, 20], np.int32)
    assert blk.mean_density(hits, events) == pytest.approx(0.35)
    assert blk.mean_density(np.zeros(4, np.int32), np.zeros(4, np.int32)) == 0.0


def test_two_share_and_group_size_rule():
    L = np.array([[3, 7], [5, -1], [-1, -1], [0, 9]], np.int32)
    assert blk.two_share(L) == pytest.approx(2 / 3)          # 3 protected groups, 2 with a second channel
    assert blk.two_share(np.full((4, 2), -1, np.int32)) == 0.0
    assert blk.choose_group_size({64: 0.5, 32: 0.05, 16: 0.0}) == 32   # largest G within tolerance
    assert blk.choose_group_size({64: 0.1, 32: 0.0, 16: 0.0}) == 64    # the tolerance is inclusive
    assert blk.choose_group_size({64: 0.6, 32: 0.4, 16: 0.45}) == 32   # none qualifies: smallest share
    assert blk.choose_group_size({64: 0.3, 32: 0.3, 16: 0.3}) == 64    # ties: the larger G


def test_group_size_rule_on_the_oracles_tables():
    """The rule on tables the oracle builds: outliers planted one per 32-channel block (the QKV
    recipe) keep G = 32 (at G = 64 about half the protected groups hold two); one per 64-channel
    block allows G = 64."""
    import synth
    q = synth.qkv(S=16)
    shares = {G: blk.two_share(oracle.build_table_multi(q.calib, G, 2)[0]) for G in (64, 32, 16)}
    assert shares[64] > 0.3 and shares[32] == 0.0
    assert blk.choose_group_size(shares) == 32
    rng = np.random.default_rng(3)
    H = 1024
    plant = synth.Plant(np.arange(0, H // 32, 2), rng.integers(0, 32, H // 64), rng.uniform(40, 100, H // 64))
    cal = synth.draw_x_bernoulli_spikes(512, H, plant, 4, None)
    shares = {G: blk.two_share(oracle.build_table_multi(cal, G, 2)[0]) for G in (64, 32, 16)}
    assert shares[64] == 0.0
    assert blk.choose_group_size(shares) == 64
