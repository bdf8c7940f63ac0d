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
