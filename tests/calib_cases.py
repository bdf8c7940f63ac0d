"""Hand-built calibration rows that pin the two rules of the table builder a shared mistake could
flip in the oracle and the device alike (OSC page §3.1, Algorithm 1, read as: a row is an event
when the group's largest |x| is strictly above alpha times the group's mean |x|; the event channel
is the lowest arg-max; with m entries per group, the m largest |x| taken lower channel first among
equal magnitudes).

Every value is exact in bf16, and every sum, mean and alpha * mean below is exact in fp64, so the
boundary cases sit exactly on the threshold.  The expected tables are derived by hand in the
comments (alpha = 5, rho = 0.35, G = 32), not computed by any implementation.
"""
import numpy as np

G = 32
ALPHA = 5.0
RHO = 0.35


def _group(spec, n_fill=0, fill=1.0):
    """One calibration row of a group: channels from `spec` {channel: value}, then `n_fill` channels
    of `fill` in the lowest free slots, the rest 0."""
    g = np.zeros(G, np.float64)
    for c, v in spec.items():
        g[c] = v
    free = [c for c in range(G) if c not in spec]
    for c in free[:n_fill]:
        g[c] = fill
    return g


# (name, row of the group, expected L for m = 1, expected L for m = 2)
GROUPS = [
    # in-row tie: |-50| = |50| at channels 3 and 11; 30 ones: mean = 130/32 = 4.0625, 5 * mean =
    # 20.3125 < 50, so every row is an event of the LOWEST arg-max, channel 3 (the last arg-max, or a
    # '>=' scan, would give 11).  m = 2: both are events, ranked 3 then 11.
    ("tie_pair", _group({3: -50.0, 11: 50.0}, n_fill=30), [3], [3, 11]),
    # exactly on the threshold: 5 and 27 ones, 4 zeros: sum 32, mean 1, 5 * mean = 5 = max.  Not an
    # event (strict '>'): no events, L = -1.
    ("on_threshold", _group({20: 5.0}, n_fill=27), [-1], [-1, -1]),
    # just above it: 5 and 26 ones: mean 31/32, 5 * mean = 4.84375 < 5: an event of channel 20
    ("above_threshold", _group({20: 5.0}, n_fill=26), [20], [20, -1]),
    # the second channel exactly on the threshold: 40, 10 and 14 ones: sum 64, mean 2, 5 * mean = 10.
    # Channel 4 (40) is an event on every row, channel 7 (10) never is.
    ("second_on_threshold", _group({4: 40.0, 7: 10.0}, n_fill=14), [4], [4, -1]),
    # one fewer one: sum 63, mean 1.96875, 5 * mean = 9.84375 < 10: both are events
    ("second_above_threshold", _group({4: 40.0, 7: 10.0}, n_fill=13), [4], [4, 7]),
    # three-way tie at 50 on channels 5, 9, 20 and 29 ones: sum 179, 5 * mean = 27.96875 < 50.
    # m = 1: channel 5; m = 2: the two lowest, 5 then 9 (never 20)
    ("tie_triple", _group({20: 50.0, 9: -50.0, 5: 50.0}, n_fill=29), [5], [5, 9]),
    # tie between the first and the last channel: offset 0 is a valid entry and wins
    ("tie_ends", _group({0: -64.0, 31: 64.0}, n_fill=30), [0], [0, 31]),
]


def calibration_rows(R: int = 64) -> np.ndarray:
    """R identical calibration rows holding every group above side by side: [R, G * len(GROUPS)]
    float64, exact in bf16."""
    row = np.concatenate([g for _, g, _, _ in GROUPS])
    return np.tile(row, (R, 1))


def expected(m: int) -> np.ndarray:
    """The hand-derived table slice: [K] for m = 1, [K, 2] for m = 2."""
    if m == 1:
        return np.array([e1[0] for _, _, e1, _ in GROUPS], np.int32)
    return np.array([e2 for _, _, _, e2 in GROUPS], np.int32)


def expected_events(R: int = 64) -> np.ndarray:
    """Rows with at least one event per group (m-independent here: every row of a group is alike)."""
    return np.array([0 if e1[0] < 0 else R for _, _, e1, _ in GROUPS], np.int32)
