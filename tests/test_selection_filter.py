"""The threshold the Block-Sparse selection filters long rows with (host
check of the invariant, no GPU): with a row's keys dealt to 64 lanes (block
c = lane + 64 u in slot u of lane `lane`, absent blocks key 0), the k-th
largest T' of the 128 per-lane top-2 keys is at most the row's k-th largest
key T for every k <= 128, so the keys >= T' contain the whole selection."""
import numpy as np
import pytest


def per_lane_top2_threshold(keys: np.ndarray, k: int) -> int:
    lanes = keys.reshape(-1, 64).T                       # [lane, slot]
    top2 = -np.sort(-lanes, axis=1)[:, :2].reshape(-1)   # 128 values, distinct slots
    return int(np.sort(top2)[::-1][k - 1])


@pytest.mark.parametrize("kind", ["random", "ties", "few_values", "hot", "short"])
def test_threshold_never_exceeds_the_kth_key(kind):
    rng = np.random.default_rng(11)
    for trial in range(200):
        R = int(rng.choice([16, 32, 64]))
        n = int(rng.integers(1, 64 * R + 1)) if kind == "short" else int(rng.integers(64 * R // 2, 64 * R + 1))
        keys = np.zeros(64 * R, np.int64)
        if kind == "random":
            keys[:n] = rng.integers(1, 2 ** 32, n)
        elif kind == "ties":
            keys[:n] = 0x9000_0000
        elif kind == "few_values":
            keys[:n] = 0x8000_0000 + rng.integers(0, 3, n)
        elif kind == "hot":
            keys[:n] = 0x8000_0000 + rng.integers(0, 1000, n)
            keys[rng.choice(n, min(n, 16), replace=False)] += 10 ** 6
        else:
            keys[:n] = rng.integers(1, 2 ** 32, n)
        a = n - 1
        keys[0] = keys[a] = 0xFFFF_FFFF  # forced blocks
        for k in (1, 2, 20, 100, 128):
            kk = min(k, n)
            T = int(np.sort(keys[:n])[::-1][kk - 1])
            Tp = per_lane_top2_threshold(keys, kk)
            assert Tp <= T, (kind, trial, n, kk)
            assert np.count_nonzero(keys[:n] >= Tp) >= kk
