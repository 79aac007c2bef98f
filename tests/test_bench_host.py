"""Host-side logic of bench.py (no GPU): the graph step count and the lock-step work
statistics reported with the prefill roofline."""
import numpy as np

import bench


def test_graph_steps_divides_and_caps():
    for steps in (1, 5, 7, 13, 20, 50, 200, 1000):
        s = bench.graph_steps(steps)
        assert steps % s == 0 and 1 <= s <= 16
        assert steps // s >= min(20, steps)  # at least 20 timed replays when K allows it
        # the largest such divisor
        assert all(steps % d or steps // d < min(20, steps) for d in range(s + 1, min(16, steps) + 1))
    assert bench.graph_steps(20) == 1 and bench.graph_steps(200) == 10


class _Ev:
    def __init__(self, t):
        self.t = t

    def elapsed_time(self, other):
        return other.t - self.t


def test_median_of_event_pairs():
    pairs = [(_Ev(0.0), _Ev(x)) for x in (5.0, 1.0, 3.0)]
    assert bench.median_ms(pairs) == (3.0, 3.0)
    pairs.append((_Ev(10.0), _Ev(17.0)))
    assert bench.median_ms(pairs) == (4.0, 4.0)


def test_baseline_rows_strata():
    head, ends, rest = bench.baseline_rows(1000, 16, 4, seed=3)
    assert head == list(range(32))
    assert ends == [p for p in range(1000 - 128, 1000) if (p + 1) % 16 == 0] + [999]
    assert sorted(head + ends + rest) == list(range(1000))  # every row once


def test_tie_band_rule():
    assert not bench._tie_band(np.array([3.0, 2.0, 1.0]), 3)       # every block kept
    assert bench._tie_band(np.array([1.0, 0.9995, 0.0]), 1)         # gap 5e-4 relative
    assert not bench._tie_band(np.array([1.0, 0.99, 0.0]), 1)       # gap 1e-2 relative


def test_compulsory_bytes_of_prefill():
    from block_sparse_attention_37_amd import synth as S
    w = S.WORKLOADS["long_prefill_bf16_128k"]
    T = w.seq
    want = T * (32 * 128 * 2 * 2 + 64 * 4 + 32 * 4) + T * 4 * 128 * 2 * 2
    assert bench.compulsory_bytes(w) == want


def _brute(sel, pos, block, step):
    tot = 0
    for t0 in range(0, len(pos), step):
        rows = [i for i in range(t0, min(len(pos), t0 + step)) if pos[i] >= 0]
        blocks = set()
        for i in rows:
            n = (pos[i] + 1) // block
            blocks |= {int(j) for j in sel[i] if 0 <= j < n}
            if (pos[i] + 1) % block:
                blocks.add(int(pos[i] // block))
        tot += len(blocks) * len(rows)
    return tot


def test_union_stats_matches_brute_force():
    rng = np.random.default_rng(0)
    for _ in range(60):
        block = int(rng.choice([4, 8, 16]))
        n_q = int(rng.integers(1, 90))
        kv_len = n_q + int(rng.integers(-10, 20))  # below n_q: padding rows in front
        k = int(rng.integers(1, 6))
        pos = np.arange(n_q) + kv_len - n_q
        sel = np.full((n_q, k), -1)
        for i, p in enumerate(pos):
            n = (p + 1) // block if p >= 0 else 0
            m = min(k, n)
            if m:
                sel[i, :m] = np.sort(rng.choice(n, m, replace=False))
        mq, pw = 8, 2
        tile, wave, need = bench.union_stats(sel, pos, block, mq, pw)
        assert tile == _brute(sel, pos, block, mq)
        assert wave == _brute(sel, pos, block, pw)
        assert need == sum(int((sel[i] >= 0).sum()) + int((pos[i] + 1) % block != 0)
                           for i in range(n_q) if pos[i] >= 0)
        assert need <= wave <= tile  # a wave's union covers its rows; a tile's covers its waves'


def test_prefill_tile_shape():
    assert bench.prefill_tile_shape(16, 2, 128) == (32, 4)   # G = 8: 4 positions per wave
    assert bench.prefill_tile_shape(32, 1, 64) == (8, 1)     # G = 32
    assert bench.prefill_tile_shape(16, 2, 256) == (16, 2)   # 16-row tiles at D = 256
    assert bench.prefill_tile_shape(32, 1, 256) == (8, 1)    # two 16-row tiles of one position
