"""CPU tests of the decode's split plan, through the library's host replay
(qkmla_plan_segments / qkmla_plan_merge_sources use the same plan helpers as
the kernels): every tile of every valid sequence is processed exactly once,
each workgroup stays inside its range, partial slots are never written twice,
and the merge reads exactly the partials that were written."""
import os

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
pytestmark = pytest.mark.skipif(
    not os.path.exists(os.path.join(ROOT, "mla_latent_decode_amd", "libqkmla.so")),
    reason="libqkmla.so not built")

TILE = 32


def _tiles(L, L_cap):
    return (L + TILE - 1) // TILE if 1 <= L <= L_cap else 0


def _check_plan(lens, L_cap, n_wg):
    from mla_latent_decode_amd import ops
    segs = ops.plan_segments(lens, L_cap, n_wg)
    ntiles = [_tiles(L, L_cap) for L in lens]
    N = sum(ntiles)
    prefix = np.concatenate([[0], np.cumsum(ntiles)])
    covered = [np.zeros(n, dtype=np.int32) for n in ntiles]
    written = set()
    per_wg = {}
    for p, b, t0, t1, kind in segs:
        assert 0 <= p < n_wg and 0 <= b < len(lens)
        assert 0 <= t0 < t1 <= ntiles[b], (p, b, t0, t1)
        covered[b][t0:t1] += 1
        # inside the workgroup's range of the flattened tile order
        lo, hi = (p * N) // n_wg, ((p + 1) * N) // n_wg
        assert lo <= prefix[b] + t0 and prefix[b] + t1 <= hi
        whole = (t0 == 0 and t1 == ntiles[b])
        assert (kind == -1) == whole
        if kind >= 0:
            assert (p, kind) not in written
            written.add((p, kind))
        per_wg.setdefault(p, []).append((prefix[b] + t0, prefix[b] + t1, kind))
    for c in covered:
        assert np.all(c == 1)
    for p, lst in per_wg.items():
        # contiguous, in order, covering the whole range
        lo, hi = (p * N) // n_wg, ((p + 1) * N) // n_wg
        assert lst[0][0] == lo and lst[-1][1] == hi
        for (a0, a1, _), (b0, b1, _) in zip(lst, lst[1:]):
            assert a1 == b0
        kinds = [k for _, _, k in lst]
        assert all(k == -1 for k in kinds[1:-1])        # middle segments are whole
        if len(kinds) > 1:
            assert kinds[0] in (-1, 0) and kinds[-1] in (-1, 1)
    # merge sources = written partials of each sequence
    for b, L in enumerate(lens):
        src = {tuple(x) for x in ops.plan_merge_sources(lens, L_cap, n_wg, b)}
        want = {(p, k) for p, bb, _, _, k in segs if bb == b and k >= 0}
        assert src == want, (b, src, want)
    return segs


@pytest.mark.parametrize("seed", range(40))
def test_random_plans(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 200))
    L_cap = int(rng.integers(1, 5000))
    lens = rng.integers(-3, L_cap + 40, size=B)          # includes invalid lengths
    n_wg = int(rng.choice([1, 2, 7, 64, 256, 1000, int(rng.integers(1, 3000))]))
    _check_plan(lens, L_cap, n_wg)


@pytest.mark.parametrize("lens,L_cap,n_wg", [
    ([4096] * 16, 4096, 256),                 # 16 x 4k: every sequence split 16 ways
    ([32768] * 4, 32768, 256),
    ([262144], 262144, 256),                  # one sequence over all workgroups
    ([45, 200], 200, 14),                     # more workgroups than tiles
    ([31, 33, 95, 97, 1, 2], 97, 24),
    ([700, 333, 64], 700, 1),                 # one workgroup, three segments
    ([0, 5, 0, 7], 10, 3),                    # invalid lengths only skip
])
def test_workload_plans(lens, L_cap, n_wg):
    segs = _check_plan(lens, L_cap, n_wg)
    assert len(segs) > 0


def test_ragged_workload_plan_balances_tiles():
    from mla_latent_decode_amd import ops
    rng = np.random.default_rng(1004)
    lens = rng.integers(1024, 16384, size=64, endpoint=True)
    segs = _check_plan(lens, 16384, 256)
    per_wg = np.zeros(256, dtype=np.int64)
    for p, b, t0, t1, k in segs:
        per_wg[p] += t1 - t0
    assert per_wg.max() - per_wg.min() <= 1          # tile-balanced
    # at most two partials per workgroup
    assert max(np.bincount(segs[segs[:, 4] >= 0][:, 0], minlength=256)) <= 2
