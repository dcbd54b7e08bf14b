"""Pins of the oracle's waypoint-path reward and its BFS tile path ("boesch.dev DDNet RL post", Reward
Engineering, Version 2: progress along a BFS waypoint path as a high-water mark, a distance-from-path
penalty beyond a 128-unit (about 4 tile) grace zone, +100 finish).

The constants are readings (the oracle's header lists them): the nearest waypoint is searched at the
high-water index and the 8 after it, progress pays 256 units per waypoint, the penalty is one unit per
16 sub-units beyond 1024, and Version 2 has no checkpoint bonus and no time penalty. The values below are
worked by hand on hand-drawn maps; the BFS is pinned by a hand-traced open grid and against scipy's
shortest-path distances.
"""
import numpy as np
import pytest
from scipy.sparse import csr_matrix
from scipy.sparse.csgraph import shortest_path

import oracle

NOOP, RIGHT = 0, 8
F = {name: i for i, name in enumerate(oracle.STATE_FIELDS)}


def flat_map(h=16, w=64, floor_h=4):
    m = np.zeros((h, w), np.uint8)
    m[h - floor_h:, :] = 1
    return m


def v2_env(m, waypoints, ckpts=((16, 11),), fs=1, n=1):
    wp = np.asarray(waypoints, np.int32).reshape(1, -1, 2)
    e = oracle.OracleEnv(m[None], np.asarray(ckpts, np.int32).reshape(1, -1, 2),
                         np.array([[256, 12 * 256 - 192]], np.int32), n, frame_skip=fs, reward_mode=1,
                         waypoints=wp, wp_lens=np.array([wp.shape[1]], np.int32))
    e.reset()
    return e


def test_bfs_open_grid_hand_traced():
    # right is tried before down: the path runs along the top row, then down the last column
    path = oracle.bfs_path(np.zeros((3, 3), np.uint8), (0, 0), (2, 2))
    assert path.tolist() == [[0, 0], [1, 0], [2, 0], [2, 1], [2, 2]]


def test_bfs_blocked_and_unreachable():
    g = np.zeros((3, 5), np.uint8)
    g[:, 2] = 1                                    # a full wall
    assert oracle.bfs_path(g, (0, 0), (4, 0)) is None
    g[2, 2] = 0                                    # a gap at the bottom
    p = oracle.bfs_path(g, (0, 0), (4, 0))
    assert len(p) == 9 and [2, 2] in p.tolist()
    assert oracle.bfs_path(g, (2, 0), (4, 0)) is None            # start inside the wall
    g[1, 4] = 2                                    # platforms block too
    assert len(oracle.bfs_path(g, (0, 0), (4, 0))) == 9
    with pytest.raises(ValueError):
        oracle.bfs_path(g, (0, 0), (4, 0), max_len=8)


def _grid_graph(g):
    h, w = g.shape
    free = (g != 1) & (g != 2)
    rows, cols = [], []
    for r in range(h):
        for c in range(w):
            if not free[r, c]:
                continue
            for dr, dc in ((0, 1), (1, 0)):
                rr, cc = r + dr, c + dc
                if rr < h and cc < w and free[rr, cc]:
                    rows += [r * w + c, rr * w + cc]
                    cols += [rr * w + cc, r * w + c]
    return csr_matrix((np.ones(len(rows)), (rows, cols)), shape=(h * w, h * w))


@pytest.mark.parametrize("seed", range(6))
def test_bfs_is_a_valid_shortest_path(seed):
    rng = np.random.default_rng(seed)
    g = (rng.random((12, 20)) < 0.25).astype(np.uint8) * rng.integers(1, 4, (12, 20)).astype(np.uint8)
    g[0, 0] = g[11, 19] = 0
    dist = shortest_path(_grid_graph(g), unweighted=True, indices=0)[11 * 20 + 19]
    p = oracle.bfs_path(g, (0, 0), (19, 11))
    if not np.isfinite(dist):
        assert p is None
        return
    assert len(p) == dist + 1
    assert p[0].tolist() == [0, 0] and p[-1].tolist() == [19, 11]
    assert (np.abs(np.diff(p, axis=0)).sum(1) == 1).all()        # 4-neighbour steps
    assert all(g[r, c] not in (1, 2) for c, r in p)


def test_progress_along_the_floor_path():
    # path (1,11) .. (16,11) along the floor; walking right (single ticks), x = 264, 280, 304, 336, 376,
    # 424, ...: the box centre x + 96 passes the midpoint 512 between waypoints 0 (centre 384) and 1
    # (centre 640) at tick 6, and 768 at tick 12 (x = 712); each step pays 256 units = 0.25
    m = flat_map()
    path = oracle.bfs_path(m, (1, 11), (16, 11))
    assert path.tolist() == [[c, 11] for c in range(1, 17)]
    e = v2_env(m, path)
    rews = [e.step([RIGHT])[0][0] for _ in range(12)]
    assert rews == [0.0] * 5 + [0.25] + [0.0] * 5 + [0.25]
    assert e.state[0, F["path"]] == 2


def test_distance_penalty_beyond_the_grace_zone():
    # a single far waypoint (20, 11): standing at spawn the box centre is (352, 2976), the waypoint's
    # centre (5248, 2944); d = floor(sqrt(4896^2 + 32^2)) = 4896, so (4896 - 1024) >> 4 = 242 units a tick
    e = v2_env(flat_map(), [[20, 11]], fs=3)
    rew, done = e.step([NOOP])
    assert rew[0] == -726 / 1024 and done[0] == 0
    assert e.state[0, F["x"]] == 256 and e.state[0, F["path"]] == 0


def test_finish_pays_100_without_checkpoint_bonus_or_time_penalty():
    # the finish checkpoint at column 3: reached at tick 12 (centre column floor(808 / 256) = 3); frame-
    # skip 3 decisions pay 0, 0.25 (waypoint 1 at tick 6), 0, and 100 + 0.25 (waypoint 2 and the finish)
    m = flat_map()
    path = oracle.bfs_path(m, (1, 11), (3, 11))
    e = v2_env(m, path, ckpts=((3, 11),), fs=3)
    out = [e.step([RIGHT]) for _ in range(4)]
    assert [r[0] for r, _ in out] == [0.0, 0.25, 0.0, 100.25]
    assert [d[0] for _, d in out] == [0.0, 0.0, 0.0, 1.0]
    assert e.state[0, F["path"]] == 0 and e.state[0, F["x"]] == 256     # reset in place


def test_search_window_is_the_high_water_index_and_eight_after():
    # waypoint 0 at the spawn, waypoints 1..8 far above, waypoint 9 = (2, 11) next on the floor: walking
    # right it becomes the nearest (tick 6: 120 sub-units against 136 to waypoint 0) but lies one past
    # the window, so the high-water mark stays at 0 and no reward is paid; a window of 9 would pay 2.25
    path = [[1, 11]] + [[1, 1]] * 8 + [[2, 11]]
    e = v2_env(flat_map(), path)
    rews = [e.step([RIGHT])[0][0] for _ in range(12)]
    assert rews == [0.0] * 12 and e.state[0, F["path"]] == 0
    # with the high-water mark at 1, waypoint 0 leaves the window and waypoint 9 (282 sub-units away at
    # tick 1, against about 2600 for waypoints 1..8) is the nearest at once: 8 waypoints, 2.0
    e = v2_env(flat_map(), path)
    e.state[0, F["path"]] = 1
    rews = [e.step([RIGHT])[0][0] for _ in range(6)]
    assert rews == [8 * 0.25] + [0.0] * 5 and e.state[0, F["path"]] == 9


def test_version_one_is_unchanged_by_the_path_field():
    m = flat_map()
    e1 = oracle.OracleEnv(m[None], np.array([[[16, 11]]], np.int32), np.array([[256, 2880]], np.int32), 1,
                          frame_skip=1)
    e1.reset()
    r = e1.step([RIGHT])[0][0]
    assert r == (8 - 1) / 1024 and e1.state[0, F["path"]] == 0


def test_shortened_table_clamps_the_high_water_index():
    # Walking right along the floor path (1,11) .. (16,11) at single ticks: x = 424 + 48 (t - 6) from tick 6,
    # so after 30 ticks x = 1576 and the box centre x + 96 = 1672 has passed the midpoints 512, 768, 1024,
    # 1280 and 1536: the high-water index is 5 and the ticks paid 5 x 0.25. The table is then cut to its
    # first waypoint (the length a later rl_env_set_waypoints may give). The index past the new end is
    # clamped to the last waypoint, 0, whose centre is (384, 2944); the next tick (no input: vx 48 -> 40,
    # x = 1616) puts the centre at (1712, 2976): d = floor(sqrt(1328^2 + 32^2)) = 1328, past the grace zone
    # by 304, so the tick costs 304 >> 4 = 19 units and pays no progress.
    m = flat_map()
    path = oracle.bfs_path(m, (1, 11), (16, 11))
    e = v2_env(m, path)
    rews = [e.step([RIGHT])[0][0] for _ in range(30)]
    assert sum(rews) == 5 * 0.25 and e.state[0, F["x"]] == 1576 and e.state[0, F["path"]] == 5
    e.wp_lens[0] = 1
    rew, done = e.step([NOOP])
    assert e.state[0, F["x"]] == 1616 and e.state[0, F["y"]] == 2880
    assert rew[0] == -19 / 1024 and done[0] == 0
    assert e.state[0, F["path"]] == 0
    # lengthening the table again resumes the search at the clamped index: waypoints 0 .. 8 are in reach,
    # and after the next tick (vx 40 -> 32, x = 1648) the nearest to the centre (1744, 2976) is waypoint 5
    # (centre 1664): 5 waypoints of progress, 5 x 0.25
    e.wp_lens[0] = len(path)
    rew, _ = e.step([NOOP])
    assert e.state[0, F["x"]] == 1648 and rew[0] == 5 * 0.25 and e.state[0, F["path"]] == 5
