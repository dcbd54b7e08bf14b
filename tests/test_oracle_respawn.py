"""Pins of the oracle's adaptive checkpoint respawn ("boesch.dev DDNet RL post", Checkpoint Respawning: a
rolling buffer of episode outcomes, spawns sampled from the top-performing episodes, 20% of resets from
the beginning, spawns capped at the frontier proven reachable from the start).

Readings (the oracle's header lists them): 64 outcomes per map; the top quarter of the buffer, taken
uniformly; resets sample the buffer as it stood at the start of the step, and the step's ended episodes
enter it afterwards in env order. The draws are SplitMix64 outputs (Steele, Lea and Flood 2014), pinned
here by the generator's published first outputs from seed 0; the choices below are applied by hand to
hand-built buffers.
"""
import numpy as np
import pytest

import oracle

F = {name: i for i, name in enumerate(oracle.STATE_FIELDS)}
M64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15


def splitmix_output(state):
    """SplitMix64's output function, from its publication."""
    z = state & M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def draw(seed, counter, n, i):
    return splitmix_output(seed + 2 * GOLDEN * (counter * (1 << 24) + n) + i * GOLDEN)


def flat_env(n, k_ckpts=12, tl=1, seed=7, fs=1):
    """n envs on one flat map (floor top at row 12) with k_ckpts checkpoints every 16 columns."""
    w = 16 * (k_ckpts + 1)
    m = np.zeros((16, w), np.uint8)
    m[12:, :] = 1
    cols = 16 * (np.arange(k_ckpts) + 1)
    ckpts = np.stack([cols, np.full(k_ckpts, 11)], axis=1).astype(np.int32)[None]
    stands = np.stack([cols * 256 + 32, np.full(k_ckpts, 12 * 256 - 192)], axis=1).astype(np.int32)[None]
    e = oracle.OracleEnv(m[None], ckpts, np.array([[256, 12 * 256 - 192]], np.int32), n, frame_skip=fs,
                         time_limit=tl, respawn_mode=1, ckpt_spawns=stands, respawn_seed=seed)
    e.reset()
    return e, stands[0]


def test_generator_published_outputs():
    # SplitMix64 seeded with 0: its first three outputs
    assert [splitmix_output(i * GOLDEN) for i in (1, 2, 3)] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4,
                                                               0x06C45D188009454F]
    assert oracle.respawn_draw(0, 0, 0, 1) == 0xE220A8397B1DCDAF
    assert oracle.respawn_draw(0, 0, 0, 2) == 0x6E789E6AA1B965F4
    for seed, counter, n, i in ((7, 3, 5, 1), (2 ** 63 + 11, 1000, 65535, 2), (1, 0, 16_777_215, 1)):
        assert oracle.respawn_draw(seed, counter, n, i) == draw(seed, counter, n, i)


def test_empty_buffer_starts_at_the_spawn_and_records_the_outcome():
    e, _ = flat_env(3)
    rew, done = e.step([8, 8, 8])                     # one tick each, then the time limit
    assert (done == 1).all()
    assert (e.state[:, F["x"]] == 256).all() and (e.state[:, F["from_start"]] == 1).all()
    assert e.fill[0] == 3 and e.head[0] == 3 and (e.ring[0, :3] == 0).all() and e.frontier[0] == 0


def test_top_quarter_choice_frontier_and_append_order():
    n, seed = 64, 7
    e, stands = flat_env(n, seed=seed)
    e.ring[0, :16] = [9, 9, 8, 8, 8, 1, 1, 2, 2, 3, 0, 0, 0, 4, 4, 5]
    e.fill[0], e.head[0], e.frontier[0] = 16, 16, 10
    # by hand: q = 16 / 4 = 4; from the top, 9 is reached by 2 entries, 8 by 5 >= 4: the candidates are
    # the two 9s then the three 8s; pick = (u2 >> 32) % 5 takes 9 for picks 0, 1 and 8 for 2, 3, 4; the
    # frontier (10) and K - 1 (11) do not bind; 20% of draws (u1 >> 32 < 858993459) start at the spawn
    expect = []
    for i in range(n):
        if (draw(seed, 0, i, 1) >> 32) < 858993459:
            expect.append(0)
        else:
            expect.append(9 if (draw(seed, 0, i, 2) >> 32) % 5 < 2 else 8)
    expect = np.array(expect)
    assert set(expect.tolist()) == {0, 8, 9}
    e.step(np.full(n, 8, np.int32))
    s = e.state
    np.testing.assert_array_equal(s[:, F["next_ckpt"]], expect)
    np.testing.assert_array_equal(s[:, F["from_start"]], (expect == 0).astype(np.int32))
    want_x = np.where(expect == 0, 256, stands[np.maximum(expect - 1, 0), 0])
    np.testing.assert_array_equal(s[:, F["x"]], want_x)
    np.testing.assert_array_equal(s[:, F["best_x"]], want_x)
    # the step's 64 outcomes (all 0: the reset episodes passed nothing) filled the ring
    assert e.fill[0] == 64 and e.head[0] == (16 + 64) % 64 and (e.ring[0] == 0).all()
    # next step: every episode ends again with outcome = its start checkpoint, appended in env order;
    # only episodes that began at the spawn may raise the frontier (theirs are 0)
    e.step(np.full(n, 8, np.int32))
    np.testing.assert_array_equal(np.roll(e.ring[0], -e.head[0]), expect)
    assert e.frontier[0] == 10


@pytest.mark.parametrize("frontier,want", [(3, 3), (20, 11), (0, 0)])
def test_caps_at_the_frontier_and_before_the_finish(frontier, want):
    e, _ = flat_env(200)
    e.ring[0, :] = 12                                  # every buffered episode finished (K = 12)
    e.fill[0], e.frontier[0] = 64, frontier
    e.step(np.full(200, 8, np.int32))
    nxt = e.state[:, F["next_ckpt"]]
    assert set(np.unique(nxt).tolist()) <= {0, want}
    assert (nxt == want).sum() > 100                   # about 80% of resets respawn


def test_frontier_rises_only_from_episodes_that_began_at_the_spawn():
    e, _ = flat_env(2, tl=10)
    # env 0 began at the spawn and has passed 4 checkpoints; env 1 respawned at 7 and has passed 9;
    # both end at this tick (tick 9 of a 10-tick limit)
    for i, (nxt, fs_) in enumerate(((4, 1), (9, 0))):
        e.state[i, F["next_ckpt"]], e.state[i, F["from_start"]], e.state[i, F["tick"]] = nxt, fs_, 9
    e.step([0, 0])
    assert e.ring[0, :2].tolist() == [4, 9] and e.frontier[0] == 4


def test_twenty_percent_start_at_the_spawn():
    n = 4000
    e, _ = flat_env(n, seed=123)
    e.ring[0, :] = 5
    e.fill[0], e.frontier[0] = 64, 5
    e.step(np.full(n, 8, np.int32))
    frac = float((e.state[:, F["next_ckpt"]] == 0).mean())
    assert abs(frac - 0.2) < 4 * np.sqrt(0.16 / n)


def test_invariants_over_a_long_run():
    from resident_rl_rollout_amd import inputs
    ms = inputs.make_mapset([7, 8, 9], 32, 120)
    n = 300
    e = oracle.OracleEnv(ms.maps, ms.ckpts, ms.spawns, n, time_limit=240, respawn_mode=1,
                         ckpt_spawns=ms.ckpt_spawns, respawn_seed=99)
    e.reset()
    rng = np.random.default_rng(1)
    k = ms.ckpts.shape[1]
    prev_front = e.frontier.copy()
    respawned = 0
    for t in range(400):
        front_before = e.frontier.copy()
        acts = np.where(rng.random(n) < 0.8, 8 + rng.integers(0, 4, n), rng.integers(0, 12, n)).astype(np.int32)
        _, done = e.step(acts)
        s = e.state
        maps_ = np.arange(n) % 3
        started = s[done == 1]
        ks = started[:, F["next_ckpt"]]
        assert (ks <= np.minimum(front_before[maps_[done == 1]], k - 1)).all()
        assert ((ks == 0) == (started[:, F["from_start"]] == 1)).all()
        respawned += int((ks > 0).sum())
        assert (e.frontier >= prev_front).all()
        prev_front = e.frontier.copy()
        assert ((e.ring >= 0) & (e.ring <= k)).all()
    assert respawned > 0 and e.frontier.max() > 0
