"""Pins of the oracle's platformer against hand-worked episodes and invariants.

No page gives the environment's outputs, so the physics constants and the tick order are readings (see
the oracle's header). These tests fix the oracle to that reading with values worked out by hand on
hand-drawn maps: a flat walk (velocity ramp 8, 16, ..., 48), a jump (apex 540 sub-units after 9 ticks,
period 19 while held), a wall stop (snap to col*256 - 192), freeze lock-out (exactly 30 ticks after
leaving the tile), checkpoints in order (+10) and the finish (+100, done, reset), the time limit, the
frame-skip sum ("boesch.dev DDNet RL post", How it works each tick: frame-skip 3 with rewards summed
between decisions), the observation layout ("What the agent sees and does") and pixels.
Units: 1 tile = 256 sub-units; rewards are integer units times 2^-10.
"""
import itertools
import math

import numpy as np
import pytest

import oracle
from resident_rl_rollout_amd import inputs

NOOP, LEFT, RIGHT, JUMP, HOOK = 0, 4, 8, 2, 1
F = {name: i for i, name in enumerate(oracle.STATE_FIELDS)}


def flat_map(h=16, w=64, floor_h=4):
    m = np.zeros((h, w), np.uint8)
    m[h - floor_h:, :] = 1
    return m


def make_env(m, ckpts=((16, 11),), spawn=None, n=1, fs=3, tl=2000, sprites=None):
    h, w = m.shape
    if spawn is None:
        spawn = (256, 12 * 256 - 192)      # standing on a floor whose top row is 12
    e = oracle.OracleEnv(m[None], np.asarray(ckpts, np.int32).reshape(1, -1, 2),
                         np.asarray(spawn, np.int32).reshape(1, 2), n, frame_skip=fs, time_limit=tl,
                         sprites=sprites)
    e.reset()
    return e


def ramp(k):
    """Distance walked on flat ground after k ticks from rest: sum_{i<=k} min(8i, 48)."""
    return sum(min(8 * i, 48) for i in range(1, k + 1))


def test_flat_walk_velocity_ramp_and_progress_reward():
    e = make_env(flat_map(), fs=1)
    x0 = 256
    for k in range(1, 15):
        rew, done = e.step([RIGHT])
        s = e.state[0]
        assert s[F["vx"]] == min(8 * k, 48)
        assert s[F["x"]] == x0 + ramp(k)
        assert s[F["y"]] == 12 * 256 - 192 and s[F["vy"]] == 0
        assert s[F["grounded"]] == 1 and s[F["facing"]] == 1
        # progress: one unit per sub-unit past the high-water mark, minus one unit per tick
        assert rew[0] == (min(8 * k, 48) - 1) / 1024 and done[0] == 0
    # pushing left first brakes by 8 per tick (still paying for the ground gained), then walks back
    # left, which pays nothing for progress, only the time cost; facing follows the push at once
    for j in range(1, 21):
        rew, _ = e.step([LEFT])
        assert e.state[0, F["vx"]] == max(48 - 8 * j, -48)
        assert rew[0] == (max(48 - 8 * j, 0) - 1) / 1024
        assert e.state[0, F["facing"]] == -1
    assert e.state[0, F["best_x"]] == x0 + ramp(14) + 40 + 32 + 24 + 16 + 8


def test_ceiling_bump_snaps_below_the_tile():
    # A solid row 10 right above the standing box (rows 11 .. 11.99, y = 2880). The jump's first tick gives
    # vy = -120 + 12 = -108 and ny = 2772, whose top row 10 is solid: the box snaps to the ceiling's
    # underside, y = 11 * 256 = 2816, and vy = 0. It then falls under gravity, vy = 12, 24, 36:
    # y = 2828, 2852, and 2888 would reach row 12, so the box lands at 2880 with vy = 0 on the fourth tick.
    m = flat_map()
    m[10, :] = 1
    e = make_env(m, fs=1)
    ys, vys = [], []
    for a in [JUMP, NOOP, NOOP, NOOP, NOOP]:
        e.step([a])
        ys.append(int(e.state[0, F["y"]]))
        vys.append(int(e.state[0, F["vy"]]))
    assert ys == [2816, 2828, 2852, 2880, 2880]
    assert vys == [0, 12, 24, 0, 0]
    assert e.state[0, F["grounded"]] == 1


def test_jump_apex_and_period():
    e = make_env(flat_map(), fs=1)
    y0 = 12 * 256 - 192
    ys = []
    for _ in range(38):
        e.step([JUMP])
        ys.append(e.state[0, F["y"]])
    # vy after gravity on tick k of a jump is -120 + 12k, so y_k = y0 - 120k + 6k(k+1) for k = 1..19,
    # the landing tick 19 ends exactly on the floor and the held jump starts the next one.
    expect = [y0 - 120 * k + 6 * k * (k + 1) for k in range(1, 20)] * 2
    assert ys == expect
    assert min(ys) == y0 - 540 and ys[8] == ys[9] == y0 - 540


def test_wall_stop_snaps_to_tile_edge():
    m = flat_map()
    m[:, 5] = 1                          # a wall filling column 5
    e = make_env(m, fs=1)
    for k in range(1, 25):
        e.step([RIGHT])
        s = e.state[0]
        if 256 + ramp(k) + 191 < 5 * 256 and k < 20:
            assert s[F["x"]] == 256 + ramp(k) and s[F["wall_right"]] == 0
        else:
            assert k >= 20                # 256 + ramp(20) + 191 = 1287 reaches column 5
            assert s[F["x"]] == 5 * 256 - 192 and s[F["vx"]] == 0 and s[F["wall_right"]] == 1


def test_freeze_tile_in_spawn_cell_locks_input():
    m = flat_map()
    m[11, 1] = 3                          # freeze tile where the player stands
    e = make_env(m, fs=3)
    # the counter is armed at the end of the first tick, so that tick's input would still act: start
    # with a no-op, after which every input is ignored while the player keeps touching the tile
    for d in range(10):
        rew, done = e.step([NOOP if d == 0 else RIGHT + JUMP])
        s = e.state[0]
        assert s[F["x"]] == 256 and s[F["y"]] == 12 * 256 - 192
        assert s[F["freeze_ticks"]] == 30 and rew[0] == -3 / 1024 and done[0] == 0
        assert s[F["jump_held"]] == 0 and s[F["hook_ticks"]] == 0


def test_freeze_lasts_exactly_30_ticks_after_leaving():
    m = flat_map()
    m[6, 1] = 3                           # a freeze tile the falling player passes through
    e = make_env(m, spawn=(256, 2 * 256), fs=1)
    # fall from y = 512: y_k = 512 + sum min(12i, 160), until the floor stops it at 12*256 - 192
    ys, y, k = [], 512, 0
    while True:
        k += 1
        y = min(y + min(12 * k, 160), 12 * 256 - 192)
        ys.append(y)
        if y == 12 * 256 - 192:
            break
    landing = len(ys)
    touching = [i + 1 for i, yy in enumerate(ys) if 6 * 256 - 191 <= yy <= 6 * 256 + 255]
    tau = touching[-1]                    # the last tick whose box overlaps the freeze row
    assert tau < landing < tau + 31
    for t in range(1, tau + 40):
        e.step([NOOP if t <= landing else RIGHT])
        s = e.state[0]
        if t <= landing:
            assert s[F["y"]] == ys[t - 1]
        if t <= tau:
            assert s[F["freeze_ticks"]] == (30 if t in touching else 0)
        elif t <= tau + 30:
            assert s[F["freeze_ticks"]] == 30 - (t - tau) and s[F["x"]] == 256
        elif t == tau + 31:
            assert s[F["x"]] == 264 and s[F["vx"]] == 8


def test_checkpoints_in_order_and_finish_resets():
    e = make_env(flat_map(), ckpts=((16, 11), (32, 11)), fs=3)
    # x_k = 256 + ramp(k) reaches ckpt column 16 (x + 96 >= 4096) at tick 81 = decision 27, tick 3,
    # and column 32 (x + 96 >= 8192) at tick 166 = decision 56, tick 1 of 3.
    assert 256 + ramp(80) + 96 < 4096 <= 256 + ramp(81) + 96
    assert 256 + ramp(165) + 96 < 8192 <= 256 + ramp(166) + 96
    total = 0
    for d in range(1, 57):
        rew, done = e.step([RIGHT])
        units = rew[0] * 1024
        assert units == int(units)
        total += int(units)
        k0, k1 = 3 * (d - 1), min(3 * d, 166)
        progress = ramp(k1) - ramp(k0)
        if d == 27:
            assert units == progress + 10240 - 3 and e.state[0, F["next_ckpt"]] == 1
        elif d == 56:
            assert units == progress + 10240 + 102400 - 1 and done[0] == 1
        else:
            assert units == progress - 3 and done[0] == 0
    assert total == ramp(166) + 2 * 10240 + 102400 - 166
    s = e.state[0]
    assert (s[F["x"]], s[F["y"]], s[F["tick"]], s[F["next_ckpt"]], s[F["best_x"]]) == (256, 2880, 0, 0, 256)
    assert s[F["last_action"]] == 0 and s[F["grounded"]] == 1
    obs = e.obs_tiles()
    fresh = make_env(flat_map(), ckpts=((16, 11), (32, 11)), fs=3).obs_tiles()
    np.testing.assert_array_equal(obs, fresh)


def test_time_limit_truncates_on_tick_2000():
    e = make_env(flat_map(), fs=3, tl=2000)
    for d in range(1, 667):
        rew, done = e.step([NOOP])
        assert rew[0] == -3 / 1024 and done[0] == 0
    rew, done = e.step([NOOP])            # decision 667: ticks 1999 and 2000
    assert rew[0] == -2 / 1024 and done[0] == 1
    assert e.state[0, F["tick"]] == 0


def test_time_limit_one_ends_every_decision():
    # a 1-tick limit: every decision runs one tick, is truncated and resets at the spawn; standing still
    # earns only the time penalty, a rightward tick 8 sub-units of progress less it
    e = make_env(flat_map(), fs=3, tl=1)
    for a, units in ((NOOP, -1), (RIGHT, 8 - 1), (RIGHT, 8 - 1), (LEFT, -1)):
        rew, done = e.step([a])
        assert rew[0] == units / 1024 and done[0] == 1
        assert e.state[0, F["tick"]] == 0 and e.state[0, F["x"]] == 256 and e.state[0, F["vx"]] == 0


def test_out_of_range_actions_are_noops():
    m = inputs.make_map(5, 32, 64)[0]
    e1 = make_env(m, n=4, fs=3, spawn=(256, (32 - 8) * 256 - 192))
    e2 = make_env(m, n=4, fs=3, spawn=(256, (32 - 8) * 256 - 192))
    for _ in range(5):
        r1, d1 = e1.step([-1, 12, 99, -2 ** 31])
        r2, d2 = e2.step([0, 0, 0, 0])
        np.testing.assert_array_equal(r1, r2)
    np.testing.assert_array_equal(e1.state, e2.state)


def test_frame_skip_is_the_sum_of_single_ticks():
    ms = inputs.make_mapset([11], 32, 128)
    acts = inputs.make_actions(12, 40, 256)
    e3 = oracle.OracleEnv(ms.maps, ms.ckpts, ms.spawns, 256, frame_skip=3)
    e1 = oracle.OracleEnv(ms.maps, ms.ckpts, ms.spawns, 256, frame_skip=1)
    e3.reset()
    e1.reset()
    alive = np.ones(256, bool)
    for a in acts:
        r3, d3 = e3.step(a)
        r1 = np.zeros(256)
        d1 = np.zeros(256)
        for _ in range(3):
            r, d = e1.step(a)
            r1 += r
            d1 += d
        alive &= (d3 == 0) & (d1 == 0)
        for f in range(oracle.NF):
            if oracle.STATE_FIELDS[f] == "tick":
                continue
            np.testing.assert_array_equal(e3.state[alive, f], e1.state[alive, f])
        np.testing.assert_array_equal(r3[alive], r1[alive].astype(np.float32))
    assert alive.sum() > 200


def test_tile_window_stack_and_checkpoint_dims_at_spawn():
    m = flat_map()
    m[5, 10] = 2                         # a platform marker
    e = make_env(m)
    o = e.obs_tiles()[0]
    win = o[:1333].reshape(31, 43)
    # the player's tile is (row 11, col 1): window (r, c) shows map (r - 4, c - 20); outside is SOLID
    for r in range(31):
        for c in range(43):
            mr, mc = r - 4, c - 20
            inside = 0 <= mr < 16 and 0 <= mc < 64
            assert win[r, c] == (m[mr, mc] if inside else 1)
    assert win[9, 30] == 2 and win[0, 0] == 1 and win[15, 21] == 0 and win[16, 21] == 1
    spawn_frame = [1.0, 11.25, 0, 0, 1, 1, 0, 0, 0, 0, 0, 0, 0, 0, 0]
    np.testing.assert_array_equal(o[1333:1393].reshape(4, 15), [spawn_frame] * 4)
    # dx = ((16 + 1/2) * 256 - (256 + 96)) / 256, dy = ((11 + 1/2) * 256 - (2880 + 96)) / 256
    np.testing.assert_array_equal(o[1393:], [15.125, -0.125, 0.0, 1.0])


def test_stack_is_newest_first():
    e = make_env(flat_map(), fs=3)
    e.step([RIGHT])
    e.step([RIGHT + HOOK])
    st = e.obs_tiles()[0, 1333:1393].reshape(4, 15)
    np.testing.assert_array_equal(st[:, 0], np.float32([424, 304, 256, 256]) / 256)
    np.testing.assert_array_equal(st[:, 13], np.float32([6, 3, 0, 0]) / 2048)
    np.testing.assert_array_equal(st[:, 14], [9, 8, 0, 0])
    np.testing.assert_array_equal(st[:, 8], [1, 0, 0, 0])      # hook held
    np.testing.assert_array_equal(st[:, 9], [3, 0, 0, 0])      # hook ticks
    np.testing.assert_array_equal(st[:, 2], np.float32([48, 24, 0, 0]) / 256)


def test_pixels_on_a_hand_map():
    m = flat_map()
    m[10, 3] = 2
    sprites = np.zeros((16, 8, 8), np.uint8)
    for k in range(16):
        sprites[k] = 10 * k + 5
    sprites[1] = 100 + np.arange(64, dtype=np.uint8).reshape(8, 8)   # a patterned SOLID sprite
    e = make_env(m, sprites=sprites)
    px = e.obs_pixels()[0]
    assert (px[0] == px[1]).all() and (px[0] == px[3]).all()     # reset: 4 copies of the spawn frame
    f = px[0].astype(int)
    # camera top-left: ((256 + 96) // 32 - 42, (2880 + 96) // 32 - 42) = (-31, 51)
    for py in range(84):
        for qx in range(84):
            wx, wy = qx - 31, py + 51
            if 39 <= qx <= 44 and 39 <= py <= 44:        # the player box, pixels [8, 13] x [90, 95]
                expect = 255
            elif wx < 0 or wy >= 96:                     # left of the map, or the floor: SOLID
                expect = 100 + (wy % 8) * 8 + (wx % 8)
            elif 80 <= wy <= 87 and 24 <= wx <= 31:      # the platform at (row 10, col 3)
                expect = 25
            else:
                expect = 5
            assert f[py, qx] == expect, (py, qx)
    assert f[0, 0] == 100 + 3 * 8 + 1
    e.step([RIGHT])                       # x = 304: camera x = (304 + 96) // 32 - 42 = -30
    px2 = e.obs_pixels()[0]
    # box pixels [304 // 32, 495 // 32] = [9, 15], at camera columns 9 + 30 .. 15 + 30
    assert (px2[0, 39:45, 39:46] == 255).all() and px2[0, 39, 38] != 255 and px2[0, 39, 46] != 255
    np.testing.assert_array_equal(px2[1], px[0])


def test_exhaustive_four_decisions_keep_invariants():
    # All 12^4 action sequences from one spawn on a small generated map. No page gives these outputs:
    # this checks invariants of the reading (parity unpinned beyond them).
    ms = inputs.make_mapset([21], 32, 128)
    seqs = np.array(list(itertools.product(range(12), repeat=4)), np.int32)
    n = len(seqs)
    e = oracle.OracleEnv(ms.maps, ms.ckpts, ms.spawns, n, frame_skip=3)
    e.reset()
    tiles = ms.maps[0]

    def solid(r, c):
        return True if (r < 0 or r >= 32 or c < 0 or c >= 128) else tiles[r, c] in (1, 2)

    prev = e.state.copy()
    for d in range(4):
        rew, done = e.step(seqs[:, d])
        s = e.state
        assert (done == 0).all()
        assert (np.abs(s[:, F["vx"]]) <= 48).all()
        assert ((s[:, F["vy"]] >= -120) & (s[:, F["vy"]] <= 160)).all()
        assert (s[:, F["best_x"]] >= prev[:, F["best_x"]]).all() and (s[:, F["best_x"]] >= s[:, F["x"]]).all()
        assert (s[:, F["tick"]] == 3 * (d + 1)).all()
        units = (rew * 1024).astype(np.int64)
        np.testing.assert_array_equal(
            units, (s[:, F["best_x"]] - prev[:, F["best_x"]]) + 10240 * (s[:, F["next_ckpt"]] - prev[:, F["next_ckpt"]]) - 3)
        for i in range(0, n, 97):
            x, y = s[i, F["x"]], s[i, F["y"]]
            for r in range(y // 256, (y + 191) // 256 + 1):
                for c in range(x // 256, (x + 191) // 256 + 1):
                    assert not solid(r, c)
            under = any(solid((y + 192) // 256, c) for c in range(x // 256, (x + 191) // 256 + 1))
            assert s[i, F["grounded"]] == int(under)
        prev = s.copy()
    assert len({tuple(r) for r in e.state[:, :4]}) > 100


def test_two_runs_are_identical_and_reset_mask_is_selective():
    ms = inputs.make_mapset([31, 32], 32, 128)
    acts = inputs.make_actions(33, 30, 64)
    runs = []
    for _ in range(2):
        e = oracle.OracleEnv(ms.maps, ms.ckpts, ms.spawns, 64)
        e.reset()
        for a in acts:
            e.step(a)
        runs.append((e.state.copy(), e.obs_tiles()))
    np.testing.assert_array_equal(runs[0][0], runs[1][0])
    np.testing.assert_array_equal(runs[0][1], runs[1][1])
    before = e.state.copy()
    mask = np.zeros(64, np.uint8)
    mask[::3] = 1
    e.reset(mask)
    np.testing.assert_array_equal(e.state[mask == 0], before[mask == 0])
    assert (e.state[mask == 1, F["tick"]] == 0).all()
    # env n plays map n mod 2: odd envs spawn on map 1
    np.testing.assert_array_equal(e.state[mask == 1, F["y"]], ms.spawns[np.arange(64)[mask == 1] % 2, 1])
