"""Pins of the oracle's grapple hook (hook mode) against hand-worked episodes.

The DDNet post ("What the agent sees and does") lists a hook button and a continuous aim (an angle and a
magnitude) among the actions, and the hook's state among the observed player state; it gives no hook
mechanics. The oracle's reading (its header and the hook step of its tick): the aim is the vector
(dx, dy) in sub-units (its polar form is the angle and magnitude); a new press with a non-zero aim fires
the tip from the box centre at HOOK_SPEED = 256 sub-units a tick along the aim (each component
truncated toward zero after dividing by floor(|aim|)); the tip attaches in the first tile it lands in that
blocks movement (solid, platform, or outside the map), and is lost after 10 ticks in flight; an attached
hook pulls the box centre toward the tip by 24 sub/tick^2 (same rounding), each velocity component then
bounded by 160; letting go retracts it; a held button does not fire again; frozen players cannot hook.
In hook mode frame dimension 9 is the hook's phase (0 idle, 1 flying, 2 attached).
Units: 1 tile = 256 sub-units.
"""
import numpy as np

import oracle
from resident_rl_rollout_amd import inputs

NOOP, HOOK = 0, 1
F = {name: i for i, name in enumerate(oracle.STATE_FIELDS)}
Y0 = 12 * 256 - 192          # standing on a floor whose top row is 12
CX, CY = 256 + 96, Y0 + 96   # box centre at the spawn (352, 2976)


def flat_map(h=16, w=64):
    m = np.zeros((h, w), np.uint8)
    m[12:, :] = 1
    return m


def make_env(m, spawn=(256, Y0), n=1, fs=1, hook_mode=1):
    e = oracle.OracleEnv(m[None], np.array([[[40, 11]]], np.int32), np.asarray(spawn, np.int32).reshape(1, 2),
                         n, frame_skip=fs, time_limit=2000, hook_mode=hook_mode)
    e.reset()
    return e


def aim(dx, dy, n=1):
    return np.full(n, inputs.pack_aim(dx, dy), np.int32)


def hook_state(e):
    s = e.state[0]
    return (int(s[F["hook_phase"]]), int(s[F["hook_x"]]), int(s[F["hook_y"]]), int(s[F["hook_vx"]]),
            int(s[F["hook_vy"]]), int(s[F["hook_flight"]]))


def test_aim_packing():
    a = inputs.pack_aim([0, -1, 300, -32768], [-100, 1, -400, 32767])
    assert a.dtype == np.int32
    dx = (a.astype(np.int64) & 0xFFFF).astype(np.uint16).view(np.int16)
    dy = ((a.astype(np.int64) >> 16) & 0xFFFF).astype(np.uint16).view(np.int16)
    assert dx.tolist() == [0, -1, 300, -32768] and dy.tolist() == [-100, 1, -400, 32767]


def test_straight_up_to_a_ceiling_then_pulled_against_it():
    m = flat_map()
    m[6, :] = 1                                   # a ceiling: row 6 spans y 1536 .. 1791
    e = make_env(m)
    a = aim(0, -100)
    # ticks 1-4: the tip climbs a tile a tick from the centre (2976 - 256 k, rows 10, 9, 8, 7) while the
    # player stands; tick 5: it lands at y 1696 in row 6 and attaches; the pull (-24) beats gravity (+12)
    for k in range(1, 5):
        e.step([HOOK], a)
        assert hook_state(e) == (1, CX, CY - 256 * k, 0, -256, k)
        assert e.state[0, F["y"]] == Y0 and e.state[0, F["vy"]] == 0
    e.step([HOOK], a)
    assert hook_state(e) == (2, CX, 1696, 0, -256, 5)
    assert e.state[0, F["vy"]] == -12 and e.state[0, F["y"]] == Y0 - 12 and e.state[0, F["grounded"]] == 0
    # tick 5 + j: vy = -12 (j + 1) and y = Y0 - 6 (j + 1)(j + 2), until y would pass 1792 (the ceiling's
    # underside) on tick 17 (j = 12): the box then snaps to 1792 and stays pinned there
    for j in range(1, 12):
        e.step([HOOK], a)
        assert e.state[0, F["vy"]] == -12 * (j + 1) and e.state[0, F["y"]] == Y0 - 6 * (j + 1) * (j + 2)
        assert hook_state(e)[0] == 2
    for _ in range(4):
        e.step([HOOK], a)
        assert e.state[0, F["y"]] == 7 * 256 and e.state[0, F["vy"]] == 0
    # letting go retracts the hook at once; the fall starts
    e.step([NOOP], a)
    assert hook_state(e)[0] == 0 and e.state[0, F["vy"]] == 12 and e.state[0, F["y"]] == 7 * 256 + 12


def test_a_miss_is_lost_after_ten_ticks_and_a_held_button_does_not_fire_again():
    e = make_env(flat_map())
    a = aim(0, -100)
    for k in range(1, 10):
        e.step([HOOK], a)
        assert hook_state(e)[0] == 1 and hook_state(e)[5] == k
    e.step([HOOK], a)                             # tick 10: row 1, still air: lost
    assert hook_state(e)[0] == 0 and hook_state(e)[2] == CY - 2560
    for _ in range(5):                            # still held: nothing fires
        e.step([HOOK], a)
        assert hook_state(e)[0] == 0
    assert e.state[0, F["hook_ticks"]] == 15
    e.step([NOOP], a)                             # release, then press: a new shot from the centre
    e.step([HOOK], a)
    assert hook_state(e) == (1, CX, CY - 256, 0, -256, 1)


def test_zero_aim_never_fires():
    e = make_env(flat_map())
    for _ in range(6):
        e.step([HOOK], aim(0, 0))
        assert hook_state(e) == (0, 0, 0, 0, 0, 0)
    assert e.state[0, F["hook_ticks"]] == 6 and e.state[0, F["hook_held"]] == 1


def test_diagonal_aim_truncates_toward_zero():
    # |(300, -400)| = 500: velocity (300 * 256 / 500, -400 * 256 / 500) = (153.6, -204.8) -> (153, -204)
    e = make_env(flat_map())
    a = aim(300, -400)
    for k in range(1, 4):
        e.step([HOOK], a)
        assert hook_state(e) == (1, CX + 153 * k, CY - 204 * k, 153, -204, k)
    # a length that is not a whole number: |(1, 2)| = 2.236..., floor 2: (128, 256)
    e2 = make_env(flat_map())
    e2.step([HOOK], aim(1, 2))
    assert hook_state(e2)[3:5] == (128, 256)


def test_outside_the_map_holds_and_pulls_the_player_to_the_edge():
    e = make_env(flat_map())
    a = aim(-100, 0)
    e.step([HOOK], a)                             # tip x 96: column 0, air
    assert hook_state(e) == (1, CX - 256, CY, -256, 0, 1)
    e.step([HOOK], a)                             # tip x -160: column -1, outside the map: attached
    assert hook_state(e)[:3] == (2, CX - 512, CY)
    # the pull of tick 2 takes vx from 0 to -24 (x 232). Each later tick the ground friction first moves
    # vx toward 0 by 8, then the pull (the tip level with the centre, so exactly -24) takes it back:
    # -16 a tick net, bounded by -160, until the box meets column -1
    assert e.state[0, F["vx"]] == -24 and e.state[0, F["x"]] == 256 - 24
    vx, x = -24, 256 - 24
    while True:
        e.step([HOOK], a)
        vx = max(vx + 8 - 24, -160)
        nx = x + vx
        if nx < 0:                                # column -1 blocks: the box stops at x = 0
            assert e.state[0, F["x"]] == 0 and e.state[0, F["vx"]] == 0
            break
        x = nx
        assert e.state[0, F["x"]] == x and e.state[0, F["vx"]] == vx
    assert e.state[0, F["wall_left"]] == 1 and hook_state(e)[0] == 2


def test_platforms_hold_the_hook_and_freeze_tiles_do_not():
    for tile, phase_at_5 in ((2, 2), (3, 1)):
        m = flat_map()
        m[6, :] = tile
        e = make_env(m)
        for _ in range(5):
            e.step([HOOK], aim(0, -100))
        assert hook_state(e)[0] == phase_at_5, tile


def test_frozen_players_cannot_hook():
    m = flat_map()
    m[11, 1] = 3                                  # a freeze tile where the player stands
    e = make_env(m)
    e.step([NOOP], aim(0, -100))                  # the first tick arms the counter
    for _ in range(5):
        e.step([HOOK], aim(0, -100))
        assert hook_state(e)[0] == 0 and e.state[0, F["hook_held"]] == 0


def test_frame_skip_keeps_the_aim_for_the_decision():
    # FS = 3 equals three FS = 1 decisions with the same action and aim
    m = flat_map()
    m[6, :] = 1
    a3, a1 = make_env(m, fs=3), make_env(m, fs=1)
    rng = np.random.default_rng(5)
    for _ in range(40):
        act = [int(rng.integers(0, 12))]
        am = aim(int(rng.integers(-300, 301)), int(rng.integers(-300, 301)))
        r3, _ = a3.step(act, am)
        r1 = sum(a1.step(act, am)[0][0] for _ in range(3))
        assert r3[0] == np.float32(r1)
        np.testing.assert_array_equal(a3.state[:, :F["last_action"]], a1.state[:, :F["last_action"]])
        np.testing.assert_array_equal(a3.state[:, F["hook_phase"]:], a1.state[:, F["hook_phase"]:])


def test_observed_phase_and_hook_mode_off():
    m = flat_map()
    m[6, :] = 1
    e = make_env(m)
    for _ in range(5):
        e.step([HOOK], aim(0, -100))
    obs = e.obs_tiles()[0]
    frames = obs[31 * 43:31 * 43 + 60].reshape(4, 15)
    assert frames[:, 9].tolist() == [2, 1, 1, 1]       # newest first: attached, then flying
    # hook mode off: the aim is ignored, the hook fields stay zero and dim 9 is the held-tick count
    rng = np.random.default_rng(9)
    ms = inputs.make_mapset([3], 32, 128)
    off = oracle.OracleEnv(ms.maps, ms.ckpts, ms.spawns, 50)
    off2 = oracle.OracleEnv(ms.maps, ms.ckpts, ms.spawns, 50)
    off.reset()
    off2.reset()
    aims = inputs.make_aims(3, 30, 50)
    for t in range(30):
        acts = rng.integers(0, 12, 50).astype(np.int32)
        assert [x.tolist() for x in off.step(acts, aims[t])] == [x.tolist() for x in off2.step(acts)]
    np.testing.assert_array_equal(off.state, off2.state)
    assert (off.state[:, F["hook_phase"]:] == 0).all()
    assert (off.obs_tiles()[:, 31 * 43 + 9] == off.state[:, F["hook_ticks"]]).all()
