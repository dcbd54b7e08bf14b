"""GPU parity of the grapple hook (hook mode, rl_env_step_aim) against the oracle: bit-exact state (the
hook's phase, tip, flight velocity and ticks flown included), observations, rewards and dones, with the
same seeded maps, actions and aims on both sides."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from resident_rl_rollout_amd import binding, inputs
from tests.gpu_helpers import PairedEnvs, waypoint_table

pytestmark = pytest.mark.gpu
F = {name: i for i, name in enumerate(oracle.STATE_FIELDS)}


def hook_inputs(seed, steps, n, p_hook=0.7):
    """Actions with the hook bit set with probability p_hook (so presses, holds and releases all occur)
    and aims mostly upward (70% in the upper half-plane), magnitudes 64 .. 4096, 5% zero."""
    rng = np.random.default_rng(seed)
    acts = (4 * rng.integers(0, 3, (steps, n)) + 2 * rng.integers(0, 2, (steps, n))
            + (rng.random((steps, n)) < p_hook)).astype(np.int32)
    aims = inputs.make_aims(seed + 1, steps, n)
    up = rng.random((steps, n)) < 0.7
    dy = (aims.astype(np.int64) >> 16)
    dx = ((aims.astype(np.int64) & 0xFFFF) ^ 0x8000) - 0x8000
    dy = np.where(up, -np.abs(dy), dy)
    return acts, inputs.pack_aim(dx, dy)


def run(pe, acts, aims, what, obs_every=1, obs_envs=None):
    """Steps both sides, checking everything; returns the phase counts, the largest speed, and how far past
    the 8x8 collision neighbourhood (3 rows up, 2 columns left of the starting box) a decision probed."""
    pe.check_obs(f"{what} reset")
    phases = np.zeros(3, np.int64)
    vmax = 0
    beyond = 0
    for s in range(len(acts)):
        x0, y0 = pe.ora.state[:, F["x"]].copy(), pe.ora.state[:, F["y"]].copy()
        r, d = pe.step(acts[s], None if aims is None else aims[s])
        x1, y1 = pe.ora.state[:, F["x"]], pe.ora.state[:, F["y"]]
        live = d == 0
        left = (x0 >> 8) - ((x1 - 1) >> 8) - 2          # wall probe columns past c0 - 2
        up = (y0 >> 8) - (y1 >> 8) - 3                  # ceiling probe rows past r0 - 3
        if live.any():
            beyond = max(beyond, int(np.maximum(left, up)[live].max()))
        pe.check_step(r, d, f"{what} step {s}")
        pe.check_state(f"{what} step {s}")
        if obs_every and (s % obs_every == 0 or s == len(acts) - 1):
            pe.check_obs(f"{what} step {s}", obs_envs)
        phases += np.bincount(pe.ora.state[:, F["hook_phase"]], minlength=3)
        vmax = max(vmax, int(np.abs(pe.ora.state[:, [F["vx"], F["vy"]]]).max()))
    return phases, vmax, beyond


def test_tiny_workload_with_the_hook(gpu_lib):
    ms = inputs.make_mapset([1], 32, 128)
    pe = PairedEnvs(ms, 64, hook_mode=binding.HOOK_GRAPPLE)
    acts, aims = hook_inputs(2, 128, 64)
    phases, _, _ = run(pe, acts, aims, "tiny hook")
    assert phases[1] > 0 and phases[2] > 0        # tips flew and held


@pytest.mark.parametrize("fs", [1, 3, 4, 5])
def test_hook_frame_skip_and_fast_swings(fs, gpu_lib):
    # up to 3 ticks at hook speeds (at most 160 a tick) keep every collision probe inside the 8x8
    # neighbourhood, which those launches rely on; frame-skip 4 and 5 take probes past it (read from the
    # map instead)
    ms = inputs.make_mapset([4, 5, 6], 48, 96)
    pe = PairedEnvs(ms, 300, frame_skip=fs, time_limit=400, hook_mode=binding.HOOK_GRAPPLE)
    acts, aims = hook_inputs(10 + fs, 120, 300, p_hook=0.85)
    phases, vmax, beyond = run(pe, acts, aims, f"hook fs={fs}", obs_every=9)
    assert phases[2] > 0 and vmax > 100
    if fs <= 3:
        assert beyond <= 0
    if fs == 5:
        assert beyond > 0


def test_hook_workload_full_size(gpu_lib):
    ms = inputs.make_mapset(range(100, 164), 256, 1024)
    pe = PairedEnvs(ms, 65536, hook_mode=binding.HOOK_GRAPPLE)
    acts, aims = hook_inputs(3, 12, 65536)
    rng = np.random.default_rng(0)
    envs = np.concatenate([np.arange(64), rng.choice(65536, 448, replace=False), np.arange(65536 - 64, 65536)])
    pe.check_obs("hook full reset", envs)
    for s in range(len(acts)):
        r, d = pe.step(acts[s], aims[s])
        pe.check_step(r, d, f"hook full step {s}")
        if s in (0, 5, len(acts) - 1):
            pe.check_state(f"hook full step {s}")
            pe.check_obs(f"hook full step {s}", envs)
    assert (pe.ora.state[:, F["hook_phase"]] == 2).sum() > 1000


def test_hook_with_pixels(gpu_lib):
    ms = inputs.make_mapset(range(100, 104), 256, 1024)
    pe = PairedEnvs(ms, 256, obs_mode=binding.OBS_PIXELS, sprites=inputs.make_sprites(30),
                    hook_mode=binding.HOOK_GRAPPLE)
    acts, aims = hook_inputs(4, 40, 256)
    run(pe, acts, aims, "hook pixels", obs_every=4)


def test_hook_with_waypoints_and_respawn(gpu_lib):
    ms = inputs.make_mapset([7, 8, 9], 32, 40)
    wpt, lens = waypoint_table(ms)
    pe = PairedEnvs(ms, 300, time_limit=30, reward_mode=binding.REWARD_WAYPOINTS, waypoints=wpt, wp_lens=lens,
                    respawn_mode=binding.RESPAWN_ADAPTIVE, respawn_seed=77, hook_mode=binding.HOOK_GRAPPLE)
    acts, aims = hook_inputs(5, 150, 300)
    phases, _, _ = run(pe, acts, aims, "hook + waypoints + respawn", obs_every=5)
    assert phases[2] > 0


def test_hook_mode_without_aims_never_fires(gpu_lib):
    ms = inputs.make_mapset([1], 32, 128)
    pe = PairedEnvs(ms, 128, hook_mode=binding.HOOK_GRAPPLE)
    acts, _ = hook_inputs(6, 40, 128)
    phases, _, _ = run(pe, acts, None, "hook without aims", obs_every=10)
    assert phases[1] == 0 and phases[2] == 0


def test_aims_need_hook_mode(gpu_lib):
    ms = inputs.make_mapset([1], 32, 128)
    env = binding.Env(ms.maps, ms.ckpts, ms.spawns, 8)
    obs = env.new_obs()
    r = torch.empty(8, dtype=torch.float32, device="cuda")
    a = torch.zeros(8, dtype=torch.int32, device="cuda")
    with pytest.raises(binding.RLError, match="grapple"):
        env.step(a, obs, r, r.clone(), aim=torch.zeros(8, dtype=torch.int32, device="cuda"))
    with pytest.raises(binding.RLError, match="hook_mode"):
        binding.Env(ms.maps, ms.ckpts, ms.spawns, 8, hook_mode=2)
    # a misaligned aim array is refused before anything is enqueued
    hk = binding.Env(ms.maps, ms.ckpts, ms.spawns, 8, hook_mode=binding.HOOK_GRAPPLE)
    aim = torch.zeros(9, dtype=torch.int32, device="cuda")
    P = lambda x: ctypes.c_void_p(x.data_ptr())
    rc = binding.lib().rl_env_step_aim(hk._handle, P(a), ctypes.c_void_p(aim.data_ptr() + 2), P(obs), P(r), P(r),
                                       None)
    assert rc == -2 and "aligned" in binding.lib().rl_last_error().decode()


def test_masked_reset_while_hooks_fly_and_hold(gpu_lib):
    # a masked reset puts every third env back at its spawn with the hook idle and the tip cleared, while the
    # other envs' tips keep flying or holding; the run then continues on both sides
    ms = inputs.make_mapset([7, 8], 32, 128)
    pe = PairedEnvs(ms, 333, hook_mode=binding.HOOK_GRAPPLE)
    acts, aims = hook_inputs(31, 40, 333, p_hook=0.85)
    run(pe, acts[:14], aims[:14], "hook before the reset", obs_every=0)
    phase = pe.ora.state[:, F["hook_phase"]]
    mask = (np.arange(333) % 3 == 0).astype(np.uint8)
    assert (phase[mask == 1] != 0).any() and (phase[mask == 0] != 0).any()
    pe.gpu.reset(pe.obs, mask=torch.from_numpy(mask).cuda())
    pe.ora.reset(mask)
    pe.check_state("hook masked reset")
    pe.check_obs("hook masked reset")
    assert (pe.ora.state[mask == 1][:, F["hook_phase"]] == 0).all()
    phases, _, _ = run(pe, acts[14:], aims[14:], "hook after the reset", obs_every=5)
    assert phases[1] > 0 and phases[2] > 0
