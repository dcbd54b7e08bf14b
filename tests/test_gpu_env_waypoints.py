"""GPU parity of the waypoint-path reward mode ("boesch.dev DDNet RL post", Reward Engineering, Version 2)
against the oracle: bit-exact state (including the path high-water index), observations, rewards and
dones, tiles and pixels, with each map's BFS tile path as the waypoint table."""
import numpy as np
import pytest

from resident_rl_rollout_amd import binding, inputs
from tests.gpu_helpers import PairedEnvs, waypoint_table

pytestmark = pytest.mark.gpu
F = {name: i for i, name in enumerate(("x", "y", "vx", "vy", "facing", "freeze_ticks", "hook_ticks", "hook_held",
                                       "jump_held", "grounded", "wall_left", "wall_right", "tick", "next_ckpt",
                                       "best_x", "last_action", "path"))}


def _pair(ms, n, **kw):
    table, lens = waypoint_table(ms)
    return PairedEnvs(ms, n, reward_mode=binding.REWARD_WAYPOINTS, waypoints=table, wp_lens=lens, **kw)


def _run(pe, actions, what, obs_every=1):
    pe.check_obs(f"{what} reset")
    for s, a in enumerate(actions):
        r, d = pe.step(a)
        pe.check_step(r, d, f"{what} step {s}")
        pe.check_state(f"{what} step {s}")
        if obs_every and (s % obs_every == 0 or s == len(actions) - 1):
            pe.check_obs(f"{what} step {s}")


def _rightward(seed, t, n, p_right=0.7):
    rng = np.random.default_rng(seed)
    return np.where(rng.random((t, n)) < p_right, 8 + rng.integers(0, 4, (t, n)),
                    rng.integers(0, 12, (t, n))).astype(np.int32)


def test_tiny_workload_waypoints(gpu_lib):
    ms = inputs.make_mapset([1], 32, 128)
    pe = _pair(ms, 64)
    _run(pe, inputs.make_actions(2, 128, 64), "tiny waypoints")


def test_progress_penalty_and_finishes(gpu_lib):
    # mostly rightward play on short maps: progress along the path, finishes and resets, and envs that
    # jump or wander past the grace zone
    ms = inputs.make_mapset([7, 8, 9], 32, 40)
    pe = _pair(ms, 300, time_limit=400)
    acts = _rightward(3, 200, 300)
    _run(pe, acts, "waypoints resets", obs_every=5)
    st = pe.gpu.read_state().cpu().numpy()
    assert st[:, F["path"]].max() > 0


@pytest.mark.parametrize("fs", [1, 5])
def test_frame_skip_settings_waypoints(fs, gpu_lib):
    ms = inputs.make_mapset([4, 5], 48, 96)
    pe = _pair(ms, 200, frame_skip=fs, time_limit=90)
    _run(pe, inputs.make_actions(6, 60, 200), f"waypoints fs={fs}", obs_every=7)


def test_env_step_workload_waypoints(gpu_lib):
    # 65536 envs on 64 seeded 256x1024 maps, 12 decisions, every env compared
    ms = inputs.make_mapset(range(100, 164), 256, 1024)
    pe = _pair(ms, 65536)
    _run(pe, _rightward(11, 12, 65536), "waypoints 65536", obs_every=4)


def test_pixels_waypoints(gpu_lib):
    ms = inputs.make_mapset([4, 5], 48, 96)
    pe = _pair(ms, 256, obs_mode=binding.OBS_PIXELS, sprites=inputs.make_sprites(30))
    _run(pe, _rightward(12, 24, 256), "waypoints pixels", obs_every=6)


def test_step_without_waypoints_is_rejected(gpu_lib):
    ms = inputs.make_mapset([1], 32, 128)
    table, lens = waypoint_table(ms)
    env = binding.Env(ms.maps, ms.ckpts, ms.spawns, 8)
    with pytest.raises(binding.RLError, match="waypoint"):
        binding.check(binding.lib().rl_env_set_waypoints(env._handle, None, None, None))
    import ctypes
    cfg = binding.EnvConfig(8, 1, 32, 128, ms.ckpts.shape[1], 3, 2000, 0, 1397, 1, table.shape[1])
    nb = ctypes.c_size_t()
    binding.check(binding.lib().rl_env_state_bytes(ctypes.byref(cfg), ctypes.byref(nb)))
    import torch
    state = torch.empty(nb.value, dtype=torch.uint8, device="cuda")
    h = ctypes.c_void_p()
    maps = torch.from_numpy(ms.maps).cuda()
    ck = torch.from_numpy(ms.ckpts).cuda()
    sp = torch.from_numpy(ms.spawns).cuda()
    binding.check(binding.lib().rl_env_create(ctypes.byref(cfg), maps.data_ptr(), ck.data_ptr(), sp.data_ptr(), None,
                                              state.data_ptr(), nb.value, None, ctypes.byref(h)))
    obs = torch.empty((8, 1397), device="cuda")
    a = torch.zeros(8, dtype=torch.int32, device="cuda")
    r = torch.empty(8, device="cuda")
    with pytest.raises(binding.RLError, match="rl_env_set_waypoints"):
        binding.check(binding.lib().rl_env_step(h, a.data_ptr(), obs.data_ptr(), r.data_ptr(), r.data_ptr(), None))
    binding.lib().rl_env_destroy(h)


def test_shortened_table_mid_episode(gpu_lib):
    # mostly rightward play until the high-water indexes are well along the paths, then a table cut below
    # them through rl_env_set_waypoints (the index is clamped to the new last waypoint), then the full
    # table again: bit-exact against the oracle given the same lengths at the same decisions
    ms = inputs.make_mapset([7, 8, 9], 32, 40)
    table, lens = waypoint_table(ms)
    pe = PairedEnvs(ms, 300, reward_mode=binding.REWARD_WAYPOINTS, waypoints=table, wp_lens=lens.copy(),
                    time_limit=10 ** 6)           # a copy: the oracle keeps its lengths array and reads it each step
    acts = _rightward(11, 150, 300, p_right=0.9)
    _run(pe, acts[:50], "before the cut", obs_every=10)
    st = pe.gpu.read_state().cpu().numpy()
    short = np.maximum(1, lens // 4).astype(np.int32)
    assert (st[:, F["path"]] > short[np.arange(300) % 3] - 1).any()      # some indexes lie past the new end
    pe.gpu.set_waypoints(table, short)
    pe.ora.wp_lens[:] = short
    _run(pe, acts[50:100], "shortened table", obs_every=10)
    pe.gpu.set_waypoints(table, lens)
    pe.ora.wp_lens[:] = lens
    _run(pe, acts[100:], "full table again", obs_every=10)
