"""GPU parity of the adaptive checkpoint respawn ("boesch.dev DDNet RL post", Checkpoint Respawning)
against the oracle: bit-exact state (including the from-start flag), observations, rewards, dones and each
map's outcome buffer, fill, write position and frontier."""
import numpy as np
import pytest

from resident_rl_rollout_amd import binding, inputs
from tests.gpu_helpers import PairedEnvs, waypoint_table

pytestmark = pytest.mark.gpu


def _rightward(seed, t, n, p_right=0.8):
    rng = np.random.default_rng(seed)
    return np.where(rng.random((t, n)) < p_right, 8 + rng.integers(0, 4, (t, n)),
                    rng.integers(0, 12, (t, n))).astype(np.int32)


def _run(pe, actions, what, obs_every=1, buf_every=1):
    pe.check_obs(f"{what} reset")
    for s, a in enumerate(actions):
        r, d = pe.step(a)
        pe.check_step(r, d, f"{what} step {s}")
        pe.check_state(f"{what} step {s}")
        if buf_every and (s % buf_every == 0 or s == len(actions) - 1):
            pe.check_respawn(f"{what} step {s}")
        if obs_every and (s % obs_every == 0 or s == len(actions) - 1):
            pe.check_obs(f"{what} step {s}")


def test_respawn_short_maps(gpu_lib):
    # 3 maps with 7 checkpoints; 80-decision episodes, so outcomes accumulate and respawns follow
    ms = inputs.make_mapset([7, 8, 9], 32, 120)
    pe = PairedEnvs(ms, 300, time_limit=240, respawn_mode=binding.RESPAWN_ADAPTIVE, respawn_seed=99)
    _run(pe, _rightward(1, 400, 300), "respawn", obs_every=10, buf_every=5)
    st = pe.gpu.read_state().cpu().numpy()
    assert (st[:, 17] == 0).any(), "no episode restarted at a checkpoint"


def test_respawn_with_waypoint_reward(gpu_lib):
    ms = inputs.make_mapset([4, 5], 48, 150)
    table, lens = waypoint_table(ms)
    pe = PairedEnvs(ms, 256, time_limit=300, respawn_mode=binding.RESPAWN_ADAPTIVE, respawn_seed=2 ** 63 + 5,
                    reward_mode=binding.REWARD_WAYPOINTS, waypoints=table, wp_lens=lens)
    _run(pe, _rightward(2, 350, 256), "respawn+waypoints", obs_every=25, buf_every=10)


def test_respawn_pixels(gpu_lib):
    ms = inputs.make_mapset([7, 8], 32, 120)
    pe = PairedEnvs(ms, 128, time_limit=150, respawn_mode=binding.RESPAWN_ADAPTIVE, respawn_seed=3,
                    obs_mode=binding.OBS_PIXELS, sprites=inputs.make_sprites(30))
    _run(pe, _rightward(3, 200, 128), "respawn pixels", obs_every=20, buf_every=10)


def test_respawn_mass_resets_full_size(gpu_lib):
    # 65536 envs on 64 maps with a 100-tick limit: every env ends at decisions 34 and 68, so each map takes
    # 1024 outcomes at once (only the last 64 stay in its buffer); the first round's finds of checkpoint 1
    # open the frontier for the second round's respawns
    ms = inputs.make_mapset(range(100, 164), 256, 1024)
    pe = PairedEnvs(ms, 65536, time_limit=100, respawn_mode=binding.RESPAWN_ADAPTIVE, respawn_seed=17)
    _run(pe, _rightward(4, 75, 65536, p_right=0.95), "respawn 65536", obs_every=15, buf_every=1)
    assert (pe.ora.frontier > 0).any() and (pe.ora.state[:, 17] == 0).any()


def test_respawn_needs_spots(gpu_lib):
    import ctypes

    import torch
    ms = inputs.make_mapset([1], 32, 128)
    k = ms.ckpts.shape[1]
    cfg = binding.EnvConfig(8, 1, 32, 128, k, 3, 2000, 0, 1397, 0, 0, 1, 5)
    nb = ctypes.c_size_t()
    binding.check(binding.lib().rl_env_state_bytes(ctypes.byref(cfg), ctypes.byref(nb)))
    state = torch.empty(nb.value, dtype=torch.uint8, device="cuda")
    h = ctypes.c_void_p()
    maps, ck, sp = (torch.from_numpy(x).cuda() for x in (ms.maps, ms.ckpts, ms.spawns))
    binding.check(binding.lib().rl_env_create(ctypes.byref(cfg), maps.data_ptr(), ck.data_ptr(), sp.data_ptr(), None,
                                              state.data_ptr(), nb.value, None, ctypes.byref(h)))
    obs = torch.empty((8, 1397), device="cuda")
    a = torch.zeros(8, dtype=torch.int32, device="cuda")
    r = torch.empty(8, device="cuda")
    with pytest.raises(binding.RLError, match="rl_env_set_respawn_spots"):
        binding.check(binding.lib().rl_env_step(h, a.data_ptr(), obs.data_ptr(), r.data_ptr(), r.data_ptr(), None))
    binding.lib().rl_env_destroy(h)
