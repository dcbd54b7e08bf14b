"""GPU parity of env_step + obs_gather (tiles and pixels) against the oracle: bit-exact state, observations,
rewards and dones, with the same seeded maps and actions on both sides."""
import itertools

import numpy as np
import pytest
import torch

from resident_rl_rollout_amd import binding, inputs
from tests.gpu_helpers import PairedEnvs

pytestmark = pytest.mark.gpu


def _run_and_check(pe, actions, what, obs_every=1, obs_envs=None):
    pe.check_obs(f"{what} reset")
    for s, a in enumerate(actions):
        r, d = pe.step(a)
        pe.check_step(r, d, f"{what} step {s}")
        pe.check_state(f"{what} step {s}")
        if obs_every and (s % obs_every == 0 or s == len(actions) - 1):
            pe.check_obs(f"{what} step {s}", obs_envs)


def test_tiny_workload_all_steps(gpu_lib):
    # N=64, one 32x128 map, 128 decisions of uniform actions
    ms = inputs.make_mapset([1], 32, 128)
    pe = PairedEnvs(ms, 64)
    _run_and_check(pe, inputs.make_actions(2, 128, 64), "tiny")


def test_short_time_limit_and_finish_resets(gpu_lib):
    # frequent truncation (25 ticks) and a map with checkpoints close to the spawn so finishes happen
    ms = inputs.make_mapset([7, 8, 9], 32, 40)
    pe = PairedEnvs(ms, 300, time_limit=25)
    rng = np.random.default_rng(3)
    acts = np.where(rng.random((150, 300)) < 0.7, 8 + rng.integers(0, 4, (150, 300)),
                    rng.integers(0, 12, (150, 300))).astype(np.int32)
    _run_and_check(pe, acts, "resets")
    pe2 = PairedEnvs(ms, 300, time_limit=10 ** 6)
    done_total = 0
    for s, a in enumerate(acts):
        r, d = pe2.step(a)
        pe2.check_step(r, d, f"finish step {s}")
        done_total += int(d.sum())
    pe2.check_state("finish")
    pe2.check_obs("finish")
    assert done_total > 0


def test_time_limit_one_ends_every_decision(gpu_lib):
    # every decision is one tick, truncated, and resets in place: all dones set every step, state and
    # observations those of the oracle (the new episodes' first)
    ms = inputs.make_mapset([4, 5, 6], 48, 96)
    pe = PairedEnvs(ms, 301, time_limit=1)
    acts = inputs.make_actions(12, 20, 301)
    pe.check_obs("tl=1 reset")
    for s, a in enumerate(acts):
        r, d = pe.step(a)
        pe.check_step(r, d, f"tl=1 step {s}")
        assert (d == 1.0).all()
        pe.check_state(f"tl=1 step {s}")
        pe.check_obs(f"tl=1 step {s}")


@pytest.mark.parametrize("fs", [1, 2, 5])
def test_frame_skip_settings(fs, gpu_lib):
    ms = inputs.make_mapset([4, 5], 48, 96)
    pe = PairedEnvs(ms, 200, frame_skip=fs, time_limit=90)
    _run_and_check(pe, inputs.make_actions(6, 60, 200), f"fs={fs}", obs_every=7)


def test_exhaustive_four_decisions(gpu_lib):
    ms = inputs.make_mapset([21], 32, 128)
    seqs = np.array(list(itertools.product(range(12), repeat=4)), np.int32)
    pe = PairedEnvs(ms, len(seqs))
    _run_and_check(pe, seqs.T.copy(), "12^4")


def test_out_of_range_actions_and_ragged_batch(gpu_lib):
    ms = inputs.make_mapset([13], 32, 64)
    pe = PairedEnvs(ms, 77)
    rng = np.random.default_rng(1)
    acts = rng.integers(-20, 30, (40, 77)).astype(np.int32)
    acts[:, 0] = -2 ** 31
    acts[:, 1] = 2 ** 31 - 1
    _run_and_check(pe, acts, "out of range")


def test_single_env_and_padded_obs_stride(gpu_lib):
    ms = inputs.make_mapset([2], 32, 128)
    pe = PairedEnvs(ms, 1, obs_stride=1408)
    pe.obs.fill_(-7.0)
    pe.gpu.reset(pe.obs)
    _run_and_check(pe, inputs.make_actions(3, 50, 1), "n=1 stride 1408")
    assert (pe.obs[:, 1397:] == -7.0).all()


def test_env_step_workload_full_size(gpu_lib):
    # 65536 envs on 64 maps of 256x1024, the bench's launch configuration; every env's state, reward and
    # done each step, and every observation at the first, a middle and the last step.
    ms = inputs.make_mapset(range(100, 164), 256, 1024)
    pe = PairedEnvs(ms, 65536)
    acts = inputs.make_actions(4, 24, 65536)
    pe.check_obs("full reset")
    for s, a in enumerate(acts):
        r, d = pe.step(a)
        pe.check_step(r, d, f"full step {s}")
        pe.check_state(f"full step {s}")
        if s in (0, 11, len(acts) - 1):
            pe.check_obs(f"full step {s}")


def test_time_limit_2000_inside_the_run(gpu_lib):
    # 700 decisions cross the 2000-tick limit (decision 667) on every env: auto-reset in the stream.
    ms = inputs.make_mapset(range(100, 108), 256, 1024)
    pe = PairedEnvs(ms, 2048)
    acts = inputs.make_actions(5, 700, 2048)
    dones = 0
    for s, a in enumerate(acts):
        r, d = pe.step(a)
        pe.check_step(r, d, f"step {s}")
        dones += int(d.sum())
        if s % 50 == 0 or s in (666, 667, 699):
            pe.check_state(f"step {s}")
            pe.check_obs(f"step {s}", envs=slice(0, 2048, 7))
    assert dones >= 2048


def test_masked_reset_and_snapshot_resume(gpu_lib):
    ms = inputs.make_mapset([40, 41], 32, 128)
    pe = PairedEnvs(ms, 500)
    acts = inputs.make_actions(42, 60, 500)
    for a in acts[:20]:
        pe.step(a)
    mask = (np.arange(500) % 3 == 0).astype(np.uint8)
    pe.gpu.reset(pe.obs, mask=torch.from_numpy(mask).cuda())
    pe.ora.reset(mask)
    pe.check_state("masked reset")
    pe.check_obs("masked reset")
    # snapshot = state buffer + step counter; resuming from it reproduces the same trajectory
    snap, counter = pe.gpu.state.clone(), pe.gpu.step_counter
    outs = []
    for rep in range(2):
        if rep == 1:
            pe.gpu.state.copy_(snap)
            pe.gpu.step_counter = counter
        for a in acts[20:]:
            pe.gpu.step(torch.from_numpy(a).cuda(), pe.obs, pe.rew, pe.done)
        outs.append((pe.gpu.read_state().cpu().numpy(), pe.obs.cpu().numpy()))
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    np.testing.assert_array_equal(outs[0][1], outs[1][1])


def test_pixels_small(gpu_lib):
    ms = inputs.make_mapset(range(100, 104), 256, 1024)
    sprites = inputs.make_sprites(30)
    pe = PairedEnvs(ms, 256, obs_mode=binding.OBS_PIXELS, sprites=sprites)
    _run_and_check(pe, inputs.make_actions(31, 40, 256), "pixels")


def test_pixels_ragged_batch_and_padded_stride(gpu_lib):
    # 257 envs (a partial wave in the physics kernel) and rows of 28228 bytes (not a 16-byte multiple)
    ms = inputs.make_mapset(range(110, 113), 256, 1024)
    sprites = inputs.make_sprites(31)
    pe = PairedEnvs(ms, 257, obs_mode=binding.OBS_PIXELS, sprites=sprites, obs_stride=28228)
    _run_and_check(pe, inputs.make_actions(33, 30, 257), "pixels n=257 stride 28228", obs_every=5)


def test_pixels_workload_full_size(gpu_lib):
    ms = inputs.make_mapset(range(100, 164), 256, 1024)
    sprites = inputs.make_sprites(30)
    pe = PairedEnvs(ms, 16384, obs_mode=binding.OBS_PIXELS, sprites=sprites)
    acts = inputs.make_actions(32, 12, 16384)
    pe.check_obs("pixels full reset")
    for s, a in enumerate(acts):
        r, d = pe.step(a)
        pe.check_step(r, d, f"pixels full step {s}")
        if s in (0, len(acts) - 1):
            pe.check_state(f"pixels full step {s}")
            pe.check_obs(f"pixels full step {s}")


def test_step_block_layout(gpu_lib):
    # one contiguous [actions | obs | rewards | dones] block per step, sub-arrays 256-byte aligned
    ms = inputs.make_mapset([1], 32, 128)
    env = binding.Env(ms.maps, ms.ckpts, ms.spawns, 100)
    offs, total = env.step_layout()
    assert offs[0] == 0 and all(o % 256 == 0 for o in offs) and total % 256 == 0
    assert offs[1] >= 400 and offs[2] >= offs[1] + 100 * 1397 * 4 and offs[3] >= offs[2] + 400
    block = torch.empty(total, dtype=torch.uint8, device="cuda")
    acts = block[offs[0]:offs[0] + 400].view(torch.int32)
    obs = block[offs[1]:offs[1] + 100 * 1397 * 4].view(torch.float32).view(100, 1397)
    rew = block[offs[2]:offs[2] + 400].view(torch.float32)
    dn = block[offs[3]:offs[3] + 400].view(torch.float32)
    acts.copy_(torch.from_numpy(inputs.make_actions(1, 1, 100)[0]))
    env.step(acts, obs, rew, dn)
    ref = PairedEnvs(ms, 100)
    r, d = ref.step(inputs.make_actions(1, 1, 100)[0])
    np.testing.assert_array_equal(obs.cpu().numpy(), ref.oracle_obs())
    np.testing.assert_array_equal(rew.cpu().numpy(), r)
