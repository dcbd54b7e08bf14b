"""GPU parity of the full-size workloads in the launch configurations the bench times.

- The full rollout, chained through device buffers: 65536 envs x 128 decisions on the 64 seeded 256x1024
  maps into one resident [actions | obs | rewards | dones] rollout allocation, then GAE with whole-batch
  statistics over the device's own rewards and dones, then the loss over 16 shuffled minibatches of
  524288 with the normalisation applied inline, from the permutation (the boundary's perm input) and from
  the per-sample minibatch numbers. The oracle steps all 65536 envs too: every env's rewards and dones at
  every decision and its final state are compared bit for bit, every observation of three decisions,
  every GAE element, the statistics, and all 16 minibatches' loss scalars.
- The env-step workload for its whole timed length: 65536 envs for 1334 decisions (two full 667-decision
  episodes, so every env is truncated and reset twice inside the run), three stated 256-env ranges
  paired with the oracle at every decision.
- The pixel workload for its 128 decisions: 16384 envs, two stated 512-env ranges paired with the oracle.
Every output buffer is poisoned before it is written, so a store a kernel skipped cannot pass.
"""
import numpy as np
import pytest
import torch

import oracle
from resident_rl_rollout_amd import binding, inputs
from tests.gpu_helpers import SubsetPairs, assert_gae_close, assert_loss_close, poison

pytestmark = pytest.mark.gpu

N, T, MAPS, H, W, MB = 65536, 128, 64, 256, 1024, 16
G32, L32 = float(np.float32(0.99)), float(np.float32(0.95))


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
def test_rollout_workload_chained_full_shape(gpu_lib):
    ms = inputs.make_mapset(range(100, 100 + MAPS), H, W)
    b = T * N
    pi = inputs.make_policy_inputs(20, b)
    values, last = inputs.make_values(21, T, N)
    acts = pi.actions.reshape(T, N)

    # the GPU rollout, exactly as the bench lays it out and launches it
    env = binding.Env(ms.maps, ms.ckpts, ms.spawns, N)
    a_bytes, o_bytes = T * N * 4, T * N * 1397 * 4
    offs = [0, a_bytes, a_bytes + o_bytes, a_bytes + o_bytes + a_bytes]
    buf = torch.empty(offs[3] + a_bytes, dtype=torch.uint8, device="cuda")
    actions = buf[offs[0]:offs[1]].view(torch.int32).view(T, N)
    obs = buf[offs[1]:offs[2]].view(torch.float32).view(T, N, 1397)
    rewards = buf[offs[2]:offs[3]].view(torch.float32).view(T, N)
    dones = buf[offs[3]:].view(torch.float32).view(T, N)
    poison(obs, rewards, dones, binding.OBS_TILES, 0)
    actions.copy_(torch.from_numpy(acts))
    env.reset(obs[0])
    for t in range(T):
        env.step(actions[t], obs[t], rewards[t], dones[t])

    ora = oracle.OracleEnv(ms.maps, ms.ckpts, ms.spawns, N)
    ora.reset()
    r_ref, d_ref = np.empty((T, N), np.float32), np.empty((T, N), np.float32)
    for t in range(T):
        r_ref[t], d_ref[t] = ora.step(acts[t])
        if t in (0, T // 2 - 1, T - 1):
            np.testing.assert_array_equal(obs[t].cpu().numpy().view(np.uint32), ora.obs_tiles().view(np.uint32),
                                          err_msg=f"observations after decision {t}")
    np.testing.assert_array_equal(rewards.cpu().numpy(), r_ref, err_msg="rewards")
    np.testing.assert_array_equal(dones.cpu().numpy(), d_ref, err_msg="dones")
    np.testing.assert_array_equal(env.read_state().cpu().numpy(), ora.state, err_msg="final state")
    env.close()

    # GAE with whole-batch statistics over the device's rewards and dones
    vd, ld = torch.from_numpy(values).cuda(), torch.from_numpy(last).cuda()
    adv, ret, stats = binding.gae(rewards, vd, dones, ld, 0.99, 0.95, normalize=2)
    ra, rr = oracle.gae(r_ref, values, d_ref, last, G32, L32)
    assert_gae_close(adv.cpu().numpy(), ra, "advantages, every element")
    assert_gae_close(ret.cpu().numpy(), rr, "returns, every element")
    na, mean, std = oracle.normalize(ra)
    st = stats.cpu().numpy()
    assert st[0] == b
    assert abs(st[1] - mean) <= 1e-5 * (abs(mean) + std) and abs(st[2] - std) <= 1e-5 * std
    del buf, obs

    # the loss over 16 minibatches, normalised inline: from the permutation and from minibatch numbers
    mb = b // MB
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    logits, old_logp, new_v, perm = dev(pi.new_logits), dev(pi.old_logp), dev(pi.new_values), dev(pi.perm)
    idx = dev(inputs.minibatch_index(pi.perm, mb))
    args = (logits, actions.reshape(-1), old_logp, adv.reshape(-1), ret.reshape(-1), new_v)
    out_perm = binding.ppo_loss(*args, perm, mb, adv_stats=stats).cpu().numpy()
    out_idx = binding.ppo_loss(*args, None, mb, adv_stats=stats, mb_index=idx).cpu().numpy()
    na, rr = na.reshape(-1), rr.reshape(-1)
    for m in range(MB):
        s = pi.perm[m * mb:(m + 1) * mb]
        ref, scale = oracle.ppo_loss(pi.new_logits[s], pi.actions[s], pi.old_logp[s], na[s], rr[s],
                                     pi.new_values[s], None, mb)
        assert_loss_close(out_perm[m:m + 1], ref, scale, f"minibatch {m} from perm")
        assert_loss_close(out_idx[m:m + 1], ref, scale, f"minibatch {m} from minibatch numbers")
    np.testing.assert_array_equal(out_perm, out_idx)     # the same sets, summed in the same order


@pytest.mark.timeout(600)
def test_env_workload_whole_timed_length(gpu_lib):
    steps = 1334
    ms = inputs.make_mapset(range(100, 100 + MAPS), H, W)
    env = binding.Env(ms.maps, ms.ckpts, ms.spawns, N, time_limit=2000)
    ranges = [(0, 256), (N // 2 - 128, N // 2 + 128), (N - 256, N)]
    sp = SubsetPairs(env, ms, ranges, time_limit=2000)
    obs = env.new_obs()
    rew = torch.empty(N, dtype=torch.float32, device="cuda")
    done = torch.empty_like(rew)
    env.reset(obs)
    sp.check_obs(obs, "reset")
    acts = inputs.make_actions(4, steps, N)
    a_dev = torch.empty(N, dtype=torch.int32, device="cuda")
    dones = 0
    for s in range(steps):
        a_dev.copy_(torch.from_numpy(acts[s]))
        poison(obs, rew, done, binding.OBS_TILES, s)
        env.step(a_dev, obs, rew, done)
        r, d = sp.step(acts[s])
        np.testing.assert_array_equal(rew[sp.sel].cpu().numpy(), r, err_msg=f"rewards at decision {s}")
        np.testing.assert_array_equal(done[sp.sel].cpu().numpy(), d, err_msg=f"dones at decision {s}")
        dones += int(d.sum())
        if s % 100 == 0 or s in (665, 666, 667, 1332, 1333):
            sp.check_state(f"decision {s}")
        if s in (0, 666, 667, 1333):
            sp.check_obs(obs, f"decision {s}")
    assert dones >= 2 * len(sp.sel_np)          # every paired env truncated at least twice
    env.close()


@pytest.mark.timeout(600)
def test_pixel_workload_whole_length(gpu_lib):
    n = 16384
    ms = inputs.make_mapset(range(100, 100 + MAPS), H, W)
    sprites = inputs.make_sprites(30)
    env = binding.Env(ms.maps, ms.ckpts, ms.spawns, n, obs_mode=binding.OBS_PIXELS, sprites=sprites)
    ranges = [(0, 512), (n - 512, n)]
    sp = SubsetPairs(env, ms, ranges, sprites=sprites)
    obs = env.new_obs()
    rew = torch.empty(n, dtype=torch.float32, device="cuda")
    done = torch.empty_like(rew)
    env.reset(obs)
    sp.check_obs(obs, "pixels reset")
    acts = inputs.make_actions(22, T, n)
    a_dev = torch.empty(n, dtype=torch.int32, device="cuda")
    for s in range(T):
        a_dev.copy_(torch.from_numpy(acts[s]))
        poison(obs, rew, done, binding.OBS_PIXELS, s)
        env.step(a_dev, obs, rew, done)
        r, d = sp.step(acts[s])
        np.testing.assert_array_equal(rew[sp.sel].cpu().numpy(), r, err_msg=f"pixel rewards at decision {s}")
        np.testing.assert_array_equal(done[sp.sel].cpu().numpy(), d, err_msg=f"pixel dones at decision {s}")
        sp.check_state(f"pixels decision {s}")
        if s % 8 == 0 or s == T - 1:
            sp.check_obs(obs, f"pixels decision {s}")
    env.close()
