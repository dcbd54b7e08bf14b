"""GPU parity of the whole hot path chained through device buffers, at the tiny workload: 64 envs on one
seeded 32x128 map, 128 decisions of uniform actions written into a resident [T] rollout buffer; GAE
(gamma 0.99, lambda 0.95) with whole-batch statistics over the rewards and dones the env produced; the loss
over 16 shuffled minibatches with the normalisation applied inline, and its gradient. Each stage is checked
against the oracle run on the same inputs: bit-exact for the env, the stated tolerances for the rest."""
import numpy as np
import pytest
import torch

import oracle
from resident_rl_rollout_amd import binding, inputs
from tests.gpu_helpers import assert_gae_close, assert_grad_close, assert_loss_close

pytestmark = pytest.mark.gpu

T, N, MB = 128, 64, 512
GAMMA, LAMBDA = 0.99, 0.95


def test_tiny_workload_end_to_end(gpu_lib):
    ms = inputs.make_mapset([1], 32, 128)
    env = binding.Env(ms.maps, ms.ckpts, ms.spawns, N)
    ora = oracle.OracleEnv(ms.maps, ms.ckpts, ms.spawns, N)
    ora.reset()
    obs = torch.empty((T + 1, N, binding.OBS_TILES_SIZE), dtype=torch.float32, device="cuda")
    rew = torch.empty((T, N), dtype=torch.float32, device="cuda")
    dn = torch.empty_like(rew)
    acts = inputs.make_actions(2, T, N)
    env.reset(obs[0])
    want_obs = {0: ora.obs_tiles()}
    r_ref, d_ref = np.empty((T, N), np.float32), np.empty((T, N), np.float32)
    a_dev = torch.from_numpy(acts).cuda()
    for t in range(T):
        env.step(a_dev[t], obs[t + 1], rew[t], dn[t])
        r_ref[t], d_ref[t] = ora.step(acts[t])
        if t % 16 == 15 or t == T - 1:
            want_obs[t + 1] = ora.obs_tiles()
    np.testing.assert_array_equal(rew.cpu().numpy(), r_ref)
    np.testing.assert_array_equal(dn.cpu().numpy(), d_ref)
    np.testing.assert_array_equal(env.read_state().cpu().numpy(), ora.state)
    got_obs = obs.cpu().numpy()
    for t, want in want_obs.items():
        np.testing.assert_array_equal(got_obs[t], want, err_msg=f"observation after decision {t}")
    assert d_ref.sum() > 0 or r_ref.std() > 0      # the rollout did something

    # GAE on the device's own rewards and dones, statistics for the loss
    values, last = inputs.make_values(3, T, N)
    adv, ret, stats = binding.gae(rew, torch.from_numpy(values).cuda(), dn, torch.from_numpy(last).cuda(),
                                  GAMMA, LAMBDA, normalize=2)
    ra, rr = oracle.gae(r_ref, values, d_ref, last, float(np.float32(GAMMA)), float(np.float32(LAMBDA)))
    na, mean, std = oracle.normalize(ra)
    assert_gae_close(adv.cpu().numpy(), ra, "advantages")
    assert_gae_close(ret.cpu().numpy(), rr, "returns")
    st = stats.cpu().numpy()
    assert st[0] == T * N
    assert abs(st[1] - mean) <= 1e-5 * (abs(mean) + std) and abs(st[2] - std) <= 1e-5 * std

    # the loss and its gradient over 16 minibatches, normalisation applied inline from the statistics
    b = T * N
    pi = inputs.make_policy_inputs(4, b)
    idx = torch.from_numpy(inputs.minibatch_index(pi.perm, MB)).cuda()
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    args = (dev(pi.new_logits), dev(pi.actions), dev(pi.old_logp), adv.reshape(-1), ret.reshape(-1),
            dev(pi.new_values), None, MB)
    out = binding.ppo_loss(*args, adv_stats=stats, mb_index=idx)
    ref, scale = oracle.ppo_loss(pi.new_logits, pi.actions, pi.old_logp, na.reshape(-1), rr.reshape(-1),
                                 pi.new_values, pi.perm, MB)
    assert out.shape == (b // MB, 4)
    assert_loss_close(out.cpu().numpy(), ref, scale, "loss")
    out_g, dl, dv = binding.ppo_loss_grad(*args, adv_stats=stats, mb_index=idx)
    assert_loss_close(out_g.cpu().numpy(), ref, scale, "loss beside the gradient")
    g = oracle.ppo_loss_grad(pi.new_logits, pi.actions, pi.old_logp, na.reshape(-1), rr.reshape(-1),
                             pi.new_values, pi.perm, MB)
    assert_grad_close(dl.cpu().numpy(), dv.cpu().numpy(), g, na.reshape(-1), "gradient")
