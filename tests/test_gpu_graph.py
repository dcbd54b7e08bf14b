"""Steps captured in a HIP graph (through torch's CUDAGraph on ROCm) and replayed: the decision counter lives
in the state buffer and each step launch advances it on the device, so every replay continues where the
last one stopped (ring heads, and the adaptive respawn's draws keyed by the counter). Each replay's
observations, rewards, dones and final state are compared bit for bit with the oracle stepping on with the
same actions; the outputs are poisoned before each replay, and eager work and a synchronisation run
between the replays."""
import numpy as np
import pytest
import torch

import oracle
from resident_rl_rollout_amd import binding, inputs
from tests.gpu_helpers import poison

pytestmark = pytest.mark.gpu

T = 128


def _capture_and_replay(ms, n, steps, replays, what, sprites=None, **env_kw):
    obs_mode = binding.OBS_PIXELS if sprites is not None else binding.OBS_TILES
    ora_kw = {k: v for k, v in env_kw.items() if k in ("time_limit", "respawn_mode", "respawn_seed")}
    if env_kw.get("respawn_mode"):
        env_kw["ckpt_spawns"] = ms.ckpt_spawns
        ora_kw["ckpt_spawns"] = ms.ckpt_spawns
    env = binding.Env(ms.maps, ms.ckpts, ms.spawns, n, obs_mode=obs_mode, sprites=sprites, **env_kw)
    ora = oracle.OracleEnv(ms.maps, ms.ckpts, ms.spawns, n, sprites=sprites, **ora_kw)
    ora.reset()
    size = binding.OBS_TILES_SIZE if obs_mode == binding.OBS_TILES else binding.OBS_PIXELS_SIZE
    obs = torch.empty((steps, n, size), dtype=env.obs_dtype, device="cuda")
    rew = torch.empty((steps, n), dtype=torch.float32, device="cuda")
    dn = torch.empty_like(rew)
    acts_np = inputs.make_actions(50, steps, n)
    if env_kw.get("time_limit", 2000) < 100:                 # mostly rightward: checkpoints and restarts
        acts_np = np.where(np.random.default_rng(51).random((steps, n)) < 0.7, 8 + acts_np % 4, acts_np)
    acts = torch.from_numpy(np.ascontiguousarray(acts_np, np.int32)).cuda()
    env.reset(obs[0])
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(graph, stream=side):
        for t in range(steps):
            env.step(acts[t], obs[t], rew[t], dn[t])
    assert int(env.read_step_counter()[0]) == 0           # capturing ran nothing
    for rep in range(replays):
        poison(obs, rew, dn, obs_mode, rep)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert int(env.read_step_counter()[0]) == (rep + 1) * steps, f"{what}: device counter after replay {rep}"
        r_ref = np.empty((steps, n), np.float32)
        d_ref = np.empty((steps, n), np.float32)
        got_obs = obs.cpu().numpy()
        for t in range(steps):
            r_ref[t], d_ref[t] = ora.step(acts_np[t])
            if t % 16 == 0 or t == steps - 1:
                want = ora.obs_tiles() if sprites is None else ora.obs_pixels().reshape(n, -1)
                np.testing.assert_array_equal(got_obs[t].view(np.uint8), want.view(np.uint8),
                                              err_msg=f"{what}: replay {rep} observations of decision {t}")
        np.testing.assert_array_equal(rew.cpu().numpy(), r_ref, err_msg=f"{what}: replay {rep} rewards")
        np.testing.assert_array_equal(dn.cpu().numpy(), d_ref, err_msg=f"{what}: replay {rep} dones")
        np.testing.assert_array_equal(env.read_state().cpu().numpy(), ora.state, err_msg=f"{what}: replay {rep} state")
        if env_kw.get("respawn_mode"):
            ring, fill, head, front = (x.cpu().numpy() for x in env.read_respawn())
            np.testing.assert_array_equal(fill, ora.fill, err_msg=f"{what}: respawn fill")
            np.testing.assert_array_equal(front, ora.frontier, err_msg=f"{what}: respawn frontier")
        # eager work between the replays
        (torch.ones(1 << 20, device="cuda") * 3.0).sum().item()
    return env, ora, d_ref


def test_captured_steps_replay_tiny_workload(gpu_lib):
    ms = inputs.make_mapset([1], 32, 128)
    _capture_and_replay(ms, 64, T, 3, "tiny")


def test_eager_steps_after_replays_continue_from_the_device_counter(gpu_lib):
    # replays advance only the device's copy of the counter: later steps outside a capture must read it
    # (the ring head and the respawn draws), not the host's count
    ms = inputs.make_mapset([7, 8, 9], 32, 40)
    env, ora, _ = _capture_and_replay(ms, 300, 6, 2, "respawn", time_limit=40,
                                      respawn_mode=binding.RESPAWN_ADAPTIVE, respawn_seed=78)
    assert env.step_counter == 6                     # the host counted the captured launches once
    acts_np = inputs.make_actions(52, 30, 300)
    obs = torch.empty((300, binding.OBS_TILES_SIZE), dtype=torch.float32, device="cuda")
    rew = torch.empty(300, dtype=torch.float32, device="cuda")
    dn = torch.empty_like(rew)
    for t in range(30):
        env.step(torch.from_numpy(np.ascontiguousarray(acts_np[t], np.int32)).cuda(), obs, rew, dn)
        r_ref, d_ref = ora.step(acts_np[t])
        np.testing.assert_array_equal(rew.cpu().numpy(), r_ref, err_msg=f"eager step {t}: rewards")
        np.testing.assert_array_equal(dn.cpu().numpy(), d_ref, err_msg=f"eager step {t}: dones")
        np.testing.assert_array_equal(obs.cpu().numpy().view(np.uint8), ora.obs_tiles().view(np.uint8),
                                      err_msg=f"eager step {t}: observations")
    np.testing.assert_array_equal(env.read_state().cpu().numpy(), ora.state)
    assert int(env.read_step_counter()[0]) == 12 + 30


def test_captured_steps_replay_with_adaptive_respawn(gpu_lib):
    # short maps and a 40-tick limit: episodes end and restart at checkpoints drawn with counter-keyed draws
    ms = inputs.make_mapset([7, 8, 9], 32, 40)
    _, ora, _ = _capture_and_replay(ms, 300, 48, 3, "respawn", time_limit=40, respawn_mode=binding.RESPAWN_ADAPTIVE,
                                    respawn_seed=77)
    assert ora.fill.sum() > 0


def test_captured_steps_replay_pixels(gpu_lib):
    ms = inputs.make_mapset(range(100, 104), 256, 1024)
    _capture_and_replay(ms, 256, 24, 2, "pixels", sprites=inputs.make_sprites(30))


def test_counter_set_before_capture_is_refused_inside_it(gpu_lib):
    ms = inputs.make_mapset([1], 32, 128)
    env = binding.Env(ms.maps, ms.ckpts, ms.spawns, 64)
    obs = env.new_obs()
    rew = torch.empty(64, dtype=torch.float32, device="cuda")
    dn = torch.empty_like(rew)
    a = torch.zeros(64, dtype=torch.int32, device="cuda")
    env.reset(obs)
    env.step_counter = 40
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with pytest.raises(binding.RLError, match="outside the capture"):
        with torch.cuda.graph(graph, stream=torch.cuda.Stream()):
            env.step(a, obs, rew, dn)
    torch.cuda.synchronize()
    env.step(a, obs, rew, dn)            # applied eagerly: the device counter continues from 40
    assert int(env.read_step_counter()[0]) == 41
    graph2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph2, stream=torch.cuda.Stream()):
        env.step(a, obs, rew, dn)
    graph2.replay()
    graph2.replay()
    torch.cuda.synchronize()
    assert int(env.read_step_counter()[0]) == 43


def test_captured_learn_phase_replays_bit_for_bit(gpu_lib):
    # GAE with the deferred statistics, the loss from a permutation (its sort, then the stream pass placing
    # its own bins, with launch-time LDS) and the loss
    # gradient from minibatch numbers, recorded into one graph: no call may allocate, synchronise or leave
    # a memset in the graph, so every replay must give the eager call's bits. Outputs are poisoned before
    # each replay; eager work and a synchronisation run between the replays.
    t, n = 64, 4096
    b, mb = t * n, t * n // 16
    gi = inputs.make_gae_inputs(61, t, n)
    pi = inputs.make_policy_inputs(62, b)
    d = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    r, v, dn, lv = d(gi.rewards), d(gi.values), d(gi.dones), d(gi.last_values)
    logits, acts, old, nv, perm = d(pi.new_logits), d(pi.actions), d(pi.old_logp), d(pi.new_values), d(pi.perm)
    idx = d(inputs.minibatch_index(pi.perm, mb))
    adv = torch.empty((t, n), dtype=torch.float32, device="cuda")
    ret = torch.empty_like(adv)
    stats = torch.zeros(binding.gae_stats_bytes(t, n) // 8, dtype=torch.float64, device="cuda")
    out = torch.empty((16, 4), dtype=torch.float32, device="cuda")
    out_g = torch.empty_like(out)
    dl = torch.empty((b, 12), dtype=torch.float32, device="cuda")
    dv = torch.empty(b, dtype=torch.float32, device="cuda")
    ws = torch.zeros(binding.ppo_loss_workspace_bytes(b, mb), dtype=torch.uint8, device="cuda")

    def learn():
        binding.gae(r, v, dn, lv, 0.99, 0.95, normalize=3, adv=adv, ret=ret, adv_stats=stats)
        binding.ppo_loss(logits, acts, old, adv.view(-1), ret.view(-1), nv, perm, mb, adv_stats=stats, out=out,
                         ws=ws)
        binding.ppo_loss_grad(logits, acts, old, adv.view(-1), ret.view(-1), nv, None, mb, adv_stats=stats,
                              out=out_g, dlogits=dl, dvalues=dv, ws=ws, mb_index=idx)

    learn()
    torch.cuda.synchronize()
    outs = (adv, ret, out, out_g, dl, dv)
    want = [x.clone() for x in outs]
    want_stats = stats.clone()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=side):
        learn()
    for rep in range(3):
        for x in outs:
            x.fill_(float("nan"))
        stats[:2].fill_(float("nan"))     # the header's spare doubles are never written
        stats[4:].fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, x, w in zip(("adv", "ret", "loss", "loss of the gradient call", "dlogits", "dvalues"), outs, want):
            torch.testing.assert_close(x, w, rtol=0, atol=0, msg=f"replay {rep}: {name}")
        torch.testing.assert_close(stats, want_stats, rtol=0, atol=0, msg=f"replay {rep}: statistics")
        (torch.ones(1 << 20, device="cuda") * 3.0).sum().item()
