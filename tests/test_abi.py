"""The C ABI without a GPU: librl.so loads, exports every function include/rl.h declares, and rejects
invalid arguments with the documented status before any HIP call."""
import ctypes
import os
import re

import pytest

from resident_rl_rollout_amd import binding

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "rl.h")


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"\b(rl_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("rl_env_create", "rl_env_reset", "rl_env_step", "rl_env_destroy", "rl_gae", "rl_ppo_loss",
                     "rl_policy_forward", "rl_rollout", "rl_last_error"):
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(binding.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert sorted(n for n, _, _ in binding.SIGNATURES) == declared_functions()


def _cfg(**kw):
    base = dict(num_envs=64, num_maps=1, map_h=32, map_w=128, num_ckpts=7, frame_skip=3, time_limit=2000,
                obs_mode=0, obs_stride=1397, reward_mode=0, max_waypoints=0, respawn_mode=0, respawn_seed=0,
                hook_mode=0)
    base.update(kw)
    return binding.EnvConfig(*[base[k] for k, _ in binding.EnvConfig._fields_])


@pytest.mark.parametrize("kw,code,msg", [
    (dict(num_envs=0), -1, "num_envs"), (dict(num_maps=0), -1, "num_maps"), (dict(map_h=0), -1, "map_h"),
    (dict(map_w=70000), -1, "map_w"), (dict(num_ckpts=-1), -1, "num_ckpts"), (dict(frame_skip=0), -1, "frame_skip"),
    (dict(frame_skip=6), -1, "frame_skip"), (dict(time_limit=0), -1, "time_limit"), (dict(obs_mode=2), -1, "obs_mode"),
    (dict(obs_stride=1396), -1, "obs_stride"), (dict(obs_mode=1, obs_stride=28226), -2, "multiple of 4"),
    (dict(num_envs=(1 << 24) + 1), -1, "num_envs"), (dict(reward_mode=2), -1, "reward_mode"),
    (dict(reward_mode=1, max_waypoints=0), -1, "max_waypoints"),
    (dict(reward_mode=1, max_waypoints=(1 << 20) + 1), -1, "max_waypoints"),
    (dict(respawn_mode=2), -1, "respawn_mode"), (dict(respawn_mode=1, num_ckpts=0), -1, "checkpoints"),
    (dict(respawn_mode=1, num_ckpts=1025), -1, "checkpoints"), (dict(hook_mode=2), -1, "hook_mode"),
    (dict(hook_mode=-1), -1, "hook_mode"),
])
def test_config_validation(kw, code, msg):
    lib = binding.lib()
    n = ctypes.c_size_t()
    assert lib.rl_env_state_bytes(ctypes.byref(_cfg(**kw)), ctypes.byref(n)) == code
    assert msg in lib.rl_last_error().decode()


def test_sizes_and_layout():
    lib = binding.lib()
    n, e, b = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.rl_env_obs_size(ctypes.byref(_cfg()), ctypes.byref(n), ctypes.byref(e)) == 0
    assert (n.value, e.value) == (1397, 4)
    assert lib.rl_env_obs_size(ctypes.byref(_cfg(obs_mode=1, obs_stride=28224)), ctypes.byref(n), ctypes.byref(e)) == 0
    assert (n.value, e.value) == (28224, 1)
    offs = (ctypes.c_size_t * 4)()
    assert lib.rl_step_layout(ctypes.byref(_cfg(num_envs=65536)), offs, ctypes.byref(b)) == 0
    assert list(offs) == [0, 262144, 262144 + 65536 * 5588, 262144 + 65536 * 5588 + 262144]
    assert b.value == offs[3] + 262144
    assert lib.rl_env_state_bytes(ctypes.byref(_cfg()), ctypes.byref(n)) == 0 and n.value % 256 == 0


def test_entry_points_reject_before_any_hip_call():
    lib = binding.lib()
    out = ctypes.c_void_p()
    fake = ctypes.c_void_p(4096)
    # rl_env_create: NULL maps, misaligned state, too-small state
    assert lib.rl_env_create(ctypes.byref(_cfg()), None, fake, fake, None, fake, 1 << 30, None, ctypes.byref(out)) == -1
    assert lib.rl_env_create(ctypes.byref(_cfg()), fake, fake, fake, None, ctypes.c_void_p(4100), 1 << 30, None,
                             ctypes.byref(out)) == -2
    assert lib.rl_env_create(ctypes.byref(_cfg()), fake, fake, fake, None, fake, 100, None, ctypes.byref(out)) == -3
    assert lib.rl_env_create(ctypes.byref(_cfg(obs_mode=1, obs_stride=28224)), fake, fake, fake, None, fake, 1 << 30,
                             None, ctypes.byref(out)) == -1
    assert lib.rl_env_step(None, fake, fake, fake, fake, None) == -1
    assert lib.rl_env_step_aim(None, fake, fake, fake, fake, fake, None) == -1
    assert lib.rl_env_set_waypoints(None, fake, fake, None) == -1
    assert lib.rl_env_set_respawn_spots(None, fake, None) == -1
    assert lib.rl_env_read_respawn(None, fake, fake, fake, fake, None) == -1
    assert lib.rl_env_reset(None, None, None, None) == -1
    # rl_gae: sizes, NULLs, enum, workspace
    assert lib.rl_gae(fake, fake, fake, fake, 0, 5, 0.99, 0.95, fake, fake, 0, None, None, 0, None) == -1
    assert lib.rl_gae(None, fake, fake, fake, 4, 5, 0.99, 0.95, fake, fake, 0, None, None, 0, None) == -1
    assert lib.rl_gae(fake, fake, fake, fake, 4, 5, 0.99, 0.95, fake, fake, 4, fake, fake, 1 << 20, None) == -1
    assert lib.rl_gae(fake, fake, fake, fake, 4, 5, 0.99, 0.95, fake, fake, 3, None, None, 0, None) == -1
    assert lib.rl_gae(fake, fake, fake, fake, 4, 5, 0.99, 0.95, fake, fake, 2, fake, None, 0, None) == -1
    assert lib.rl_adv_stats_finish(None, fake, None) == -1
    assert lib.rl_adv_stats_finish(ctypes.c_void_p(4100), fake, None) == -2
    assert lib.rl_gae(fake, fake, fake, fake, 4, 5, 0.99, 0.95, fake, fake, 1, fake, fake, 8, None) == -3
    assert lib.rl_gae(fake, ctypes.c_void_p(4098), fake, fake, 4, 5, 0.99, 0.95, fake, fake, 0, None, None, 0, None) == -2
    # rl_vtrace: sizes, NULLs, clip thresholds, alignment
    assert lib.rl_vtrace(fake, fake, fake, fake, fake, 0, 5, 0.99, 1.0, 1.0, 1.0, 1.0, fake, fake, None) == -1
    assert lib.rl_vtrace(fake, fake, fake, fake, None, 4, 5, 0.99, 1.0, 1.0, 1.0, 1.0, fake, fake, None) == -1
    assert lib.rl_vtrace(fake, fake, fake, fake, fake, 4, 5, 0.99, 1.0, -1.0, 1.0, 1.0, fake, fake, None) == -1
    assert lib.rl_vtrace(fake, fake, fake, fake, ctypes.c_void_p(4098), 4, 5, 0.99, 1.0, 1.0, 1.0, 1.0, fake, fake,
                         None) == -2
    # rl_ppo_loss: B % mb, A range, alignment, workspace
    args = [fake] * 6 + [None, None, None]
    assert lib.rl_ppo_loss(*args, 100, 12, 30, 0.2, 0.5, 0.01, fake, fake, 1 << 20, None) == -1
    assert "multiple" in lib.rl_last_error().decode()
    assert lib.rl_ppo_loss(*args, 100, 65, 10, 0.2, 0.5, 0.01, fake, fake, 1 << 20, None) == -1
    assert lib.rl_ppo_loss(ctypes.c_void_p(4100), *args[1:], 100, 12, 10, 0.2, 0.5, 0.01, fake, fake, 1 << 20,
                           None) == -2
    assert lib.rl_ppo_loss(*args, 100, 12, 10, 0.2, 0.5, 0.01, fake, fake, 8, None) == -3
    both = [fake] * 8 + [None]
    assert lib.rl_ppo_loss(*both, 100, 12, 10, 0.2, 0.5, 0.01, fake, fake, 1 << 20, None) == -1
    assert "not both" in lib.rl_last_error().decode()
    idx = [fake] * 6 + [None, fake, None]
    assert lib.rl_ppo_loss(*idx, 6500, 12, 100, 0.2, 0.5, 0.01, fake, fake, 1 << 30, None) == -1
    assert "at most 64" in lib.rl_last_error().decode()
    # rl_ppo_loss_grad: the gradient buffers are required; dlogits 16-byte aligned when A % 4 == 0
    g = [fake] * 6 + [None, None, None]
    assert lib.rl_ppo_loss_grad(*g, 100, 12, 10, 0.2, 0.5, 0.01, fake, None, fake, fake, 1 << 20, None) == -1
    assert "dlogits" in lib.rl_last_error().decode()
    assert lib.rl_ppo_loss_grad(*g, 100, 12, 10, 0.2, 0.5, 0.01, fake, ctypes.c_void_p(4100), fake, fake, 1 << 20,
                                None) == -2
    assert lib.rl_ppo_loss_grad(*g, 100, 12, 30, 0.2, 0.5, 0.01, fake, fake, fake, fake, 1 << 20, None) == -1
    # the stand-in policy and the rollout driver
    assert lib.rl_policy_weights_bytes(ctypes.byref(need := ctypes.c_size_t())) == 0
    assert need.value == 128 * 1408 * 2 + 13 * 128 * 4
    assert lib.rl_policy_pack(None, fake, fake, None) == -1
    assert lib.rl_policy_pack(fake, fake, ctypes.c_void_p(4096 + 16), None) == -2
    assert lib.rl_policy_forward(None, fake, 10, 1397, 0, 0, 0, fake, fake, fake, None) == -1
    assert lib.rl_policy_forward(fake, fake, 10, 1396, 0, 0, 0, fake, fake, fake, None) == -1
    assert lib.rl_policy_forward(fake, fake, 10, 1397, 0, -1, 0, fake, fake, fake, None) == -1
    assert lib.rl_policy_forward(fake, fake, 10, 1397, 0, 0, (1 << 24) - 5, fake, fake, fake, None) == -1
    assert lib.rl_policy_forward(fake, None, 10, 1397, 0, 0, 0, fake, fake, fake, None) == -1
    assert lib.rl_policy_forward(fake, fake, 0, 1397, 0, 0, 0, None, None, None, None) == 0   # n = 0: nothing
    assert lib.rl_policy_forward(fake, ctypes.c_void_p(4098), 10, 1397, 0, 0, 0, fake, fake, fake, None) == -2
    grp = (binding.RolloutGroup * 2)()
    assert lib.rl_rollout(fake, 0, grp, 0, 0, 1, 1) == -1
    assert lib.rl_rollout(fake, 0, grp, 9, 0, 1, 1) == -1
    assert lib.rl_rollout(fake, 0, grp, 1, 0, 1, 1) == -1          # no env
    assert lib.rl_rollout(fake, 0, grp, 1, -1, 1, 1) == -1
    assert lib.rl_env_get_config(None, None) == -1
    # strided GAE / V-trace: a row stride below the width
    assert lib.rl_gae_strided(fake, fake, fake, fake, 4, 64, 63, 0.99, 0.95, fake, fake, 0, None, None, 0, None) == -1
    assert "row stride" in lib.rl_last_error().decode()
    assert lib.rl_vtrace_strided(fake, fake, fake, fake, fake, 4, 64, 10, 0.99, 1.0, 1.0, 1.0, 1.0, fake, fake,
                                 None) == -1
    assert lib.rl_policy_forward(fake, fake, 10, 1397, 0, 0, 0, ctypes.c_void_p(4098), fake, fake, None) == -2
    assert lib.rl_ppo_loss_workspace_bytes(100, 10, ctypes.byref(need)) == 0 and need.value > 8
    assert lib.rl_gae_workspace_bytes(128, 2048, ctypes.byref(need)) == 0 and need.value >= 16 * 128


def test_waypoint_path_host_bfs_matches_the_oracle():
    # the library's BFS (host C++) and the oracle's, written apart, pick the same unique path
    import numpy as np

    import oracle
    rng = np.random.default_rng(4)
    for trial in range(8):
        g = (rng.random((20, 40)) < 0.3).astype(np.uint8) * rng.integers(1, 4, (20, 40)).astype(np.uint8)
        g[5, 0] = g[14, 39] = 0
        ref = oracle.bfs_path(g, (0, 5), (39, 14))
        if ref is None:
            with pytest.raises(binding.RLError, match="unreachable"):
                binding.waypoint_path(g, (0, 5), (39, 14))
        else:
            np.testing.assert_array_equal(binding.waypoint_path(g, (0, 5), (39, 14)), ref)
    g = np.zeros((3, 3), np.uint8)
    assert binding.waypoint_path(g, (0, 0), (2, 2)).tolist() == [[0, 0], [1, 0], [2, 0], [2, 1], [2, 2]]
    with pytest.raises(binding.RLError, match="max_len"):
        binding.waypoint_path(g, (0, 0), (2, 2), max_len=4)
    g[1, 1] = 1
    with pytest.raises(binding.RLError, match="blocked"):
        binding.waypoint_path(g, (1, 1), (2, 2))


def test_store_probe_rejects_bad_arguments():
    lib = binding.lib()
    buf = ctypes.c_void_p(4096)   # never dereferenced: every call below fails its checks first
    assert lib.rl_store_probe(None, 64, 16, None) == -1
    assert lib.rl_store_probe(ctypes.c_void_p(4100), 64, 16, None) == -2
    assert lib.rl_store_probe(buf, 60, 16, None) == -1
    assert lib.rl_store_probe(buf, 64, 24, None) == -1
    assert lib.rl_store_probe(buf, 0, 16, None) == -1
    assert "multiples of 16" in lib.rl_last_error().decode()


def test_read_probe_rejects_bad_arguments():
    lib = binding.lib()
    buf = ctypes.c_void_p(4096)   # never dereferenced: every call below fails its checks first
    sink = ctypes.c_void_p(8192)
    assert lib.rl_read_probe(None, 64, 16, sink, None) == -1
    assert lib.rl_read_probe(buf, 64, 16, None, None) == -1
    assert lib.rl_read_probe(ctypes.c_void_p(4100), 64, 16, sink, None) == -2
    assert lib.rl_read_probe(buf, 64, 16, ctypes.c_void_p(8194), None) == -2
    assert lib.rl_read_probe(buf, 60, 16, sink, None) == -1
    assert lib.rl_read_probe(buf, 64, 24, sink, None) == -1
    assert "multiples of 16" in lib.rl_last_error().decode()


def test_deferred_statistics_size():
    # a header of 4 doubles, then (sum A, sum A^2) of every scan block: 256 blocks of 256 envs at 65536 x
    # 128, 128 blocks of 16 envs at 2048 x 128, 1 block of 16 envs at one env
    for t, n, blocks in ((128, 65536, 256), (128, 2048, 128), (1, 1, 1)):
        assert binding.gae_stats_bytes(t, n) == 8 * (4 + 2 * blocks)


def test_noalloc_loss_refuses_before_any_device_call():
    # the size checks of rl_ppo_loss_noalloc run before it looks up its device array, so they answer on a
    # machine without a GPU; the pointers are never dereferenced
    lib = binding.lib()
    p = ctypes.c_void_p(4096)
    args = lambda b, mb, perm: (p, p, p, p, p, p, perm, None, None, b, 12, mb, 0.2, 0.5, 0.01, p, None)
    assert lib.rl_ppo_loss_noalloc(*args(1000, 300, None)) == -1                  # B not a multiple of mb
    assert "multiple" in lib.rl_last_error().decode()
    assert lib.rl_ppo_loss_noalloc(*args(1 << 24, 1 << 20, p)) == -3              # 68 MiB with a perm
    assert "fixed device array" in lib.rl_last_error().decode()
    # at 16 minibatches the array admits a perm of up to 15,630,336 samples (the workspace size, a host-only
    # call, says so); one minibatch row more is refused for its size
    big = 15630336
    need = ctypes.c_size_t()
    assert lib.rl_ppo_loss_workspace_bytes(big, big // 16, ctypes.byref(need)) == 0 and need.value <= 64 << 20
    assert lib.rl_ppo_loss_workspace_bytes(big + 16, (big + 16) // 16, ctypes.byref(need)) == 0
    assert need.value > 64 << 20
    assert lib.rl_ppo_loss_noalloc(*args(big + 16, (big + 16) // 16, p)) == -3
