"""Shared helpers of the GPU parity tests: tolerance checks and paired GPU / oracle env batches."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from resident_rl_rollout_amd import binding, inputs


def assert_gae_close(got, ref, what, rel=1e-5):
    """|g - o| <= rel * (|o| + rms(o)) per element: the scale floor keeps the bound meaningful for
    values near zero (normalised advantages have mean 0)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    err = np.abs(got - ref)
    bound = rel * (np.abs(ref) + rms)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; worst at {i}: "
                             f"got {got[i]!r} want {ref[i]!r} (bound {bound[i]:.3g})")


def assert_loss_close(got, ref, scale, what, rel=1e-4):
    """|g - o| <= rel * (|o| + mean |summand|) per minibatch scalar."""
    got = np.asarray(got, np.float64)
    bound = rel * (np.abs(ref) + scale)
    err = np.abs(got - ref)
    assert (err <= bound).all(), f"{what}: err {err[err > bound]} bound {bound[err > bound]}"


def assert_grad_close(dlogits, dvalues, g, adv, what, rel=1e-4, clip_eps=0.2, edge_rel=1e-5):
    """Loss-gradient parity against the oracle's LossGrad g: per element |got - want| <= rel * (|want| +
    summand magnitudes). Where float rounding decides which side of the min a sample takes (its ratio
    within edge_rel of the band edge that applies to its advantage's sign), the row may match either
    side: the oracle's row, or that row with the surrogate's part switched."""
    dl = np.asarray(dlogits, np.float64)
    dv = np.asarray(dvalues, np.float64)
    assert dl.shape == g.dlogits.shape and dv.shape == g.dvalues.shape, what
    bound = rel * (np.abs(g.dlogits) + g.gscale)
    ok = (np.abs(dl - g.dlogits) <= bound).all(axis=1)
    edge = np.where(np.asarray(adv) >= 0, 1.0 + clip_eps, 1.0 - clip_eps)
    ambiguous = np.abs(g.ratio - edge) <= edge_rel * edge
    if (~ok & ambiguous).any():
        rows = np.nonzero(~ok & ambiguous)[0]
        # the other side of the min: remove the surrogate part if the oracle kept it, add it otherwise
        sides = [g.dlogits[rows] - g.dpg[rows], g.dlogits[rows] + g.dpg[rows]]
        alt_ok = np.zeros(rows.size, bool)
        for alt in sides:
            alt_ok |= (np.abs(dl[rows] - alt) <= rel * (np.abs(alt) + g.gscale[rows])).all(axis=1)
        ok[rows] = alt_ok
    if not ok.all():
        i = int(np.nonzero(~ok)[0][0])
        j = int(np.argmax(np.abs(dl[i] - g.dlogits[i]) - bound[i]))
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} gradient rows outside tolerance; first "
                             f"sample {i} logit {j}: got {dl[i, j]!r} want {g.dlogits[i, j]!r} "
                             f"(bound {bound[i, j]:.3g}, ratio {g.ratio[i]!r})")
    vbound = rel * (np.abs(g.dvalues) + g.vscale)
    verr = np.abs(dv - g.dvalues)
    if (verr > vbound).any():
        i = int(np.argmax(verr - vbound))
        raise AssertionError(f"{what}: value gradient of sample {i}: got {dv[i]!r} want {g.dvalues[i]!r}")
    return int(ambiguous.sum())


def path_goal(grid, col, row):
    """The finish tile, or the nearest tile above it in its column that a box can pass (a platform may
    cover the finish checkpoint's tile; the finish itself is reached by column)."""
    while row > 0 and grid[row, col] in (1, 2):
        row -= 1
    return col, row


def waypoint_table(ms: inputs.MapSet):
    """Each map's BFS tile path (the oracle's) from the spawn's box-centre tile to its finish tile (see
    path_goal), padded to the longest: (int32[M][KW][2], int32[M])."""
    paths = []
    for m in range(ms.maps.shape[0]):
        x, y = ms.spawns[m]
        start = ((int(x) + 96) >> 8, (int(y) + 96) >> 8)
        goal = path_goal(ms.maps[m], int(ms.ckpts[m, -1, 0]), int(ms.ckpts[m, -1, 1]))
        p = oracle.bfs_path(ms.maps[m], start, goal)
        assert p is not None, f"map {m}: finish unreachable"
        paths.append(p)
    kw = max(len(p) for p in paths)
    table = np.zeros((len(paths), kw, 2), np.int32)
    for m, p in enumerate(paths):
        table[m, :len(p)] = p
        table[m, len(p):] = p[-1]
    return table, np.array([len(p) for p in paths], np.int32)


def poison(obs, rew, done, obs_mode, step):
    """Fill a step's outputs with values no step writes, so that every element a parity check compares
    must have been written by that step: NaN for float observations, rewards and dones; for u8 pixels
    (where every byte value can occur) a byte that changes with the step, so a skipped store leaves the
    previous step's poison, which differs. Padding past the observation is left alone (no step may write
    it)."""
    size = binding.OBS_TILES_SIZE if obs_mode == binding.OBS_TILES else binding.OBS_PIXELS_SIZE
    if obs_mode == binding.OBS_TILES:
        obs[..., :size].fill_(float("nan"))
    else:
        obs[..., :size].fill_((37 * step + 11) & 0xFF)
    rew.fill_(float("nan"))
    done.fill_(float("nan"))


class SubsetPairs:
    """One GPU env batch of n envs beside oracle batches of stated env ranges (env_offset keys each
    range's maps and draws as global envs), for the full-size workloads the oracle cannot step whole."""

    def __init__(self, gpu_env, ms, ranges, **oracle_kw):
        self.gpu = gpu_env
        self.ranges = ranges
        self.oras = [oracle.OracleEnv(ms.maps, ms.ckpts, ms.spawns, hi - lo, env_offset=lo, **oracle_kw)
                     for lo, hi in ranges]
        for o in self.oras:
            o.reset()
        self.sel_np = np.concatenate([np.arange(lo, hi) for lo, hi in ranges])
        self.sel = torch.from_numpy(self.sel_np).cuda()

    def step(self, actions_np):
        outs = [o.step(actions_np[lo:hi]) for o, (lo, hi) in zip(self.oras, self.ranges)]
        return np.concatenate([r for r, _ in outs]), np.concatenate([d for _, d in outs])

    def check_state(self, what):
        got = self.gpu.read_state()[self.sel].cpu().numpy()
        want = np.concatenate([o.state for o in self.oras])
        if not np.array_equal(got, want):
            e, f = np.argwhere(got != want)[0]
            raise AssertionError(f"{what}: state of env {self.sel_np[e]} field {oracle.STATE_FIELDS[f]}: gpu "
                                 f"{got[e]} oracle {want[e]}")

    def check_obs(self, obs, what):
        got = obs[self.sel].cpu().numpy()
        if self.gpu.obs_mode == binding.OBS_TILES:
            want = np.concatenate([o.obs_tiles() for o in self.oras])
            got = got[:, :binding.OBS_TILES_SIZE]
        else:
            want = np.concatenate([o.obs_pixels().reshape(len(o.state), -1) for o in self.oras])
            got = got[:, :binding.OBS_PIXELS_SIZE]
        if not np.array_equal(got.view(np.uint8), want.view(np.uint8)):
            bad = np.argwhere(got != want)
            raise AssertionError(f"{what}: obs differ at {len(bad)} elements, first (row in the subset, element) "
                                 f"{bad[:5].tolist()}")


class PairedEnvs:
    """The same env batch on the GPU (through the C ABI) and in the oracle, stepped with the same actions."""

    def __init__(self, ms: inputs.MapSet, n, *, frame_skip=3, time_limit=2000, obs_mode=binding.OBS_TILES,
                 sprites=None, obs_stride=None, reward_mode=0, waypoints=None, wp_lens=None, respawn_mode=0,
                 respawn_seed=0, hook_mode=0):
        spots = ms.ckpt_spawns if respawn_mode else None
        self.gpu = binding.Env(ms.maps, ms.ckpts, ms.spawns, n, frame_skip=frame_skip, time_limit=time_limit,
                               obs_mode=obs_mode, sprites=sprites, obs_stride=obs_stride, reward_mode=reward_mode,
                               waypoints=waypoints, wp_lens=wp_lens, respawn_mode=respawn_mode, ckpt_spawns=spots,
                               respawn_seed=respawn_seed, hook_mode=hook_mode)
        self.ora = oracle.OracleEnv(ms.maps, ms.ckpts, ms.spawns, n, frame_skip=frame_skip,
                                    time_limit=time_limit, sprites=sprites, reward_mode=reward_mode,
                                    waypoints=waypoints, wp_lens=wp_lens, respawn_mode=respawn_mode,
                                    ckpt_spawns=spots, respawn_seed=respawn_seed, hook_mode=hook_mode)
        self.ora.reset()
        self.n = n
        self.obs_mode = obs_mode
        self.obs = self.gpu.new_obs()
        self.rew = torch.empty(n, dtype=torch.float32, device="cuda")
        self.done = torch.empty(n, dtype=torch.float32, device="cuda")
        self.gpu.reset(self.obs)

    def oracle_obs(self):
        if self.obs_mode == binding.OBS_TILES:
            return self.ora.obs_tiles()
        return self.ora.obs_pixels().reshape(self.n, -1)

    def gpu_obs(self):
        size = binding.OBS_TILES_SIZE if self.obs_mode == binding.OBS_TILES else binding.OBS_PIXELS_SIZE
        return self.obs[:, :size].cpu().numpy()

    def step(self, actions_np, aim_np=None):
        a = torch.from_numpy(np.ascontiguousarray(actions_np, np.int32)).cuda()
        aim = None if aim_np is None else torch.from_numpy(np.ascontiguousarray(aim_np, np.int32)).cuda()
        self.steps = getattr(self, "steps", 0) + 1
        poison(self.obs, self.rew, self.done, self.obs_mode, self.steps)
        self.gpu.step(a, self.obs, self.rew, self.done, aim=aim)
        r, d = self.ora.step(actions_np, aim_np)
        return r, d

    def check_state(self, what):
        got = self.gpu.read_state().cpu().numpy()
        if not np.array_equal(got, self.ora.state):
            bad = np.argwhere(got != self.ora.state)
            e, f = bad[0]
            raise AssertionError(f"{what}: state differs in {len(bad)} fields; first env {e} field "
                                 f"{oracle.STATE_FIELDS[f]}: gpu {got[e]} oracle {self.ora.state[e]}")

    def check_respawn(self, what):
        ring, fill, head, front = (t.cpu().numpy() for t in self.gpu.read_respawn())
        np.testing.assert_array_equal(fill, self.ora.fill, err_msg=f"{what}: respawn fill")
        np.testing.assert_array_equal(head, self.ora.head, err_msg=f"{what}: respawn head")
        np.testing.assert_array_equal(front, self.ora.frontier, err_msg=f"{what}: respawn frontier")
        for m in range(len(fill)):
            np.testing.assert_array_equal(ring[m, :fill[m]], self.ora.ring[m, :fill[m]],
                                          err_msg=f"{what}: respawn ring of map {m}")

    def check_step(self, r, d, what):
        np.testing.assert_array_equal(self.rew.cpu().numpy(), r, err_msg=f"{what}: rewards")
        np.testing.assert_array_equal(self.done.cpu().numpy(), d, err_msg=f"{what}: dones")

    def check_obs(self, what, envs=None):
        got = self.gpu_obs()
        ref = self.oracle_obs()
        if envs is not None:
            got, ref = got[envs], ref[envs]
        if not np.array_equal(got.view(np.uint8), ref.view(np.uint8)):
            bad = np.argwhere(got != ref)
            raise AssertionError(f"{what}: obs differ at {len(bad)} elements, first {bad[:5].tolist()}")
