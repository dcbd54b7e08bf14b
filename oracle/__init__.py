"""CPU oracle of the rollout hot path: numpy wrappers over the plain C in ``oracle.c``.

TEST INFRASTRUCTURE, NOT PRODUCT CODE: only the tests, the smoke check and the bench's CPU-baseline leg
import this package. It shares no code with the HIP path and never imports it.

``build()`` compiles ``oracle.c`` with gcc (-O2, no floating-point contraction) into ``liboracle.so``
next to it; the wrappers build it on first use when it is missing. The environment variable
``RL_ORACLE_LIB`` names another build of the same source to load instead (the tests' sanitizer and
planted-mistake builds); it is loaded as it is, never rebuilt.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
GCC_FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared", "-Wall", "-Wextra"]
_lib = None

NF = 24            # canonical state fields per env
RESPAWN_BUF = 64   # outcomes in each map's respawn buffer
STACK = 4
FRAME_DIMS = 15
OBS_TILES = 31 * 43 + STACK * FRAME_DIMS + 4   # 1397
PIX = 84
STATE_FIELDS = ("x", "y", "vx", "vy", "facing", "freeze_ticks", "hook_ticks", "hook_held", "jump_held",
                "grounded", "wall_left", "wall_right", "tick", "next_ckpt", "best_x", "last_action", "path",
                "from_start", "hook_phase", "hook_x", "hook_y", "hook_vx", "hook_vy", "hook_flight")


def build() -> str:
    """Compile the oracle into liboracle.so (always recompiles)."""
    tmp = _LIB_PATH + ".tmp"
    subprocess.check_call(["gcc", *GCC_FLAGS, "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Cfg(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in
                ("num_envs", "env_offset", "num_maps", "map_h", "map_w", "num_ckpts", "frame_skip",
                 "time_limit", "reward_mode", "max_waypoints", "respawn_mode", "hook_mode")]


def _load():
    global _lib
    if _lib is not None:
        return _lib
    override = os.environ.get("RL_ORACLE_LIB")
    if override:
        lib = ctypes.CDLL(override)
    else:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
    p = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    cfgp = ctypes.POINTER(_Cfg)
    lib.oracle_env_reset.argtypes = [cfgp, p, p, p, p]
    lib.oracle_env_step.argtypes = [cfgp, p, p, p, p, p, p, p, p, p, p, ctypes.c_uint64, i64, p,
                                    p, p, p, p, p, p]
    lib.oracle_bfs_path.argtypes = [p, i32, i32, i32, i32, i32, i32, p, i32, p, p]
    lib.oracle_respawn_draw.argtypes = [ctypes.c_uint64, i64, i32, i32]
    lib.oracle_respawn_draw.restype = ctypes.c_uint64
    lib.oracle_env_obs_tiles.argtypes = [cfgp, p, p, p, p, p, i64]
    lib.oracle_env_obs_pixels.argtypes = [cfgp, p, p, p, p]
    lib.oracle_gae.argtypes = [p, p, p, p, i32, i32, f64, f64, p, p]
    lib.oracle_normalize.argtypes = [p, i64, f64, p, p, p]
    lib.oracle_ppo_loss.argtypes = [p, p, p, p, p, p, p, i64, i32, i32, f64, f64, f64, p, p]
    lib.oracle_ppo_loss_grad.argtypes = [p, p, p, p, p, p, p, i64, i32, i32, f64, f64, f64, p, p, p, p, p, p]
    lib.oracle_vtrace.argtypes = [p, p, p, p, p, i32, i32, f64, f64, f64, f64, f64, p, p]
    lib.oracle_policy_forward.argtypes = [p, i64, i64, p, p, ctypes.c_uint64, i64, i64, p, p, p]
    lib.oracle_policy_gumbel.argtypes = [ctypes.c_uint64, i64, i64, i32, p]
    lib.oracle_policy_gumbel.restype = f64
    for fn in (lib.oracle_env_reset, lib.oracle_env_step, lib.oracle_env_obs_tiles,
               lib.oracle_env_obs_pixels, lib.oracle_gae, lib.oracle_normalize, lib.oracle_ppo_loss,
               lib.oracle_ppo_loss_grad, lib.oracle_vtrace, lib.oracle_bfs_path, lib.oracle_policy_forward):
        fn.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


class OracleEnv:
    """A batch of envs held in numpy arrays: canonical state int32[N][NF] and the frame stack
    f32[N][4][15] (newest first)."""

    def __init__(self, maps, ckpts, spawns, num_envs, frame_skip=3, time_limit=2000, sprites=None,
                 env_offset=0, reward_mode=0, waypoints=None, wp_lens=None, respawn_mode=0, ckpt_spawns=None,
                 respawn_seed=0, hook_mode=0):
        self.maps = _c(maps, np.uint8)
        self.ckpts = _c(ckpts, np.int32).reshape(self.maps.shape[0], -1, 2)
        self.spawns = _c(spawns, np.int32).reshape(self.maps.shape[0], 2)
        self.sprites = None if sprites is None else _c(sprites, np.uint8)
        m, h, w = self.maps.shape
        if reward_mode == 1:
            self.waypoints = _c(waypoints, np.int32).reshape(m, -1, 2)
            self.wp_lens = _c(wp_lens, np.int32).reshape(m)
            assert (self.wp_lens >= 1).all() and (self.wp_lens <= self.waypoints.shape[1]).all()
            kw = self.waypoints.shape[1]
        else:
            self.waypoints = self.wp_lens = None
            kw = 0
        self.cfg = _Cfg(num_envs, env_offset, m, h, w, self.ckpts.shape[1], frame_skip, time_limit, reward_mode, kw,
                        respawn_mode, hook_mode)
        # adaptive respawn: each map's outcome ring, fill, write position and frontier; the decision counter
        self.ckpt_spawns = None if ckpt_spawns is None else _c(ckpt_spawns, np.int32).reshape(m, -1, 2)
        assert respawn_mode == 0 or (self.ckpt_spawns is not None and self.ckpts.shape[1] >= 1)
        self.ring = np.zeros((m, RESPAWN_BUF), np.int32)
        self.fill = np.zeros(m, np.int32)
        self.head = np.zeros(m, np.int32)
        self.frontier = np.zeros(m, np.int32)
        self.respawn_seed = int(respawn_seed) & (2 ** 64 - 1)
        self.counter = 0
        self.ended = np.zeros(num_envs, np.int32)
        self.n = num_envs
        self.state = np.zeros((num_envs, NF), np.int32)
        self.stack = np.zeros((num_envs, STACK, FRAME_DIMS), np.float32)
        self._lib = _load()

    def reset(self, mask=None):
        mask = None if mask is None else _c(mask, np.uint8)
        self._lib.oracle_env_reset(ctypes.byref(self.cfg), _ptr(self.spawns), _ptr(mask),
                                   _ptr(self.state), _ptr(self.stack))

    def step(self, actions, aim=None):
        """Advance every env one decision; returns (rewards f32[N], dones f32[N]). aim: hook mode's aim of
        every env, int32[N] packing dx (low 16 bits) and dy (high 16 bits), or None for no aim."""
        actions = _c(actions, np.int32)
        assert actions.shape == (self.n,)
        if aim is not None:
            aim = _c(aim, np.int32)
            assert aim.shape == (self.n,)
        rew = np.empty(self.n, np.float32)
        done = np.empty(self.n, np.float32)
        self._lib.oracle_env_step(ctypes.byref(self.cfg), _ptr(self.maps), _ptr(self.ckpts),
                                  _ptr(self.spawns), _ptr(self.waypoints), _ptr(self.wp_lens),
                                  _ptr(self.ckpt_spawns), _ptr(self.ring), _ptr(self.fill), _ptr(self.head),
                                  _ptr(self.frontier), self.respawn_seed, self.counter, _ptr(self.ended),
                                  _ptr(actions), _ptr(aim), _ptr(self.state), _ptr(self.stack), _ptr(rew),
                                  _ptr(done))
        self.counter += 1
        return rew, done

    def obs_tiles(self, out=None):
        if out is None:
            out = np.empty((self.n, OBS_TILES), np.float32)
        assert out.dtype == np.float32 and out.flags.c_contiguous and out.shape[0] == self.n
        self._lib.oracle_env_obs_tiles(ctypes.byref(self.cfg), _ptr(self.maps), _ptr(self.ckpts),
                                       _ptr(self.state), _ptr(self.stack), _ptr(out), out.shape[1])
        return out

    def obs_pixels(self, out=None):
        assert self.sprites is not None
        if out is None:
            out = np.empty((self.n, STACK, PIX, PIX), np.uint8)
        assert out.dtype == np.uint8 and out.flags.c_contiguous and out.shape[0] == self.n
        self._lib.oracle_env_obs_pixels(ctypes.byref(self.cfg), _ptr(self.maps), _ptr(self.sprites),
                                        _ptr(self.stack), _ptr(out))
        return out


def bfs_path(grid, start, goal, max_len=None):
    """The oracle's BFS tile path over one map grid u8[H][W] from start (col, row) to goal (col, row):
    int32[L][2] of (col, row), or None when unreachable / blocked. Raises if longer than max_len."""
    g = _c(grid, np.uint8)
    h, w = g.shape
    max_len = h * w if max_len is None else max_len
    path = np.empty((max_len, 2), np.int32)
    n = ctypes.c_int32()
    scratch = np.empty(2 * h * w, np.int32)
    rc = _load().oracle_bfs_path(_ptr(g), h, w, int(start[0]), int(start[1]), int(goal[0]), int(goal[1]),
                                 _ptr(path), max_len, ctypes.byref(n), _ptr(scratch))
    if rc == -1:
        return None
    if rc == -3:
        raise ValueError("path longer than max_len")
    return path[:n.value].copy()


def gae(rewards, values, dones, last_values, gamma, lam):
    """GAE by its definition sum, float64. Returns (adv, ret) float64[T][N]."""
    r, v, d = (_c(a, np.float32) for a in (rewards, values, dones))
    vl = _c(last_values, np.float32)
    t, n = r.shape
    adv = np.empty((t, n), np.float64)
    ret = np.empty((t, n), np.float64)
    _load().oracle_gae(_ptr(r), _ptr(v), _ptr(d), _ptr(vl), t, n, float(gamma), float(lam),
                       _ptr(adv), _ptr(ret))
    return adv, ret


def normalize(adv, eps=1e-8):
    """Whole-batch advantage normalisation, float64. Returns (normalised, mean, std)."""
    a = _c(adv, np.float64)
    out = np.empty_like(a)
    mean = ctypes.c_double()
    std = ctypes.c_double()
    _load().oracle_normalize(_ptr(a), a.size, float(eps), _ptr(out), ctypes.byref(mean), ctypes.byref(std))
    return out, mean.value, std.value


def ppo_loss(logits, actions, old_logp, adv, ret, new_values, perm, minibatch, clip_eps=0.2,
             vf_coef=0.5, ent_coef=0.01):
    """Per-minibatch PPO loss scalars, float64. Returns (out[num_mb][4], scale[num_mb][4]) with columns
    (pg, value, entropy, total)."""
    lg = _c(logits, np.float64)
    b, a = lg.shape
    act = _c(actions, np.int32).reshape(b)
    olp = _c(old_logp, np.float64).reshape(b)
    ad = _c(adv, np.float64).reshape(b)
    rt = _c(ret, np.float64).reshape(b)
    nv = _c(new_values, np.float64).reshape(b)
    pm = None if perm is None else _c(perm, np.int32).reshape(b)
    assert b % minibatch == 0
    nmb = b // minibatch
    out = np.empty((nmb, 4), np.float64)
    scale = np.empty((nmb, 4), np.float64)
    _load().oracle_ppo_loss(_ptr(lg), _ptr(act), _ptr(olp), _ptr(ad), _ptr(rt), _ptr(nv), _ptr(pm), b, a,
                            minibatch, float(clip_eps), float(vf_coef), float(ent_coef), _ptr(out), _ptr(scale))
    return out, scale


class LossGrad:
    """Per-sample gradient of each minibatch's total loss, float64, in storage order, with the tests'
    extras (see oracle_ppo_loss_grad)."""

    def __init__(self, dlogits, dvalues, gscale, vscale, dpg, ratio):
        self.dlogits, self.dvalues, self.gscale, self.vscale, self.dpg, self.ratio = (
            dlogits, dvalues, gscale, vscale, dpg, ratio)


def ppo_loss_grad(logits, actions, old_logp, adv, ret, new_values, perm, minibatch, clip_eps=0.2,
                  vf_coef=0.5, ent_coef=0.01):
    """dL_m/dlogits [B][A] and dL_m/dV [B] for the minibatch m that holds each sample."""
    lg = _c(logits, np.float64)
    b, a = lg.shape
    act = _c(actions, np.int32).reshape(b)
    olp = _c(old_logp, np.float64).reshape(b)
    ad = _c(adv, np.float64).reshape(b)
    rt = _c(ret, np.float64).reshape(b)
    nv = _c(new_values, np.float64).reshape(b)
    pm = None if perm is None else _c(perm, np.int32).reshape(b)
    assert b % minibatch == 0
    g = LossGrad(np.empty((b, a)), np.empty(b), np.empty((b, a)), np.empty(b), np.empty((b, a)), np.empty(b))
    _load().oracle_ppo_loss_grad(_ptr(lg), _ptr(act), _ptr(olp), _ptr(ad), _ptr(rt), _ptr(nv), _ptr(pm), b, a,
                                 minibatch, float(clip_eps), float(vf_coef), float(ent_coef), _ptr(g.dlogits),
                                 _ptr(g.dvalues), _ptr(g.gscale), _ptr(g.vscale), _ptr(g.dpg), _ptr(g.ratio))
    return g


def vtrace(rewards, values, dones, last_values, log_rhos, gamma, lam=1.0, rho_bar=1.0, c_bar=1.0,
           pg_rho_bar=1.0):
    """V-trace targets vs[T][N] and policy-gradient advantages pg[T][N], float64, by the definition sum."""
    r = _c(rewards, np.float32)
    t, n = r.shape
    v = _c(values, np.float32)
    d = _c(dones, np.float32)
    lv = _c(last_values, np.float32).reshape(n)
    lr = _c(log_rhos, np.float32)
    vs = np.empty((t, n), np.float64)
    pg = np.empty((t, n), np.float64)
    _load().oracle_vtrace(_ptr(r), _ptr(v), _ptr(d), _ptr(lv), _ptr(lr), t, n, float(gamma), float(lam),
                          float(rho_bar), float(c_bar), float(pg_rho_bar), _ptr(vs), _ptr(pg))
    return vs, pg


def respawn_draw(seed, counter, n, i):
    """The oracle's i-th respawn draw of global env n at decision `counter` (uint64)."""
    return int(_load().oracle_respawn_draw(int(seed) & (2 ** 64 - 1), int(counter), int(n), int(i)))


POLICY_HIDDEN = 128
POLICY_ACTIONS = 12


def policy_forward(obs, enc_w, dec_w, seed, t, env_offset=0):
    """The stand-in policy's inference for rows of obs (float32 [n][>= 1397]): returns (out float64
    [n][13] = 12 logits then the value, actions int32 [n], logp float64 [n])."""
    lib = _load()
    obs = _c(obs, np.float32)
    n, stride = obs.shape
    enc_w = _c(enc_w, np.float32).reshape(POLICY_HIDDEN, OBS_TILES)
    dec_w = _c(dec_w, np.float32).reshape(POLICY_ACTIONS + 1, POLICY_HIDDEN)
    out = np.empty((n, POLICY_ACTIONS + 1), np.float64)
    actions = np.empty(n, np.int32)
    logp = np.empty(n, np.float64)
    rc = lib.oracle_policy_forward(_ptr(obs), n, stride, _ptr(enc_w), _ptr(dec_w), int(seed) & ((1 << 64) - 1),
                                   int(t), int(env_offset), _ptr(out), _ptr(actions), _ptr(logp))
    if rc != 0:
        raise ValueError("oracle_policy_forward rejected its arguments")
    return out, actions, logp


def policy_gumbel(seed, t, n, j):
    """(g, u): the Gumbel variate of global env n, decision t, logit j, and its uniform draw."""
    u = ctypes.c_double()
    g = _load().oracle_policy_gumbel(int(seed) & ((1 << 64) - 1), int(t), int(n), int(j), ctypes.byref(u))
    return g, u.value
