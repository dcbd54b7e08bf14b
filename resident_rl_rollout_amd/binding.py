"""Python binding of librl.so: argument marshalling only.

Every function here forwards to the C ABI declared in include/rl.h with the same name. PyTorch is used
only to own device memory (tensors) and to name the stream (the current HIP stream); every step of the
rollout path runs in the library's HIP kernels. If librl.so is missing the binding raises: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librl.so")

OBS_TILES, OBS_PIXELS = 0, 1
STATE_FIELDS = 24
REWARD_CHECKPOINTS, REWARD_WAYPOINTS = 0, 1
RESPAWN_OFF, RESPAWN_ADAPTIVE = 0, 1
HOOK_OFF, HOOK_GRAPPLE = 0, 1
RESPAWN_BUF = 64
OBS_TILES_SIZE = 1397
OBS_PIXELS_SIZE = 28224

_lib = None


class RLError(RuntimeError):
    """A non-zero status from the library, with its rl_last_error() text."""


class EnvConfig(ctypes.Structure):
    _fields_ = [("num_envs", ctypes.c_int32), ("num_maps", ctypes.c_int32), ("map_h", ctypes.c_int32),
                ("map_w", ctypes.c_int32), ("num_ckpts", ctypes.c_int32), ("frame_skip", ctypes.c_int32),
                ("time_limit", ctypes.c_int32), ("obs_mode", ctypes.c_int32), ("obs_stride", ctypes.c_int64),
                ("reward_mode", ctypes.c_int32), ("max_waypoints", ctypes.c_int32),
                ("respawn_mode", ctypes.c_int32), ("respawn_seed", ctypes.c_uint64), ("hook_mode", ctypes.c_int32)]


POLICY_HIDDEN, POLICY_ACTIONS = 128, 12
ROLLOUT_MAX_GROUPS = 8


class RolloutGroup(ctypes.Structure):
    _fields_ = [("env", ctypes.c_void_p), ("obs0", ctypes.c_void_p), ("obs", ctypes.c_void_p),
                ("actions", ctypes.c_void_p), ("logp", ctypes.c_void_p), ("values", ctypes.c_void_p),
                ("rewards", ctypes.c_void_p), ("dones", ctypes.c_void_p), ("row", ctypes.c_int64),
                ("obs_row", ctypes.c_int64), ("env_offset", ctypes.c_int64), ("stream", ctypes.c_void_p)]


# (name, restype, argtypes) of every symbol include/rl.h declares.
_P, _I32, _I64, _F32, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_CFG = ctypes.POINTER(EnvConfig)
SIGNATURES = [
    ("rl_env_state_bytes", ctypes.c_int, [_CFG, ctypes.POINTER(_SZ)]),
    ("rl_env_obs_size", ctypes.c_int, [_CFG, ctypes.POINTER(_SZ), ctypes.POINTER(_SZ)]),
    ("rl_step_layout", ctypes.c_int, [_CFG, ctypes.POINTER(_SZ), ctypes.POINTER(_SZ)]),
    ("rl_env_create", ctypes.c_int, [_CFG, _P, _P, _P, _P, _P, _SZ, _P, ctypes.POINTER(_P)]),
    ("rl_env_reset", ctypes.c_int, [_P, _P, _P, _P]),
    ("rl_env_set_waypoints", ctypes.c_int, [_P, _P, _P, _P]),
    ("rl_env_set_respawn_spots", ctypes.c_int, [_P, _P, _P]),
    ("rl_env_read_respawn", ctypes.c_int, [_P, _P, _P, _P, _P, _P]),
    ("rl_waypoint_path", ctypes.c_int, [_P, _I32, _I32, _I32, _I32, _I32, _I32, _P, _I32, ctypes.POINTER(_I32)]),
    ("rl_env_step", ctypes.c_int, [_P, _P, _P, _P, _P, _P]),
    ("rl_env_step_aim", ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P]),
    ("rl_env_read_state", ctypes.c_int, [_P, _P, _P]),
    ("rl_env_get_step_counter", ctypes.c_int, [_P, ctypes.POINTER(_I64)]),
    ("rl_env_set_step_counter", ctypes.c_int, [_P, _I64]),
    ("rl_env_read_step_counter", ctypes.c_int, [_P, _P, _P]),
    ("rl_env_get_config", ctypes.c_int, [_P, _CFG]),
    ("rl_env_destroy", None, [_P]),
    ("rl_gae_workspace_bytes", ctypes.c_int, [_I32, _I32, ctypes.POINTER(_SZ)]),
    ("rl_gae_stats_bytes", ctypes.c_int, [_I32, _I32, ctypes.POINTER(_SZ)]),
    ("rl_adv_stats_finish", ctypes.c_int, [_P, _P, _P]),
    ("rl_gae", ctypes.c_int, [_P, _P, _P, _P, _I32, _I32, _F32, _F32, _P, _P, _I32, _P, _P, _SZ, _P]),
    ("rl_vtrace", ctypes.c_int, [_P, _P, _P, _P, _P, _I32, _I32, _F32, _F32, _F32, _F32, _F32, _P, _P, _P]),
    ("rl_gae_strided", ctypes.c_int, [_P, _P, _P, _P, _I32, _I32, _I64, _F32, _F32, _P, _P, _I32, _P, _P, _SZ, _P]),
    ("rl_vtrace_strided", ctypes.c_int, [_P, _P, _P, _P, _P, _I32, _I32, _I64, _F32, _F32, _F32, _F32, _F32, _P, _P,
                                         _P]),
    ("rl_ppo_loss_workspace_bytes", ctypes.c_int, [_I64, _I32, ctypes.POINTER(_SZ)]),
    ("rl_ppo_loss", ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I32, _I32, _F32, _F32, _F32, _P,
                                   _P, _SZ, _P]),
    ("rl_ppo_loss_noalloc", ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I32, _I32, _F32, _F32, _F32,
                                           _P, _P]),
    ("rl_ppo_loss_grad", ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I32, _I32, _F32, _F32, _F32,
                                        _P, _P, _P, _P, _SZ, _P]),
    ("rl_policy_weights_bytes", ctypes.c_int, [ctypes.POINTER(_SZ)]),
    ("rl_policy_pack", ctypes.c_int, [_P, _P, _P, _P]),
    ("rl_policy_forward", ctypes.c_int, [_P, _P, _I64, _I64, ctypes.c_uint64, _I64, _I64, _P, _P, _P, _P]),
    ("rl_rollout", ctypes.c_int, [_P, ctypes.c_uint64, ctypes.POINTER(RolloutGroup), _I32, _I32, _I32, _I32]),
    ("rl_store_probe", ctypes.c_int, [_P, _I64, _I64, _P]),
    ("rl_read_probe", ctypes.c_int, [_P, _I64, _I64, _P, _P]),
    ("rl_last_error", ctypes.c_char_p, []),
]


def lib():
    """The loaded library with every signature declared; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m resident_rl_rollout_amd.build` "
                           "(there is no non-HIP fallback)")
    handle = ctypes.CDLL(LIB_PATH)
    for name, res, args in SIGNATURES:
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    _lib = handle
    return handle


def check(rc: int) -> None:
    if rc != 0:
        raise RLError(f"status {rc}: {lib().rl_last_error().decode()}")


def stream_ptr(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def dptr(t, dtype=None, what="tensor"):
    """Device pointer of a contiguous CUDA tensor (None passes through as NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{what} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{what} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _dev(x, dtype, device):
    if isinstance(x, np.ndarray):
        x = torch.from_numpy(np.ascontiguousarray(x))
    return x.to(device=device, dtype=dtype).contiguous()


_workspaces: dict = {}


def workspace(kind: str, nbytes: int, device, stream=None) -> torch.Tensor:
    """A device workspace per (kind, size, device, stream), reused by every call of that kind on that
    stream: calls on one stream run in order, so they never overlap, while calls on two streams get two
    workspaces."""
    key = (kind, int(nbytes), str(device), stream_ptr(stream).value)
    ws = _workspaces.get(key)
    if ws is None:
        ws = torch.zeros(max(int(nbytes), 8), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


class Env:
    """A batch of platformer envs over a device state buffer owned by this object."""

    def __init__(self, maps, ckpts, spawns, num_envs, *, frame_skip=3, time_limit=2000, obs_mode=OBS_TILES,
                 sprites=None, obs_stride=None, device="cuda", stream=None, reward_mode=REWARD_CHECKPOINTS,
                 waypoints=None, wp_lens=None, respawn_mode=RESPAWN_OFF, ckpt_spawns=None, respawn_seed=0,
                 hook_mode=HOOK_OFF):
        """reward_mode REWARD_WAYPOINTS needs waypoints int32[M][KW][2] and wp_lens int32[M] (copied to the
        device and set on the env after creation). hook_mode HOOK_GRAPPLE takes aims in step()."""
        L = lib()
        self.device = torch.device(device)
        self.maps = _dev(maps, torch.uint8, self.device)
        m, h, w = self.maps.shape
        ck = _dev(ckpts, torch.int32, self.device).reshape(m, -1, 2)
        self.ckpts = ck
        self.spawns = _dev(spawns, torch.int32, self.device).reshape(m, 2)
        self.sprites = None if sprites is None else _dev(sprites, torch.uint8, self.device).reshape(16, 8, 8)
        self.obs_mode = obs_mode
        size = OBS_TILES_SIZE if obs_mode == OBS_TILES else OBS_PIXELS_SIZE
        self.obs_stride = size if obs_stride is None else int(obs_stride)
        kw = 0
        if reward_mode == REWARD_WAYPOINTS:
            wpt = _dev(waypoints, torch.int32, self.device).reshape(m, -1, 2)
            kw = wpt.shape[1]
        self.cfg = EnvConfig(num_envs, m, h, w, ck.shape[1], frame_skip, time_limit, obs_mode, self.obs_stride,
                             reward_mode, kw, respawn_mode, int(respawn_seed) & (2 ** 64 - 1), hook_mode)
        nbytes = ctypes.c_size_t()
        check(L.rl_env_state_bytes(ctypes.byref(self.cfg), ctypes.byref(nbytes)))
        self.state = torch.empty(nbytes.value, dtype=torch.uint8, device=self.device)
        self.num_envs = num_envs
        self._handle = ctypes.c_void_p()
        check(L.rl_env_create(ctypes.byref(self.cfg), dptr(self.maps), dptr(self.ckpts) if ck.numel() else None,
                              dptr(self.spawns), dptr(self.sprites), dptr(self.state), nbytes.value,
                              stream_ptr(stream), ctypes.byref(self._handle)))
        if reward_mode == REWARD_WAYPOINTS:
            self.set_waypoints(wpt, wp_lens, stream)
        self.respawn_mode = respawn_mode
        if respawn_mode == RESPAWN_ADAPTIVE:
            self.ckpt_spawns = _dev(ckpt_spawns, torch.int32, self.device).reshape(m, -1, 2)
            check(L.rl_env_set_respawn_spots(self._handle, dptr(self.ckpt_spawns), stream_ptr(stream)))

    def set_waypoints(self, waypoints, wp_lens, stream=None):
        """rl_env_set_waypoints: each map's path table int32[M][max_waypoints][2] (the width the env was
        created with) and its lengths int32[M]; may be called again between steps."""
        m = self.maps.shape[0]
        wpt = _dev(waypoints, torch.int32, self.device).reshape(m, -1, 2)
        if wpt.shape[1] != self.cfg.max_waypoints:
            raise ValueError(f"waypoint table has {wpt.shape[1]} entries per map, the env {self.cfg.max_waypoints}")
        self.waypoints = wpt
        self.wp_lens = _dev(wp_lens, torch.int32, self.device).reshape(m)
        check(lib().rl_env_set_waypoints(self._handle, dptr(self.waypoints), dptr(self.wp_lens), stream_ptr(stream)))

    @property
    def obs_dtype(self):
        return torch.float32 if self.obs_mode == OBS_TILES else torch.uint8

    def new_obs(self, steps=None):
        shape = (self.num_envs, self.obs_stride) if steps is None else (steps, self.num_envs, self.obs_stride)
        return torch.empty(shape, dtype=self.obs_dtype, device=self.device)

    def reset(self, obs=None, mask=None, stream=None):
        check(lib().rl_env_reset(self._handle, dptr(mask, torch.uint8, "mask"), dptr(obs, self.obs_dtype, "obs"),
                                 stream_ptr(stream)))

    def step(self, actions, obs, rewards, dones, stream=None, aim=None):
        """rl_env_step, or rl_env_step_aim when aim (device int32[N], dx | dy << 16) is given."""
        if aim is None:
            check(lib().rl_env_step(self._handle, dptr(actions, torch.int32, "actions"),
                                    dptr(obs, self.obs_dtype, "obs"), dptr(rewards, torch.float32, "rewards"),
                                    dptr(dones, torch.float32, "dones"), stream_ptr(stream)))
        else:
            check(lib().rl_env_step_aim(self._handle, dptr(actions, torch.int32, "actions"),
                                        dptr(aim, torch.int32, "aim"), dptr(obs, self.obs_dtype, "obs"),
                                        dptr(rewards, torch.float32, "rewards"), dptr(dones, torch.float32, "dones"),
                                        stream_ptr(stream)))

    def read_state(self, stream=None):
        out = torch.empty((self.num_envs, STATE_FIELDS), dtype=torch.int32, device=self.device)
        check(lib().rl_env_read_state(self._handle, dptr(out), stream_ptr(stream)))
        return out

    def read_respawn(self, stream=None):
        """(ring int32[M][64], fill, head, frontier int32[M]) of the adaptive respawn."""
        m = self.maps.shape[0]
        ring = torch.empty((m, RESPAWN_BUF), dtype=torch.int32, device=self.device)
        meta = torch.empty((3, m), dtype=torch.int32, device=self.device)
        check(lib().rl_env_read_respawn(self._handle, dptr(ring), dptr(meta[0]), dptr(meta[1]), dptr(meta[2]),
                                        stream_ptr(stream)))
        return ring, meta[0], meta[1], meta[2]

    @property
    def step_counter(self) -> int:
        c = ctypes.c_int64()
        check(lib().rl_env_get_step_counter(self._handle, ctypes.byref(c)))
        return c.value

    @step_counter.setter
    def step_counter(self, value: int):
        check(lib().rl_env_set_step_counter(self._handle, int(value)))

    def read_step_counter(self, stream=None):
        """The device decision counter (advanced by every step launch, graph replays included)."""
        out = torch.empty(1, dtype=torch.int64, device=self.device)
        check(lib().rl_env_read_step_counter(self._handle, dptr(out), stream_ptr(stream)))
        return out

    def step_layout(self):
        offs = (ctypes.c_size_t * 4)()
        total = ctypes.c_size_t()
        check(lib().rl_step_layout(ctypes.byref(self.cfg), offs, ctypes.byref(total)))
        return list(offs), total.value

    def close(self):
        if getattr(self, "_handle", None) is not None and self._handle.value:
            lib().rl_env_destroy(self._handle)
            self._handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def waypoint_path(grid, start, goal, max_len=None):
    """rl_waypoint_path on one host map grid u8[H][W]: the BFS tile path from start (col, row) to goal
    (col, row) as int32[L][2] (col, row) pairs."""
    import numpy as np
    g = np.ascontiguousarray(grid, np.uint8)
    h, w = g.shape
    max_len = h * w if max_len is None else int(max_len)
    out = np.empty((max_len, 2), np.int32)
    n = ctypes.c_int32()
    check(lib().rl_waypoint_path(g.ctypes.data_as(_P), h, w, int(start[0]), int(start[1]), int(goal[0]),
                                 int(goal[1]), out.ctypes.data_as(_P), max_len, ctypes.byref(n)))
    return out[:n.value].copy()


def gae_workspace_bytes(t: int, n: int) -> int:
    b = ctypes.c_size_t()
    check(lib().rl_gae_workspace_bytes(t, n, ctypes.byref(b)))
    return b.value


def _rows(x, what, ld=None):
    """Address and row stride of a [T][N] float32 device view whose rows are contiguous; every such
    argument of one call must share the row stride."""
    if not isinstance(x, torch.Tensor) or not x.is_cuda or x.dtype != torch.float32 or x.dim() != 2:
        raise TypeError(f"{what} must be a 2-D float32 device tensor")
    if x.stride(1) != 1 or (x.shape[0] > 1 and x.stride(0) < x.shape[1]):
        raise ValueError(f"{what}: rows must be contiguous")
    stride = x.stride(0) if x.shape[0] > 1 else (ld if ld is not None else x.shape[1])
    if ld is not None and stride != ld:
        raise ValueError(f"{what}: row stride {stride} differs from the other arrays' {ld}")
    return ctypes.c_void_p(x.data_ptr()), stride


def gae_stats_bytes(t: int, n: int) -> int:
    b = ctypes.c_size_t()
    check(lib().rl_gae_stats_bytes(t, n, ctypes.byref(b)))
    return b.value


def adv_stats_finish(adv_stats, out=None, stream=None):
    """rl_adv_stats_finish: {count, mean, std} (float64[3] device tensor) of an adv_stats buffer in either
    form."""
    out = torch.empty(3, dtype=torch.float64, device=adv_stats.device) if out is None else out
    check(lib().rl_adv_stats_finish(dptr(adv_stats, torch.float64, "adv_stats"), dptr(out, torch.float64, "out"),
                                    stream_ptr(stream)))
    return out


def gae(rewards, values, dones, last_values, gamma, lam, normalize=0, adv=None, ret=None, adv_stats=None,
        ws=None, stream=None):
    """rl_gae over [T][N] float32 device tensors; returns (adv, ret, adv_stats). The [T][N] arguments may be
    column ranges of wider arrays (rows contiguous, one shared row stride): then rl_gae_strided runs. With
    normalize = 3, adv_stats holds the deferred form (rl_gae_stats_bytes bytes)."""
    t, n = rewards.shape
    dev = rewards.device
    adv = torch.empty((t, n), dtype=torch.float32, device=dev) if adv is None else adv
    ret = torch.empty((t, n), dtype=torch.float32, device=dev) if ret is None else ret
    if normalize and adv_stats is None:
        size = 3 if normalize != 3 else gae_stats_bytes(t, n) // 8
        adv_stats = torch.zeros(size, dtype=torch.float64, device=dev)
    if normalize in (1, 2) and ws is None:
        ws = workspace("gae", gae_workspace_bytes(t, n), dev, stream)
    r_p, ld = _rows(rewards, "rewards")
    ptrs = [r_p] + [_rows(x, name, ld)[0] for x, name in ((values, "values"), (dones, "dones"))]
    out = [_rows(x, name, ld)[0] for x, name in ((adv, "adv"), (ret, "ret"))]
    check(lib().rl_gae_strided(*ptrs, dptr(last_values, torch.float32, "last_values"), t, n, ld, float(gamma),
                               float(lam), *out, int(normalize), dptr(adv_stats, torch.float64, "adv_stats"),
                               dptr(ws), 0 if ws is None else ws.numel(), stream_ptr(stream)))
    return adv, ret, adv_stats


def vtrace(rewards, values, dones, last_values, log_rhos, gamma, lam=1.0, rho_bar=1.0, c_bar=1.0, pg_rho_bar=1.0,
           vs=None, pg_adv=None, stream=None):
    """rl_vtrace over [T][N]; returns (vs, pg_adv)."""
    t, n = rewards.shape
    vs = torch.empty((t, n), dtype=torch.float32, device=rewards.device) if vs is None else vs
    pg_adv = torch.empty((t, n), dtype=torch.float32, device=rewards.device) if pg_adv is None else pg_adv
    r_p, ld = _rows(rewards, "rewards")
    ins = [r_p] + [_rows(x, name, ld)[0] for x, name in ((values, "values"), (dones, "dones"))]
    check(lib().rl_vtrace_strided(*ins, dptr(last_values, torch.float32, "last_values"),
                                  _rows(log_rhos, "log_rhos", ld)[0], t, n, ld, float(gamma), float(lam),
                                  float(rho_bar), float(c_bar), float(pg_rho_bar), _rows(vs, "vs", ld)[0],
                                  _rows(pg_adv, "pg_adv", ld)[0], stream_ptr(stream)))
    return vs, pg_adv


def ppo_loss_workspace_bytes(b: int, mb: int) -> int:
    nb = ctypes.c_size_t()
    check(lib().rl_ppo_loss_workspace_bytes(b, mb, ctypes.byref(nb)))
    return nb.value


def ppo_loss(logits, actions, old_logp, adv, ret, new_values, perm, minibatch, clip_eps=0.2, vf_coef=0.5,
             ent_coef=0.01, adv_stats=None, out=None, ws=None, stream=None, mb_index=None):
    """rl_ppo_loss; returns out float32[B/minibatch][4] = (pg, value, entropy, total) per minibatch.
    Minibatches come from `perm` (int32 gather), or from `mb_index` (uint16 minibatch of each sample,
    read in storage order), or are contiguous when both are None."""
    b, a = logits.shape
    dev = logits.device
    out = torch.empty((b // minibatch, 4), dtype=torch.float32, device=dev) if out is None else out
    if ws is None:
        ws = workspace("ppo", ppo_loss_workspace_bytes(b, minibatch), dev, stream)
    check(lib().rl_ppo_loss(dptr(logits, torch.float32, "logits"), dptr(actions, torch.int32, "actions"),
                            dptr(old_logp, torch.float32, "old_logp"), dptr(adv, torch.float32, "adv"),
                            dptr(ret, torch.float32, "ret"), dptr(new_values, torch.float32, "new_values"),
                            dptr(perm, torch.int32, "perm"), dptr(mb_index, torch.uint16, "mb_index"),
                            dptr(adv_stats, torch.float64, "adv_stats"),
                            b, a, minibatch, float(clip_eps), float(vf_coef), float(ent_coef),
                            dptr(out, torch.float32, "out"), dptr(ws), ws.numel(), stream_ptr(stream)))
    return out


def ppo_loss_noalloc(logits, actions, old_logp, adv, ret, new_values, perm, minibatch, clip_eps=0.2, vf_coef=0.5,
                     ent_coef=0.01, adv_stats=None, out=None, stream=None, mb_index=None):
    """rl_ppo_loss_noalloc: ppo_loss with the library's fixed device workspace instead of a workspace
    argument (pass `out` to allocate nothing here either)."""
    b, a = logits.shape
    out = torch.empty((b // minibatch, 4), dtype=torch.float32, device=logits.device) if out is None else out
    check(lib().rl_ppo_loss_noalloc(dptr(logits, torch.float32, "logits"), dptr(actions, torch.int32, "actions"),
                                    dptr(old_logp, torch.float32, "old_logp"), dptr(adv, torch.float32, "adv"),
                                    dptr(ret, torch.float32, "ret"), dptr(new_values, torch.float32, "new_values"),
                                    dptr(perm, torch.int32, "perm"), dptr(mb_index, torch.uint16, "mb_index"),
                                    dptr(adv_stats, torch.float64, "adv_stats"),
                                    b, a, minibatch, float(clip_eps), float(vf_coef), float(ent_coef),
                                    dptr(out, torch.float32, "out"), stream_ptr(stream)))
    return out


def ppo_loss_grad(logits, actions, old_logp, adv, ret, new_values, perm, minibatch, clip_eps=0.2, vf_coef=0.5,
                  ent_coef=0.01, adv_stats=None, out=None, dlogits=None, dvalues=None, ws=None, stream=None,
                  mb_index=None):
    """rl_ppo_loss_grad; returns (out [B/minibatch][4], dlogits [B][A], dvalues [B]): the loss scalars and
    the gradient of each minibatch's total with respect to its samples' logits and values."""
    b, a = logits.shape
    dev = logits.device
    out = torch.empty((b // minibatch, 4), dtype=torch.float32, device=dev) if out is None else out
    dlogits = torch.empty((b, a), dtype=torch.float32, device=dev) if dlogits is None else dlogits
    dvalues = torch.empty(b, dtype=torch.float32, device=dev) if dvalues is None else dvalues
    if ws is None:
        ws = workspace("ppo", ppo_loss_workspace_bytes(b, minibatch), dev, stream)
    check(lib().rl_ppo_loss_grad(dptr(logits, torch.float32, "logits"), dptr(actions, torch.int32, "actions"),
                                 dptr(old_logp, torch.float32, "old_logp"), dptr(adv, torch.float32, "adv"),
                                 dptr(ret, torch.float32, "ret"), dptr(new_values, torch.float32, "new_values"),
                                 dptr(perm, torch.int32, "perm"), dptr(mb_index, torch.uint16, "mb_index"),
                                 dptr(adv_stats, torch.float64, "adv_stats"),
                                 b, a, minibatch, float(clip_eps), float(vf_coef), float(ent_coef),
                                 dptr(out, torch.float32, "out"), dptr(dlogits, torch.float32, "dlogits"),
                                 dptr(dvalues, torch.float32, "dvalues"), dptr(ws), ws.numel(), stream_ptr(stream)))
    return out, dlogits, dvalues


def _rows_view(t, dtype, what, inner):
    """Device address and dim-0 stride (elements) of a [T][...] view whose inner `inner` elements per
    row are contiguous."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != dtype:
        raise TypeError(f"{what} must be a {dtype} device tensor")
    flat_inner = t[0].numel() if t.dim() > 1 else 1
    if flat_inner != inner or not t[0].is_contiguous():
        raise ValueError(f"{what}: each decision's {inner} elements must be contiguous")
    return ctypes.c_void_p(t.data_ptr()), t.stride(0)


class Policy:
    """Packed stand-in policy weights on the device (rl_policy_pack): the encoder float32 [128][1397]
    (stored as bfloat16) and the decoder float32 [13][128] (12 logits, then the value)."""

    def __init__(self, enc_w, dec_w, seed=0, device="cuda", stream=None):
        L = lib()
        nb = ctypes.c_size_t()
        check(L.rl_policy_weights_bytes(ctypes.byref(nb)))
        self.device = torch.device(device)
        self.seed = int(seed) & ((1 << 64) - 1)
        self.packed = torch.empty(nb.value, dtype=torch.uint8, device=self.device)
        self._enc = _dev(enc_w, torch.float32, self.device).reshape(POLICY_HIDDEN, OBS_TILES_SIZE).contiguous()
        self._dec = _dev(dec_w, torch.float32, self.device).reshape(POLICY_ACTIONS + 1, POLICY_HIDDEN).contiguous()
        check(L.rl_policy_pack(dptr(self._enc), dptr(self._dec), dptr(self.packed), stream_ptr(stream)))

    def forward(self, obs, t, env_offset=0, actions=None, logp=None, values=None, stream=None):
        """rl_policy_forward on obs float32 [n][stride]; returns (actions int32, logp, values float32 [n])."""
        if obs.dim() != 2 or obs.stride(1) != 1:
            raise ValueError("obs must be [n][stride] with contiguous rows")
        n = obs.shape[0]
        if actions is None:
            actions = torch.empty(n, dtype=torch.int32, device=self.device)
        if logp is None:
            logp = torch.empty(n, dtype=torch.float32, device=self.device)
        if values is None:
            values = torch.empty(n, dtype=torch.float32, device=self.device)
        if obs.dtype != torch.float32 or not obs.is_cuda:
            raise TypeError("obs must be a float32 device tensor")
        check(lib().rl_policy_forward(dptr(self.packed), ctypes.c_void_p(obs.data_ptr()), n, obs.stride(0),
                                      self.seed, int(t), int(env_offset), dptr(actions, torch.int32, "actions"),
                                      dptr(logp, torch.float32, "logp"), dptr(values, torch.float32, "values"),
                                      stream_ptr(stream)))
        return actions, logp, values


def rollout_group(env, obs0, obs, actions, logp, values, rewards, dones, env_offset=0, stream=None):
    """An rl_rollout_group over [T][n...] views (each decision's block contiguous; dim 0 may stride over
    a wider [T][N] rollout)."""
    n, d = env.num_envs, env.obs_stride
    g = RolloutGroup()
    g.env = env._handle
    g.obs0 = None if obs0 is None else dptr(obs0, torch.float32, "obs0")
    g.obs, g.obs_row = _rows_view(obs, torch.float32, "obs", n * d)
    g.actions, g.row = _rows_view(actions, torch.int32, "actions", n)
    for name, t in (("logp", logp), ("values", values), ("rewards", rewards), ("dones", dones)):
        addr, row = _rows_view(t, torch.float32, name, n)
        if row != g.row:
            raise ValueError(f"{name} must have the same decision stride as actions")
        setattr(g, name, addr)
    g.env_offset = int(env_offset)
    g.stream = stream_ptr(stream)
    g._keep = (obs0, obs, actions, logp, values, rewards, dones)
    return g


def rollout(policy, groups, t0, steps, alternate=True):
    """rl_rollout: decisions t0 .. t0 + steps - 1 of every group (see rollout_group)."""
    arr = (RolloutGroup * len(groups))(*groups)
    check(lib().rl_rollout(dptr(policy.packed), policy.seed, arr, len(groups), int(t0), int(steps),
                           1 if alternate else 0))


def read_probe(buf, chunk, sink, stream=None):
    """rl_read_probe over a device tensor: 16-byte loads, one `chunk`-byte contiguous chunk per block; `sink`
    is a device uint32 / int32 tensor of at least one element."""
    nbytes = buf.numel() * buf.element_size()
    check(lib().rl_read_probe(dptr(buf), nbytes, int(chunk), dptr(sink), stream_ptr(stream)))


def store_probe(buf, chunk, stream=None):
    """rl_store_probe over a device tensor: 16-byte stores, one `chunk`-byte contiguous chunk per block."""
    nbytes = buf.numel() * buf.element_size()
    check(lib().rl_store_probe(dptr(buf), nbytes, int(chunk), stream_ptr(stream)))
