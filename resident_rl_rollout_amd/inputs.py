"""Seeded synthetic inputs for the rollout hot path.

This module draws the random inputs that both the HIP path and the CPU oracle consume: tile maps,
checkpoint and spawn tables, sprite patterns, actions, rewards / values / dones, policy logits and
minibatch permutations. It holds none of the path's own arithmetic (no physics, no observation
layout, no GAE, no loss); it imports neither the HIP binding nor the oracle.

The one piece of policy arithmetic here is the stand-in policy's sampling: actions are drawn by
Gumbel-max from the old logits and their old log-probability is taken in float64 and rounded to
float32. Sampling and recording the old probability belong to the collect phase that runs the
network ("Teaching Mario to speedrun", section 6, the whole-algorithm listing), not to the loss.

Tile codes used by the generated maps: 0 air, 1 solid floor, 2 platform (solid), 3 freeze (passable).
Positions are in sub-units: one tile is 256 sub-units, the player box is 192 x 192.
"""
from __future__ import annotations

import dataclasses

import numpy as np

TILE_AIR, TILE_SOLID, TILE_PLATFORM, TILE_FREEZE = 0, 1, 2, 3
NUM_ACTIONS = 12


@dataclasses.dataclass
class MapSet:
    maps: np.ndarray      # u8[M][H][W], row 0 at the top
    ckpts: np.ndarray     # int32[M][K][2] = (col, row)
    spawns: np.ndarray    # int32[M][2]    = (x, y) in sub-units
    ckpt_spawns: np.ndarray = None   # int32[M][K][2] = (x, y) standing spot at each checkpoint

    @property
    def num_maps(self) -> int:
        return int(self.maps.shape[0])

    @property
    def map_h(self) -> int:
        return int(self.maps.shape[1])

    @property
    def map_w(self) -> int:
        return int(self.maps.shape[2])

    @property
    def num_ckpts(self) -> int:
        return int(self.ckpts.shape[1])


def make_map(seed: int, h: int, w: int, p_platform: float = 0.10, p_freeze: float = 0.02):
    """One seeded map: a floor whose height is a clipped random walk in [4, 12] (8 on columns 0-2),
    and, in the air above the floor from column 3 on, platform tiles with probability p_platform and
    freeze tiles with probability p_freeze. Returns (tiles u8[h][w], floor heights int[w])."""
    rng = np.random.default_rng(seed)
    steps = rng.integers(-1, 2, size=w)
    heights = np.empty(w, dtype=np.int64)
    hcur = 8
    for c in range(w):
        if c >= 3:
            hcur = int(np.clip(hcur + steps[c], 4, 12))
        heights[c] = hcur
    heights = np.minimum(heights, h - 2)
    tiles = np.zeros((h, w), dtype=np.uint8)
    rows = np.arange(h)[:, None]
    floor = rows >= (h - heights)[None, :]
    tiles[floor] = TILE_SOLID
    u = rng.random((h, w))
    air_above = (~floor) & (np.arange(w)[None, :] >= 3)
    tiles[air_above & (u < p_platform)] = TILE_PLATFORM
    tiles[air_above & (u >= p_platform) & (u < p_platform + p_freeze)] = TILE_FREEZE
    return tiles, heights


def make_mapset(seeds, h: int, w: int) -> MapSet:
    """Maps for the given seeds, with checkpoint k at column 16(k+1) on the row just above the floor
    (K = (w-1)//16 per map) and the spawn standing on the floor at column 1."""
    k = (w - 1) // 16
    maps, ckpts, spawns, stands = [], [], [], []
    for s in seeds:
        tiles, heights = make_map(int(s), h, w)
        maps.append(tiles)
        cols = 16 * (np.arange(k) + 1)
        ckpts.append(np.stack([cols, h - heights[cols] - 1], axis=1))
        spawns.append([256, (h - int(heights[1])) * 256 - 192])
        # standing spot at each checkpoint: the box centred in the checkpoint's column, on the floor or
        # on the platform stack that covers it (tile codes 1 and 2 block)
        st = []
        for c in cols:
            r = h - int(heights[c]) - 1
            while r > 0 and tiles[r, c] in (1, 2):
                r -= 1
            st.append([int(c) * 256 + 32, (r + 1) * 256 - 192])
        stands.append(st)
    return MapSet(np.ascontiguousarray(np.stack(maps)).astype(np.uint8),
                  np.asarray(ckpts, dtype=np.int32).reshape(len(seeds), k, 2),
                  np.asarray(spawns, dtype=np.int32),
                  np.asarray(stands, dtype=np.int32).reshape(len(seeds), k, 2))


def make_sprites(seed: int = 30) -> np.ndarray:
    """16 seeded 8x8 grayscale sprite patterns, uniform u8."""
    return np.random.default_rng(seed).integers(0, 256, size=(16, 8, 8), dtype=np.uint8)


def make_actions(seed: int, steps: int, n: int) -> np.ndarray:
    """Uniform random actions int32[steps][n] in [0, 12)."""
    return np.random.default_rng(seed).integers(0, NUM_ACTIONS, size=(steps, n), dtype=np.int32)


@dataclasses.dataclass
class GaeInputs:
    rewards: np.ndarray      # f32[T][N]
    values: np.ndarray       # f32[T][N]
    dones: np.ndarray        # f32[T][N], 0 or 1
    last_values: np.ndarray  # f32[N]


def make_gae_inputs(seed: int, t: int, n: int, p_spike: float = 0.05, p_done: float = 0.01) -> GaeInputs:
    """Rewards ~ N(0,1) with +1 added to a p_spike fraction, values ~ N(0,1), dones ~ Bernoulli(p_done),
    bootstrap values ~ N(0,1); all float32."""
    rng = np.random.default_rng(seed)
    r = rng.standard_normal((t, n), dtype=np.float32)
    r += (rng.random((t, n)) < p_spike).astype(np.float32)
    v = rng.standard_normal((t, n), dtype=np.float32)
    d = (rng.random((t, n)) < p_done).astype(np.float32)
    vl = rng.standard_normal(n, dtype=np.float32)
    return GaeInputs(r, v, d, vl)


def make_log_rhos(seed: int, t: int, n: int, spread: float = 0.6) -> np.ndarray:
    """Log importance ratios log pi - log mu of the taken actions, U(-spread, spread), float32: ratios from
    0.55 to 1.82, so both sides of rho_bar = c_bar = 1 occur (the stand-in policy's new-minus-old logits
    move by at most 0.3 each, which bounds the log-ratio by 0.6)."""
    rng = np.random.default_rng(seed)
    return rng.uniform(-spread, spread, (t, n)).astype(np.float32)


@dataclasses.dataclass
class PolicyInputs:
    new_logits: np.ndarray   # f32[B][A]
    actions: np.ndarray      # int32[B]
    old_logp: np.ndarray     # f32[B]
    new_values: np.ndarray   # f32[B]
    perm: np.ndarray         # int32[B], a seeded shuffle of 0..B-1


def make_policy_inputs(seed: int, b: int, a: int = NUM_ACTIONS, delta: float = 0.3,
                       chunk: int = 1 << 20) -> PolicyInputs:
    """Stand-in policy outputs: old logits ~ N(0,1), new = old + U(-delta, delta); the action is sampled
    from the old logits by Gumbel-max and its old log-probability recorded (float64, rounded to f32);
    new values ~ N(0,1); a seeded permutation for minibatch shuffling. Rows are drawn in chunks of
    `chunk` (old logits, then the perturbation, then the Gumbel noise, per chunk) to bound temporaries."""
    rng = np.random.default_rng(seed)
    new = np.empty((b, a), np.float32)
    act = np.empty(b, np.int32)
    old_logp = np.empty(b, np.float32)
    for lo in range(0, b, chunk):
        hi = min(b, lo + chunk)
        rows = hi - lo
        old = rng.standard_normal((rows, a), dtype=np.float32)
        pert = rng.random((rows, a), dtype=np.float32) * np.float32(2 * delta) - np.float32(delta)
        new[lo:hi] = old + pert
        gumbel = -np.log(-np.log(rng.random((rows, a))))
        o64 = old.astype(np.float64)
        k = np.argmax(o64 + gumbel, axis=1)
        m = o64.max(axis=1, keepdims=True)
        lse = m[:, 0] + np.log(np.exp(o64 - m).sum(axis=1))
        act[lo:hi] = k
        old_logp[lo:hi] = o64[np.arange(rows), k] - lse
    new_v = rng.standard_normal(b, dtype=np.float32)
    perm = rng.permutation(b).astype(np.int32)
    return PolicyInputs(new, act, old_logp, new_v, perm)


def minibatch_index(perm: np.ndarray, mb: int) -> np.ndarray:
    """The same minibatch split as `perm` (minibatch m = perm[m*mb : (m+1)*mb]) as the minibatch number of
    every sample, uint16[B]."""
    idx = np.empty(perm.shape[0], np.uint16)
    idx[perm] = (np.arange(perm.shape[0]) // mb).astype(np.uint16)
    return idx


def pack_aim(dx, dy) -> np.ndarray:
    """Hook mode's aim per env as int32: dx in the low 16 bits, dy in the high 16 bits (both int16)."""
    dx = np.asarray(dx, np.int64)
    dy = np.asarray(dy, np.int64)
    assert ((dx >= -32768) & (dx <= 32767) & (dy >= -32768) & (dy <= 32767)).all()
    return ((dx & 0xFFFF) | ((dy & 0xFFFF) << 16)).astype(np.uint32).view(np.int32)


def make_aims(seed: int, steps: int, n: int, zero_frac: float = 0.05) -> np.ndarray:
    """Synthetic continuous aims, int32[steps][n] packed by pack_aim: angle uniform over the circle,
    magnitude uniform in [64, 4096] sub-units (a quarter tile to 16 tiles), rounded to integers; a
    fraction zero_frac of them exactly (0, 0)."""
    rng = np.random.default_rng(seed)
    ang = rng.uniform(0.0, 2.0 * np.pi, (steps, n))
    mag = rng.uniform(64.0, 4096.0, (steps, n))
    dx = np.rint(mag * np.cos(ang)).astype(np.int64)
    dy = np.rint(mag * np.sin(ang)).astype(np.int64)
    zero = rng.random((steps, n)) < zero_frac
    dx[zero] = 0
    dy[zero] = 0
    return pack_aim(dx, dy)


def make_values(seed: int, t: int, n: int):
    """Stand-in value head outputs: values f32[T][N] and bootstrap values f32[N], both ~ N(0,1)."""
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((t, n), dtype=np.float32),
            rng.standard_normal(n, dtype=np.float32))


def make_policy_weights(seed: int, enc_std: float = 0.01):
    """Seeded stand-in weights of the inference: encoder f32[128][1397] ~ N(0, enc_std^2) (observation
    norms are about 100, so hidden units come out about N(0, 1)) and decoder f32[13][128] ~ N(0, 1/128)
    (logits and value about N(0, 1))."""
    rng = np.random.default_rng(seed)
    enc = (rng.standard_normal((128, 1397)) * enc_std).astype(np.float32)
    dec = (rng.standard_normal((13, 128)) / np.sqrt(128.0)).astype(np.float32)
    return enc, dec


# The five workloads, by what they are. Sizes only; the generators above draw their contents.
WORKLOADS = {
    "tiny": dict(n=64, t=128, maps=1, map_h=32, map_w=128, map_seed0=1, action_seed=2, value_seed=3),
    "gae_ppo": dict(n=2048, t=128, seed=10, minibatch=8192),
    "env_step": dict(n=65536, maps=64, map_h=256, map_w=1024, map_seed0=100, action_seed=4,
                     time_limit=2000),
    "rollout": dict(n=65536, t=128, maps=64, map_h=256, map_w=1024, map_seed0=100, policy_seed=20,
                    minibatches=16),
    "pixels": dict(n=16384, t=128, maps=64, map_h=256, map_w=1024, map_seed0=100, sprite_seed=30,
                   policy_seed=20),
}
