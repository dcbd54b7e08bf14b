"""Throughput of the GPU-resident PPO rollout hot path on one MI355X.

One timed step is one whole rollout of the full-rollout workload: 65536 envs on 64 seeded 256x1024 tile
maps step 128 times (env_step + obs_gather writing 31x43 tile windows, 4x15 frame stacks and checkpoint
dims into a resident [actions | obs | rewards | dones] rollout buffer), then GAE (gamma 0.99, lambda 0.95)
with whole-batch advantage normalisation, then the PPO clipped-surrogate / value / entropy loss over 16
shuffled minibatches of 524288 samples. Policy outputs (actions sampled from seeded old logits, new
logits, values) are seeded N(0,1) stand-ins, generated before timing and resident in HBM.

Prints one JSON line: env-steps/s of the whole job, the roofline of the env step (the dominant kernel),
GAE + loss GB/s, and the CPU oracle timed on a bounded sample of the same workload, single-threaded and in
one process per host core of the GPU's share (the oracle itself is unchanged; envs and minibatches are
independent). GAE and loss GB/s come
from separate repetitions after a read-only cache flush (their own HBM efficiency); their times inside the
rollout, which also absorb the write-back of the rollout's last observations, are reported beside them.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--workload rollout|pixels|infer]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
N_ENVS, HORIZON, N_MAPS, MAP_H, MAP_W, MINIBATCHES = 65536, 128, 64, 256, 1024, 16
GAMMA, LAMBDA = 0.99, 0.95

# Algorithmic HBM bytes per unit. The fused tile step per env: the observation row, the action, the
# current ring slot (5 words) and the two slots before it, the two extra words read and written, the new
# slot, the reward and the done.
ENV_BYTES_PER_ENV_STEP = 1397 * 4 + 4 + 20 + 40 + 8 + 20 + 8 + 4 + 4    # 5696
ENV_BYTES_WAYPOINTS = 4 + 4   # the path index, read and written (the 0.5 MB waypoint table stays in cache)
ENV_BYTES_RESPAWN = 4 + 4 + 4  # the from-start flag read, the step's outcome written and read back by the append
ENV_BYTES_HOOK = 4 + 12 + 12   # the aim read; the hook's tip x, y and flight velocity read and written
# The pixel step per env (two kernels): the physics reads the action, the current slot and the extras and
# writes the new slot, the extras, the reward and the done; the render reads (x, y) of the four stacked
# slots and writes the 4 x 84 x 84 frame bytes.
PIX_ENVS = 16384
PIX_BYTES_PER_ENV_STEP = 4 * 84 * 84 + (4 + 20 + 8) + (20 + 8 + 4 + 4) + 4 * 8   # 28324
GAE_BYTES_PER_ELEM = 5 * 4                            # r, v, d in; adv, ret out (statistics only: normalised in the loss)
VTRACE_BYTES_PER_ELEM = 6 * 4                        # r, v, d, log rho in; vs, pg advantage out
GRAD_BYTES_PER_SAMPLE = 12 * 4 + 4                   # the gradient row and the value gradient, written
# The stand-in inference per env: the observation row read; the action, its log-probability and the value
# written. Per launch also the packed weights once (bfloat16 encoder 128 x 1408, float32 decoder 13 x 128);
# blocks re-read them from L2, which HBM does not see.
POLICY_BYTES_PER_ENV = 1397 * 4 + 3 * 4               # 5600
POLICY_WEIGHT_BYTES = 128 * 1408 * 2 + 13 * 128 * 4   # 367104
POLICY_SEED = 31
LOSS_BYTES_PER_SAMPLE = {"stream": 12 * 4 + 5 * 4 + 2,  # logits row; action, old logp, adv, ret, value; minibatch id
                         # up to 16 minibatches: the same without the id, + the permutation entry read, its
                         # sorted entry written and read back (the stream blocks place their own numbers)
                         "perm": 12 * 4 + 5 * 4 + 3 * 4,
                         # 17 to 64: + the 2-byte minibatch id written (and read, as in "stream")
                         "perm_placed": 12 * 4 + 5 * 4 + 2 + 3 * 4 + 2}


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20, help="timed rollouts")
    p.add_argument("--warmup", type=int, default=5, help="untimed rollouts")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-envs", type=int, default=None,
                   help="envs in the oracle's bounded sample (default 16384 for the rollout, 512 for pixels)")
    p.add_argument("--iso-reps", type=int, default=20, help="isolated GAE / loss repetitions (median and min reported)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="first run one plain 1 GiB device-to-device copy, whose rocprofv3 FETCH_SIZE / WRITE_SIZE "
                        "scale the counters of the other kernels")
    p.add_argument("--schedule", choices=("double", "alternate", "single"), default="double",
                   help="infer workload: the schedule whose throughput is `value` (all three are measured)")
    p.add_argument("--workload", choices=("rollout", "pixels", "infer"), default="rollout",
                   help="rollout: the tile-observation full rollout (the default bench line); pixels: 16384 envs "
                        "x 128 steps rendering 4 x 84 x 84 u8 frames, then GAE")
    p.add_argument("--reward", choices=("checkpoints", "waypoints"), default="checkpoints",
                   help="the rollout's reward: checkpoints (+10 each, x progress, time penalty) or the waypoint "
                        "path (progress along each map's BFS tile path, grace-zone distance penalty)")
    p.add_argument("--respawn", choices=("off", "adaptive"), default="off",
                   help="adaptive checkpoint respawn (each map's outcome buffer, top-quarter restarts, frontier cap)")
    p.add_argument("--hook", choices=("off", "grapple"), default="off",
                   help="grapple hook aimed by seeded continuous aims (rl_env_step_aim)")
    p.add_argument("--no-pixels", action="store_true",
                   help="skip the short run of the pixel workload reported beside the default line")
    p.add_argument("--loss-mode", choices=("stream", "perm"), default="stream",
                   help="minibatches as per-sample minibatch ids read in storage order, or given by a permutation "
                        "(turned into the same ids on the device, then the same pass)")
    return p.parse_args()


def source_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(kernel_key):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None when the kernel source has
    changed since they were taken (or none were taken)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(kernel_key)
    if not rec:
        return None
    src = os.path.join(ROOT, rec["source"])
    if not os.path.exists(src) or source_sha(src) != rec["source_sha"]:
        return None
    return rec["hbm_bytes_per_launch"]


def path_goal(grid, col, row):
    """A map's path goal: the finish checkpoint's tile, or the nearest tile above it in its column that a
    box can pass (a platform may cover the checkpoint's tile; the finish itself is reached by column)."""
    while row > 0 and grid[row, col] in (1, 2):
        row -= 1
    return col, row


def path_ends(ms, m):
    x, y = ms.spawns[m]
    start = ((int(x) + 96) >> 8, (int(y) + 96) >> 8)
    return start, path_goal(ms.maps[m], int(ms.ckpts[m, -1, 0]), int(ms.ckpts[m, -1, 1]))


def pad_paths(paths):
    kw = max(len(p) for p in paths)
    table = np.zeros((len(paths), kw, 2), np.int32)
    for m, p in enumerate(paths):
        table[m, :len(p)] = p
        table[m, len(p):] = p[-1]
    return table, np.array([len(p) for p in paths], np.int32)


def oracle_waypoints(ms):
    """The oracle's own BFS paths, for the CPU leg."""
    import oracle
    return pad_paths([oracle.bfs_path(ms.maps[m], *path_ends(ms, m)) for m in range(ms.maps.shape[0])])


RESPAWN_SEED = 2024


def _env_kw():
    return {k: _SHARED[k] for k in ("reward_mode", "waypoints", "wp_lens", "respawn_mode", "ckpt_spawns",
                                    "respawn_seed", "hook_mode") if k in _SHARED}


def _aim(t, lo, hi):
    aims = _SHARED.get("aims")
    return None if aims is None else aims[t, lo:hi]


def cpu_baseline(ms, policy_actions, values, last_values, pi, n_sample):
    """The oracle as it stands, single-threaded, on the first n_sample envs of the same workload: 128
    steps with tile observations, GAE by its definition with normalisation, and the loss over the
    sample's batch in minibatches of the same share. Returns env-steps/s of the whole path."""
    import oracle
    n = n_sample
    t0 = time.perf_counter()
    env = oracle.OracleEnv(ms.maps, ms.ckpts, ms.spawns, n, **_env_kw())
    env.reset()
    obs = np.empty((n, 1397), np.float32)
    rew = np.empty((HORIZON, n), np.float32)
    dn = np.empty((HORIZON, n), np.float32)
    for t in range(HORIZON):
        rew[t], dn[t] = env.step(policy_actions[t, :n], _aim(t, 0, n))
        env.obs_tiles(obs)
    adv, ret = oracle.gae(rew, values[:, :n], dn, last_values[:n], float(np.float32(GAMMA)),
                          float(np.float32(LAMBDA)))
    na, _, _ = oracle.normalize(adv)
    b = HORIZON * n
    sel = np.arange(HORIZON)[:, None] * N_ENVS + np.arange(n)[None, :]
    sel = sel.reshape(-1)
    perm = np.random.default_rng(5).permutation(b).astype(np.int32)
    oracle.ppo_loss(pi.new_logits[sel], policy_actions[:, :n].reshape(-1), pi.old_logp[sel], na.reshape(-1),
                    ret.reshape(-1), pi.new_values[sel], perm, b // MINIBATCHES)
    dt = time.perf_counter() - t0
    return b / dt, dt


CPU_WORKERS = 16     # the host-core share of one GPU
_SHARED = {}         # inputs the forked workers read (copy-on-write)


def _env_shard(lo_hi):
    """Worker: the oracle's env step + tile observations for envs [lo, hi), then GAE over the shard."""
    import oracle
    lo, hi = lo_hi
    g = _SHARED
    n = hi - lo
    env = oracle.OracleEnv(g["ms"].maps, g["ms"].ckpts, g["ms"].spawns, n, env_offset=lo, **_env_kw())
    env.reset()
    obs = np.empty((n, 1397), np.float32)
    rew = np.empty((HORIZON, n), np.float32)
    dn = np.empty((HORIZON, n), np.float32)
    for t in range(HORIZON):
        rew[t], dn[t] = env.step(g["actions"][t, lo:hi], _aim(t, lo, hi))
        env.obs_tiles(obs)
    adv, ret = oracle.gae(rew, g["values"][:, lo:hi], dn, g["last_values"][lo:hi], float(np.float32(GAMMA)),
                          float(np.float32(LAMBDA)))
    return adv, ret


def _loss_minibatch(args):
    """Worker: the oracle's loss for one minibatch (its sample indices into the rollout batch)."""
    import oracle
    rows, adv, ret = args
    g = _SHARED
    pi = g["pi"]
    out, _ = oracle.ppo_loss(pi.new_logits[rows], g["actions"].reshape(-1)[rows], pi.old_logp[rows], adv, ret,
                             pi.new_values[rows], None, rows.size)
    return out[0]


def cpu_baseline_all_cores(ms, policy_actions, values, last_values, pi, n, workers):
    """The same bounded sample as cpu_baseline, with the single-threaded oracle run in `workers` forked
    processes: envs are independent (env shards with GAE per shard), and so are the loss minibatches."""
    import multiprocessing as mp

    import oracle
    _SHARED.update(ms=ms, actions=policy_actions, values=values, last_values=last_values, pi=pi)
    t0 = time.perf_counter()
    bounds = np.linspace(0, n, workers + 1).astype(int)
    with mp.get_context("fork").Pool(workers) as pool:
        parts = pool.map(_env_shard, [(int(a), int(z)) for a, z in zip(bounds[:-1], bounds[1:])])
        adv = np.concatenate([p[0] for p in parts], axis=1)
        ret = np.concatenate([p[1] for p in parts], axis=1)
        na, _, _ = oracle.normalize(adv)
        b = HORIZON * n
        sel = (np.arange(HORIZON)[:, None] * N_ENVS + np.arange(n)[None, :]).reshape(-1)
        perm = np.random.default_rng(5).permutation(b)
        mb = b // MINIBATCHES
        tasks = []
        for m in range(MINIBATCHES):
            k = perm[m * mb:(m + 1) * mb]
            tasks.append((sel[k], na.reshape(-1)[k], ret.reshape(-1)[k]))
        pool.map(_loss_minibatch, tasks)
    dt = time.perf_counter() - t0
    return b / dt, dt


def calibration_copy(torch, dev):
    """One plain device-to-device copy of 1 GiB: the known byte count that scales the HBM counters."""
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def pixel_rollouts(torch, binding, dev, ms, sprites, policy_actions, values, last_values, steps, warmup):
    """The pixel workload on the GPU: 16384 envs x 128 steps rendering 4 x 84 x 84 u8 frames into a resident
    rollout buffer, then GAE with whole-batch statistics; `warmup` untimed and `steps` timed rollouts.
    Returns the whole-job rate, the per-launch env step times and the step's roofline."""
    n = PIX_ENVS
    env = binding.Env(ms.maps, ms.ckpts, ms.spawns, n, frame_skip=3, time_limit=2000, obs_mode=binding.OBS_PIXELS,
                      sprites=sprites, device=dev)
    # rollout buffer: one allocation of [actions T*N | obs T*N*28224 (u8) | rewards T*N | dones T*N]
    a_bytes = HORIZON * n * 4
    o_bytes = HORIZON * n * 4 * 84 * 84
    offs = [0, a_bytes, a_bytes + o_bytes, a_bytes + o_bytes + a_bytes]
    buf = torch.empty(offs[3] + a_bytes, dtype=torch.uint8, device=dev)
    actions = buf[offs[0]:offs[1]].view(torch.int32).view(HORIZON, n)
    obs = buf[offs[1]:offs[2]].view(HORIZON, n, 4 * 84 * 84)
    rewards = buf[offs[2]:offs[3]].view(torch.float32).view(HORIZON, n)
    dones = buf[offs[3]:].view(torch.float32).view(HORIZON, n)
    actions.copy_(torch.from_numpy(policy_actions))
    values_d = torch.from_numpy(values).to(dev)
    last_d = torch.from_numpy(last_values).to(dev)
    adv = torch.empty((HORIZON, n), dtype=torch.float32, device=dev)
    ret = torch.empty_like(adv)
    stats = torch.zeros(3, dtype=torch.float64, device=dev)
    env.reset(obs[0])
    torch.cuda.synchronize()

    def rollout(ev=None):
        # one event pair around the 128 back-to-back env launches: events between launches would add
        # their own barrier and timestamp packets to every step
        if ev is not None:
            ev["env"][0].record()
        for t in range(HORIZON):
            env.step(actions[t], obs[t], rewards[t], dones[t])
        if ev is not None:
            ev["env"][1].record()
            ev["gae"][0].record()
        binding.gae(rewards, values_d, dones, last_d, GAMMA, LAMBDA, normalize=2, adv=adv, ret=ret, adv_stats=stats)
        if ev is not None:
            ev["gae"][1].record()

    for _ in range(warmup):
        rollout()
    torch.cuda.synchronize()
    mk = lambda: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    events = [{"env": mk(), "gae": mk()} for _ in range(steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(steps):
        rollout(events[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    env.close()
    del buf

    env_ms = np.array([ev["env"][0].elapsed_time(ev["env"][1]) / HORIZON for ev in events])   # per launch
    gae_ms = np.array([ev["gae"][0].elapsed_time(ev["gae"][1]) for ev in events])
    env_avg_s = float(env_ms.mean()) * 1e-3
    launch_bytes = n * PIX_BYTES_PER_ENV_STEP
    achieved = launch_bytes / env_avg_s / 1e9
    return {
        "workload": "pixel rollout: 16384 envs x 128 steps on 64 seeded 256x1024 maps, frame-skip 3, 4 x 84 x 84 u8 "
                    "frames from 16 seeded 8x8 sprites into a resident rollout buffer, then GAE with whole-batch "
                    "statistics",
        "value": steps * HORIZON * n / wall,
        "ms_per_step": wall / steps * 1e3,
        "steps": steps,
        "roofline": {"kernel": "env_step + pixel render (one rl_env_step: k_step, k_obs_pixels)", "bound": "hbm",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": load_traffic("env_step+pixels"), "bytes_per_launch": launch_bytes,
                     "avg_launch_us": env_avg_s * 1e6},
        "env_launch_us": launch_stats(env_ms),
        "gae_us_in_rollout": float(gae_ms.mean()) * 1e3,
    }


def launch_stats(per_launch_ms):
    """Mean, median and min over the timed rollouts of the average launch time (each rollout's loop of 128
    launches over 128), in microseconds."""
    a = np.asarray(per_launch_ms) * 1e3
    return {"mean": float(a.mean()), "median": float(np.median(a)), "min": float(a.min()), "max": float(a.max()),
            "rollouts": int(a.size)}


def cpu_info():
    """The host's CPU model and core counts (the oracle legs' machine)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = None
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "usable_cpus": usable, "oracle_workers": CPU_WORKERS}


def hbm_ceiling(torch, binding, dev, store_bytes, row_chunk, reps=9):
    """Same-run ceilings of plain HBM traffic, medians of `reps` timed launches: stores of `store_bytes`
    (the observation bytes of one env step) into successive slices of a 4 GiB buffer (so that no slice is
    still cached when it is written again) by torch's fill and by the library's store probe at several
    granularities (bytes one block writes before it exits: 4 KB, 16 KB, `row_chunk` = what one env-step
    block writes, and four times that), a 1 GiB device-to-device copy (read + write bytes counted), a 1 GiB
    sum (a reduction's read), and the library's read probe over 1 GiB at 4 KB, 64 KB and 1 MB per block."""
    slab = torch.empty(1 << 30, dtype=torch.float32, device=dev)
    n = store_bytes // 4
    nslices = (1 << 30) // n
    src, dst = slab[:1 << 28], slab[1 << 28:2 << 28]
    slab.zero_()
    torch.cuda.synchronize()

    def timed(fn):
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        z.record()
        torch.cuda.synchronize()
        return a.elapsed_time(z) * 1e-3

    store = [timed(lambda i=i: slab[(i % nslices) * n:(i % nslices + 1) * n].fill_(1.0)) for i in range(reps + 1)][1:]
    n16 = n // 4 * 4   # 16-byte multiple of the slice
    chunks = {}
    store_sizes = {"4KB": 4096, "16KB": 16384, "env_block": row_chunk, "4_env_blocks": 4 * row_chunk}
    for name, chunk in store_sizes.items():
        chunks[name] = [timed(lambda i=i: binding.store_probe(slab[(i % nslices) * n:(i % nslices) * n + n16], chunk))
                        for i in range(reps + 1)][1:]
    copy = [timed(lambda: dst.copy_(src)) for _ in range(reps + 1)][1:]
    read = [timed(lambda: src.sum()) for _ in range(reps + 1)][1:]
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    reads = {}
    read_sizes = {"4KB": 4096, "64KB": 1 << 16, "1MB": 1 << 20}
    for name, chunk in read_sizes.items():
        # successive 1 GiB quarters of the 4 GiB buffer, so that no read finds its bytes cached
        reads[name] = [timed(lambda i=i: binding.read_probe(slab[(i % 4) * (1 << 28):(i % 4 + 1) * (1 << 28)], chunk,
                                                             sink)) for i in range(reps + 1)][1:]
    del slab
    torch.cuda.empty_cache()
    gbs = lambda nbytes, ts: nbytes / float(np.median(ts)) / 1e9
    return {"store_GB/s": gbs(n * 4, store), "store_bytes": n * 4,
            "store_4KB_blocks_GB/s": gbs(n16 * 4, chunks["4KB"]),
            "store_env_block_GB/s": gbs(n16 * 4, chunks["env_block"]), "env_block_bytes": row_chunk,
            "copy_GB/s": gbs(2 * (1 << 30), copy), "sum_read_GB/s": gbs(1 << 30, read),
            "read_4KB_blocks_GB/s": gbs(1 << 30, reads["4KB"]), "read_1MB_blocks_GB/s": gbs(1 << 30, reads["1MB"]),
            "store_probe_sweep_GB/s": {f"{v}B": gbs(n16 * 4, chunks[k]) for k, v in store_sizes.items()},
            "read_probe_sweep_GB/s": {f"{v}B": gbs(1 << 30, reads[k]) for k, v in read_sizes.items()},
            "kernels": "torch fill_ (store), rl_store_probe (store_4KB_blocks, store_env_block), torch copy_, "
                       "torch sum, rl_read_probe (read_4KB_blocks, read_1MB_blocks)",
            "reps": reps, "peak_GB/s": HBM_PEAK_GBS}


def tiny_record(torch, binding, inputs, dev, steps, warmup):
    """The tiny workload (N = 64, T = 128, one 32 x 128 map): rollouts of 128 env steps into a resident buffer,
    then GAE with the deferred statistics. Launch-latency bound (64 envs fill one wave), so not an HBM test;
    per-rollout event pairs, median and min."""
    t, n = HORIZON, 64
    ms1 = inputs.make_mapset([1], 32, 128)
    env = binding.Env(ms1.maps, ms1.ckpts, ms1.spawns, n, frame_skip=3, time_limit=2000, device=dev)
    acts = torch.from_numpy(np.ascontiguousarray(inputs.make_actions(2, t, n), np.int32)).to(dev)
    values, last = inputs.make_values(3, t, n)
    values_d, last_d = torch.from_numpy(values).to(dev), torch.from_numpy(last).to(dev)
    obs = torch.empty((t, n, binding.OBS_TILES_SIZE), dtype=torch.float32, device=dev)
    rew = torch.empty((t, n), dtype=torch.float32, device=dev)
    dn = torch.empty_like(rew)
    adv, ret = torch.empty_like(rew), torch.empty_like(rew)
    stats = torch.zeros(binding.gae_stats_bytes(t, n) // 8, dtype=torch.float64, device=dev)
    env.reset(obs[0])
    times = []
    for k in range(warmup + steps):
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(t):
            env.step(acts[i], obs[i], rew[i], dn[i])
        binding.gae(rew, values_d, dn, last_d, GAMMA, LAMBDA, normalize=3, adv=adv, ret=ret, adv_stats=stats)
        z.record()
        torch.cuda.synchronize()
        if k >= warmup:
            times.append(a.elapsed_time(z))
    env.close()
    ms_ = np.array(times)
    return {"workload": "tiny: 64 envs x 128 steps on one seeded 32x128 map (seed 1), actions (2), values (3), "
                        "GAE with the deferred statistics; launch-latency bound, not an HBM test",
            "value": t * n / (float(np.median(ms_)) * 1e-3), "unit": "env-steps/s",
            "rollout_ms": {"median": float(np.median(ms_)), "min": float(ms_.min())},
            "us_per_env_step_launch": float(np.median(ms_)) * 1e3 / t, "steps": steps, "warmup": warmup}


def env_episodes_record(torch, binding, inputs, dev, ms):
    """The env-step workload as its own run: 65536 envs on the 64 bench maps, 16 warm-up steps then 1334 timed
    steps (two whole 667-decision episodes at the 2000-tick limit, so every env resets inside the timed span),
    each writing its observations into one resident [N][1397] block. One event pair around the 1334 launches."""
    warm, timed, n = 16, 1334, N_ENVS
    env = binding.Env(ms.maps, ms.ckpts, ms.spawns, n, frame_skip=3, time_limit=2000, device=dev)
    acts = torch.from_numpy(np.ascontiguousarray(inputs.make_actions(4, warm + timed, n), np.int32)).to(dev)
    obs = torch.empty((n, binding.OBS_TILES_SIZE), dtype=torch.float32, device=dev)
    rew = torch.empty((warm + timed, n), dtype=torch.float32, device=dev)
    dn = torch.empty_like(rew)
    env.reset(obs)
    for i in range(warm):
        env.step(acts[i], obs, rew[i], dn[i])
    a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for i in range(warm, warm + timed):
        env.step(acts[i], obs, rew[i], dn[i])
    z.record()
    torch.cuda.synchronize()
    ms_ = a.elapsed_time(z)
    ends = int(dn[warm:].sum().item())
    env.close()
    per_s = ms_ * 1e-3 / timed
    achieved = n * ENV_BYTES_PER_ENV_STEP / per_s / 1e9
    return {"workload": "env step: 65536 envs on 64 seeded 256x1024 maps, actions (seed 4), frame-skip 3, 2000-tick "
                        "limit, 16 warm-up + 1334 timed steps, obs f32[N][1397] rewritten each step",
            "value": timed * n / (ms_ * 1e-3), "unit": "env-steps/s", "ms": ms_, "avg_launch_us": per_s * 1e6,
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": achieved / HBM_PEAK_GBS},
            "episode_ends_in_timed_span": ends}


def config2_record(torch, binding, inputs, dev, reps):
    """The GAE+PPO workload (N = 2048, T = 128, 32 minibatches of 8192): rl_gae with statistics, and the loss
    normalised inline from the permutation and from minibatch numbers; medians of `reps` back-to-back
    launches. 5.2 MB + 18.9 MB stay in the caches: latency-bound, not an HBM test."""
    t, n, mb = 128, 2048, 8192
    b = t * n
    gi = inputs.make_gae_inputs(10, t, n)
    pi = inputs.make_policy_inputs(10, b)
    d = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    r, v, dn, vl = d(gi.rewards), d(gi.values), d(gi.dones), d(gi.last_values)
    logits, acts, old, nv, perm = d(pi.new_logits), d(pi.actions), d(pi.old_logp), d(pi.new_values), d(pi.perm)
    idx = d(inputs.minibatch_index(pi.perm, mb))
    adv = torch.empty((t, n), dtype=torch.float32, device=dev)
    ret = torch.empty_like(adv)
    stats = torch.zeros(binding.gae_stats_bytes(t, n) // 8, dtype=torch.float64, device=dev)   # deferred form
    out = torch.empty((b // mb, 4), dtype=torch.float32, device=dev)
    calls = {
        "gae": lambda: binding.gae(r, v, dn, vl, GAMMA, LAMBDA, normalize=3, adv=adv, ret=ret, adv_stats=stats),
        "loss_perm": lambda: binding.ppo_loss(logits, acts, old, adv.view(-1), ret.view(-1), nv, perm, mb,
                                              adv_stats=stats, out=out),
        "loss_stream": lambda: binding.ppo_loss(logits, acts, old, adv.view(-1), ret.view(-1), nv, None, mb,
                                                adv_stats=stats, out=out, mb_index=idx),
    }
    res = {"workload": "GAE+PPO: N=2048, T=128, minibatch 8192 (32 minibatches), perm seeded; cache-resident, "
                       "latency-bound (not an HBM test)"}
    nbytes = {"gae": b * GAE_BYTES_PER_ELEM + n * 4, "loss_perm": b * LOSS_BYTES_PER_SAMPLE["perm_placed"],
              "loss_stream": b * LOSS_BYTES_PER_SAMPLE["stream"]}
    for name, fn in calls.items():
        for _ in range(3):
            fn()
        ts = []
        for _ in range(reps):
            a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            z.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(z) * 1e-3)
        med = float(np.median(ts))
        res[name] = {"us": med * 1e6, "min_us": float(np.min(ts)) * 1e6, "GB/s": nbytes[name] / med / 1e9}
    return res


def cpu_baseline_pixels(ms, sprites, policy_actions, values, last_values, n):
    """The oracle, single-threaded, on the first n envs of the pixel workload: 128 steps with pixel
    observations, then GAE by its definition with normalisation. Returns env-steps/s."""
    import oracle
    t0 = time.perf_counter()
    env = oracle.OracleEnv(ms.maps, ms.ckpts, ms.spawns, n, sprites=sprites)
    env.reset()
    obs = np.empty((n, 4 * 84 * 84), np.uint8)
    rew = np.empty((HORIZON, n), np.float32)
    dn = np.empty((HORIZON, n), np.float32)
    for t in range(HORIZON):
        rew[t], dn[t] = env.step(policy_actions[t, :n])
        env.obs_pixels(obs)
    adv, _ = oracle.gae(rew, values[:, :n], dn, last_values[:n], float(np.float32(GAMMA)), float(np.float32(LAMBDA)))
    oracle.normalize(adv)
    dt = time.perf_counter() - t0
    return HORIZON * n / dt, dt


def _pix_shard(lo_hi):
    """Worker: the oracle's env step + pixel render for envs [lo, hi), then GAE over the shard."""
    import oracle
    lo, hi = lo_hi
    g = _SHARED
    n = hi - lo
    env = oracle.OracleEnv(g["ms"].maps, g["ms"].ckpts, g["ms"].spawns, n, sprites=g["sprites"], env_offset=lo)
    env.reset()
    obs = np.empty((n, 4 * 84 * 84), np.uint8)
    rew = np.empty((HORIZON, n), np.float32)
    dn = np.empty((HORIZON, n), np.float32)
    for t in range(HORIZON):
        rew[t], dn[t] = env.step(g["actions"][t, lo:hi])
        env.obs_pixels(obs)
    adv, _ = oracle.gae(rew, g["values"][:, lo:hi], dn, g["last_values"][lo:hi], float(np.float32(GAMMA)),
                        float(np.float32(LAMBDA)))
    return adv


def cpu_baseline_pixels_all_cores(ms, sprites, policy_actions, values, last_values, n, workers):
    """cpu_baseline_pixels' sample in `workers` forked processes of the single-threaded oracle."""
    import multiprocessing as mp

    import oracle
    _SHARED.update(ms=ms, sprites=sprites, actions=policy_actions, values=values, last_values=last_values)
    t0 = time.perf_counter()
    bounds = np.linspace(0, n, workers + 1).astype(int)
    with mp.get_context("fork").Pool(workers) as pool:
        parts = pool.map(_pix_shard, [(int(a), int(z)) for a, z in zip(bounds[:-1], bounds[1:])])
    oracle.normalize(np.concatenate(parts, axis=1))
    dt = time.perf_counter() - t0
    return HORIZON * n / dt, dt


def main_pixels(args):
    from resident_rl_rollout_amd import inputs

    n = PIX_ENVS
    ms = inputs.make_mapset(range(100, 100 + N_MAPS), MAP_H, MAP_W)
    sprites = inputs.make_sprites(30)
    policy_actions = inputs.make_actions(22, HORIZON, n)
    values, last_values = inputs.make_values(23, HORIZON, n)
    # CPU legs first: no fork after the GPU runtime is initialised
    cpu = cpu_all = None
    if not args.no_cpu_baseline:
        n_s = min(args.cpu_envs, n)
        rate, dt = cpu_baseline_pixels(ms, sprites, policy_actions, values, last_values, n_s)
        cpu = {"value": rate, "unit": "env-steps/s", "cores": 1, "kind": "oracle",
               "sample": f"first {n_s} of the 16384 envs x 128 steps (env step + 4 x 84 x 84 pixel render), GAE + "
                         f"normalisation over [128][{n_s}]; {dt:.1f} s single-threaded"}
        workers = min(CPU_WORKERS, os.cpu_count() or 1)
        rate, dt = cpu_baseline_pixels_all_cores(ms, sprites, policy_actions, values, last_values, n_s, workers)
        cpu_all = {"value": rate, "unit": "env-steps/s", "cores": workers, "kind": "oracle",
                   "sample": f"the same sample in {workers} processes of the single-threaded oracle (env shards); "
                             f"{dt:.1f} s wall"}

    import torch

    from resident_rl_rollout_amd import binding

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    binding.lib()
    if args.calibrate_copy:
        calibration_copy(torch, dev)
    rec = pixel_rollouts(torch, binding, dev, ms, sprites, policy_actions, values, last_values, args.steps,
                         args.warmup)
    out = {
        "metric": "env-steps/s incl. 84x84 u8 pixel obs write at 16384 envs",
        "value": rec["value"],
        "unit": "env-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i32+u8+f32",
        "data": "synthetic",
        "config": {"workload": rec["workload"], "num_envs": n, "horizon": HORIZON},
        "roofline": rec["roofline"],
        "env_launch_us": rec["env_launch_us"],
        "gae_us_in_rollout": rec["gae_us_in_rollout"],
        "cpu_baseline": cpu,
        "cpu_baseline_all_cores": cpu_all,
        "host": cpu_info(),
    }
    print(json.dumps(out), flush=True)


def cpu_baseline_infer(ms, enc, dec, pi, n_sample):
    """The oracle as it stands, single-threaded, on the first n_sample envs of the inference workload:
    per decision the stand-in inference on the env's observations, then the env step on its actions;
    the bootstrap inference, GAE over the inferred values with normalisation, and the loss over the
    sample's batch. Returns env-steps/s of the whole path."""
    import oracle
    n = n_sample
    t0 = time.perf_counter()
    env = oracle.OracleEnv(ms.maps, ms.ckpts, ms.spawns, n, **_env_kw())
    env.reset()
    obs = env.obs_tiles()
    rew = np.empty((HORIZON, n), np.float32)
    dn = np.empty((HORIZON, n), np.float32)
    val = np.empty((HORIZON, n), np.float32)
    act = np.empty((HORIZON, n), np.int32)
    logp = np.empty((HORIZON, n), np.float32)
    for t in range(HORIZON):
        out, act[t], logp[t] = oracle.policy_forward(obs, enc, dec, POLICY_SEED, t)
        val[t] = out[:, 12]
        rew[t], dn[t] = env.step(act[t])
        env.obs_tiles(obs)
    out, _, _ = oracle.policy_forward(obs, enc, dec, POLICY_SEED, HORIZON)
    adv, ret = oracle.gae(rew, val, dn, out[:, 12].astype(np.float32), float(np.float32(GAMMA)),
                          float(np.float32(LAMBDA)))
    na, _, _ = oracle.normalize(adv)
    b = HORIZON * n
    sel = (np.arange(HORIZON)[:, None] * N_ENVS + np.arange(n)[None, :]).reshape(-1)
    perm = np.random.default_rng(5).permutation(b).astype(np.int32)
    oracle.ppo_loss(pi.new_logits[sel], act.reshape(-1), logp.reshape(-1), na.reshape(-1), ret.reshape(-1),
                    pi.new_values[sel], perm, b // MINIBATCHES)
    dt = time.perf_counter() - t0
    return b / dt, dt


def main_infer(args):
    """Rollouts with the stand-in inference in the loop: per decision the inference on the last
    observations and the env step on its actions (rl_rollout), then a bootstrap inference, GAE over the
    inferred values and the loss with the rollout's actions and log-probabilities. Three schedules of the
    same work: single-buffered (one group of 65536 envs), double-buffered (two groups of 32768 on two
    streams), and double-buffered with the groups taking turns at the inference."""
    from resident_rl_rollout_amd import inputs

    n, T = N_ENVS, HORIZON
    ms = inputs.make_mapset(range(100, 100 + N_MAPS), MAP_H, MAP_W)
    enc, dec = inputs.make_policy_weights(POLICY_SEED)
    b = T * n
    pi = inputs.make_policy_inputs(20, b)
    cpu = None
    if not args.no_cpu_baseline:
        n_s = min(args.cpu_envs, n)
        rate, dt = cpu_baseline_infer(ms, enc, dec, pi, n_s)
        cpu = {"value": rate, "unit": "env-steps/s", "cores": 1, "kind": "oracle",
               "sample": f"first {n_s} of the 65536 envs x 128 decisions (stand-in inference + env step + tile obs), "
                         f"bootstrap inference, GAE + normalisation over [128][{n_s}], loss over the sample's "
                         f"{T * n_s} samples in 16 minibatches; {dt:.1f} s single-threaded"}

    import torch

    from resident_rl_rollout_amd import binding

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    binding.lib()
    pol = binding.Policy(enc, dec, seed=POLICY_SEED, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    obs = torch.empty((T, n, 1397), **f32)
    actions = torch.empty((T, n), dtype=torch.int32, device=dev)
    logp, values, rewards, dones = (torch.empty((T, n), **f32) for _ in range(4))
    obs0 = torch.empty((n, 1397), **f32)
    last_values = torch.empty(n, **f32)
    boot_act = torch.empty(n, dtype=torch.int32, device=dev)
    boot_logp = torch.empty(n, **f32)
    adv = torch.empty((T, n), **f32)
    ret = torch.empty_like(adv)
    stats = torch.zeros(binding.gae_stats_bytes(T, n) // 8, dtype=torch.float64, device=dev)   # deferred form
    loss_out = torch.empty((MINIBATCHES, 4), **f32)
    logits, new_v = (torch.from_numpy(x).to(dev) for x in (pi.new_logits, pi.new_values))
    mb_index = torch.from_numpy(inputs.minibatch_index(pi.perm, b // MINIBATCHES)).to(dev)
    main_stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    if args.calibrate_copy:
        calibration_copy(torch, dev)

    def schedule(groups, alternate):
        per = n // groups
        envs = [binding.Env(ms.maps, ms.ckpts, ms.spawns, per, frame_skip=3, time_limit=2000, device=dev)
                for _ in range(groups)]
        for g, e in enumerate(envs):
            e.reset(obs0[g * per:(g + 1) * per])
        streams = [torch.cuda.Stream(device=dev) for _ in range(groups)]
        torch.cuda.synchronize()

        def groups_from(start):
            out = []
            for g, e in enumerate(envs):
                sl = slice(g * per, (g + 1) * per)
                out.append(binding.rollout_group(e, start[sl], obs[:, sl], actions[:, sl], logp[:, sl], values[:, sl],
                                                 rewards[:, sl], dones[:, sl], env_offset=g * per, stream=streams[g]))
            return out
        first, later = groups_from(obs0), groups_from(obs[T - 1])
        state = {"k": 0}

        def rollout():
            grp = first if state["k"] == 0 else later
            for s_ in streams:                 # the previous loss has read the buffers this rollout rewrites
                s_.wait_stream(main_stream)
            binding.rollout(pol, grp, 0, T, alternate=alternate)
            for g, s_ in enumerate(streams):   # the bootstrap value of each group, on its own stream
                sl = slice(g * per, (g + 1) * per)
                pol.forward(obs[T - 1, sl], t=envs[g].step_counter, env_offset=g * per, actions=boot_act[sl],
                            logp=boot_logp[sl], values=last_values[sl], stream=s_)
            for s_ in streams:
                main_stream.wait_stream(s_)
            binding.gae(rewards, values, dones, last_values, GAMMA, LAMBDA, normalize=3, adv=adv, ret=ret,
                        adv_stats=stats)
            binding.ppo_loss(logits, actions.view(-1), logp.view(-1), adv.view(-1), ret.view(-1), new_v, None,
                             b // MINIBATCHES, adv_stats=stats, out=loss_out, mb_index=mb_index)
            state["k"] += 1

        for _ in range(args.warmup):
            rollout()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            rollout()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        for e in envs:
            e.close()
        return {"value": args.steps * T * n / wall, "ms_per_step": wall / args.steps * 1e3}

    results = {"single": schedule(1, False), "double": schedule(2, False), "alternate": schedule(2, True)}

    # the inference kernel alone over a resident observation block, after a read-only cache flush
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    flush.zero_()
    iso = []
    for rep in range(args.iso_reps):
        flush.sum()
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        pol.forward(obs[T // 2], t=rep, actions=boot_act, logp=boot_logp, values=last_values)
        z.record()
        torch.cuda.synchronize()
        iso.append(a.elapsed_time(z))
    del flush
    pol_s = float(np.median(iso)) * 1e-3
    launch_bytes = n * POLICY_BYTES_PER_ENV + POLICY_WEIGHT_BYTES
    achieved = launch_bytes / pol_s / 1e9
    chosen = results[args.schedule]
    out = {
        "metric": "env-steps/s of the whole rollout with the stand-in inference in the loop",
        "value": chosen["value"],
        "unit": "env-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": chosen["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i32+f32 env, bf16 x bf16 -> f32 encoder",
        "data": "synthetic",
        "config": {"workload": "inference rollout: 65536 envs x 128 decisions on 64 seeded 256x1024 maps; per "
                               "decision a stand-in policy (seeded encoder 1397 -> 128, decoder -> 12 logits + "
                               "value, Gumbel-max sampling) then the env step; bootstrap inference, GAE, loss in "
                               "16 minibatches",
                   "schedule": args.schedule, "num_envs": n, "horizon": T, "minibatches": MINIBATCHES},
        "schedules": {k: {"value": v["value"], "ms_per_step": v["ms_per_step"],
                          "vs_single": v["value"] / results["single"]["value"]} for k, v in results.items()},
        "roofline": {"kernel": "stand-in inference (rl_policy_forward: k_policy_forward) at 65536 envs", "bound": "hbm",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": load_traffic("policy_forward"), "bytes_per_launch": launch_bytes,
                     "avg_launch_us": pol_s * 1e6},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.cpu_envs is None:
        args.cpu_envs = {"pixels": 2048, "infer": 1024}.get(args.workload, 32768)   # 10-15 s single-threaded
    if args.workload == "pixels":
        return main_pixels(args)
    if args.workload == "infer":
        return main_infer(args)
    from resident_rl_rollout_amd import inputs

    # ---- seeded inputs (host) ----
    ms = inputs.make_mapset(range(100, 100 + N_MAPS), MAP_H, MAP_W)
    b = HORIZON * N_ENVS
    pi = inputs.make_policy_inputs(20, b)
    values, last_values = inputs.make_values(21, HORIZON, N_ENVS)
    policy_actions = pi.actions.reshape(HORIZON, N_ENVS)
    hook = args.hook == "grapple"
    aims = inputs.make_aims(22, HORIZON, N_ENVS) if hook else None

    # The CPU legs run before this process first touches the GPU: the all-core leg forks workers, and a
    # process whose GPU runtime is initialised must not fork them.
    cpu = cpu_all = None
    waypoints = args.reward == "waypoints"
    respawn = args.respawn == "adaptive"
    if not args.no_cpu_baseline:
        if waypoints:
            table, lens = oracle_waypoints(ms)
            _SHARED.update(reward_mode=1, waypoints=table, wp_lens=lens)
        if respawn:
            _SHARED.update(respawn_mode=1, ckpt_spawns=ms.ckpt_spawns, respawn_seed=RESPAWN_SEED)
        if hook:
            _SHARED.update(hook_mode=1, aims=aims)
        n_s = min(args.cpu_envs, N_ENVS)
        rate, dt = cpu_baseline(ms, policy_actions, values, last_values, pi, n_s)
        cpu = {"value": rate, "unit": "env-steps/s", "cores": 1, "kind": "oracle",
               "sample": f"first {n_s} of the 65536 envs x 128 steps (env step + tile obs), GAE + normalisation "
                         f"over [128][{n_s}], loss over the sample's {HORIZON * n_s} samples in 16 minibatches; "
                         f"{dt:.1f} s single-threaded"}
        workers = min(CPU_WORKERS, os.cpu_count() or 1)
        rate, dt = cpu_baseline_all_cores(ms, policy_actions, values, last_values, pi, n_s, workers)
        cpu_all = {"value": rate, "unit": "env-steps/s", "cores": workers, "kind": "oracle",
                   "sample": f"the same sample in {workers} processes of the single-threaded oracle: env shards, "
                             f"GAE per shard, one process per loss minibatch; {dt:.1f} s wall"}

    import torch

    from resident_rl_rollout_amd import binding

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    binding.lib()

    wp_kw = {}
    if waypoints:   # the library's host BFS: each map's tile path from the spawn to the finish
        table, lens = pad_paths([binding.waypoint_path(ms.maps[m], *path_ends(ms, m)) for m in range(N_MAPS)])
        wp_kw = dict(reward_mode=binding.REWARD_WAYPOINTS, waypoints=table, wp_lens=lens)
    if respawn:
        wp_kw.update(respawn_mode=binding.RESPAWN_ADAPTIVE, ckpt_spawns=ms.ckpt_spawns, respawn_seed=RESPAWN_SEED)
    if hook:
        wp_kw.update(hook_mode=binding.HOOK_GRAPPLE)
    env = binding.Env(ms.maps, ms.ckpts, ms.spawns, N_ENVS, frame_skip=3, time_limit=2000, device=dev, **wp_kw)
    aims_d = torch.from_numpy(aims).to(dev) if hook else None
    # rollout buffer: one allocation of [actions T*N | obs T*N*1397 | rewards T*N | dones T*N]
    a_bytes = HORIZON * N_ENVS * 4
    o_bytes = HORIZON * N_ENVS * 1397 * 4
    offs = [0, a_bytes, a_bytes + o_bytes, a_bytes + o_bytes + a_bytes]
    buf = torch.empty(offs[3] + a_bytes, dtype=torch.uint8, device=dev)
    actions = buf[offs[0]:offs[1]].view(torch.int32).view(HORIZON, N_ENVS)
    obs = buf[offs[1]:offs[2]].view(torch.float32).view(HORIZON, N_ENVS, 1397)
    rewards = buf[offs[2]:offs[3]].view(torch.float32).view(HORIZON, N_ENVS)
    dones = buf[offs[3]:].view(torch.float32).view(HORIZON, N_ENVS)
    actions.copy_(torch.from_numpy(policy_actions))
    t_ = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    logits, old_logp, new_v, perm = t_(pi.new_logits), t_(pi.old_logp), t_(pi.new_values), t_(pi.perm)
    mb_index = t_(inputs.minibatch_index(pi.perm, b // MINIBATCHES))
    values_d, last_d = t_(values), t_(last_values)
    adv = torch.empty((HORIZON, N_ENVS), dtype=torch.float32, device=dev)
    ret = torch.empty_like(adv)
    stats = torch.zeros(binding.gae_stats_bytes(HORIZON, N_ENVS) // 8, dtype=torch.float64, device=dev)   # deferred
    loss_out = torch.empty((MINIBATCHES, 4), dtype=torch.float32, device=dev)
    dlogits = torch.empty((b, 12), dtype=torch.float32, device=dev)
    log_rhos = torch.from_numpy(inputs.make_log_rhos(24, HORIZON, N_ENVS)).to(dev)
    vs_out = torch.empty((HORIZON, N_ENVS), dtype=torch.float32, device=dev)
    pgadv_out = torch.empty_like(vs_out)
    dvalues = torch.empty(b, dtype=torch.float32, device=dev)
    mb = b // MINIBATCHES
    env.reset(obs[0])
    torch.cuda.synchronize()
    if args.calibrate_copy:
        calibration_copy(torch, dev)

    def rollout(ev=None):
        # one event pair around the 128 back-to-back env launches: events between launches would add
        # their own barrier and timestamp packets to every step
        if ev is not None:
            ev["env"][0].record()
        for t in range(HORIZON):
            env.step(actions[t], obs[t], rewards[t], dones[t], aim=None if aims_d is None else aims_d[t])
        if ev is not None:
            ev["env"][1].record()
            ev["gae"][0].record()
        binding.gae(rewards, values_d, dones, last_d, GAMMA, LAMBDA, normalize=3, adv=adv, ret=ret, adv_stats=stats)
        if ev is not None:
            ev["gae"][1].record()
            ev["loss"][0].record()
        if args.loss_mode == "stream":
            binding.ppo_loss(logits, actions.view(-1), old_logp, adv.view(-1), ret.view(-1), new_v, None, mb,
                             adv_stats=stats, out=loss_out, mb_index=mb_index)
        else:
            binding.ppo_loss(logits, actions.view(-1), old_logp, adv.view(-1), ret.view(-1), new_v, perm, mb,
                             adv_stats=stats, out=loss_out)
        if ev is not None:
            ev["loss"][1].record()

    for _ in range(args.warmup):
        rollout()
    torch.cuda.synchronize()

    mk = lambda: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    events = [{"env": mk(), "gae": mk(), "loss": mk()} for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(args.steps):
        rollout(events[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start

    # GAE and loss alone: before each repetition a 1 GiB read evicts the 256 MB Infinity Cache without
    # leaving dirty lines behind (a write-based flush, or the rollout's observation writes, leaves up to
    # 256 MB to be written back during the next kernel).
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    flush.zero_()
    iso = {"gae": [], "scan": [], "loss": [], "perm": [], "grad": [], "vtrace": []}
    for rep in range(args.iso_reps):
        for which in ("gae", "scan", "loss", "perm", "grad", "vtrace"):
            flush.sum()
            a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            if which == "gae":   # scan + deferred statistics: what the rollout runs
                binding.gae(rewards, values_d, dones, last_d, GAMMA, LAMBDA, normalize=3, adv=adv, ret=ret,
                            adv_stats=stats)
            elif which == "scan":   # the scan kernel alone: no statistics, no second launch
                binding.gae(rewards, values_d, dones, last_d, GAMMA, LAMBDA, normalize=0, adv=adv, ret=ret)
            elif which == "vtrace":  # V-trace targets and advantages over the same [T][N] rollout
                binding.vtrace(rewards, values_d, dones, last_d, log_rhos, GAMMA, 1.0, vs=vs_out, pg_adv=pgadv_out)
            elif which == "grad":   # the loss with its per-sample gradient in the same pass (stream mode)
                binding.ppo_loss_grad(logits, actions.view(-1), old_logp, adv.view(-1), ret.view(-1), new_v, None,
                                      mb, adv_stats=stats, out=loss_out, dlogits=dlogits, dvalues=dvalues,
                                      mb_index=mb_index)
            elif which == "perm" or args.loss_mode == "perm":   # the boundary's permutation input
                binding.ppo_loss(logits, actions.view(-1), old_logp, adv.view(-1), ret.view(-1), new_v, perm, mb,
                                 adv_stats=stats, out=loss_out)
            else:
                binding.ppo_loss(logits, actions.view(-1), old_logp, adv.view(-1), ret.view(-1), new_v, None, mb,
                                 adv_stats=stats, out=loss_out, mb_index=mb_index)
            z.record()
            torch.cuda.synchronize()
            iso[which].append(a.elapsed_time(z))
    del flush

    # the same 128-launch env loop captured once in a HIP graph (torch's CUDAGraph) and replayed: the decision
    # counter lives on the device, so each replay continues the episodes
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=side):
        for t in range(HORIZON):
            env.step(actions[t], obs[t], rewards[t], dones[t], aim=None if aims_d is None else aims_d[t])
    graph.replay()
    torch.cuda.synchronize()
    g_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, z in g_ev:
        a.record()
        graph.replay()
        z.record()
    torch.cuda.synchronize()
    graph_ms = np.array([a.elapsed_time(z) for a, z in g_ev])
    del graph

    # one more loop of 128 env launches, each between its own event pair: the spread of single launches
    # (the packets of 256 events add about 2 us to each launch, so these read high against the loop's mean)
    per_launch = []
    for t in range(HORIZON):
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        env.step(actions[t], obs[t], rewards[t], dones[t], aim=None if aims_d is None else aims_d[t])
        z.record()
        per_launch.append((a, z))
    torch.cuda.synchronize()
    per_launch_us = np.array([a.elapsed_time(z) * 1e3 for a, z in per_launch])
    env.close()
    del buf, obs, actions, rewards, dones   # the rollout buffer (47 GB): the ceiling and the pixel run follow
    torch.cuda.empty_cache()
    ceiling = hbm_ceiling(torch, binding, dev, N_ENVS * 1397 * 4, 16 * 1397 * 4)
    cfg2 = config2_record(torch, binding, inputs, dev, args.iso_reps)
    cfg1 = tiny_record(torch, binding, inputs, dev, 20, 5)
    cfg3 = env_episodes_record(torch, binding, inputs, dev, ms)

    env_ms = np.array([ev["env"][0].elapsed_time(ev["env"][1]) / HORIZON for ev in events])   # per launch
    gae_ms = np.array([ev["gae"][0].elapsed_time(ev["gae"][1]) for ev in events])
    loss_ms = np.array([ev["loss"][0].elapsed_time(ev["loss"][1]) for ev in events])
    env_steps = args.steps * HORIZON * N_ENVS
    value = env_steps / wall

    env_launch_bytes = N_ENVS * (ENV_BYTES_PER_ENV_STEP + (ENV_BYTES_WAYPOINTS if waypoints else 0)
                                 + (ENV_BYTES_RESPAWN if respawn else 0) + (ENV_BYTES_HOOK if hook else 0))
    env_key = ("env_step+obs_gather" + ("+waypoints" if waypoints else "") + ("+respawn" if respawn else "")
               + ("+hook" if hook else ""))
    env_avg_s = float(env_ms.mean()) * 1e-3
    achieved = env_launch_bytes / env_avg_s / 1e9
    gae_bytes = b * GAE_BYTES_PER_ELEM + N_ENVS * 4
    loss_bytes = b * LOSS_BYTES_PER_SAMPLE[args.loss_mode]
    gae_s, loss_s = float(np.median(iso["gae"])) * 1e-3, float(np.median(iso["loss"])) * 1e-3
    perm_s = float(np.median(iso["perm"])) * 1e-3
    perm_bytes = b * LOSS_BYTES_PER_SAMPLE["perm"]
    stream_s = loss_s if args.loss_mode == "stream" else None
    scan_s = float(np.median(iso["scan"])) * 1e-3
    grad_s = float(np.median(iso["grad"])) * 1e-3
    vt_s = float(np.median(iso["vtrace"])) * 1e-3
    vt_bytes = b * VTRACE_BYTES_PER_ELEM + N_ENVS * 4
    vt_gbs = vt_bytes / vt_s / 1e9
    grad_bytes = b * (LOSS_BYTES_PER_SAMPLE["stream"] + GRAD_BYTES_PER_SAMPLE)
    grad_gbs = grad_bytes / grad_s / 1e9
    scan_gbs = gae_bytes / scan_s / 1e9
    gae_gbs = gae_bytes / gae_s / 1e9
    loss_gbs = loss_bytes / loss_s / 1e9
    gl_gbs = (gae_bytes + loss_bytes) / (gae_s + loss_s) / 1e9

    out = {
        "metric": "env-steps/s incl. obs write at 65536 envs; GAE+loss GB/s vs HBM peak",
        "value": value,
        "unit": "env-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i32+f32",
        "data": "synthetic",
        "config": {"workload": "full rollout: 65536 envs x 128 steps on 64 seeded 256x1024 maps, frame-skip 3, "
                               "tile obs (31x43 + 4x15 + 4) into a resident rollout buffer, GAE + whole-batch "
                               "normalisation, PPO loss over 16 shuffled minibatches of 524288"
                               + (", waypoint-path reward" if waypoints else "")
                               + (", adaptive checkpoint respawn" if respawn else "")
                               + (", grapple hook with seeded continuous aims" if hook else ""),
                   "num_envs": N_ENVS, "horizon": HORIZON, "minibatches": MINIBATCHES,
                   "loss_mode": args.loss_mode, "normalisation": "partial statistics in GAE (deferred), reduced and applied inside the loss",
                   "reward": args.reward, "respawn": args.respawn, "hook": args.hook},
        "roofline": {"kernel": "env_step+obs_gather (one rl_env_step)", "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": load_traffic(env_key),
                     "bytes_per_launch": env_launch_bytes, "avg_launch_us": env_avg_s * 1e6,
                     "frac_of_store_ceiling": achieved / ceiling["store_GB/s"],
                     "frac_of_env_block_store_ceiling": achieved / ceiling["store_env_block_GB/s"],
                     "frac_of_copy_ceiling": achieved / ceiling["copy_GB/s"]},
        "hbm_ceiling": ceiling,
        "env_step_us": float(env_ms.mean()) * 1e3,
        "env_launch_us": launch_stats(env_ms),
        "env_loop_128_ms": {"uncaptured_mean": float(env_ms.mean()) * HORIZON,
                            "captured_graph_median": float(np.median(graph_ms)),
                            "captured_graph_min": float(graph_ms.min()), "replays": int(graph_ms.size)},
        "env_launch_us_one_event_pair_each": {"median": float(np.median(per_launch_us)),
                                              "min": float(per_launch_us.min()), "max": float(per_launch_us.max()),
                                              "launches": int(per_launch_us.size)},
        "gae": {"us": gae_s * 1e6, "min_us": float(np.min(iso["gae"])) * 1e3, "GB/s": gae_gbs,
                "frac": gae_gbs / HBM_PEAK_GBS, "bytes": gae_bytes,
                "us_in_rollout": float(gae_ms.mean()) * 1e3, "scan_us": scan_s * 1e6,
                "scan_min_us": float(np.min(iso["scan"])) * 1e3, "scan_GB/s": scan_gbs,
                "scan_frac": scan_gbs / HBM_PEAK_GBS, "scan_frac_of_copy_ceiling": scan_gbs / ceiling["copy_GB/s"],
                "scan_traffic": load_traffic("gae_scan")},
        "loss": {"us": loss_s * 1e6, "min_us": float(np.min(iso["loss"])) * 1e3, "GB/s": loss_gbs,
                 "frac": loss_gbs / HBM_PEAK_GBS, "bytes": loss_bytes,
                 "frac_of_read_ceiling": loss_gbs / ceiling["read_1MB_blocks_GB/s"],
                 "us_in_rollout": float(loss_ms.mean()) * 1e3,
                 "traffic": load_traffic("ppo_loss") if args.loss_mode == "stream" else None},
        "loss_perm": {"us": perm_s * 1e6, "min_us": float(np.min(iso["perm"])) * 1e3, "GB/s": perm_bytes / perm_s / 1e9,
                      "frac": perm_bytes / perm_s / 1e9 / HBM_PEAK_GBS, "bytes": perm_bytes,
                      "vs_minibatch_numbers": None if stream_s is None else perm_s / stream_s,
                      # the sort and the stream pass that places its own bins, from the counter runs
                      "traffic": (lambda a, c: None if a is None or c is None else a + c)(
                          load_traffic("ppo_loss_perm_sort"), load_traffic("ppo_loss_perm_stream"))},
        "loss_grad": {"us": grad_s * 1e6, "GB/s": grad_gbs, "frac": grad_gbs / HBM_PEAK_GBS, "bytes": grad_bytes,
                      "traffic": load_traffic("ppo_loss_grad")},
        "vtrace": {"us": vt_s * 1e6, "GB/s": vt_gbs, "frac": vt_gbs / HBM_PEAK_GBS, "bytes": vt_bytes,
                   "traffic": load_traffic("vtrace")},
        "gae_loss_GB/s": gl_gbs,
        "gae_loss_frac": gl_gbs / HBM_PEAK_GBS,
        "loss_check": loss_out[0].tolist(),
        "cpu_baseline": cpu,
        "cpu_baseline_all_cores": cpu_all,
        "host": cpu_info(),
        "gae_ppo_n2048": cfg2,
        "tiny_n64": cfg1,
        "env_n65536_1334_steps": cfg3,
    }
    if not args.no_pixels:   # the pixel workload's own rate beside the headline (a short run of it)
        pix_actions = inputs.make_actions(22, HORIZON, PIX_ENVS)
        pix_values, pix_last = inputs.make_values(23, HORIZON, PIX_ENVS)
        out["pixels_n16384"] = pixel_rollouts(torch, binding, dev, ms, inputs.make_sprites(30), pix_actions,
                                              pix_values, pix_last, 3, 1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
