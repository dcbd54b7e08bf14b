"""GPU parity of the stand-in inference (rl_policy_forward) and of the rollout driver (rl_rollout) against
the oracle, and equality of the double-buffered rollout (two env groups on two streams) with the
single-buffered one.

Tolerances follow from the arithmetic. The kernel sums the encoder's 1397 bfloat16 products in float32,
so a hidden unit is within K u = 1397 * 2^-24 (about 8.3e-5) of sum |x_k w_hk|, and an output within
1e-4 of out_abs = sum_h |hidden|_h |d_jh| (the decoder's own rounding is another 128 u). The Gumbel
variates come from float32 log1p / log (a few ulp). Where those bounds leave two logits' scores closer
than their combined error, either choice is correct: the test checks that the kernel's action is then
one whose oracle score lies within that error of the best, and that it matches exactly elsewhere.
Values and log-probabilities are compared within the same bounds, log-probabilities at the kernel's
action. Env outputs (observations, rewards, dones) are bit-exact: the oracle env is driven with the
kernel's actions once they have been checked.
"""
import numpy as np
import pytest
import torch

import oracle
from resident_rl_rollout_amd import binding, inputs

pytestmark = pytest.mark.gpu

OBS = 1397
A = 12


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def check_policy(obs, enc, dec, seed, t, env_offset, actions, logp, values, what):
    """Checks kernel outputs for rows obs [n][>= 1397] against the oracle, within the bounds above."""
    obs = np.asarray(obs, np.float32)
    out, act_o, logp_o = oracle.policy_forward(obs, enc, dec, seed, t, env_offset)
    hid_abs = np.abs(_bf16(obs[:, :OBS])) @ np.abs(_bf16(enc)).T
    out_abs = hid_abs @ np.abs(dec.astype(np.float64)).T
    tol = 1e-4 * out_abs + 1e-6
    g = np.array([[oracle.policy_gumbel(seed, t, env_offset + e, j)[0] for j in range(A)] for e in range(len(obs))])
    score = out[:, :A] + g
    err = tol[:, :A] + 1e-6 * (1.0 + np.abs(g))
    a = np.asarray(actions).astype(np.int64)
    rows = np.arange(len(obs))
    best = score.max(axis=1)
    assert ((a >= 0) & (a < A)).all(), what
    valid = score[rows, a] >= best - (err[rows, a] + err[rows, act_o])
    assert valid.all(), f"{what}: {int((~valid).sum())} actions outside the scores' error"
    exact = (a == act_o)
    if len(obs) >= 1000:                                    # near ties are rare
        assert exact.mean() > 0.99, f"{what}: only {exact.mean():.4f} of actions equal the oracle's"
    lse = np.log(np.exp(out[:, :A] - out[:, :A].max(1, keepdims=True)).sum(1)) + out[:, :A].max(1)
    lp_want = out[rows, a] - lse
    lp_tol = 2 * tol[:, :A].max(axis=1) + 1e-6 * (1 + np.abs(lp_want))
    assert (np.abs(np.asarray(logp, np.float64) - lp_want) <= lp_tol).all(), f"{what}: logp"
    assert (np.abs(np.asarray(values, np.float64) - out[:, A]) <= tol[:, A] + 1e-7).all(), f"{what}: values"
    return int((~exact).sum())


@pytest.mark.parametrize("n,stride,offset", [(1, OBS, 0), (63, OBS, 5), (64, OBS, 0), (65, 1400, 1000),
                                             (1000, OBS, 0), (4113, 1408, 77)])
def test_forward_matches_oracle_on_random_observations(gpu_lib, n, stride, offset):
    rng = np.random.default_rng(n + stride)
    obs = (rng.standard_normal((n, stride)) * 3).astype(np.float32)
    obs[:, :1333] = rng.integers(0, 4, (n, 1333))        # window cells are small tile codes
    enc, dec = inputs.make_policy_weights(n, enc_std=0.02)
    pol = binding.Policy(enc, dec, seed=99)
    a, lp, v = pol.forward(torch.from_numpy(obs).cuda(), t=3, env_offset=offset)
    check_policy(obs, enc, dec, 99, 3, offset, a.cpu().numpy(), lp.cpu().numpy(), v.cpu().numpy(),
                 f"n={n} stride={stride} offset={offset}")


def test_wide_launches_equal_narrow_ones_and_the_oracle(gpu_lib):
    # 65536 envs and more take 128-env blocks, smaller launches 64-env blocks: per-env results are the same
    n = 65536 + 77
    gen = torch.Generator(device="cuda").manual_seed(3)
    obs = torch.randint(0, 4, (n, OBS), generator=gen, device="cuda").float()
    obs[:, 1333:] = torch.randn((n, OBS - 1333), generator=gen, device="cuda") * 20
    enc, dec = inputs.make_policy_weights(12)
    pol = binding.Policy(enc, dec, seed=8)
    a, lp, v = pol.forward(obs, t=5)
    parts = [pol.forward(obs[lo:hi], t=5, env_offset=lo) for lo, hi in ((0, 40000), (40000, n))]
    for got, want in zip((a, lp, v), (torch.cat([p_[k] for p_ in parts]) for k in range(3))):
        assert torch.equal(got, want)
    # against the oracle: the first two blocks, the ragged last block, and single rows in between
    segments = [(0, 130), (n - 200, n)] + [(int(r), int(r) + 1) for r in np.random.default_rng(0).choice(n - 200, 40)]
    for lo, hi in segments:
        check_policy(obs[lo:hi].cpu().numpy(), enc, dec, 8, 5, lo, a[lo:hi].cpu().numpy(), lp[lo:hi].cpu().numpy(),
                     v[lo:hi].cpu().numpy(), f"rows {lo}..{hi}")


def test_forward_reads_exactly_the_observation_row(gpu_lib):
    # a padded stride with poison past element 1397 and a last row at the very end of its allocation
    n, stride = 130, 1400
    rng = np.random.default_rng(7)
    obs = rng.standard_normal((n, stride)).astype(np.float32)
    obs[:, OBS:] = 1e30
    enc, dec = inputs.make_policy_weights(3)
    pol = binding.Policy(enc, dec, seed=1)
    d = torch.from_numpy(obs).cuda()
    a, lp, v = pol.forward(d, t=0)
    assert torch.isfinite(lp).all() and torch.isfinite(v).all()
    check_policy(obs, enc, dec, 1, 0, 0, a.cpu().numpy(), lp.cpu().numpy(), v.cpu().numpy(), "padded stride")
    tail = torch.from_numpy(obs[:, :OBS].copy()).cuda()      # stride 1397: the last row ends the buffer
    a2, lp2, v2 = pol.forward(tail, t=0)
    assert torch.equal(a, a2) and torch.equal(lp, lp2) and torch.equal(v, v2)


def test_one_hot_weights_give_the_rounded_observation(gpu_lib):
    # decoder output j = hidden j = bf16(obs[k_j]) exactly (one product per sum), value = bf16(obs[k_12])
    cols = [0, 5, 100, 1332, 1333, 1392, 1396, 7, 8, 9, 10, 11, 1395]
    enc = np.zeros((128, OBS), np.float32)
    enc[np.arange(13), cols] = 1.0
    dec = np.zeros((13, 128), np.float32)
    dec[np.arange(13), np.arange(13)] = 1.0
    rng = np.random.default_rng(2)
    obs = (rng.standard_normal((200, OBS)) * np.exp(rng.uniform(-8, 8, (200, 1)))).astype(np.float32)
    pol = binding.Policy(enc, dec, seed=4)
    a, lp, v = pol.forward(torch.from_numpy(obs).cuda(), t=1)
    np.testing.assert_array_equal(v.cpu().numpy().astype(np.float64), _bf16(obs[:, 1395]))
    check_policy(obs, enc, dec, 4, 1, 0, a.cpu().numpy(), lp.cpu().numpy(), v.cpu().numpy(), "one-hot")


def test_sampled_actions_follow_the_softmax(gpu_lib):
    from scipy import stats
    from scipy.special import softmax
    logits = np.array([2.0, -1.0, 0.5, 0.0, -3.0, 1.5, 0.25, -0.5, 1.0, -2.0, 0.75, 3.0], np.float32)
    n = 1 << 18
    obs = torch.zeros((n, OBS), dtype=torch.float32, device="cuda")
    obs[:, 0] = 1.0
    enc = np.zeros((128, OBS), np.float32)
    enc[0, 0] = 1.0
    dec = np.zeros((13, 128), np.float32)
    dec[:12, 0] = logits
    pol = binding.Policy(enc, dec, seed=2024)
    a, lp, _ = pol.forward(obs, t=11)
    counts = np.bincount(a.cpu().numpy(), minlength=A)
    assert stats.chisquare(counts, softmax(logits.astype(np.float64)) * n).pvalue > 1e-4
    want = logits.astype(np.float64)[a.cpu().numpy()] - np.log(np.exp(logits.astype(np.float64)).sum())
    np.testing.assert_allclose(lp.cpu().numpy(), want, rtol=0, atol=5e-6)


def _mapset():
    return inputs.make_mapset(range(40, 44), 48, 192)


def _buffers(n, t):
    f = dict(dtype=torch.float32, device="cuda")
    return dict(obs=torch.empty((t, n, OBS), **f), actions=torch.empty((t, n), dtype=torch.int32, device="cuda"),
                logp=torch.empty((t, n), **f), values=torch.empty((t, n), **f), rewards=torch.empty((t, n), **f),
                dones=torch.empty((t, n), **f))


def _run(policy, ms, n, t, groups, alternate, time_limit=21, splits=None):
    """A rollout of t decisions over n envs split into `groups` equal groups (one stream each)."""
    per = n // groups
    envs = [binding.Env(ms.maps, ms.ckpts, ms.spawns, per, time_limit=time_limit) for _ in range(groups)]
    obs0 = torch.empty((n, OBS), dtype=torch.float32, device="cuda")
    for g, e in enumerate(envs):
        e.reset(obs0[g * per:(g + 1) * per])
    b = _buffers(n, t)
    streams = [torch.cuda.Stream() for _ in range(groups)]
    torch.cuda.synchronize()
    grp = []
    for g, e in enumerate(envs):
        sl = slice(g * per, (g + 1) * per)
        grp.append(binding.rollout_group(e, obs0[sl], b["obs"][:, sl], b["actions"][:, sl], b["logp"][:, sl],
                                         b["values"][:, sl], b["rewards"][:, sl], b["dones"][:, sl],
                                         env_offset=g * per, stream=streams[g]))
    for t0, steps in (splits or [(0, t)]):
        binding.rollout(policy, grp, t0, steps, alternate=alternate)
    torch.cuda.synchronize()
    b["obs0"] = obs0
    return b


def test_rollout_matches_the_oracle(gpu_lib):
    ms = _mapset()
    n, t = 256, 12
    enc, dec = inputs.make_policy_weights(5)
    pol = binding.Policy(enc, dec, seed=77)
    b = _run(pol, ms, n, t, 1, False)
    ora = oracle.OracleEnv(ms.maps, ms.ckpts, ms.spawns, n, time_limit=21)
    ora.reset()
    prev = ora.obs_tiles()
    np.testing.assert_array_equal(b["obs0"].cpu().numpy(), prev)
    near_ties = 0
    for s in range(t):
        act = b["actions"][s].cpu().numpy()
        near_ties += check_policy(prev, enc, dec, 77, s, 0, act, b["logp"][s].cpu().numpy(),
                                  b["values"][s].cpu().numpy(), f"decision {s}")
        r, d = ora.step(act)
        np.testing.assert_array_equal(b["rewards"][s].cpu().numpy(), r)
        np.testing.assert_array_equal(b["dones"][s].cpu().numpy(), d)
        prev = ora.obs_tiles()
        np.testing.assert_array_equal(b["obs"][s].cpu().numpy(), prev, err_msg=f"decision {s}")
    assert b["dones"].sum() > 0                             # the 21-tick limit ends episodes mid-rollout


@pytest.mark.parametrize("groups,alternate", [(2, True), (2, False), (4, True)])
def test_double_buffered_equals_single_buffered(gpu_lib, groups, alternate):
    ms = _mapset()
    n, t = 512, 10
    enc, dec = inputs.make_policy_weights(6)
    pol = binding.Policy(enc, dec, seed=5)
    one = _run(pol, ms, n, t, 1, False)
    many = _run(pol, ms, n, t, groups, alternate)
    for k in one:
        assert torch.equal(one[k], many[k]), f"{groups} groups, alternate={alternate}: {k} differs"


def test_double_buffered_at_the_bench_size(gpu_lib):
    # 65536 envs on the bench's map set for 3 decisions: the single-buffered rollout takes the 128-env
    # inference blocks, the two 32768-env groups the 64-env blocks; every buffer must agree bit for bit
    ms = inputs.make_mapset(range(100, 164), 256, 1024)
    enc, dec = inputs.make_policy_weights(31)
    pol = binding.Policy(enc, dec, seed=31)
    one = _run(pol, ms, 65536, 3, 1, False, time_limit=2000)
    two = _run(pol, ms, 65536, 3, 2, False, time_limit=2000)
    for k in one:
        assert torch.equal(one[k], two[k]), k
    # the first decision's inference against the oracle on the first and last 128 envs
    for lo in (0, 65536 - 128):
        sl = slice(lo, lo + 128)
        check_policy(one["obs0"][sl].cpu().numpy(), enc, dec, 31, 0, lo, one["actions"][0, sl].cpu().numpy(),
                     one["logp"][0, sl].cpu().numpy(), one["values"][0, sl].cpu().numpy(), f"envs {lo}..")


def test_rollout_resumes_across_calls(gpu_lib):
    ms = _mapset()
    n, t = 192, 9
    enc, dec = inputs.make_policy_weights(8)
    pol = binding.Policy(enc, dec, seed=6)
    whole = _run(pol, ms, n, t, 2, True)
    parts = _run(pol, ms, n, t, 2, True, splits=[(0, 4), (4, 0), (4, 5)])
    for k in whole:
        assert torch.equal(whole[k], parts[k]), k


def test_rollout_rejects_mismatched_groups(gpu_lib):
    ms = _mapset()
    enc, dec = inputs.make_policy_weights(9)
    pol = binding.Policy(enc, dec)
    e1 = binding.Env(ms.maps, ms.ckpts, ms.spawns, 64)
    e2 = binding.Env(ms.maps, ms.ckpts, ms.spawns, 64)
    b = _buffers(128, 2)
    obs0 = torch.zeros((128, OBS), dtype=torch.float32, device="cuda")
    e2.step(torch.zeros(64, dtype=torch.int32, device="cuda"), b["obs"][0, 64:], b["rewards"][0, 64:],
            b["dones"][0, 64:])                                # e2 is one decision ahead
    torch.cuda.synchronize()
    g = [binding.rollout_group(e, obs0[i * 64:(i + 1) * 64], b["obs"][:, i * 64:(i + 1) * 64],
                               b["actions"][:, i * 64:(i + 1) * 64], b["logp"][:, i * 64:(i + 1) * 64],
                               b["values"][:, i * 64:(i + 1) * 64], b["rewards"][:, i * 64:(i + 1) * 64],
                               b["dones"][:, i * 64:(i + 1) * 64], env_offset=64 * i) for i, e in enumerate((e1, e2))]
    with pytest.raises(binding.RLError, match="decision counter"):
        binding.rollout(pol, g, 0, 1)
    bad = binding.rollout_group(e1, obs0[:64], b["obs"][:, :64], b["actions"][:, :64], b["logp"][:, :64],
                                b["values"][:, :64], b["rewards"][:, :64], b["dones"][:, :64])
    bad.logp = bad.logp + 2                                   # misaligned: refused before anything is enqueued
    with pytest.raises(binding.RLError, match="4-byte aligned"):
        binding.rollout(pol, [bad], 0, 1)
    pix = binding.Env(ms.maps, ms.ckpts, ms.spawns, 64, obs_mode=binding.OBS_PIXELS, sprites=inputs.make_sprites())
    gp = binding.RolloutGroup()
    gp.env = pix._handle
    with pytest.raises(binding.RLError, match="tile observations"):
        binding.rollout(pol, [gp], 0, 1)
