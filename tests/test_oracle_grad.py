"""Pins of the oracle's PPO loss gradient, each independent of the formula the oracle writes out:

- central finite differences of the oracle's own loss forward (a different computation: no derivative
  is formed);
- reverse-mode autograd of the same loss written with torch operations in float64 on the CPU (the pages'
  own test method for a fused loss gradient: "Teaching Mario to speedrun", section 8, checks every
  gradient against an autograd implementation);
- a hand-worked two-action example, and invariants (rows of the logits gradient sum to zero, uniform
  logits carry no entropy gradient, a clipped sample keeps only the entropy part).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from resident_rl_rollout_amd import inputs

EPS, VF, ENT = 0.2, 0.5, 0.01


def _case(seed, b, a=12):
    pi = inputs.make_policy_inputs(seed, b, a)
    rng = np.random.default_rng(seed + 1)
    adv = rng.standard_normal(b)
    ret = rng.standard_normal(b)
    return pi, adv, ret


def _total(pi, logits, nv, adv, ret, mb, m):
    out, _ = oracle.ppo_loss(logits, pi.actions, pi.old_logp, adv, ret, nv, pi.perm, mb)
    return out[m, 3]


def test_hand_worked_two_actions():
    # z = (0, 0), action 0, old prob 1/2: ratio 1, p = (1/2, 1/2), H = ln 2, A = 1, one sample
    # dL/dz0 = -A r (1 - 1/2) + 0.01 * 1/2 * (ln 1/2 + ln 2) = -1/2; dL/dz1 = -A r (0 - 1/2) = +1/2
    # dL/dV = 0.5 * 2 * (V - R) with V = 1, R = 0: 1
    g = oracle.ppo_loss_grad(np.zeros((1, 2)), np.array([0], np.int32), np.array([math.log(0.5)]), np.array([1.0]),
                             np.array([0.0]), np.array([1.0]), None, 1)
    np.testing.assert_allclose(g.dlogits, [[-0.5, 0.5]], rtol=0, atol=1e-15)
    assert g.dvalues[0] == pytest.approx(1.0, rel=1e-15)
    assert g.ratio[0] == pytest.approx(1.0, rel=1e-15)


def test_matches_finite_differences_of_the_loss():
    b, mb, a = 48, 12, 12
    pi, adv, ret = _case(3, b, a)
    logits = pi.new_logits.astype(np.float64)
    nv = pi.new_values.astype(np.float64)
    g = oracle.ppo_loss_grad(logits, pi.actions, pi.old_logp, adv, ret, nv, pi.perm, mb)
    where = np.empty(b, np.int64)                     # minibatch of each sample
    where[pi.perm] = np.arange(b) // mb
    h = 1e-5
    checked = 0
    for i in range(b):
        if min(abs(g.ratio[i] - (1 + EPS)), abs(g.ratio[i] - (1 - EPS))) < 1e-2:
            continue                                  # the loss has a kink at the band edges
        m = where[i]
        for j in range(a):
            zp, zm = logits.copy(), logits.copy()
            zp[i, j] += h
            zm[i, j] -= h
            fd = (_total(pi, zp, nv, adv, ret, mb, m) - _total(pi, zm, nv, adv, ret, mb, m)) / (2 * h)
            assert abs(fd - g.dlogits[i, j]) < 1e-8, (i, j, fd, g.dlogits[i, j])
        vp, vm = nv.copy(), nv.copy()
        vp[i] += h
        vm[i] -= h
        fd = (_total(pi, logits, vp, adv, ret, mb, m) - _total(pi, logits, vm, adv, ret, mb, m)) / (2 * h)
        assert abs(fd - g.dvalues[i]) < 1e-8
        checked += 1
    assert checked > b // 2
    # a sample of another minibatch does not move this minibatch's loss
    i = int(pi.perm[0])
    other = int(pi.perm[mb])
    zp = logits.copy()
    zp[other, 0] += 1.0
    assert _total(pi, zp, nv, adv, ret, mb, where[i]) == _total(pi, logits, nv, adv, ret, mb, where[i])


@pytest.mark.parametrize("b,mb,a,use_perm", [(96, 32, 12, True), (40, 8, 5, True), (30, 30, 3, False),
                                             (64, 16, 12, False)])
def test_matches_autograd(b, mb, a, use_perm):
    pi, adv, ret = _case(b + a, b, a)
    perm = pi.perm if use_perm else None
    g = oracle.ppo_loss_grad(pi.new_logits, pi.actions, pi.old_logp, adv, ret, pi.new_values, perm, mb)

    z = torch.tensor(pi.new_logits, dtype=torch.float64, requires_grad=True)
    v = torch.tensor(pi.new_values, dtype=torch.float64, requires_grad=True)
    order = torch.as_tensor(perm if use_perm else np.arange(b), dtype=torch.long)
    act = torch.as_tensor(pi.actions, dtype=torch.long)
    old = torch.tensor(pi.old_logp, dtype=torch.float64)
    A_ = torch.tensor(adv)
    R_ = torch.tensor(ret)
    logp_all = torch.log_softmax(z, dim=1)
    logp = logp_all.gather(1, act[:, None])[:, 0]
    ratio = torch.exp(logp - old)
    pg = -torch.minimum(ratio * A_, torch.clamp(ratio, 1 - EPS, 1 + EPS) * A_)
    ent = -(logp_all.exp() * logp_all).sum(1)
    vl = (v - R_) ** 2
    total = 0
    for m in range(b // mb):
        idx = order[m * mb:(m + 1) * mb]
        total = total + pg[idx].mean() + VF * vl[idx].mean() - ENT * ent[idx].mean()
    total.backward()
    np.testing.assert_allclose(g.dlogits, z.grad.numpy(), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(g.dvalues, v.grad.numpy(), rtol=1e-12, atol=1e-15)


def test_invariants():
    b, mb = 256, 64
    pi, adv, ret = _case(11, b)
    g = oracle.ppo_loss_grad(pi.new_logits, pi.actions, pi.old_logp, adv, ret, pi.new_values, pi.perm, mb)
    # softmax is unchanged by a constant added to a row, so every row of the gradient sums to zero
    assert np.abs(g.dlogits.sum(1)).max() < 1e-15
    # the surrogate's part is zero exactly on the clipped side of the band
    clipped_side = np.where(adv > 0, g.ratio > 1 + EPS, g.ratio < 1 - EPS)
    assert clipped_side.any() and (~clipped_side).any()
    g0 = oracle.ppo_loss_grad(pi.new_logits, pi.actions, pi.old_logp, np.zeros(b), ret, pi.new_values, pi.perm, mb)
    np.testing.assert_allclose(g.dlogits[clipped_side], g0.dlogits[clipped_side], rtol=0, atol=1e-17)
    np.testing.assert_allclose(g.dlogits[~clipped_side], (g0.dlogits + g.dpg)[~clipped_side], rtol=1e-13, atol=1e-17)
    # value gradient is 2 vf (V - R) / mb exactly
    np.testing.assert_allclose(g.dvalues, 2 * VF * (pi.new_values.astype(np.float64) - ret) / mb, rtol=1e-15)


def test_uniform_logits_have_no_entropy_gradient():
    b = 24
    logits = np.zeros((b, 12))
    actions = (np.arange(b) % 12).astype(np.int32)
    old = np.full(b, -math.log(12.0))                       # ratio 1: every sample on the unclipped branch
    g = oracle.ppo_loss_grad(logits, actions, old, np.zeros(b), np.zeros(b), np.zeros(b), None, b)
    assert np.abs(g.dlogits).max() < 1e-18
    adv = np.linspace(-1, 1, b)
    g = oracle.ppo_loss_grad(logits, actions, old, adv, np.zeros(b), np.zeros(b), None, b)
    onehot = np.eye(12)[actions]
    np.testing.assert_allclose(g.dlogits, -(adv[:, None] * (onehot - 1 / 12)) / b, rtol=1e-13, atol=1e-18)
