"""Pins of the oracle's PPO loss forward against closed forms and hand-worked values.

The loss is the one in "Teaching Mario to speedrun", section 6 ("Don't move too far at once"):
ratio = new/old probability, loss_pi = -min(ratio*A, clip(ratio, 1-0.2, 1+0.2)*A), loss_V = (V - R)^2,
loss = loss_pi + 0.5 loss_V - 0.01 entropy; the coefficients match PlayTrain's Table 8.
"""
import math

import numpy as np
import pytest

import oracle

A = 12
LN12 = math.log(12.0)


def _uniform_case(adv, ratio, b_values=None, ret=None):
    """Uniform logits (logp = -ln 12 for every action) and old_logp set so the ratio is `ratio`."""
    adv = np.asarray(adv, np.float64)
    b = adv.size
    logits = np.zeros((b, A), np.float32)
    actions = np.arange(b, dtype=np.int32) % A
    old_logp = np.full(b, -LN12 - math.log(ratio), np.float64).astype(np.float32)
    nv = np.zeros(b, np.float32) if b_values is None else np.asarray(b_values, np.float32)
    rt = np.zeros(b) if ret is None else np.asarray(ret, np.float64)
    return logits, actions, old_logp, adv, rt, nv


def _ratio_exact(old_logp):
    return math.exp(-LN12 - float(old_logp))


def test_uniform_logits_entropy_is_ln12():
    out, _ = oracle.ppo_loss(*_uniform_case(np.zeros(8), 1.0), None, 8)
    assert out[0, 2] == pytest.approx(LN12, rel=1e-14)
    assert round(LN12, 12) == 2.484906649788


def test_ratio_one_gives_minus_mean_advantage():
    adv = np.array([0.5, -1.25, 2.0, 0.0, -0.75, 1.5, 3.0, -2.0])
    case = _uniform_case(adv, 1.0)
    out, _ = oracle.ppo_loss(*case, None, 8)
    r = _ratio_exact(case[2][0])          # float32 rounding of old_logp leaves r within 1e-7 of 1
    assert abs(r - 1.0) < 1e-6
    assert out[0, 0] == pytest.approx(-r * adv.mean(), rel=1e-12, abs=1e-15)


@pytest.mark.parametrize("adv,ratio,expect", [
    (1.0, 1.5, lambda r: -(1.2) * 1.0),      # A>0, ratio above 1+eps: clipped
    (-1.0, 0.5, lambda r: -(0.8) * -1.0),    # A<0, ratio below 1-eps: clipped
    (1.0, 0.5, lambda r: -r * 1.0),          # A>0, ratio below 1-eps: unclipped (the pessimistic min)
    (-1.0, 1.5, lambda r: -r * -1.0),        # A<0, ratio above 1+eps: unclipped
    (2.0, 1.1, lambda r: -r * 2.0),          # inside the band
    (-2.0, 0.9, lambda r: -r * -2.0),
])
def test_clip_regions(adv, ratio, expect):
    case = _uniform_case([adv], ratio)
    out, _ = oracle.ppo_loss(*case, None, 1)
    r = _ratio_exact(case[2][0])
    assert out[0, 0] == pytest.approx(expect(r), rel=1e-12)


@pytest.mark.parametrize("ratio", [0.8, 1.2])
def test_clip_boundaries_coincide(ratio):
    # At ratio = 1 +- eps both branches of the min are equal: the result is continuous there.
    for adv in (1.0, -1.0):
        below = oracle.ppo_loss(*_uniform_case([adv], ratio * (1 - 1e-6)), None, 1)[0][0, 0]
        above = oracle.ppo_loss(*_uniform_case([adv], ratio * (1 + 1e-6)), None, 1)[0][0, 0]
        assert abs(below - above) < 1e-5


def test_two_action_hand_example():
    # logits (0, ln 3): p = (1/4, 3/4); action 1: logp = ln(3/4); entropy = ln 4 - (3/4) ln 3.
    logits = np.array([[0.0, math.log(3.0)]], np.float32)
    z1 = float(logits[0, 1])
    lse = math.log(1.0 + math.exp(z1))
    old_logp = np.array([math.log(0.75)], np.float32)
    out, _ = oracle.ppo_loss(logits, np.array([1], np.int32), old_logp, np.array([1.0]), np.array([0.0]),
                             np.array([0.0], np.float32), None, 1)
    p1 = math.exp(z1 - lse)
    h = -(1 - p1) * math.log(1 - p1) - p1 * math.log(p1)
    assert h == pytest.approx(math.log(4.0) - 0.75 * math.log(3.0), rel=1e-6)
    assert out[0, 2] == pytest.approx(h, rel=1e-12)
    ratio = math.exp((z1 - lse) - float(old_logp[0]))
    assert out[0, 0] == pytest.approx(-ratio, rel=1e-12)


def test_value_loss_and_total_coefficients():
    b = 4
    case = list(_uniform_case(np.zeros(b), 1.0, b_values=[1.0, 2.0, 3.0, 4.0], ret=[1.0, 0.0, 5.0, 1.0]))
    out, _ = oracle.ppo_loss(*case, None, b, vf_coef=0.5, ent_coef=0.01)
    # (0^2 + 2^2 + 2^2 + 3^2) / 4
    assert out[0, 1] == pytest.approx(17.0 / 4.0, rel=1e-15)
    assert out[0, 3] == pytest.approx(out[0, 0] + 0.5 * 17.0 / 4.0 - 0.01 * LN12, rel=1e-14)
    out2, _ = oracle.ppo_loss(*case, None, b, vf_coef=2.0, ent_coef=0.25)
    assert out2[0, 3] == pytest.approx(out2[0, 0] + 2.0 * 17.0 / 4.0 - 0.25 * LN12, rel=1e-14)
    case[4] = np.asarray(case[5], np.float64)   # V = R: no value loss
    out3, _ = oracle.ppo_loss(*case, None, b)
    assert out3[0, 1] == 0.0


def test_large_logits_do_not_overflow():
    logits = np.full((3, A), 1000.0, np.float32)
    logits[:, 0] = 999.0
    out, _ = oracle.ppo_loss(logits, np.zeros(3, np.int32), np.zeros(3, np.float32), np.zeros(3),
                             np.zeros(3), np.zeros(3, np.float32), None, 3)
    # p_0 = e^-1 / (e^-1 + 11)
    p0 = math.exp(-1.0) / (math.exp(-1.0) + 11.0)
    ps = np.array([p0] + [1.0 / (math.exp(-1.0) + 11.0)] * 11)
    assert out[0, 2] == pytest.approx(-(ps * np.log(ps)).sum(), rel=1e-12)
    assert np.isfinite(out).all()


def _random_batch(seed, b):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((b, A)).astype(np.float32)
    actions = rng.integers(0, A, b).astype(np.int32)
    old_logp = (-LN12 + 0.2 * rng.standard_normal(b)).astype(np.float32)
    return (logits, actions, old_logp, rng.standard_normal(b), rng.standard_normal(b),
            rng.standard_normal(b).astype(np.float32))


def test_minibatch_is_the_permuted_set():
    # Minibatch m is the set {perm[m*mb + k]}: equal to contiguous minibatches of the pre-gathered
    # arrays, and unchanged when the order inside a minibatch changes.
    b, mb = 96, 24
    batch = _random_batch(8, b)
    perm = np.random.default_rng(9).permutation(b).astype(np.int32)
    out, _ = oracle.ppo_loss(*batch, perm, mb)
    gathered = [x[perm] for x in batch]
    out2, _ = oracle.ppo_loss(*gathered, None, mb)
    np.testing.assert_allclose(out, out2, rtol=1e-13, atol=1e-15)
    perm2 = perm.reshape(-1, mb)[:, ::-1].copy().reshape(-1)
    out3, _ = oracle.ppo_loss(*batch, perm2, mb)
    np.testing.assert_allclose(out, out3, rtol=1e-13, atol=1e-15)
    # one minibatch of the whole batch is the mean of the per-minibatch means
    whole, _ = oracle.ppo_loss(*batch, None, b)
    np.testing.assert_allclose(whole[0], out.mean(axis=0), rtol=1e-12, atol=1e-15)


def test_single_sample_brute_force():
    # Every per-sample term from first principles for one sample with a closed-form softmax.
    z = np.log(np.arange(1, A + 1, dtype=np.float64)).astype(np.float32)   # p_j = (j+1)/78
    p = np.arange(1, A + 1) / 78.0
    a = 5
    old = np.float32(math.log(0.1))
    out, scale = oracle.ppo_loss(z[None], np.array([a], np.int32), np.array([old]), np.array([-0.5]),
                                 np.array([0.25]), np.array([1.0], np.float32), None, 1)
    ratio = p[a] / math.exp(float(old))                  # (6/78) / 0.1 = 0.769...: below 1 - eps
    assert ratio < 0.8
    pg = -min(ratio * -0.5, 0.8 * -0.5)
    assert out[0, 0] == pytest.approx(pg, rel=1e-6)
    assert out[0, 1] == pytest.approx(0.75 ** 2, rel=1e-15)
    assert out[0, 2] == pytest.approx(-(p * np.log(p)).sum(), rel=1e-6)
    assert scale[0, 0] == pytest.approx(abs(out[0, 0]), rel=1e-15)
