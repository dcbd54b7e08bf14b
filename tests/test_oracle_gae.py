"""Pins of the oracle's GAE and advantage normalisation against what the pages and the mathematics fix.

GAE is defined in "Teaching Mario to speedrun", section 6 (Better advantages); the discounted return in
section 4 (Reward) and its reverse accumulation in section 5. None of these checks calls the oracle's
formula a second time: they use hand-worked values, closed forms and a different algorithm (the
reverse recursion) that must agree with the definition sum.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "gae_worked_example.json")


def _col(x):
    return np.asarray(x, dtype=np.float32).reshape(-1, 1)


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_worked_examples(case):
    adv, ret = oracle.gae(_col(case["rewards"]), _col(case["values"]), _col(case["dones"]),
                          np.float32([case["last_value"]]), case["gamma"], case["lambda"])
    np.testing.assert_allclose(adv[:, 0], case["advantages"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(ret[:, 0], case["returns"], rtol=0, atol=1e-12)


def _rand(seed, t, n, p_done=0.0):
    rng = np.random.default_rng(seed)
    r = rng.standard_normal((t, n)).astype(np.float32)
    v = rng.standard_normal((t, n)).astype(np.float32)
    d = (rng.random((t, n)) < p_done).astype(np.float32)
    vl = rng.standard_normal(n).astype(np.float32)
    return r, v, d, vl


def test_lambda_one_is_discounted_return_plus_bootstrap():
    # lambda = 1 and no dones: R_t = sum_k gamma^k r_{t+k} + gamma^(T-t) V_T, whatever V is.
    t, n, g = 9, 5, 0.9
    r, v, d, vl = _rand(1, t, n)
    _, ret = oracle.gae(r, v, d, vl, g, 1.0)
    for j in range(n):
        for s in range(t):
            expect = sum(g ** k * float(r[s + k, j]) for k in range(t - s)) + g ** (t - s) * float(vl[j])
            assert ret[s, j] == pytest.approx(expect, rel=1e-12, abs=1e-12)
    _, ret2 = oracle.gae(r, -3.0 * v + 1.0, d, vl, g, 1.0)
    np.testing.assert_allclose(ret2, ret, rtol=1e-12, atol=1e-12)


def test_lambda_zero_is_one_step_td_error():
    t, n, g = 7, 4, 0.97
    r, v, d, vl = _rand(2, t, n, p_done=0.3)
    adv, _ = oracle.gae(r, v, d, vl, g, 0.0)
    r, v, d, vl = (x.astype(np.float64) for x in (r, v, d, vl))
    vnext = np.concatenate([v[1:], vl[None]], axis=0)
    delta = r + g * vnext * (1.0 - d) - v
    np.testing.assert_allclose(adv, delta, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("gamma,all_done", [(0.0, False), (0.99, True)])
def test_no_future_gives_reward_minus_value(gamma, all_done):
    t, n = 6, 3
    r, v, d, vl = _rand(3, t, n)
    if all_done:
        d[:] = 1.0
    adv, ret = oracle.gae(r, v, d, vl, gamma, 0.95)
    np.testing.assert_allclose(adv, r.astype(np.float64) - v, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ret, r.astype(np.float64), rtol=1e-12, atol=1e-12)


def test_definition_sum_equals_reverse_recursion():
    # A_t = delta_t + gamma*lambda*(1-d_t)*A_{t+1}, A_T = 0: a different algorithm, same quantity.
    t, n, g, lam = 33, 6, 0.99, 0.95
    r, v, d, vl = _rand(4, t, n, p_done=0.1)
    adv, ret = oracle.gae(r, v, d, vl, g, lam)
    r, v, d, vl = (x.astype(np.float64) for x in (r, v, d, vl))
    a = np.zeros(n)
    for s in range(t - 1, -1, -1):
        vn = vl if s == t - 1 else v[s + 1]
        delta = r[s] + g * vn * (1.0 - d[s]) - v[s]
        a = delta + g * lam * (1.0 - d[s]) * a
        np.testing.assert_allclose(adv[s], a, rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(ret[s], a + v[s], rtol=1e-11, atol=1e-11)


def test_done_isolates_episodes():
    # Nothing after the step in which an episode ended may reach the advantages before it.
    t, n = 10, 2
    r, v, d, vl = _rand(5, t, n)
    d[4, :] = 1.0
    adv, _ = oracle.gae(r, v, d, vl, 0.99, 0.95)
    r2, v2, vl2 = r.copy(), v.copy(), vl + 5.0
    r2[5:] += 3.0
    v2[5:] -= 2.0
    adv2, _ = oracle.gae(r2, v2, d, vl2, 0.99, 0.95)
    np.testing.assert_array_equal(adv[:5], adv2[:5])
    assert not np.allclose(adv[5:], adv2[5:])


def test_columns_are_independent():
    t, n = 12, 8
    r, v, d, vl = _rand(6, t, n, p_done=0.1)
    adv, _ = oracle.gae(r, v, d, vl, 0.99, 0.95)
    for j in range(n):
        a1, _ = oracle.gae(r[:, j:j + 1], v[:, j:j + 1], d[:, j:j + 1], vl[j:j + 1], 0.99, 0.95)
        np.testing.assert_array_equal(a1[:, 0], adv[:, j])


def test_normalize_small_example():
    # A = [1, 2, 3, 4]: mean 2.5, population variance 1.25.
    out, mean, std = oracle.normalize(np.array([1.0, 2.0, 3.0, 4.0]), eps=0.0)
    assert mean == 2.5 and std == pytest.approx(math.sqrt(1.25), rel=1e-15)
    np.testing.assert_allclose(out, (np.array([1, 2, 3, 4]) - 2.5) / math.sqrt(1.25), rtol=1e-15)


def test_normalize_moments_and_affine_invariance():
    a = np.random.default_rng(7).standard_normal(10007) * 3.0 + 0.7
    out, mean, std = oracle.normalize(a)
    assert abs(out.mean()) < 1e-12
    assert out.std() == pytest.approx(1.0, abs=1e-7)  # eps = 1e-8 is added to std
    out2, _, _ = oracle.normalize(2.5 * a - 11.0)
    np.testing.assert_allclose(out2, out, rtol=1e-7, atol=1e-7)


def test_normalize_epsilon_is_added_to_std():
    # Constant advantages: std = 0, so the result is 0 / eps = 0, not a division by zero.
    out, mean, std = oracle.normalize(np.full(17, 3.0), eps=1e-8)
    assert std == 0.0 and mean == 3.0
    np.testing.assert_array_equal(out, np.zeros(17))


def test_normalize_epsilon_placement_at_small_std():
    # A = [a, -a]: mean 0 and population std a, so (A - mean) / (std + eps) = +-a / (a + eps). At a = 1e-4
    # and eps = 1e-8 that is +-1 / (1 + 1e-4) = +-0.99990001; the other common placement,
    # (A - mean) / sqrt(std^2 + eps), would give +-1e-4 / sqrt(2e-8) = +-0.7071, so this case tells them apart.
    a = 1e-4
    out, mean, std = oracle.normalize(np.array([a, -a]), eps=1e-8)
    assert mean == 0.0 and std == a
    np.testing.assert_allclose(out, [1.0 / (1.0 + 1e-4), -1.0 / (1.0 + 1e-4)], rtol=1e-14)
    assert abs(out[0] - a / math.sqrt(a * a + 1e-8)) > 0.25
