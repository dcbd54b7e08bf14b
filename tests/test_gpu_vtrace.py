"""GPU parity of rl_vtrace against the float64 oracle (the definition sum).

Tolerance (float32 scan against the float64 definition, as for GAE): |g - o| <= 1e-5 (|o| + rms(o)) per
element of vs and pg_adv.
"""
import numpy as np
import pytest
import torch

import oracle
from resident_rl_rollout_amd import binding, inputs
from tests.gpu_helpers import assert_gae_close

pytestmark = pytest.mark.gpu

PARAMS = {"torchbeast": (0.99, 1.0, 1.0, 1.0, 1.0), "clipped": (0.99, 0.95, 1.0, 0.9, 1.2)}


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _case(t, n, seed):
    gi = inputs.make_gae_inputs(seed, t, n)
    lr = inputs.make_log_rhos(seed + 1, t, n)
    return gi, lr


def _check(gi, lr, prm, what, cols=None):
    g, lam, rb, cb, pb = prm
    g = float(np.float32(g))
    lam = float(np.float32(lam))
    vs, pg = binding.vtrace(_t(gi.rewards), _t(gi.values), _t(gi.dones), _t(gi.last_values), _t(lr), g, lam, rb, cb, pb)
    vs, pg = vs.cpu().numpy(), pg.cpu().numpy()
    r, v, d, vl, l_ = gi.rewards, gi.values, gi.dones, gi.last_values, lr
    if cols is not None:
        r, v, d, vl, l_ = r[:, cols], v[:, cols], d[:, cols], vl[cols], l_[:, cols]
        vs, pg = vs[:, cols], pg[:, cols]
    # the kernel forms g * lambda * min(c_bar, ratio) in float32 from float32 gamma and lambda
    ovs, opg = oracle.vtrace(r, v, d, vl, l_, g, lam, float(np.float32(rb)), float(np.float32(cb)),
                             float(np.float32(pb)))
    assert_gae_close(vs, ovs, f"{what}: vs")
    assert_gae_close(pg, opg, f"{what}: pg_adv")


@pytest.mark.parametrize("prm", list(PARAMS), ids=list(PARAMS))
@pytest.mark.parametrize("t,n", [(128, 2048), (128, 40000), (1, 1), (37, 1000), (200, 100), (300, 77),
                                 (700, 50), (129, 4096), (64, 6144)])
def test_vtrace_matches_oracle(t, n, prm, gpu_lib):
    gi, lr = _case(t, n, 40 + t + n)
    _check(gi, lr, PARAMS[prm], f"vtrace {prm} T={t} N={n}")


def test_vtrace_full_rollout_shape_sampled(gpu_lib):
    # 65536 x 128 (the full rollout's shape and launch), compared on 384 sampled env columns
    t, n = 128, 65536
    gi, lr = _case(t, n, 77)
    cols = np.sort(np.random.default_rng(5).choice(n, 384, replace=False))
    _check(gi, lr, PARAMS["clipped"], "vtrace 65536x128", cols=cols)


def test_vtrace_on_policy_equals_gae_returns(gpu_lib):
    # every ratio 1: vs is GAE(lambda)'s return (both through the C ABI, against the GAE oracle)
    t, n = 128, 4096
    gi = inputs.make_gae_inputs(3, t, n)
    zero = np.zeros((t, n), np.float32)
    g, lam = float(np.float32(0.99)), float(np.float32(0.95))
    vs, _ = binding.vtrace(_t(gi.rewards), _t(gi.values), _t(gi.dones), _t(gi.last_values), _t(zero), g, lam)
    _, ret = oracle.gae(gi.rewards, gi.values, gi.dones, gi.last_values, g, lam)
    assert_gae_close(vs.cpu().numpy(), ret, "on-policy vtrace")


def test_vtrace_all_dones_and_determinism(gpu_lib):
    t, n = 64, 3000
    gi, lr = _case(t, n, 9)
    gi.dones[:] = 1.0
    _check(gi, lr, PARAMS["clipped"], "all dones")
    a = binding.vtrace(_t(gi.rewards), _t(gi.values), _t(gi.dones), _t(gi.last_values), _t(lr), 0.99)
    b = binding.vtrace(_t(gi.rewards), _t(gi.values), _t(gi.dones), _t(gi.last_values), _t(lr), 0.99)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x.cpu().numpy(), y.cpu().numpy())
