"""GPU parity of gae_scan, the advantage statistics and normalisation against the float64 oracle.

Tolerance (GAE / returns, float32 kernels against the float64 definition): |g - o| <= 1e-5 (|o| + rms(o))
per element; the statistics within 1e-6 relative.
"""
import numpy as np
import pytest
import torch

import oracle
from resident_rl_rollout_amd import binding, inputs
from tests.gpu_helpers import assert_gae_close, assert_loss_close

pytestmark = pytest.mark.gpu

G, LAM = float(np.float32(0.99)), float(np.float32(0.95))


def _run(gi, normalize, cols=None):
    dev = "cuda"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    adv, ret, st = binding.gae(t(gi.rewards), t(gi.values), t(gi.dones), t(gi.last_values), G, LAM,
                               normalize=normalize)
    torch.cuda.synchronize()
    return adv.cpu().numpy(), ret.cpu().numpy(), None if st is None else st.cpu().numpy()


def _oracle(gi, cols=None):
    r, v, d, vl = gi.rewards, gi.values, gi.dones, gi.last_values
    if cols is not None:
        r, v, d, vl = r[:, cols], v[:, cols], d[:, cols], vl[cols]
    return oracle.gae(r, v, d, vl, G, LAM)


@pytest.mark.parametrize("t,n", [(128, 2048), (128, 64), (1, 1), (37, 1000), (128, 70000), (300, 513),
                                 (700, 100), (1500, 33), (129, 4096), (128, 20000)])
def test_gae_matches_oracle(t, n, gpu_lib):
    gi = inputs.make_gae_inputs(10 + t + n, t, n)
    adv, ret, _ = _run(gi, 0)
    ra, rr = _oracle(gi)
    assert_gae_close(adv, ra, f"adv T={t} N={n}")
    assert_gae_close(ret, rr, f"ret T={t} N={n}")


@pytest.mark.parametrize("normalize", [1, 2])
def test_normalised_advantages_and_stats(normalize, gpu_lib):
    gi = inputs.make_gae_inputs(10, 128, 2048)
    adv, ret, st = _run(gi, normalize)
    ra, rr = _oracle(gi)
    na, mean, std = oracle.normalize(ra)
    assert st[0] == 128 * 2048
    assert st[1] == pytest.approx(mean, rel=1e-6, abs=1e-7)
    assert st[2] == pytest.approx(std, rel=1e-6)
    assert_gae_close(ret, rr, "ret")
    assert_gae_close(adv, na if normalize == 1 else ra, f"adv normalize={normalize}")


def test_full_rollout_shape_every_element(gpu_lib):
    # T=128, N=65536 in the launch configuration the bench times: every element of the raw and normalised
    # advantages and the returns against the oracle's definition sum over the whole batch, and the
    # whole-batch statistics against the oracle's normalisation
    t, n = 128, 65536
    gi = inputs.make_gae_inputs(20, t, n)
    adv_raw, ret, _ = _run(gi, 0)
    adv_n, ret2, st = _run(gi, 1)
    ra, rr = _oracle(gi)
    assert_gae_close(adv_raw, ra, "adv, every element")
    assert_gae_close(ret, rr, "ret, every element")
    np.testing.assert_array_equal(ret, ret2)
    na, mean, std = oracle.normalize(ra)
    assert st[0] == t * n
    assert abs(st[1] - mean) <= 1e-5 * (abs(mean) + std) and abs(st[2] - std) <= 1e-5 * std
    assert_gae_close(adv_n, na, "normalised, every element")


def test_normalisation_at_a_small_spread(gpu_lib):
    # advantages of about 1e-5: the epsilon (1e-8) is a tenth of a percent of the std, and its placement
    # decides the result ((A - mean) / (std + eps), against about 1e-4 for sqrt(std^2 + eps)); both the
    # materialised normalisation and the one applied inside the loss follow the oracle
    gi = inputs.make_gae_inputs(12, 64, 3000)
    for a in (gi.rewards, gi.values, gi.last_values):
        a *= np.float32(1e-5)
    adv_n, ret, st = _run(gi, 1)
    ra, rr = _oracle(gi)
    na, mean, std = oracle.normalize(ra)
    assert 5e-6 < std < 1e-4
    assert_gae_close(adv_n, na, "normalised at a small spread")
    b = 64 * 3000
    pi = inputs.make_policy_inputs(13, b)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    adv_raw, _, stats = binding.gae(t(gi.rewards), t(gi.values), t(gi.dones), t(gi.last_values), G, LAM,
                                    normalize=2)
    out = binding.ppo_loss(t(pi.new_logits), t(pi.actions), t(pi.old_logp), adv_raw.reshape(-1),
                           t(rr.astype(np.float32)).reshape(-1), t(pi.new_values), t(pi.perm), b // 4,
                           adv_stats=stats).cpu().numpy()
    ref, scale = oracle.ppo_loss(pi.new_logits, pi.actions, pi.old_logp, na.reshape(-1),
                                 rr.astype(np.float32).reshape(-1), pi.new_values, pi.perm, b // 4)
    assert_loss_close(out, ref, scale, "loss with the small-spread normalisation inline")


def test_all_dones_and_zero_gamma(gpu_lib):
    gi = inputs.make_gae_inputs(5, 64, 300)
    gi.dones[:] = 1.0
    adv, ret, _ = _run(gi, 0)
    np.testing.assert_allclose(adv, gi.rewards.astype(np.float64) - gi.values, rtol=0, atol=1e-6)
    np.testing.assert_allclose(ret, gi.rewards, rtol=0, atol=1e-6)


def test_nan_propagates_without_crash(gpu_lib):
    gi = inputs.make_gae_inputs(6, 16, 128)
    gi.rewards[7, 3] = np.nan
    adv, ret, _ = _run(gi, 0)
    assert np.isnan(adv[:8, 3]).all() and np.isfinite(adv[8:, 3]).all()
    assert np.isfinite(np.delete(adv, 3, axis=1)).all()


def test_deterministic_stats(gpu_lib):
    gi = inputs.make_gae_inputs(7, 128, 20000)
    a1, _, s1 = _run(gi, 1)
    a2, _, s2 = _run(gi, 1)
    np.testing.assert_array_equal(a1, a2)
    np.testing.assert_array_equal(s1, s2)


@pytest.mark.parametrize("t,n", [(128, 65536), (129, 65536), (128, 2048), (37, 1000), (1500, 33), (1, 1)])
def test_deferred_statistics_equal_the_finished_ones(t, n, gpu_lib):
    # normalize = 3 leaves the scan blocks' partial sums in adv_stats; finishing them (here, and inside the
    # loss) must give the very bits normalize = 2 gives, and the scan's outputs must not change
    gi = inputs.make_gae_inputs(30 + t + n, t, n)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    args = (dev(gi.rewards), dev(gi.values), dev(gi.dones), dev(gi.last_values), G, LAM)
    adv2, ret2, st2 = binding.gae(*args, normalize=2)
    adv3, ret3, st3 = binding.gae(*args, normalize=3)
    assert st3.numel() * 8 == binding.gae_stats_bytes(t, n) and float(st3[0]) < 0
    torch.testing.assert_close(adv3, adv2, rtol=0, atol=0)
    torch.testing.assert_close(ret3, ret2, rtol=0, atol=0)
    np.testing.assert_array_equal(binding.adv_stats_finish(st3).cpu().numpy(), st2.cpu().numpy())
    np.testing.assert_array_equal(binding.adv_stats_finish(st2).cpu().numpy(), st2.cpu().numpy())
    b = t * n
    mb = b // next(k for k in (16, 8, 4, 2, 1) if b % k == 0)
    pi = inputs.make_policy_inputs(31 + t, b)
    la = (dev(pi.new_logits), dev(pi.actions), dev(pi.old_logp), adv2.reshape(-1), ret2.reshape(-1),
          dev(pi.new_values))
    idx = dev(inputs.minibatch_index(pi.perm, mb))
    for kw in (dict(perm=dev(pi.perm)), dict(perm=None, mb_index=idx), dict(perm=None)):
        perm = kw.pop("perm")
        o2 = binding.ppo_loss(*la, perm, mb, adv_stats=st2, **kw).cpu().numpy()
        o3 = binding.ppo_loss(*la, perm, mb, adv_stats=st3, **kw).cpu().numpy()
        np.testing.assert_array_equal(o3, o2)
        g2 = binding.ppo_loss_grad(*la, perm, mb, adv_stats=st2, **kw)
        g3 = binding.ppo_loss_grad(*la, perm, mb, adv_stats=st3, **kw)
        for x2, x3 in zip(g2, g3):
            torch.testing.assert_close(x3, x2, rtol=0, atol=0)
    np.testing.assert_array_equal(binding.adv_stats_finish(st3).cpu().numpy(), st2.cpu().numpy())
