"""GPU parity of rl_ppo_loss_grad (the loss scalars and, in the same pass, each sample's gradient of its
minibatch's total loss) against the float64 oracle.

Tolerance: per element |g - o| <= 1e-4 (|o| + magnitude of its summands); rows whose ratio sits within
float rounding of a clip-band edge may take either side of the minimum (see assert_grad_close).
"""
import numpy as np
import pytest
import torch

import oracle
from resident_rl_rollout_amd import binding, inputs
from tests.gpu_helpers import assert_grad_close, assert_loss_close

pytestmark = pytest.mark.gpu


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _case(seed, b, a=12):
    pi = inputs.make_policy_inputs(seed, b, a)
    rng = np.random.default_rng(seed + 1)
    adv = rng.standard_normal(b).astype(np.float32)
    ret = rng.standard_normal(b).astype(np.float32)
    return pi, adv, ret


def _gpu(pi, adv, ret, mb, mode, stats=None):
    perm = _dev(pi.perm) if mode == "perm" else None
    idx = _dev(inputs.minibatch_index(pi.perm, mb)) if mode == "stream" else None
    out, dl, dv = binding.ppo_loss_grad(_dev(pi.new_logits), _dev(pi.actions), _dev(pi.old_logp), _dev(adv),
                                        _dev(ret), _dev(pi.new_values), perm, mb,
                                        adv_stats=None if stats is None else _dev(stats), mb_index=idx)
    return out.cpu().numpy(), dl.cpu().numpy(), dv.cpu().numpy()


def _check(pi, adv, ret, mb, mode, what, stats=None, adv_ref=None):
    out, dl, dv = _gpu(pi, adv, ret, mb, mode, stats)
    a_ref = adv if adv_ref is None else adv_ref
    perm = None if mode == "contiguous" else pi.perm
    ref, scale = oracle.ppo_loss(pi.new_logits, pi.actions, pi.old_logp, a_ref, ret, pi.new_values, perm, mb)
    assert_loss_close(out, ref, scale, what)
    g = oracle.ppo_loss_grad(pi.new_logits, pi.actions, pi.old_logp, a_ref, ret, pi.new_values, perm, mb)
    assert_grad_close(dl, dv, g, a_ref, what)
    return out, dl, dv


@pytest.mark.parametrize("b,mb,a,mode", [
    (262144, 8192, 12, "stream"), (262144, 8192, 12, "perm"), (30000, 3000, 5, "stream"),
    (600, 200, 3, "stream"), (4096, 4096, 7, "stream"), (1, 1, 12, "stream"), (1000, 10, 12, "perm"),
    (8192, 1024, 64, "contiguous"), (40000, 2500, 12, "stream"), (7, 1, 12, "perm"),
    (3000000, 187500, 12, "stream")])
def test_grad_matches_oracle(b, mb, a, mode, gpu_lib):
    pi, adv, ret = _case(b + 3 * mb + a, b, a)
    _check(pi, adv, ret, mb, mode, f"grad {mode} B={b} mb={mb} A={a}")


def test_full_rollout_batch_inline_normalisation(gpu_lib):
    # 128 x 65536 samples, 16 minibatches, advantages normalised on the fly from the GAE statistics
    b, mb = 128 * 65536, 524288
    pi, adv, ret = _case(31, b)
    raw = (adv * 1.3 + 0.2).astype(np.float32)
    norm, mean, std = oracle.normalize(raw.astype(np.float64))
    _check(pi, raw, ret, mb, "stream", "grad full batch", stats=np.array([b, mean, std]), adv_ref=norm)


def test_forward_scalars_equal_the_loss_entry_point(gpu_lib):
    b, mb = 65536, 8192
    pi, adv, ret = _case(5, b)
    idx = _dev(inputs.minibatch_index(pi.perm, mb))
    args = (_dev(pi.new_logits), _dev(pi.actions), _dev(pi.old_logp), _dev(adv), _dev(ret), _dev(pi.new_values), None,
            mb)
    fwd = binding.ppo_loss(*args, mb_index=idx).cpu().numpy()
    out, _, _ = binding.ppo_loss_grad(*args, mb_index=idx)
    ref, scale = oracle.ppo_loss(pi.new_logits, pi.actions, pi.old_logp, adv, ret, pi.new_values, pi.perm, mb)
    assert_loss_close(fwd, ref, scale, "forward")
    assert_loss_close(out.cpu().numpy(), ref, scale, "forward with gradient")


def test_clip_sides_and_uniform_logits(gpu_lib):
    # uniform logits: no entropy gradient; ratio 1.5 / 0.5 puts each sample on a known side of the band
    b = 256
    logits = np.zeros((b, 12), np.float32)
    actions = (np.arange(b) % 12).astype(np.int32)
    ratios = np.where(np.arange(b) % 2 == 0, 1.5, 0.5)
    old_logp = (-np.log(12.0) - np.log(ratios)).astype(np.float32)
    adv = np.where(np.arange(b) % 4 < 2, 1.0, -1.0).astype(np.float32)
    zeros = np.zeros(b, np.float32)
    pi = inputs.PolicyInputs(logits, actions, old_logp, zeros, np.arange(b, dtype=np.int32))
    out, dl, dv = _check(pi, adv, zeros, b, "contiguous", "clip sides")
    clipped_side = np.where(adv > 0, ratios > 1.2, ratios < 0.8)
    assert clipped_side.any() and (~clipped_side).any()
    assert np.abs(dl[clipped_side]).max() < 1e-9        # only the entropy part, zero for uniform logits
    assert np.abs(dl[~clipped_side]).max() > 1e-4
    np.testing.assert_array_equal(dv, np.zeros(b, np.float32))


def test_deterministic(gpu_lib):
    pi, adv, ret = _case(9, 100000)
    r1 = _gpu(pi, adv, ret, 10000, "stream")
    r2 = _gpu(pi, adv, ret, 10000, "stream")
    for x, y in zip(r1, r2):
        np.testing.assert_array_equal(x, y)


def test_rejects_missing_gradient_buffers(gpu_lib):
    pi, adv, ret = _case(1, 64)
    lib = binding.lib()
    t = [_dev(x) for x in (pi.new_logits, pi.actions, pi.old_logp, adv, ret, pi.new_values)]
    out = torch.empty((1, 4), device="cuda")
    ws = torch.empty(binding.ppo_loss_workspace_bytes(64, 64), dtype=torch.uint8, device="cuda")
    rc = lib.rl_ppo_loss_grad(*[x.data_ptr() for x in t], None, None, None, 64, 12, 64, 0.2, 0.5, 0.01,
                              out.data_ptr(), None, None, ws.data_ptr(), ws.numel(), None)
    assert rc == -1 and "dlogits" in lib.rl_last_error().decode()
