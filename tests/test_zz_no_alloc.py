"""rl_ppo_loss_noalloc (the loss for callers that cannot allocate: its workspace is the library's fixed
device array) against rl_ppo_loss with a workspace argument, through the C ABI: the same kernels, so the
scalars must be equal bit for bit, and within the loss tolerance of the float64 oracle. Each case makes
two calls in a row on the shared array, the second with a smaller input, so that nothing a call leaves in
the array can leak into the next."""
import numpy as np
import pytest
import torch

import oracle
from resident_rl_rollout_amd import binding, inputs
from tests.gpu_helpers import assert_loss_close

pytestmark = pytest.mark.gpu


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _case(seed, b, a=12):
    pi = inputs.make_policy_inputs(seed, b, a)
    rng = np.random.default_rng(seed + 1)
    adv = rng.standard_normal(b).astype(np.float32)
    ret = rng.standard_normal(b).astype(np.float32)
    return pi, adv, ret


def _check(pi, adv, ret, mb, use_perm, what):
    args = (_dev(pi.new_logits), _dev(pi.actions), _dev(pi.old_logp), _dev(adv), _dev(ret), _dev(pi.new_values))
    perm = _dev(pi.perm) if use_perm else None
    idx = None if use_perm else _dev(inputs.minibatch_index(pi.perm, mb))
    want = binding.ppo_loss(*args, perm, mb, mb_index=idx).cpu().numpy()
    out = torch.full((pi.new_logits.shape[0] // mb, 4), float("nan"), dtype=torch.float32, device="cuda")
    got = binding.ppo_loss_noalloc(*args, perm, mb, mb_index=idx, out=out).cpu().numpy()
    np.testing.assert_array_equal(got, want, err_msg=f"{what}: no-allocation entry vs workspace entry")
    ref, scale = oracle.ppo_loss(pi.new_logits, pi.actions, pi.old_logp, adv, ret, pi.new_values, pi.perm, mb)
    assert_loss_close(got, ref, scale, f"{what}: no-allocation entry vs oracle")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("use_perm", [True, False])
def test_noalloc_loss_equals_workspace_loss_on_two_calls(use_perm, gpu_lib):
    # a large call (with perm: 2^22 samples, 256 bins of staging in the array), then a small ragged one
    for seed, b, mb in [(31, 1 << 22, 1 << 18), (32, 49616, 3101)]:
        pi, adv, ret = _case(seed, b)
        _check(pi, adv, ret, mb, use_perm, f"B={b} mb={mb} perm={use_perm}")


@pytest.mark.timeout(300)
def test_noalloc_loss_full_batch_with_perm(gpu_lib):
    # 128 x 65536 samples in 16 shuffled minibatches: the perm conversion fills 52 of the array's 64 MiB;
    # then a second, smaller call with minibatch numbers
    pi, adv, ret = _case(33, 128 * 65536)
    _check(pi, adv, ret, 524288, True, "full batch, perm")
    pi, adv, ret = _case(34, 65536 * 4)
    _check(pi, adv, ret, 65536, False, "second call, minibatch numbers")


def test_noalloc_loss_refuses_more_than_its_array(gpu_lib):
    # 2^24 samples with a perm need about 112 MiB of workspace: refused before anything is launched, so
    # out keeps its contents (the inputs are allocated at full size all the same)
    b, mb = 1 << 24, 1 << 20
    logits = torch.empty((b, 12), dtype=torch.float32, device="cuda")
    f = torch.empty(b, dtype=torch.float32, device="cuda")
    acts = torch.zeros(b, dtype=torch.int32, device="cuda")
    perm = torch.arange(b, dtype=torch.int32, device="cuda")
    out = torch.full((b // mb, 4), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(binding.RLError, match="fixed device array"):
        binding.ppo_loss_noalloc(logits, acts, f, f, f, f, perm, mb, out=out)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    # the same size without the perm needs only the partials and runs (and matches the workspace entry)
    idx = (torch.arange(b, device="cuda") // mb).to(torch.int16).view(torch.uint16)
    logits.normal_()
    f.normal_()
    want = binding.ppo_loss(logits, acts, f, f, f, f, None, mb, mb_index=idx)
    got = binding.ppo_loss_noalloc(logits, acts, f, f, f, f, None, mb, mb_index=idx)
    torch.testing.assert_close(got, want, rtol=0, atol=0)
