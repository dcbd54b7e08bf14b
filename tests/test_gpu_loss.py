"""GPU parity of ppo_loss against the float64 oracle.

Tolerance: |g - o| <= 1e-4 (|o| + mean_i |summand_i|) per minibatch scalar.
"""
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


def _gpu(pi, adv, ret, mb, use_perm=True, stats=None, a=12, stream=False):
    idx = _dev(inputs.minibatch_index(pi.perm, mb)) if stream else None
    out = binding.ppo_loss(_dev(pi.new_logits), _dev(pi.actions), _dev(pi.old_logp), _dev(adv), _dev(ret),
                           _dev(pi.new_values), _dev(pi.perm) if (use_perm and not stream) else None, mb,
                           adv_stats=None if stats is None else _dev(stats), mb_index=idx)
    return out.cpu().numpy()


@pytest.mark.parametrize("b,mb,use_perm,a", [(262144, 8192, True, 12), (262144, 8192, False, 12),
                                             (4096, 4096, True, 12), (1000, 10, True, 12), (7, 1, True, 12),
                                             (30000, 3000, True, 5), (8192, 1024, False, 64), (600, 200, True, 3)])
def test_loss_matches_oracle(b, mb, use_perm, a, gpu_lib):
    pi, adv, ret = _case(b + mb + a, b, a)
    got = _gpu(pi, adv, ret, mb, use_perm)
    ref, scale = oracle.ppo_loss(pi.new_logits, pi.actions, pi.old_logp, adv, ret, pi.new_values,
                                 pi.perm if use_perm else None, mb)
    assert got.shape == ref.shape
    assert_loss_close(got, ref, scale, f"B={b} mb={mb} perm={use_perm} A={a}")


@pytest.mark.parametrize("b,mb,a", [(262144, 8192, 12), (30000, 3000, 5), (600, 200, 3), (64000, 1000, 12),
                                    (40000, 2500, 12), (1, 1, 12), (4096, 4096, 7),
                                    (3000000, 187500, 12)])   # blocks end partway through a load-ahead group
def test_stream_mode_matches_oracle(b, mb, a, gpu_lib):
    # the minibatch split given as each sample's minibatch number, read in storage order
    pi, adv, ret = _case(b + 7 * mb + a, b, a)
    got = _gpu(pi, adv, ret, mb, stream=True)
    ref, scale = oracle.ppo_loss(pi.new_logits, pi.actions, pi.old_logp, adv, ret, pi.new_values, pi.perm, mb)
    assert_loss_close(got, ref, scale, f"stream B={b} mb={mb} A={a}")


def test_stream_mode_inline_normalisation_full_batch(gpu_lib):
    # the bench's configuration: 128 x 65536 samples, 16 minibatches, normalisation applied on the fly
    b, mb = 128 * 65536, 524288
    pi, adv, ret = _case(21, b)
    raw = (adv * 1.7 - 0.4).astype(np.float32)
    norm, mean, std = oracle.normalize(raw.astype(np.float64))
    got = _gpu(pi, raw, ret, mb, stats=np.array([b, mean, std]), stream=True)
    ref, scale = oracle.ppo_loss(pi.new_logits, pi.actions, pi.old_logp, norm, ret, pi.new_values, pi.perm, mb)
    assert_loss_close(got, ref, scale, "stream + inline normalisation")
    got2 = _gpu(pi, raw, ret, mb, stats=np.array([b, mean, std]), stream=True)
    np.testing.assert_array_equal(got, got2)


def test_inline_normalisation_matches_normalised_input(gpu_lib):
    b, mb = 65536, 8192
    pi, adv, ret = _case(3, b)
    raw = (adv * 2.5 + 0.3).astype(np.float32)
    norm, mean, std = oracle.normalize(raw.astype(np.float64))
    stats = np.array([b, mean, std], np.float64)
    got = _gpu(pi, raw, ret, mb, stats=stats)
    ref, scale = oracle.ppo_loss(pi.new_logits, pi.actions, pi.old_logp, norm, ret, pi.new_values, pi.perm, mb)
    assert_loss_close(got, ref, scale, "inline normalisation")


def test_full_rollout_batch_sixteen_minibatches(gpu_lib):
    # The bench's launch configuration: B = 128 x 65536 samples in 16 shuffled minibatches.
    b, mb = 128 * 65536, 524288
    pi, adv, ret = _case(20, b)
    got = _gpu(pi, adv, ret, mb)
    ref, scale = oracle.ppo_loss(pi.new_logits, pi.actions, pi.old_logp, adv, ret, pi.new_values, pi.perm, mb)
    assert_loss_close(got, ref, scale, "16 minibatches")


def test_clip_and_entropy_special_cases(gpu_lib):
    # uniform logits: entropy ln 12; ratio set on both sides of the clip band
    b = 256
    logits = np.zeros((b, 12), np.float32)
    actions = (np.arange(b) % 12).astype(np.int32)
    ratios = np.where(np.arange(b) % 2 == 0, 1.5, 0.5)
    old_logp = (-np.log(12.0) - np.log(ratios)).astype(np.float32)
    adv = np.where(np.arange(b) % 4 < 2, 1.0, -1.0).astype(np.float32)
    ret = np.zeros(b, np.float32)
    nv = np.zeros(b, np.float32)
    pi = inputs.PolicyInputs(logits, actions, old_logp, nv, np.arange(b, dtype=np.int32))
    got = _gpu(pi, adv, ret, b)
    ref, scale = oracle.ppo_loss(logits, actions, old_logp, adv, ret, nv, None, b)
    assert_loss_close(got, ref, scale, "clip cases")
    assert got[0, 2] == pytest.approx(np.log(12.0), rel=1e-6)
    assert got[0, 1] == 0.0


def test_deterministic(gpu_lib):
    pi, adv, ret = _case(9, 100000)
    o1 = _gpu(pi, adv, ret, 10000)
    o2 = _gpu(pi, adv, ret, 10000)
    np.testing.assert_array_equal(o1, o2)


def test_rejects_bad_arguments(gpu_lib):
    pi, adv, ret = _case(1, 100)
    with pytest.raises(binding.RLError, match="multiple"):
        _gpu(pi, adv, ret, 30)


@pytest.mark.parametrize("b,mb", [(16384, 4096), (60000, 3000), (4000, 1000)])
def test_minibatch_numbers_past_the_last_count_as_the_last(b, mb, gpu_lib):
    # 4, 20 and 4 minibatches, fewer than the 16 / 32 / 64 per-thread slots of the stream pass: every
    # sample of the last minibatch is renumbered to a value past it (up to 65535); the header reads those
    # as the last minibatch, so the sets, and the oracle's scalars from the permutation, are unchanged
    pi, adv, ret = _case(b + 3, b)
    nmb = b // mb
    idx = inputs.minibatch_index(pi.perm, mb)
    rng = np.random.default_rng(b)
    slots = 16 if nmb <= 16 else (32 if nmb <= 32 else 64)
    last = np.nonzero(idx == nmb - 1)[0]
    half = last.size // 2
    idx[last[:half]] = rng.integers(nmb, slots, half).astype(np.uint16)           # slots the pass never sums
    idx[last[half:]] = rng.integers(slots, 65536, last.size - half).astype(np.uint16)   # past every slot
    out = binding.ppo_loss(_dev(pi.new_logits), _dev(pi.actions), _dev(pi.old_logp), _dev(adv), _dev(ret),
                           _dev(pi.new_values), None, mb, mb_index=_dev(idx)).cpu().numpy()
    ref, scale = oracle.ppo_loss(pi.new_logits, pi.actions, pi.old_logp, adv, ret, pi.new_values, pi.perm, mb)
    assert_loss_close(out, ref, scale, f"B={b} mb={mb} renumbered last minibatch")


@pytest.mark.parametrize("b,mb", [(49616, 3101), (1 << 20, 1 << 16), (262144, 4096), (5, 5), (16384 * 5 + 16, 10242)])
def test_perm_conversion_equals_minibatch_numbers(b, mb, gpu_lib):
    # the perm is turned into minibatch numbers on the device (sorted into bins by destination; up to 16
    # minibatches the stream pass places its own chunk, else 2-byte numbers are written for it; these sizes
    # give one bin, several, ragged last bins, and both routes); the scalars must equal, bit for bit, those
    # of the same split given as minibatch numbers, and the oracle's within tolerance
    pi, adv, ret = _case(b + 7, b)
    args = (_dev(pi.new_logits), _dev(pi.actions), _dev(pi.old_logp), _dev(adv), _dev(ret), _dev(pi.new_values))
    out_perm = binding.ppo_loss(*args, _dev(pi.perm), mb).cpu().numpy()
    out_idx = binding.ppo_loss(*args, None, mb, mb_index=_dev(inputs.minibatch_index(pi.perm, mb))).cpu().numpy()
    np.testing.assert_array_equal(out_perm, out_idx)
    ref, scale = oracle.ppo_loss(pi.new_logits, pi.actions, pi.old_logp, adv, ret, pi.new_values, pi.perm, mb)
    assert_loss_close(out_perm, ref, scale, f"B={b} mb={mb} from perm")
    _, dl_p, dv_p = binding.ppo_loss_grad(*args, _dev(pi.perm), mb)
    _, dl_i, dv_i = binding.ppo_loss_grad(*args, None, mb, mb_index=_dev(inputs.minibatch_index(pi.perm, mb)))
    torch.testing.assert_close(dl_p, dl_i, rtol=0, atol=0)
    torch.testing.assert_close(dv_p, dv_i, rtol=0, atol=0)



def _perm_vs_index(b, mb, perm, seed):
    pi, adv, ret = _case(seed, b, a=4)
    args = (_dev(pi.new_logits), _dev(pi.actions), _dev(pi.old_logp), _dev(adv), _dev(ret), _dev(pi.new_values))
    out_perm = binding.ppo_loss(*args, _dev(perm), mb).cpu().numpy()
    out_idx = binding.ppo_loss(*args, None, mb, mb_index=_dev(inputs.minibatch_index(perm, mb))).cpu().numpy()
    return pi, adv, ret, out_perm, out_idx


@pytest.mark.parametrize("b,mb,kind", [(1 << 20, 1 << 16, "identity"), (1 << 20, 1 << 16, "reversed"),
                                       (300000, 20000, "rotated"), (262144, 4096, "identity"),
                                       (100480, 100480 // 40, "reversed")])
def test_perm_conversion_with_long_runs(b, mb, kind, gpu_lib):
    # perms that are not shuffles send a position block's entries to few bins, so the runs the conversion
    # reads are thousands of entries long, far past the 64 a wave reads at once; the scalars must still
    # equal those of the same split given as minibatch numbers, and the oracle's within tolerance
    base = np.arange(b, dtype=np.int32)
    perm = {"identity": base, "reversed": base[::-1].copy(), "rotated": np.roll(base, b // 3)}[kind]
    pi, adv, ret, out_perm, out_idx = _perm_vs_index(b, mb, perm, b % 1000 + 3)
    np.testing.assert_array_equal(out_perm, out_idx)
    ref, scale = oracle.ppo_loss(pi.new_logits, pi.actions, pi.old_logp, adv, ret, pi.new_values, perm, mb)
    assert_loss_close(out_perm, ref, scale, f"B={b} mb={mb} {kind} perm")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("b,nmb", [((1 << 23) + 16, 16), ((1 << 23) + 16, 48), (1 << 24, 16)])
def test_perm_conversion_two_rounds_of_bins(b, nmb, gpu_lib):
    # just past 2^23 samples the stream pass takes two rounds of 512 blocks (1024 bins) at 16 minibatches,
    # and 513 sort rows; at 48 minibatches the placed numbers; at 2^24, the largest sorted batch, 1024 bins
    # (the most the sort holds) and 1024 sort rows: bit for bit the minibatch-number results (those are
    # checked against the oracle at other sizes)
    rng = np.random.default_rng(b)
    perm = rng.permutation(b).astype(np.int32)
    _, _, _, out_perm, out_idx = _perm_vs_index(b, b // nmb, perm, 17)
    np.testing.assert_array_equal(out_perm, out_idx)
    assert np.isfinite(out_perm).all()


@pytest.mark.timeout(300)
def test_perm_conversion_past_the_binned_sizes(gpu_lib):
    # more than 1024 bins of 16384 samples: the perm takes the direct scatter; the scalars must still equal
    # those of the same split given as minibatch numbers, and the oracle's within tolerance
    b = (1 << 24) + (1 << 16)
    mb = b // 8
    pi, adv, ret = _case(91, b, a=4)
    args = (_dev(pi.new_logits), _dev(pi.actions), _dev(pi.old_logp), _dev(adv), _dev(ret), _dev(pi.new_values))
    out_perm = binding.ppo_loss(*args, _dev(pi.perm), mb).cpu().numpy()
    out_idx = binding.ppo_loss(*args, None, mb, mb_index=_dev(inputs.minibatch_index(pi.perm, mb))).cpu().numpy()
    np.testing.assert_array_equal(out_perm, out_idx)
    ref, scale = oracle.ppo_loss(pi.new_logits, pi.actions, pi.old_logp, adv, ret, pi.new_values, pi.perm, mb)
    assert_loss_close(out_perm, ref, scale, f"B={b} mb={mb} from perm (direct scatter)")

@pytest.mark.parametrize("mode", ["perm", "stream", "contiguous"])
def test_nan_logits_spoil_only_their_minibatch(mode, gpu_lib):
    # a NaN in one sample's logits makes its minibatch's policy, entropy and total terms NaN and leaves the
    # value term and every other minibatch finite, as in the oracle (no crash, no spread across minibatches)
    b, mb = 65536, 8192
    pi, adv, ret = _case(77, b)
    logits = pi.new_logits.copy()
    s = int(pi.perm[3 * mb + 5]) if mode != "contiguous" else 3 * mb + 5    # a sample of minibatch 3
    logits[s, 7] = np.nan
    args = (_dev(logits), _dev(pi.actions), _dev(pi.old_logp), _dev(adv), _dev(ret), _dev(pi.new_values))
    if mode == "perm":
        out = binding.ppo_loss(*args, _dev(pi.perm), mb).cpu().numpy()
    elif mode == "stream":
        out = binding.ppo_loss(*args, None, mb, mb_index=_dev(inputs.minibatch_index(pi.perm, mb))).cpu().numpy()
    else:
        out = binding.ppo_loss(*args, None, mb).cpu().numpy()
    ref, _ = oracle.ppo_loss(logits, pi.actions, pi.old_logp, adv, ret, pi.new_values,
                             None if mode == "contiguous" else pi.perm, mb)
    assert np.isnan(out[3, [0, 2, 3]]).all() and np.isfinite(out[3, 1])
    np.testing.assert_array_equal(np.isnan(out), np.isnan(ref))
    assert np.isfinite(np.delete(out, 3, axis=0)).all()
