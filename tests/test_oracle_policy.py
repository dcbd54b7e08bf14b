"""Pins of the oracle's stand-in policy inference: the encoder / decoder shape of PufferLib 5.0's default
policy ("Teaching Mario to speedrun", s.8: a bias-free linear encoder to 128 numbers, one decoder matrix to
the logits plus the value) and the heads of s.6 (logits sampled through a softmax, plus the value).

Readings (the oracle's header lists them): the encoder reads bfloat16-rounded observations and weights;
the sample is the Gumbel-max form of softmax sampling with SplitMix64 draws keyed by (decision, global env,
logit). Pinned here by: torch's bfloat16 conversion on one-hot weights, a float64 library matmul on the
rounded operands, the generator's published first outputs, the Gumbel distribution's mean and variance,
and action frequencies against the softmax they should follow.
"""
import math

import numpy as np
import pytest
import torch
from scipy import stats
from scipy.special import logsumexp, softmax

import oracle

OBS = oracle.OBS_TILES
H = oracle.POLICY_HIDDEN
A = oracle.POLICY_ACTIONS
M64 = (1 << 64) - 1


def bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def one_hot_policy(cols):
    """Encoder row h reads observation element cols[h] (h < len(cols)); decoder output j = hidden j."""
    enc = np.zeros((H, OBS), np.float32)
    for h, k in enumerate(cols):
        enc[h, k] = 1.0
    dec = np.zeros((A + 1, H), np.float32)
    dec[np.arange(A + 1), np.arange(A + 1)] = 1.0
    return enc, dec


def test_bf16_rounding_matches_torch():
    cols = [0, 5, 100, 1332, 1333, 1392, 1396, 7, 8, 9, 10, 11, 12]
    enc, dec = one_hot_policy(cols)
    ties = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x42FF8000, 0x3F80FFFF, 0x00018000,
                     0x7F7F7FFF, 0x3E2AAAAB], np.uint32).view(np.float32)
    rng = np.random.default_rng(1)
    obs = (rng.standard_normal((64, OBS)) * np.exp(rng.uniform(-20, 20, (64, 1)))).astype(np.float32)
    obs[:len(ties), 5] = ties                         # exact ties round to even, just-below rounds down
    obs[:, 1396] = rng.integers(0, 9, 64)             # tile codes are exact in bfloat16
    out, _, _ = oracle.policy_forward(obs, enc, dec, seed=3, t=0)
    np.testing.assert_array_equal(out[:, :len(cols)], bf16(obs[:, cols]))
    assert (out[:, len(cols):] == 0).all()


def test_encoder_and_decoder_match_a_library_matmul():
    rng = np.random.default_rng(2)
    n, stride = 200, OBS + 11                          # a padded row stride
    obs = rng.standard_normal((n, stride)).astype(np.float32)
    enc = (rng.standard_normal((H, OBS)) / math.sqrt(OBS)).astype(np.float32)
    dec = (rng.standard_normal((A + 1, H)) / math.sqrt(H)).astype(np.float32)
    out, _, logp = oracle.policy_forward(obs, enc, dec, seed=9, t=4)
    hidden = bf16(obs[:, :OBS]) @ bf16(enc).T
    want = hidden @ dec.astype(np.float64).T
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-12)


def test_generator_published_outputs_key_the_first_draws():
    # decision 0, env 0: logit j reads the (j + 1)-th SplitMix64 output from seed 0
    for j, x in enumerate((0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F)):
        g, u = oracle.policy_gumbel(0, 0, 0, j)
        assert u == (2 * (x >> 41) + 1) / 2 ** 24
        assert g == -math.log(-math.log(u))


def test_gumbel_variates_have_the_gumbel_moments():
    gs = np.array([oracle.policy_gumbel(11, t, n, j)[0] for t in range(2) for n in range(1000) for j in range(A)])
    assert abs(gs.mean() - 0.5772156649) < 5 * math.sqrt(math.pi ** 2 / 6 / gs.size)
    assert abs(gs.var() - math.pi ** 2 / 6) < 0.05
    us = np.array([oracle.policy_gumbel(11, 5, n, 3)[1] for n in range(5000)])
    assert stats.kstest(us, "uniform").pvalue > 1e-4


@pytest.mark.parametrize("logits", [[0.0] * A, [2.0, -1.0, 0.5, 0.0, -3.0, 1.5, 0.25, -0.5, 1.0, -2.0, 0.75, 3.0]])
def test_sampled_actions_follow_the_softmax(logits):
    # every env sees observation element 0 = 1, so hidden 0 = 1 and the logits are decoder column 0
    n = 20000
    obs = np.zeros((n, OBS), np.float32)
    obs[:, 0] = 1.0
    enc = np.zeros((H, OBS), np.float32)
    enc[0, 0] = 1.0
    dec = np.zeros((A + 1, H), np.float32)
    dec[:A, 0] = logits
    dec[A, 0] = -0.75                                  # the value head
    out, act, logp = oracle.policy_forward(obs, enc, dec, seed=12345, t=7)
    p = softmax(np.asarray(logits, np.float64))
    counts = np.bincount(act, minlength=A)
    assert stats.chisquare(counts, p * n).pvalue > 1e-4
    np.testing.assert_allclose(logp, np.asarray(logits)[act] - logsumexp(logits), rtol=0, atol=1e-12)
    assert (out[:, A] == -0.75).all()


def test_draws_are_keyed_by_global_env_and_decision():
    rng = np.random.default_rng(4)
    obs = rng.standard_normal((300, OBS)).astype(np.float32)
    enc = (rng.standard_normal((H, OBS)) / 40).astype(np.float32)
    dec = (rng.standard_normal((A + 1, H)) / 12).astype(np.float32)
    _, act, logp = oracle.policy_forward(obs, enc, dec, seed=5, t=2)
    _, act_b, logp_b = oracle.policy_forward(obs[120:], enc, dec, seed=5, t=2, env_offset=120)
    np.testing.assert_array_equal(act[120:], act_b)
    np.testing.assert_array_equal(logp[120:], logp_b)
    _, act_t, _ = oracle.policy_forward(obs, enc, dec, seed=5, t=3)
    assert (act_t != act).mean() > 0.3                 # a new decision draws anew


def test_planted_mistakes_fail_the_pins():
    # a sign slip in the Gumbel variate (g = +ln(-ln u)) would bias toward low-probability actions:
    # the frequencies under it differ from the softmax, which the test above would reject
    logits = np.array([2.0, -1.0, 0.5, 0.0, -3.0, 1.5, 0.25, -0.5, 1.0, -2.0, 0.75, 3.0])
    n = 3000
    wrong = np.empty(n, int)
    for e in range(n):
        g = np.array([oracle.policy_gumbel(1, 0, e, j)[0] for j in range(A)])
        wrong[e] = np.argmax(logits - g)
    counts = np.bincount(wrong, minlength=A)
    assert stats.chisquare(counts, softmax(logits) * n).pvalue < 1e-6
