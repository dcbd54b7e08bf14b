"""GPU parity of the strided GAE and V-trace entry points (rl_gae_strided, rl_vtrace_strided): a minibatch
of envs as a column range of the [T][N] rollout, with its fresh values in the same layout, gives the same
bits as the contiguous call on a copy of those columns, matches the oracle, and leaves every other column
untouched ("Teaching Mario to speedrun", s.8: advantages computed per minibatch from fresh values)."""
import numpy as np
import pytest
import torch

import oracle
from resident_rl_rollout_amd import binding, inputs
from tests.gpu_helpers import assert_gae_close

pytestmark = pytest.mark.gpu
G, L = float(np.float32(0.99)), float(np.float32(0.95))


def _rollout(seed, t, n):
    gi = inputs.make_gae_inputs(seed, t, n)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return dev(gi.rewards), dev(gi.values), dev(gi.dones), dev(gi.last_values)


@pytest.mark.parametrize("t,n,n0,w", [(128, 65536, 4096, 8192), (128, 4096, 1000, 333), (37, 1000, 13, 211),
                                      (600, 512, 100, 64), (1, 300, 7, 5)])
@pytest.mark.parametrize("normalize", [0, 1, 2, 3])
def test_gae_on_a_column_range(gpu_lib, t, n, n0, w, normalize):
    r, v, d, vl = _rollout(t + n + w, t, n)
    fresh = v.clone()
    fresh[:, n0:n0 + w] += 0.25                        # the minibatch's fresh values, in the rollout's layout
    sl = slice(n0, n0 + w)
    adv = torch.full((t, n), -7.0, device="cuda")
    ret = torch.full((t, n), -7.0, device="cuda")
    a, rt, st = binding.gae(r[:, sl], fresh[:, sl], d[:, sl], vl[sl].contiguous(), G, L, normalize=normalize,
                            adv=adv[:, sl], ret=ret[:, sl])
    # the same call on contiguous copies: the same kernel for the same (T, N), so the same bits
    a2, r2, st2 = binding.gae(r[:, sl].contiguous(), fresh[:, sl].contiguous(), d[:, sl].contiguous(),
                              vl[sl].contiguous(), G, L, normalize=normalize)
    assert torch.equal(adv[:, sl], a2) and torch.equal(ret[:, sl], r2)
    if normalize:
        assert torch.equal(st, st2)
    if normalize == 3:
        # the deferred partial sums of a column range finish to the statistics normalize = 2 leaves
        _, _, st_fin = binding.gae(r[:, sl].contiguous(), fresh[:, sl].contiguous(), d[:, sl].contiguous(),
                                   vl[sl].contiguous(), G, L, normalize=2)
        assert torch.equal(binding.adv_stats_finish(st), st_fin)
    others = torch.ones(n, dtype=torch.bool)
    others[sl] = False
    assert (adv[:, others.cuda()] == -7.0).all() and (ret[:, others.cuda()] == -7.0).all()
    ra, rr = oracle.gae(r[:, sl].cpu().numpy(), fresh[:, sl].cpu().numpy(), d[:, sl].cpu().numpy(),
                        vl[sl].cpu().numpy(), G, L)
    assert_gae_close(ret[:, sl].cpu().numpy(), rr, "strided returns")
    if normalize == 1:
        na, _, _ = oracle.normalize(ra)
        assert_gae_close(adv[:, sl].cpu().numpy(), na, "strided normalised advantages")
    else:
        assert_gae_close(adv[:, sl].cpu().numpy(), ra, "strided advantages")


@pytest.mark.parametrize("t,n,n0,w", [(128, 65536, 2048, 16384), (200, 1000, 31, 97), (700, 256, 3, 9)])
def test_vtrace_on_a_column_range(gpu_lib, t, n, n0, w):
    r, v, d, vl = _rollout(t * 3 + w, t, n)
    lr = torch.from_numpy(inputs.make_log_rhos(t + n, t, n)).cuda()
    sl = slice(n0, n0 + w)
    vs = torch.full((t, n), 5.0, device="cuda")
    pg = torch.full((t, n), 5.0, device="cuda")
    binding.vtrace(r[:, sl], v[:, sl], d[:, sl], vl[sl].contiguous(), lr[:, sl], G, 0.9, 1.0, 1.0, 1.0,
                   vs=vs[:, sl], pg_adv=pg[:, sl])
    vs2, pg2 = binding.vtrace(r[:, sl].contiguous(), v[:, sl].contiguous(), d[:, sl].contiguous(),
                              vl[sl].contiguous(), lr[:, sl].contiguous(), G, 0.9, 1.0, 1.0, 1.0)
    assert torch.equal(vs[:, sl], vs2) and torch.equal(pg[:, sl], pg2)
    others = torch.ones(n, dtype=torch.bool)
    others[sl] = False
    assert (vs[:, others.cuda()] == 5.0).all() and (pg[:, others.cuda()] == 5.0).all()
    ovs, opg = oracle.vtrace(r[:, sl].cpu().numpy(), v[:, sl].cpu().numpy(), d[:, sl].cpu().numpy(),
                             vl[sl].cpu().numpy(), lr[:, sl].cpu().numpy(), G, 0.9, 1.0, 1.0, 1.0)
    assert_gae_close(vs[:, sl].cpu().numpy(), ovs, "strided vs")
    assert_gae_close(pg[:, sl].cpu().numpy(), opg, "strided pg advantages")


def test_rejects_a_row_stride_below_the_width(gpu_lib):
    r, v, d, vl = _rollout(1, 4, 64)
    lib = binding.lib()
    p = lambda x: binding.dptr(x)
    assert lib.rl_gae_strided(p(r), p(v), p(d), p(vl), 4, 64, 63, 0.99, 0.95, p(r), p(v), 0, None, None, 0,
                              None) == -1
    assert "row stride" in lib.rl_last_error().decode()
