"""GPU greedy acceptance (gdn_accept_greedy) against the oracle, bit-exact
(integer work), and chained on the device into gdn_commit.

"Add request-owned eight-way MTP serving for Qwen 35B" (MTPLX PR #245),
Follow-up: the greedy cohort route keeps draft IDs on the device and moves
only token-ID arrays; What was broken item 2: keep in {0, 1, 2} at T = 2.
"""
import numpy as np
import pytest

import oracle
from gated_deltanet_recurrence_conv_amd import workloads as W
from gpu_util import act_dtype, dev, dims_pair, host, torch_mod

pytestmark = pytest.mark.gpu


def B():
    from gated_deltanet_recurrence_conv_amd import binding
    return binding


def ids(rng, sh, p_match):
    """Targets over a 151k vocabulary; each draft equals the target one
    position earlier with probability p_match, else a different id."""
    target = rng.integers(0, 151_000, size=(sh.B, sh.T)).astype(np.int32)
    draft = target[:, :sh.T - 1].copy()
    miss = rng.random((sh.B, sh.T - 1)) >= p_match
    draft[miss] = (draft[miss] + 1 + rng.integers(0, 1000, size=int(miss.sum()))) % 151_000
    return draft.astype(np.int32), target


@pytest.mark.parametrize("T,rows,p", [(2, 8, 0.8), (4, 8, 0.8), (3, 64, 0.5), (4, 300, 0.9),
                                      (1, 5, 0.0)])
def test_accept_matches_oracle(T, rows, p):
    torch = torch_mod()
    sh = W.COHORT.with_(T=T, B=rows, S=T + 1, inactive=(1,) if rows > 1 else ())
    rng = np.random.default_rng(7000 + T * 100 + rows)
    draft, target = ids(rng, sh, p)
    active = np.ones(rows, np.uint8)
    active[list(sh.inactive)] = 0
    bd, od = dims_pair(sh)
    keep = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    nxt = torch.full((rows,), -1, dtype=torch.int32, device="cuda")
    B().gdn_accept_greedy(bd, dev(draft) if T > 1 else None, dev(target), keep, dev(active), nxt)
    torch.cuda.synchronize()
    k_ref, n_ref = oracle.accept_greedy(od, draft, target, active)
    assert np.array_equal(host(keep), k_ref)
    assert np.array_equal(host(nxt), n_ref)


def test_accept_feeds_commit_on_device():
    """accept -> commit with no host round trip equals commit with the keep
    computed on the host."""
    torch = torch_mod()
    sh = W.COHORT
    inp = W.verify_inputs(sh, seed=7100)
    rng = np.random.default_rng(7101)
    draft, target = ids(rng, sh, 0.7)
    bd, od = dims_pair(sh)
    A = act_dtype(sh.act)
    x, cs = dev(inp["x"], A), dev(inp["conv_state"], A)
    cur = dev(inp["cur"], torch.int32)
    act = dev(inp["active"], torch.uint8)
    keep = torch.empty(sh.B, dtype=torch.int32, device="cuda")
    B().gdn_accept_greedy(bd, dev(draft), dev(target), keep, act)
    B().gdn_commit(bd, x, cs, cur, keep, act)
    torch.cuda.synchronize()
    k_ref, _ = oracle.accept_greedy(od, draft, target, inp["active"])
    cs_ref, cur_ref, err = oracle.commit(od, inp["x"], inp["conv_state"], inp["cur"], k_ref,
                                         inp["active"])
    assert err == 0
    assert np.array_equal(host(keep), k_ref)
    assert np.array_equal(host(cur), cur_ref)
    assert np.array_equal(host(cs).astype(np.float64), cs_ref)
