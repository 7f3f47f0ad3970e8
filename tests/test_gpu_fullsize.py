"""Parity at the benchmark's full sizes and launch configuration: the B8/T2
cohort over 30 layer pools in one grouped verify, one grouped commit, the
fused commit + verify of the next cycle, the verify with the fused gated
RMSNorm, and the B8/T4 rewind over 30 layers.
The oracle recomputes sampled layers (0, 14, 29) one by one; every other
layer is checked by properties that hold at any size (inactive rows and the
snapshot slot untouched, finite outputs).  Inputs are drawn on the device
with torch's seeded generator, like the benchmark's pools.

Tolerance: normwise per (layer, row, head) block 2e-3 (bf16 inputs, fp32
state); commit, cur and conv cache bit-exact.
"""
import numpy as np
import pytest

import oracle
from gated_deltanet_recurrence_conv_amd import workloads as W
from gpu_util import dims_pair, host, out_err, state_err, torch_mod

pytestmark = pytest.mark.gpu

L_FULL = 30
SAMPLED = (0, 14, 29)


def B():
    from gated_deltanet_recurrence_conv_amd import binding
    return binding


def pools(sh, seed):
    torch = torch_mod()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    bf = torch.bfloat16
    C, L = sh.C, L_FULL

    def act(shape, scale=1.0):
        return (scale * torch.randn(shape, generator=gen, device="cuda")).to(bf)

    t = dict(x=act((L, sh.B, sh.T, C)), conv_w=act((L, C, 4), 0.5),
             conv_state=act((L, sh.B, 3, C)))
    t["g"] = (-torch.nn.functional.softplus(
        torch.randn((L, sh.B, sh.T, sh.HV), generator=gen, device="cuda"))).to(bf)
    t["beta"] = torch.sigmoid(torch.randn((L, sh.B, sh.T, sh.HV), generator=gen,
                                          device="cuda")).to(bf)
    t["state"] = 0.1 * torch.randn((L, sh.B, sh.S, sh.HV, sh.DK, sh.DV), generator=gen,
                                   device="cuda")
    t["cur"] = torch.randint(0, sh.S, (L, sh.B), generator=gen, device="cuda",
                             dtype=torch.int32)
    return t


def layer(t, l):
    """Host copies (float64 for activations) of one layer's inputs."""
    return {k: host(v[l:l + 1]) for k, v in t.items()}


def test_cohort_thirty_layers_grouped_verify_commit_and_next_cycle():
    torch = torch_mod()
    sh = W.COHORT
    t = pools(sh, 9001)
    act = np.ones(sh.B, np.uint8)
    act[list(sh.inactive)] = 0
    act_d = torch.from_numpy(act).cuda()
    before = {l: layer(t, l) for l in SAMPLED}
    cur0 = host(t["cur"]).copy()
    cs0 = t["conv_state"].clone()
    bd, _ = dims_pair(sh, L=L_FULL)
    _, od1 = dims_pair(sh, L=1)
    o = torch.full((L_FULL, sh.B, sh.T, sh.HV, sh.DV), float("nan"), device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    # snapshot slots of every layer, for the untouched check
    snap_slots = torch.gather(t["state"], 2, t["cur"].long().view(L_FULL, sh.B, 1, 1, 1, 1)
                              .expand(L_FULL, sh.B, 1, sh.HV, sh.DK, sh.DV)).clone()
    B().gdn_verify(bd, t["x"], t["conv_w"], None, t["conv_state"], t["g"], t["beta"], t["state"],
                   t["cur"], o, act_d, err)
    rng = np.random.default_rng(9002)
    keep = W.keep_uniform(rng, sh, act)
    keep_d = torch.from_numpy(keep).cuda()
    B().gdn_commit(bd, t["x"], t["conv_state"], t["cur"], keep_d, act_d, err)
    torch.cuda.synchronize()
    assert int(host(err)[0]) == 0
    o_h = host(o)
    a = act.astype(bool)
    assert np.all(np.isfinite(o_h[:, a])) and np.all(np.isnan(o_h[:, ~a]))
    # the pre-verification slot of every row of every layer is untouched
    snap_after = torch.gather(t["state"], 2, torch.from_numpy(cur0).cuda().long()
                              .view(L_FULL, sh.B, 1, 1, 1, 1)
                              .expand(L_FULL, sh.B, 1, sh.HV, sh.DK, sh.DV))
    assert torch.equal(snap_after, snap_slots)
    cur_h, cs_h = host(t["cur"]), host(t["conv_state"])
    for l in SAMPLED:
        inp = before[l]
        st_ref, o_ref, e = oracle.verify(od1, inp["x"], inp["conv_w"], None, inp["conv_state"],
                                         inp["g"], inp["beta"], inp["state"], inp["cur"], act)
        assert e == 0
        st_l = host(t["state"][l:l + 1])
        assert out_err(o_h[l:l + 1][:, a], o_ref[:, a]) <= 2e-3
        for b in np.nonzero(a)[0]:
            c0 = int(inp["cur"][0, b])
            for s in range(1, sh.T + 1):
                slot = (c0 + s) % sh.S
                assert state_err(st_l[:, b, slot], st_ref[:, b, slot]) <= 2e-3
        cs_ref, cur_ref, e = oracle.commit(od1, inp["x"], inp["conv_state"], inp["cur"], keep, act)
        assert e == 0
        assert np.array_equal(cur_h[l:l + 1], cur_ref)
        assert np.array_equal(cs_h[l:l + 1].astype(np.float64), cs_ref)

    # the next cycle as the fused commit + verify: commits this keep from the
    # snapshot (S = 3 slots stay; only slot cur is written) and verifies new inputs
    t2 = pools(sh, 9003)
    for k in ("x", "g", "beta"):
        t[k + "_next"] = t2[k]
    del t2
    # restart from the pre-verification state: cur and conv cache as before the commit
    # (verify never writes slot cur, so the snapshots are still in place)
    t["cur"].copy_(torch.from_numpy(cur0).cuda())
    t["conv_state"].copy_(cs0)
    o2 = torch.full_like(o, float("nan"))
    B().gdn_verify_lazy(bd, t["x"], t["g"], t["beta"], keep_d, t["x_next"], t["conv_w"], None,
                        t["conv_state"], t["g_next"], t["beta_next"], t["state"], t["cur"], o2,
                        act_d, err)
    torch.cuda.synchronize()
    assert int(host(err)[0]) == 0
    o2_h = host(o2)
    assert np.all(np.isfinite(o2_h[:, a])) and np.all(np.isnan(o2_h[:, ~a]))
    for l in SAMPLED:
        inp = before[l]
        st1, cs1, _, e1 = oracle.rewind(od1, inp["x"], inp["conv_w"], None, inp["conv_state"],
                                        inp["g"], inp["beta"], inp["state"], inp["cur"], keep)
        assert e1 == 0
        nxt = {k: host(t[k + "_next"][l:l + 1]) for k in ("x", "g", "beta")}
        _, o_ref, e2 = oracle.verify(od1, nxt["x"], inp["conv_w"], None, cs1, nxt["g"],
                                     nxt["beta"], st1, inp["cur"], act)
        assert e2 == 0
        assert np.array_equal(host(t["conv_state"][l:l + 1]).astype(np.float64), cs1)
        st_l = host(t["state"][l:l + 1])
        for b in range(sh.B):
            c0 = int(inp["cur"][0, b])
            assert state_err(st_l[:, b, c0], st1[:, b, c0]) <= 2e-3
        assert out_err(o2_h[l:l + 1][:, a], o_ref[:, a]) <= 2e-3


def test_rewind_b8_t4_thirty_layers():
    torch = torch_mod()
    sh = W.REWIND
    t = pools(sh, 9101)
    before = {l: layer(t, l) for l in SAMPLED}
    rng = np.random.default_rng(9102)
    keep = W.keep_uniform(rng, sh)
    keep[0], keep[1] = 0, sh.T
    bd, _ = dims_pair(sh, L=L_FULL)
    _, od1 = dims_pair(sh, L=1)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    B().gdn_rewind(bd, t["x"], t["conv_w"], None, t["conv_state"], t["g"], t["beta"], t["state"],
                   t["cur"], torch.from_numpy(keep).cuda(), None, err)
    torch.cuda.synchronize()
    assert int(host(err)[0]) == 0
    for l in SAMPLED:
        inp = before[l]
        st_ref, cs_ref, _, e = oracle.rewind(od1, inp["x"], inp["conv_w"], None, inp["conv_state"],
                                             inp["g"], inp["beta"], inp["state"], inp["cur"], keep)
        assert e == 0
        st_l = host(t["state"][l:l + 1])
        assert np.array_equal(host(t["conv_state"][l:l + 1]).astype(np.float64), cs_ref)
        for b in range(sh.B):
            c0 = int(inp["cur"][0, b])
            if keep[b] == 0:
                assert np.array_equal(st_l[:, b], inp["state"][:, b])
            else:
                assert state_err(st_l[:, b, c0], st_ref[:, b, c0]) <= 2e-3


def test_cohort_thirty_layers_verify_with_fused_gated_norm():
    """gdn_verify_gated_norm over the 30 layer pools (the bench's fused-norm
    launch): candidates bit-equal to the plain grouped verify on every layer,
    y against the oracle's verify followed by its gated RMSNorm on the sampled
    layers, inactive rows untouched."""
    torch = torch_mod()
    sh = W.COHORT
    t = pools(sh, 9201)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(9202)
    z = torch.randn((L_FULL, sh.B, sh.T, sh.HV, sh.DV), generator=gen, device="cuda").to(torch.bfloat16)
    w = (1.0 + 0.1 * torch.randn((L_FULL, sh.DV), generator=gen, device="cuda")).to(torch.bfloat16)
    act = np.ones(sh.B, np.uint8)
    act[list(sh.inactive)] = 0
    act_d = torch.from_numpy(act).cuda()
    before = {l: layer(t, l) for l in SAMPLED}
    bd, _ = dims_pair(sh, L=L_FULL)
    _, od1 = dims_pair(sh, L=1)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    st_plain = t["state"].clone()
    o = torch.full((L_FULL, sh.B, sh.T, sh.HV, sh.DV), float("nan"), device="cuda")
    B().gdn_verify(bd, t["x"], t["conv_w"], None, t["conv_state"], t["g"], t["beta"], st_plain,
                   t["cur"], o, act_d, err)
    y = torch.full_like(o, float("nan"))
    B().gdn_verify_gated_norm(bd, t["x"], t["conv_w"], None, t["conv_state"], t["g"], t["beta"],
                              t["state"], t["cur"], z, w, y, eps=1e-6, active=act_d, err=err)
    torch.cuda.synchronize()
    assert int(host(err)[0]) == 0
    assert torch.equal(t["state"], st_plain)
    y_h = host(y).astype(np.float64)
    a = act.astype(bool)
    assert np.all(np.isfinite(y_h[:, a])) and np.all(np.isnan(y_h[:, ~a]))
    z_h, w_h = host(z), host(w)
    for l in SAMPLED:
        inp = before[l]
        _, o_ref, e = oracle.verify(od1, inp["x"], inp["conv_w"], None, inp["conv_state"],
                                    inp["g"], inp["beta"], inp["state"], inp["cur"], act)
        assert e == 0
        y_ref = oracle.gated_rmsnorm(od1, o_ref, z_h[l:l + 1], w_h[l:l + 1],
                                     eps=float(np.float32(1e-6)), active=act)
        num = np.max(np.abs(y_h[l:l + 1][:, a] - y_ref[:, a]), axis=-1)
        den = np.maximum(np.max(np.abs(y_ref[:, a]), axis=-1), 1e-30)
        assert np.max(num / den) <= 2e-3
