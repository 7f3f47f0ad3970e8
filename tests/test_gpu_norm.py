"""GPU gated RMSNorm epilogue (gdn_gated_rmsnorm) against the oracle.

"MTP inference: review and commit structure" (eole docs), Functional commits
item 4: the gated RMSNorm that follows the mixer.  fp32 o: normwise per
(layer, row, token, head) block within 1e-5 of the fp64 oracle; bf16 o: within
one bf16 unit of the oracle's value; inactive rows untouched; in place equals
out of place bit for bit; chained after verify on the device.
"""
import numpy as np
import pytest

import oracle
from gated_deltanet_recurrence_conv_amd import workloads as W
from gpu_util import act_dtype, block_err, dev, dims_pair, host, torch_mod

pytestmark = pytest.mark.gpu


def B():
    from gated_deltanet_recurrence_conv_amd import binding
    return binding


def inputs(sh, seed):
    rng = np.random.default_rng(seed)
    shp = (sh.L, sh.B, sh.T, sh.HV, sh.DV)
    o = rng.standard_normal(shp).astype(np.float32) * 0.3
    z = W.bf16_round(rng.standard_normal(shp).astype(np.float32))
    w = W.bf16_round((1.0 + 0.1 * rng.standard_normal((sh.L, sh.DV))).astype(np.float32))
    return o, z, w


@pytest.mark.parametrize("DV,out", [(128, "f32"), (64, "f32"), (32, "f32"), (16, "f32"), (128, "bf16")])
def test_gated_rmsnorm_matches_oracle(DV, out):
    torch = torch_mod()
    sh = W.COHORT.with_(L=2, DV=DV, DK=128 if DV == 128 else DV, out=out)
    o, z, w = inputs(sh, 8000 + DV)
    if out == "bf16":
        o = W.bf16_round(o)
    active = np.ones(sh.B, np.uint8)
    active[[1, 6]] = 0
    bd, od = dims_pair(sh, out=out)
    O = act_dtype(out)
    y = torch.full(o.shape, float("nan"), device="cuda", dtype=O)
    B().gdn_gated_rmsnorm(bd, dev(o, O), dev(z, torch.bfloat16), dev(w, torch.bfloat16), y,
                          eps=1e-6, active=dev(active))
    torch.cuda.synchronize()
    ref = oracle.gated_rmsnorm(od, o, z, w, eps=float(np.float32(1e-6)), active=active)
    yg = host(y).astype(np.float64)
    a = active.astype(bool)
    assert np.all(np.isnan(yg[:, ~a]))
    if out == "f32":
        assert block_err(yg[:, a], ref[:, a], (-1,)) <= 1e-5
    else:
        r = W.bf16_round(ref[:, a].astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(yg[:, a] - r) <= np.abs(r) * 2 ** -7 + 1e-30)


@pytest.mark.parametrize("DV", [16, 32, 64, 128])
def test_gated_rmsnorm_ragged_row_count(DV):
    """45 (layer, row, token, head) rows: not a multiple of the rows a wave
    takes at any d_v, so the last wave is partly past the end; rows 1 and 3
    inactive."""
    torch = torch_mod()
    sh = W.Shape("pfn", L=1, B=5, T=3, HV=3, HK=1, DK=16, DV=DV, S=1, out="f32")
    o, z, w = inputs(sh, 8200 + DV)
    active = np.array([1, 0, 1, 0, 1], np.uint8)
    bd, od = dims_pair(sh)
    y = torch.full(o.shape, float("nan"), device="cuda")
    B().gdn_gated_rmsnorm(bd, dev(o, torch.float32), dev(z, torch.bfloat16), dev(w, torch.bfloat16), y,
                          eps=1e-6, active=dev(active))
    torch.cuda.synchronize()
    ref = oracle.gated_rmsnorm(od, o, z, w, eps=float(np.float32(1e-6)), active=active)
    yg = host(y).astype(np.float64)
    a = active.astype(bool)
    assert np.all(np.isnan(yg[:, ~a]))
    assert block_err(yg[:, a], ref[:, a], (-1,)) <= 1e-5


def test_gated_rmsnorm_in_place_after_verify():
    """verify -> norm in place on its o, against the same norm out of place."""
    torch = torch_mod()
    sh = W.COHORT
    inp = W.verify_inputs(sh, seed=8100)
    _, z, w = inputs(sh, 8101)
    bd, _ = dims_pair(sh)
    A = act_dtype(sh.act)
    o = torch.full((sh.L, sh.B, sh.T, sh.HV, sh.DV), float("nan"), device="cuda")
    act = dev(inp["active"], torch.uint8)
    B().gdn_verify(bd, dev(inp["x"], A), dev(inp["conv_w"], A), None, dev(inp["conv_state"], A),
                   dev(inp["g"], A), dev(inp["beta"], A), dev(inp["state"], torch.float32),
                   dev(inp["cur"], torch.int32), o, act)
    zd, wd = dev(z, torch.bfloat16), dev(w, torch.bfloat16)
    y = torch.full_like(o, float("nan"))
    B().gdn_gated_rmsnorm(bd, o, zd, wd, y, active=act)
    o_before = o.clone()
    B().gdn_gated_rmsnorm(bd, o, zd, wd, o, active=act)
    torch.cuda.synchronize()
    assert np.array_equal(host(o), host(y), equal_nan=True)
    a = inp["active"].astype(bool)
    assert np.all(np.isnan(host(o_before)[:, ~a]))
