"""GPU tests of verify and fused commit + verify with the gated RMSNorm
epilogue inside the same launch (gdn_verify_gated_norm,
gdn_verify_lazy_gated_norm), through the C ABI.

"MTP inference: review and commit structure" (eole docs), Functional commits
item 4: the gated RMSNorm that follows the mixer.  Checked:

  * y against the oracle's verify followed by its gated RMSNorm (2e-3 per
    (layer, row, token, head) block with bf16 inputs, 1e-5 with fp32 inputs);
  * y against the two-launch GPU path (verify, then gdn_gated_rmsnorm on the
    fp32 o): 1e-5 per block -- only the order of the sum of squares differs;
  * candidate states, the snapshot slot and the error word bit for bit equal
    to gdn_verify's, committed state and conv cache bit for bit equal to
    gdn_verify_lazy's;
  * inactive rows leave y untouched.
"""
import numpy as np
import pytest

import oracle
from gated_deltanet_recurrence_conv_amd import workloads as W
from gpu_util import act_dtype, block_err, dev, dims_pair, host, tol, torch_mod

pytestmark = pytest.mark.gpu

EPS = 1e-6


def B():
    from gated_deltanet_recurrence_conv_amd import binding
    return binding


def norm_inputs(sh, seed):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((sh.L, sh.B, sh.T, sh.HV, sh.DV)).astype(np.float32)
    w = (1.0 + 0.1 * rng.standard_normal((sh.L, sh.DV))).astype(np.float32)
    if sh.act == "bf16":
        z, w = W.bf16_round(z), W.bf16_round(w)
    return z, w


def tok_err(x, ref):
    """normwise error per (layer, row, token, head) block of d_v values"""
    return block_err(x, ref, (-1,))


SHAPES = {
    "cohort": W.COHORT,
    "cohort_l2_dv64": W.COHORT.with_(L=2, DV=64, HV=8, HK=4),
    "t4_dv32": W.REWIND.with_(DV=32, HV=4, HK=2),
    "dk64_dv16": W.COHORT.with_(DK=64, DV=16, HV=4, HK=1, T=3, S=4),
    "tiny_f32": W.TINY,
}


@pytest.mark.parametrize("name", list(SHAPES))
def test_verify_gated_norm(name):
    torch = torch_mod()
    sh = SHAPES[name]
    inp = W.verify_inputs(sh, seed=9000 + len(name))
    z, w = norm_inputs(sh, 9100 + len(name))
    bd, od = dims_pair(sh)
    A = act_dtype(sh.act)
    act_np = inp.get("active")
    act = None if act_np is None else dev(act_np, torch.uint8)
    a = np.ones(sh.B, bool) if act_np is None else act_np.astype(bool)
    shp = (sh.L, sh.B, sh.T, sh.HV, sh.DV)
    common = [dev(inp["x"], A), dev(inp["conv_w"], A), None, dev(inp["conv_state"], A),
              dev(inp["g"], A), dev(inp["beta"], A)]
    cur = dev(inp["cur"], torch.int32)
    zd, wd = dev(z, A), dev(w, A)

    st1 = dev(inp["state"], torch.float32)
    y = torch.full(shp, float("nan"), device="cuda", dtype=act_dtype(sh.out))
    e1 = torch.zeros(1, dtype=torch.int32, device="cuda")
    B().gdn_verify_gated_norm(bd, *common, st1, cur, zd, wd, y, eps=EPS, active=act, err=e1)

    st2 = dev(inp["state"], torch.float32)
    o = torch.full(shp, float("nan"), device="cuda", dtype=act_dtype(sh.out))
    e2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    B().gdn_verify(bd, *common, st2, cur, o, act, e2)
    y2 = torch.full_like(o, float("nan"))
    B().gdn_gated_rmsnorm(bd, o, zd, wd, y2, eps=EPS, active=act)
    torch.cuda.synchronize()

    assert int(host(e1)[0]) == 0 and int(host(e2)[0]) == 0
    assert np.array_equal(host(st1), host(st2))             # candidates and snapshot
    yg = host(y).astype(np.float64)
    assert np.all(np.isnan(yg[:, ~a]))
    assert np.all(np.isfinite(yg[:, a]))

    st_ref, o_ref, err = oracle.verify(od, inp["x"], inp["conv_w"], None, inp["conv_state"],
                                       inp["g"], inp["beta"], inp["state"], inp["cur"], act_np)
    assert err == 0
    y_ref = oracle.gated_rmsnorm(od, o_ref, z, w, eps=float(np.float32(EPS)), active=act_np)
    e = tok_err(yg[:, a], y_ref[:, a])
    print("%s: y err vs oracle %.3e" % (name, e))
    assert e <= tol(sh.act)
    if sh.out == "f32":
        assert tok_err(yg[:, a], host(y2).astype(np.float64)[:, a]) <= 1e-5


def test_verify_gated_norm_bf16_output():
    """bf16 y: the norm is taken on the fp32 outputs, then rounded once, so y
    is within one bf16 unit of the fp32-output call's value."""
    torch = torch_mod()
    sh = W.COHORT.with_(HV=8, HK=4)
    inp = W.verify_inputs(sh, seed=9200)
    z, w = norm_inputs(sh, 9201)
    A = act_dtype(sh.act)
    shp = (sh.L, sh.B, sh.T, sh.HV, sh.DV)
    ys = {}
    for out in ("f32", "bf16"):
        bd, _ = dims_pair(sh, out=out)
        st = dev(inp["state"], torch.float32)
        y = torch.full(shp, float("nan"), device="cuda", dtype=act_dtype(out))
        B().gdn_verify_gated_norm(bd, dev(inp["x"], A), dev(inp["conv_w"], A), None,
                                  dev(inp["conv_state"], A), dev(inp["g"], A), dev(inp["beta"], A),
                                  st, dev(inp["cur"], torch.int32), dev(z, A), dev(w, A), y,
                                  eps=EPS, active=dev(inp["active"], torch.uint8))
        torch.cuda.synchronize()
        ys[out] = host(y).astype(np.float64)
    a = inp["active"].astype(bool)
    r = W.bf16_round(ys["f32"][:, a].astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(ys["bf16"][:, a] - r) <= np.abs(r) * 2 ** -7 + 1e-30)
    assert np.all(np.isnan(ys["bf16"][:, ~a]))


@pytest.mark.parametrize("shape", ["cohort", "rewind"])
def test_verify_lazy_gated_norm(shape):
    """The fused commit + verify with the norm epilogue against
    gdn_verify_lazy followed by gdn_gated_rmsnorm on the same inputs."""
    torch = torch_mod()
    sh = W.COHORT if shape == "cohort" else W.REWIND.with_(S=1)
    prev = W.verify_inputs(sh, seed=9300)
    new = W.verify_inputs(sh, seed=9301)
    rng = np.random.default_rng(9302)
    keep = rng.integers(0, sh.T + 1, size=sh.B).astype(np.int32)
    keep[0], keep[-1] = 0, sh.T
    cur = rng.integers(0, sh.S, size=(sh.L, sh.B)).astype(np.int32)
    active = new["active"] if new.get("active") is not None else np.ones(sh.B, np.uint8)
    z, w = norm_inputs(sh, 9303)
    bd, _ = dims_pair(sh)
    A = act_dtype(sh.act)
    shp = (sh.L, sh.B, sh.T, sh.HV, sh.DV)

    def run(fused):
        st = dev(prev["state"], torch.float32)
        cs = dev(prev["conv_state"], A)
        out = torch.full(shp, float("nan"), device="cuda", dtype=act_dtype(sh.out))
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        args = [bd, dev(prev["x"], A), dev(prev["g"], A), dev(prev["beta"], A), dev(keep),
                dev(new["x"], A), dev(prev["conv_w"], A), None, cs, dev(new["g"], A),
                dev(new["beta"], A), st, dev(cur, torch.int32)]
        if fused:
            B().gdn_verify_lazy_gated_norm(*args, dev(z, A), dev(w, A), out, eps=EPS,
                                           active=dev(active), err=err)
        else:
            B().gdn_verify_lazy(*args, out, dev(active), err)
            B().gdn_gated_rmsnorm(bd, out, dev(z, A), dev(w, A), out, eps=EPS, active=dev(active))
        torch.cuda.synchronize()
        assert int(host(err)[0]) == 0
        return host(st), host(cs), host(out).astype(np.float64)

    st1, cs1, y1 = run(True)
    st2, cs2, y2 = run(False)
    assert np.array_equal(st1, st2)
    assert np.array_equal(cs1, cs2)
    a = active.astype(bool)
    assert np.all(np.isnan(y1[:, ~a]))
    assert tok_err(y1[:, a], y2[:, a]) <= 1e-5
