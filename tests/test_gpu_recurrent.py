"""GPU parity of verify / commit / rewind against the CPU oracle, through the
C ABI, plus the bit-exact invariants the pages fix:

  * keep=0 and inactive rows leave the snapshot, conv cache and outputs
    untouched ("Add request-owned eight-way MTP serving for Qwen 35B", What
    was broken items 2 and 4);
  * a B8 cohort equals eight B1 calls (same page, item 6);
  * rewind over the accepted prefix equals the verify candidate and a direct
    forward ("perf(qwen): full-context MTP draft prefill and replay-free
    rewind", Summary item 4 and Tests);
  * prefix windows agree (no look-ahead).

Tolerance (normwise per (layer, row, head) block): 2e-3 with bf16 inputs and
fp32 state, 1e-5 with fp32 inputs; integer and copied data bit-exact.
"""
import numpy as np
import pytest

import oracle
from gated_deltanet_recurrence_conv_amd import workloads as W
from gpu_util import (act_dtype, dev, dims_pair, host, out_err, state_err, tol, torch_mod)

pytestmark = pytest.mark.gpu


def B():
    from gated_deltanet_recurrence_conv_amd import binding
    return binding


class Run:
    """Device copies of one verify workload."""

    def __init__(self, sh, inp, out=None):
        torch = torch_mod()
        A = act_dtype(sh.act)
        self.sh = sh
        self.x = dev(inp["x"], A)
        self.w = dev(inp["conv_w"], A)
        self.cs = dev(inp["conv_state"], A)
        self.g = dev(inp["g"], A)
        self.beta = dev(inp["beta"], A)
        self.state = dev(inp["state"], torch.float32)
        self.cur = dev(inp["cur"], torch.int32)
        self.active = dev(inp["active"], torch.uint8)
        out = sh.out if out is None else out
        self.o = torch.full((sh.L, sh.B, sh.T, sh.HV, sh.DV), float("nan"), device="cuda",
                            dtype=act_dtype(out))
        self.err = torch.zeros(1, dtype=torch.int32, device="cuda")


def run_verify(r, bd, active=True):
    B().gdn_verify(bd, r.x, r.w, None, r.cs, r.g, r.beta, r.state, r.cur, r.o,
                   r.active if active else None, r.err)


def oracle_verify(od, inp, active=True):
    return oracle.verify(od, inp["x"], inp["conv_w"], None, inp["conv_state"], inp["g"],
                         inp["beta"], inp["state"], inp["cur"],
                         inp["active"] if active else None)


def test_library_is_the_native_one():
    b = B()
    assert "gfx950" in b.gdn_version()
    torch = torch_mod()
    assert torch.cuda.get_device_properties(0).gcnArchName.startswith("gfx950")


@pytest.mark.parametrize("keep", [0, 1, 2])
def test_tiny_fp32_all_keeps(keep):
    """The tiny case: B=1, 2 value heads, 1 qk head, d=16, T=2, fp32; every keep."""
    sh = W.TINY
    inp = W.verify_inputs(sh, seed=1000)
    bd, od = dims_pair(sh)
    r = Run(sh, inp)
    run_verify(r, bd)
    torch_mod().cuda.synchronize()
    st_ref, o_ref, err = oracle_verify(od, inp)
    assert err == 0 and int(host(r.err)[0]) == 0
    assert out_err(host(r.o), o_ref) <= 1e-5
    assert state_err(host(r.state), st_ref) <= 1e-5
    # the snapshot slot is bit-identical
    assert np.array_equal(host(r.state)[:, :, 0], inp["state"][:, :, 0])
    keep_a = np.full(sh.B, keep, np.int32)
    B().gdn_commit(bd, r.x, r.cs, r.cur, dev(keep_a), r.active, r.err)
    cs_ref, cur_ref, err = oracle.commit(od, inp["x"], inp["conv_state"], inp["cur"], keep_a,
                                         inp["active"])
    assert err == 0 and int(host(r.err)[0]) == 0
    assert np.array_equal(host(r.cur), cur_ref)
    assert np.array_equal(host(r.cs).astype(np.float64), cs_ref)
    if keep == 0:
        assert np.array_equal(host(r.cs), inp["conv_state"])
    # the committed slot holds the oracle's state after `keep` tokens
    c = int(host(r.cur)[0, 0])
    ref_committed = inp["state"][0, 0, 0] if keep == 0 else st_ref[0, 0, keep]
    assert state_err(host(r.state)[0, 0, c], ref_committed) <= 1e-5


def test_cohort_b8_t2_bf16_verify_commit():
    """The B8/T2 verify cohort: 32 value heads, 16 qk heads, d=128, bf16
    inputs, fp32 state; rows 1 and 6 inactive; keep ~ U{0,1,2}."""
    sh = W.COHORT
    inp = W.verify_inputs(sh, seed=1001)
    bd, od = dims_pair(sh)
    r = Run(sh, inp)
    snap = host(r.state).copy()
    run_verify(r, bd)
    torch_mod().cuda.synchronize()
    st_ref, o_ref, err = oracle_verify(od, inp)
    st_gpu, o_gpu = host(r.state), host(r.o)
    act = inp["active"].astype(bool)
    assert int(host(r.err)[0]) == 0
    assert out_err(o_gpu[:, act], o_ref[:, act]) <= 2e-3
    assert state_err(st_gpu[:, act], st_ref[:, act]) <= 2e-3
    # inactive rows: every candidate slot and every output untouched
    assert np.array_equal(st_gpu[:, ~act], snap[:, ~act])
    assert np.all(np.isnan(o_gpu[:, ~act]))
    # snapshot slot of every row untouched
    assert np.array_equal(st_gpu[:, :, 0], snap[:, :, 0])
    rng = np.random.default_rng(7)
    keep = W.keep_uniform(rng, sh, inp["active"])
    B().gdn_commit(bd, r.x, r.cs, r.cur, dev(keep), r.active, r.err)
    cs_ref, cur_ref, err = oracle.commit(od, inp["x"], inp["conv_state"], inp["cur"], keep,
                                         inp["active"])
    assert err == 0 and int(host(r.err)[0]) == 0
    assert np.array_equal(host(r.cur), cur_ref)
    assert np.array_equal(host(r.cs).astype(np.float64), cs_ref)


def test_cohort_equals_eight_solo_rows_bit_exact():
    sh = W.COHORT.with_(inactive=())
    inp = W.verify_inputs(sh, seed=1002)
    bd, _ = dims_pair(sh)
    r = Run(sh, inp)
    run_verify(r, bd)
    torch = torch_mod()
    for b in range(sh.B):
        one = {k: (v[:, b:b + 1] if k not in ("conv_w", "active") else v)
               for k, v in inp.items()}
        one["active"] = inp["active"][b:b + 1]
        sh1 = sh.with_(B=1)
        bd1, _ = dims_pair(sh1)
        r1 = Run(sh1, one)
        run_verify(r1, bd1)
        torch.cuda.synchronize()
        assert np.array_equal(host(r1.state)[:, 0], host(r.state)[:, b])
        assert np.array_equal(host(r1.o)[:, 0], host(r.o)[:, b])


def test_prefix_windows_bit_exact():
    sh = W.REWIND.with_(B=2)
    inp = W.verify_inputs(sh, seed=1003)
    bd, _ = dims_pair(sh)
    r = Run(sh, inp)
    run_verify(r, bd)
    for t in range(1, sh.T):
        sub = dict(inp)
        for k in ("x", "g", "beta"):
            sub[k] = np.ascontiguousarray(inp[k][:, :, :t])
        sht = sh.with_(T=t)
        bdt, _ = dims_pair(sht, S=sh.S)
        rt = Run(sht.with_(S=sh.S), sub)
        run_verify(rt, bdt)
        torch_mod().cuda.synchronize()
        assert np.array_equal(host(rt.state)[:, :, t], host(r.state)[:, :, t])
        assert np.array_equal(host(rt.o), host(r.o)[:, :, :t])


def test_rewind_b8_t4_parity_and_equals_candidate():
    """Replay-free rewind: B=8, T=4 captured inputs, keep ~ U{0..4}."""
    sh = W.REWIND
    inp = W.verify_inputs(sh, seed=1004)
    rng = np.random.default_rng(11)
    keep = W.keep_uniform(rng, sh)
    keep[0], keep[1] = 0, sh.T          # make sure both ends appear
    inp["cur"] = rng.integers(0, sh.S, size=(sh.L, sh.B)).astype(np.int32)
    bd, od = dims_pair(sh)
    # verify (for the candidates) on one copy, rewind on another
    rv = Run(sh, inp)
    run_verify(rv, bd, active=False)
    rr = Run(sh, inp)
    snap = host(rr.state).copy()
    B().gdn_rewind(bd, rr.x, rr.w, None, rr.cs, rr.g, rr.beta, rr.state, rr.cur, dev(keep),
                   rr.o, rr.err)
    torch_mod().cuda.synchronize()
    assert int(host(rr.err)[0]) == 0
    st_ref, cs_ref, o_ref, err = oracle.rewind(od, inp["x"], inp["conv_w"], None,
                                               inp["conv_state"], inp["g"], inp["beta"],
                                               inp["state"], inp["cur"], keep)
    assert err == 0
    st_gpu, st_ver = host(rr.state), host(rv.state)
    o_gpu, o_ver = host(rr.o), host(rv.o)
    assert np.array_equal(host(rr.cs).astype(np.float64), cs_ref)
    assert np.array_equal(host(rr.cur), inp["cur"])
    for b in range(sh.B):
        c0 = int(inp["cur"][0, b])
        k = int(keep[b])
        if k == 0:
            assert np.array_equal(st_gpu[:, b], snap[:, b])
            assert np.all(np.isnan(o_gpu[:, b]))
            continue
        assert state_err(st_gpu[:, b, c0], st_ref[:, b, c0]) <= 2e-3
        assert out_err(o_gpu[:, b:b + 1, :k], o_ref[:, b:b + 1, :k]) <= 2e-3
        # bit-identical to the verify candidate after k tokens
        assert np.array_equal(st_gpu[:, b, c0], st_ver[:, b, (c0 + k) % sh.S])
        assert np.array_equal(o_gpu[:, b, :k], o_ver[:, b, :k])
        # other slots untouched
        others = [s for s in range(sh.S) if s != c0]
        assert np.array_equal(st_gpu[:, b, others], snap[:, b, others])


@pytest.mark.parametrize("DK,DV,HV,HK", [(16, 16, 4, 2), (128, 16, 4, 2), (16, 128, 4, 2),
                                         (32, 64, 4, 4), (64, 128, 8, 2), (128, 128, 2, 1)])
def test_rewind_head_shapes_fp32(DK, DV, HV, HK):
    """Rewind over head shapes and value heads per qk head (fp32, 1e-5), with
    and without outputs: the state, conv cache and outputs against the oracle,
    and the two runs' states and caches bit-identical.  (64, 128, 8, 2) needs
    more waves per qk head than one workgroup holds (the conv cache is then
    shifted by a second launch)."""
    sh = W.Shape("rw_dims", L=2, B=4, T=4, HV=HV, HK=HK, DK=DK, DV=DV, S=3, act="f32")
    inp = W.verify_inputs(sh, seed=1300 + DK + DV + HV)
    rng = np.random.default_rng(DK + DV + HV)
    keep = np.array([0, 1, sh.T, 2], np.int32)
    inp["cur"] = rng.integers(0, sh.S, size=(sh.L, sh.B)).astype(np.int32)
    bd, od = dims_pair(sh, scale=DK ** -0.5)
    st_ref, cs_ref, o_ref, err = oracle.rewind(od, inp["x"], inp["conv_w"], None,
                                               inp["conv_state"], inp["g"], inp["beta"],
                                               inp["state"], inp["cur"], keep)
    assert err == 0
    runs = []
    for with_o in (True, False):
        r = Run(sh, inp)
        B().gdn_rewind(bd, r.x, r.w, None, r.cs, r.g, r.beta, r.state, r.cur, dev(keep),
                       r.o if with_o else None, r.err)
        torch_mod().cuda.synchronize()
        assert int(host(r.err)[0]) == 0
        runs.append(r)
        assert np.array_equal(host(r.cs).astype(np.float64), cs_ref)
        st = host(r.state)
        for b in range(sh.B):
            c0 = inp["cur"][:, b]
            for l in range(sh.L):
                if keep[b] == 0:
                    assert np.array_equal(st[l, b], inp["state"][l, b])
                else:
                    assert state_err(st[l, b, c0[l]], st_ref[l, b, c0[l]]) <= 1e-5
        if with_o:
            o = host(r.o)
            for b in range(sh.B):
                k = int(keep[b])
                if k:
                    assert out_err(o[:, b:b + 1, :k], o_ref[:, b:b + 1, :k]) <= 1e-5
                assert np.all(np.isnan(o[:, b, k:]))
    assert np.array_equal(host(runs[0].state), host(runs[1].state))
    assert np.array_equal(host(runs[0].cs), host(runs[1].cs))


@pytest.mark.parametrize("DK,DV", [(16, 16), (16, 32), (32, 16), (32, 64), (64, 32),
                                   (64, 128), (128, 64), (128, 16), (16, 128)])
def test_head_dims_fp32(DK, DV):
    sh = W.Shape("dims", L=2, B=3, T=3, HV=4, HK=2, DK=DK, DV=DV, S=4, act="f32",
                 inactive=(1,))
    inp = W.verify_inputs(sh, seed=1005 + DK + DV)
    inp["cur"] = np.array([[0, 1, 3], [2, 0, 1]], np.int32)
    bd, od = dims_pair(sh, scale=DK ** -0.5)
    r = Run(sh, inp)
    run_verify(r, bd)
    torch_mod().cuda.synchronize()
    st_ref, o_ref, err = oracle_verify(od, inp)
    act = inp["active"].astype(bool)
    assert out_err(host(r.o)[:, act], o_ref[:, act]) <= 1e-5
    assert state_err(host(r.state), st_ref) <= 1e-5


def test_bias_no_silu_no_l2_bf16_out():
    sh = W.Shape("bias", L=1, B=2, T=2, HV=4, HK=4, DK=32, DV=32, S=3, act="f32", out="bf16")
    inp = W.verify_inputs(sh, seed=1010)
    rng = np.random.default_rng(3)
    cb = (0.2 * rng.standard_normal((1, sh.C))).astype(np.float32)
    for flags in (0, 1, 2):
        bd, od = dims_pair(sh, flags=flags)
        r = Run(sh, inp)
        B().gdn_verify(bd, r.x, r.w, dev(cb), r.cs, r.g, r.beta, r.state, r.cur, r.o, None,
                       r.err)
        torch_mod().cuda.synchronize()
        st_ref, o_ref, _ = oracle.verify(od, inp["x"], inp["conv_w"], cb, inp["conv_state"],
                                         inp["g"], inp["beta"], inp["state"], inp["cur"])
        assert state_err(host(r.state), st_ref) <= 1e-5
        # bf16 outputs: within one bf16 unit in the last place of the oracle's value
        o = host(r.o).astype(np.float64)
        ulp = np.abs(W.bf16_round(o_ref.astype(np.float32))).astype(np.float64) * 2.0 ** -7
        assert np.all(np.abs(o - o_ref) <= ulp + 1e-30)


def test_device_error_bits_leave_rows_untouched():
    sh = W.Shape("err", L=1, B=3, T=2, HV=2, HK=1, DK=16, DV=16, S=3, act="f32")
    inp = W.verify_inputs(sh, seed=1011)
    inp["active"] = np.array([1, 0, 1], np.uint8)
    inp["cur"] = np.array([[0, 0, 5]], np.int32)      # row 2: slot out of range
    bd, od = dims_pair(sh)
    r = Run(sh, inp)
    snap = host(r.state).copy()
    run_verify(r, bd)
    torch_mod().cuda.synchronize()
    assert int(host(r.err)[0]) == 2
    assert np.array_equal(host(r.state)[:, 2], snap[:, 2])
    keep = np.array([3, 1, 1], np.int32)                # bad keep, inactive keep, bad slot
    r.err.zero_()
    B().gdn_commit(bd, r.x, r.cs, r.cur, dev(keep), r.active, r.err)
    torch_mod().cuda.synchronize()
    _, cur_ref, err = oracle.commit(od, inp["x"], inp["conv_state"], inp["cur"], keep,
                                    inp["active"])
    assert int(host(r.err)[0]) == err == 7
    assert np.array_equal(host(r.cur), inp["cur"])
    assert np.array_equal(host(r.cs), inp["conv_state"])
    r.err.zero_()
    B().gdn_rewind(bd, r.x, r.w, None, r.cs, r.g, r.beta, r.state, r.cur,
                   dev(np.array([-1, 0, 1], np.int32)), None, r.err)
    torch_mod().cuda.synchronize()
    assert int(host(r.err)[0]) == 3
    assert np.array_equal(host(r.cs), inp["conv_state"])


def test_nan_in_one_row_stays_in_that_row():
    sh = W.COHORT.with_(inactive=())
    inp = W.verify_inputs(sh, seed=1012)
    bd, _ = dims_pair(sh)
    ra = Run(sh, inp)
    run_verify(ra, bd)
    bad = dict(inp)
    bad["state"] = inp["state"].copy()
    bad["state"][0, 3, 0, 5, 7, 9] = np.nan
    rb = Run(sh, bad)
    run_verify(rb, bd)
    torch_mod().cuda.synchronize()
    sa, sb = host(ra.state), host(rb.state)
    others = [b for b in range(sh.B) if b != 3]
    assert np.array_equal(sa[:, others], sb[:, others])
    assert np.array_equal(host(ra.o)[:, others], host(rb.o)[:, others])


def test_run_twice_identical():
    sh = W.COHORT
    inp = W.verify_inputs(sh, seed=1013)
    bd, _ = dims_pair(sh)
    r1, r2 = Run(sh, inp), Run(sh, inp)
    run_verify(r1, bd)
    run_verify(r2, bd)
    torch_mod().cuda.synchronize()
    assert np.array_equal(host(r1.state), host(r2.state))
    assert np.array_equal(host(r1.o), host(r2.o), equal_nan=True)


def test_solo_b1_t3_thirty_layers_carried_cycles():
    """B=1, T=3, 30 independent layers in one grouped call, keep by prefix
    acceptance p=0.8, state carried over 12 cycles; all layers checked."""
    sh = W.SOLO
    torch = torch_mod()
    inputs = [W.verify_inputs(sh, seed=2000 + i) for i in range(4)]
    state0 = inputs[0]["state"]
    cs0 = inputs[0]["conv_state"]
    bd, od = dims_pair(sh)
    A = act_dtype(sh.act)
    st_d = dev(state0, torch.float32)
    cs_d = dev(cs0, A)
    cur_d = torch.zeros((sh.L, sh.B), dtype=torch.int32, device="cuda")
    o_d = torch.empty((sh.L, sh.B, sh.T, sh.HV, sh.DV), dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    st_h, cs_h, cur_h = state0.astype(np.float64), cs0.astype(np.float64), np.zeros((sh.L, sh.B), np.int32)
    rng = np.random.default_rng(5)
    dev_in = [{k: dev(v, A) for k, v in inp.items() if k in ("x", "conv_w", "g", "beta")}
              for inp in inputs]
    for c in range(12):
        inp, di = inputs[c % 4], dev_in[c % 4]
        keep = W.keep_prefix_acceptance(rng, sh)
        B().gdn_verify(bd, di["x"], di["conv_w"], None, cs_d, di["g"], di["beta"], st_d, cur_d,
                       o_d, None, err)
        B().gdn_commit(bd, di["x"], cs_d, cur_d, dev(keep), None, err)
        st_h, o_ref, e1 = oracle.verify(od, inp["x"], inp["conv_w"], None, cs_h, inp["g"],
                                        inp["beta"], st_h, cur_h)
        cs_h, cur_h, e2 = oracle.commit(od, inp["x"], cs_h, cur_h, keep)
        assert e1 == 0 and e2 == 0
        torch.cuda.synchronize()
        assert out_err(host(o_d), o_ref) <= 2e-3, c
    assert int(host(err)[0]) == 0
    assert np.array_equal(host(cur_d), cur_h)
    assert np.array_equal(host(cs_d).astype(np.float64), cs_h)
    sg = host(st_d)
    for l in range(sh.L):
        c0 = int(cur_h[l, 0])
        assert state_err(sg[l, 0, c0], st_h[l, 0, c0]) <= 2e-3


def test_graph_replay_matches_eager():
    """Per-layer verify launches plus a grouped commit captured in a HIP
    graph: every replay (with eager work in between) equals the same cycle
    run eagerly, bit for bit."""
    torch = torch_mod()
    sh = W.COHORT.with_(L=3)
    inp = W.verify_inputs(sh, seed=1020)
    A = act_dtype(sh.act)
    d1, _ = dims_pair(sh, L=1)
    dL, _ = dims_pair(sh)

    def pool():
        return dict(x=dev(inp["x"], A), w=dev(inp["conv_w"], A), cs=dev(inp["conv_state"], A),
                    g=dev(inp["g"], A), be=dev(inp["beta"], A),
                    st=dev(inp["state"], torch.float32), cur=dev(inp["cur"], torch.int32),
                    act=dev(inp["active"], torch.uint8),
                    o=torch.zeros((sh.L, sh.B, sh.T, sh.HV, sh.DV), device="cuda"))

    def cycle(t, keep):
        for l in range(sh.L):
            sl = slice(l, l + 1)
            B().gdn_verify(d1, t["x"][sl], t["w"][sl], None, t["cs"][sl], t["g"][sl],
                           t["be"][sl], t["st"][sl], t["cur"][sl], t["o"][sl], t["act"])
        B().gdn_commit(dL, t["x"], t["cs"], t["cur"], keep, t["act"])

    eager, graphed = pool(), pool()
    keep_cur = torch.zeros(sh.B, dtype=torch.int32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        cycle(graphed, keep_cur)
    torch.cuda.synchronize()
    # capture does not execute: reset the graphed pool to the inputs
    for k, v in pool().items():
        graphed[k].copy_(v)
    rng = np.random.default_rng(9)
    junk = torch.randn(512, 512, device="cuda")
    for it in range(4):
        keep = dev(W.keep_uniform(rng, sh, inp["active"]), torch.int32)
        cycle(eager, keep)
        keep_cur.copy_(keep)
        graph.replay()
        junk = junk @ junk.T / 512.0          # unrelated eager work between replays
        torch.cuda.synchronize()
        for k in ("st", "cur", "cs", "o"):
            assert torch.equal(eager[k], graphed[k]), (it, k)
