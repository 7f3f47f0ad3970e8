"""GPU tests of the fused commit + verify (gdn_verify_lazy) through the C ABI.

"MTP inference: review and commit structure" (eole docs), Functional commits
item 2 and Verification and limits: a partial commit replays only the
accepted recurrent prefix.  gdn_verify_lazy(previous window, keep_prev, new
window) is defined as gdn_rewind(previous window, keep_prev) followed by
gdn_verify(new window) without candidate writes, so it is checked

  * bit for bit against those two GPU calls (same kernel arithmetic),
  * against the oracle's rewind followed by its verify (2e-3 with bf16
    inputs and fp32 state, 1e-5 with fp32 inputs),
  * over several decode cycles against the eager verify + commit ring, with a
    final rewind as the flush,

plus its edge cases: no previous window, inactive rows, device error bits.
"""
import numpy as np
import pytest

import oracle
from gated_deltanet_recurrence_conv_amd import workloads as W
from gpu_util import act_dtype, dev, dims_pair, host, out_err, state_err, tol, torch_mod

pytestmark = pytest.mark.gpu


def B():
    from gated_deltanet_recurrence_conv_amd import binding
    return binding


def two_windows(sh, seed):
    """A previous and a new window of the same shape sharing conv weights,
    conv cache and state; keep_prev over 0..T with both ends present."""
    prev = W.verify_inputs(sh, seed=seed)
    new = W.verify_inputs(sh, seed=seed + 1)
    rng = np.random.default_rng(seed + 2)
    keep = rng.integers(0, sh.T + 1, size=sh.B).astype(np.int32)
    keep[0], keep[-1] = 0, sh.T
    cur = rng.integers(0, sh.S, size=(sh.L, sh.B)).astype(np.int32)
    return prev, new, keep, cur


class Dev:
    def __init__(self, sh, prev, new, cur, active):
        torch = torch_mod()
        A = act_dtype(sh.act)
        self.xp, self.gp, self.bp = dev(prev["x"], A), dev(prev["g"], A), dev(prev["beta"], A)
        self.x, self.g, self.b = dev(new["x"], A), dev(new["g"], A), dev(new["beta"], A)
        self.w = dev(prev["conv_w"], A)
        self.cs = dev(prev["conv_state"], A)
        self.state = dev(prev["state"], torch.float32)
        self.cur = dev(cur, torch.int32)
        self.active = dev(active, torch.uint8)
        self.o = torch.full((sh.L, sh.B, sh.T, sh.HV, sh.DV), float("nan"), device="cuda",
                            dtype=act_dtype(sh.out))
        self.err = torch.zeros(1, dtype=torch.int32, device="cuda")


def lazy(r, bd, keep):
    B().gdn_verify_lazy(bd, r.xp, r.gp, r.bp, None if keep is None else dev(keep), r.x, r.w,
                        None, r.cs, r.g, r.b, r.state, r.cur, r.o, r.active, r.err)


# Head shapes beyond the cohort's, fp32 (1e-5): value heads per qk head times
# column slices per head sets how many waves a qk head's workgroup holds; the
# g4 shapes have more than one workgroup holds, so their conv cache is shifted
# by a second launch.  The kernel is built for windows of T <= 2 and of
# T <= 4 separately; both sizes run in both layouts (T = 1 and 2, T = 3 and 4).
DIM_SHAPES = {
    "cohort": W.COHORT,
    "rewind": W.REWIND,
    "d16_g2": W.Shape("d16_g2", L=2, B=3, T=3, HV=4, HK=2, DK=16, DV=16, S=4, act="f32", inactive=(1,)),
    "k128_v16": W.Shape("k128_v16", L=2, B=3, T=3, HV=4, HK=2, DK=128, DV=16, S=4, act="f32", inactive=(1,)),
    "k16_v128": W.Shape("k16_v128", L=2, B=3, T=4, HV=4, HK=2, DK=16, DV=128, S=5, act="f32"),
    "g1_v64": W.Shape("g1_v64", L=2, B=3, T=2, HV=4, HK=4, DK=32, DV=64, S=4, act="f32", inactive=(2,)),
    "g4_v128": W.Shape("g4_v128", L=2, B=3, T=3, HV=8, HK=2, DK=64, DV=128, S=4, act="f32"),
    "t1_k32": W.Shape("t1_k32", L=2, B=3, T=1, HV=4, HK=2, DK=32, DV=32, S=2, act="f32", inactive=(1,)),
    "t4_g4": W.Shape("t4_g4", L=2, B=3, T=4, HV=8, HK=2, DK=32, DV=128, S=5, act="f32", inactive=(2,)),
    "t1_g4": W.Shape("t1_g4", L=1, B=4, T=1, HV=8, HK=2, DK=64, DV=128, S=3, act="f32"),
}


@pytest.mark.parametrize("shape", list(DIM_SHAPES))
def test_lazy_equals_rewind_then_verify(shape):
    sh = DIM_SHAPES[shape]
    prev, new, keep, cur = two_windows(sh, 5100 + 100 * list(DIM_SHAPES).index(shape))
    active = new["active"]
    bd, od = dims_pair(sh)
    torch = torch_mod()
    ra = Dev(sh, prev, new, cur, active)
    snap = host(ra.state).copy()
    lazy(ra, bd, keep)
    # the same cycle as two calls
    rb = Dev(sh, prev, new, cur, active)
    B().gdn_rewind(bd, rb.xp, rb.w, None, rb.cs, rb.gp, rb.bp, rb.state, rb.cur, dev(keep),
                   None, rb.err)
    B().gdn_verify(bd, rb.x, rb.w, None, rb.cs, rb.g, rb.b, rb.state, rb.cur, rb.o, rb.active,
                   rb.err)
    torch.cuda.synchronize()
    assert int(host(ra.err)[0]) == 0 and int(host(rb.err)[0]) == 0
    sa, sb = host(ra.state), host(rb.state)
    assert np.array_equal(host(ra.cs), host(rb.cs))
    assert np.array_equal(host(ra.cur), cur)
    oa, ob = host(ra.o), host(rb.o)
    for b in range(sh.B):
        for l in range(sh.L):
            c0 = int(cur[l, b])
            assert np.array_equal(sa[l, b, c0], sb[l, b, c0])
            others = [s for s in range(sh.S) if s != c0]
            assert np.array_equal(sa[l, b, others], snap[l, b, others])   # no candidates
            if keep[b] == 0:
                assert np.array_equal(sa[l, b, c0], snap[l, b, c0])
        if active[b]:
            assert np.array_equal(oa[:, b], ob[:, b])
        else:
            assert np.all(np.isnan(oa[:, b]))
    # against the oracle: rewind, then verify from the committed state
    st1, cs1, _, e1 = oracle.rewind(od, prev["x"], prev["conv_w"], None, prev["conv_state"],
                                    prev["g"], prev["beta"], prev["state"], cur, keep)
    assert e1 == 0
    st2, o2, e2 = oracle.verify(od, new["x"], prev["conv_w"], None, cs1, new["g"], new["beta"],
                                st1, cur, active)
    assert e2 == 0
    assert np.array_equal(host(ra.cs).astype(np.float64), cs1)
    for b in range(sh.B):
        for l in range(sh.L):
            c0 = int(cur[l, b])
            assert state_err(sa[l, b, c0], st1[l, b, c0]) <= tol(sh.act)
        if active[b]:
            assert out_err(oa[:, b:b + 1], o2[:, b:b + 1]) <= tol(sh.act)


def test_lazy_tiny_fp32_against_oracle():
    sh = W.TINY.with_(B=3, T=3, S=1)
    prev, new, keep, cur = two_windows(sh, 5300)
    active = np.array([1, 0, 1], np.uint8)
    keep[1] = 2                       # an inactive row still commits its previous window
    bd, od = dims_pair(sh)
    r = Dev(sh, prev, new, cur, active)
    lazy(r, bd, keep)
    torch_mod().cuda.synchronize()
    assert int(host(r.err)[0]) == 0
    st1, cs1, _, _ = oracle.rewind(od, prev["x"], prev["conv_w"], None, prev["conv_state"],
                                   prev["g"], prev["beta"], prev["state"], cur, keep)
    # the oracle's verify writes candidates, so it runs on a copy with T spare slots
    _, od_v = dims_pair(sh, S=sh.T + 1)
    ring = np.concatenate([st1] + [np.zeros_like(st1)] * sh.T, axis=2)
    _, o2, _ = oracle.verify(od_v, new["x"], prev["conv_w"], None, cs1, new["g"], new["beta"],
                             ring, cur, active)
    assert state_err(host(r.state), st1) <= 1e-5
    assert np.array_equal(host(r.cs).astype(np.float64), cs1)
    o = host(r.o)
    assert out_err(o[:, [0, 2]], o2[:, [0, 2]]) <= 1e-5
    assert np.all(np.isnan(o[:, 1]))


def test_lazy_without_previous_window_is_verify_without_candidates():
    sh = W.COHORT
    prev, new, keep, cur = two_windows(sh, 5400)
    active = new["active"]
    bd, _ = dims_pair(sh)
    r = Dev(sh, prev, new, cur, active)
    snap, cs0 = host(r.state).copy(), host(r.cs).copy()
    lazy(r, bd, None)
    rv = Dev(sh, prev, new, cur, active)
    B().gdn_verify(bd, rv.x, rv.w, None, rv.cs, rv.g, rv.b, rv.state, rv.cur, rv.o, rv.active,
                   rv.err)
    torch_mod().cuda.synchronize()
    assert int(host(r.err)[0]) == 0
    assert np.array_equal(host(r.state), snap)       # nothing written, no candidates
    assert np.array_equal(host(r.cs), cs0)
    o, ov = host(r.o), host(rv.o)
    a = active.astype(bool)
    assert np.array_equal(o[:, a], ov[:, a])
    assert np.all(np.isnan(o[:, ~a]))


def test_lazy_cycles_match_eager_ring():
    """Twelve B1/T3 cycles over 4 layers: lazy in place (S = 1) against
    verify + commit on the ring (S = 4); outputs bit-exact every cycle, and
    after a final rewind flush the committed state and conv cache are equal."""
    torch = torch_mod()
    sh = W.SOLO.with_(L=4)
    ncyc = 12
    wins = [W.verify_inputs(sh, seed=5500 + c) for c in range(ncyc)]
    rng = np.random.default_rng(5599)
    keeps = [W.keep_prefix_acceptance(rng, sh) for _ in range(ncyc)]
    A = act_dtype(sh.act)
    bd_ring, _ = dims_pair(sh)
    bd_lazy, _ = dims_pair(sh, S=1)
    w = dev(wins[0]["conv_w"], A)
    cs_e, cs_l = dev(wins[0]["conv_state"], A), dev(wins[0]["conv_state"], A)
    st0 = wins[0]["state"][:, :, :1]
    st_e = dev(np.concatenate([st0] + [np.zeros_like(st0)] * (sh.S - 1), axis=2), torch.float32)
    st_l = dev(st0, torch.float32)
    cur_e = torch.zeros((sh.L, sh.B), dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    xs = [dev(wn["x"], A) for wn in wins]
    gs = [dev(wn["g"], A) for wn in wins]
    bs = [dev(wn["beta"], A) for wn in wins]
    ks = [dev(k) for k in keeps]
    for c in range(ncyc):
        o_e = torch.empty((sh.L, sh.B, sh.T, sh.HV, sh.DV), device="cuda")
        o_l = torch.empty_like(o_e)
        B().gdn_verify(bd_ring, xs[c], w, None, cs_e, gs[c], bs[c], st_e, cur_e, o_e, None, err)
        B().gdn_commit(bd_ring, xs[c], cs_e, cur_e, ks[c], None, err)
        if c == 0:
            B().gdn_verify_lazy(bd_lazy, None, None, None, None, xs[c], w, None, cs_l, gs[c],
                                bs[c], st_l, None, o_l, None, err)
        else:
            B().gdn_verify_lazy(bd_lazy, xs[c - 1], gs[c - 1], bs[c - 1], ks[c - 1], xs[c], w,
                                None, cs_l, gs[c], bs[c], st_l, None, o_l, None, err)
        torch.cuda.synchronize()
        assert np.array_equal(host(o_l), host(o_e)), "cycle %d" % c
    B().gdn_rewind(bd_lazy, xs[-1], w, None, cs_l, gs[-1], bs[-1], st_l, None, ks[-1], None, err)
    torch.cuda.synchronize()
    assert int(host(err)[0]) == 0
    ce = host(cur_e)
    se, sl = host(st_e), host(st_l)
    for l in range(sh.L):
        for b in range(sh.B):
            assert np.array_equal(sl[l, b, 0], se[l, b, int(ce[l, b])])
    assert np.array_equal(host(cs_l), host(cs_e))


def test_lazy_error_bits_leave_rows_untouched():
    sh = W.COHORT
    prev, new, keep, cur = two_windows(sh, 5600)
    active = np.ones(sh.B, np.uint8)
    keep[2] = sh.T + 1                # keep out of range
    cur[0, 4] = sh.S                  # slot out of range
    bd, _ = dims_pair(sh)
    r = Dev(sh, prev, new, cur, active)
    snap, cs0 = host(r.state).copy(), host(r.cs).copy()
    lazy(r, bd, keep)
    torch_mod().cuda.synchronize()
    e = int(host(r.err)[0])
    assert e & 1 and e & 2
    o = host(r.o)
    for b in (2, 4):
        assert np.array_equal(host(r.state)[:, b], snap[:, b])
        assert np.array_equal(host(r.cs)[:, b], cs0[:, b])
        assert np.all(np.isnan(o[:, b]))


def test_device_resident_decode_loop_in_a_graph():
    """A decode loop that never leaves the device, as the greedy cohort route
    of "Add request-owned eight-way MTP serving for Qwen 35B" (Follow-up)
    runs it: each cycle commits the previous window and verifies the new one
    (gdn_verify_lazy), then accepts greedily (gdn_accept_greedy) into the keep
    the next cycle commits.  Six cycles captured in one HIP graph and replayed
    from the same start state equal the same calls made eagerly, bit for bit,
    on every replay."""
    torch = torch_mod()
    sh = W.COHORT.with_(L=2, S=1)
    ncyc = 6
    A = act_dtype(sh.act)
    bd, _ = dims_pair(sh)
    wins = [W.verify_inputs(sh, seed=5700 + c) for c in range(ncyc)]
    rng = np.random.default_rng(5799)
    xs = [dev(wn["x"], A) for wn in wins]
    gs = [dev(wn["g"], A) for wn in wins]
    bs = [dev(wn["beta"], A) for wn in wins]
    targets, drafts = [], []
    for _ in range(ncyc):
        t = rng.integers(0, 151_000, size=(sh.B, sh.T)).astype(np.int32)
        dr = t[:, :sh.T - 1].copy()
        miss = rng.random(dr.shape) > 0.7
        dr[miss] += 1
        targets.append(dev(t))
        drafts.append(dev(dr))
    act = dev(wins[0]["active"], torch.uint8)
    w = dev(wins[0]["conv_w"], A)
    cs0 = dev(wins[0]["conv_state"], A)
    st0 = dev(wins[0]["state"], torch.float32)

    def fresh():
        return dict(cs=cs0.clone(), st=st0.clone(),
                    keep=torch.zeros(sh.B, dtype=torch.int32, device="cuda"),
                    nxt=torch.zeros(sh.B, dtype=torch.int32, device="cuda"),
                    o=torch.zeros((ncyc,) + (sh.L, sh.B, sh.T, sh.HV, sh.DV), device="cuda"),
                    err=torch.zeros(1, dtype=torch.int32, device="cuda"))

    def loop(r):
        for c in range(ncyc):
            prev = c > 0
            B().gdn_verify_lazy(bd, xs[c - 1] if prev else None, gs[c - 1] if prev else None,
                                bs[c - 1] if prev else None, r["keep"] if prev else None, xs[c], w,
                                None, r["cs"], gs[c], bs[c], r["st"], None, r["o"][c], act,
                                r["err"])
            B().gdn_accept_greedy(bd, drafts[c], targets[c], r["keep"], act, r["nxt"])

    eager = fresh()
    loop(eager)
    torch.cuda.synchronize()
    assert int(host(eager["err"])[0]) == 0
    g = fresh()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        loop(g)
    torch.cuda.synchronize()
    for rep in range(3):
        g["cs"].copy_(cs0)
        g["st"].copy_(st0)
        g["keep"].zero_()
        g["o"].zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in ("cs", "st", "keep", "nxt", "o"):
            assert np.array_equal(host(g[k]), host(eager[k])), (rep, k)
        assert int(host(g["err"])[0]) == 0
