"""GPU tests of gdn_prefill_conv_chunked, the prompt prefill that computes the
short conv itself, through the C ABI.

"MTP inference: review and commit structure" (eole docs), Functional commits
items 2 and 4: the short conv with its cache mutated in place; "perf(qwen):
full-context MTP draft prefill and replay-free rewind", Measurements:
prompts prefilled in 1,024-token calls.  The call is defined as gdn_conv_step
(y in the act dtype, cache committed) followed by gdn_prefill_chunked, so it
is checked

  * bit for bit against those two GPU calls: outputs, state and conv cache,
    over split calls that carry both, windows shorter than the conv (T < 3),
    tails of every chunk length, with and without bias and SiLU;
  * against the oracle's conv_step followed by its token-sequential prefill
    (2e-3 normwise, bf16 inputs and fp32 state);
  * for a row with a bad slot: the error bit, and the row left untouched,
    conv cache included.
"""
import numpy as np
import pytest

import oracle
from gated_deltanet_recurrence_conv_amd import workloads as W
from gpu_util import FLAGS, act_dtype, dev, dims_pair, host, out_err, state_err, torch_mod

pytestmark = pytest.mark.gpu


def B():
    from gated_deltanet_recurrence_conv_amd import binding
    return binding


class Dev:
    """Device copies of one prefill's inputs (the conv cache and state are
    carried across the calls of a prompt)."""

    def __init__(self, sh, inp, bias):
        torch = torch_mod()
        A = act_dtype(sh.act)
        self.x, self.g, self.beta = (dev(inp[k], A) for k in ("x", "g", "beta"))
        self.w = dev(inp["conv_w"], A)
        self.b = dev(bias, A) if bias is not None else None
        self.cs = dev(inp["conv_state"], A)
        self.state = dev(inp["state"], torch.float32)
        self.cur = dev(inp["cur"], torch.int32)
        self.err = torch.zeros(1, dtype=torch.int32, device="cuda")


def piece(t, t0, n):
    return t[:, :, t0:t0 + n].contiguous()


def run_two_calls(sh, r, calls, out, flags):
    """gdn_conv_step (y in the act dtype, cache committed) + gdn_prefill_chunked per call."""
    torch = torch_mod()
    outs, t0 = [], 0
    for n in calls:
        dc, _ = dims_pair(sh, T=n, out=sh.act, flags=flags)
        dp, _ = dims_pair(sh, T=n, out=out, flags=flags)
        y = torch.empty((sh.L, sh.B, n, sh.C), dtype=act_dtype(sh.act), device="cuda")
        B().gdn_conv_step(dc, piece(r.x, t0, n), r.w, r.b, r.cs, y, None, True, r.err)
        o = torch.full((sh.L, sh.B, n, sh.HV, sh.DV), float("nan"), device="cuda", dtype=act_dtype(out))
        ws = torch.empty(max(B().gdn_workspace_size(dp), 1), dtype=torch.uint8, device="cuda")
        B().gdn_prefill_chunked(dp, y, piece(r.g, t0, n), piece(r.beta, t0, n), r.state, r.cur, o, 64,
                                ws, r.err)
        outs.append(o)
        t0 += n
    torch.cuda.synchronize()
    return [host(o) for o in outs]


def run_fused(sh, r, calls, out, flags):
    torch = torch_mod()
    outs, t0 = [], 0
    for n in calls:
        dp, _ = dims_pair(sh, T=n, out=out, flags=flags)
        o = torch.full((sh.L, sh.B, n, sh.HV, sh.DV), float("nan"), device="cuda", dtype=act_dtype(out))
        ws = torch.empty(max(B().gdn_workspace_size(dp), 1), dtype=torch.uint8, device="cuda")
        B().gdn_prefill_conv_chunked(dp, piece(r.x, t0, n), r.w, r.b, r.cs, piece(r.g, t0, n),
                                     piece(r.beta, t0, n), r.state, r.cur, o, 64, ws, r.err)
        outs.append(o)
        t0 += n
    torch.cuda.synchronize()
    return [host(o) for o in outs]


def compare(sh, calls, seed, out="f32", bias=False, flags=FLAGS, oracle_check=True):
    inp = W.verify_inputs(sh.with_(T=sum(calls)), seed=seed)
    rng = np.random.default_rng(seed)
    inp["cur"] = rng.integers(0, sh.S, size=(sh.L, sh.B)).astype(np.int32)
    b = W._act(0.3 * rng.standard_normal((sh.L, sh.C), dtype=np.float32), sh.act) if bias else None
    ra, rb = Dev(sh, inp, b), Dev(sh, inp, b)
    oa = run_fused(sh, ra, calls, out, flags)
    ob = run_two_calls(sh, rb, calls, out, flags)
    assert int(host(ra.err)[0]) == 0 and int(host(rb.err)[0]) == 0
    for x, y in zip(oa, ob):
        assert np.array_equal(x, y, equal_nan=True)
    assert np.array_equal(host(ra.state), host(rb.state))
    assert np.array_equal(host(ra.cs), host(rb.cs))
    if not oracle_check:
        return
    # the oracle: conv step over the whole prompt, then the token-sequential prefill
    T = sum(calls)
    _, od = dims_pair(sh, T=T, flags=flags)
    y, cs = oracle.conv_step(od, inp["x"], inp["conv_w"], b, inp["conv_state"])
    y = W._act(y.astype(np.float32), sh.act)   # the conv output is stored in the act dtype
    st, o_ref, err = oracle.prefill(od, y, inp["g"], inp["beta"], inp["state"], inp["cur"])
    assert err == 0
    assert np.array_equal(host(ra.cs).astype(np.float64), cs)
    o_gpu = np.concatenate(oa, axis=2)
    assert out_err(o_gpu, o_ref) <= 2e-3
    st_gpu = host(ra.state)
    for l in range(sh.L):
        for bb in range(sh.B):
            c0 = inp["cur"][l, bb]
            assert state_err(st_gpu[l, bb, c0], st[l, bb, c0]) <= 2e-3


def test_qwen_prompt_two_calls_bf16_out():
    """B1, 2,048 tokens in two 1,024-token calls, 32 value / 16 qk heads,
    d = 128, bf16 o: the bench's prefill shape."""
    sh = W.PREFILL.with_(L=1, B=1, S=1)
    compare(sh, [1024, 1024], seed=7100, out="bf16", oracle_check=False)


def test_qwen_prompt_against_oracle():
    sh = W.PREFILL.with_(L=1, B=1, S=1)
    compare(sh, [300], seed=7101)


@pytest.mark.parametrize("DK,DV,HV,HK,calls,bias,flags", [
    (32, 128, 4, 2, [37, 64], True, FLAGS),
    (64, 32, 4, 4, [130], False, FLAGS),
    (128, 16, 2, 1, [65, 1], True, FLAGS),
    (128, 64, 8, 2, [2, 70], False, FLAGS),
    (64, 64, 4, 2, [1, 2, 100], True, FLAGS & ~1),   # SiLU off, windows shorter than the conv
])
def test_head_shapes_split_calls(DK, DV, HV, HK, calls, bias, flags):
    sh = W.Shape("pc", L=2, B=2, T=sum(calls), HV=HV, HK=HK, DK=DK, DV=DV, S=3, act="bf16")
    compare(sh, calls, seed=7200 + DK + DV + HV + len(calls), bias=bias, flags=flags)


def test_bad_slot_row_left_untouched():
    torch = torch_mod()
    sh = W.Shape("pc_err", L=1, B=3, T=80, HV=4, HK=2, DK=64, DV=64, S=2, act="bf16")
    inp = W.verify_inputs(sh, seed=7300)
    inp["cur"] = np.array([[0, 5, 1]], np.int32)   # row 1: slot out of range
    r = Dev(sh, inp, None)
    cs0, st0 = host(r.cs).copy(), host(r.state).copy()
    dp, _ = dims_pair(sh)
    o = torch.full((sh.L, sh.B, sh.T, sh.HV, sh.DV), float("nan"), device="cuda")
    ws = torch.empty(B().gdn_workspace_size(dp), dtype=torch.uint8, device="cuda")
    B().gdn_prefill_conv_chunked(dp, r.x, r.w, None, r.cs, r.g, r.beta, r.state, r.cur, o, 64, ws,
                                 r.err)
    torch.cuda.synchronize()
    assert int(host(r.err)[0]) & 2
    assert np.array_equal(host(r.cs)[:, 1], cs0[:, 1])
    assert np.array_equal(host(r.state)[:, 1], st0[:, 1])
    assert np.all(np.isnan(host(o)[:, 1]))
    # the other rows equal the two-call result
    inp_ok = dict(inp)
    rb = Dev(sh, inp_ok, None)
    ob = run_two_calls(sh, rb, [sh.T], "f32", FLAGS)[0]
    for b in (0, 2):
        assert np.array_equal(host(o)[:, b], ob[:, b])
        assert np.array_equal(host(r.cs)[:, b], host(rb.cs)[:, b])
        assert np.array_equal(host(r.state)[:, b], host(rb.state)[:, b])


def test_unsupported_shapes_are_refused():
    torch = torch_mod()
    for act, DK in (("f32", 64), ("bf16", 16)):
        sh = W.Shape("pc_uns", L=1, B=1, T=8, HV=2, HK=1, DK=DK, DV=32, S=1, act=act)
        inp = W.verify_inputs(sh, seed=7400)
        r = Dev(sh, inp, None)
        dp, _ = dims_pair(sh)
        o = torch.zeros((1, 1, 8, 2, 32), device="cuda")
        with pytest.raises(B().GdnError):
            B().gdn_prefill_conv_chunked(dp, r.x, r.w, None, r.cs, r.g, r.beta, r.state, r.cur, o, 64,
                                         None, r.err)
