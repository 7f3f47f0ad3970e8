"""GPU parity of the chunked prefill (WY/UT form on MFMA) and the standalone
conv step against the token-sequential CPU oracle, through the C ABI.

"perf(qwen): full-context MTP draft prefill and replay-free rewind"
(Measurements): 1,024-token layer-major prefill calls; "MTP inference:
review and commit structure" (Verification and limits): the chunk recurrence
differs from the sequential one only in rounding.  Tolerance: normwise per
(layer, row, head) block <= 2e-3 (bf16 inputs, fp32 state and outputs).
"""
import numpy as np
import pytest

import oracle
from gated_deltanet_recurrence_conv_amd import workloads as W
from gpu_util import act_dtype, dev, dims_pair, host, out_err, state_err, torch_mod

pytestmark = pytest.mark.gpu


def B():
    from gated_deltanet_recurrence_conv_amd import binding
    return binding


def gpu_prefill(sh, inp, T=None, state=None, out="f32", calls=None):
    """Run the prefill over inp's tokens, split into `calls` (list of lengths)."""
    torch = torch_mod()
    T = sh.T if T is None else T
    calls = [T] if calls is None else calls
    A = act_dtype(sh.act)
    st = dev(inp["state"] if state is None else state, torch.float32)
    cur = dev(inp["cur"], torch.int32)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    outs = []
    t0 = 0
    for n in calls:
        d, _ = dims_pair(sh, T=n, out=out)
        y = dev(np.ascontiguousarray(inp["y"][:, :, t0:t0 + n]), A)
        g = dev(np.ascontiguousarray(inp["g"][:, :, t0:t0 + n]), A)
        be = dev(np.ascontiguousarray(inp["beta"][:, :, t0:t0 + n]), A)
        o = torch.full((sh.L, sh.B, n, sh.HV, sh.DV), float("nan"), device="cuda",
                       dtype=act_dtype(out))
        ws = torch.empty(max(B().gdn_workspace_size(d), 1), dtype=torch.uint8, device="cuda")
        B().gdn_prefill_chunked(d, y, g, be, st, cur, o, 64, ws, err)
        outs.append(o)
        t0 += n
    torch.cuda.synchronize()
    assert int(host(err)[0]) == 0
    return host(st), np.concatenate([host(o) for o in outs], axis=2)


def oracle_prefill(sh, inp, T=None, state=None):
    T = sh.T if T is None else T
    _, od = dims_pair(sh, T=T)
    st0 = inp["state"] if state is None else state
    return oracle.prefill(od, inp["y"][:, :, :T], inp["g"][:, :, :T], inp["beta"][:, :, :T], st0,
                          inp["cur"])


@pytest.mark.parametrize("T,DK,DV,HV,HK", [(150, 64, 64, 4, 2), (1, 128, 128, 2, 1),
                                           (13, 32, 16, 2, 2), (64, 128, 32, 2, 1),
                                           (65, 64, 128, 4, 1), (1000, 128, 128, 2, 1),
                                           (640, 32, 16, 8, 4)])
def test_prefill_shapes_ragged(T, DK, DV, HV, HK):
    sh = W.Shape("pf", L=1, B=2, T=T, HV=HV, HK=HK, DK=DK, DV=DV, S=2)
    inp = W.prefill_inputs(sh, seed=3000 + T + DK + DV)
    inp["state"] = W.random_state(sh, seed=3001)
    inp["cur"] = np.array([[1, 0]], np.int32)
    st_g, o_g = gpu_prefill(sh, inp)
    st_r, o_r, err = oracle_prefill(sh, inp)
    assert err == 0
    assert out_err(o_g, o_r) <= 2e-3
    assert state_err(st_g, st_r) <= 2e-3
    # the slot that is not cur is untouched
    assert np.array_equal(st_g[0, 0, 0], inp["state"][0, 0, 0])
    assert np.array_equal(st_g[0, 1, 1], inp["state"][0, 1, 1])


def test_prefill_qwen_4096_tokens_in_1024_calls():
    """B=1, 4,096-token prompt in 1,024-token calls, chunk 64, 32 value heads,
    16 qk heads, d = 128, bf16 inputs, fp32 state from zero; every output and
    the state after each call against the token-sequential oracle."""
    sh = W.PREFILL
    inp = W.prefill_inputs(sh, seed=3100, tokens=W.PREFILL_TOKENS)
    _, od = dims_pair(sh, T=W.PREFILL_TOKENS)
    st_r, o_r, err = oracle.prefill(od, inp["y"], inp["g"], inp["beta"], inp["state"], inp["cur"])
    assert err == 0
    st_g, o_g = gpu_prefill(sh, inp, T=W.PREFILL_TOKENS, calls=[1024] * 4)
    e_o, e_s = out_err(o_g, o_r), state_err(st_g, st_r)
    print("prefill 4096: out err %.3e state err %.3e" % (e_o, e_s))
    assert e_o <= 2e-3 and e_s <= 2e-3
    # state after the first call too
    _, od1 = dims_pair(sh, T=1024)
    st1, _, _ = oracle.prefill(od1, inp["y"][:, :, :1024], inp["g"][:, :, :1024],
                               inp["beta"][:, :, :1024], inp["state"], inp["cur"])
    st_g1, _ = gpu_prefill(sh, inp, T=1024, calls=[1024])
    assert state_err(st_g1, st1) <= 2e-3


def test_prefill_carried_state_and_split_calls_bit_exact():
    """A random N(0, 0.1^2) starting state; calls of 64-multiples give the
    same bits as one call; a ragged split still matches the oracle."""
    sh = W.PREFILL.with_(HV=4, HK=2)
    inp = W.prefill_inputs(sh, seed=3200, tokens=640)
    inp["state"] = W.random_state(sh, seed=3201)
    st1, o1 = gpu_prefill(sh, inp, T=640, calls=[640])
    st2, o2 = gpu_prefill(sh, inp, T=640, calls=[256, 64, 320])
    assert np.array_equal(st1, st2)
    assert np.array_equal(o1, o2)
    st3, o3 = gpu_prefill(sh, inp, T=640, calls=[100, 413, 127])
    st_r, o_r, _ = oracle_prefill(sh, inp, T=640)
    assert out_err(o3, o_r) <= 2e-3 and state_err(st3, st_r) <= 2e-3
    assert out_err(o1, o_r) <= 2e-3 and state_err(st1, st_r) <= 2e-3


def test_prefill_4096_tokens_in_one_call():
    """The whole 4,096-token prompt in one call (64 chunks: the longest record
    chain a call builds here) from a random N(0, 0.1^2) state, 4 value heads
    on 2 qk heads at d = 128, against the token-sequential oracle; equal bit
    for bit to the same prompt in four 1,024-token calls."""
    sh = W.PREFILL.with_(HV=4, HK=2)
    inp = W.prefill_inputs(sh, seed=3150, tokens=W.PREFILL_TOKENS)
    inp["state"] = W.random_state(sh, seed=3151)
    st1, o1 = gpu_prefill(sh, inp, T=W.PREFILL_TOKENS, calls=[W.PREFILL_TOKENS])
    st4, o4 = gpu_prefill(sh, inp, T=W.PREFILL_TOKENS, calls=[1024] * 4)
    assert np.array_equal(st1, st4) and np.array_equal(o1, o4)
    st_r, o_r, err = oracle_prefill(sh, inp, T=W.PREFILL_TOKENS)
    assert err == 0
    e_o, e_s = out_err(o1, o_r), state_err(st1, st_r)
    print("prefill 4096 in one call: out err %.3e state err %.3e" % (e_o, e_s))
    assert e_o <= 2e-3 and e_s <= 2e-3


def test_prefill_bf16_output_and_scale():
    sh = W.Shape("pfo", L=2, B=1, T=200, HV=2, HK=1, DK=128, DV=64, S=1, out="bf16")
    inp = W.prefill_inputs(sh, seed=3300)
    inp["state"] = W.random_state(sh, seed=3301)
    torch = torch_mod()
    d, od = dims_pair(sh, out="bf16", scale=128 ** -0.5)
    y, g, be = (dev(inp[k], torch.bfloat16) for k in ("y", "g", "beta"))
    st = dev(inp["state"], torch.float32)
    o = torch.empty((sh.L, sh.B, sh.T, sh.HV, sh.DV), device="cuda", dtype=torch.bfloat16)
    ws = torch.empty(B().gdn_workspace_size(d), dtype=torch.uint8, device="cuda")
    B().gdn_prefill_chunked(d, y, g, be, st, None, o, 64, ws)
    torch.cuda.synchronize()
    st_r, o_r, _ = oracle.prefill(od, inp["y"], inp["g"], inp["beta"], inp["state"])
    assert state_err(host(st), st_r) <= 2e-3
    o_g = host(o).astype(np.float64)
    # bf16 output: the oracle's value rounded to bf16, within one more bf16 unit
    assert out_err(o_g, W.bf16_round(o_r.astype(np.float32))) <= 2 ** -7


def test_verify_window_matches_prefill():
    """Verify over a T-token window and the chunked prefill over the same
    tokens reach the same state and outputs (two different algorithms).  The
    conv is the identity on the current token with SiLU off, so both see the
    same bf16 q, k, v."""
    torch = torch_mod()
    sh = W.REWIND.with_(B=2, S=5, T=4)
    inp = W.verify_inputs(sh, seed=3400)
    wid = np.zeros_like(inp["conv_w"])
    wid[..., 3] = 1.0
    d, od = dims_pair(sh, flags=2)
    A = act_dtype(sh.act)
    x, w, cs = dev(inp["x"], A), dev(wid, A), dev(inp["conv_state"], A)
    g, be = dev(inp["g"], A), dev(inp["beta"], A)
    st = dev(inp["state"], torch.float32)
    cur = dev(inp["cur"], torch.int32)
    o = torch.empty((1, 2, 4, sh.HV, sh.DV), device="cuda")
    B().gdn_verify(d, x, w, None, cs, g, be, st, cur, o, None)
    st2 = dev(inp["state"], torch.float32)
    o2 = torch.empty((1, 2, 4, sh.HV, sh.DV), device="cuda")
    ws = torch.empty(B().gdn_workspace_size(d), dtype=torch.uint8, device="cuda")
    B().gdn_prefill_chunked(d, x, g, be, st2, cur, o2, 64, ws)
    torch.cuda.synchronize()
    sv = host(st)[:, :, 4]            # verify candidate after 4 tokens (cur = 0, S = 5)
    sp = host(st2)[:, :, 0]
    assert state_err(sp, sv) <= 2e-3
    assert out_err(host(o2), host(o)) <= 2e-3
    st_r, o_r, _ = oracle.verify(od, inp["x"], wid, None, inp["conv_state"], inp["g"],
                                 inp["beta"], inp["state"], inp["cur"])
    assert state_err(sp, st_r[:, :, 4]) <= 2e-3 and out_err(host(o2), o_r) <= 2e-3


@pytest.mark.parametrize("T", [1, 3, 7, 37, 1024])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_conv_step_parity(T, out):
    """The short causal conv over T tokens at the Qwen channel count
    (2*16*128 + 32*128 = 8192), rows 1 and 6 inactive, cache committed.
    T = 7 and 37 leave ragged token tiles for both tile heights; the cache
    commit takes its new rows from registers (T = 1, 3) or from x (T >= 5)."""
    torch = torch_mod()
    sh = W.COHORT.with_(T=T, B=8 if T < 1024 else 2, inactive=(1, 6) if T < 1024 else (1,))
    inp = W.verify_inputs(sh, seed=3500 + T)
    d, od = dims_pair(sh, out=out)
    A = act_dtype(sh.act)
    x, w, cs = dev(inp["x"], A), dev(inp["conv_w"], A), dev(inp["conv_state"], A)
    act = dev(inp["active"], torch.uint8)
    y = torch.full(inp["x"].shape, float("nan"), device="cuda", dtype=act_dtype(out))
    B().gdn_conv_step(d, x, w, None, cs, y, act, True)
    torch.cuda.synchronize()
    y_r, cs_r = oracle.conv_step(od, inp["x"], inp["conv_w"], None, inp["conv_state"],
                                 y_init=np.full(inp["x"].shape, np.nan), active=inp["active"])
    assert np.array_equal(host(cs).astype(np.float64), cs_r)
    yg = host(y).astype(np.float64)
    a = inp["active"].astype(bool)
    assert np.all(np.isnan(yg[:, ~a]))
    if out == "f32":
        assert np.max(np.abs(yg[:, a] - y_r[:, a])) <= 1e-5 * np.max(np.abs(y_r[:, a]))
    else:
        ref = W.bf16_round(y_r[:, a].astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(yg[:, a] - ref) <= np.abs(ref) * 2 ** -7 + 1e-30)


def test_prefill_rejects_other_chunks_and_small_workspace():
    """chunk != 64 is refused (GDN_E_SHAPE) and a workspace smaller than
    gdn_workspace_size is refused before any launch; the fp32 form (d_k = 16
    here) needs no workspace at all."""
    torch = torch_mod()
    sh = W.Shape("pfx", L=1, B=1, T=64, HV=2, HK=1, DK=32, DV=16, S=1)
    d, _ = dims_pair(sh)
    need = B().gdn_workspace_size(d)
    assert need > 0
    z = torch.zeros((1, 1, 64, sh.C), dtype=torch.bfloat16, device="cuda")
    st = torch.zeros((1, 1, 1, 2, 32, 16), device="cuda")
    o = torch.full((1, 1, 64, 2, 16), float("nan"), device="cuda")
    gg = torch.zeros((1, 1, 64, 2), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B().GdnError) as ei:
        B().gdn_prefill_chunked(d, z, gg, gg, st, None, o, 32,
                                torch.zeros(need, dtype=torch.uint8, device="cuda"))
    assert ei.value.status == 2
    with pytest.raises(ValueError):
        B().gdn_prefill_chunked(d, z, gg, gg, st, None, o, 64,
                                torch.zeros(need - 16, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert torch.isnan(o).all()
    d16, _ = dims_pair(sh.with_(DK=16))
    assert B().gdn_workspace_size(d16) == 0


def test_prefill_ragged_rows_equal_single_row_calls():
    """Eight prompts of unequal length (0 .. 1,000 tokens) in one launch into
    their own rows ("Add request-owned eight-way MTP serving for Qwen 35B",
    What was broken items 1 and 5): each row equals a single-row call of its
    own length bit for bit and the token-sequential oracle within 2e-3; a
    row of length 0 and the padding past every prompt are untouched."""
    torch = torch_mod()
    lengths = np.array([0, 1, 63, 64, 65, 200, 1000, 13], np.int32)
    T = int(lengths.max())
    sh = W.Shape("pfr", L=1, B=8, T=T, HV=4, HK=2, DK=128, DV=64, S=2)
    inp = W.prefill_inputs(sh, seed=3600)
    inp["state"] = W.random_state(sh, seed=3601)
    inp["cur"] = np.array([[0, 1, 1, 0, 1, 0, 0, 1]], np.int32)
    A = act_dtype(sh.act)
    d, _ = dims_pair(sh)
    st = dev(inp["state"], torch.float32)
    o = torch.full((1, sh.B, T, sh.HV, sh.DV), float("nan"), device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(B().gdn_workspace_size(d), dtype=torch.uint8, device="cuda")
    B().gdn_prefill_ragged(d, dev(inp["y"], A), dev(inp["g"], A), dev(inp["beta"], A), st,
                           dev(inp["cur"], torch.int32), o, dev(lengths), 64, ws, err)
    torch.cuda.synchronize()
    assert int(host(err)[0]) == 0
    st_g, o_g = host(st), host(o)
    for b, n in enumerate(lengths):
        c0 = int(inp["cur"][0, b])
        others = [s for s in range(sh.S) if s != c0]
        assert np.array_equal(st_g[:, b, others], inp["state"][:, b, others])
        assert np.all(np.isnan(o_g[:, b, n:]))
        if n == 0:
            assert np.array_equal(st_g[:, b], inp["state"][:, b])
            continue
        one = sh.with_(B=1, T=int(n))
        row = {k: np.ascontiguousarray(inp[k][:, b:b + 1, :n]) for k in ("y", "g", "beta")}
        row["state"] = np.ascontiguousarray(inp["state"][:, b:b + 1])
        row["cur"] = np.ascontiguousarray(inp["cur"][:, b:b + 1])
        st1, o1 = gpu_prefill(one, row)
        assert np.array_equal(st_g[:, b:b + 1], st1)
        assert np.array_equal(o_g[:, b:b + 1, :n], o1)
        st_r, o_r, e = oracle_prefill(one, row)
        assert e == 0
        assert state_err(st_g[:, b:b + 1, c0], st_r[:, :, c0]) <= 2e-3
        assert out_err(o_g[:, b:b + 1, :n], o_r) <= 2e-3


def test_prefill_ragged_bad_length_reported():
    torch = torch_mod()
    sh = W.Shape("pfe", L=1, B=3, T=100, HV=2, HK=1, DK=64, DV=32, S=1)
    inp = W.prefill_inputs(sh, seed=3700)
    inp["state"] = W.random_state(sh, seed=3701)
    A = act_dtype(sh.act)
    d, _ = dims_pair(sh)
    st = dev(inp["state"], torch.float32)
    o = torch.full((1, sh.B, sh.T, sh.HV, sh.DV), float("nan"), device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(B().gdn_workspace_size(d), dtype=torch.uint8, device="cuda")
    lengths = np.array([50, sh.T + 1, -1], np.int32)
    B().gdn_prefill_ragged(d, dev(inp["y"], A), dev(inp["g"], A), dev(inp["beta"], A), st, None,
                           o, dev(lengths), 64, ws, err)
    torch.cuda.synchronize()
    assert int(host(err)[0]) == 8
    st_g, o_g = host(st), host(o)
    for b in (1, 2):
        assert np.array_equal(st_g[:, b], inp["state"][:, b])
        assert np.all(np.isnan(o_g[:, b]))
    assert not np.array_equal(st_g[:, 0], inp["state"][:, 0])
    assert np.all(np.isfinite(o_g[:, 0, :50])) and np.all(np.isnan(o_g[:, 0, 50:]))


def scan_slices_per_workgroup(rows, HV, HK, DV):
    """The scan form the library launches: with the one-slice grid (rows x qk
    heads padded to a multiple of 8, x value heads per qk head x DV/16
    slices) taking r1 rounds of one workgroup per compute unit and the
    two-slice grid r2, two 16-column slices per workgroup when DV >= 32 and
    5 r2 < 3 r1, else one."""
    torch = torch_mod()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    groups = rows * HK
    blocks1 = (groups + 7) // 8 * 8 * (HV // HK) * (DV // 16)
    r1 = -(-blocks1 // cus)
    r2 = -(-(blocks1 // 2) // cus)
    return 2 if DV >= 32 and 5 * r2 < 3 * r1 else 1


@pytest.mark.parametrize("DK,DV,lengths,out", [
    (128, 128, (200, 64, 1, 131), "f32"), (128, 128, (200, 64, 1, 131), "bf16"),
    (64, 64, (70, 128, 5, 64), "f32"), (32, 32, (90, 1, 64, 65, 3, 128, 40, 7), "f32"),
    (128, 64, (150, 64, 3, 77, 12, 200, 1, 64), "f32"),
    (64, 128, (100, 65, 2, 128), "f32"), (128, 32, (33, 1, 90, 64, 70, 5, 128, 10), "f32")])
def test_prefill_two_slice_workgroups_equal_single_row_calls(DK, DV, lengths, out):
    """Ragged prompts at 32 value / 16 qk heads: 512 to 1,024 one-slice scan
    workgroups, more than the GPU holds at once, so the scan runs two column
    slices per workgroup (asserted from the device's compute-unit count).
    Each row equals a single-row call (256 or fewer workgroups: one slice per
    workgroup) bit for bit, and the token-sequential oracle within 2e-3."""
    torch = torch_mod()
    lengths = np.array(lengths, np.int32)
    T = int(lengths.max())
    nb = len(lengths)
    assert scan_slices_per_workgroup(nb, 32, 16, DV) == 2
    assert scan_slices_per_workgroup(1, 32, 16, DV) == 1
    sh = W.Shape("pf2", L=1, B=nb, T=T, HV=32, HK=16, DK=DK, DV=DV, S=2)
    inp = W.prefill_inputs(sh, seed=3700)
    inp["state"] = W.random_state(sh, seed=3701)
    inp["cur"] = (np.arange(nb, dtype=np.int32) % 2)[None, :]
    A = act_dtype(sh.act)
    d, _ = dims_pair(sh, out=out)
    st = dev(inp["state"], torch.float32)
    o = torch.full((1, sh.B, T, sh.HV, sh.DV), float("nan"), device="cuda", dtype=act_dtype(out))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(B().gdn_workspace_size(d), dtype=torch.uint8, device="cuda")
    B().gdn_prefill_ragged(d, dev(inp["y"], A), dev(inp["g"], A), dev(inp["beta"], A), st,
                           dev(inp["cur"], torch.int32), o, dev(lengths), 64, ws, err)
    torch.cuda.synchronize()
    assert int(host(err)[0]) == 0
    st_g, o_g = host(st), host(o)
    for b, n in enumerate(lengths):
        assert np.all(np.isnan(o_g[:, b, n:]))
        one = sh.with_(B=1, T=int(n))
        row = {k: np.ascontiguousarray(inp[k][:, b:b + 1, :n]) for k in ("y", "g", "beta")}
        row["state"] = np.ascontiguousarray(inp["state"][:, b:b + 1])
        row["cur"] = np.ascontiguousarray(inp["cur"][:, b:b + 1])
        st1, o1 = gpu_prefill(one, row, out=out)
        assert np.array_equal(st_g[:, b:b + 1], st1), b
        assert np.array_equal(o_g[:, b:b + 1, :n], o1), b
        st_r, o_r, e = oracle_prefill(one, row)
        assert e == 0
        c0 = int(inp["cur"][0, b])
        assert state_err(st_g[:, b, c0], st_r[:, 0, c0]) <= 2e-3, b
        if out == "f32":
            assert out_err(o_g[:, b:b + 1, :n], o_r) <= 2e-3, b
        else:   # the oracle's value rounded to bf16, within one more bf16 unit
            assert out_err(o_g[:, b:b + 1, :n].astype(np.float64),
                           W.bf16_round(o_r.astype(np.float32))) <= 2 ** -7, b


@pytest.mark.parametrize("rows", [1, 4])
def test_prefill_graph_replay_matches_eager(rows):
    """Two chained 128-token prefill calls (state carried) captured in one HIP
    graph, at B = 1 (one column slice per scan workgroup) and B = 4 (two):
    every replay, with eager work in between, equals the eager calls bit for
    bit."""
    torch = torch_mod()
    sh = W.Shape("pfg", L=1, B=rows, T=256, HV=32, HK=16, DK=128, DV=128, S=1)
    inp = W.prefill_inputs(sh, seed=3800 + rows)
    st0 = W.random_state(sh, seed=3801 + rows)
    A = act_dtype(sh.act)
    d, _ = dims_pair(sh, T=128)
    halves = [{k: dev(np.ascontiguousarray(inp[k][:, :, h * 128:(h + 1) * 128]), A)
               for k in ("y", "g", "beta")} for h in range(2)]
    ws = torch.empty(B().gdn_workspace_size(d), dtype=torch.uint8, device="cuda")

    def run(st, outs):
        for h in range(2):
            B().gdn_prefill_chunked(d, halves[h]["y"], halves[h]["g"], halves[h]["beta"], st, None,
                                    outs[h], 64, ws)

    def fresh():
        return dev(st0, torch.float32), [torch.empty((1, sh.B, 128, sh.HV, sh.DV), device="cuda")
                                         for _ in range(2)]

    st_e, o_e = fresh()
    run(st_e, o_e)
    torch.cuda.synchronize()
    st_g, o_g = fresh()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        run(st_g, o_g)
    torch.cuda.synchronize()
    junk = torch.randn(512, 512, device="cuda")
    for it in range(3):
        st_g.copy_(dev(st0, torch.float32))
        for o in o_g:
            o.fill_(float("nan"))
        graph.replay()
        junk = junk @ junk.T / 512.0          # unrelated eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(st_g, st_e), it
        for h in range(2):
            assert torch.equal(o_g[h], o_e[h]), (it, h)
