"""Pins that tie the CPU oracle to facts fixed by the pages and by the
mathematics, not to itself.

Each pin is a function of the oracle module (so the mutation test can run the
same pins against deliberately broken builds of the oracle) and raises
AssertionError when the oracle disagrees.

Page citations use the page title and section:
  [P1] "perf(qwen): full-context MTP draft prefill and replay-free rewind"
  [P2] "MTP inference: review and commit structure"
  [P3] "Add request-owned eight-way MTP serving for Qwen 35B"
"""
from __future__ import annotations

import numpy as np

import brute
from gated_deltanet_recurrence_conv_amd import workloads as W

SILU_L2 = 3


def _dims(ora, sh, **kw):
    base = dict(L=sh.L, B=sh.B, T=sh.T, HV=sh.HV, HK=sh.HK, DK=sh.DK, DV=sh.DV,
                KCONV=sh.KCONV, S=sh.S)
    base.update(kw)
    return ora.Dims(**base)


def _small(T=3, B=2, HV=4, HK=2, DK=16, DV=16, S=None, L=1, act="f32"):
    return W.Shape("pin", L=L, B=B, T=T, HV=HV, HK=HK, DK=DK, DV=DV,
                   S=(T + 1 if S is None else S), act=act)


def _close(a, b, tol, what):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    err = np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30)
    assert err <= tol, "%s: normwise error %.3e > %.1e" % (what, err, tol)


def pin_brute_force_verify(ora):
    """Brute force in explicit-matrix form agrees with the oracle on tiny
    shapes, with GQA sharing, a bias, DK != DV and a non-unit scale.
    (Method: gated delta rule; mixer rerun of [P1] Summary item 4.)"""
    for (T, HV, HK, DK, DV, scale, bias) in [(2, 2, 1, 16, 16, 1.0, False),
                                             (4, 4, 2, 16, 32, 0.25, True),
                                             (3, 6, 3, 32, 16, 1.0, True)]:
        sh = _small(T=T, HV=HV, HK=HK, DK=DK, DV=DV)
        inp = W.verify_inputs(sh, seed=11 + T)
        d = _dims(ora, sh, scale=scale)
        rng = np.random.default_rng(5)
        cb = (0.3 * rng.standard_normal((1, sh.C))).astype(np.float32) if bias else None
        cur = np.array([[1, sh.S - 1]], np.int32)
        st, o, err = ora.verify(d, inp["x"], inp["conv_w"], cb, inp["conv_state"], inp["g"],
                                inp["beta"], inp["state"], cur)
        assert err == 0
        for b in range(sh.B):
            c0 = int(cur[0, b])
            states, ob = brute.verify_row(inp["x"][0, b], inp["conv_state"][0, b],
                                          inp["conv_w"][0], None if cb is None else cb[0],
                                          inp["g"][0, b], inp["beta"][0, b],
                                          inp["state"][0, b, c0], HV, HK, DK, DV, scale)
            _close(o[0, b], ob, 1e-12, "brute o")
            for t in range(T):
                _close(st[0, b, (c0 + t + 1) % sh.S], states[t], 1e-12, "brute state t=%d" % t)
            _close(st[0, b, c0], inp["state"][0, b, c0], 0.0, "snapshot slot untouched")


def pin_retrieval_identity(ora):
    """With a=1, beta=1 and a unit key the delta rule writes v exactly at k:
    h_t^T k_t = v_t.  Pins the state orientation and the correction term."""
    sh = _small(T=5, B=1, HV=2, HK=1, DK=16, DV=16, S=1)
    inp = W.prefill_inputs(sh, seed=3)
    g = np.zeros_like(inp["g"])
    beta = np.ones_like(inp["beta"])
    st0 = W.random_state(sh, seed=4)
    y = inp["y"].astype(np.float64)
    for t in range(1, sh.T + 1):
        dt = _dims(ora, sh, T=t, l2_eps=0.0)
        st, _, _ = ora.prefill(dt, y[:, :, :t], g[:, :, :t], beta[:, :, :t], st0)
        k = y[0, 0, t - 1, sh.HK * sh.DK:2 * sh.HK * sh.DK]
        k = k / np.sqrt(k @ k)
        for h in range(sh.HV):
            v = y[0, 0, t - 1, 2 * sh.HK * sh.DK + h * sh.DV:2 * sh.HK * sh.DK + (h + 1) * sh.DV]
            _close(st[0, 0, 0, h].T @ k, v, 1e-13, "retrieval t=%d h=%d" % (t, h))


def pin_zero_decay(ora):
    """a -> 0 (g = -1000, so exp(g) == 0 exactly): the state becomes
    beta k v^T and o = scale * beta * v * (k . q), independent of the past."""
    sh = _small(T=1, B=1, HV=2, HK=1, DK=16, DV=16, S=1)
    inp = W.prefill_inputs(sh, seed=8)
    g = np.full_like(inp["g"], -1000.0)
    st0 = W.random_state(sh, seed=9)
    d = _dims(ora, sh, scale=0.5)
    st, o, _ = ora.prefill(d, inp["y"], g, inp["beta"], st0)
    y = inp["y"].astype(np.float64)[0, 0, 0]
    q = y[:sh.DK] / np.sqrt(y[:sh.DK] @ y[:sh.DK] + 1e-6)
    k = y[sh.DK:2 * sh.DK] / np.sqrt(y[sh.DK:2 * sh.DK] @ y[sh.DK:2 * sh.DK] + 1e-6)
    for h in range(sh.HV):
        v = y[2 * sh.DK + h * sh.DV:2 * sh.DK + (h + 1) * sh.DV]
        bt = float(inp["beta"][0, 0, 0, h])
        _close(st[0, 0, 0, h], bt * np.outer(k, v), 1e-14, "zero-decay state")
        _close(o[0, 0, 0, h], 0.5 * bt * v * (k @ q), 1e-14, "zero-decay output")


def pin_pure_decay(ora):
    """beta = 0: the state only decays, h_T = exp(sum g) h_0, and o_t = scale
    * exp(sum_{s<=t} g) h_0^T q_t."""
    sh = _small(T=6, B=1, HV=2, HK=1, DK=16, DV=16, S=1)
    inp = W.prefill_inputs(sh, seed=12)
    beta = np.zeros_like(inp["beta"])
    st0 = W.random_state(sh, seed=13)
    d = _dims(ora, sh)
    st, o, _ = ora.prefill(d, inp["y"], inp["g"], beta, st0)
    gs = inp["g"].astype(np.float64)[0, 0]
    y = inp["y"].astype(np.float64)[0, 0]
    for h in range(sh.HV):
        _close(st[0, 0, 0, h], np.exp(gs[:, h].sum()) * st0[0, 0, 0, h], 1e-13, "pure decay")
        for t in range(sh.T):
            q = y[t, :sh.DK] / np.sqrt(y[t, :sh.DK] @ y[t, :sh.DK] + 1e-6)
            _close(o[0, 0, t, h], np.exp(gs[:t + 1, h].sum()) * (st0[0, 0, 0, h].T @ q), 1e-13,
                   "pure-decay output")


def pin_l2_idempotent(ora):
    """Normalising already-unit q and k changes nothing beyond the eps term:
    the norm divides by sqrt(sum of squares + eps), not by the sum itself."""
    sh = _small(T=4, B=1, HV=2, HK=1, DK=16, DV=16, S=1)
    inp = W.prefill_inputs(sh, seed=21)
    y = inp["y"].astype(np.float64)
    # exact unit vectors in float64
    for m in range(2):
        blk = y[..., m * sh.DK:(m + 1) * sh.DK]
        y[..., m * sh.DK:(m + 1) * sh.DK] = blk / np.sqrt((blk ** 2).sum(-1, keepdims=True))
    st0 = W.random_state(sh, seed=22)
    on = _dims(ora, sh, flags=SILU_L2, l2_eps=0.0)
    off = _dims(ora, sh, flags=1, l2_eps=0.0)
    s1, o1, _ = ora.prefill(on, y, inp["g"], inp["beta"], st0)
    s2, o2, _ = ora.prefill(off, y, inp["g"], inp["beta"], st0)
    _close(s1, s2, 1e-14, "l2 idempotent state")
    _close(o1, o2, 1e-14, "l2 idempotent output")
    # and scaling q, k by any positive factor is undone by the norm
    y3 = y.copy()
    y3[..., :2 * sh.DK] *= 7.5
    s3, o3, _ = ora.prefill(on, y3, inp["g"], inp["beta"], st0)
    _close(s3, s1, 1e-13, "l2 scale invariance state")
    _close(o3, o1, 1e-13, "l2 scale invariance output")


def pin_conv_taps(ora):
    """Delta taps: w = e_j with SiLU off gives y_t = W[t + j], where the
    window W is [conv_state (oldest first); x].  w = e_{K-1} is the identity
    on the current token.  SiLU(1) and SiLU(-2) match their closed values.
    (Short convolution with a conv cache: [P2] Functional commits 2 and 4.)"""
    sh = _small(T=4, B=2, HV=2, HK=1, DK=16, DV=16)
    inp = W.verify_inputs(sh, seed=31)
    win = np.concatenate([inp["conv_state"], inp["x"]], axis=2).astype(np.float64)
    for j in range(4):
        w = np.zeros((1, sh.C, 4), np.float32)
        w[..., j] = 1.0
        d = _dims(ora, sh, flags=0)
        y, cs = ora.conv_step(d, inp["x"], w, None, inp["conv_state"], commit_state=False)
        _close(y, win[:, :, j:j + sh.T], 0.0, "delta tap %d" % j)
        _close(cs, inp["conv_state"], 0.0, "no commit leaves the cache")
    w = np.zeros((1, sh.C, 4), np.float32)
    w[..., 3] = 1.0
    x = np.zeros_like(inp["x"])
    x[..., 0, 0] = 1.0
    x[..., 1, 0] = -2.0
    y, _ = ora.conv_step(_dims(ora, sh, flags=1), x, w, None, inp["conv_state"],
                         commit_state=False)
    assert abs(y[0, 0, 0, 0] - 0.7310585786300049) < 1e-15, y[0, 0, 0, 0]
    assert abs(y[0, 0, 1, 0] - (-0.23840584404423515)) < 1e-15, y[0, 0, 1, 0]
    # commit_state keeps the last K-1 window rows
    _, cs = ora.conv_step(_dims(ora, sh), inp["x"], inp["conv_w"], None, inp["conv_state"],
                          commit_state=True)
    _close(cs, win[:, :, sh.T:sh.T + 3], 0.0, "conv cache after a full step")


def pin_gqa_duplication(ora):
    """Value head h reads qk head h // (HV/HK): HK < HV equals HK = HV with each
    qk head duplicated for its group of value heads."""
    sh = _small(T=3, B=1, HV=4, HK=2, DK=16, DV=16, S=1)
    inp = W.prefill_inputs(sh, seed=41)
    y = inp["y"].astype(np.float64)
    DK, HK, HV = sh.DK, sh.HK, sh.HV
    q = y[..., :HK * DK].reshape(1, 1, sh.T, HK, DK)
    k = y[..., HK * DK:2 * HK * DK].reshape(1, 1, sh.T, HK, DK)
    v = y[..., 2 * HK * DK:]
    rep = HV // HK
    qd = np.repeat(q, rep, axis=3).reshape(1, 1, sh.T, -1)
    kd = np.repeat(k, rep, axis=3).reshape(1, 1, sh.T, -1)
    yd = np.concatenate([qd, kd, v], axis=-1)
    st0 = W.random_state(sh, seed=42)
    s1, o1, _ = ora.prefill(_dims(ora, sh), y, inp["g"], inp["beta"], st0)
    s2, o2, _ = ora.prefill(_dims(ora, sh, HK=HV), yd, inp["g"], inp["beta"], st0)
    _close(s1, s2, 0.0, "gqa state")
    _close(o1, o2, 0.0, "gqa output")


def pin_keep_zero_and_commit_window(ora):
    """keep=0 leaves the snapshot and the conv cache bit-identical; keep=k
    advances the slot by k and the conv cache becomes window rows k..k+2.
    ([P3] What was broken items 2 and 4.)"""
    sh = _small(T=4, B=3, HV=2, HK=1, DK=16, DV=16, S=5)
    inp = W.verify_inputs(sh, seed=51)
    d = _dims(ora, sh)
    cur = np.array([[2, 4, 0]], np.int32)
    win = np.concatenate([inp["conv_state"], inp["x"]], axis=2).astype(np.float64)
    for keep in ([0, 0, 0], [1, 4, 2], [3, 0, 4]):
        cs, cu, err = ora.commit(d, inp["x"], inp["conv_state"], cur, np.array(keep, np.int32))
        assert err == 0
        for b, kp in enumerate(keep):
            assert cu[0, b] == (cur[0, b] + kp) % sh.S
            _close(cs[0, b], win[0, b, kp:kp + 3], 0.0, "commit window keep=%d" % kp)
        st, cs2, _, err = ora.rewind(d, inp["x"], inp["conv_w"], None, inp["conv_state"],
                                     inp["g"], inp["beta"], inp["state"], cur,
                                     np.array(keep, np.int32))
        assert err == 0
        for b, kp in enumerate(keep):
            if kp == 0:
                assert np.array_equal(st[0, b], inp["state"][0, b].astype(np.float64))
                assert np.array_equal(cs2[0, b], inp["conv_state"][0, b].astype(np.float64))
            _close(cs2[0, b], win[0, b, kp:kp + 3], 0.0, "rewind window keep=%d" % kp)


def pin_rewind_equals_prefix_forward(ora):
    """Rewind(keep=k) equals a direct forward over the accepted prefix
    ([P1] Tests), equals verify's candidate k ([P2] Verification and limits:
    partial commits replay only the accepted prefix), and equals conv_step +
    prefill over the same k tokens."""
    sh = _small(T=4, B=2, HV=4, HK=2, DK=16, DV=32, S=5)
    inp = W.verify_inputs(sh, seed=61)
    d = _dims(ora, sh)
    cur = np.array([[1, 3]], np.int32)
    stv, ov, _ = ora.verify(d, inp["x"], inp["conv_w"], None, inp["conv_state"], inp["g"],
                            inp["beta"], inp["state"], cur)
    for k in range(1, sh.T + 1):
        keep = np.array([k, k], np.int32)
        st, cs, o, err = ora.rewind(d, inp["x"], inp["conv_w"], None, inp["conv_state"],
                                    inp["g"], inp["beta"], inp["state"], cur, keep)
        assert err == 0
        for b in range(2):
            c0 = int(cur[0, b])
            _close(st[0, b, c0], stv[0, b, (c0 + k) % sh.S], 0.0, "rewind vs candidate")
            _close(o[0, b, :k], ov[0, b, :k], 0.0, "rewind outputs")
        # direct forward over the prefix: conv over k tokens, then prefill
        dk = _dims(ora, sh, T=k)
        y, cs3 = ora.conv_step(dk, inp["x"][:, :, :k], inp["conv_w"], None, inp["conv_state"])
        st0 = np.stack([inp["state"][:, b, int(cur[0, b])] for b in range(2)], 1)[:, :, None]
        sp, op, _ = ora.prefill(_dims(ora, sh, T=k, S=1), y, inp["g"][:, :, :k],
                                inp["beta"][:, :, :k], st0)
        for b in range(2):
            _close(st[0, b, int(cur[0, b])], sp[0, b, 0], 0.0, "rewind vs direct forward")
        _close(cs, cs3, 0.0, "conv cache vs direct forward")


def pin_prefix_consistency(ora):
    """Candidate t of a T-token window equals the last candidate of a
    t-token window over the same tokens (no look-ahead)."""
    sh = _small(T=4, B=1, HV=2, HK=1, DK=16, DV=16, S=5)
    inp = W.verify_inputs(sh, seed=71)
    stT, oT, _ = ora.verify(_dims(ora, sh), inp["x"], inp["conv_w"], None, inp["conv_state"],
                            inp["g"], inp["beta"], inp["state"])
    for t in range(1, sh.T):
        st, o, _ = ora.verify(_dims(ora, sh, T=t), inp["x"][:, :, :t], inp["conv_w"], None,
                              inp["conv_state"], inp["g"][:, :, :t], inp["beta"][:, :, :t],
                              inp["state"])
        _close(st[0, 0, t], stT[0, 0, t], 0.0, "prefix state")
        _close(o, oT[:, :, :t], 0.0, "prefix output")


def pin_inactive_rows_inert(ora):
    """Inactive rows write nothing in verify and commit ([P3] What was
    broken item 4; Ownership model: padding rows are inert)."""
    sh = _small(T=2, B=3, HV=2, HK=1, DK=16, DV=16, S=3)
    inp = W.verify_inputs(sh, seed=81)
    act = np.array([1, 0, 1], np.uint8)
    st_in = inp["state"].copy()
    st_in[0, :, 1:] = np.nan          # candidate slots hold a sentinel
    o_in = np.full((1, 3, 2, 2, 16), np.nan)
    st, o, err = ora.verify(_dims(ora, sh), inp["x"], inp["conv_w"], None, inp["conv_state"],
                            inp["g"], inp["beta"], st_in, active=act, o_init=o_in)
    assert err == 0
    assert np.array_equal(st[0, 1], st_in[0, 1].astype(np.float64), equal_nan=True)
    assert np.all(np.isnan(o[0, 1]))
    assert not np.any(np.isnan(o[0, 0])) and not np.any(np.isnan(o[0, 2]))
    assert not np.any(np.isnan(st[0, 0])) and not np.any(np.isnan(st[0, 2]))
    cs, cu, err = ora.commit(_dims(ora, sh), inp["x"], inp["conv_state"],
                             np.zeros((1, 3), np.int32), np.array([2, 0, 1], np.int32), act)
    assert err == 0 and cu[0, 1] == 0
    assert np.array_equal(cs[0, 1], inp["conv_state"][0, 1].astype(np.float64))


def pin_rows_separable(ora):
    """A batch of rows equals each row run alone ([P3] What was broken item 6)."""
    sh = _small(T=3, B=4, HV=2, HK=1, DK=16, DV=16, S=4)
    inp = W.verify_inputs(sh, seed=91)
    cur = np.array([[0, 1, 2, 3]], np.int32)
    stB, oB, _ = ora.verify(_dims(ora, sh), inp["x"], inp["conv_w"], None, inp["conv_state"],
                            inp["g"], inp["beta"], inp["state"], cur)
    for b in range(sh.B):
        sl = slice(b, b + 1)
        st1, o1, _ = ora.verify(_dims(ora, sh, B=1), inp["x"][:, sl], inp["conv_w"], None,
                                inp["conv_state"][:, sl], inp["g"][:, sl], inp["beta"][:, sl],
                                inp["state"][:, sl], cur[:, sl])
        _close(st1[:, 0], stB[:, b], 0.0, "row state")
        _close(o1[:, 0], oB[:, b], 0.0, "row output")


def pin_orthonormal_memory(ora):
    """a = beta = 1, h_0 = 0 and orthonormal keys: the state is the exact
    associative memory h_T = sum_s k_s v_s^T and o_t = sum_{s<=t} v_s (k_s.q_t)."""
    DK = DV = 16
    T = 6
    sh = _small(T=T, B=1, HV=1, HK=1, DK=DK, DV=DV, S=1)
    rng = np.random.default_rng(101)
    Qm, _ = np.linalg.qr(rng.standard_normal((DK, DK)))
    ks = Qm[:, :T].T
    qs = rng.standard_normal((T, DK))
    qs /= np.linalg.norm(qs, axis=1, keepdims=True)
    vs = rng.standard_normal((T, DV))
    y = np.concatenate([qs, ks, vs], axis=1)[None, None]
    g = np.zeros((1, 1, T, 1))
    beta = np.ones((1, 1, T, 1))
    st, o, _ = ora.prefill(_dims(ora, sh, l2_eps=0.0), y, g, beta,
                           np.zeros((1, 1, 1, 1, DK, DV)))
    _close(st[0, 0, 0, 0], sum(np.outer(ks[s], vs[s]) for s in range(T)), 1e-13, "memory")
    for t in range(T):
        exp_o = sum(vs[s] * (ks[s] @ qs[t]) for s in range(t + 1))
        _close(o[0, 0, t, 0], exp_o, 1e-12, "memory readout t=%d" % t)


def pin_affine_and_columns(ora):
    """For fixed q, k, g, beta the final state is affine in (h_0, V):
    h(h_0, V) = h(h_0, 0) + h(0, V); permuting value columns together with
    the state's columns permutes the outputs the same way."""
    sh = _small(T=5, B=1, HV=2, HK=1, DK=16, DV=16, S=1)
    inp = W.prefill_inputs(sh, seed=111)
    y = inp["y"].astype(np.float64)
    st0 = W.random_state(sh, seed=112).astype(np.float64)
    d = _dims(ora, sh)
    vsl = slice(2 * sh.DK, None)
    y0 = y.copy()
    y0[..., vsl] = 0.0
    sA, oA, _ = ora.prefill(d, y, inp["g"], inp["beta"], st0)
    sB, oB, _ = ora.prefill(d, y0, inp["g"], inp["beta"], st0)
    sC, oC, _ = ora.prefill(d, y, inp["g"], inp["beta"], np.zeros_like(st0))
    _close(sA, sB + sC, 1e-13, "affine state")
    _close(oA, oB + oC, 1e-13, "affine output")
    perm = np.random.default_rng(113).permutation(sh.DV)
    yp = y.copy()
    for h in range(sh.HV):
        base = 2 * sh.DK + h * sh.DV
        yp[..., base:base + sh.DV] = y[..., base + perm]
    sP, oP, _ = ora.prefill(d, yp, inp["g"], inp["beta"], st0[..., perm])
    _close(sP, sA[..., perm], 1e-14, "column permutation state")
    _close(oP, oA[..., perm], 1e-14, "column permutation output")


def pin_split_prefill(ora):
    """Prefill split into calls with the state carried equals one call."""
    sh = _small(T=12, B=1, HV=2, HK=1, DK=16, DV=16, S=1)
    inp = W.prefill_inputs(sh, seed=121)
    st0 = W.random_state(sh, seed=122)
    sA, oA, _ = ora.prefill(_dims(ora, sh), inp["y"], inp["g"], inp["beta"], st0)
    st = st0
    outs = []
    for a, b in [(0, 5), (5, 6), (6, 12)]:
        st, o, _ = ora.prefill(_dims(ora, sh, T=b - a), inp["y"][:, :, a:b], inp["g"][:, :, a:b],
                               inp["beta"][:, :, a:b], st)
        outs.append(o)
    _close(st, sA, 0.0, "split prefill state")
    _close(np.concatenate(outs, axis=2), oA, 0.0, "split prefill output")


def pin_error_bits(ora):
    """Bad keep (bit 0), bad cur (bit 1) and keep != 0 on an inactive row
    (bit 2) are reported and leave that row untouched."""
    sh = _small(T=2, B=3, HV=2, HK=1, DK=16, DV=16, S=3)
    inp = W.verify_inputs(sh, seed=131)
    d = _dims(ora, sh)
    act = np.array([1, 0, 1], np.uint8)
    cur = np.array([[0, 0, 7]], np.int32)
    cs, cu, err = ora.commit(d, inp["x"], inp["conv_state"], cur, np.array([3, 1, 1], np.int32),
                             act)
    assert err == (1 | 4 | 2), err
    assert np.array_equal(cu, cur)
    assert np.array_equal(cs, inp["conv_state"].astype(np.float64))
    st, cs, _, err = ora.rewind(d, inp["x"], inp["conv_w"], None, inp["conv_state"], inp["g"],
                                inp["beta"], inp["state"], cur, np.array([-1, 0, 1], np.int32))
    assert err == (1 | 2), err
    assert np.array_equal(st, inp["state"].astype(np.float64))


def pin_greedy_acceptance(ora):
    """Greedy acceptance of a window ("Add request-owned eight-way MTP serving
    for Qwen 35B", Follow-up; What was broken item 2): keep counts the pending
    token plus the leading drafts that equal the target's token one position
    earlier; the first mismatch ends the prefix (later matches do not count);
    an inactive row keeps 0; the next pending token is the target's token
    after the last kept position.  Every case below is written out by hand."""
    d = ora.Dims(L=1, B=7, T=4, HV=2, HK=1, DK=16, DV=16, S=5)
    target = np.array([[10, 11, 12, 13]] * 7, np.int32)
    draft = np.array([[10, 11, 12],     # all accepted
                      [99, 11, 12],     # first draft rejected
                      [10, 99, 12],     # second rejected
                      [10, 11, 99],     # third rejected
                      [99, 11, 12],     # later matches after a mismatch do not count
                      [11, 12, 13],     # drafts shifted by one: compared position by position
                      [10, 11, 12]], np.int32)
    active = np.array([1, 1, 1, 1, 1, 1, 0], np.uint8)
    keep, nxt = ora.accept_greedy(d, draft, target, active)
    assert keep.tolist() == [4, 1, 2, 3, 1, 1, 0]
    assert nxt.tolist() == [13, 10, 11, 12, 10, 10, -1]
    # T = 1: no drafts, the pending token alone
    d1 = ora.Dims(L=1, B=2, T=1, HV=2, HK=1, DK=16, DV=16, S=2)
    keep, nxt = ora.accept_greedy(d1, np.zeros((2, 0), np.int32), np.array([[5], [6]], np.int32))
    assert keep.tolist() == [1, 1] and nxt.tolist() == [5, 6]


def pin_gated_rmsnorm(ora):
    """Gated RMSNorm epilogue ("MTP inference: review and commit structure",
    Functional commits item 4) pinned by properties of its definition:
    invariance to a positive scale of o (eps = 0), oddness in o, unit mean
    square when w = 1 and the gate is saturated (SiLU(60) = 60 in double),
    a zero gate gives zero, SiLU(z) - SiLU(-z) = z, a one-hot weight keeps one
    column, the constant-vector closed form, inactive rows untouched."""
    rng = np.random.default_rng(171)
    d = ora.Dims(L=2, B=3, T=2, HV=3, HK=1, DK=16, DV=16, S=3)
    shp = (2, 3, 2, 3, 16)
    o = rng.standard_normal(shp)
    z = rng.standard_normal(shp)
    w = rng.standard_normal((2, 16))
    y = ora.gated_rmsnorm(d, o, z, w, eps=0.0)
    assert np.allclose(ora.gated_rmsnorm(d, 7.5 * o, z, w, eps=0.0), y, rtol=1e-13, atol=0)
    assert np.array_equal(ora.gated_rmsnorm(d, -o, z, w, eps=1e-6), -ora.gated_rmsnorm(d, o, z, w, eps=1e-6))
    unit = ora.gated_rmsnorm(d, o, np.full(shp, 60.0), np.ones((2, 16)), eps=0.0) / 60.0
    assert np.allclose(np.mean(unit ** 2, axis=-1), 1.0, rtol=0, atol=1e-13)
    assert np.array_equal(ora.gated_rmsnorm(d, o, np.zeros(shp), w), np.zeros(shp))
    yp, ym = ora.gated_rmsnorm(d, o, z, w, eps=0.0), ora.gated_rmsnorm(d, o, -z, w, eps=0.0)
    base = ora.gated_rmsnorm(d, o, np.full(shp, 60.0), w, eps=0.0) / 60.0   # o / rms(o) * w
    assert np.allclose(yp - ym, base * z, rtol=1e-12, atol=1e-13)
    onehot = np.zeros((2, 16))
    onehot[:, 5] = 1.0
    y1 = ora.gated_rmsnorm(d, o, z, onehot)
    assert np.count_nonzero(y1[..., np.arange(16) != 5]) == 0 and np.all(y1[..., 5] != 0)
    c = np.full(shp, 0.25)
    yc = ora.gated_rmsnorm(d, c, np.full(shp, 60.0), np.ones((2, 16)), eps=0.0625)
    assert np.allclose(yc, 0.25 / np.sqrt(0.0625 + 0.0625) * 60.0, rtol=1e-15, atol=0)
    sentinel = np.full(shp, np.nan)
    ya = ora.gated_rmsnorm(d, o, z, w, active=np.array([1, 0, 1], np.uint8), y_init=sentinel)
    assert np.all(np.isnan(ya[:, 1])) and np.all(np.isfinite(ya[:, [0, 2]]))


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
