#!/usr/bin/env python3
"""Benchmark of the Gated DeltaNet verify + commit cycle on one MI355X.

Headline: the B8/T2 verification cohort (32 value heads, 16 qk heads,
d_k = d_v = 128, bf16 inputs, fp32 state, rows 1 and 6 inactive, keep ~
U{0,1,2} drawn per cycle).  One step is one decode cycle of a 30-layer
hybrid stack: gdn_verify over the 30 GDN layers' state pools (one grouped
launch) followed by gdn_commit of every layer (one grouped launch).  The 30
pools (1.44 GiB of fp32 state) exceed the 256 MiB Infinity Cache, so state
traffic is HBM traffic.  Metric: rows*heads/s = 30 * 8 * 32 per step / time.

Also printed (in the same JSON line, under "extra"): the same cycle with one
verify launch per layer captured in a HIP graph, the solo B1/T3 30-layer
cycle, the B8/T4 rewind, the 1,024-token conv step and the chunked prefill.

  python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
L_POOL = 30


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-headline", action="store_true")
    ap.add_argument("--only", default=None,
                    help="run one secondary measurement (per_layer_graph, solo, rewind, conv_step, "
                         "prefill) and print its JSON instead of the headline line")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy three times (used to "
                         "calibrate the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def copy_probe(torch):
    n = 1 << 28                     # 2^28 fp32 = 1 GiB
    a = torch.randn(n, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4,
                      "copies": 3}), flush=True)


def counted_traffic(key):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE
    (calibrated on a plain copy) for the kernel source they were taken on;
    None when that source has changed since."""
    import hashlib
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            rec = json.load(f)[key]
        h = hashlib.sha256()
        for src in rec["sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        sha = h.hexdigest()[:16]
    except (OSError, KeyError, ValueError):
        return None
    return rec["traffic_bytes_per_launch"] if sha == rec["sha256_16"] else None


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Timer:
    """HIP events on torch's current stream, which is the stream every
    libgdn call below is launched on."""

    def __init__(self, torch):
        self.torch = torch

    def ev(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return e


def cohort_pools(torch, W, sh, L, seed):
    """L layers of the cohort: every tensor on the GPU, stacked along the layer axis."""
    big = sh.with_(L=L)
    rng = np.random.default_rng(seed)
    bf = torch.bfloat16 if sh.act == "bf16" else torch.float32
    C = sh.C

    def act(shape, scale=1.0):
        return (scale * torch.randn(shape, generator=gen, device="cuda")).to(bf)

    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    t = {}
    t["x"] = act((L, sh.B, sh.T, C))
    t["conv_w"] = act((L, C, 4), 0.5)
    t["conv_state"] = act((L, sh.B, 3, C))
    t["g"] = (-torch.nn.functional.softplus(torch.randn((L, sh.B, sh.T, sh.HV), generator=gen,
                                                        device="cuda"))).to(bf)
    t["beta"] = torch.sigmoid(torch.randn((L, sh.B, sh.T, sh.HV), generator=gen,
                                          device="cuda")).to(bf)
    t["state"] = 0.1 * torch.randn((L, sh.B, sh.S, sh.HV, sh.DK, sh.DV), generator=gen,
                                   device="cuda")
    t["cur"] = torch.zeros((L, sh.B), dtype=torch.int32, device="cuda")
    act_rows = np.ones(sh.B, np.uint8)
    for r in sh.inactive:
        act_rows[r] = 0
    t["active"] = torch.from_numpy(act_rows).cuda()
    t["o"] = torch.empty((L, sh.B, sh.T, sh.HV, sh.DV), dtype=torch.float32, device="cuda")
    t["err"] = torch.zeros(1, dtype=torch.int32, device="cuda")
    return big, t, rng, act_rows


def verify_bytes(sh, n_active_rows, L):
    """Algorithmic bytes of one grouped verify launch: per active (layer, row):
    the fp32 state read once (HV*DK*DV*4) and written T times as candidates,
    the window inputs x (T*C) and conv cache (3*C) in the act dtype, g and
    beta (2*T*HV), and the fp32 outputs (T*HV*DV*4); per layer the conv
    weights (C*4)."""
    esz = 2 if sh.act == "bf16" else 4
    tile = sh.HV * sh.DK * sh.DV * 4
    per_row = tile * (1 + sh.T) + (sh.T + 3) * sh.C * esz + 2 * sh.T * sh.HV * esz \
        + sh.T * sh.HV * sh.DV * 4
    return L * (n_active_rows * per_row + sh.C * 4 * esz)


def commit_bytes(sh, keep, active, L):
    """Per committing (layer, row): 3 conv-cache rows written and the 3
    window rows they come from read (act dtype), plus keep/active/cur."""
    esz = 2 if sh.act == "bf16" else 4
    n = int(np.sum((keep > 0) & (active > 0)))
    return L * (n * 6 * sh.C * esz + sh.B * 9)


def algorithmic_min_bytes(sh, keep, active, L):
    """The fewest bytes one verify + commit cycle can move: per active (layer,
    row) one read of its fp32 state, the window inputs x, conv cache, g and
    beta, and the fp32 outputs; per committing (layer, row) one write of its
    state and of its new conv cache; per layer the conv weights.  The
    verify + commit split writes T candidates instead of one committed state."""
    esz = 2 if sh.act == "bf16" else 4
    tile = sh.HV * sh.DK * sh.DV * 4
    n_act = int(np.sum(active > 0))
    n_com = int(np.sum((keep > 0) & (active > 0)))
    per_act = tile + (sh.T + 3) * sh.C * esz + 2 * sh.T * sh.HV * esz + sh.T * sh.HV * sh.DV * 4
    per_com = tile + 3 * sh.C * esz
    return L * (n_act * per_act + n_com * per_com + sh.C * 4 * esz)


def stream_copy_gbs(torch):
    """Device-to-device copy rate of a 1 GiB buffer (read + write bytes per
    second), the practical ceiling of a kernel that streams memory."""
    n = 1 << 28
    a = torch.empty(n, device="cuda")
    a.fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(2):
        b.copy_(a)
    tm = Timer(torch)
    e0 = tm.ev()
    reps = 5
    for _ in range(reps):
        b.copy_(a)
    e1 = tm.ev()
    torch.cuda.synchronize()
    gbs = 2 * n * 4 * reps / (e0.elapsed_time(e1) / 1e3) / 1e9
    del a, b
    torch.cuda.empty_cache()
    return gbs


def headline(torch, gb, W, args):
    """The headline cycle: one grouped verify over the 30 layer pools, then one
    grouped commit with a fresh device keep vector.  The K timed cycles are
    captured once in a HIP graph (as a decode loop issues them) and replayed,
    so the time is the GPU's, not the host's launch rate.  The verify
    kernel's average launch time for the roofline comes from a separate run
    of back-to-back verify launches (verify writes only candidate slots, so
    repeating it changes nothing)."""
    sh = W.COHORT
    big, t, rng, act_rows = cohort_pools(torch, W, sh, L_POOL, 1001)
    d = gb.make_dims(L_POOL, sh.B, sh.T, sh.HV, sh.HK, sh.DK, sh.DV, S=sh.S, act="bf16",
                     out="f32")
    n = args.steps + args.warmup
    keeps = np.stack([W.keep_uniform(rng, sh, act_rows) for _ in range(n)]).astype(np.int32)
    keep_d = torch.from_numpy(keeps).cuda()

    def step(i):
        gb.gdn_verify(d, t["x"], t["conv_w"], None, t["conv_state"], t["g"], t["beta"],
                      t["state"], t["cur"], t["o"], t["active"], t["err"])
        gb.gdn_commit(d, t["x"], t["conv_state"], t["cur"], keep_d[i], t["active"], t["err"])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        for i in range(args.warmup, n):
            step(i)
    torch.cuda.synchronize()
    tm = Timer(torch)
    start = tm.ev()
    graph.replay()
    end = tm.ev()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    assert int(t["err"].item()) == 0, "device error word set"
    # verify alone, back to back
    reps = 20
    v0 = tm.ev()
    for _ in range(reps):
        gb.gdn_verify(d, t["x"], t["conv_w"], None, t["conv_state"], t["g"], t["beta"],
                      t["state"], t["cur"], t["o"], t["active"], t["err"])
    v1 = tm.ev()
    torch.cuda.synchronize()
    verify_ms = v0.elapsed_time(v1) / reps
    assert int(t["err"].item()) == 0, "device error word set"
    n_act = int(act_rows.sum())
    vb = verify_bytes(sh, n_act, L_POOL)
    cb = float(np.mean([commit_bytes(sh, keeps[i], act_rows, L_POOL) for i in range(args.warmup, n)]))
    amin = float(np.mean([algorithmic_min_bytes(sh, keeps[i], act_rows, L_POOL)
                          for i in range(args.warmup, n)]))
    ms_step = total_ms / args.steps
    rows_heads = L_POOL * sh.B * sh.HV
    res = dict(ms_per_step=ms_step, value=rows_heads * args.steps / (total_ms / 1e3),
               verify_ms=verify_ms, verify_bytes=vb, commit_bytes=cb,
               verify_gbs=vb / (verify_ms / 1e3) / 1e9,
               cycle_gbs=(vb + cb) / (ms_step / 1e3) / 1e9,
               algorithmic_min_bytes_per_cycle=amin,
               algorithmic_min_gbs=amin / (ms_step / 1e3) / 1e9,
               active_rows_heads_per_s=L_POOL * n_act * sh.HV * args.steps / (total_ms / 1e3))
    del t, graph
    torch.cuda.empty_cache()
    return res


def lazy_cycle(torch, gb, W, args):
    """The cohort cycle with the commit folded into the next verify
    (gdn_verify_lazy): each cycle replays the previous cycle's accepted
    tokens from the snapshot, writes the committed state once in place, and
    verifies the new window without candidate writes.  Same pools, keep
    sequence and graph replay as the headline."""
    sh = W.COHORT
    big, t, rng, act_rows = cohort_pools(torch, W, sh, L_POOL, 1001)
    d = gb.make_dims(L_POOL, sh.B, sh.T, sh.HV, sh.HK, sh.DK, sh.DV, S=sh.S, act="bf16",
                     out="f32")
    n = args.steps + args.warmup
    keeps = np.stack([W.keep_uniform(rng, sh, act_rows) for _ in range(n)]).astype(np.int32)
    keep_d = torch.from_numpy(keeps).cuda()

    def cycle(i):
        # the previous window's inputs are the same pool tensors (the bench
        # does not change x between cycles); keep_prev is the previous keep
        gb.gdn_verify_lazy(d, t["x"] if i else None, t["g"] if i else None,
                           t["beta"] if i else None, keep_d[i - 1] if i else None, t["x"],
                           t["conv_w"], None, t["conv_state"], t["g"], t["beta"], t["state"],
                           t["cur"], t["o"], t["active"], t["err"])

    for i in range(args.warmup):
        cycle(i)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        for i in range(args.warmup, n):
            cycle(i)
    torch.cuda.synchronize()
    tm = Timer(torch)
    start = tm.ev()
    graph.replay()
    end = tm.ev()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    assert int(t["err"].item()) == 0, "device error word set"
    esz, tile = 2, sh.HV * sh.DK * sh.DV * 4
    byts = []
    for i in range(args.warmup, n):
        kp = keeps[i - 1]
        per = 0
        for b in range(sh.B):
            if act_rows[b] or kp[b] > 0:
                per += tile + (2 * sh.T + 3) * sh.C * esz + 4 * sh.T * sh.HV * esz
            if kp[b] > 0:
                per += tile + 6 * sh.C * esz
            if act_rows[b]:
                per += sh.T * sh.HV * sh.DV * 4
        byts.append(L_POOL * (per + sh.C * 4 * esz))
    per_cycle = float(np.mean(byts))
    del t, graph
    torch.cuda.empty_cache()
    return dict(ms_per_cycle=ms, rows_heads_per_s=L_POOL * sh.B * sh.HV / (ms / 1e3),
                bytes_per_cycle=per_cycle, gbs=per_cycle / (ms / 1e3) / 1e9,
                launches_per_cycle=2)


def per_layer_graph(torch, gb, W, args):
    """The same cycle with one verify launch per layer (as a model forward
    issues them), captured once in a HIP graph and replayed."""
    sh = W.COHORT
    big, t, rng, act_rows = cohort_pools(torch, W, sh, L_POOL, 1002)
    d1 = gb.make_dims(1, sh.B, sh.T, sh.HV, sh.HK, sh.DK, sh.DV, S=sh.S, act="bf16", out="f32")
    dL = gb.make_dims(L_POOL, sh.B, sh.T, sh.HV, sh.HK, sh.DK, sh.DV, S=sh.S, act="bf16",
                      out="f32")
    keep_cur = torch.zeros(sh.B, dtype=torch.int32, device="cuda")
    n = args.steps + args.warmup
    keeps = torch.from_numpy(np.stack([W.keep_uniform(rng, sh, act_rows) for _ in range(n)])
                             .astype(np.int32)).cuda()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())

    def cycle():
        for l in range(L_POOL):
            sl = slice(l, l + 1)
            gb.gdn_verify(d1, t["x"][sl], t["conv_w"][sl], None, t["conv_state"][sl],
                          t["g"][sl], t["beta"][sl], t["state"][sl], t["cur"][sl], t["o"][sl],
                          t["active"], t["err"])
        gb.gdn_commit(dL, t["x"], t["conv_state"], t["cur"], keep_cur, t["active"], t["err"])

    with torch.cuda.stream(s):
        cycle()                       # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        cycle()
    torch.cuda.synchronize()
    for i in range(args.warmup):
        keep_cur.copy_(keeps[i])
        graph.replay()
    torch.cuda.synchronize()
    tm = Timer(torch)
    start = tm.ev()
    for i in range(args.warmup, n):
        keep_cur.copy_(keeps[i])
        graph.replay()
    end = tm.ev()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    assert int(t["err"].item()) == 0
    res = dict(ms_per_step=ms, rows_heads_per_s=L_POOL * sh.B * sh.HV / (ms / 1e3),
               launches_per_step=L_POOL + 1)
    del graph, t
    torch.cuda.empty_cache()
    return res


def solo(torch, gb, W, args):
    """B=1, T=3 (two drafts + bonus), 30 independent layers in one grouped
    launch, keep by prefix acceptance p=0.8, state carried across cycles."""
    sh = W.SOLO
    big, t, rng, act_rows = cohort_pools(torch, W, sh.with_(L=1), sh.L, 2002)
    d = gb.make_dims(sh.L, 1, sh.T, sh.HV, sh.HK, sh.DK, sh.DV, S=sh.S, act="bf16", out="f32")
    cycles = 200
    keeps = torch.from_numpy(np.stack([W.keep_prefix_acceptance(rng, sh) for _ in range(cycles)])
                             .astype(np.int32)).cuda()

    def cyc(i):
        gb.gdn_verify(d, t["x"], t["conv_w"], None, t["conv_state"], t["g"], t["beta"],
                      t["state"], t["cur"], t["o"], None, t["err"])
        gb.gdn_commit(d, t["x"], t["conv_state"], t["cur"], keeps[i], None, t["err"])

    for i in range(10):
        cyc(i)
    torch.cuda.synchronize()
    tm = Timer(torch)
    marks = []
    start = tm.ev()
    for i in range(cycles):
        v0 = tm.ev()
        gb.gdn_verify(d, t["x"], t["conv_w"], None, t["conv_state"], t["g"], t["beta"],
                      t["state"], t["cur"], t["o"], None, t["err"])
        v1 = tm.ev()
        gb.gdn_commit(d, t["x"], t["conv_state"], t["cur"], keeps[i], None, t["err"])
        marks.append((v0, v1))
    end = tm.ev()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / cycles
    vms = float(np.mean([a.elapsed_time(b) for a, b in marks]))
    vb = verify_bytes(sh, 1, sh.L)
    assert int(t["err"].item()) == 0
    del t
    torch.cuda.empty_cache()
    return dict(ms_per_cycle=ms, rows_heads_per_s=sh.L * sh.HV / (ms / 1e3), verify_ms=vms,
                verify_gbs=vb / (vms / 1e3) / 1e9)


def rewind(torch, gb, W, args):
    """B=8, T=4 captured window, keep ~ U{0..4}, 30 layer pools in one grouped call."""
    sh = W.REWIND
    big, t, rng, act_rows = cohort_pools(torch, W, sh.with_(L=1), L_POOL, 3003)
    d = gb.make_dims(L_POOL, sh.B, sh.T, sh.HV, sh.HK, sh.DK, sh.DV, S=sh.S, act="bf16",
                     out="f32")
    reps = 20
    keeps_np = np.stack([W.keep_uniform(rng, sh) for _ in range(reps + 3)]).astype(np.int32)
    keeps = torch.from_numpy(keeps_np).cuda()
    for i in range(3):
        gb.gdn_rewind(d, t["x"], t["conv_w"], None, t["conv_state"], t["g"], t["beta"],
                      t["state"], t["cur"], keeps[i], None, t["err"])
    torch.cuda.synchronize()
    tm = Timer(torch)
    start = tm.ev()
    for i in range(3, reps + 3):
        gb.gdn_rewind(d, t["x"], t["conv_w"], None, t["conv_state"], t["g"], t["beta"],
                      t["state"], t["cur"], keeps[i], None, t["err"])
    end = tm.ev()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / reps
    tile = sh.HV * sh.DK * sh.DV * 4
    k = keeps_np[3:]
    # per committing (layer, row): state read + written, keep tokens of x/g/beta,
    # conv cache read + written (3 rows each)
    per_call = np.mean([L_POOL * sum(2 * tile + kk * (sh.C * 2 + 4 * sh.HV) + 9 * sh.C * 2
                                     for kk in row if kk > 0) for row in k])
    assert int(t["err"].item()) == 0
    del t
    torch.cuda.empty_cache()
    return dict(ms_per_call=ms, bytes_per_call=float(per_call),
                gbs=per_call / (ms / 1e3) / 1e9,
                rows_heads_per_s=L_POOL * sh.B * sh.HV / (ms / 1e3))


def conv_step(torch, gb, W, args):
    """The standalone conv over a 1,024-token prefill call, 10 buffers rotated.
    One call is ~10 us of GPU work, less than the host needs to issue it, so
    the 10 calls are captured once in a HIP graph and the graph is replayed."""
    sh = W.PREFILL
    nb = 10
    C = sh.C
    bf = torch.bfloat16
    xs = [torch.randn((1, 1, sh.T, C), device="cuda").to(bf) for _ in range(nb)]
    ys = [torch.empty((1, 1, sh.T, C), device="cuda", dtype=bf) for _ in range(nb)]
    w = (0.5 * torch.randn((1, C, 4), device="cuda")).to(bf)
    cs = torch.randn((1, 1, 3, C), device="cuda").to(bf)
    d = gb.make_dims(1, 1, sh.T, sh.HV, sh.HK, sh.DK, sh.DV, S=1, act="bf16", out="bf16")
    for i in range(nb):
        gb.gdn_conv_step(d, xs[i], w, None, cs, ys[i], None, True)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        for i in range(nb):
            gb.gdn_conv_step(d, xs[i], w, None, cs, ys[i], None, True)
    torch.cuda.synchronize()
    for _ in range(2):
        graph.replay()
    torch.cuda.synchronize()
    replays = 10
    tm = Timer(torch)
    start = tm.ev()
    for _ in range(replays):
        graph.replay()
    end = tm.ev()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / (replays * nb)
    byts = 2 * sh.T * C * 2 + C * 4 * 2 + 6 * C * 2
    return dict(tokens=sh.T, ms_per_call=ms, gbs=byts / (ms / 1e3) / 1e9)


def prefill(torch, gb, W, args):
    """Chunked prefill of 4,096-token prompts in 1,024-token calls (chunk 64),
    32 value / 16 qk heads, d = 128, bf16 inputs and outputs, fp32 state;
    10 prompt buffers (640 MiB of y) rotated so inputs come from HBM."""
    sh = W.PREFILL
    d = gb.make_dims(1, 1, sh.T, sh.HV, sh.HK, sh.DK, sh.DV, S=1, act="bf16", out="bf16")
    nb, calls = 10, W.PREFILL_TOKENS // sh.T
    C = sh.C
    bf = torch.bfloat16
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5005)
    ys, gs, bs = [], [], []
    for _ in range(nb):
        y = torch.randn((calls, 1, 1, sh.T, C), generator=gen, device="cuda")
        qk = y[..., :2 * sh.HK * sh.DK].reshape(calls, 1, 1, sh.T, 2 * sh.HK, sh.DK)
        qk /= qk.norm(dim=-1, keepdim=True)
        ys.append(y.to(bf))
        gs.append((-torch.nn.functional.softplus(torch.randn((calls, 1, 1, sh.T, sh.HV),
                                                             generator=gen, device="cuda"))).to(bf))
        bs.append(torch.sigmoid(torch.randn((calls, 1, 1, sh.T, sh.HV), generator=gen,
                                            device="cuda")).to(bf))
    st = torch.zeros((1, 1, 1, sh.HV, sh.DK, sh.DV), device="cuda")
    o = torch.empty((1, 1, sh.T, sh.HV, sh.DV), device="cuda", dtype=bf)
    ws = torch.empty(gb.gdn_workspace_size(d), dtype=torch.uint8, device="cuda")

    def prompt(i):
        st.zero_()
        for c in range(calls):
            gb.gdn_prefill_chunked(d, ys[i][c], gs[i][c], bs[i][c], st, None, o, 64, ws)

    for i in range(2):
        prompt(i)
    torch.cuda.synchronize()
    tm = Timer(torch)
    reps = 20
    marks = []
    start = tm.ev()
    for r in range(reps):
        i = r % nb
        st.zero_()
        for c in range(calls):
            e0 = tm.ev()
            gb.gdn_prefill_chunked(d, ys[i][c], gs[i][c], bs[i][c], st, None, o, 64, ws)
            e1 = tm.ev()
            marks.append((e0, e1))
    end = tm.ev()
    torch.cuda.synchronize()
    call_ms = float(np.mean([a.elapsed_time(b) for a, b in marks]))
    total_ms = start.elapsed_time(end)
    Cc, dd = 64, sh.DK
    flop_tok_head = 6 * dd * dd + 5 * Cc * dd + Cc * Cc / 3.0
    flops = flop_tok_head * sh.T * sh.HV
    byts = sh.T * C * 2 + 2 * sh.T * sh.HV * 2 + 2 * sh.HV * sh.DK * sh.DV * 4 \
        + sh.T * sh.HV * sh.DV * 2
    ai = flops / byts
    attainable = min(2500.0, ai * HBM_PEAK_GBS / 1e3)   # TFLOP/s
    tflops = flops / (call_ms / 1e3) / 1e12
    del ys, gs, bs
    torch.cuda.empty_cache()
    return dict(call_ms=call_ms, tokens_per_s=calls * sh.T * reps / (total_ms / 1e3),
                flop_per_call=flops, bytes_per_call=byts, flop_per_byte=ai,
                achieved_tflops=tflops, mfma_peak_tflops=2500.0,
                frac_of_mfma_peak=tflops / 2500.0, attainable_tflops=attainable,
                frac_of_attainable=tflops / attainable,
                hbm_gbs=byts / (call_ms / 1e3) / 1e9, workspace_bytes=ws.numel())


def prefill_ragged(torch, gb, W, args):
    """Eight prompts of unequal length (seeded, 64..1,024 tokens) prefilled in
    one 1,024-token launch into their own rows of a B8 state (32 value / 16
    qk heads, d = 128, bf16 in and out); tokens/s counts real prompt tokens."""
    sh = W.PREFILL.with_(B=8)
    d = gb.make_dims(1, sh.B, sh.T, sh.HV, sh.HK, sh.DK, sh.DV, S=1, act="bf16", out="bf16")
    rng = np.random.default_rng(1005)
    lengths = rng.integers(64, sh.T + 1, size=sh.B).astype(np.int32)
    lengths[0] = sh.T
    C = sh.C
    bf = torch.bfloat16
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5006)
    y = torch.randn((1, sh.B, sh.T, C), generator=gen, device="cuda")
    qk = y[..., :2 * sh.HK * sh.DK].reshape(1, sh.B, sh.T, 2 * sh.HK, sh.DK)
    qk /= qk.norm(dim=-1, keepdim=True)
    y = y.to(bf)
    g = (-torch.nn.functional.softplus(torch.randn((1, sh.B, sh.T, sh.HV), generator=gen,
                                                   device="cuda"))).to(bf)
    b = torch.sigmoid(torch.randn((1, sh.B, sh.T, sh.HV), generator=gen, device="cuda")).to(bf)
    st = torch.zeros((1, sh.B, 1, sh.HV, sh.DK, sh.DV), device="cuda")
    o = torch.empty((1, sh.B, sh.T, sh.HV, sh.DV), device="cuda", dtype=bf)
    ws = torch.empty(gb.gdn_workspace_size(d), dtype=torch.uint8, device="cuda")
    lens = torch.from_numpy(lengths).cuda()
    for _ in range(3):
        gb.gdn_prefill_ragged(d, y, g, b, st, None, o, lens, 64, ws)
    torch.cuda.synchronize()
    reps = 20
    tm = Timer(torch)
    start = tm.ev()
    for _ in range(reps):
        gb.gdn_prefill_ragged(d, y, g, b, st, None, o, lens, 64, ws)
    end = tm.ev()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / reps
    ntok = int(lengths.sum())
    Cc, dd = 64, sh.DK
    flops = (6 * dd * dd + 5 * Cc * dd + Cc * Cc / 3.0) * ntok * sh.HV
    del y, g, b, o, ws
    torch.cuda.empty_cache()
    return dict(lengths=lengths.tolist(), call_ms=ms, tokens_per_s=ntok / (ms / 1e3),
                achieved_tflops=flops / (ms / 1e3) / 1e12)


def gated_rmsnorm(torch, gb, W, args):
    """The gated RMSNorm epilogue over the cohort's verify outputs (30 layers x
    8 rows x 2 tokens x 32 heads x 128, fp32 o, bf16 gate and weight, written
    in place), 10 launches captured in one HIP graph."""
    sh = W.COHORT
    d = gb.make_dims(L_POOL, sh.B, sh.T, sh.HV, sh.HK, sh.DK, sh.DV, S=sh.S, act="bf16",
                     out="f32")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5007)
    shp = (L_POOL, sh.B, sh.T, sh.HV, sh.DV)
    o = torch.randn(shp, generator=gen, device="cuda")
    z = torch.randn(shp, generator=gen, device="cuda").to(torch.bfloat16)
    w = (1.0 + 0.1 * torch.randn((L_POOL, sh.DV), generator=gen, device="cuda")).to(torch.bfloat16)
    act_rows = np.ones(sh.B, np.uint8)
    for r in sh.inactive:
        act_rows[r] = 0
    active = torch.from_numpy(act_rows).cuda()
    gb.gdn_gated_rmsnorm(d, o, z, w, o, active=active)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    n = 10
    with torch.cuda.graph(graph, stream=s):
        for _ in range(n):
            gb.gdn_gated_rmsnorm(d, o, z, w, o, active=active)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    tm = Timer(torch)
    start = tm.ev()
    for _ in range(5):
        graph.replay()
    end = tm.ev()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / (5 * n)
    na = int(act_rows.sum())
    byts = L_POOL * na * sh.T * sh.HV * sh.DV * (4 + 2 + 4) + L_POOL * sh.DV * 2
    del o, z, graph
    torch.cuda.empty_cache()
    return dict(ms_per_call=ms, bytes_per_call=byts, gbs=byts / (ms / 1e3) / 1e9)


def verify_gated_norm(torch, gb, W, args):
    """Verify with the gated RMSNorm fused into its outputs
    (gdn_verify_gated_norm) against the same two steps as separate launches
    (gdn_verify, then gdn_gated_rmsnorm in place), over the cohort's 30 layer
    pools; 20 back-to-back launches of each between HIP events."""
    sh = W.COHORT
    big, t, rng, act_rows = cohort_pools(torch, W, sh, L_POOL, 1001)
    d = gb.make_dims(L_POOL, sh.B, sh.T, sh.HV, sh.HK, sh.DK, sh.DV, S=sh.S, act="bf16",
                     out="f32")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5011)
    z = torch.randn(t["o"].shape, generator=gen, device="cuda").to(torch.bfloat16)
    w = (1.0 + 0.1 * torch.randn((L_POOL, sh.DV), generator=gen, device="cuda")).to(torch.bfloat16)
    ins = [t["x"], t["conv_w"], None, t["conv_state"], t["g"], t["beta"], t["state"], t["cur"]]

    def fused():
        gb.gdn_verify_gated_norm(d, *ins, z, w, t["o"], active=t["active"], err=t["err"])

    def split():
        gb.gdn_verify(d, *ins, t["o"], t["active"], t["err"])
        gb.gdn_gated_rmsnorm(d, t["o"], z, w, t["o"], active=t["active"])

    # the fused commit + verify cycle, each call committing a fixed keep
    keep = torch.from_numpy(W.keep_uniform(rng, sh, act_rows).astype(np.int32)).cuda()
    prev = [t["x"], t["g"], t["beta"], keep, t["x"], t["conv_w"], None, t["conv_state"], t["g"],
            t["beta"], t["state"], t["cur"]]

    def lazy_fused():
        gb.gdn_verify_lazy_gated_norm(d, *prev, z, w, t["o"], active=t["active"], err=t["err"])

    def lazy_split():
        gb.gdn_verify_lazy(d, *prev, t["o"], t["active"], t["err"])
        gb.gdn_gated_rmsnorm(d, t["o"], z, w, t["o"], active=t["active"])

    tm = Timer(torch)
    res = {}
    for name, fn in (("fused", fused), ("split", split), ("fused_again", fused),
                     ("lazy_fused", lazy_fused), ("lazy_split", lazy_split)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        reps = 20
        a = tm.ev()
        for _ in range(reps):
            fn()
        b = tm.ev()
        torch.cuda.synchronize()
        res[name] = a.elapsed_time(b) / reps
    assert int(t["err"].item()) == 0, "device error word set"
    n_act = int(act_rows.sum())
    byts = verify_bytes(sh, n_act, L_POOL) + L_POOL * (n_act * sh.T * sh.HV * sh.DV * 2 + sh.DV * 2)
    ms = min(res["fused"], res["fused_again"])
    del t, z, w
    torch.cuda.empty_cache()
    return dict(fused_ms=ms, split_ms=res["split"], bytes_per_call=byts,
                gbs=byts / (ms / 1e3) / 1e9, lazy_fused_ms=res["lazy_fused"],
                lazy_split_ms=res["lazy_split"])


def cpu_baseline(W, budget_s=12.0):
    """The oracle as it stands (single-threaded C, float64) on a bounded
    sample of the headline workload: whole verify + commit layer-cycles of
    the B8/T2 cohort (8 rows x 32 heads each) until the time budget is used."""
    import oracle
    sh = W.COHORT
    inp = W.verify_inputs(sh, seed=4242)
    od = oracle.Dims(L=1, B=sh.B, T=sh.T, HV=sh.HV, HK=sh.HK, DK=sh.DK, DV=sh.DV, S=sh.S)
    rng = np.random.default_rng(1)
    st, cs, cur = inp["state"], inp["conv_state"], inp["cur"]
    n = 0
    t0 = time.perf_counter()
    while True:
        keep = W.keep_uniform(rng, sh, inp["active"])
        st, _, _ = oracle.verify(od, inp["x"], inp["conv_w"], None, cs, inp["g"], inp["beta"],
                                 st, cur, inp["active"])
        cs, cur, _ = oracle.commit(od, inp["x"], cs, cur, keep, inp["active"])
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 400:
            break
    single = n * sh.B * sh.HV / el

    # The same oracle calls fanned out over the host's cores, one independent
    # layer-cycle stream per thread (the C oracle runs outside the GIL).
    import concurrent.futures as cf
    workers = max(1, min(os.cpu_count() or 1, 16))
    par_budget = budget_s * 0.75

    def stream(seed):
        r = np.random.default_rng(seed)
        s_, c_, u_ = inp["state"].copy(), inp["conv_state"].copy(), inp["cur"].copy()
        k = 0
        t_end = time.perf_counter() + par_budget
        while time.perf_counter() < t_end:
            kp = W.keep_uniform(r, sh, inp["active"])
            s_, _, _ = oracle.verify(od, inp["x"], inp["conv_w"], None, c_, inp["g"], inp["beta"],
                                     s_, u_, inp["active"])
            c_, u_, _ = oracle.commit(od, inp["x"], c_, u_, kp, inp["active"])
            k += 1
        return k

    t1 = time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        counts = list(ex.map(stream, range(100, 100 + workers)))
    el2 = time.perf_counter() - t1
    return dict(value=single, unit="rows*heads/s", cores=1, kind="oracle",
                sample="%d verify+commit layer-cycles of the B8/T2 cohort (8 rows x 32 heads, "
                       "6 active) in %.1f s, single-threaded float64 C oracle incl. marshalling; "
                       "host: %s, %d cpus" % (n, el, platform.processor() or platform.machine(),
                                              os.cpu_count() or 0),
                all_cores=dict(value=sum(counts) * sh.B * sh.HV / el2, cores=workers,
                               sample="%d layer-cycles over %d threads in %.1f s, one independent "
                                      "cycle stream per thread" % (sum(counts), workers, el2)))


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures a single GPU: the path has no cross-GPU exchange, so "
              "--gpus %d is not supported" % max(args.gpus, world), file=sys.stderr)
        sys.exit(2)
    import torch

    from gated_deltanet_recurrence_conv_amd import binding as gb
    from gated_deltanet_recurrence_conv_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_probe:
        copy_probe(torch)
        return
    log("bench: %s on %s" % (gb.gdn_version(), torch.cuda.get_device_name(0)))
    sections = {"per_layer_graph": per_layer_graph, "solo": solo, "rewind": rewind,
                "conv_step": conv_step, "prefill": prefill, "lazy": lazy_cycle,
                "prefill_ragged": prefill_ragged, "gated_rmsnorm": gated_rmsnorm,
                "verify_gated_norm": verify_gated_norm}
    if args.only:
        print(json.dumps({args.only: sections[args.only](torch, gb, W, args)}), flush=True)
        return
    log("bench: headline B8/T2 cohort x %d layers, %d steps" % (L_POOL, args.steps))
    h = headline(torch, gb, W, args)
    log("bench: headline %.4f ms/step  verify %.1f GB/s" % (h["ms_per_step"], h["verify_gbs"]))
    extra = {}
    if not args.only_headline:
        for name, fn in (("lazy_commit_verify_b8_t2", lazy_cycle),
                         ("per_layer_graph_b8_t2", per_layer_graph), ("solo_b1_t3_l30", solo),
                         ("rewind_b8_t4", rewind), ("conv_step_t1024", conv_step),
                         ("prefill_b1_4096_in_1024_calls", prefill),
                         ("prefill_ragged_b8_up_to_1024", prefill_ragged),
                         ("gated_rmsnorm_b8_t2_l30", gated_rmsnorm),
                         ("verify_gated_norm_b8_t2_l30", verify_gated_norm)):
            log("bench: %s" % name)
            extra[name] = fn(torch, gb, W, args)
            log("bench: %s -> %s" % (name, json.dumps(extra[name])))
    cpu = None
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle)")
        cpu = cpu_baseline(W)
    vb = h["verify_bytes"]
    log("bench: device copy rate")
    copy_gbs = stream_copy_gbs(torch)
    rec = {
        "metric": "GDN verify+commit rows*heads/s (B8,T2,32 heads) + achieved HBM GB/s vs peak",
        "value": h["value"],
        "unit": "rows*heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": h["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {"workload": "qwen_verify_cohort_b8_t2_hv32_hk16_d128 x %d layer pools "
                               "(grouped verify + grouped commit per cycle)" % L_POOL,
                   "rows": 8, "active_rows": 6, "T": 2, "value_heads": 32, "qk_heads": 16,
                   "d_k": 128, "d_v": 128, "layers": L_POOL, "inputs": "bf16",
                   "state": "fp32", "keep": "U{0,1,2} per cycle"},
        "roofline": {"bound": "hbm", "kernel": "gdn::recurrent_kernel<128,128,bf16> (verify)",
                     "achieved": h["verify_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": h["verify_gbs"] / HBM_PEAK_GBS,
                     "traffic": counted_traffic("recurrent_kernel_verify_b8_t2_l30"),
                     "algorithmic_bytes_per_launch": vb,
                     "avg_launch_ms": h["verify_ms"],
                     "stream_copy_gbs": copy_gbs,
                     "frac_of_stream": h["verify_gbs"] / copy_gbs},
        "cycle_gbs": h["cycle_gbs"],
        "algorithmic_min_bytes_per_cycle": h["algorithmic_min_bytes_per_cycle"],
        "algorithmic_min_gbs": h["algorithmic_min_gbs"],
        "active_rows_heads_per_s": h["active_rows_heads_per_s"],
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
