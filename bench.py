#!/usr/bin/env python3
"""Benchmark of the Gated DeltaNet verify + commit cycle on one MI355X.

Headline: the B8/T2 verification cohort (32 value heads, 16 qk heads,
d_k = d_v = 128, bf16 inputs, fp32 state, rows 1 and 6 inactive, keep ~
U{0,1,2} drawn per cycle) in a 30-layer hybrid stack, issued the way a model
forward issues it: one gdn_verify per GDN layer (layer l+1's inputs exist
only once layer l has run), then, once acceptance has fixed keep, one
gdn_commit over all 30 layers.  The 30 layer pools (1.44 GiB of fp32 state)
exceed the 256 MiB Infinity Cache, so state traffic is HBM traffic.
Metric: rows*heads/s = 30 layers * 8 rows * 32 heads per cycle / time; the
8 rows include the 2 inactive ones (active_rows_heads_per_s counts only 6).

Every other measurement goes under "extra", each with its own roofline and,
where the oracle can run it, a CPU baseline: the same cycle with one grouped
verify launch over the 30 layers, the fused commit + verify (per layer and
grouped), the solo B1/T3 30-layer cycle, the B8/T4 rewind, the 1,024-token
conv step, the chunked prefill (B1, 4,096 tokens in 1,024-token calls), the
ragged B8 prefill, the gated RMSNorm and its fused forms, and the measured
ceilings (hand-written HBM stream kernels and a bf16 MFMA loop).

  python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--only NAME]
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
BF16_MFMA_PEAK_TFLOPS = 2500.0
L_POOL = 30


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-headline", action="store_true")
    ap.add_argument("--only", default=None,
                    help="run one measurement (a key of SECTIONS) and print its JSON instead of "
                         "the headline line")
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
    (calibrated on a plain copy) for the kernel sources they were taken on;
    None when that record is missing or a source has changed since."""
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
    libgdn call below is launched on (graphs are replayed on it too)."""

    def __init__(self, torch):
        self.torch = torch

    def ev(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return e


def graph_of(torch, fn):
    """Captures fn() once in a HIP graph (on a side stream, after one eager
    warm-up call) and returns it."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        fn()
    torch.cuda.synchronize()
    return graph


def time_graph(torch, graph, reps, warm=2):
    """Average ms per replay of a captured graph, replays back to back
    between two HIP events."""
    for _ in range(warm):
        graph.replay()
    torch.cuda.synchronize()
    tm = Timer(torch)
    a = tm.ev()
    for _ in range(reps):
        graph.replay()
    b = tm.ev()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def roofline(bound, achieved, peak, unit, traffic_key, measured_peak=None, **kw):
    r = {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
         "frac": achieved / peak, "traffic": counted_traffic(traffic_key) if traffic_key else None}
    if measured_peak:
        r["measured_peak"] = measured_peak
        r["frac_of_measured"] = achieved / measured_peak
    r.update(kw)
    return r


def cohort_pools(torch, W, sh, L, seed):
    """L layers of a verify workload: every tensor on the GPU, stacked along the layer axis."""
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
    """Algorithmic bytes of one verify launch over L layers: per active
    (layer, row): the fp32 state read once (HV*DK*DV*4) and written T times as
    candidates, the window inputs x (T*C) and conv cache (3*C) in the act
    dtype, g and beta (2*T*HV), and the fp32 outputs (T*HV*DV*4); per layer
    the conv weights (C*4)."""
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


def lazy_bytes(sh, keep_prev, act_rows, L):
    """Algorithmic bytes of one fused commit + verify cycle over L layers: per
    (layer, row) that replays or verifies, one state read and the 3 conv-cache
    rows; per replayed token its x row and g, beta (keep_prev tokens of the
    previous window); per active row the new window's x, g, beta and its fp32
    outputs; per committing row one state write and the 3 new conv-cache rows;
    per layer the conv weights.  (The kernels also read the previous window's
    unreplayed rows and, on 30-layer grids, re-read the new cache rows in the
    shift launch: counted traffic, not algorithmic bytes.)"""
    esz = 2 if sh.act == "bf16" else 4
    tile = sh.HV * sh.DK * sh.DV * 4
    tok = sh.C * esz + 2 * sh.HV * esz          # one token's x row, g and beta
    per = 0
    for b in range(sh.B):
        kp = int(keep_prev[b])
        if act_rows[b] or kp > 0:
            per += tile + 3 * sh.C * esz + kp * tok
        if kp > 0:
            per += tile + 3 * sh.C * esz
        if act_rows[b]:
            per += sh.T * tok + sh.T * sh.HV * sh.DV * 4
    return L * (per + sh.C * 4 * esz)


def rewind_bytes(sh, keep, L):
    """Algorithmic bytes of one rewind over L layers: per committing (layer,
    row) the state tile read and written back, the keep replayed tokens' x
    rows and g, beta, the 3 conv-cache rows read and the 3 new ones written;
    per layer the conv weights.  (On 30-layer grids the shift launch re-reads
    the new cache rows: counted traffic, not algorithmic bytes.)"""
    esz = 2 if sh.act == "bf16" else 4
    tile = sh.HV * sh.DK * sh.DV * 4
    per = sum(2 * tile + int(kk) * (sh.C * esz + 2 * sh.HV * esz) + 6 * sh.C * esz for kk in keep if kk > 0)
    return L * (per + sh.C * 4 * esz)


# ---------------------------------------------------------------------------
# Measured ceilings: hand-written stream kernels and a bf16 MFMA loop.

def ceilings(torch, gb, W, args):
    """Sustained HBM rates of hand-written stream kernels for the read:write
    mixes of the path's kernels (read-only, write-only, copy 1:1, 1:2 as
    verify at T=2, 1:3 as verify at T=3, 2:1), each over buffers of 512 MiB
    to 1 GiB, best over a small sweep of grid size, vectors per thread,
    non-temporal vs plain access and grid-stride vs per-workgroup contiguous
    blocks; and the dense bf16 MFMA rate of a loop of
    independent v_mfma_f32_16x16x32_bf16 chains."""
    from gated_deltanet_recurrence_conv_amd import ceiling as ce
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    mixes = {"read": (1, 0), "write": (0, 1), "copy": (1, 1), "r1w2": (1, 2), "r1w3": (1, 3),
             "r2w1": (2, 1)}
    total_bytes = 1 << 30
    res = {"cus": cus}
    for name, (nr, nw) in mixes.items():
        nbuf = nr + nw
        per = (total_bytes // max(1, nbuf)) // 16 * 16 if nbuf > 1 else total_bytes
        n_vec = per // 16
        bufs = [torch.empty(per // 4, dtype=torch.float32, device="cuda") for _ in range(nbuf)]
        for bb in bufs:
            bb.fill_(1.0)
        sink = torch.empty(cus * 64 * 4, dtype=torch.float32, device="cuda")
        srcs, dsts = bufs[:nr], bufs[nr:]
        best = (0.0, None)
        configs = [(mult, unroll, nt, False) for mult in (4, 8, 16) for unroll in (2, 4, 8)
                   for nt in (True, False)]
        configs += [(mult, unroll, nt, True) for mult in (2, 4, 8) for unroll in (1, 2, 4)
                    for nt in (True, False)]
        for mult, unroll, nt, blocked in configs:
            grid = cus * mult
            if not dsts and grid * 4 > sink.numel():
                continue

            def run():
                ce.gdn_ceiling_stream(srcs, dsts, n_vec, sink=sink, grid=grid,
                                      unroll=unroll, nontemporal=nt, blocked=blocked)
            run()
            torch.cuda.synchronize()
            tm = Timer(torch)
            reps = 4
            a = tm.ev()
            for _ in range(reps):
                run()
            b = tm.ev()
            torch.cuda.synchronize()
            ms = a.elapsed_time(b) / reps
            gbs = n_vec * 16 * nbuf / (ms / 1e3) / 1e9
            if gbs > best[0]:
                best = (gbs, dict(grid_per_cu=mult, unroll=unroll, nontemporal=nt,
                                  blocked=blocked))
        res[name + "_gbs"] = best[0]
        res[name + "_config"] = best[1]
        del bufs, sink
        torch.cuda.empty_cache()
    out = torch.empty(cus * 4 * 256 * 32, dtype=torch.float32, device="cuda")
    best = 0.0
    for mult in (1, 2, 4):
        grid, iters = cus * mult, 4000
        ce.gdn_ceiling_mfma_bf16(out, grid, iters)
        torch.cuda.synchronize()
        tm = Timer(torch)
        a = tm.ev()
        ce.gdn_ceiling_mfma_bf16(out, grid, iters)
        b = tm.ev()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        best = max(best, grid * 4 * iters * 8 * 16384 / (ms / 1e3) / 1e12)
    res["mfma_bf16_tflops"] = best
    del out
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------
# The oracle beside the GPU: single-threaded and fanned out over host cores.

def oracle_rate(make_stream, units_per_call, unit, sample, budget_s):
    """Runs an oracle call stream for about budget_s on one thread, then one
    independent stream per host thread (up to 16; the C oracle runs outside
    the GIL) for 3/4 of that.  make_stream(seed) returns a function doing one
    call (or one fixed group of calls) of units_per_call units."""
    import concurrent.futures as cf
    step = make_stream(0)
    n = 0
    t0 = time.perf_counter()
    while True:
        step()
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    workers = max(1, min(os.cpu_count() or 1, 16))
    par_budget = budget_s * 0.75

    def stream(seed):
        f = make_stream(seed)
        k = 0
        t_end = time.perf_counter() + par_budget
        while time.perf_counter() < t_end:
            f()
            k += 1
        return k

    t1 = time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        counts = list(ex.map(stream, range(100, 100 + workers)))
    el2 = time.perf_counter() - t1
    return dict(value=n * units_per_call / el, unit=unit, cores=1, kind="oracle",
                sample="%d calls of %s in %.1f s, single-threaded float64 C oracle incl. "
                       "marshalling; host: %s, %d cpus" % (n, sample, el,
                                                           platform.processor() or platform.machine(),
                                                           os.cpu_count() or 0),
                all_cores=dict(value=sum(counts) * units_per_call / el2, cores=workers,
                               sample="%d calls over %d threads in %.1f s, one independent stream "
                                      "per thread" % (sum(counts), workers, el2)))


def cpu_cohort(W, budget_s):
    """verify + commit layer-cycles of the B8/T2 cohort (8 rows x 32 heads, 6 active)."""
    import oracle
    sh = W.COHORT
    inp = W.verify_inputs(sh, seed=4242)
    od = oracle.Dims(L=1, B=sh.B, T=sh.T, HV=sh.HV, HK=sh.HK, DK=sh.DK, DV=sh.DV, S=sh.S)

    def make(seed):
        r = np.random.default_rng(seed)
        s = dict(st=inp["state"].copy(), cs=inp["conv_state"].copy(), cur=inp["cur"].copy())

        def step():
            keep = W.keep_uniform(r, sh, inp["active"])
            s["st"], _, _ = oracle.verify(od, inp["x"], inp["conv_w"], None, s["cs"], inp["g"],
                                          inp["beta"], s["st"], s["cur"], inp["active"])
            s["cs"], s["cur"], _ = oracle.commit(od, inp["x"], s["cs"], s["cur"], keep, inp["active"])
        return step
    return oracle_rate(make, sh.B * sh.HV, "rows*heads/s",
                       "one verify+commit layer-cycle of the B8/T2 cohort (8 rows x 32 heads, 6 "
                       "active)", budget_s)


def cpu_solo(W, budget_s):
    """verify + commit layer-cycles of the solo B1/T3 shape (one of its 30
    independent layers per call), keep by prefix acceptance p = 0.8."""
    import oracle
    sh = W.SOLO.with_(L=1)
    inp = W.verify_inputs(sh, seed=4343)
    od = oracle.Dims(L=1, B=1, T=sh.T, HV=sh.HV, HK=sh.HK, DK=sh.DK, DV=sh.DV, S=sh.S)

    def make(seed):
        r = np.random.default_rng(seed)
        s = dict(st=inp["state"].copy(), cs=inp["conv_state"].copy(), cur=inp["cur"].copy())

        def step():
            keep = W.keep_prefix_acceptance(r, sh)
            s["st"], _, _ = oracle.verify(od, inp["x"], inp["conv_w"], None, s["cs"], inp["g"],
                                          inp["beta"], s["st"], s["cur"], None)
            s["cs"], s["cur"], _ = oracle.commit(od, inp["x"], s["cs"], s["cur"], keep, None)
        return step
    return oracle_rate(make, sh.HV, "rows*heads/s",
                       "one verify+commit layer-cycle of the solo B1/T3 shape (1 row x 32 heads)",
                       budget_s)


def cpu_rewind(W, budget_s):
    """Rewind calls of the B8/T4 shape (one layer per call), keep ~ U{0..4}."""
    import oracle
    sh = W.REWIND
    inp = W.verify_inputs(sh, seed=4444)
    od = oracle.Dims(L=1, B=sh.B, T=sh.T, HV=sh.HV, HK=sh.HK, DK=sh.DK, DV=sh.DV, S=sh.S)

    def make(seed):
        r = np.random.default_rng(seed)

        def step():
            keep = W.keep_uniform(r, sh)
            oracle.rewind(od, inp["x"], inp["conv_w"], None, inp["conv_state"], inp["g"],
                          inp["beta"], inp["state"], inp["cur"], keep)
        return step
    return oracle_rate(make, sh.B * sh.HV, "rows*heads/s",
                       "one B8/T4 rewind layer-call (8 rows x 32 heads, keep ~ U{0..4})", budget_s)


def cpu_prefill(W, budget_s):
    """Token-sequential prefill of the Qwen head shape (32 value / 16 qk heads,
    d = 128), 64 tokens per call with the state carried."""
    import oracle
    sh = W.PREFILL
    n = 64
    inp = W.prefill_inputs(sh, seed=4545, tokens=n)
    od = oracle.Dims(L=1, B=1, T=n, HV=sh.HV, HK=sh.HK, DK=sh.DK, DV=sh.DV, S=1)

    def make(seed):
        s = dict(st=inp["state"].copy())

        def step():
            s["st"], _, _ = oracle.prefill(od, inp["y"], inp["g"], inp["beta"], s["st"], inp["cur"])
        return step
    return oracle_rate(make, n, "tokens/s",
                       "a 64-token prefill call at 32 value / 16 qk heads, d = 128, state carried",
                       budget_s)


# ---------------------------------------------------------------------------
# GPU legs.

def per_layer_cycle(torch, gb, W, args, ceil):
    """The headline cycle, as a model forward issues it: gdn_verify on each of
    the 30 layers in turn (one launch per layer), then one gdn_commit over all
    30 layers with the cycle's keep (acceptance needs the last layer's
    logits, so no layer commits before every layer has verified).  The K
    timed cycles (fresh keep each) are captured once in a HIP graph and
    replayed, so the time is the GPU's, not the host's launch rate.  The
    per-launch verify time for the roofline comes from a graph of 30
    per-layer verify launches replayed back to back (verify writes only
    candidate slots, so repeating it changes nothing)."""
    sh = W.COHORT
    big, t, rng, act_rows = cohort_pools(torch, W, sh, L_POOL, 1001)
    d1 = gb.make_dims(1, sh.B, sh.T, sh.HV, sh.HK, sh.DK, sh.DV, S=sh.S, act="bf16", out="f32")
    dL = gb.make_dims(L_POOL, sh.B, sh.T, sh.HV, sh.HK, sh.DK, sh.DV, S=sh.S, act="bf16",
                      out="f32")
    n = args.steps + args.warmup
    keeps = np.stack([W.keep_uniform(rng, sh, act_rows) for _ in range(n)]).astype(np.int32)
    keep_d = torch.from_numpy(keeps).cuda()

    def verify_layers():
        for l in range(L_POOL):
            sl = slice(l, l + 1)
            gb.gdn_verify(d1, t["x"][sl], t["conv_w"][sl], None, t["conv_state"][sl],
                          t["g"][sl], t["beta"][sl], t["state"][sl], t["cur"][sl], t["o"][sl],
                          t["active"], t["err"])

    def cycle(i):
        verify_layers()
        gb.gdn_commit(dL, t["x"], t["conv_state"], t["cur"], keep_d[i], t["active"], t["err"])

    for i in range(args.warmup):
        cycle(i)
    torch.cuda.synchronize()

    def timed():
        for i in range(args.warmup, n):
            cycle(i)
    graph = graph_of(torch, timed)
    tm = Timer(torch)
    start = tm.ev()
    graph.replay()
    end = tm.ev()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    assert int(t["err"].item()) == 0, "device error word set"
    del graph
    vgraph = graph_of(torch, verify_layers)
    verify_ms = time_graph(torch, vgraph, 10) / L_POOL
    assert int(t["err"].item()) == 0, "device error word set"
    n_act = int(act_rows.sum())
    vb = verify_bytes(sh, n_act, 1)
    cb = float(np.mean([commit_bytes(sh, keeps[i], act_rows, L_POOL) for i in range(args.warmup, n)]))
    amin = float(np.mean([algorithmic_min_bytes(sh, keeps[i], act_rows, L_POOL)
                          for i in range(args.warmup, n)]))
    ms_step = total_ms / args.steps
    res = dict(ms_per_step=ms_step, value=L_POOL * sh.B * sh.HV / (ms_step / 1e3),
               active_rows_heads_per_s=L_POOL * n_act * sh.HV / (ms_step / 1e3),
               launches_per_step=L_POOL + 1, verify_ms_per_layer=verify_ms,
               verify_bytes_per_layer=vb, commit_bytes=cb,
               cycle_gbs=(L_POOL * vb + cb) / (ms_step / 1e3) / 1e9,
               algorithmic_min_bytes_per_cycle=amin,
               algorithmic_min_gbs=amin / (ms_step / 1e3) / 1e9)
    res["roofline"] = roofline("hbm", vb / (verify_ms / 1e3) / 1e9, HBM_PEAK_GBS, "GB/s",
                               "recurrent_kernel_verify_b8_t2_l1",
                               measured_peak=ceil.get("r1w2_gbs"),
                               kernel="gdn::recurrent_kernel<128,128,bf16> (verify, one layer)",
                               algorithmic_bytes_per_launch=vb, avg_launch_ms=verify_ms)
    del t, vgraph
    torch.cuda.empty_cache()
    return res


def grouped_cycle(torch, gb, W, args, ceil):
    """The cycle with one grouped verify launch over the 30 layer pools and one
    grouped commit (a launch shape for independent layers; a model forward
    issues per-layer verifies), graph-replayed as the headline."""
    sh = W.COHORT
    big, t, rng, act_rows = cohort_pools(torch, W, sh, L_POOL, 1001)
    d = gb.make_dims(L_POOL, sh.B, sh.T, sh.HV, sh.HK, sh.DK, sh.DV, S=sh.S, act="bf16",
                     out="f32")
    n = args.steps + args.warmup
    keeps = np.stack([W.keep_uniform(rng, sh, act_rows) for _ in range(n)]).astype(np.int32)
    keep_d = torch.from_numpy(keeps).cuda()

    def verify():
        gb.gdn_verify(d, t["x"], t["conv_w"], None, t["conv_state"], t["g"], t["beta"],
                      t["state"], t["cur"], t["o"], t["active"], t["err"])

    def step(i):
        verify()
        gb.gdn_commit(d, t["x"], t["conv_state"], t["cur"], keep_d[i], t["active"], t["err"])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    def timed():
        for i in range(args.warmup, n):
            step(i)
    graph = graph_of(torch, timed)
    tm = Timer(torch)
    start = tm.ev()
    graph.replay()
    end = tm.ev()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    assert int(t["err"].item()) == 0, "device error word set"
    reps = 20
    v0 = tm.ev()
    for _ in range(reps):
        verify()
    v1 = tm.ev()
    torch.cuda.synchronize()
    verify_ms = v0.elapsed_time(v1) / reps
    n_act = int(act_rows.sum())
    vb = verify_bytes(sh, n_act, L_POOL)
    cb = float(np.mean([commit_bytes(sh, keeps[i], act_rows, L_POOL) for i in range(args.warmup, n)]))
    amin = float(np.mean([algorithmic_min_bytes(sh, keeps[i], act_rows, L_POOL)
                          for i in range(args.warmup, n)]))
    ms_step = total_ms / args.steps
    res = dict(ms_per_step=ms_step, rows_heads_per_s=L_POOL * sh.B * sh.HV / (ms_step / 1e3),
               active_rows_heads_per_s=L_POOL * n_act * sh.HV / (ms_step / 1e3),
               launches_per_step=2, verify_ms=verify_ms, verify_bytes=vb, commit_bytes=cb,
               cycle_gbs=(vb + cb) / (ms_step / 1e3) / 1e9,
               algorithmic_min_bytes_per_cycle=amin,
               algorithmic_min_gbs=amin / (ms_step / 1e3) / 1e9)
    res["roofline"] = roofline("hbm", vb / (verify_ms / 1e3) / 1e9, HBM_PEAK_GBS, "GB/s",
                               "recurrent_kernel_verify_b8_t2_l30",
                               measured_peak=ceil.get("r1w2_gbs"),
                               kernel="gdn::recurrent_kernel<128,128,bf16> (verify, 30 layers)",
                               algorithmic_bytes_per_launch=vb, avg_launch_ms=verify_ms)
    del t, graph
    torch.cuda.empty_cache()
    return res


def lazy_legs(torch, gb, W, args, ceil):
    """The cohort cycle with the commit folded into the next verify
    (gdn_verify_lazy): each cycle replays the previous cycle's accepted
    tokens from the snapshot, writes the committed state once in place, and
    verifies the new window without candidate writes.  Per layer (30 calls
    per cycle, as a model forward issues them) and grouped (one call over the
    30 layers); the headline's pools, 3 untimed and 20 timed cycles of seeded
    keeps, replayed from a graph.  The sample is fixed (not --steps) so that
    the bytes priced here and the counters of a profiled run come from the
    same keep vectors.  A one-layer call is one launch (its workgroups, one per qk head, also
    shift the conv cache); the 30-layer call is two (the replay-and-verify
    kernel and the conv-cache shift).  The roofline prices the whole cycle's
    bytes against its time."""
    sh = W.COHORT
    big, t, rng, act_rows = cohort_pools(torch, W, sh, L_POOL, 1001)
    d1 = gb.make_dims(1, sh.B, sh.T, sh.HV, sh.HK, sh.DK, sh.DV, S=sh.S, act="bf16", out="f32")
    dL = gb.make_dims(L_POOL, sh.B, sh.T, sh.HV, sh.HK, sh.DK, sh.DV, S=sh.S, act="bf16",
                      out="f32")
    warm, cycles = 3, 20
    n = warm + cycles
    keeps = np.stack([W.keep_uniform(rng, sh, act_rows) for _ in range(n)]).astype(np.int32)
    keep_d = torch.from_numpy(keeps).cuda()

    def call(d, sl, i):
        # the previous window's inputs are the same pool tensors (the bench
        # does not change x between cycles); keep_prev is the previous keep
        gb.gdn_verify_lazy(d, t["x"][sl] if i else None, t["g"][sl] if i else None,
                           t["beta"][sl] if i else None, keep_d[i - 1] if i else None, t["x"][sl],
                           t["conv_w"][sl], None, t["conv_state"][sl], t["g"][sl], t["beta"][sl],
                           t["state"][sl], t["cur"][sl], t["o"][sl], t["active"], t["err"])

    def cycle_layers(i):
        for l in range(L_POOL):
            call(d1, slice(l, l + 1), i)

    def cycle_grouped(i):
        call(dL, slice(0, L_POOL), i)

    res = {}
    byts = float(np.mean([lazy_bytes(sh, keeps[i - 1], act_rows, L_POOL) for i in range(warm, n)]))
    for name, cyc, launches, tkey in (("per_layer", cycle_layers, L_POOL, "lazy_per_layer_b8_t2_l30"),
                                      ("grouped", cycle_grouped, 2, "lazy_b8_t2_l30")):
        for i in range(warm):
            cyc(i)
        torch.cuda.synchronize()

        def timed():
            for i in range(warm, n):
                cyc(i)
        graph = graph_of(torch, timed)
        tm = Timer(torch)
        start = tm.ev()
        graph.replay()
        end = tm.ev()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / cycles
        assert int(t["err"].item()) == 0, "device error word set"
        del graph
        gbs = byts / (ms / 1e3) / 1e9
        res[name] = dict(ms_per_cycle=ms, rows_heads_per_s=L_POOL * sh.B * sh.HV / (ms / 1e3),
                         bytes_per_cycle=byts, gbs=gbs, launches_per_cycle=launches,
                         roofline=roofline("hbm", gbs, HBM_PEAK_GBS, "GB/s", tkey,
                                           measured_peak=ceil.get("copy_gbs"),
                                           kernel="recurrent_kernel (lazy) + window_kernel, whole cycle"))
    del t
    torch.cuda.empty_cache()
    return res


def solo(torch, gb, W, args, ceil):
    """B=1, T=3 (two drafts + bonus), 30 independent layers in one grouped
    launch, keep by prefix acceptance p=0.8, state carried across cycles."""
    sh = W.SOLO
    big, t, rng, act_rows = cohort_pools(torch, W, sh.with_(L=1), sh.L, 2002)
    d = gb.make_dims(sh.L, 1, sh.T, sh.HV, sh.HK, sh.DK, sh.DV, S=sh.S, act="bf16", out="f32")
    cycles = 200
    keeps = torch.from_numpy(np.stack([W.keep_prefix_acceptance(rng, sh) for _ in range(cycles)])
                             .astype(np.int32)).cuda()

    def verify():
        gb.gdn_verify(d, t["x"], t["conv_w"], None, t["conv_state"], t["g"], t["beta"],
                      t["state"], t["cur"], t["o"], None, t["err"])

    def cyc(i):
        verify()
        gb.gdn_commit(d, t["x"], t["conv_state"], t["cur"], keeps[i], None, t["err"])

    for i in range(10):
        cyc(i)
    torch.cuda.synchronize()

    def timed():
        for i in range(cycles):
            cyc(i)
    graph = graph_of(torch, timed)
    tm = Timer(torch)
    start = tm.ev()
    graph.replay()
    end = tm.ev()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / cycles
    del graph
    vgraph = graph_of(torch, lambda: [verify() for _ in range(20)])
    vms = time_graph(torch, vgraph, 5) / 20
    vb = verify_bytes(sh, 1, sh.L)
    assert int(t["err"].item()) == 0
    del t, vgraph
    torch.cuda.empty_cache()
    return dict(ms_per_cycle=ms, rows_heads_per_s=sh.L * sh.HV / (ms / 1e3), verify_ms=vms,
                verify_bytes=vb,
                roofline=roofline("hbm", vb / (vms / 1e3) / 1e9, HBM_PEAK_GBS, "GB/s",
                                  "recurrent_kernel_verify_b1_t3_l30",
                                  measured_peak=ceil.get("r1w3_gbs"),
                                  kernel="gdn::recurrent_kernel<128,128,bf16> (verify, B1/T3, 30 layers)",
                                  algorithmic_bytes_per_launch=vb, avg_launch_ms=vms))


def rewind(torch, gb, W, args, ceil):
    """B=8, T=4 captured window, keep ~ U{0..4}, 30 layer pools in one grouped
    call (the replay kernel, then the conv-cache shift); 20 calls with fresh
    keep vectors captured in one HIP graph."""
    sh = W.REWIND
    big, t, rng, act_rows = cohort_pools(torch, W, sh.with_(L=1), L_POOL, 3003)
    d = gb.make_dims(L_POOL, sh.B, sh.T, sh.HV, sh.HK, sh.DK, sh.DV, S=sh.S, act="bf16",
                     out="f32")
    reps = 20
    keeps_np = np.stack([W.keep_uniform(rng, sh) for _ in range(reps + 3)]).astype(np.int32)
    keeps = torch.from_numpy(keeps_np).cuda()

    def call(i):
        gb.gdn_rewind(d, t["x"], t["conv_w"], None, t["conv_state"], t["g"], t["beta"],
                      t["state"], t["cur"], keeps[i], None, t["err"])

    for i in range(3):
        call(i)
    torch.cuda.synchronize()
    graph = graph_of(torch, lambda: [call(i) for i in range(3, reps + 3)])
    ms = time_graph(torch, graph, 1, warm=1) / reps
    per_call = np.mean([rewind_bytes(sh, row, L_POOL) for row in keeps_np[3:]])
    assert int(t["err"].item()) == 0
    del t, graph
    torch.cuda.empty_cache()
    gbs = per_call / (ms / 1e3) / 1e9
    return dict(ms_per_call=ms, bytes_per_call=float(per_call), gbs=gbs,
                rows_heads_per_s=L_POOL * sh.B * sh.HV / (ms / 1e3),
                roofline=roofline("hbm", gbs, HBM_PEAK_GBS, "GB/s", "rewind_b8_t4_l30",
                                  measured_peak=ceil.get("copy_gbs"),
                                  kernel="gdn::recurrent_kernel (rewind) + gdn::window_kernel, per call",
                                  algorithmic_bytes_per_launch=float(per_call), avg_launch_ms=ms))


def conv_step(torch, gb, W, args, ceil):
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
    graph = graph_of(torch, lambda: [gb.gdn_conv_step(d, xs[i], w, None, cs, ys[i], None, True)
                                     for i in range(nb)])
    ms = time_graph(torch, graph, 10) / nb
    byts = 2 * sh.T * C * 2 + C * 4 * 2 + 6 * C * 2
    gbs = byts / (ms / 1e3) / 1e9
    return dict(tokens=sh.T, ms_per_call=ms, bytes_per_call=byts, gbs=gbs,
                roofline=roofline("hbm", gbs, HBM_PEAK_GBS, "GB/s", "conv_kernel_t1024_c8192",
                                  measured_peak=ceil.get("copy_gbs"), kernel="gdn::conv_kernel<bf16,4>",
                                  algorithmic_bytes_per_launch=byts, avg_launch_ms=ms))


def prefill_flops(tokens, HV, d, chunk=64):
    """Algorithmic flops of the chunked form per token-head (triangular-aware):
    6 d^2 + 5 C d + C^2 / 3."""
    return (6 * d * d + 5 * chunk * d + chunk * chunk / 3.0) * tokens * HV


def prefill(torch, gb, W, args, ceil):
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
    # per-call time: the calls of 10 prompts captured in one graph (the state
    # is not re-zeroed inside it, so only prefill launches are timed; it stays
    # bounded, the gates decay it)
    graph = graph_of(torch, lambda: [gb.gdn_prefill_chunked(d, ys[i][c], gs[i][c], bs[i][c], st,
                                                            None, o, 64, ws)
                                     for i in range(nb) for c in range(calls)])
    prompt_ms = time_graph(torch, graph, 3) / nb
    del graph
    # per-call time by HIP events around each eager call
    tm = Timer(torch)
    marks = []
    for r in range(8):
        i = r % nb
        st.zero_()
        for c in range(calls):
            e0 = tm.ev()
            gb.gdn_prefill_chunked(d, ys[i][c], gs[i][c], bs[i][c], st, None, o, 64, ws)
            e1 = tm.ev()
            marks.append((e0, e1))
    torch.cuda.synchronize()
    call_ms_events = float(np.mean([a.elapsed_time(b) for a, b in marks]))
    call_ms = prompt_ms / calls
    flops = prefill_flops(sh.T, sh.HV, sh.DK)
    byts = sh.T * C * 2 + 2 * sh.T * sh.HV * 2 + 2 * sh.HV * sh.DK * sh.DV * 4 \
        + sh.T * sh.HV * sh.DV * 2
    ai = flops / byts
    attainable = min(BF16_MFMA_PEAK_TFLOPS, ai * HBM_PEAK_GBS / 1e3)   # TFLOP/s
    tflops = flops / (call_ms / 1e3) / 1e12
    gbs = byts / (call_ms / 1e3) / 1e9
    meas = None
    if ceil.get("mfma_bf16_tflops") and ceil.get("copy_gbs"):
        meas = min(ceil["mfma_bf16_tflops"], ai * ceil["copy_gbs"] / 1e3)
    del ys, gs, bs
    torch.cuda.empty_cache()
    return dict(call_ms=call_ms, call_ms_eager_events=call_ms_events,
                tokens_per_s=sh.T / (call_ms / 1e3),
                flop_per_call=flops, bytes_per_call=byts, flop_per_byte=ai,
                achieved_tflops=tflops, frac_of_mfma_peak=tflops / BF16_MFMA_PEAK_TFLOPS,
                attainable_tflops=attainable, frac_of_attainable=tflops / attainable,
                hbm_gbs=gbs, workspace_bytes=ws.numel(),
                roofline=roofline("hbm", gbs, HBM_PEAK_GBS, "GB/s", "prefill_b1_t1024",
                                  kernel="prefill_prep_kernel + prefill_scan_kernel, per call",
                                  algorithmic_bytes_per_launch=byts, avg_launch_ms=call_ms,
                                  achieved_tflops=tflops, attainable_tflops=attainable,
                                  measured_attainable_tflops=meas,
                                  frac_of_measured_attainable=(tflops / meas) if meas else None))


def prefill_ragged(torch, gb, W, args, ceil):
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
    graph = graph_of(torch, lambda: [gb.gdn_prefill_ragged(d, y, g, b, st, None, o, lens, 64, ws)
                                     for _ in range(10)])
    ms = time_graph(torch, graph, 2) / 10
    ntok = int(lengths.sum())
    flops = prefill_flops(ntok, sh.HV, sh.DK)
    byts = ntok * (C * 2 + 2 * sh.HV * 2 + sh.HV * sh.DV * 2) + 2 * sh.B * sh.HV * sh.DK * sh.DV * 4
    attainable = min(BF16_MFMA_PEAK_TFLOPS, flops / byts * HBM_PEAK_GBS / 1e3)
    tflops = flops / (ms / 1e3) / 1e12
    del y, g, b, o, ws, graph
    torch.cuda.empty_cache()
    gbs = byts / (ms / 1e3) / 1e9
    return dict(lengths=lengths.tolist(), call_ms=ms, tokens_per_s=ntok / (ms / 1e3),
                achieved_tflops=tflops, attainable_tflops=attainable,
                frac_of_attainable=tflops / attainable, bytes_per_call=byts,
                roofline=roofline("hbm", gbs, HBM_PEAK_GBS, "GB/s", "prefill_ragged_b8_t1024",
                                  kernel="prefill_prep_kernel + prefill_scan_kernel, per call",
                                  algorithmic_bytes_per_launch=byts, avg_launch_ms=ms,
                                  achieved_tflops=tflops, attainable_tflops=attainable))


def conv_prefill(torch, gb, W, args, ceil):
    """The prompt path from the raw projection: B1 4,096-token prompts in
    1,024-token calls (32 value / 16 qk heads, d = 128, bf16 in and out),
    gdn_prefill_conv_chunked against gdn_conv_step + gdn_prefill_chunked,
    each as the calls of 10 prompt buffers captured in one HIP graph (the
    state and conv cache run on across them)."""
    sh = W.PREFILL
    nb, calls = 10, W.PREFILL_TOKENS // sh.T
    C = sh.C
    d = gb.make_dims(1, 1, sh.T, sh.HV, sh.HK, sh.DK, sh.DV, S=1, act="bf16", out="bf16")
    bf = torch.bfloat16
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5013)
    xs = [(torch.randn((calls, 1, 1, sh.T, C), generator=gen, device="cuda")).to(bf) for _ in range(nb)]
    gs = [(-torch.nn.functional.softplus(torch.randn((calls, 1, 1, sh.T, sh.HV), generator=gen,
                                                     device="cuda"))).to(bf) for _ in range(nb)]
    bs = [torch.sigmoid(torch.randn((calls, 1, 1, sh.T, sh.HV), generator=gen, device="cuda")).to(bf)
          for _ in range(nb)]
    w = (0.5 * torch.randn((1, C, 4), generator=gen, device="cuda")).to(bf)
    cs = torch.zeros((1, 1, 3, C), device="cuda", dtype=bf)
    st = torch.zeros((1, 1, 1, sh.HV, sh.DK, sh.DV), device="cuda")
    o = torch.empty((1, 1, sh.T, sh.HV, sh.DV), device="cuda", dtype=bf)
    y = torch.empty((1, 1, sh.T, C), device="cuda", dtype=bf)
    ws = torch.empty(gb.gdn_workspace_size(d), dtype=torch.uint8, device="cuda")

    def fused(i, c):
        gb.gdn_prefill_conv_chunked(d, xs[i][c], w, None, cs, gs[i][c], bs[i][c], st, None, o, 64, ws)

    def two(i, c):
        gb.gdn_conv_step(d, xs[i][c], w, None, cs, y, None, True)
        gb.gdn_prefill_chunked(d, y, gs[i][c], bs[i][c], st, None, o, 64, ws)

    res = {}
    for name, fn in (("fused", fused), ("conv_step_then_prefill", two)):
        for i in range(2):
            for c in range(calls):
                fn(i, c)
        torch.cuda.synchronize()
        graph = graph_of(torch, lambda: [fn(i, c) for i in range(nb) for c in range(calls)])
        res[name + "_call_ms"] = time_graph(torch, graph, 3) / (nb * calls)
        del graph
    res["tokens_per_s_fused"] = sh.T / (res["fused_call_ms"] / 1e3)
    res["saved_fraction"] = 1.0 - res["fused_call_ms"] / res["conv_step_then_prefill_call_ms"]
    del xs, gs, bs, ws
    torch.cuda.empty_cache()
    return res


def prefill_gated_norm(torch, gb, W, args, ceil):
    """The gated RMSNorm after a 1,024-token prefill call (B1, 32 value / 16
    qk heads, d = 128, bf16 in and out): the call alone against the call
    followed by gdn_gated_rmsnorm over its outputs (o written in place), each
    as 10 calls captured in one HIP graph.  The difference is the most a norm
    fused into the prefill could save."""
    sh = W.PREFILL
    d = gb.make_dims(1, 1, sh.T, sh.HV, sh.HK, sh.DK, sh.DV, S=1, act="bf16", out="bf16")
    bf = torch.bfloat16
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5012)
    y = torch.randn((1, 1, sh.T, sh.C), generator=gen, device="cuda")
    qk = y[..., :2 * sh.HK * sh.DK].reshape(1, 1, sh.T, 2 * sh.HK, sh.DK)
    qk /= qk.norm(dim=-1, keepdim=True)
    y = y.to(bf)
    g = (-torch.nn.functional.softplus(torch.randn((1, 1, sh.T, sh.HV), generator=gen, device="cuda"))).to(bf)
    b = torch.sigmoid(torch.randn((1, 1, sh.T, sh.HV), generator=gen, device="cuda")).to(bf)
    z = torch.randn((1, 1, sh.T, sh.HV, sh.DV), generator=gen, device="cuda").to(bf)
    w = (1.0 + 0.1 * torch.randn((1, sh.DV), generator=gen, device="cuda")).to(bf)
    st = torch.zeros((1, 1, 1, sh.HV, sh.DK, sh.DV), device="cuda")
    o = torch.empty((1, 1, sh.T, sh.HV, sh.DV), device="cuda", dtype=bf)
    ws = torch.empty(gb.gdn_workspace_size(d), dtype=torch.uint8, device="cuda")

    def call():
        gb.gdn_prefill_chunked(d, y, g, b, st, None, o, 64, ws)

    def call_norm():
        call()
        gb.gdn_gated_rmsnorm(d, o, z, w, o)

    res = {}
    for name, fn in (("prefill", call), ("prefill_then_norm", call_norm)):
        fn()
        torch.cuda.synchronize()
        graph = graph_of(torch, lambda: [fn() for _ in range(10)])
        res[name + "_ms"] = time_graph(torch, graph, 5) / 10
        del graph
    res["norm_ms"] = res["prefill_then_norm_ms"] - res["prefill_ms"]
    res["norm_bytes"] = sh.T * sh.HV * sh.DV * 2 * 3 + sh.DV * 2
    del y, g, b, z, o, ws
    torch.cuda.empty_cache()
    return res


def gated_rmsnorm(torch, gb, W, args, ceil):
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
    n = 10
    graph = graph_of(torch, lambda: [gb.gdn_gated_rmsnorm(d, o, z, w, o, active=active)
                                     for _ in range(n)])
    ms = time_graph(torch, graph, 5, warm=1) / n
    na = int(act_rows.sum())
    byts = L_POOL * na * sh.T * sh.HV * sh.DV * (4 + 2 + 4) + L_POOL * sh.DV * 2
    del o, z, graph
    torch.cuda.empty_cache()
    return dict(ms_per_call=ms, bytes_per_call=byts, gbs=byts / (ms / 1e3) / 1e9)


def verify_gated_norm(torch, gb, W, args, ceil):
    """Verify with the gated RMSNorm fused into its outputs
    (gdn_verify_gated_norm) against the same two steps as separate launches
    (gdn_verify, then gdn_gated_rmsnorm in place), and the same for the fused
    commit + verify, over the cohort's 30 layer pools.  Each variant is timed
    twice, interleaved (20 back-to-back calls between HIP events each time),
    and reported as the better of its two runs."""
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
    runs = {}
    order = (("fused", fused), ("split", split), ("lazy_fused", lazy_fused),
             ("lazy_split", lazy_split))
    for _ in range(2):
        for name, fn in order:
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            reps = 20
            a = tm.ev()
            for _ in range(reps):
                fn()
            b = tm.ev()
            torch.cuda.synchronize()
            runs.setdefault(name, []).append(a.elapsed_time(b) / reps)
    assert int(t["err"].item()) == 0, "device error word set"
    n_act = int(act_rows.sum())
    byts = verify_bytes(sh, n_act, L_POOL) + L_POOL * (n_act * sh.T * sh.HV * sh.DV * 2 + sh.DV * 2)
    best = {k: min(v) for k, v in runs.items()}
    del t, z, w
    torch.cuda.empty_cache()
    return dict(fused_ms=best["fused"], split_ms=best["split"], bytes_per_call=byts,
                gbs=byts / (best["fused"] / 1e3) / 1e9, lazy_fused_ms=best["lazy_fused"],
                lazy_split_ms=best["lazy_split"], runs_ms=runs)


SECTIONS = {"per_layer": per_layer_cycle, "grouped": grouped_cycle, "lazy": lazy_legs,
            "solo": solo, "rewind": rewind, "conv_step": conv_step, "prefill": prefill,
            "prefill_ragged": prefill_ragged, "gated_rmsnorm": gated_rmsnorm,
            "verify_gated_norm": verify_gated_norm, "prefill_gated_norm": prefill_gated_norm,
            "conv_prefill": conv_prefill,
            "ceilings": ceilings}

EXTRA = (("grouped_verify_commit_b8_t2_l30", "grouped"), ("lazy_commit_verify_b8_t2", "lazy"),
         ("solo_b1_t3_l30", "solo"), ("rewind_b8_t4_l30", "rewind"),
         ("conv_step_t1024", "conv_step"), ("prefill_b1_4096_in_1024_calls", "prefill"),
         ("prefill_ragged_b8_up_to_1024", "prefill_ragged"),
         ("gated_rmsnorm_b8_t2_l30", "gated_rmsnorm"),
         ("verify_gated_norm_b8_t2_l30", "verify_gated_norm"),
         ("prefill_gated_norm_b1_t1024", "prefill_gated_norm"),
         ("conv_prefill_b1_4096_in_1024_calls", "conv_prefill"))

CPU_LEGS = {"solo_b1_t3_l30": cpu_solo, "rewind_b8_t4_l30": cpu_rewind,
            "prefill_b1_4096_in_1024_calls": cpu_prefill}


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
    if args.only:
        ceil = {}
        print(json.dumps({args.only: SECTIONS[args.only](torch, gb, W, args, ceil)}), flush=True)
        return
    ceil = {}
    if not args.only_headline:
        log("bench: ceilings")
        ceil = ceilings(torch, gb, W, args)
        log("bench: ceilings -> %s" % json.dumps(ceil))
    log("bench: headline B8/T2 cohort x %d layers, per-layer verify, %d steps" % (L_POOL, args.steps))
    h = per_layer_cycle(torch, gb, W, args, ceil)
    log("bench: headline %.4f ms/step  verify %.2f us/layer (%.1f GB/s)"
        % (h["ms_per_step"], h["verify_ms_per_layer"] * 1e3, h["roofline"]["achieved"]))
    extra = {}
    if not args.only_headline:
        for name, key in EXTRA:
            log("bench: %s" % name)
            extra[name] = SECTIONS[key](torch, gb, W, args, ceil)
            log("bench: %s -> %s" % (name, json.dumps(extra[name])))
        extra["ceilings"] = ceil
    cpu = None
    if not args.no_cpu_baseline:
        log("bench: cpu baselines (oracle)")
        cpu = cpu_cohort(W, 10.0)
        if not args.only_headline:
            for name, fn in CPU_LEGS.items():
                extra[name]["cpu_baseline"] = fn(W, 5.0)
                log("bench: cpu %s -> %.1f %s" % (name, extra[name]["cpu_baseline"]["value"],
                                                  extra[name]["cpu_baseline"]["unit"]))
    roof = dict(h["roofline"])
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
                               "(per-layer verify, then one commit over all layers, per cycle)"
                               % L_POOL,
                   "rows": 8, "active_rows": 6, "T": 2, "value_heads": 32, "qk_heads": 16,
                   "d_k": 128, "d_v": 128, "layers": L_POOL, "inputs": "bf16",
                   "state": "fp32", "keep": "U{0,1,2} per cycle",
                   "value_counts": "all 8 rows incl. the 2 inactive ones (see active_rows_heads_per_s)"},
        "roofline": roof,
        "active_rows_heads_per_s": h["active_rows_heads_per_s"],
        "cycle_gbs": h["cycle_gbs"],
        "algorithmic_min_bytes_per_cycle": h["algorithmic_min_bytes_per_cycle"],
        "algorithmic_min_gbs": h["algorithmic_min_gbs"],
        "cpu_baseline": cpu,
        "headline_detail": h,
        "extra": extra,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
