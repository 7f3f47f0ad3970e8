"""The bench's roofline denominators, checked on the CPU against hand counts:
the algorithmic bytes of a verify launch, of a fused commit + verify cycle and
of a rewind, the prefill's algorithmic flops, and the rule that a counted
traffic record is used only while its kernel sources are unchanged."""
import hashlib
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from gated_deltanet_recurrence_conv_amd import workloads as W  # noqa: E402


def test_verify_bytes_of_the_thirty_layer_cohort():
    # per active (layer, row): the 2 MiB state read once and written as two
    # candidates, 2 window rows + 3 cache rows of 8,192 bf16 channels, g and
    # beta of 2 tokens x 32 heads, and 2 x 32 x 128 fp32 outputs
    state = 32 * 128 * 128 * 4
    per_row = 3 * state + 5 * 8192 * 2 + 2 * 2 * 32 * 2 + 2 * 32 * 128 * 4
    assert per_row == 6_406_400
    per_layer = 6 * per_row + 8192 * 4 * 2           # six active rows, conv weights
    assert bench.verify_bytes(W.COHORT, 6, 1) == per_layer == 38_503_936
    assert bench.verify_bytes(W.COHORT, 6, 30) == 1_155_118_080


def small_shape(T):
    # C = 2 * 1 * 16 + 2 * 16 = 64 channels, a 2 KiB state per row
    return W.Shape("acct", L=1, B=4, T=T, HV=2, HK=1, DK=16, DV=16, S=3, act="bf16")


def test_lazy_bytes_by_hand():
    sh = small_shape(2)
    # row 0: verifies only; row 1: replays 1 token and verifies; row 2: inactive,
    # replays 2 tokens; row 3: inactive, nothing to replay
    keep_prev, active = [0, 1, 2, 0], [1, 1, 0, 0]
    state, cache, tok, out = 2048, 3 * 64 * 2, 64 * 2 + 2 * 2 * 2, 2 * 2 * 16 * 4
    row0 = state + cache + 2 * tok + out
    row1 = state + cache + 1 * tok + (state + cache) + 2 * tok + out
    row2 = state + cache + 2 * tok + (state + cache)
    assert (row0, row1, row2) == (2960, 5528, 5136)
    weights = 64 * 4 * 2
    assert bench.lazy_bytes(sh, keep_prev, active, 3) == 3 * (row0 + row1 + row2 + weights) == 42_408


def test_rewind_bytes_by_hand():
    sh = small_shape(4)
    # per committing row: state read and written, keep tokens (x row, g, beta),
    # 3 cache rows read and 3 written; per layer the weights
    r1 = 2 * 2048 + 1 * (64 * 2 + 2 * 2 * 2) + 6 * 64 * 2
    r3 = 2 * 2048 + 3 * (64 * 2 + 2 * 2 * 2) + 6 * 64 * 2
    assert (r1, r3) == (5000, 5272)
    assert bench.rewind_bytes(sh, [0, 1, 3, 0], 2) == 2 * (r1 + r3 + 512) == 21_568


def test_prefill_flops_of_a_1024_token_call():
    # 6 d^2 + 5 C d + C^2 / 3 per token-head at d = 128, chunk C = 64
    per = 6 * 128 * 128 + 5 * 64 * 128 + 64 * 64 / 3
    assert bench.prefill_flops(1024, 32, 128) == pytest.approx(per * 1024 * 32)
    assert bench.prefill_flops(1024, 32, 128) == pytest.approx(4.608142e9, rel=1e-6)


def test_traffic_record_only_for_unchanged_sources(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("kernel source\n")
    sha = hashlib.sha256(src.read_bytes()).hexdigest()[:16]
    (tmp_path / "profiles").mkdir()
    rec = {"k": {"sources": ["k.hip"], "sha256_16": sha, "traffic_bytes_per_launch": 1234}}
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.counted_traffic("k") == 1234
    assert bench.counted_traffic("missing") is None
    src.write_text("kernel source, changed\n")
    assert bench.counted_traffic("k") is None


def test_every_traffic_record_names_existing_sources_and_a_profile():
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        recs = json.load(f)
    for key, r in recs.items():
        for s in r["sources"]:
            assert os.path.exists(os.path.join(ROOT, s)), (key, s)
        assert os.path.exists(os.path.join(ROOT, r["profile"])), (key, r["profile"])
        assert r["traffic_bytes_per_launch"] > 0
