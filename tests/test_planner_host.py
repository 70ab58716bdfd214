"""The library's THD layout planner (host code behind the C ABI) against the
oracle's planner: identical span tables, rank costs and chosen candidate on
random packed batches (integer work: bit-exact), the input rules, the
contiguous mode, and the per-rank view.  No GPU is used."""

import numpy as np
import pytest

import synth


@pytest.fixture(scope="module")
def cam():
    import context_attention_movement_amd as m
    m.library()
    return m


def _batch(seed, b):
    rng = np.random.default_rng(1000 + seed)
    n_short = int(rng.integers(0, 30))
    lens = list(rng.integers(0, 24, size=n_short)) + list(rng.integers(24, 900, size=int(rng.integers(0, 5))))
    rng.shuffle(lens)
    if sum(lens) == 0:
        lens = [50]
    return synth.cu_seqlens([int(x) * b for x in lens])


def _same(p, q):
    assert p.grid == q["grid"]
    assert np.array_equal(p.span_start_host, q["span_start"])
    assert np.array_equal(p.span_rank_host, q["span_rank"])
    assert np.array_equal(p.span_local_host, q["span_local"])
    assert np.array_equal(p.rank_off_host, q["rank_off"])
    assert np.array_equal(p.rank_cost, q["rank_cost"])


@pytest.mark.parametrize("seed", range(60))
def test_planner_matches_oracle(cam, orc, seed):
    b = [1, 4, 16, 64][seed % 4]
    cu = _batch(seed, b)
    N = int(cu[-1]) // b
    wt, wc = [(1.0, 1.0), (0.0, 1.0), (3.5, 0.25), (1.0, 0.0)][seed % 4]
    for W in (1, 2, 3, 5, 8, 16):
        if N < W:
            continue
        for min_split, max_chunks in ((16 * b, 64), (4 * b, 6), (1 * b, 3)):
            cfg = cam.ThdPlannerConfig(block_size=b, min_split_tokens=min_split, max_chunks_per_rank=max_chunks,
                                       token_weight=wt, causal_weight=wc)
            p = cam.thd_plan(cu, W, cfg)
            q = orc.thd_plan(cu, W, b, min_split, max_chunks, wt, wc)
            _same(p, q)


def test_thd_workload_plan_matches_oracle(cam, orc):
    """The packed THD benchmark batch (20 short + 2 long sequences, 131072
    tokens, lengths rounded to 64-token blocks) over 8 ranks."""
    lens = synth.thd_lengths(20, 131072, seed=synth.BASE_SEED + 4, align=64)
    cu = synth.cu_seqlens(lens)
    p = cam.thd_plan(cu, 8, cam.ThdPlannerConfig(block_size=64, min_split_tokens=8192))
    q = orc.thd_plan(cu, 8, 64, 8192)
    _same(p, q)
    assert p.grid > 0, "the planned layout should beat the contiguous cut on this batch"


def test_contiguous_mode(cam):
    cu = synth.cu_seqlens([64 * x for x in (3, 17, 5, 40, 1)])
    N = int(cu[-1]) // 64
    for W in (1, 2, 3, 7):
        p = cam.thd_plan(cu, W, cam.ThdPlannerConfig(block_size=64, min_split_tokens=64, contiguous=True))
        assert p.grid == 0
        bounds = sorted({64 * (r * N // W) for r in range(W + 1)} | set(int(c) for c in cu))
        assert p.span_start_host.tolist() == [x for x in bounds if x <= int(cu[-1])]
        for s in range(p.n_spans):
            t = int(p.span_start_host[s])
            assert p.span_rank_host[s] == max(r for r in range(W) if 64 * (r * N // W) <= t)


def test_rejections(cam):
    cu = synth.cu_seqlens([1 << 12])
    C = cam.ThdPlannerConfig
    with pytest.raises(cam.CamError, match="multiple of block_size"):
        cam.thd_plan(cu, 4, C(block_size=4, min_split_tokens=6))
    for bad in (C(max_chunks_per_rank=0), C(block_size=0), C(min_split_tokens=0), C(token_weight=float("nan")),
                C(causal_weight=-1.0), C(token_weight=0.0, causal_weight=0.0)):
        with pytest.raises(cam.CamError):
            cam.thd_plan(cu, 4, bad)
    with pytest.raises(cam.CamError):
        cam.thd_plan(cu, 0)
    with pytest.raises(TypeError):
        cam.thd_plan(cu, True)
    with pytest.raises(TypeError):
        cam.thd_plan(cu, 4, C(block_size=True))
    with pytest.raises(cam.CamError, match="not a multiple"):
        cam.thd_plan(synth.cu_seqlens([128, 100]), 2, C(block_size=64, min_split_tokens=128))
    with pytest.raises(cam.CamError, match="aligned blocks for"):
        cam.thd_plan(synth.cu_seqlens([64, 64, 64]), 4, C(block_size=64, min_split_tokens=128))
    plan = cam.thd_plan(cu, 4)
    with pytest.raises(ValueError, match="rank must be in"):
        plan.for_rank(4)


def test_for_rank_lists_slab_order(cam):
    lens = [64 * x for x in (3, 200, 2, 5, 150, 1)]
    cu = synth.cu_seqlens(lens)
    plan = cam.thd_plan(cu, 3, cam.ThdPlannerConfig(block_size=64, min_split_tokens=64 * 16))
    for r in range(3):
        spans = plan.for_rank(r)
        assert sum(n for _, _, n in spans) == plan.tokens_on_rank(r)
        assert all(0 <= a and a + n <= lens[i] for i, a, n in spans)
        keys = [(i, a) for i, a, _ in spans]
        assert keys == sorted(keys)


def test_first_positions_match_oracle(cam, orc):
    for seed in range(10):
        cu = _batch(seed, 4)
        N = int(cu[-1]) // 4
        for W in (1, 3, 8):
            if N < W:
                continue
            q = orc.thd_plan(cu, W, 4, 64)
            plan = cam.ThdPlan(W, int(cu[-1]), cu, q["span_start"], q["span_rank"], q["span_local"], q["rank_off"],
                               q["rank_cost"], q["grid"])
            assert np.array_equal(plan.first_pos_host, orc.plan_first_positions(cu, q, W))


@pytest.mark.parametrize("name", sorted(p.name for p in (__import__("pathlib").Path(__file__).resolve().parent
                                                          / "golden").glob("thd_plan_*.json")))
def test_planner_equals_hand_worked_plans(cam, name):
    """The library's planner gives each hand-worked plan exactly (the plans
    that reach the rebalancing steps included)."""
    import json
    from pathlib import Path
    g = json.loads((Path(__file__).resolve().parent / "golden" / name).read_text())
    i, e = g["input"], g["expected"]
    cfg = cam.ThdPlannerConfig(block_size=i["block_size"], min_split_tokens=i["min_split_tokens"],
                               max_chunks_per_rank=i["max_chunks_per_rank"], token_weight=i["token_weight"],
                               causal_weight=i["causal_weight"])
    p = cam.thd_plan(synth.cu_seqlens(i["lengths"]), i["world_size"], cfg)
    assert p.grid == e["grid"]
    assert p.span_start_host.tolist() == e["span_start"]
    assert p.span_rank_host.tolist() == e["span_rank"]
    assert p.span_local_host.tolist() == e["span_local"]
    assert p.rank_off_host.tolist() == e["rank_off"]
    assert p.rank_cost.tolist() == e["rank_cost"]
