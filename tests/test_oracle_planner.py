"""Pins of the oracle's THD layout planner and planned-span relayout.

Planner: the input rules the page lists; the hand-worked plan in
tests/golden/thd_plan_small.json; on random packed batches (non-power-of-two
rank counts included) the invariants the page states -- every token placed
once, block-aligned spans, every rank holding its balanced share of blocks,
short samples on one rank when they fit, at most max_chunks_per_rank spans
per rank (unless the contiguous layout wins), the same output for the same
input -- with rank costs
recomputed exactly from the spans, and never worse than the contiguous
layout (computed here from the balanced-shard closed form); brute force over
every capacity-respecting block assignment bounds the plan on tiny batches.

Span relayout: with the spans of the per-sequence split it equals the pinned
varlen relayout bit for bit; round trip and exactly-once coverage; per-element
brute force on a tiny case."""

import itertools
import json
from pathlib import Path

import numpy as np
import pytest

import synth

GOLDEN = Path(__file__).resolve().parent / "golden"


def _exact_costs(plan, cu, wt=1.0, wc=1.0):
    """Per rank (tokens, causal work) from the spans, in Python integers."""
    W = plan["rank_off"].size - 1
    tok = [0] * W
    caus = [0] * W
    ss, sr = plan["span_start"], plan["span_rank"]
    for s in range(sr.size):
        a, e = int(ss[s]), int(ss[s + 1])
        i = int(np.searchsorted(cu, a, side="right")) - 1
        k0, k1 = a - int(cu[i]), e - int(cu[i])
        tok[int(sr[s])] += e - a
        caus[int(sr[s])] += sum(range(k0 + 1, k1 + 1))
    return tok, caus


def _contiguous_max(cu, W, b, wt=1.0, wc=1.0):
    T = int(cu[-1])
    N = T // b
    worst = 0.0
    for r in range(W):
        lo, hi = (r * N // W) * b, ((r + 1) * N // W) * b
        c = 0
        for t in range(lo, hi):
            i = int(np.searchsorted(cu, t, side="right")) - 1
            c += t - int(cu[i]) + 1
        worst = max(worst, wt * (hi - lo) + wc * c)
    return worst


def _check_invariants(plan, cu, W, b, min_split, max_chunks):
    T = int(cu[-1])
    N = T // b
    ss, sr, sl, ro = plan["span_start"], plan["span_rank"], plan["span_local"], plan["rank_off"]
    assert ss[0] == 0 and ss[-1] == T and np.all(np.diff(ss) > 0)
    assert np.all(ss % b == 0), "spans must be block-aligned"
    cap = np.array([((r + 1) * N // W - r * N // W) * b for r in range(W)])
    assert np.array_equal(np.diff(ro), cap) and ro[0] == 0, "rank capacities must be the exact balanced split"
    for s in range(sr.size):  # a span never crosses a sequence boundary
        i = int(np.searchsorted(cu, ss[s], side="right")) - 1
        assert ss[s + 1] <= cu[i + 1]
    fill = np.zeros(W, dtype=np.int64)
    for s in range(sr.size):  # slabs list their spans in packed order, back to back
        r = int(sr[s])
        assert sl[s] == fill[r]
        fill[r] += ss[s + 1] - ss[s]
    assert np.array_equal(fill, cap)
    tok, caus = _exact_costs(plan, cu)
    assert np.array_equal(np.array(tok), cap)
    for r in range(W):
        assert plan["rank_cost"][r] == float(tok[r]) * 1.0 + float(caus[r]) * 1.0
    if plan["grid"] > 0:
        assert np.all(np.bincount(sr, minlength=W) <= max_chunks)
    assert plan["rank_cost"].max() <= _contiguous_max(cu, W, b) + 1e-9


GOLDEN_PLANS = sorted(p.name for p in GOLDEN.glob("thd_plan_*.json"))


def _golden_plan(orc_mod, name):
    g = json.loads((GOLDEN / name).read_text())
    i = g["input"]
    cu = synth.cu_seqlens(i["lengths"])
    return g["expected"], orc_mod.thd_plan(cu, i["world_size"], i["block_size"], i["min_split_tokens"],
                                           i["max_chunks_per_rank"], i["token_weight"], i["causal_weight"])


def _matches(e, p):
    return (p["grid"] == e["grid"] and all(p[k].tolist() == e[k] for k in
                                           ("span_start", "span_rank", "span_local", "rank_off"))
            and p["rank_cost"].tolist() == e["rank_cost"])


@pytest.mark.parametrize("name", GOLDEN_PLANS)
def test_golden_hand_plan(orc, name):
    e, p = _golden_plan(orc, name)
    assert p["grid"] == e["grid"]
    for k in ("span_start", "span_rank", "span_local", "rank_off"):
        assert p[k].tolist() == e[k], k
    assert p["rank_cost"].tolist() == e["rank_cost"]


# Planted mistakes (in a copy of the oracle built here, never in the product):
# each hand-worked plan must catch the rebalancing step it reaches taking the
# other choice.
MUTANTS = {
    # C1 takes the top blocks where the bottom ones are cheaper and vice versa
    "c1_flipped": ("            if (ml < mh) {", "            if (!(ml < mh)) {"),
    # C2 lays a short's pieces into the lowest rank with room, not the cheapest
    "c2_lowest_rank": ("                int64_t u = cheapest_with_room(&L, 1);\n                int64_t k = capb[u] - blk[u];",
                       "                int64_t u = 0;\n                while (capb[u] - blk[u] < 1)\n                    ++u;\n"
                       "                int64_t k = capb[u] - blk[u];"),
}
CAUGHT_BY = {"c1_flipped": ["thd_plan_c1_bottom.json", "thd_plan_c1_top.json"],
             "c2_lowest_rank": ["thd_plan_c2_split_short.json"]}


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_golden_plans_catch_planted_rebalancing_mistakes(orc, tmp_path, mutant):
    from oracle_mutant import build_oracle_mutant

    old, new = MUTANTS[mutant]
    mod = build_oracle_mutant(orc, tmp_path, old, new, mutant)
    for name in GOLDEN_PLANS:
        e, p = _golden_plan(mod, name)
        if name in CAUGHT_BY[mutant]:
            assert not _matches(e, p), f"{name} does not catch {mutant}"


@pytest.mark.parametrize("kw,W,kind", [
    (dict(min_split_tokens=6, block_size=4), 4, "config"),     # min_split not block-aligned
    (dict(max_chunks_per_rank=0), 4, "config"),
    (dict(block_size=0), 4, "config"),
    (dict(min_split_tokens=0), 4, "config"),
    (dict(token_weight=float("nan")), 4, "config"),
    (dict(causal_weight=-1.0), 4, "config"),
    (dict(token_weight=0.0, causal_weight=0.0), 4, "config"),
    (dict(), 0, "config"),
])
def test_rejects_invalid_config(orc, kw, W, kind):
    args = dict(block_size=64, min_split_tokens=128)
    args.update(kw)
    with pytest.raises(ValueError, match=kind):
        orc.thd_plan(synth.cu_seqlens([1 << 12]), W, **args)


def test_rejects_misaligned_lengths_and_too_few_blocks(orc):
    with pytest.raises(ValueError, match="lengths"):
        orc.thd_plan(synth.cu_seqlens([128, 100]), 2, block_size=64, min_split_tokens=128)
    with pytest.raises(ValueError, match="blocks"):
        orc.thd_plan(synth.cu_seqlens([64, 64, 64]), 4, block_size=64, min_split_tokens=128)


def _random_batch(seed, b):
    rng = np.random.default_rng(seed)
    n_short = int(rng.integers(0, 12))
    shorts = list(rng.integers(0, 20, size=n_short))
    longs = list(rng.integers(20, 300, size=int(rng.integers(0, 4))))
    lens = shorts + longs
    rng.shuffle(lens)
    if not lens or sum(lens) == 0:
        lens = [40]
    return synth.cu_seqlens([int(x) * b for x in lens])


@pytest.mark.parametrize("seed", range(40))
def test_invariants_random_batches(orc, seed):
    b = [1, 4, 16][seed % 3]
    cu = _random_batch(seed, b)
    N = int(cu[-1]) // b
    for W in (1, 2, 3, 5, 8):
        if N < W:
            continue
        p = orc.thd_plan(cu, W, block_size=b, min_split_tokens=16 * b, max_chunks_per_rank=12)
        _check_invariants(p, cu, W, b, 16 * b, 12)
        q = orc.thd_plan(cu, W, block_size=b, min_split_tokens=16 * b, max_chunks_per_rank=12)
        for k in p:
            assert np.array_equal(np.asarray(p[k]), np.asarray(q[k])), "the plan must be deterministic"


def test_short_samples_kept_whole(orc):
    """Shorts that fit beside the long sequences stay in one span each."""
    b = 16
    lens = [40 * b, 3 * b, 200 * b, 5 * b, 2 * b, 1 * b, 7 * b, 150 * b]
    cu = synth.cu_seqlens(lens)
    for W in (2, 3, 4, 6):
        p = orc.thd_plan(cu, W, block_size=b, min_split_tokens=32 * b)
        if p["grid"] == 0:
            continue
        for i, L in enumerate(lens):
            if L < 32 * b:
                inside = (p["span_start"][:-1] >= cu[i]) & (p["span_start"][:-1] < cu[i + 1])
                assert inside.sum() == 1, (W, i)


def test_long_sequence_snake_direction(orc):
    """One long sequence alone, 2W equal chunks (grid 2 chosen or not, the
    chunk -> rank map of every candidate follows the alternating snake):
    with causal weight only, the snake pairs early and late chunks, so every
    rank's cost is equal and the planner picks it over the contiguous cut."""
    W, b = 4, 1
    cu = synth.cu_seqlens([8 * W])
    p = orc.thd_plan(cu, W, block_size=b, min_split_tokens=2, token_weight=0.0, causal_weight=1.0)
    assert p["grid"] >= 2
    # chunk c of 2W chunks of W blocks... the chosen grid's first 2W chunk owners
    owners = [int(p["span_rank"][np.searchsorted(p["span_start"], t, side="right") - 1]) for t in range(0, 8 * W)]
    rounds = [owners[c * (8 * W) // (2 * W)] for c in range(2 * W)] if p["grid"] == 2 else None
    if rounds is not None:
        assert rounds == [0, 1, 2, 3, 3, 2, 1, 0]
    costs = p["rank_cost"]
    assert costs.max() < _contiguous_max(cu, W, b, wt=0.0, wc=1.0)


def test_brute_force_bound_tiny(orc):
    """The plan is a valid exact-capacity assignment, so its maximum rank cost
    is at least the optimum over all block assignments, found by brute force."""
    for lens, W in (([3, 1, 2], 2), ([4, 2], 3), ([2, 2, 1, 1], 2), ([5, 1], 2)):
        cu = synth.cu_seqlens(lens)
        N = sum(lens)
        blocks = [(i, k) for i, L in enumerate(lens) for k in range(L)]
        cap = [(r + 1) * N // W - r * N // W for r in range(W)]
        best = None
        for assign in itertools.product(range(W), repeat=N):
            if [assign.count(r) for r in range(W)] != cap:
                continue
            cost = [0.0] * W
            for (i, k), r in zip(blocks, assign):
                cost[r] += 1.0 + (k + 1)
            m = max(cost)
            best = m if best is None else min(best, m)
        p = orc.thd_plan(cu, W, block_size=1, min_split_tokens=3)
        assert p["rank_cost"].max() >= best - 1e-12
        assert p["rank_cost"].max() <= _contiguous_max(cu, W, 1)


# -- planned-span relayout -------------------------------------------------------

def _spans_of_sequence_split(orc, cu, P):
    """The per-sequence P-way split as a span table (piece p of each sequence
    on rank p, local rows from the varlen plan)."""
    rank_cu, rank_off = orc.varlen_plan(cu, P)
    starts, ranks, local = [], [], []
    for i in range(cu.size - 1):
        L = int(cu[i + 1] - cu[i])
        for p in range(P):
            a, e = p * L // P, (p + 1) * L // P
            if a < e:
                starts.append(int(cu[i]) + a)
                ranks.append(p)
                local.append(int(rank_cu[p][i]))
    order = np.argsort(starts, kind="stable")
    return {"span_start": np.array([starts[k] for k in order] + [int(cu[-1])], dtype=np.int32),
            "span_rank": np.array([ranks[k] for k in order], dtype=np.int32),
            "span_local": np.array([local[k] for k in order], dtype=np.int32),
            "rank_off": np.ascontiguousarray(rank_off, dtype=np.int64)}


@pytest.mark.parametrize("P,B", [(2, 1), (4, 3), (8, 2)])
def test_span_relayout_equals_sequence_split_relayout(orc, P, B):
    H, D = 8, 4
    cu = synth.cu_seqlens([5, 0, 17, 3, 40, 1])
    T = int(cu[-1])
    plan = _spans_of_sequence_split(orc, cu, P)
    x = synth.iota32(B * T * H * D)
    assert np.array_equal(orc.span_seq_to_head(x, plan, P, B, H, D), orc.varlen_seq_to_head(x, cu, P, B, H, D))
    y = synth.iota32(B * T * H * D)
    assert np.array_equal(orc.span_head_to_seq(y, plan, P, B, H, D), orc.varlen_head_to_seq(y, cu, P, B, H, D))


@pytest.mark.parametrize("W,B", [(3, 1), (4, 2), (8, 3)])
def test_span_relayout_round_trip_and_coverage(orc, W, B):
    b, H, D = 4, W * 2, 3
    cu = synth.cu_seqlens([4 * x for x in (3, 60, 1, 7, 90, 2)])
    plan = orc.thd_plan(cu, W, block_size=b, min_split_tokens=32)
    T = int(cu[-1])
    x = synth.iota32(B * T * H * D)
    y = orc.span_seq_to_head(x, plan, W, B, H, D)
    assert np.array_equal(np.sort(y.reshape(-1)), x)
    assert np.array_equal(orc.span_head_to_seq(y, plan, W, B, H, D).reshape(-1), x)


def test_span_relayout_brute_force(orc):
    W, B, H, D, b = 3, 2, 6, 2, 1
    cu = synth.cu_seqlens([2, 9, 1, 4])
    plan = orc.thd_plan(cu, W, block_size=b, min_split_tokens=4)
    T = int(cu[-1])
    Hp = H // W
    x = synth.iota32(B * T * H * D).reshape(B * T, H, D)
    y = orc.span_seq_to_head(x, plan, W, B, H, D)
    ss, sr, sl, ro = plan["span_start"], plan["span_rank"], plan["span_local"], plan["rank_off"]
    for t in range(T):
        s = int(np.searchsorted(ss, t, side="right")) - 1
        p = int(sr[s])
        l = int(sl[s]) + t - int(ss[s])
        Tp = int(ro[p + 1] - ro[p])
        for bb in range(B):
            row = B * int(ro[p]) + bb * Tp + l
            for r in range(W):
                assert np.array_equal(y[r, bb, t], x[row, r * Hp:(r + 1) * Hp])


def _trace_batch(seed):
    """Random packed batches shaped to reach the rebalancing steps.  Seeds
    below 12: one to three long sequences and small shorts, so that the snake
    overfills ranks (C1).  Seeds from 12: mostly shorts near a rank's share,
    so that some fit nowhere whole (C2)."""
    rng = np.random.default_rng(7000 + seed)
    W = int(rng.integers(2, 9))
    b = int(rng.choice([1, 2, 4]))
    min_split = 16 * b
    if seed < 12:
        longs = [int(x) for x in rng.integers(16, 80, size=int(rng.integers(1, 4)))]
        share = max(2, (sum(longs) + 12 * W) // W)
        shorts = [int(x) for x in rng.integers(1, min(16, share + 2), size=int(rng.integers(W, 3 * W + 1)))]
    else:
        longs = [int(rng.integers(16, 60))] if rng.integers(0, 2) else []
        shorts = [int(x) for x in rng.integers(4, 16, size=int(rng.integers(W + 1, 2 * W + 3)))]
    lens = longs + shorts
    rng.shuffle(lens)
    return synth.cu_seqlens([x * b for x in lens]), W, b, min_split


def _range_cost(a, e, b, wt, wc):
    """Cost of blocks [a, e) of a sequence in exact integers: wt per token plus
    wc * (k + 1) for each token position k."""
    return wt * (e - a) * b + wc * sum(range(a * b + 1, e * b + 1))


@pytest.mark.parametrize("seed", range(24))
def test_rebalancing_decisions_recomputed_in_integers(orc, seed):
    """Every C1 move and C2 piece of every grid candidate, recomputed from the
    recorded loads in Python integers: C1 takes the overfull rank with the
    lowest index, sends min(its excess, the room of the cheapest rank with
    room) blocks to that rank, and of the two candidate moves (the top of the
    highest long span, the bottom of the lowest) takes the one whose larger
    cost of the pair is smaller (ties: the top); C2 lays a short's next piece
    into the cheapest rank with room (ties: the lowest), as far as its room
    allows; each record's loads are the previous record's after its move."""
    cu, W, b, min_split = _trace_batch(seed)
    lens = np.diff(cu) // b
    N = int(lens.sum())
    cap = [(r + 1) * N // W - r * N // W for r in range(W)]
    n_c1 = n_c1_distinct = n_c2 = 0
    for wt, wc in ((1, 1), (3, 1), (1, 4), (0, 1), (2, 0)):
        for g in range(1, 7):
            _, recs = orc.thd_plan_candidate_trace(cu, W, g, b, min_split, float(wt), float(wc))
            prev = None
            for t in recs:
                blk, caus = list(t["blk"]), list(t["caus"])
                if prev is not None:
                    assert (blk, caus) == prev, "a record's loads must follow from the previous move"
                cost = [wt * blk[r] * b + wc * caus[r] for r in range(W)]
                room = [cap[r] - blk[r] for r in range(W)]
                with_room = [r for r in range(W) if room[r] >= 1]
                to = min(with_room, key=lambda r: (cost[r], r))
                assert t["to"] == to
                a, e = t["moved_a"], t["moved_e"]
                moved_caus = sum(range(a * b + 1, e * b + 1))
                if t["step"] == 1:
                    over = [r for r in range(W) if blk[r] > cap[r]][0]
                    assert t["over"] == over
                    amount = min(blk[over] - cap[over], room[to])
                    assert t["amount"] == amount
                    n_top = min(amount, t["top_e"] - t["top_a"])
                    n_bot = min(amount, t["bot_e"] - t["bot_a"])
                    c_top = _range_cost(t["top_e"] - n_top, t["top_e"], b, wt, wc)
                    c_bot = _range_cost(t["bot_a"], t["bot_a"] + n_bot, b, wt, wc)
                    via_top = max(cost[over] - c_top, cost[to] + c_top)
                    via_bot = max(cost[over] - c_bot, cost[to] + c_bot)
                    take_bottom = via_bot < via_top
                    assert bool(t["chose_bottom"]) == take_bottom, (t, via_top, via_bot)
                    if take_bottom:
                        assert (t["moved_seq"], a, e) == (t["bot_seq"], t["bot_a"], t["bot_a"] + n_bot)
                    else:
                        assert (t["moved_seq"], a, e) == (t["top_seq"], t["top_e"] - n_top, t["top_e"])
                    n_c1 += 1
                    n_c1_distinct += via_top != via_bot
                    blk[over] -= e - a
                    caus[over] -= moved_caus
                else:
                    assert t["step"] == 2
                    assert t["amount"] == e - a == min(room[to], int(lens[t["moved_seq"]]) - a)
                    n_c2 += 1
                blk[to] += e - a
                caus[to] += moved_caus
                prev = (blk, caus)
    if seed < 12:
        assert n_c1 > 0 and n_c1_distinct > 0, "the batch must reach C1 with two different candidate costs"
    if seed % 3 == 0:
        print(f"seed {seed}: W={W} b={b}: {n_c1} C1 moves ({n_c1_distinct} with distinct costs), {n_c2} C2 pieces")


def test_rebalancing_traces_reach_c2(orc):
    """Across the traced batches, shorts that fit nowhere whole occur (C2)."""
    total = 0
    for seed in range(12, 24):
        cu, W, b, min_split = _trace_batch(seed)
        for g in range(1, 7):
            _, recs = orc.thd_plan_candidate_trace(cu, W, g, b, min_split)
            total += sum(t["step"] == 2 for t in recs)
    assert total >= 50, total
