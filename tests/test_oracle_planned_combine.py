"""Pins of the oracle's causal combine over a THD layout plan.

- With the per-sequence split written as a plan, the first positions are the
  piece starts and the planned combine equals the pinned varlen combine bit
  for bit.
- The planned validity rule equals brute force (rank p holds a key of the
  token's sequence at or before it), and the combine of brute-force
  per-rank causal attention partials equals full causal attention.
- The typed planned combine and its gradient equal the rounded double forms
  row by row under that rule."""

import numpy as np
import pytest

import synth


def _split_plan(orc, cu, P):
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


def _owner(plan, t):
    s = int(np.searchsorted(plan["span_start"], t, side="right")) - 1
    return int(plan["span_rank"][s])


def test_sequence_split_plan_reduces_to_piece_rule(orc):
    P = 4
    cu = synth.cu_seqlens([5, 0, 17, 3, 40, 1, 2])
    plan = _split_plan(orc, cu, P)
    first = orc.plan_first_positions(cu, plan, P)
    for i in range(cu.size - 1):
        L = int(cu[i + 1] - cu[i])
        for p in range(P):
            a, e = p * L // P, (p + 1) * L // P
            assert first[p, i] == (a if a < e else np.iinfo(np.int32).max)
    assert np.array_equal(orc.plan_mask(cu, first, P), orc.causal_mask(cu, P))
    T, H, D = int(cu[-1]), 3, 16
    po = synth.bits(synth.normal((P, T, H, D), seed=1))
    pl = synth.partial_lse((P, T, H), seed=2).numpy()
    a = orc.lse_combine_planned(po, pl, cu, first)
    b = orc.lse_combine(po, pl, cu=cu)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("lengths,W,b,min_split", [([5, 9, 3], 3, 1, 4), ([12, 2, 7, 1], 2, 1, 6),
                                                   ([8, 8, 16], 4, 2, 8)])
def test_rule_and_combine_against_brute_force_attention(orc, lengths, W, b, min_split):
    cu = synth.cu_seqlens(lengths)
    T = int(cu[-1])
    plan = orc.thd_plan(cu, W, block_size=b, min_split_tokens=min_split)
    first = orc.plan_first_positions(cu, plan, W)
    mask = orc.plan_mask(cu, first, W)
    owner = np.array([_owner(plan, t) for t in range(T)])
    rng = np.random.default_rng(len(lengths) * 10 + W)
    D = 8
    q, k, v = (rng.normal(size=(T, D)) for _ in range(3))
    for i in range(cu.size - 1):
        c0, c1 = int(cu[i]), int(cu[i + 1])
        for t in range(c0, c1):
            keys = np.arange(c0, t + 1)
            s = q[t] @ k[keys].T / np.sqrt(D)
            full = np.exp(s - s.max()) @ v[keys] / np.exp(s - s.max()).sum()
            parts_o = np.zeros((W, 1, D))
            parts_l = np.full((W, 1), -np.inf)
            for p in range(W):
                mine = keys[owner[keys] == p]
                assert mask[p, t] == (mine.size > 0), (p, t)
                if mine.size:
                    sp = q[t] @ k[mine].T / np.sqrt(D)
                    m = sp.max()
                    parts_o[p, 0] = np.exp(sp - m) @ v[mine] / np.exp(sp - m).sum()
                    parts_l[p, 0] = m + np.log(np.exp(sp - m).sum())
            out, _ = orc.combine_f64(parts_o, parts_l)
            assert np.allclose(out[0], full, rtol=0, atol=1e-12)


def test_typed_planned_combine_and_gradient_rowwise(orc):
    W, H, D = 3, 2, 16
    cu = synth.cu_seqlens([6, 1, 11, 4])
    T = int(cu[-1])
    plan = orc.thd_plan(cu, W, block_size=1, min_split_tokens=5)
    first = orc.plan_first_positions(cu, plan, W)
    po = synth.bits(synth.normal((W, T, H, D), seed=3))
    pl = synth.partial_lse((W, T, H), seed=4).numpy()
    go = synth.bits(synth.normal((T, H, D), seed=5))
    gl = synth.normal((T, H), seed=6, dtype="fp32").numpy()
    out, lse = orc.lse_combine_planned(po, pl, cu, first)
    d_po, d_pl = orc.lse_combine_planned_backward(po, pl, go, gl, cu, first)
    dec = orc.half_bits_to_double
    for t in range(T):
        valid = np.array([orc.plan_piece_valid(cu, first, p, t) for p in range(W)], dtype=np.int32)
        for h in range(H):
            o = np.stack([dec(po[p, t, h]) for p in range(W)])
            l = np.where(valid == 1, pl[:, t, h].astype(np.float64), -np.inf)
            ro, rl = orc.combine_f64(o[:, None, :], l[:, None])
            assert np.array_equal(out[t, h], orc.double_to_bf16_bits(ro[0]))
            assert lse[t, h] == np.float32(rl[0])
            g_o, g_l = orc.combine_row_backward_f64(o, l, dec(go[t, h]), float(gl[t, h]), valid)
            assert np.array_equal(d_po[:, t, h], orc.double_to_bf16_bits(g_o))
            assert np.array_equal(d_pl[:, t, h], g_l.astype(np.float32))
