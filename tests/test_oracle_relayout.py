"""Pins of the oracle's Ulysses relayouts (dense and cu_seqlens varlen).

Dense: the global-tensor closed form (numpy reshape/transpose), a hand-written
golden case, the round trip, exactly-once coverage with an index payload, and
pure-Python brute force on tiny shapes.  Varlen: reduction to dense for one
sequence, the plan by brute-force counting, round trip and coverage."""

import json
from pathlib import Path

import numpy as np
import pytest

import synth

GOLDEN = Path(__file__).resolve().parent / "golden"

DENSE_SHAPES = [  # (P, B, S, H, D)
    (1, 1, 4, 3, 5),
    (2, 1, 4, 2, 1),
    (2, 3, 8, 4, 8),
    (3, 2, 9, 6, 4),
    (4, 3, 12, 8, 16),
    (4, 1, 8, 4, 2),
    (8, 2, 16, 8, 3),
]


def _closed_form_s2h(X, P):
    """X: global [B][S][H][D].  Rank j's sequence slab is X[:, jS/P:(j+1)S/P];
    rank r's head slab is X[:, :, rH/P:(r+1)H/P]."""
    B, S, H, D = X.shape
    seq_side = X.reshape(B, P, S // P, H, D).transpose(1, 0, 2, 3, 4)
    head_side = X.reshape(B, S, P, H // P, D).transpose(2, 0, 1, 3, 4)
    return np.ascontiguousarray(seq_side), np.ascontiguousarray(head_side)


@pytest.mark.parametrize("shape", DENSE_SHAPES)
def test_dense_matches_global_closed_form(orc, shape):
    P, B, S, H, D = shape
    X = synth.bits(synth.normal((B, S, H, D), seed=1000 + P * 7 + S))
    seq_side, head_side = _closed_form_s2h(X, P)
    assert np.array_equal(orc.seq_to_head(seq_side, P, B, S, H, D), head_side)
    assert np.array_equal(orc.head_to_seq(head_side, P, B, S, H, D), seq_side)


def test_dense_golden_hand_case(orc):
    g = json.loads((GOLDEN / "relayout_p2_s4_h2_d1.json").read_text())
    s = g["shape"]
    x = np.array(g["seq_side"], dtype=np.uint32)
    y = orc.seq_to_head(x, s["P"], s["B"], s["S"], s["H"], s["D"])
    assert y.reshape(-1).tolist() == g["head_side"]
    back = orc.head_to_seq(np.array(g["head_side"], dtype=np.uint32), s["P"], s["B"], s["S"], s["H"], s["D"])
    assert back.reshape(-1).tolist() == g["seq_side"]


@pytest.mark.parametrize("shape", DENSE_SHAPES)
def test_dense_round_trip_and_exactly_once(orc, shape):
    P, B, S, H, D = shape
    n = B * S * H * D
    x = synth.iota32(n)
    y = orc.seq_to_head(x, P, B, S, H, D)
    # every source index appears exactly once
    assert np.array_equal(np.sort(y.reshape(-1)), x)
    assert np.array_equal(orc.head_to_seq(y, P, B, S, H, D).reshape(-1), x)
    z = orc.head_to_seq(x, P, B, S, H, D)
    assert np.array_equal(np.sort(z.reshape(-1)), x)
    assert np.array_equal(orc.seq_to_head(z, P, B, S, H, D).reshape(-1), x)


@pytest.mark.parametrize("shape", [(2, 1, 4, 2, 2), (3, 2, 6, 3, 1), (2, 2, 6, 4, 3)])
def test_dense_brute_force(orc, shape):
    P, B, S, H, D = shape
    Sp, Hp = S // P, H // P
    x = synth.iota32(B * S * H * D).reshape(P, B, Sp, H, D)
    y = orc.seq_to_head(x, P, B, S, H, D)
    for r in range(P):
        for b in range(B):
            for t in range(S):
                for h in range(Hp):
                    for d in range(D):
                        # token t of the global sequence lives on rank t // Sp
                        assert y[r, b, t, h, d] == x[t // Sp, b, t % Sp, r * Hp + h, d]


# --------------------------- varlen -----------------------------------------

def _brute_plan(lengths, P):
    """Pieces by direct enumeration: piece p of a length-L sequence is
    positions k with floor(p*L/P) <= k < floor((p+1)*L/P)."""
    pieces = []  # per sequence, per rank: list of positions
    for L in lengths:
        pieces.append([[k for k in range(L) if (p * L) // P <= k < ((p + 1) * L) // P] for p in range(P)])
    T_p = [sum(len(pieces[i][p]) for i in range(len(lengths))) for p in range(P)]
    return pieces, T_p


VARLEN_CASES = [  # (lengths, P, B, H, D)
    ([7], 2, 1, 4, 2),
    ([5, 0, 9, 1, 3], 3, 2, 3, 2),
    ([1, 2, 3], 4, 1, 4, 1),
    ([17, 33, 2, 64], 4, 3, 8, 4),
    ([40, 3, 0, 0, 12, 7], 8, 1, 8, 2),
]


@pytest.mark.parametrize("case", VARLEN_CASES)
def test_varlen_plan_by_counting(orc, case):
    lengths, P, *_ = case
    cu = synth.cu_seqlens(lengths)
    rank_cu, rank_off = orc.varlen_plan(cu, P)
    pieces, T_p = _brute_plan(lengths, P)
    assert sum(T_p) == cu[-1]
    assert rank_off.tolist() == [sum(T_p[:p]) for p in range(P + 1)]
    for p in range(P):
        acc = 0
        for i in range(len(lengths)):
            assert rank_cu[p, i] == acc
            acc += len(pieces[i][p])
        assert rank_cu[p, len(lengths)] == T_p[p]


@pytest.mark.parametrize("case", VARLEN_CASES)
def test_varlen_brute_force_and_round_trip(orc, case):
    lengths, P, B, H, D = case
    cu = synth.cu_seqlens(lengths)
    T = int(cu[-1])
    Hp = H // P
    pieces, T_p = _brute_plan(lengths, P)
    x = synth.iota32(B * T * H * D).reshape(B * T, H, D)
    y = orc.varlen_seq_to_head(x, cu, P, B, H, D)
    # brute force: rank p's slab [B][T_p] starts at token row B * sum(T_0..T_{p-1})
    R = 0
    for p in range(P):
        l = 0
        rows = []
        for i, L in enumerate(lengths):
            for k in pieces[i][p]:
                rows.append((l, int(cu[i]) + k))
                l += 1
        for b in range(B):
            for (l, t) in rows:
                src_row = B * R + b * T_p[p] + l
                for r in range(P):
                    assert np.array_equal(y[r, b, t], x[src_row, r * Hp:(r + 1) * Hp])
        R += T_p[p]
    assert np.array_equal(np.sort(y.reshape(-1)), x.reshape(-1))
    back = orc.varlen_head_to_seq(y, cu, P, B, H, D)
    assert np.array_equal(back, x)


@pytest.mark.parametrize("P,B,T,H,D", [(2, 3, 8, 4, 8), (4, 1, 12, 8, 3), (3, 2, 9, 6, 2)])
def test_varlen_single_sequence_is_dense(orc, P, B, T, H, D):
    cu = np.array([0, T], dtype=np.int32)
    x = synth.bits(synth.normal((P, B, T // P, H, D), seed=55))
    dense = orc.seq_to_head(x, P, B, T, H, D)
    var = orc.varlen_seq_to_head(x.reshape(B * T, H, D), cu, P, B, H, D)
    assert np.array_equal(dense, var)
    back_dense = orc.head_to_seq(dense, P, B, T, H, D)
    back_var = orc.varlen_head_to_seq(dense, cu, P, B, H, D)
    assert np.array_equal(back_dense.reshape(-1), back_var.reshape(-1))


def test_owner_closed_form_equals_linear_search():
    # The owner of position k in a length-L sequence, floor(((k+1)P - 1)/L),
    # is the rank whose piece [floor(pL/P), floor((p+1)L/P)) contains k.
    for P in (1, 2, 3, 4, 7, 8, 16):
        for L in range(1, 70):
            for k in range(L):
                lin = [p for p in range(P) if (p * L) // P <= k < ((p + 1) * L) // P]
                assert lin == [((k + 1) * P - 1) // L]
