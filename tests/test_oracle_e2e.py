"""Tiny end-to-end chain on the oracle alone (P = 2, S = 256, H = 8, D = 64):
relayout round trip of Q, K, V; each logical rank attends every query over its
half of the keys; max/sum-aware pack over heads; combine over the emulated
exchange; head->seq of the combined output; compared with brute-force full
attention within the stated tolerances."""

import numpy as np

import synth

P, S, H, D = 2, 256, 8, 64


def row_rel_err(got, ref):
    """Per row: max |g - o| / max |o| (rows where the reference is all zero
    must match exactly); returns the largest over rows."""
    num = np.max(np.abs(got - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    assert np.all(num[den == 0] == 0)
    return float(np.max(num[den > 0] / den[den > 0]))


def test_tiny_chain_matches_full_attention(orc):
    g = [synth.bits(synth.normal((S, H, D), seed=synth.BASE_SEED + i)) for i in range(3)]
    X = np.stack(g)  # [3][S][H][D]
    seq_side = np.ascontiguousarray(X.reshape(3, P, S // P, H, D).transpose(1, 0, 2, 3, 4))
    hs = orc.seq_to_head(seq_side, P, 3, S, H, D)
    assert np.array_equal(orc.head_to_seq(hs, P, 3, S, H, D), seq_side)
    q, k, v = g
    outs, ms, ss = [], [], []
    for p in range(P):
        o, m, s = orc.attention(q, k, v, p * S // P, (p + 1) * S // P)
        outs.append(orc.round_half(o))
        ms.append(m.astype(np.float32))
        ss.append(s.astype(np.float32))
    ob = np.stack(outs)  # [P][T][H][D] bf16 bits
    packed = orc.lse_pack(ob, np.stack(ms), np.stack(ss), scatter_dim=1)
    comb, lse = orc.lse_combine_packed(packed, P, S, H, D, scatter_dim=1)
    # combined output is head-sharded [P][S][H/P][D]: bring it back to [S][H][D]
    back = orc.head_to_seq(comb.reshape(P, 1, S, H // P, D), P, 1, S, H, D).reshape(S, H, D)
    full_o, full_m, full_s = orc.attention(q, k, v, 0, S)
    got = orc.half_bits_to_double(back)
    assert row_rel_err(got.reshape(-1, D), full_o.reshape(-1, D)) <= 8e-3
    lse_global = lse.reshape(P, S, H // P).transpose(1, 0, 2).reshape(S, H)
    assert np.max(np.abs(lse_global - (full_m + np.log(full_s)))) <= 1e-5
