"""Pins of the oracle's Q/K/V projection into the head-sharded layout:
numpy's float64 matrix product of the decoded operands, rounded with the
(pinned) RNE routine and placed by the global-tensor closed form of the
all-to-all; the same product in the sequence-sharded layout followed by the
oracle's pinned seq->head relayout; per-element brute force on a tiny case."""

import numpy as np
import pytest

import synth


@pytest.mark.parametrize("S,K,P,B,H,D,dt", [(24, 64, 2, 3, 4, 8, "bf16"), (17, 32, 4, 1, 8, 16, "bf16"),
                                            (9, 16, 3, 2, 6, 4, "fp16")])
def test_matches_library_product_and_closed_form(orc, S, K, P, B, H, D, dt):
    x = synth.bits(synth.normal((S, K), seed=S + K, dtype=dt))
    w = synth.bits(synth.normal((B * H * D, K), seed=S + K + 1, std=0.1, dtype=dt))
    got = orc.qkv_projection(x, w, P, B, H, D, dt)
    prod = orc.half_bits_to_double(x, dt) @ orc.half_bits_to_double(w, dt).T      # [S][B*H*D]
    rounded = orc.double_to_bf16_bits(prod) if dt == "bf16" else orc.double_to_fp16_bits(prod)
    want = rounded.reshape(S, B, P, H // P, D).transpose(2, 1, 0, 3, 4)
    # numpy sums in another order: the double results may differ in their last
    # bits, which changes a rounding only next to a tie -- at most one unit
    # in the last place, in a tiny fraction of the elements
    want = np.ascontiguousarray(want)
    diff = got != want
    assert diff.mean() <= 1e-3
    g, wv = orc.half_bits_to_double(got, dt), orc.half_bits_to_double(want, dt)
    ulp = np.abs(wv) * (2.0 ** -7 if dt == "bf16" else 2.0 ** -10)
    assert np.all(np.abs(g - wv)[diff] <= ulp[diff])
    if S % P == 0:
        # the same values produced in the sequence-sharded layout, then relaid
        stacked = rounded.reshape(P, S // P, B, H, D).transpose(0, 2, 1, 3, 4)   # [P][B][S/P][H][D]
        relaid = orc.seq_to_head(np.ascontiguousarray(stacked), P, B, S, H, D)
        assert np.array_equal(relaid, want)


def test_brute_force_tiny(orc):
    S, K, P, B, H, D = 4, 8, 2, 2, 2, 2
    x = synth.bits(synth.normal((S, K), seed=1))
    w = synth.bits(synth.normal((B * H * D, K), seed=2))
    got = orc.qkv_projection(x, w, P, B, H, D)
    xd, wd = orc.half_bits_to_double(x), orc.half_bits_to_double(w)
    Hp = H // P
    for r in range(P):
        for b in range(B):
            for t in range(S):
                for hp in range(Hp):
                    for d in range(D):
                        n = (b * H + r * Hp + hp) * D + d
                        v = sum(xd[t, k] * wd[n, k] for k in range(K))
                        assert got[r, b, t, hp, d] == orc.double_to_bf16_bits(np.array([v]))[0]
