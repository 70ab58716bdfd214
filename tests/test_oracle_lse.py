"""Pins of the oracle's LSE formation, max/sum-aware pack and stable combine.

- LSE and combine closed forms written out by hand (tests/golden).
- Pack O-region against the slicing closed form; L-region against the legacy
  path: materialize LSE, then permute/reshape, then pack, computed here with
  Python's own math.log.
- Combine: P = 1 identity, brute-force attention split into KV chunks equals
  the LSE combine of the chunks, invariances (shift, permutation, neutral
  -inf partial, duplication adds ln 2, associativity), invalid statistics.
- Causal piece validity against brute-force attention (a partial is valid iff
  its masked attention has a visible key)."""

import itertools
import json
import math
from pathlib import Path

import numpy as np
import pytest
import torch

import synth

GOLDEN = Path(__file__).resolve().parent / "golden"


def _num(v):
    return {"inf": math.inf, "-inf": -math.inf, "nan": math.nan, "-0": -0.0}.get(v, v) if isinstance(v, str) else v


def test_lse_golden_cases(orc):
    g = json.loads((GOLDEN / "lse_and_combine_closed_forms.json").read_text())
    for c in g["lse_cases"]:
        got = orc.lse_from_stats(np.float32(_num(c["max"])), np.float32(_num(c["sum"])))
        want = _num(c["lse"])
        if math.isinf(want):
            assert got == want, c
        else:
            assert abs(got - want) < 1e-7, c


def test_combine_golden_cases(orc):
    g = json.loads((GOLDEN / "lse_and_combine_closed_forms.json").read_text())
    for c in g["combine_cases"]:
        lse = np.array([_num(v) for v in c["lse"]], dtype=np.float64)
        o = np.array([[_num(v) for v in row] for row in c["o"]], dtype=np.float64)
        P, D = o.shape
        out, l = orc.combine_f64(o.reshape(P, 1, D), lse.reshape(P, 1))
        want = np.array([_num(v) for v in c["out"]])
        assert not np.isnan(out).any(), c
        assert np.allclose(out[0], want, rtol=0, atol=1e-14), c
        if math.isinf(_num(c["lse_out"])):
            assert l[0] == -math.inf and np.all(np.signbit(out) == False), c  # noqa: E712
        else:
            assert abs(l[0] - _num(c["lse_out"])) < 1e-14, c


# ----------------------------- pack -----------------------------------------

def _stats(P, T, H, seed, corrupt=0.0):
    out, m, s, idx = synth.dcp_partials(P, T, H, 8, seed, corrupt_frac=corrupt)
    return m.numpy(), s.numpy(), idx


@pytest.mark.parametrize("scatter_dim", [0, 1])
@pytest.mark.parametrize("P,T,H,Dv", [(2, 4, 4, 8), (4, 8, 8, 16), (3, 6, 6, 5), (1, 3, 2, 4)])
def test_pack_matches_slicing_and_legacy_path(orc, scatter_dim, P, T, H, Dv):
    o, m, s, _ = synth.dcp_partials(P, T, H, Dv, seed=77 + P + T, corrupt_frac=0.2)
    ob = synth.bits(o)
    m = m.numpy()
    s = s.numpy()
    packed = orc.lse_pack(ob, m, s, scatter_dim)
    O, L = orc.packed_regions(packed, P, T, H, Dv, scatter_dim)
    # legacy path: materialize LSE, then permute/reshape into the same slices
    lse = np.empty((P, T, H), dtype=np.float32)
    for p, t, h in itertools.product(range(P), range(T), range(H)):
        mm, ss = float(m[p, t, h]), float(s[p, t, h])
        ok = math.isfinite(mm) and math.isfinite(ss) and ss > 0
        lse[p, t, h] = np.float32(mm + math.log(ss)) if ok else -np.inf
    for p in range(P):
        for r in range(P):
            if scatter_dim == 1:
                Hp = H // P
                o_sl = ob[p][:, r * Hp:(r + 1) * Hp, :].reshape(-1, Dv)
                l_sl = lse[p][:, r * Hp:(r + 1) * Hp].reshape(-1)
            else:
                Tp = T // P
                o_sl = ob[p][r * Tp:(r + 1) * Tp].reshape(-1, Dv)
                l_sl = lse[p][r * Tp:(r + 1) * Tp].reshape(-1)
            assert np.array_equal(O[p, r], o_sl)
            assert np.array_equal(L[p, r], l_sl)


def test_pack_chunk_geometry(orc):
    # MLA decode shape: rows = T * H / P = 2048, O = 2048*512*2, L = 2048*4
    assert orc.pack_rows(8, 128, 128, 1) == 2048
    assert orc.pack_chunk_bytes(8, 128, 128, 512, 1) == 2_097_152 + 8_192
    # ragged rows pad each region to 16 bytes
    assert orc.pack_chunk_bytes(2, 3, 2, 3, 1) == 32 + 16


def test_pack_noncontiguous_strides(orc):
    P, T, H, Dv = 2, 4, 4, 8
    o, m, s, _ = synth.dcp_partials(P, T, H, Dv, seed=5, corrupt_frac=0.25)
    ob = synth.bits(o)
    # out stored as [P][H][T][Dv] and viewed as [P][T][H][Dv]; stats stored [H][P][T]
    ob_store = np.ascontiguousarray(ob.transpose(0, 2, 1, 3))
    ob_view = ob_store.transpose(0, 2, 1, 3)
    m_store = np.ascontiguousarray(m.numpy().transpose(2, 0, 1))
    s_store = np.ascontiguousarray(s.numpy().transpose(2, 0, 1))
    m_view = m_store.transpose(1, 2, 0)
    s_view = s_store.transpose(1, 2, 0)
    for sd in (0, 1):
        ref = orc.lse_pack(np.ascontiguousarray(ob), np.ascontiguousarray(m.numpy()),
                           np.ascontiguousarray(s.numpy()), sd)
        got = orc.lse_pack(ob_view, m_view, s_view, sd)
        O1, L1 = orc.packed_regions(ref, P, T, H, Dv, sd)
        O2, L2 = orc.packed_regions(got, P, T, H, Dv, sd)
        assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_pack_special_cases_and_denormal(orc):
    specials = [(math.inf, 1.0), (-math.inf, 1.0), (math.nan, 1.0), (0.5, math.nan), (0.5, math.inf),
                (0.5, 0.0), (0.5, -0.0), (0.5, -2.0), (0.5, 1e-45), (0.5, 1e-40)]
    for mm, ss in specials:
        v = orc.lse_from_stats(np.float32(mm), np.float32(ss))
        if ss in (1e-45, 1e-40):
            assert math.isfinite(v) and abs(v - (0.5 + math.log(float(np.float32(ss))))) < 1e-12
        else:
            assert v == -math.inf


# ----------------------------- combine --------------------------------------

def test_p1_identity_exact(orc):
    T, H, D = 5, 3, 16
    o = synth.bits(synth.normal((1, T, H, D), seed=9))
    l = synth.partial_lse((1, T, H), seed=10).numpy()
    l[0, 1, 2] = -np.inf
    l[0, 3, 0] = np.nan
    out, lse = orc.lse_combine(o, l)
    for t in range(T):
        for h in range(H):
            if np.isfinite(l[0, t, h]):
                assert np.array_equal(out[t, h], o[0, t, h])
                assert lse[t, h] == l[0, t, h]
            else:
                assert np.all(out[t, h] == 0)  # +0.0 bits
                assert lse[t, h] == -np.inf


def _qkv(T, H, D, seed):
    return [synth.bits(synth.normal((T, H, D), seed=seed + i)) for i in range(3)]


@pytest.mark.parametrize("T,H,D,cuts", [(16, 2, 8, [0, 8, 16]), (13, 3, 4, [0, 1, 5, 5, 13]),
                                        (20, 1, 16, [0, 3, 7, 12, 20])])
def test_brute_force_attention_equals_chunk_combine(orc, T, H, D, cuts):
    q, k, v = _qkv(T, H, D, seed=300 + T)
    full_o, full_m, full_s = orc.attention(q, k, v, 0, T)
    full_lse = full_m + np.log(full_s)
    parts_o, parts_l = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        o, m, s = orc.attention(q, k, v, a, b)
        with np.errstate(divide="ignore"):
            parts_l.append(np.where(s > 0, m + np.log(np.where(s > 0, s, 1.0)), -np.inf))
        parts_o.append(o)
    P = len(parts_o)
    out, lse = orc.combine_f64(np.stack(parts_o).reshape(P, T * H, D), np.stack(parts_l).reshape(P, T * H))
    assert np.max(np.abs(out - full_o.reshape(T * H, D))) <= 1e-12
    assert np.max(np.abs(lse - full_lse.reshape(-1))) <= 1e-12


@pytest.mark.parametrize("lengths,P", [([9, 1, 16], 4), ([5, 12], 8), ([3], 2)])
def test_causal_varlen_attention_equals_masked_combine(orc, lengths, P):
    """Per sequence, causal attention over the whole sequence equals the
    combine of causal attention over its P KV pieces, with exactly the pieces
    orc_causal_piece_valid admits (those with a visible key)."""
    cu = synth.cu_seqlens(lengths)
    H, D = 2, 4
    for i, L in enumerate(lengths):
        q, k, v = _qkv(L, H, D, seed=40 + i)
        full_o, full_m, full_s = orc.attention(q, k, v, 0, L, causal=True)
        po, pl = [], []
        for p in range(P):
            a, b = (p * L) // P, ((p + 1) * L) // P
            o, m, s = orc.attention(q, k, v, a, b, causal=True)
            for kk in range(L):
                visible = s[kk, 0] > 0
                assert visible == orc.causal_piece_valid(cu, P, p, int(cu[i]) + kk)
            with np.errstate(divide="ignore"):
                pl.append(np.where(s > 0, m + np.log(np.where(s > 0, s, 1.0)), -np.inf))
            po.append(o)
        out, lse = orc.combine_f64(np.stack(po).reshape(P, L * H, D), np.stack(pl).reshape(P, L * H))
        assert np.max(np.abs(out - full_o.reshape(L * H, D))) <= 1e-12
        assert np.max(np.abs(lse - (full_m + np.log(full_s)).reshape(-1))) <= 1e-12


def _rand_parts(P, R, D, seed):
    g = np.random.default_rng(seed)
    return g.standard_normal((P, R, D)), g.standard_normal((P, R)) * 2


def test_combine_invariances(orc):
    P, R, D = 4, 7, 5
    o, l = _rand_parts(P, R, D, 1)
    base_o, base_l = orc.combine_f64(o, l)
    # shift every LSE by c: out unchanged, lse shifted by c
    so, sl = orc.combine_f64(o, l + 3.25)
    assert np.allclose(so, base_o, rtol=0, atol=1e-13) and np.allclose(sl, base_l + 3.25, rtol=0, atol=1e-13)
    # permutation of partials
    perm = [2, 0, 3, 1]
    po, pl = orc.combine_f64(o[perm], l[perm])
    assert np.allclose(po, base_o, rtol=0, atol=1e-13) and np.allclose(pl, base_l, rtol=0, atol=1e-13)
    # a -inf partial (with garbage O) is neutral
    o2 = np.concatenate([o, np.full((1, R, D), np.nan)])
    l2 = np.concatenate([l, np.full((1, R), -np.inf)])
    no, nl = orc.combine_f64(o2, l2)
    assert np.array_equal(no, base_o) and np.array_equal(nl, base_l)
    # duplicating every partial adds ln 2 to the LSE
    do, dl = orc.combine_f64(np.concatenate([o, o]), np.concatenate([l, l]))
    assert np.allclose(do, base_o, rtol=0, atol=1e-13) and np.allclose(dl, base_l + math.log(2), rtol=0, atol=1e-13)
    # associativity: combine(combine(A, B), C) == combine(A, B, C)
    ab_o, ab_l = orc.combine_f64(o[:2], l[:2])
    abc_o, abc_l = orc.combine_f64(np.stack([ab_o, o[2], o[3]]), np.stack([ab_l, l[2], l[3]]))
    assert np.allclose(abc_o, base_o, rtol=0, atol=1e-13) and np.allclose(abc_l, base_l, rtol=0, atol=1e-13)


def test_invalid_statistics_give_neg_inf_and_no_nan(orc):
    """Pack rows built from invalid statistics get -inf LSE; the combine never
    reads those partials' O rows (poisoned with NaN here) and an all-invalid
    row comes out as +0 with lse -inf."""
    P, T, H, Dv = 2, 4, 2, 8
    o, m, s, _ = synth.dcp_partials(P, T, H, Dv, seed=3, corrupt_frac=0.0)
    ob = synth.bits(o).copy()
    m = m.numpy().copy()
    s = s.numpy().copy()
    # token 1 head 0: rank 0 invalid (sum <= 0); token 2 head 1: both ranks invalid
    s[0, 1, 0] = -1.0
    ob[0, 1, 0] = 0x7FC0
    m[0, 2, 1] = np.nan
    s[1, 2, 1] = np.inf
    ob[0, 2, 1] = 0x7FC0
    ob[1, 2, 1] = 0xFFC1
    for sd in (0, 1):
        packed = orc.lse_pack(ob, m, s, sd)
        out, lse = orc.lse_combine_packed(packed, P, T, H, Dv, sd)
        vals = orc.half_bits_to_double(out)
        assert not np.isnan(vals).any()
        O, L = orc.packed_regions(packed, P, T, H, Dv, sd)
        n_inf = int(np.isneginf(L).sum())
        assert n_inf == 3
        assert np.isneginf(lse).sum() == 1
        row = np.nonzero(np.isneginf(lse))[0][0]
        assert np.all(out[row] == 0)


def test_typed_combine_is_rounded_f64_combine(orc):
    """The strided bf16 combine equals the double combine of the decoded inputs
    rounded once, under strided (non-contiguous) storage of every operand."""
    P, T, H, D = 3, 6, 4, 8
    o = synth.bits(synth.normal((P, H, T, D), seed=21))  # stored [P][H][T][D]
    l = synth.partial_lse((T, P, H), seed=22).numpy()  # stored [T][P][H]
    l[2, 1, 3] = -np.inf
    l[4, :, 0] = np.nan
    o_view = o.transpose(0, 2, 1, 3)
    l_view = l.transpose(1, 0, 2)
    out, lse = orc.lse_combine(o_view, l_view)
    dec = orc.half_bits_to_double(np.ascontiguousarray(o_view)).reshape(P, T * H, D)
    ref_o, ref_l = orc.combine_f64(dec, np.ascontiguousarray(l_view).astype(np.float64).reshape(P, T * H))
    assert np.array_equal(out.reshape(T * H, D), orc.round_half(ref_o))
    assert np.array_equal(lse.reshape(-1), ref_l.astype(np.float32))


def test_packed_combine_equals_generic_on_received_views(orc):
    P, T, H, Dv = 4, 8, 8, 16
    o, m, s, _ = synth.dcp_partials(P, T, H, Dv, seed=13, corrupt_frac=0.1)
    ob, m, s = synth.bits(o), m.numpy(), s.numpy()
    for sd in (0, 1):
        packed = orc.lse_pack(ob, m, s, sd)
        out, lse = orc.lse_combine_packed(packed, P, T, H, Dv, sd)
        O, L = orc.packed_regions(packed, P, T, H, Dv, sd)
        rows = O.shape[2]
        for r in range(P):
            go, gl = orc.lse_combine(np.ascontiguousarray(O[:, r]).reshape(P, rows, 1, Dv),
                                     np.ascontiguousarray(L[:, r]).reshape(P, rows, 1))
            assert np.array_equal(go.reshape(rows, Dv), out[r * rows:(r + 1) * rows])
            assert np.array_equal(gl.reshape(rows), lse[r * rows:(r + 1) * rows])


def test_varlen_combine_skips_masked_partials(orc):
    lengths, P, H, D = [5, 11, 2, 0, 7], 4, 2, 8
    cu = synth.cu_seqlens(lengths)
    T = int(cu[-1])
    o = synth.bits(synth.normal((P, T, H, D), seed=31)).copy()
    l = synth.partial_lse((P, T, H), seed=32).numpy().copy()
    mask = orc.causal_mask(cu, P)
    o_clean, l_clean = o.copy(), l.copy()
    o[~mask] = 0x7FC0  # NaN poison in every masked partial row
    l[~mask] = np.nan
    out, lse = orc.lse_combine(o, l, cu=cu)
    # equal to the plain combine of the unpoisoned data with masked LSEs set to -inf
    l_ref = np.where(mask[:, :, None], l_clean, -np.inf).astype(np.float32)
    ref_o, ref_l = orc.lse_combine(o_clean, l_ref)
    assert np.array_equal(out, ref_o) and np.array_equal(lse, ref_l)
    # a sampled window addressed from its first row gives the same rows
    a, b = 4, 13
    wo, wl = orc.lse_combine(np.ascontiguousarray(o[:, a:b]), np.ascontiguousarray(l[:, a:b]), cu=cu, t_begin=a)
    assert np.array_equal(wo, out[a:b]) and np.array_equal(wl, lse[a:b])


# ------------------- combine with sequence-sharded output -------------------

def test_token_rows_match_varlen_relayout(orc):
    """The rank-major row of each token is where the varlen head->seq relayout
    puts that token's row (checked with an index payload over P = 1 heads)."""
    for lengths, P in (([5, 0, 9, 1, 3], 3), ([17, 33, 2, 64], 4), ([3], 8)):
        cu = synth.cu_seqlens(lengths)
        T = int(cu[-1])
        rows = orc.varlen_token_rows(cu, P)
        assert np.array_equal(np.sort(rows), np.arange(T))
        # head-sharded payload whose value is the token index, one head per rank
        x = np.broadcast_to(np.arange(T, dtype=np.uint32)[None, None, :, None, None], (P, 1, T, 1, 1)).copy()
        y = orc.varlen_head_to_seq(x, cu, P, 1, P, 1).reshape(T, P)
        assert np.array_equal(y[rows, 0], np.arange(T))


@pytest.mark.parametrize("sd", [0, 1])
def test_packed_seq_is_combine_then_head_to_seq(orc, sd):
    P, T, H, Dv = 4, 8, 8, 16
    o, m, s, _ = synth.dcp_partials(P, T, H, Dv, seed=17, corrupt_frac=0.1)
    packed = orc.lse_pack(synth.bits(o), m.numpy(), s.numpy(), sd)
    out, lse = orc.lse_combine_packed_seq(packed, P, T, H, Dv, sd)
    comb, clse = orc.lse_combine_packed(packed, P, T, H, Dv, sd)
    if sd == 0:
        assert np.array_equal(out.reshape(-1, Dv), comb) and np.array_equal(lse.reshape(-1), clse)
    else:
        # destination-major [P][T][H/P][Dv] moved by the dense head->seq relayout (B = 1)
        ref = orc.head_to_seq(comb.reshape(P, 1, T, H // P, Dv), P, 1, T, H, Dv).reshape(T, H, Dv)
        assert np.array_equal(out, ref)
        lref = orc.head_to_seq(clse.reshape(P, 1, T, H // P, 1), P, 1, T, H, 1).reshape(T, H)
        assert np.array_equal(lse, lref)
