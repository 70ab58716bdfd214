"""Pins of the oracle's training-side functions.

The gradient of the stable combine (orc_combine_row_backward_f64 and its typed
strided form) is pinned against: central finite differences of the oracle's
own forward combine; PyTorch float64 autograd through logsumexp/softmax; the
hand-derived closed forms in tests/golden/combine_gradient_closed_forms.json;
the invariants that follow from the definition (the dL sum to g_lse, a shift
of every LSE changes nothing, a masked or invalid partial gets exactly zero).

The relayout's gradient is its inverse relayout: pinned against PyTorch
autograd through the global-tensor closed form of the permutation, and by the
adjoint identity <S x, y> = <x, S^T y> with exact integer payloads."""

import json
import math
from pathlib import Path

import numpy as np
import pytest
import torch

import synth

GOLDEN = Path(__file__).resolve().parent / "golden"


def _num(v):
    return float(v) if not isinstance(v, str) else {"inf": math.inf, "-inf": -math.inf, "nan": math.nan}[v]


def _row(seed, P, D, n_invalid=0):
    rng = np.random.default_rng(seed)
    o = rng.normal(size=(P, D))
    lse = rng.normal(scale=2.0, size=P)
    g = rng.normal(size=D)
    valid = np.ones(P, dtype=np.int32)
    valid[rng.permutation(P)[:n_invalid]] = 0
    return o, lse, g, valid


def _forward_objective(orc, o, lse, valid, g, g_lse):
    """F = <g, out> + g_lse * lse_out of the oracle's forward combine (one row)."""
    o_m = np.where(valid[:, None] == 1, o, np.nan)          # masked rows must not be read
    l_m = np.where(valid == 1, lse, -np.inf)
    out, lse_out = orc.combine_f64(o_m[:, None, :], l_m[:, None])
    return float(np.dot(g, out[0]) + g_lse * lse_out[0])


def test_golden_closed_forms(orc):
    g = json.loads((GOLDEN / "combine_gradient_closed_forms.json").read_text())
    for c in g["cases"]:
        o = np.array([[_num(v) for v in r] for r in c["o"]])
        lse = np.array([_num(v) for v in c["lse"]])
        d_o, d_l = orc.combine_row_backward_f64(o, lse, np.array(c["g"]), c["g_lse"])
        assert np.allclose(d_o, np.array(c["d_o"]), rtol=0, atol=1e-15), c["why"]
        assert np.allclose(d_l, np.array(c["d_lse"]), rtol=0, atol=1e-15), c["why"]
        assert not np.isnan(d_o).any() and not np.isnan(d_l).any()


@pytest.mark.parametrize("P,D,n_invalid,g_lse", [(1, 3, 0, 0.7), (2, 5, 0, 0.0), (5, 7, 2, -1.3),
                                                 (8, 16, 3, 0.5), (8, 4, 0, 0.0)])
def test_finite_differences_of_forward(orc, P, D, n_invalid, g_lse):
    o, lse, g, valid = _row(100 + 17 * P + D, P, D, n_invalid)
    d_o, d_l = orc.combine_row_backward_f64(o, lse, g, g_lse, valid)
    h = 1e-6
    for p in range(P):
        for d in range(D):
            op, om = o.copy(), o.copy()
            op[p, d] += h
            om[p, d] -= h
            fd = (_forward_objective(orc, op, lse, valid, g, g_lse)
                  - _forward_objective(orc, om, lse, valid, g, g_lse)) / (2 * h)
            assert abs(fd - d_o[p, d]) <= 1e-7 * (1 + abs(fd)), (p, d, fd, d_o[p, d])
        lp, lm = lse.copy(), lse.copy()
        lp[p] += h
        lm[p] -= h
        fd = (_forward_objective(orc, o, lp, valid, g, g_lse)
              - _forward_objective(orc, o, lm, valid, g, g_lse)) / (2 * h)
        assert abs(fd - d_l[p]) <= 1e-7 * (1 + abs(fd)), (p, fd, d_l[p])
        if not valid[p]:
            assert d_l[p] == 0.0 and not d_o[p].any()


@pytest.mark.parametrize("P,D", [(2, 8), (4, 32), (8, 128)])
def test_torch_autograd_float64(orc, P, D):
    o, lse, g, _ = _row(7 * P + D, P, D)
    g_lse = 0.375
    ot = torch.tensor(o, dtype=torch.float64, requires_grad=True)
    lt = torch.tensor(lse, dtype=torch.float64, requires_grad=True)
    lse_out = torch.logsumexp(lt, dim=0)
    out = (torch.softmax(lt, dim=0)[:, None] * ot).sum(0)
    obj = (out * torch.tensor(g)).sum() + g_lse * lse_out
    go, gl = torch.autograd.grad(obj, (ot, lt))
    d_o, d_l = orc.combine_row_backward_f64(o, lse, g, g_lse)
    assert np.allclose(d_o, go.numpy(), rtol=1e-13, atol=1e-14)
    assert np.allclose(d_l, gl.numpy(), rtol=1e-12, atol=1e-13)


def test_invariants(orc):
    o, lse, g, valid = _row(5, 6, 9, n_invalid=2)
    d_o, d_l = orc.combine_row_backward_f64(o, lse, g, 1.25, valid)
    assert abs(d_l.sum() - 1.25) < 1e-13                          # the weights sum to one
    d_o2, d_l2 = orc.combine_row_backward_f64(o, lse + 40.0, g, 1.25, valid)
    assert np.allclose(d_o, d_o2, atol=1e-15) and np.allclose(d_l, d_l2, atol=1e-13)
    inv = valid == 0
    assert (d_o[inv] == 0).all() and (d_l[inv] == 0).all()
    # a NaN-poisoned row of an invalid partial changes nothing
    o_bad = o.copy()
    o_bad[inv] = np.nan
    d_o3, d_l3 = orc.combine_row_backward_f64(o_bad, lse, g, 1.25, valid)
    assert np.array_equal(d_o, d_o3) and np.array_equal(d_l, d_l3)
    # the gradient is linear in (g, g_lse)
    d_o4, d_l4 = orc.combine_row_backward_f64(o, lse, 3.0 * g, 3.75, valid)
    assert np.allclose(d_o4, 3 * d_o, atol=1e-14) and np.allclose(d_l4, 3 * d_l, atol=1e-13)


@pytest.mark.parametrize("with_g_lse", [False, True])
@pytest.mark.parametrize("causal", [False, True])
def test_typed_backward_is_rounded_f64_backward(orc, causal, with_g_lse):
    P, H, D = 4, 3, 16
    lengths = [3, 9, 1, 12]
    cu = synth.cu_seqlens(lengths)
    T = int(cu[-1])
    po = synth.bits(synth.normal((P, T, H, D), seed=91))
    pl = synth.partial_lse((P, T, H), seed=92).numpy()
    pl[1, 5, 2] = -np.inf
    pl[3, 0, 0] = np.nan
    go = synth.bits(synth.normal((T, H, D), seed=93))
    gl = synth.normal((T, H), seed=94, dtype="fp32").numpy() if with_g_lse else None
    d_po, d_pl = orc.lse_combine_backward(po, pl, go, gl, cu=cu if causal else None)
    dec = orc.half_bits_to_double
    for t in range(T):
        for h in range(H):
            valid = np.array([orc.causal_piece_valid(cu, P, p, t) if causal else 1 for p in range(P)],
                             dtype=np.int32)
            o = np.stack([dec(po[p, t, h]) for p in range(P)])
            lse = pl[:, t, h].astype(np.float64)
            lse = np.where(valid == 1, lse, -np.inf)
            d_o, d_l = orc.combine_row_backward_f64(np.nan_to_num(o), lse, dec(go[t, h]),
                                                    float(gl[t, h]) if gl is not None else 0.0, valid)
            assert np.array_equal(d_po[:, t, h], orc.double_to_bf16_bits(d_o)), (t, h)
            assert np.array_equal(d_pl[:, t, h], d_l.astype(np.float32)), (t, h)


def test_typed_backward_window_and_strides(orc):
    """A window of rows [t0, t1) of strided (LSE [P][H][T]) inputs gives the
    same values as the whole batch."""
    P, T, H, D = 3, 10, 2, 8
    po = synth.bits(synth.normal((P, T, H, D), seed=31))
    pl_ht = synth.partial_lse((P, H, T), seed=32).numpy()
    pl = pl_ht.transpose(0, 2, 1)
    go = synth.bits(synth.normal((T, H, D), seed=33))
    full_o, full_l = orc.lse_combine_backward(po, pl, go)
    t0, t1 = 3, 8
    w_o, w_l = orc.lse_combine_backward(po[:, t0:t1], pl[:, t0:t1], go[t0:t1], t_begin=t0)
    assert np.array_equal(w_o, full_o[:, t0:t1]) and np.array_equal(w_l, full_l[:, t0:t1])


# -- the relayout's gradient -----------------------------------------------------

@pytest.mark.parametrize("P,B,S,H,D", [(2, 3, 8, 4, 8), (4, 1, 8, 8, 2), (3, 2, 9, 6, 4)])
def test_relayout_gradient_is_inverse_relayout(orc, P, B, S, H, D):
    """Autograd through the global-tensor form of the all-to-all: the gradient
    of y = seq_to_head(x) for upstream dy equals head_to_seq(dy), and the other
    way round, exactly (a permutation moves values without arithmetic)."""
    X = synth.normal((B, S, H, D), seed=P + S, dtype="fp32").double()

    def s2h(x_seq):  # [P][B][S/P][H][D] -> [P][B][S][H/P][D]
        glob = x_seq.permute(1, 0, 2, 3, 4).reshape(B, S, H, D)
        return glob.reshape(B, S, P, H // P, D).permute(2, 0, 1, 3, 4)

    def h2s(y_head):  # inverse
        glob = y_head.permute(1, 2, 0, 3, 4).reshape(B, S, H, D)
        return glob.reshape(B, P, S // P, H, D).permute(1, 0, 2, 3, 4)

    x_seq = X.reshape(B, P, S // P, H, D).permute(1, 0, 2, 3, 4).contiguous().requires_grad_(True)
    dy = synth.normal((P, B, S, H // P, D), seed=77, dtype="fp32").double()
    (gx,) = torch.autograd.grad(s2h(x_seq), x_seq, dy)
    want = orc.head_to_seq(dy.numpy().view(np.uint64), P, B, S, H, D)
    assert np.array_equal(gx.numpy().view(np.uint64), want)

    y_head = s2h(x_seq.detach()).contiguous().requires_grad_(True)
    dx = synth.normal((P, B, S // P, H, D), seed=78, dtype="fp32").double()
    (gy,) = torch.autograd.grad(h2s(y_head), y_head, dx)
    want = orc.seq_to_head(dx.numpy().view(np.uint64), P, B, S, H, D)
    assert np.array_equal(gy.numpy().view(np.uint64), want)


def test_relayout_adjoint_identity(orc):
    """<S x, y> = <x, S^T y> with S^T = head_to_seq, in exact integer arithmetic."""
    P, B, S, H, D = 4, 2, 12, 8, 3
    rng = np.random.default_rng(3)
    x = rng.integers(-1000, 1000, size=(P, B, S // P, H, D)).astype(np.int64)
    y = rng.integers(-1000, 1000, size=(P, B, S, H // P, D)).astype(np.int64)
    lhs = int((orc.seq_to_head(x.view(np.uint64), P, B, S, H, D).view(np.int64) * y).sum())
    rhs = int((x * orc.head_to_seq(y.view(np.uint64), P, B, S, H, D).view(np.int64)).sum())
    assert lhs == rhs


def test_varlen_relayout_adjoint_identity(orc):
    P, B, H, D = 4, 2, 8, 2
    cu = synth.cu_seqlens([5, 1, 0, 11, 3])
    T = int(cu[-1])
    rng = np.random.default_rng(4)
    x = rng.integers(-1000, 1000, size=(B * T * H * D,)).astype(np.int64)
    y = rng.integers(-1000, 1000, size=(B * T * H * D,)).astype(np.int64)
    sx = orc.varlen_seq_to_head(x.view(np.uint64), cu, P, B, H, D).view(np.int64).reshape(-1)
    ty = orc.varlen_head_to_seq(y.view(np.uint64), cu, P, B, H, D).view(np.int64).reshape(-1)
    assert int((sx * y).sum()) == int((x * ty).sum())
