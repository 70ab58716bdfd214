"""GPU parity of the training-side path against the oracle, through the C ABI.

- lse_combine_backward / lse_combine_varlen_backward: the gradient of the
  partial outputs within 8e-3 per-row relative error (one rounding of w_p g),
  exact zeros for partials outside the valid set; the gradient of the partial
  LSEs within 1e-5 of the row scale sum_d |g_d| max_p |O_pd| + |g_lse|; no NaN,
  invalid or masked partials' rows never read (NaN-poisoned).
- The autograd functions: the relayout's gradient is the inverse relayout, bit
  for bit (dense and varlen, the benchmark's forward/backward training pair);
  the combine's autograd gradient is the kernel's and matches the oracle.
"""

import numpy as np
import pytest
import torch

import synth
from helpers import (window_pool, announce, assert_bits_equal, assert_grad_lse_close, assert_rows_close, grad_lse_scale,
                     to_host_bits)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cam():
    import context_attention_movement_amd as m
    m.library()
    assert torch.cuda.is_available()
    return m


def _check_backward(orc, po, pl, go, gl, d_po, d_pl, cu=None, t_begin=0, dt="bf16", tag=""):
    """Compare GPU gradients (device tensors d_po, d_pl) of the rows
    [t_begin, t_begin + T') with the oracle on host copies of the inputs."""
    pob, gob = to_host_bits(po), to_host_bits(go)
    pln = pl.detach().cpu().numpy()
    gln = gl.detach().cpu().numpy() if gl is not None else None
    ro, rl = orc.lse_combine_backward(pob, pln, gob, gln, dtype=dt, cu=cu, t_begin=t_begin)
    P, T, H, D = po.shape
    got_o = orc.half_bits_to_double(to_host_bits(d_po), dt).reshape(P, T * H, D)
    want_o = orc.half_bits_to_double(ro, dt).reshape(P, T * H, D)
    assert_rows_close(got_o.reshape(-1, D), want_o.reshape(-1, D), f"{tag}: d_part_out")
    zero = want_o == 0
    assert np.all(got_o[zero] == 0), f"{tag}: d_part_out not exactly zero outside the valid set"
    scale = grad_lse_scale(orc.half_bits_to_double(pob, dt).reshape(P, T * H, D),
                           orc.half_bits_to_double(gob, dt).reshape(T * H, D),
                           None if gln is None else gln.reshape(-1).astype(np.float64))
    return assert_grad_lse_close(d_pl.detach().cpu().numpy().reshape(P, -1), rl.reshape(P, -1), scale,
                                 f"{tag}: d_part_lse")


CASES = [  # (P, T, H, D, dtype)
    (2, 33, 3, 64, "bf16"),
    (8, 40, 4, 128, "bf16"),
    (8, 9, 5, 512, "bf16"),      # 1 KB rows: one wave per row
    (3, 17, 2, 24, "fp16"),      # 48-byte rows: 16-byte accesses, 3 lanes
    (5, 11, 3, 6, "bf16"),       # 12-byte rows: 4-byte accesses
    (4, 7, 2, 3, "fp16"),        # 6-byte rows: 2-byte accesses
    (1, 13, 3, 16, "bf16"),      # P = 1: dO = g, dL = g_lse
    (16, 6, 4, 64, "bf16"),
    (64, 3, 2, 32, "bf16"),      # the largest P
    (64, 3, 2, 512, "bf16"),     # the largest P with 1 KB rows (the wide-row form)
    # rows of a wave or more (the row-stream form): a ragged second pass, two
    # full passes, 8-byte accesses, a rank count that is not a power of two
    (8, 9, 3, 520, "bf16"),      # 1040-byte rows: 65 vectors
    (4, 6, 2, 1024, "fp16"),     # 2 KB rows
    (8, 5, 3, 516, "bf16"),      # 1032-byte rows: 8-byte accesses, 129 vectors
    (33, 4, 2, 512, "fp16"),
]


@pytest.mark.parametrize("with_g_lse", [True, False])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "P{}T{}H{}D{}{}".format(*c))
def test_combine_backward(cam, orc, case, with_g_lse):
    P, T, H, D, dt = case
    announce(f"combine backward {case} g_lse={with_g_lse}")
    po = synth.normal((P, T, H, D), seed=500 + P + T, dtype=dt)
    pl = synth.partial_lse((P, T, H), seed=501 + P)
    # invalid statistics: -inf, +inf and NaN LSEs with NaN-poisoned rows
    rng = np.random.default_rng(P * 100 + T)
    n_bad = max(1, (P * T * H) // 20)
    flat = rng.permutation(P * T * H)[:n_bad]
    kinds = [float("-inf"), float("inf"), float("nan")]
    for i, f in enumerate(flat):
        p, r = divmod(int(f), T * H)
        t, h = divmod(r, H)
        pl[p, t, h] = kinds[i % 3]
        po[p, t, h] = float("nan")
    if P > 1:  # one row with no valid partial at all
        pl[:, T // 2, 0] = float("-inf")
    go = synth.normal((T, H, D), seed=502 + T, dtype=dt)
    gl = synth.normal((T, H), seed=503, dtype="fp32") if with_g_lse else None
    d_po, d_pl = cam.lse_combine_backward(po.cuda(), pl.cuda(), go.cuda(), None if gl is None else gl.cuda())
    torch.cuda.synchronize()
    _check_backward(orc, po, pl, go, gl, d_po, d_pl, dt=dt, tag=str(case))
    if P == 1:
        # P = 1: the partial's gradient is the upstream gradient itself
        valid = torch.isfinite(pl[0])
        assert torch.equal(d_po[0].cpu()[valid], go[valid])


@pytest.mark.parametrize("D", [64, 512])
def test_combine_backward_strided(cam, orc, D):
    """LSE [P][H][T] and partials inside a wider buffer; gradients into strided
    views (rows under a wave and rows of a whole wave)."""
    P, T, H = 4, 21, 6
    announce(f"combine backward strided D={D}")
    po = synth.normal((P, T, H, D + 32), seed=61).cuda()[..., 16:16 + D]
    pl = synth.partial_lse((P, H, T), seed=62).cuda().transpose(1, 2)
    go = synth.normal((T, H, D), seed=63).cuda()
    gl = synth.normal((H, T), seed=64, dtype="fp32").cuda().t()
    assert po.stride(2) == D + 32 and pl.stride(1) == 1 and gl.stride(0) == 1
    d_po_buf = torch.full((P, T, H, D + 8), 7.0, dtype=torch.bfloat16, device="cuda")
    d_pl_buf = torch.full((P, H, T), 7.0, dtype=torch.float32, device="cuda")
    d_po, d_pl = cam.lse_combine_backward(po, pl, go, gl,
                                          d_part_out=d_po_buf[..., :D], d_part_lse=d_pl_buf.transpose(1, 2))
    torch.cuda.synchronize()
    assert torch.all(d_po_buf[..., D:] == 7.0), "wrote outside the strided gradient view"
    _check_backward(orc, po, pl, go, gl, d_po, d_pl, tag="strided")


@pytest.mark.parametrize("D", [128, 520])
@pytest.mark.parametrize("P", [2, 4, 8])
def test_varlen_backward_masked_not_read(cam, orc, P, D):
    """Ragged lengths with zero-length and shorter-than-P sequences: masked
    partials get exact zero gradients and their rows are never read (rows
    under a wave, and rows of more than a wave)."""
    H = 4
    lengths = [0, 1, 3, P - 1, 37, 5, 0, 64, 2 * P + 1, 11]
    cu = synth.cu_seqlens(lengths)
    T = int(cu[-1])
    announce(f"varlen backward P={P} T={T} D={D}")
    po = synth.normal((P, T, H, D), seed=70 + P)
    pl = synth.partial_lse((P, T, H), seed=71 + P)
    mask = orc.causal_mask(cu, P)
    for p in range(P):
        for t in range(T):
            if not mask[p, t]:
                pl[p, t] = float("nan")
                po[p, t] = float("nan")
    go = synth.normal((T, H, D), seed=72)
    gl = synth.normal((T, H), seed=73, dtype="fp32")
    cu_d = torch.from_numpy(cu).cuda()
    d_po, d_pl = cam.lse_combine_backward(po.cuda(), pl.cuda(), go.cuda(), gl.cuda(), cu_seqlens=cu_d)
    torch.cuda.synchronize()
    _check_backward(orc, po, pl, go, gl, d_po, d_pl, cu=cu, tag=f"varlen P={P} D={D}")


def test_backward_many_short_rows(cam, orc):
    """Rows of 16 bytes, more than 2^22 of them (6.3 million rows over 2
    partials): invalid statistics and an upstream LSE gradient; every row of
    both gradients against the oracle."""
    P, T, H, D = 2, (1 << 21) + 37, 3, 8
    announce(f"combine backward, {T * H} short rows")
    po = synth.normal((P, T, H, D), seed=synth.BASE_SEED + 91)
    pl = synth.partial_lse((P, T, H), seed=synth.BASE_SEED + 92)
    rng = np.random.default_rng(synth.BASE_SEED + 93)
    bad = torch.from_numpy(rng.random((P, T, H)) < 0.02)
    pl[bad] = float("-inf")
    po[bad] = float("nan")
    go = synth.normal((T, H, D), seed=synth.BASE_SEED + 94)
    gl = synth.normal((T, H), seed=synth.BASE_SEED + 95, dtype="fp32")
    d_po = torch.full((P, T, H, D), 7.0, dtype=torch.bfloat16, device="cuda")
    d_pl = torch.full((P, T, H), 7.0, dtype=torch.float32, device="cuda")
    cam.lse_combine_backward(po.cuda(), pl.cuda(), go.cuda(), gl.cuda(), d_part_out=d_po, d_part_lse=d_pl)
    torch.cuda.synchronize()
    _check_backward(orc, po, pl, go, gl, d_po, d_pl, tag="many short rows")


def test_mla_shape_backward_full_size(cam, orc):
    """The combine's gradient at the MLA decode shape (P = 8, T = 128, H = 128,
    Dv = 512: rows of 1 KB, the row-stream form), with invalid statistics, an
    upstream LSE gradient and the gradient written into a gapped partial
    stack; every row against the oracle."""
    P, T, H, D = 8, 128, 128, 512
    announce("MLA-shape combine backward, every row")
    po = synth.normal((P, T, H, D), seed=synth.BASE_SEED + 81)
    pl = synth.partial_lse((P, T, H), seed=synth.BASE_SEED + 82)
    rng = np.random.default_rng(synth.BASE_SEED + 83)
    bad = rng.random((P, T, H)) < 0.01
    pl[torch.from_numpy(bad)] = float("-inf")
    po[torch.from_numpy(bad)] = float("nan")
    go = synth.normal((T, H, D), seed=synth.BASE_SEED + 84)
    gl = synth.normal((T, H), seed=synth.BASE_SEED + 85, dtype="fp32")
    buf = torch.full((P * (T * H * D + 4096),), 7.0, dtype=torch.bfloat16, device="cuda")
    d_po = buf.as_strided((P, T, H, D), (T * H * D + 4096, H * D, D, 1))
    d_po, d_pl = cam.lse_combine_backward(po.cuda(), pl.cuda(), go.cuda(), gl.cuda(), d_part_out=d_po)
    torch.cuda.synchronize()
    gaps = buf.view(P, T * H * D + 4096)[:, T * H * D:]
    assert torch.all(gaps == 7.0), "wrote into the gaps between partials"
    _check_backward(orc, po, pl, go, gl, d_po, d_pl, tag="MLA shape")


def test_thd_backward_full_size(cam, orc):
    """Packed THD at full size (131072 tokens, H = 32, D = 128, 8 KV-piece
    partials, the launch the benchmark times): the gradient of the whole batch
    on the GPU, every row of both gradients against the oracle."""
    P, H, D = 8, 32, 128
    lens = synth.thd_lengths(20, 131072, seed=synth.BASE_SEED + 4)
    cu = synth.cu_seqlens(lens)
    T = int(cu[-1])
    announce("THD combine backward full size, every row")
    g = synth._gen(synth.BASE_SEED + 78, "cuda")
    po = torch.randn((P, T, H, D), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    pl = torch.randn((P, T, H), generator=g, device="cuda", dtype=torch.float32).mul_(2.0)
    go = torch.randn((T, H, D), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    gl = torch.randn((T, H), generator=g, device="cuda", dtype=torch.float32)
    cu_d = torch.from_numpy(cu).cuda()
    d_po, d_pl = cam.lse_combine_backward(po, pl, go, gl, cu_seqlens=cu_d)
    torch.cuda.synchronize()
    po_h, pl_h, go_h, gl_h = to_host_bits(po), pl.cpu().numpy(), to_host_bits(go), gl.cpu().numpy()
    dpo_h, dpl_h = to_host_bits(d_po), d_pl.cpu().numpy()
    del po, d_po

    def check(a, e):
        ro, rl = orc.lse_combine_backward(po_h[:, a:e], pl_h[:, a:e], go_h[a:e], gl_h[a:e], cu=cu, t_begin=a)
        n = (e - a) * H
        got_o = orc.half_bits_to_double(np.ascontiguousarray(dpo_h[:, a:e])).reshape(P, n, D)
        want_o = orc.half_bits_to_double(ro).reshape(P, n, D)
        w = assert_rows_close(got_o.reshape(-1, D), want_o.reshape(-1, D), f"THD d_part_out [{a}, {e})")
        zero = want_o == 0
        assert np.all(got_o[zero] == 0), f"THD d_part_out [{a}, {e}) not exactly zero outside the valid set"
        scale = grad_lse_scale(orc.half_bits_to_double(np.ascontiguousarray(po_h[:, a:e])).reshape(P, n, D),
                               orc.half_bits_to_double(go_h[a:e]).reshape(n, D),
                               gl_h[a:e].reshape(-1).astype(np.float64))
        le = assert_grad_lse_close(np.ascontiguousarray(dpl_h[:, a:e]).reshape(P, -1), rl.reshape(P, -1), scale,
                                   f"THD d_part_lse [{a}, {e})")
        return w, le

    res = window_pool(T, check, n_windows=128)
    print(f"THD backward, all {T * H} rows: worst d_part_out row {max(r[0] for r in res):.3e}, "
          f"worst d_part_lse / scale {max(r[1] for r in res):.3e}", flush=True)


def test_backward_into_empty_partials(cam, orc):
    """The gradient written into the library's partial-stack layout (64 MiB
    partials, so 1 MiB gaps): every row against the oracle, and the gaps
    between the partials untouched."""
    P, H, D = 8, 32, 128
    lens = synth.thd_lengths(6, 8192, seed=synth.BASE_SEED + 5, lo=64, hi=1024)
    cu = synth.cu_seqlens(lens)
    T = int(cu[-1])
    announce(f"combine backward into empty_partials, T={T}")
    g = synth._gen(synth.BASE_SEED + 79, "cuda")
    po = torch.randn((P, T, H, D), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    pl = torch.randn((P, T, H), generator=g, device="cuda", dtype=torch.float32).mul_(2.0)
    go = torch.randn((T, H, D), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    d_po = cam.empty_partials(P, T, H, D)
    n = T * H * D
    gap = d_po.stride(0) - n
    assert gap == (1 << 19)
    base = torch.full((P * d_po.stride(0),), 7.0, dtype=torch.bfloat16, device="cuda")
    d_po = base.as_strided((P, T, H, D), d_po.stride())
    _, d_pl = cam.lse_combine_backward(po, pl, go, None, cu_seqlens=torch.from_numpy(cu).cuda(), d_part_out=d_po)
    torch.cuda.synchronize()
    assert torch.all(base.view(P, n + gap)[:, n:] == 7.0), "wrote into the gaps between the partials"
    _check_backward(orc, po, pl, go, None, d_po, d_pl, cu=cu, tag="into empty_partials")


# -- autograd -------------------------------------------------------------------

def test_relayout_training_pair_gradients_exact(cam, orc):
    """The benchmark's training pair: y1 = seq_to_head(x), y2 = head_to_seq(y);
    autograd gradients for upstream (dx, dy) equal the oracle's inverse
    relayouts of them bit for bit."""
    from context_attention_movement_amd import autograd as ag
    P, B, S, H, D = 4, 3, 64, 8, 128
    announce("relayout training pair")
    x = synth.normal((P, B, S // P, H, D), seed=81).cuda().requires_grad_(True)
    y = synth.normal((P, 1, S, H // P, D), seed=82).cuda().requires_grad_(True)
    dx = synth.normal((P, B, S, H // P, D), seed=83)
    dy = synth.normal((P, 1, S // P, H, D), seed=84)
    gx, gy = torch.autograd.grad((ag.seq_to_head(x, P), ag.head_to_seq(y, P)), (x, y), (dx.cuda(), dy.cuda()))
    torch.cuda.synchronize()
    assert_bits_equal(to_host_bits(gx), orc.head_to_seq(synth.bits(dx), P, B, S, H, D), "grad of seq->head")
    assert_bits_equal(to_host_bits(gy), orc.seq_to_head(synth.bits(dy), P, 1, S, H, D), "grad of head->seq")


def test_varlen_relayout_gradients_exact(cam, orc):
    from context_attention_movement_amd import autograd as ag
    P, B, H, D = 4, 3, 8, 64
    cu = synth.cu_seqlens([5, 0, 17, 3, 40])
    T = int(cu[-1])
    announce("varlen relayout gradients")
    plan = cam.ulysses_varlen_plan(cu, P)
    x = synth.normal((B * T, H, D), seed=85).cuda().requires_grad_(True)
    y = synth.normal((P, 1, T, H // P, D), seed=86).cuda().requires_grad_(True)
    dx = synth.normal((P, B, T, H // P, D), seed=87)
    dy = synth.normal((T, H, D), seed=88)
    gx, gy = torch.autograd.grad((ag.seq_to_head_varlen(x, plan, B), ag.head_to_seq_varlen(y, plan)), (x, y),
                                 (dx.cuda(), dy.cuda()))
    torch.cuda.synchronize()
    assert_bits_equal(to_host_bits(gx), orc.varlen_head_to_seq(synth.bits(dx), cu, P, B, H, D), "grad varlen s2h")
    assert_bits_equal(to_host_bits(gy), orc.varlen_seq_to_head(synth.bits(dy), cu, P, 1, H, D), "grad varlen h2s")


@pytest.mark.parametrize("causal", [False, True])
def test_combine_autograd(cam, orc, causal):
    """A loss over both outputs of the combine: autograd through the C ABI
    gives the kernel's gradient, which matches the oracle."""
    from context_attention_movement_amd import autograd as ag
    P, H, D = 4, 3, 64
    cu = synth.cu_seqlens([9, 2, 14])
    T = int(cu[-1])
    announce(f"combine autograd causal={causal}")
    po = synth.normal((P, T, H, D), seed=91)
    pl = synth.partial_lse((P, T, H), seed=92)
    go = synth.normal((T, H, D), seed=93)
    gl = synth.normal((T, H), seed=94, dtype="fp32")
    po_d = po.cuda().requires_grad_(True)
    pl_d = pl.cuda().requires_grad_(True)
    cu_d = torch.from_numpy(cu).cuda() if causal else None
    out, lse = ag.lse_combine(po_d, pl_d, cu_d)
    d_po, d_pl = torch.autograd.grad((out, lse), (po_d, pl_d), (go.cuda(), gl.cuda()))
    k_po, k_pl = cam.lse_combine_backward(po.cuda(), pl.cuda(), go.cuda(), gl.cuda(), cu_seqlens=cu_d)
    torch.cuda.synchronize()
    assert torch.equal(d_po, k_po) and torch.equal(d_pl, k_pl)
    _check_backward(orc, po, pl, go, gl, d_po, d_pl, cu=cu if causal else None, tag="autograd")
