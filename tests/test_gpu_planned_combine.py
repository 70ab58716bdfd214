"""GPU parity of the causal combine over a THD layout plan (and its
gradient) against the oracle: ragged planned batches with masked partials
NaN-poisoned (never read), 256-byte and 1 KB rows, fp16; the packed THD batch
planned over 8 ranks at full size, every row; the per-sequence split
given as a plan equals the varlen combine bit for bit; autograd."""

import numpy as np
import pytest
import torch

import synth
from helpers import (window_pool, announce, assert_grad_lse_close, assert_lse_close, assert_rows_close, from_host_bits,
                     grad_lse_scale, to_host_bits)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cam():
    import context_attention_movement_amd as m
    m.library()
    assert torch.cuda.is_available()
    return m


def _plan(cam, orc, cu, W, **kw):
    q = orc.thd_plan(cu, W, **kw)
    plan = cam.ThdPlan(W, int(cu[-1]), cu, q["span_start"], q["span_rank"], q["span_local"], q["rank_off"],
                       q["rank_cost"], q["grid"]).to("cuda")
    return q, orc.plan_first_positions(cu, q, W), plan


CASES = [  # (lengths in blocks, block, W, H, D, dtype)
    ([3, 40, 1, 7, 90, 2], 4, 3, 4, 128, "bf16"),
    ([0, 12, 5, 33, 1, 0, 64], 1, 8, 2, 512, "bf16"),     # 1 KB rows: the row-stream kernel
    ([9, 27, 4], 2, 5, 3, 64, "fp16"),
    ([6, 1, 1], 1, 2, 2, 40, "bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"W{c[2]}H{c[3]}D{c[4]}{c[5]}")
def test_planned_combine(cam, orc, case):
    lens, b, W, H, D, dt = case
    cu = synth.cu_seqlens([x * b for x in lens])
    T = int(cu[-1])
    announce(f"planned combine {case}")
    q, first, plan = _plan(cam, orc, cu, W, block_size=b, min_split_tokens=8 * b)
    mask = orc.plan_mask(cu, first, W)
    o = synth.bits(synth.normal((W, T, H, D), seed=T + W, dtype=dt)).copy()
    l = synth.partial_lse((W, T, H), seed=T + W + 1).numpy().copy()
    o[~mask] = 0x7FC0 if dt == "bf16" else 0x7E00
    l[~mask] = np.nan
    ro, rl = orc.lse_combine_planned(o, l, cu, first, dtype=dt)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float16
    out, lse = cam.lse_combine_planned(from_host_bits(o, tdt), torch.from_numpy(l).cuda(), plan)
    torch.cuda.synchronize()
    assert_rows_close(orc.half_bits_to_double(to_host_bits(out), dt).reshape(-1, D),
                      orc.half_bits_to_double(ro, dt).reshape(-1, D), "planned combine")
    assert_lse_close(lse.cpu().numpy(), rl, "planned combine lse")
    # the gradient under the same rule
    go = synth.bits(synth.normal((T, H, D), seed=T + 7, dtype=dt))
    gl = synth.normal((T, H), seed=T + 8, dtype="fp32").numpy()
    d_po, d_pl = cam.lse_combine_backward(from_host_bits(o, tdt), torch.from_numpy(l).cuda(),
                                          from_host_bits(go, tdt), torch.from_numpy(gl).cuda(), plan=plan)
    torch.cuda.synchronize()
    wo, wl = orc.lse_combine_planned_backward(o, l, go, gl, cu, first, dtype=dt)
    assert_rows_close(orc.half_bits_to_double(to_host_bits(d_po), dt).reshape(-1, D),
                      orc.half_bits_to_double(wo, dt).reshape(-1, D), "planned d_part_out")
    od = orc.half_bits_to_double(o, dt)
    od[np.isnan(od)] = 0.0
    scale = grad_lse_scale(od.reshape(W, T * H, D), orc.half_bits_to_double(go, dt).reshape(T * H, D),
                           gl.reshape(-1).astype(np.float64))
    assert_grad_lse_close(d_pl.cpu().numpy().reshape(W, -1), wl.reshape(W, -1), scale, "planned d_part_lse")


def test_sequence_split_as_plan_equals_varlen_combine(cam, orc):
    P, H, D = 4, 3, 128
    cu = synth.cu_seqlens([5, 0, 17, 3, 40, 1, 2])
    T = int(cu[-1])
    announce("split-as-plan vs varlen combine")
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
    ss = np.array([starts[k] for k in order] + [T], dtype=np.int32)
    plan = cam.ThdPlan(P, T, cu, ss, np.array([ranks[k] for k in order], dtype=np.int32),
                       np.array([local[k] for k in order], dtype=np.int32), np.asarray(rank_off, dtype=np.int64),
                       np.zeros(P), 0).to("cuda")
    po = synth.normal((P, T, H, D), seed=3).cuda()
    pl = synth.partial_lse((P, T, H), seed=4).cuda()
    a_o, a_l = cam.lse_combine_planned(po, pl, plan)
    b_o, b_l = cam.lse_combine_varlen(po, pl, torch.from_numpy(cu).cuda())
    torch.cuda.synchronize()
    assert torch.equal(a_o, b_o) and torch.equal(a_l, b_l)


def test_planned_thd_combine_full_size(cam, orc):
    """The planned THD batch at full size (8-rank plan of 131072 tokens in
    64-token blocks): every row and LSE against the oracle's planned combine."""
    P, H, D = 8, 32, 128
    lens = synth.thd_lengths(20, 131072, seed=synth.BASE_SEED + 4, align=64)
    cu = synth.cu_seqlens(lens)
    T = int(cu[-1])
    announce("planned THD combine full size, every row")
    q, first, plan = _plan(cam, orc, cu, P, block_size=64, min_split_tokens=8192)
    g = synth._gen(synth.BASE_SEED + 91, "cuda")
    po = torch.randn((P, T, H, D), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    pl = torch.randn((P, T, H), generator=g, device="cuda", dtype=torch.float32).mul_(2.0)
    out, lse = cam.lse_combine_planned(po, pl, plan)
    torch.cuda.synchronize()
    po_h, pl_h = to_host_bits(po), pl.cpu().numpy()
    out_h, lse_h = to_host_bits(out), lse.cpu().numpy()
    del po

    def check(a, e):
        ro, rl = orc.lse_combine_planned(po_h[:, a:e], pl_h[:, a:e], cu, first, t_begin=a)
        w = assert_rows_close(orc.half_bits_to_double(out_h[a:e]).reshape(-1, D),
                              orc.half_bits_to_double(ro).reshape(-1, D), f"planned THD rows [{a}, {e})")
        return w, assert_lse_close(lse_h[a:e], rl, f"planned THD lse [{a}, {e})")

    res = window_pool(T, check)
    print(f"planned THD combine, all {T * H} rows: worst row {max(r[0] for r in res):.3e}, "
          f"lse err {max(r[1] for r in res):.3e}", flush=True)


def test_planned_thd_backward_full_size(cam, orc):
    """The gradient of the combine over the 8-rank plan of the full THD batch:
    every row of both gradients against the oracle's planned gradient."""
    P, H, D = 8, 32, 128
    lens = synth.thd_lengths(20, 131072, seed=synth.BASE_SEED + 4, align=64)
    cu = synth.cu_seqlens(lens)
    T = int(cu[-1])
    announce("planned THD combine backward full size, every row")
    q, first, plan = _plan(cam, orc, cu, P, block_size=64, min_split_tokens=8192)
    g = synth._gen(synth.BASE_SEED + 92, "cuda")
    po = torch.randn((P, T, H, D), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    pl = torch.randn((P, T, H), generator=g, device="cuda", dtype=torch.float32).mul_(2.0)
    go = torch.randn((T, H, D), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    gl = torch.randn((T, H), generator=g, device="cuda", dtype=torch.float32)
    d_po, d_pl = cam.lse_combine_backward(po, pl, go, gl, plan=plan)
    torch.cuda.synchronize()
    po_h, pl_h, go_h, gl_h = to_host_bits(po), pl.cpu().numpy(), to_host_bits(go), gl.cpu().numpy()
    dpo_h, dpl_h = to_host_bits(d_po), d_pl.cpu().numpy()
    del po, d_po

    def check(a, e):
        ro, rl = orc.lse_combine_planned_backward(po_h[:, a:e], pl_h[:, a:e], go_h[a:e], gl_h[a:e], cu, first,
                                                  t_begin=a)
        n = (e - a) * H
        got_o = orc.half_bits_to_double(np.ascontiguousarray(dpo_h[:, a:e])).reshape(P, n, D)
        want_o = orc.half_bits_to_double(ro).reshape(P, n, D)
        w = assert_rows_close(got_o.reshape(-1, D), want_o.reshape(-1, D), f"planned d_part_out [{a}, {e})")
        assert np.all(got_o[want_o == 0] == 0), f"planned d_part_out [{a}, {e}) not exactly zero outside the valid set"
        scale = grad_lse_scale(orc.half_bits_to_double(np.ascontiguousarray(po_h[:, a:e])).reshape(P, n, D),
                               orc.half_bits_to_double(go_h[a:e]).reshape(n, D),
                               gl_h[a:e].reshape(-1).astype(np.float64))
        le = assert_grad_lse_close(np.ascontiguousarray(dpl_h[:, a:e]).reshape(P, -1), rl.reshape(P, -1), scale,
                                   f"planned d_part_lse [{a}, {e})")
        return w, le

    res = window_pool(T, check, n_windows=128)
    print(f"planned THD backward, all {T * H} rows: worst d_part_out row {max(r[0] for r in res):.3e}, "
          f"worst d_part_lse / scale {max(r[1] for r in res):.3e}", flush=True)


def test_planned_combine_autograd(cam, orc):
    from context_attention_movement_amd import autograd as ag
    W, H, D = 3, 2, 64
    cu = synth.cu_seqlens([6, 1, 11, 4])
    T = int(cu[-1])
    announce("planned combine autograd")
    q, first, plan = _plan(cam, orc, cu, W, block_size=1, min_split_tokens=5)
    po = synth.normal((W, T, H, D), seed=11).cuda().requires_grad_(True)
    pl = synth.partial_lse((W, T, H), seed=12).cuda().requires_grad_(True)
    go = synth.normal((T, H, D), seed=13).cuda()
    gl = synth.normal((T, H), seed=14, dtype="fp32").cuda()
    out, lse = ag.lse_combine(po, pl, plan=plan)
    d_po, d_pl = torch.autograd.grad((out, lse), (po, pl), (go, gl))
    k_po, k_pl = cam.lse_combine_backward(po.detach(), pl.detach(), go, gl, plan=plan)
    torch.cuda.synchronize()
    assert torch.equal(d_po, k_po) and torch.equal(d_pl, k_pl)
