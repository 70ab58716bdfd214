"""HIP graph capture of the entry points beyond the step: the planned-span
relayout, the combine written to sequence shards, a ring of online merges
(the accumulator reset by a fill kernel inside the graph) and the combine
gradient.  The graph is replayed several times with sentinels in every
output and new inputs at the same addresses, eager work in between, and each
replay is compared with the oracle."""

import numpy as np
import pytest
import torch

import synth
from helpers import (announce, assert_bits_equal, assert_grad_lse_close, assert_lse_close, assert_rows_close,
                     grad_lse_scale, to_host_bits)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cam():
    import context_attention_movement_amd as m
    m.library()
    assert torch.cuda.is_available()
    return m


def test_graph_replay_training_and_extension_ops(cam, orc):
    announce("graph capture: planned relayout, fused combine, ring merges, combine gradient")
    P, H, D, B = 4, 8, 64, 2
    lens = [16 * x for x in (3, 20, 1, 9, 30)]
    cu = synth.cu_seqlens(lens)
    T = int(cu[-1])
    q = orc.thd_plan(cu, P, block_size=16, min_split_tokens=128)
    plan = cam.ThdPlan(P, T, cu, q["span_start"], q["span_rank"], q["span_local"], q["rank_off"],
                       q["rank_cost"], q["grid"]).to("cuda")
    vplan = cam.ulysses_varlen_plan(cu, P)
    cu_d = torch.from_numpy(cu).cuda()

    x = synth.normal((B * T, H, D), seed=1).cuda()
    y = torch.empty((P, B, T, H // P, D), dtype=torch.bfloat16, device="cuda")
    po = synth.normal((P, T, H, D), seed=2).cuda()
    pl = synth.partial_lse((P, T, H), seed=3).cuda()
    comb = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    comb_lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    acc = torch.empty((T, H, D), dtype=torch.float32, device="cuda")
    acc_lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ring_out = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    go = synth.normal((T, H, D), seed=4).cuda()
    gl = synth.normal((T, H), seed=5, dtype="fp32").cuda()
    dpo = torch.empty_like(po)
    dpl = torch.empty_like(pl)

    def step():
        cam.ulysses_seq_to_head_spans(x, plan, B, out=y)
        cam.lse_combine_varlen_seq(po, pl, vplan, out=comb, lse_out=comb_lse)
        acc_lse.fill_(float("-inf"))
        for hop in range(P):
            cam.lse_merge(acc, acc_lse, po[hop], pl[hop], out_final=ring_out if hop == P - 1 else None)
        cam.lse_combine_backward(po, pl, go, gl, cu_seqlens=cu_d, d_part_out=dpo, d_part_lse=dpl)

    def check(tag):
        assert_bits_equal(to_host_bits(y), orc.span_seq_to_head(to_host_bits(x), q, P, B, H, D), f"{tag}: spans")
        pob, pln = to_host_bits(po), pl.cpu().numpy()
        ro, rl = orc.lse_combine_varlen_seq(pob, pln, cu)
        assert_rows_close(orc.half_bits_to_double(to_host_bits(comb)).reshape(-1, D),
                          orc.half_bits_to_double(ro).reshape(-1, D), f"{tag}: fused combine")
        assert_lse_close(comb_lse.cpu().numpy(), rl, f"{tag}: fused combine lse")
        ro2, rl2 = orc.lse_combine(pob, pln)
        assert_rows_close(orc.half_bits_to_double(to_host_bits(ring_out)).reshape(-1, D),
                          orc.half_bits_to_double(ro2).reshape(-1, D), f"{tag}: ring")
        assert_lse_close(acc_lse.cpu().numpy(), rl2, f"{tag}: ring lse")
        gob, gln = to_host_bits(go), gl.cpu().numpy()
        do, dl = orc.lse_combine_backward(pob, pln, gob, gln, cu=cu)
        assert_rows_close(orc.half_bits_to_double(to_host_bits(dpo)).reshape(-1, D),
                          orc.half_bits_to_double(do).reshape(-1, D), f"{tag}: d_part_out")
        scale = grad_lse_scale(orc.half_bits_to_double(pob).reshape(P, T * H, D),
                               orc.half_bits_to_double(gob).reshape(T * H, D), gln.reshape(-1).astype(np.float64))
        assert_grad_lse_close(dpl.cpu().numpy().reshape(P, -1), dl.reshape(P, -1), scale, f"{tag}: d_part_lse")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    check("eager")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for i in range(3):
        for t in (y, comb, ring_out, dpo):
            t.view(torch.int16).fill_(0x7FC0 - i)
        for t in (comb_lse, acc, dpl):
            t.fill_(12345.0)
        graph.replay()
        torch.cuda.synchronize()
        check(f"replay {i}")
        x.copy_(synth.normal((B * T, H, D), seed=10 + i).cuda())
        po.copy_(synth.normal((P, T, H, D), seed=20 + i).cuda())
        pl.copy_(synth.partial_lse((P, T, H), seed=30 + i).cuda())
        go.copy_(synth.normal((T, H, D), seed=40 + i).cuda())
        torch.cuda.synchronize()


def test_graph_replay_planned_combine_and_projection(cam, orc):
    """HIP graph capture of the combine over a THD plan, its gradient and the
    Q/K/V projection into the head-sharded layout (two tiles along each
    dimension and a ragged row tail); every replay, with sentinels in the
    outputs and new inputs at the same addresses, is compared with an eager
    call on the same inputs (bit for bit: same kernels) and the combine with
    the oracle."""
    announce("graph capture: planned combine, its gradient, projection")
    P, H, D = 4, 8, 64
    lens = [16 * x for x in (3, 20, 1, 9, 30)]
    cu = synth.cu_seqlens(lens)
    T = int(cu[-1])
    q = orc.thd_plan(cu, P, block_size=16, min_split_tokens=128)
    plan = cam.ThdPlan(P, T, cu, q["span_start"], q["span_rank"], q["span_local"], q["rank_off"],
                       q["rank_cost"], q["grid"]).to("cuda")
    first = orc.plan_first_positions(cu, q, P)
    po = synth.normal((P, T, H, D), seed=2).cuda()
    pl = synth.partial_lse((P, T, H), seed=3).cuda()
    go = synth.normal((T, H, D), seed=4).cuda()
    gl = synth.normal((T, H), seed=5, dtype="fp32").cuda()
    comb = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    comb_lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    dpo, dpl = torch.empty_like(po), torch.empty_like(pl)
    S, K, Pp, B, Hh, Dh = 300, 128, 2, 3, 4, 64   # N = 768: three column tiles; two row tiles, ragged
    xs = synth.normal((S, K), seed=6).cuda()
    ws = synth.normal((B * Hh * Dh, K), seed=7, std=0.1).cuda()
    proj = torch.empty((Pp, B, S, Hh // Pp, Dh), dtype=torch.bfloat16, device="cuda")

    def step():
        cam.lse_combine_planned(po, pl, plan, out=comb, lse_out=comb_lse)
        cam.lse_combine_backward(po, pl, go, gl, d_part_out=dpo, d_part_lse=dpl, plan=plan)
        cam.qkv_projection_head_sharded(xs, ws, Pp, B, Hh, Dh, out=proj)

    def eager():
        o, l = cam.lse_combine_planned(po, pl, plan)
        a, b = cam.lse_combine_backward(po, pl, go, gl, plan=plan)
        j = cam.qkv_projection_head_sharded(xs, ws, Pp, B, Hh, Dh)
        torch.cuda.synchronize()
        return o, l, a, b, j

    def check(tag):
        o, l, a, b, j = eager()
        for got, want, what in ((comb, o, "combine"), (comb_lse, l, "combine lse"), (dpo, a, "d_part_out"),
                                (dpl, b, "d_part_lse"), (proj, j, "projection")):
            assert torch.equal(got, want), f"{tag}: {what} differs from the eager call"
        ro, rl = orc.lse_combine_planned(to_host_bits(po), pl.cpu().numpy(), cu, first)
        assert_rows_close(orc.half_bits_to_double(to_host_bits(comb)).reshape(-1, D),
                          orc.half_bits_to_double(ro).reshape(-1, D), f"{tag}: planned combine")
        assert_lse_close(comb_lse.cpu().numpy(), rl, f"{tag}: planned combine lse")

    eager()   # first calls (function attributes) outside the capture
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for i in range(3):
        for t in (comb, dpo, proj):
            t.view(torch.int16).fill_(0x7FC0 - i)
        for t in (comb_lse, dpl):
            t.fill_(12345.0)
        graph.replay()
        torch.cuda.synchronize()
        check(f"replay {i}")
        po.copy_(synth.normal((P, T, H, D), seed=20 + i).cuda())
        pl.copy_(synth.partial_lse((P, T, H), seed=30 + i).cuda())
        go.copy_(synth.normal((T, H, D), seed=40 + i).cuda())
        xs.copy_(synth.normal((S, K), seed=50 + i).cuda())
        torch.cuda.synchronize()
