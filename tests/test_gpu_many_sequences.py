"""Packed batches with more sequences (or planned spans) than the kernels
stage in LDS (1024 cu_seqlens entries): the tables are then searched in
global memory (64-wide by a wave, then a gallop per lane).  Varlen relayout, causal combine (256-byte and 1 KB rows),
the combine written to sequence shards, the combine gradient and the
planned relayout, each against the oracle."""

import numpy as np
import pytest
import torch

import synth
from helpers import (announce, assert_bits_equal, assert_grad_lse_close, assert_lse_close, assert_rows_close,
                     from_host_bits, grad_lse_scale, to_host_bits)

pytestmark = pytest.mark.gpu

NSEQ = 1500


@pytest.fixture(scope="module")
def cam():
    import context_attention_movement_amd as m
    m.library()
    assert torch.cuda.is_available()
    return m


@pytest.fixture(scope="module")
def batch():
    lengths = synth.random_lengths(NSEQ, seed=77, lo=0, hi=24)
    lengths[100] = 900          # one long sequence among many short ones
    return synth.cu_seqlens(lengths)


def test_varlen_relayout_many_sequences(cam, orc, batch):
    cu = batch
    P, B, H, D = 8, 2, 8, 64
    T = int(cu[-1])
    announce(f"varlen relayout nseq={NSEQ} T={T}")
    plan = cam.ulysses_varlen_plan(cu, P)
    x = synth.normal((B * T, H, D), seed=1).cuda()
    y = cam.ulysses_seq_to_head_varlen(x, plan, B)
    z = cam.ulysses_head_to_seq_varlen(y, plan)
    torch.cuda.synchronize()
    xh = to_host_bits(x)
    assert_bits_equal(to_host_bits(y), orc.varlen_seq_to_head(xh, cu, P, B, H, D), "many-seq seq->head")
    assert_bits_equal(to_host_bits(z), xh, "many-seq round trip")


@pytest.mark.parametrize("D", [128, 512])
def test_varlen_combine_many_sequences(cam, orc, batch, D):
    cu = batch
    P, H = 8, 2
    T = int(cu[-1])
    announce(f"varlen combine nseq={NSEQ} D={D}")
    o = synth.bits(synth.normal((P, T, H, D), seed=2 + D)).copy()
    l = synth.partial_lse((P, T, H), seed=3 + D).numpy().copy()
    mask = orc.causal_mask(cu, P)
    o[~mask] = 0x7FC0
    l[~mask] = np.nan
    ro, rl = orc.lse_combine(o, l, cu=cu)
    cu_d = torch.from_numpy(cu).cuda()
    out, lse = cam.lse_combine_varlen(from_host_bits(o, torch.bfloat16), torch.from_numpy(l).cuda(), cu_d)
    torch.cuda.synchronize()
    assert_rows_close(orc.half_bits_to_double(to_host_bits(out)).reshape(-1, D),
                      orc.half_bits_to_double(ro).reshape(-1, D), "many-seq combine")
    assert_lse_close(lse.cpu().numpy(), rl, "many-seq combine lse")
    # the same rows written to the sequence shards of the varlen relayout
    plan = cam.ulysses_varlen_plan(cu, P)
    so, sl = cam.lse_combine_varlen_seq(from_host_bits(o, torch.bfloat16), torch.from_numpy(l).cuda(), plan)
    torch.cuda.synchronize()
    wo, wl = orc.lse_combine_varlen_seq(o, l, cu)
    assert_rows_close(orc.half_bits_to_double(to_host_bits(so)).reshape(-1, D),
                      orc.half_bits_to_double(wo).reshape(-1, D), "many-seq fused combine")
    assert_lse_close(sl.cpu().numpy(), wl, "many-seq fused lse")


def test_varlen_backward_many_sequences(cam, orc, batch):
    cu = batch
    P, H, D = 8, 2, 128
    T = int(cu[-1])
    announce(f"varlen combine gradient nseq={NSEQ}")
    po = synth.normal((P, T, H, D), seed=5)
    pl = synth.partial_lse((P, T, H), seed=6)
    go = synth.normal((T, H, D), seed=7)
    gl = synth.normal((T, H), seed=8, dtype="fp32")
    d_po, d_pl = cam.lse_combine_backward(po.cuda(), pl.cuda(), go.cuda(), gl.cuda(),
                                          cu_seqlens=torch.from_numpy(cu).cuda())
    torch.cuda.synchronize()
    pob, gob = synth.bits(po), synth.bits(go)
    ro, rl = orc.lse_combine_backward(pob, pl.numpy(), gob, gl.numpy(), cu=cu)
    assert_rows_close(orc.half_bits_to_double(to_host_bits(d_po)).reshape(-1, D),
                      orc.half_bits_to_double(ro).reshape(-1, D), "many-seq d_part_out")
    scale = grad_lse_scale(orc.half_bits_to_double(pob).reshape(P, T * H, D),
                           orc.half_bits_to_double(gob).reshape(T * H, D), gl.numpy().reshape(-1).astype(np.float64))
    assert_grad_lse_close(d_pl.cpu().numpy().reshape(P, -1), rl.reshape(P, -1), scale, "many-seq d_part_lse")


def test_planned_relayout_many_spans(cam, orc):
    lengths = synth.random_lengths(1300, seed=9, lo=1, hi=12)
    cu = synth.cu_seqlens(lengths)
    W, B, H, D = 8, 1, 8, 64
    q = orc.thd_plan(cu, W, block_size=1, min_split_tokens=64)
    assert q["span_rank"].size > 1024
    announce(f"planned relayout with {q['span_rank'].size} spans")
    T = int(cu[-1])
    plan = cam.ThdPlan(W, T, cu, q["span_start"], q["span_rank"], q["span_local"], q["rank_off"],
                       q["rank_cost"], q["grid"]).to("cuda")
    x = synth.normal((B * T, H, D), seed=10).cuda()
    y = cam.ulysses_seq_to_head_spans(x, plan, B)
    z = cam.ulysses_head_to_seq_spans(y, plan)
    torch.cuda.synchronize()
    xh = to_host_bits(x)
    assert_bits_equal(to_host_bits(y), orc.span_seq_to_head(xh, q, W, B, H, D), "many-span seq->head")
    assert_bits_equal(to_host_bits(z), xh, "many-span round trip")
