"""Empty and degenerate inputs through every entry point that launches: a
zero-size call returns without launching or writing (sentinels survive), and
degenerate shapes (one partial, one head per rank, a single-token batch)
match the oracle."""

import numpy as np
import pytest
import torch

import synth
from helpers import announce, assert_bits_equal, assert_lse_close, assert_rows_close, to_host_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cam():
    import context_attention_movement_amd as m
    m.library()
    assert torch.cuda.is_available()
    return m


def test_zero_sized_calls_launch_nothing(cam):
    announce("zero-sized calls")
    dev = "cuda"
    bf = torch.bfloat16
    sentinel = torch.full((16,), 7.0, device=dev)
    # combine over zero tokens / zero heads
    po = torch.empty((4, 0, 3, 64), dtype=bf, device=dev)
    pl = torch.empty((4, 0, 3), dtype=torch.float32, device=dev)
    out, lse = cam.lse_combine(po, pl)
    assert out.numel() == 0 and lse.numel() == 0
    d_po, d_pl = cam.lse_combine_backward(po, pl, torch.empty((0, 3, 64), dtype=bf, device=dev))
    assert d_po.numel() == 0 and d_pl.numel() == 0
    acc = torch.empty((0, 3, 64), dtype=torch.float32, device=dev)
    cam.lse_merge(acc, torch.empty((0, 3), device=dev), po[0], pl[0])
    # empty packed exchange
    o = torch.empty((2, 0, 4, 64), dtype=bf, device=dev)
    m = torch.empty((2, 0, 4), device=dev)
    packed = cam.lse_pack(o, m, m.clone(), 1)
    assert packed.numel() == 0
    # projection of zero tokens
    x = torch.empty((0, 64), dtype=bf, device=dev)
    w = torch.zeros((256, 64), dtype=bf, device=dev)
    y = cam.qkv_projection_head_sharded(x, w, 2, 1, 4, 64)
    assert y.numel() == 0
    # planned relayout of an empty batch is rejected by the planner (no blocks)
    with pytest.raises(cam.CamError):
        cam.thd_plan([0], 2)
    torch.cuda.synchronize()
    assert torch.all(sentinel == 7.0)


def test_single_partial_and_single_head_per_rank(cam, orc):
    announce("P = 1 combine, H/P = 1 relayout, one-token batch")
    # one partial: the combine is the identity on valid rows
    po = synth.normal((1, 5, 2, 64), seed=1)
    pl = synth.partial_lse((1, 5, 2), seed=2)
    pl[0, 3, 1] = float("-inf")
    out, lse = cam.lse_combine(po.cuda(), pl.cuda())
    torch.cuda.synchronize()
    ro, rl = orc.lse_combine(synth.bits(po), pl.numpy())
    assert_bits_equal(to_host_bits(out), ro, "P = 1 combine")
    assert_lse_close(lse.cpu().numpy(), rl, "P = 1 lse")
    # one head per rank
    P, B, S, H, D = 4, 2, 8, 4, 16
    x = synth.relayout_seq_side(P, B, S, H, D, seed=3).cuda()
    y = cam.ulysses_seq_to_head(x, P)
    torch.cuda.synchronize()
    assert_bits_equal(to_host_bits(y), orc.seq_to_head(to_host_bits(x), P, B, S, H, D), "H/P = 1")
    # a batch of one token over 8 ranks (seven empty pieces)
    cu = synth.cu_seqlens([1])
    plan = cam.ulysses_varlen_plan(cu, 8)
    z = synth.normal((1, 8, 32), seed=4).cuda()
    zz = cam.ulysses_seq_to_head_varlen(z, plan, 1)
    torch.cuda.synchronize()
    assert_bits_equal(to_host_bits(zz), orc.varlen_seq_to_head(to_host_bits(z), cu, 8, 1, 8, 32), "one token")
    po = synth.normal((8, 1, 2, 64), seed=5)
    pl = synth.partial_lse((8, 1, 2), seed=6)
    out, lse = cam.lse_combine_varlen(po.cuda(), pl.cuda(), torch.from_numpy(cu).cuda())
    torch.cuda.synchronize()
    ro, rl = orc.lse_combine(synth.bits(po), pl.numpy(), cu=cu)
    assert_rows_close(orc.half_bits_to_double(to_host_bits(out)).reshape(-1, 64),
                      orc.half_bits_to_double(ro).reshape(-1, 64), "one-token combine")
    assert_lse_close(lse.cpu().numpy(), rl, "one-token lse")
