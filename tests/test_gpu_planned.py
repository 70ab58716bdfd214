"""GPU parity of the relayout over THD layout plans against the oracle's
planned-span relayout, bit for bit: small ragged batches (2/4/8/16-byte
accesses, several rank counts and planes), the packed THD batch at full size
(every element), the round trip, and autograd (the gradient is the inverse
relayout).  The span tables come from the oracle's planner."""

import numpy as np
import pytest
import torch

import synth
from helpers import announce, assert_bits_equal, to_host_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cam():
    import context_attention_movement_amd as m
    m.library()
    assert torch.cuda.is_available()
    return m


def _plan_from_oracle(cam, orc, cu, W, **kw):
    q = orc.thd_plan(cu, W, **kw)
    plan = cam.ThdPlan(W, int(cu[-1]), np.asarray(cu, dtype=np.int32), q["span_start"], q["span_rank"],
                       q["span_local"], q["rank_off"], q["rank_cost"], q["grid"])
    return q, plan.to("cuda")


CASES = [  # (lengths in blocks, block size, W, B, H, D, dtype)
    ([3, 40, 1, 7, 90, 2], 4, 3, 1, 6, 64, torch.bfloat16),
    ([3, 40, 1, 7, 90, 2], 4, 4, 3, 8, 128, torch.bfloat16),
    ([0, 12, 5, 33, 1, 0, 64], 1, 8, 2, 16, 8, torch.float16),     # 16-byte runs of 8 elements x 2 heads
    ([6, 1, 1], 1, 2, 1, 4, 3, torch.bfloat16),                    # 6-byte runs: 2-byte accesses
    ([9, 27, 4], 2, 5, 2, 10, 2, torch.float32),                   # 8-byte runs, 5 ranks
    ([3, 40, 1, 7, 90, 2], 4, 4, 2, 16, 128, torch.bfloat16),      # 1 KB runs: the wave-uniform row map
    ([20, 1, 9], 8, 3, 1, 6, 256, torch.bfloat16),                 # 1 KB runs over 3 ranks
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"W{c[2]}B{c[3]}H{c[4]}D{c[5]}")
def test_span_relayout_bit_exact(cam, orc, case):
    lens, b, W, B, H, D, dt = case
    cu = synth.cu_seqlens([x * b for x in lens])
    T = int(cu[-1])
    announce(f"span relayout {case}")
    q, plan = _plan_from_oracle(cam, orc, cu, W, block_size=b, min_split_tokens=8 * b)
    x = synth.normal((B * T, H, D), seed=T + W, dtype={torch.bfloat16: "bf16", torch.float16: "fp16",
                                                         torch.float32: "fp32"}[dt])
    y = cam.ulysses_seq_to_head_spans(x.cuda(), plan, B)
    z = cam.ulysses_head_to_seq_spans(y, plan)
    torch.cuda.synchronize()
    want = orc.span_seq_to_head(synth.bits(x), q, W, B, H, D)
    assert_bits_equal(to_host_bits(y), want, "seq->head over spans")
    assert_bits_equal(to_host_bits(z), synth.bits(x), "round trip")
    w = synth.normal((W, B, T, H // W, D), seed=5 + T, dtype="fp32").to(dt)
    back = cam.ulysses_head_to_seq_spans(w.cuda(), plan)
    torch.cuda.synchronize()
    assert_bits_equal(to_host_bits(back), orc.span_head_to_seq(synth.bits(w), q, W, B, H, D), "head->seq over spans")


def test_planned_thd_full_size(cam, orc):
    """The packed THD batch (131072 tokens in 64-token blocks, H = 32, D = 128,
    Q/K/V planes) planned over 8 ranks: every element of both directions."""
    P, B, H, D = 8, 3, 32, 128
    lens = synth.thd_lengths(20, 131072, seed=synth.BASE_SEED + 4, align=64)
    cu = synth.cu_seqlens(lens)
    T = int(cu[-1])
    announce("planned THD relayout full size")
    q, plan = _plan_from_oracle(cam, orc, cu, P, block_size=64, min_split_tokens=8192)
    assert q["grid"] > 0
    g = synth._gen(synth.BASE_SEED + 90, "cuda")
    x = torch.randn((B * T, H, D), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    y = cam.ulysses_seq_to_head_spans(x, plan, B)
    torch.cuda.synchronize()
    xb = to_host_bits(x)
    assert_bits_equal(to_host_bits(y), orc.span_seq_to_head(xb, q, P, B, H, D), "planned THD seq->head")
    z = cam.ulysses_head_to_seq_spans(y, plan)
    torch.cuda.synchronize()
    assert_bits_equal(to_host_bits(z), xb, "planned THD round trip")


def test_planned_relayout_autograd(cam, orc):
    from context_attention_movement_amd import autograd as ag
    W, B, H, D = 4, 2, 8, 64
    cu = synth.cu_seqlens([16 * x for x in (3, 20, 1, 9, 30)])
    T = int(cu[-1])
    announce("planned relayout autograd")
    q, plan = _plan_from_oracle(cam, orc, cu, W, block_size=16, min_split_tokens=128)
    x = synth.normal((B * T, H, D), seed=31).cuda().requires_grad_(True)
    y = synth.normal((W, B, T, H // W, D), seed=32).cuda().requires_grad_(True)
    dx = synth.normal((W, B, T, H // W, D), seed=33)
    dy = synth.normal((B * T, H, D), seed=34)
    gx, gy = torch.autograd.grad((ag.seq_to_head_spans(x, plan, B), ag.head_to_seq_spans(y, plan)), (x, y),
                                 (dx.cuda(), dy.cuda()))
    torch.cuda.synchronize()
    assert_bits_equal(to_host_bits(gx), orc.span_head_to_seq(synth.bits(dx), q, W, B, H, D), "grad of s2h")
    assert_bits_equal(to_host_bits(gy), orc.span_seq_to_head(synth.bits(dy), q, W, B, H, D), "grad of h2s")
