"""GPU parity of the Ulysses relayouts (dense and cu_seqlens varlen) against
the oracle: bit-exact, every element, at tiny and ragged multi-tile sizes and
at the full video-DiT and packed-THD workload sizes."""

import numpy as np
import pytest
import torch

import synth
from helpers import announce, assert_bits_equal, from_host_bits, to_host_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cam():
    import context_attention_movement_amd as m
    m.library()
    assert torch.cuda.is_available()
    return m


DENSE = [  # (P, B, S, H, D, dtype)
    (2, 3, 256, 8, 64, torch.bfloat16),        # tiny check shape, Q/K/V planes
    (1, 2, 40, 3, 16, torch.bfloat16),         # P = 1: plain copy
    (3, 2, 3 * 1111, 6, 40, torch.bfloat16),   # ragged slab tail, 160-byte runs
    (4, 1, 4 * 777, 4, 13, torch.float16),     # odd D: 2-byte accesses
    (4, 3, 4 * 301, 8, 6, torch.bfloat16),     # 24-byte runs: 8-byte accesses
    (8, 1, 8 * 129, 8, 128, torch.bfloat16),   # H/P = 1
    (2, 2, 2 * 2000, 4, 64, torch.float32),    # 4-byte payload
]


@pytest.mark.parametrize("case", DENSE, ids=lambda c: "P{}B{}S{}H{}D{}{}".format(*c[:5], str(c[5])[6:]))
def test_dense_relayout_bit_exact(cam, orc, case):
    P, B, S, H, D, dt = case
    announce(f"dense relayout {case}")
    if dt == torch.float32:
        x_host = synth.iota32(B * S * H * D).reshape(P, B, S // P, H, D)
        x = from_host_bits(x_host, torch.float32)
    else:
        x = synth.relayout_seq_side(P, B, S, H, D, seed=synth.BASE_SEED + S,
                                    dtype="bf16" if dt == torch.bfloat16 else "fp16").cuda()
        x_host = to_host_bits(x)
    y = cam.ulysses_seq_to_head(x, P)
    torch.cuda.synchronize()
    want = orc.seq_to_head(x_host, P, B, S, H, D)
    assert_bits_equal(to_host_bits(y), want, "seq->head")
    z = cam.ulysses_head_to_seq(y, P)
    torch.cuda.synchronize()
    assert_bits_equal(to_host_bits(z), x_host, "round trip")
    # inverse direction on an independent head-sharded operand
    h = synth.relayout_head_side(P, B, S, H, D, seed=7, dtype="bf16").cuda() if dt != torch.float32 else \
        from_host_bits(synth.iota32(B * S * H * D).reshape(P, B, S, H // P, D), torch.float32)
    s = cam.ulysses_head_to_seq(h, P)
    torch.cuda.synchronize()
    assert_bits_equal(to_host_bits(s), orc.head_to_seq(to_host_bits(h), P, B, S, H, D), "head->seq")


def test_dense_relayout_misaligned_views(cam, orc):
    """Sub-views whose base is only 2-byte aligned take the narrow access path."""
    P, B, S, H, D = 2, 1, 64, 4, 16
    announce("dense relayout misaligned base")
    buf = synth.normal((B * S * H * D + 1,), seed=3).cuda()
    x = buf[1:].view(P, B, S // P, H, D)
    out_buf = torch.empty(B * S * H * D + 3, dtype=torch.bfloat16, device="cuda")
    y = out_buf[3:].view(P, B, S, H // P, D)
    cam.ulysses_seq_to_head(x, P, out=y)
    torch.cuda.synchronize()
    assert_bits_equal(to_host_bits(y), orc.seq_to_head(to_host_bits(x), P, B, S, H, D), "misaligned")


@pytest.mark.parametrize("P,S,H,B", [(4, 32760, 24, 3), (4, 32760, 24, 1), (8, 75600, 48, 3), (8, 75600, 48, 1)])
def test_video_dit_full_size(cam, orc, P, S, H, B):
    """The video-DiT operands at full size: Q/K/V (B = 3) seq->head and the
    attention output (B = 1) head->seq, every element compared."""
    D = 128
    announce(f"video DiT P={P} S={S} H={H} B={B}")
    g = synth._gen(synth.BASE_SEED + P, "cuda")
    if B == 3:
        x = torch.randn((P, B, S // P, H, D), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
        y = cam.ulysses_seq_to_head(x, P)
        torch.cuda.synchronize()
        want = orc.seq_to_head(to_host_bits(x), P, B, S, H, D)
    else:
        x = torch.randn((P, B, S, H // P, D), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
        y = cam.ulysses_head_to_seq(x, P)
        torch.cuda.synchronize()
        want = orc.head_to_seq(to_host_bits(x), P, B, S, H, D)
    assert_bits_equal(to_host_bits(y), want, f"video P={P} B={B}")


VARLEN = [  # (lengths, P, B, H, D, dtype)
    ([7], 2, 1, 4, 64, torch.bfloat16),
    ([5, 0, 9, 1, 3, 0], 3, 2, 3, 16, torch.bfloat16),           # empty and sub-P sequences
    ([300, 1, 2, 3, 513, 1000], 4, 3, 8, 40, torch.bfloat16),
    (list(range(1, 60)), 8, 1, 8, 7, torch.float16),              # odd D, many tiny sequences
    ([4096, 17, 2048, 333], 8, 2, 32, 128, torch.bfloat16),
    ([1000, 999], 4, 1, 4, 32, torch.float32),
    # rows of a multiple of 64 16-byte vectors: the wave-uniform row-map kernel
    ([1, 2, 3, 129, 64, 700, 0], 2, 3, 4, 256, torch.bfloat16),   # 1 KB runs, sub-P and empty sequences
    ([5, 1000, 0, 33], 2, 1, 16, 128, torch.bfloat16),            # 2 KB runs
    ([77, 3, 500], 4, 2, 8, 128, torch.float32),                  # 1 KB runs of 4-byte elements
]


@pytest.mark.parametrize("case", VARLEN, ids=lambda c: f"n{len(c[0])}P{c[1]}B{c[2]}H{c[3]}D{c[4]}")
def test_varlen_relayout_bit_exact(cam, orc, case):
    lengths, P, B, H, D, dt = case
    announce(f"varlen relayout {case[1:]} nseq={len(lengths)}")
    cu = synth.cu_seqlens(lengths)
    T = int(cu[-1])
    plan = cam.ulysses_varlen_plan(cu, P)
    if dt == torch.float32:
        x = from_host_bits(synth.iota32(B * T * H * D).reshape(B * T, H, D), torch.float32)
    else:
        x = synth.normal((B * T, H, D), seed=11 + T, dtype="bf16" if dt == torch.bfloat16 else "fp16").cuda()
    y = cam.ulysses_seq_to_head_varlen(x, plan, B)
    torch.cuda.synchronize()
    xh = to_host_bits(x)
    assert_bits_equal(to_host_bits(y), orc.varlen_seq_to_head(xh, cu, P, B, H, D), "varlen seq->head")
    z = cam.ulysses_head_to_seq_varlen(y, plan)
    torch.cuda.synchronize()
    assert_bits_equal(to_host_bits(z), xh, "varlen round trip")


def test_varlen_single_sequence_matches_dense(cam):
    P, B, T, H, D = 4, 3, 4 * 500, 8, 64
    announce("varlen nseq=1 vs dense")
    x = synth.relayout_seq_side(P, B, T, H, D, seed=5).cuda()
    dense = cam.ulysses_seq_to_head(x, P)
    plan = cam.ulysses_varlen_plan([0, T], P)
    var = cam.ulysses_seq_to_head_varlen(x.view(B * T, H, D), plan, B)
    torch.cuda.synchronize()
    assert torch.equal(dense.view(torch.int16), var.view(torch.int16))


@pytest.mark.parametrize("B", [3, 1])
def test_thd_full_size(cam, orc, B):
    """Packed THD: 20 short sequences plus 2 long ones, 131072 tokens, H = 32,
    D = 128, P = 8; Q/K/V (B = 3) seq->head and O (B = 1) head->seq."""
    P, H, D = 8, 32, 128
    lens = synth.thd_lengths(20, 131072, seed=synth.BASE_SEED + 4)
    cu = synth.cu_seqlens(lens)
    T = int(cu[-1])
    announce(f"THD full size B={B}")
    plan = cam.ulysses_varlen_plan(cu, P)
    g = synth._gen(synth.BASE_SEED + 40 + B, "cuda")
    if B == 3:
        x = torch.randn((B * T, H, D), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
        y = cam.ulysses_seq_to_head_varlen(x, plan, B)
        torch.cuda.synchronize()
        want = orc.varlen_seq_to_head(to_host_bits(x), cu, P, B, H, D)
    else:
        x = torch.randn((P, B, T, H // P, D), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
        y = cam.ulysses_head_to_seq_varlen(x, plan)
        torch.cuda.synchronize()
        want = orc.varlen_head_to_seq(to_host_bits(x), cu, P, B, H, D)
    assert_bits_equal(to_host_bits(y), want, f"THD B={B}")


def test_copy_kernel(cam):
    announce("copy kernel")
    x = synth.normal((3, 1000, 8, 64), seed=1).cuda()
    y = torch.empty_like(x)
    cam.copy(x, y)
    torch.cuda.synchronize()
    assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_empty_inputs(cam):
    announce("empty inputs")
    x = torch.empty((2, 0, 4, 8, 16), dtype=torch.bfloat16, device="cuda")
    assert cam.ulysses_seq_to_head(x, 2).numel() == 0
    plan = cam.ulysses_varlen_plan([0], 2)
    y = torch.empty((0, 4, 8), dtype=torch.bfloat16, device="cuda")
    assert cam.ulysses_seq_to_head_varlen(y, plan, 1).numel() == 0


def test_host_plan_rejected_before_launch(cam):
    # a plan built with its tables on the host is refused for device data
    # (the check runs in the binding; no kernel is launched)
    announce("host plan with device data")
    T, H, D, P = 64, 8, 16, 2
    plan = cam.ulysses_varlen_plan([0, 20, T], P, device="cpu")
    x = torch.zeros((T, H, D), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="the plan's tables are on cpu"):
        cam.ulysses_seq_to_head_varlen(x, plan, 1)
    po = torch.zeros((P, T, H, D), dtype=torch.bfloat16, device="cuda")
    pl = torch.zeros((P, T, H), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="the plan's tables are on cpu"):
        cam.lse_combine_varlen_seq(po, pl, plan)
