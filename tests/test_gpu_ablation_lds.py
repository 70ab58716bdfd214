"""GPU parity of the LDS-staged seq->head kernel (kept to measure the choice
of direct 16-byte moves for the relayout against staging whole sequence-side
rows in LDS): bit-exact against the oracle, with tiles that end inside a slab,
several rows per tile, and the full video-DiT P = 4 shape; its rejections."""

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


CASES = [  # (P, B, S, H, D, rows_per_tile)
    (2, 3, 256, 8, 64, 4),
    (4, 2, 4 * 37, 8, 64, 5),      # 37 rows per slab: the last tile holds 2 rows
    (3, 1, 3 * 50, 6, 32, 1),      # one row per tile
    (8, 1, 8 * 9, 16, 128, 8),     # 9 rows per slab, 8 rows per tile
    (1, 2, 100, 4, 64, 7),         # P = 1
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "P{}B{}S{}H{}D{}R{}".format(*c))
def test_lds_staged_seq_to_head_bit_exact(cam, orc, case):
    P, B, S, H, D, R = case
    announce(f"LDS-staged seq->head {case}")
    x = synth.relayout_seq_side(P, B, S, H, D, seed=synth.BASE_SEED + S + R).cuda()
    y = cam.ablation_seq_to_head_lds(x, P, R)
    torch.cuda.synchronize()
    assert_bits_equal(to_host_bits(y), orc.seq_to_head(to_host_bits(x), P, B, S, H, D), "LDS-staged seq->head")


def test_lds_staged_seq_to_head_video_p4_full(cam, orc):
    """The video DiT P = 4 Q/K/V operand [4][3][8190][24][128] bf16, every
    element, at the rows-per-tile setting the benchmark times (4)."""
    P, B, S, H, D = 4, 3, 32760, 24, 128
    announce("LDS-staged seq->head, video P=4 full size")
    g = synth._gen(synth.BASE_SEED + 55, "cuda")
    x = torch.randn((P, B, S // P, H, D), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    y = cam.ablation_seq_to_head_lds(x, P, 4)
    ref = cam.ulysses_seq_to_head(x, P)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), "LDS-staged kernel differs from the direct one"
    xh = to_host_bits(x)
    want = orc.seq_to_head(xh, P, B, S, H, D)
    assert_bits_equal(to_host_bits(y), want, "LDS-staged seq->head, video P=4")


def test_lds_staged_rejections(cam):
    x = torch.zeros((2, 1, 4, 4, 5), dtype=torch.bfloat16, device="cuda")   # 10-byte runs
    with pytest.raises(cam.CamError, match="ALIGNMENT"):
        cam.ablation_seq_to_head_lds(x, 2, 2)
    x = torch.zeros((2, 1, 4, 4, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(cam.CamError, match="UNSUPPORTED"):
        cam.ablation_seq_to_head_lds(x, 2, 0)
    with pytest.raises(cam.CamError, match="UNSUPPORTED"):
        cam.ablation_seq_to_head_lds(x, 2, 1000)   # 1000 rows of 512 bytes: beyond 64 KiB
