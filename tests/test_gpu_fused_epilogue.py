"""GPU parity of the combine that writes the sequence-sharded layout directly
(the combine fused with the head->seq relayout of its result) against the
oracle's composition of the two: packed exchange with token-major output,
and the causal varlen combine with rank-major (sequence-sharded) output."""

import math

import numpy as np
import pytest
import torch

import synth
from helpers import window_pool, announce, assert_lse_close, assert_rows_close, from_host_bits, to_host_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cam():
    import context_attention_movement_amd as m
    m.library()
    assert torch.cuda.is_available()
    return m


CASES = [(2, 256, 8, 64, "bf16"), (8, 24, 16, 512, "bf16"), (4, 12, 8, 40, "fp16"), (3, 9, 6, 5, "bf16"),
         (8, 128, 128, 512, "bf16")]


@pytest.mark.parametrize("sd", [1, 0])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "P{}T{}H{}Dv{}{}".format(*c))
def test_packed_seq_output(cam, orc, case, sd):
    P, T, H, Dv, dt = case
    if sd == 0 and T % P:
        pytest.skip("T not divisible by P")
    announce(f"combine packed -> token-major {case} scatter_dim={sd}")
    o, m, s, _ = synth.dcp_partials(P, T, H, Dv, seed=4321 + P, dtype=dt, corrupt_frac=0.05)
    ob = synth.bits(o).copy()
    mn, sn = m.numpy(), s.numpy()
    with np.errstate(invalid="ignore"):
        ob[~(np.isfinite(mn) & np.isfinite(sn) & (sn > 0))] = 0x7FC3  # invalid rows must not be read
    if T * H >= 8:
        sn[:, 1, :] = -1.0  # whole token invalid on every rank
    packed = orc.lse_pack(ob, mn, sn, sd)
    ro, rl = orc.lse_combine_packed_seq(packed, P, T, H, Dv, sd, dtype=dt)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float16
    out, lse = cam.lse_combine_packed_seq(torch.from_numpy(packed).cuda(), P, T, H, Dv, sd, dtype=tdt)
    torch.cuda.synchronize()
    assert_rows_close(orc.half_bits_to_double(to_host_bits(out), dt).reshape(-1, Dv),
                      orc.half_bits_to_double(ro, dt).reshape(-1, Dv), "token-major combine")
    assert_lse_close(lse.cpu().numpy(), rl, "token-major lse")


VARLEN = [([5, 11, 2, 0, 7, 300, 64], 8, 4, 64), ([1, 2, 3], 4, 2, 128), ([1000, 999, 3], 4, 3, 16), ([40], 2, 8, 8)]


@pytest.mark.parametrize("case", VARLEN, ids=lambda c: f"n{len(c[0])}P{c[1]}H{c[2]}D{c[3]}")
def test_varlen_seq_output(cam, orc, case):
    lengths, P, H, D = case
    announce(f"varlen combine -> rank-major {case}")
    cu = synth.cu_seqlens(lengths)
    T = int(cu[-1])
    o = synth.bits(synth.normal((P, T, H, D), seed=91)).copy()
    l = synth.partial_lse((P, T, H), seed=92).numpy().copy()
    mask = orc.causal_mask(cu, P)
    o[~mask] = 0x7FC0
    l[~mask] = np.nan
    ro, rl = orc.lse_combine_varlen_seq(o, l, cu)
    plan = cam.ulysses_varlen_plan(cu, P)
    out, lse = cam.lse_combine_varlen_seq(from_host_bits(o, torch.bfloat16), torch.from_numpy(l).cuda(), plan)
    torch.cuda.synchronize()
    assert_rows_close(orc.half_bits_to_double(to_host_bits(out)).reshape(-1, D),
                      orc.half_bits_to_double(ro).reshape(-1, D), "rank-major combine")
    assert_lse_close(lse.cpu().numpy(), rl, "rank-major lse")


def test_varlen_seq_full_size(cam, orc):
    """Packed THD at full size, combined straight into the rank-major
    (sequence-sharded) rows: every token row is written exactly once (the
    output starts as NaN) and every row and LSE equals the oracle's combine
    placed by the oracle's row map."""
    P, H, D = 8, 32, 128
    lens = synth.thd_lengths(20, 131072, seed=synth.BASE_SEED + 4)
    cu = synth.cu_seqlens(lens)
    T = int(cu[-1])
    announce("THD combine -> rank-major, full size, every row")
    g = synth._gen(synth.BASE_SEED + 78, "cuda")
    po = torch.randn((P, T, H, D), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    pl = torch.randn((P, T, H), generator=g, device="cuda", dtype=torch.float32).mul_(2.0)
    plan = cam.ulysses_varlen_plan(cu, P)
    out = torch.full((T, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    cam.lse_combine_varlen_seq(po, pl, plan, out=out, lse_out=lse)
    torch.cuda.synchronize()
    rows = orc.varlen_token_rows(cu, P)
    assert np.array_equal(np.sort(rows), np.arange(T)), "the oracle's row map is a permutation"
    po_h, pl_h = to_host_bits(po), pl.cpu().numpy()
    out_h, lse_h = to_host_bits(out), lse.cpu().numpy()
    del po

    def check(a, e):
        ro, rl = orc.lse_combine(po_h[:, a:e], pl_h[:, a:e], cu=cu, t_begin=a)
        got = out_h[rows[a:e]]
        w = assert_rows_close(orc.half_bits_to_double(got).reshape(-1, D), orc.half_bits_to_double(ro).reshape(-1, D),
                              f"THD rank-major rows of tokens [{a}, {e})")
        return w, assert_lse_close(lse_h[rows[a:e]], rl, f"THD rank-major lse of tokens [{a}, {e})")

    res = window_pool(T, check)
    print(f"THD rank-major combine, all {T * H} rows: worst row {max(r[0] for r in res):.3e}, "
          f"lse err {max(r[1] for r in res):.3e}", flush=True)
