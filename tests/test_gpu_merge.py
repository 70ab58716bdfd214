"""GPU parity of the online two-way merge (ring / context-parallel
accumulation) against the oracle: one merge against the double combine of
the two inputs, and a ring of P hops against the one-shot combine of all P
partials (the combine is associative; pinned in test_oracle_lse)."""

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


@pytest.mark.parametrize("T,H,D,dt", [(37, 3, 64, "bf16"), (5, 8, 128, "fp16"), (64, 2, 512, "bf16"), (9, 4, 4, "bf16")])
def test_single_merge(cam, orc, T, H, D, dt):
    announce(f"merge T={T} H={H} D={D} {dt}")
    g = torch.Generator().manual_seed(T * 7 + D)
    acc = torch.randn((T, H, D), generator=g)
    acc_l = torch.randn((T, H), generator=g) * 2
    part = synth.normal((T, H, D), seed=T + D, dtype=dt)
    part_l = synth.partial_lse((T, H), seed=T + D + 1)
    # validity cases: empty accumulator, invalid partial, both invalid
    acc_l[1, :] = -np.inf
    acc[1, :] = float("nan")          # an empty accumulator's payload is ignored
    part_l[2, 0] = float("nan")
    part_l[3, :] = float("inf")
    acc_l[3, 1 % H] = -np.inf
    pb = synth.bits(part).copy()
    bad = ~np.isfinite(part_l.numpy())
    pb[bad] = 0x7FC1                  # an invalid partial's row is never read
    # oracle: the double combine of the two partials
    ref_o, ref_l = orc.combine_f64(np.stack([acc.double().numpy(), orc.half_bits_to_double(pb, dt)]).reshape(2, T * H, D),
                                   np.stack([acc_l.double().numpy(), part_l.double().numpy()]).reshape(2, T * H))
    a_d, al_d = acc.cuda(), acc_l.cuda()
    fin = torch.empty((T, H, D), dtype=part.dtype, device="cuda")
    cam.lse_merge(a_d, al_d, from_host_bits(pb, part.dtype), part_l.cuda(), out_final=fin)
    torch.cuda.synchronize()
    got = a_d.cpu().double().numpy().reshape(T * H, D)
    assert not np.isnan(got).any()
    num = np.max(np.abs(got - ref_o), axis=1)
    den = np.max(np.abs(ref_o), axis=1)
    assert np.all(num[den == 0] == 0) and np.max(num[den > 0] / den[den > 0]) <= 1e-5   # fp32 accumulator
    assert_lse_close(al_d.cpu().numpy(), ref_l, "merge lse")
    assert_rows_close(orc.half_bits_to_double(to_host_bits(fin), dt).reshape(-1, D), ref_o, "merge rounded payload")


@pytest.mark.parametrize("P,T,H,D", [(8, 300, 4, 128), (4, 64, 8, 64), (2, 33, 2, 512)])
def test_ring_of_merges_equals_one_shot_combine(cam, orc, P, T, H, D):
    announce(f"ring of {P} merges T={T} H={H} D={D}")
    po = synth.normal((P, T, H, D), seed=P * 100 + T)
    pl = synth.partial_lse((P, T, H), seed=P * 100 + T + 1)
    pl[P - 1, 5, 0] = -np.inf     # an invalid partial in the middle of a row
    pl[:, 7, :] = -np.inf         # a row with no valid partial
    pb = synth.bits(po).copy()
    pb[~np.isfinite(pl.numpy())] = 0xFFC0
    ro, rl = orc.lse_combine(pb, pl.numpy())
    acc = torch.full((T, H, D), float("nan"), device="cuda")
    acc_l = torch.full((T, H), float("-inf"), device="cuda")
    fin = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    pd, pld = from_host_bits(pb, torch.bfloat16), pl.cuda()
    for hop in range(P):   # the partial that arrives at this hop
        cam.lse_merge(acc, acc_l, pd[hop], pld[hop], out_final=fin if hop == P - 1 else None)
    torch.cuda.synchronize()
    assert_rows_close(orc.half_bits_to_double(to_host_bits(fin)).reshape(-1, D),
                      orc.half_bits_to_double(ro).reshape(-1, D), "ring result")
    err = assert_lse_close(acc_l.cpu().numpy(), rl, "ring lse")
    print(f"ring P={P} lse err {err:.2e}", flush=True)


def test_ring_full_thd_size(cam, orc):
    """The ring at the packed THD batch's full size (131072 tokens, H = 32,
    D = 128, 8 hops, fp32 accumulator; the shape the benchmark times): every
    final rounded row and LSE against the oracle's one-shot combine of the
    same 8 partials."""
    P, H, D = 8, 32, 128
    lens = synth.thd_lengths(20, 131072, seed=synth.BASE_SEED + 4)
    cu = synth.cu_seqlens(lens)
    T = int(cu[-1])
    announce("ring of 8 merges, full THD size, every row")
    g = synth._gen(synth.BASE_SEED + 78, "cuda")
    po = torch.randn((P, T, H, D), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    pl = torch.randn((P, T, H), generator=g, device="cuda", dtype=torch.float32).mul_(2.0)
    pl[3, 1000:1100, :] = float("-inf")   # a stretch where one hop brings nothing
    acc = torch.empty((T, H, D), device="cuda")
    acc_l = torch.full((T, H), float("-inf"), device="cuda")
    fin = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    for hop in range(P):
        cam.lse_merge(acc, acc_l, po[hop], pl[hop], out_final=fin if hop == P - 1 else None)
    torch.cuda.synchronize()
    del acc
    po_h, pl_h = to_host_bits(po), pl.cpu().numpy()
    fin_h, accl_h = to_host_bits(fin), acc_l.cpu().numpy()
    del po

    def check(a, e):
        ro, rl = orc.lse_combine(po_h[:, a:e], pl_h[:, a:e])
        w = assert_rows_close(orc.half_bits_to_double(fin_h[a:e]).reshape(-1, D),
                              orc.half_bits_to_double(ro).reshape(-1, D), f"ring rows [{a}, {e})")
        return w, assert_lse_close(accl_h[a:e], rl, f"ring lse [{a}, {e})")

    res = window_pool(T, check)
    print(f"ring of 8, all {T * H} rows: worst row {max(r[0] for r in res):.3e}, "
          f"lse err {max(r[1] for r in res):.3e}", flush=True)
