"""GPU parity of the max/sum-aware LSE pack and the stable LSE combine
against the oracle: packed O-region bit-exact, LSE within 1e-5 absolute with
identical -inf positions, combined payload within 8e-3 per-row relative
error; invalid partials never read; MLA decode and packed-THD workloads at
full size, every row (the THD oracle runs over token windows on the host's
cores)."""

import math

import numpy as np
import pytest
import torch

import synth
from helpers import (window_pool, announce, assert_bits_equal, assert_lse_close, assert_rows_close, from_host_bits,
                     to_host_bits)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cam():
    import context_attention_movement_amd as m
    m.library()
    assert torch.cuda.is_available()
    return m


def _pack_and_check(cam, orc, o, m, s, sd, tag):
    """o, m, s: host torch tensors (any strides).  Packs on the GPU and
    compares with the oracle's pack of the same values."""
    P, T, H, Dv = o.shape
    ob = synth.bits(o)
    packed_ref = orc.lse_pack(ob, m.contiguous().numpy(), s.contiguous().numpy(), sd)
    od, md, sdv = o.cuda(), m.cuda(), s.cuda()
    packed = cam.lse_pack(od, md, sdv, sd)
    torch.cuda.synchronize()
    got = to_host_bits(packed)
    O1, L1 = orc.packed_regions(packed_ref, P, T, H, Dv, sd)
    O2, L2 = orc.packed_regions(got, P, T, H, Dv, sd)
    assert_bits_equal(O2, O1, f"{tag}: packed O-region")
    err = assert_lse_close(L2, L1, f"{tag}: packed L-region")
    return packed_ref, packed, err


PACK = [  # (P, T, H, Dv, dtype)
    (2, 256, 8, 64, "bf16"),
    (8, 24, 16, 512, "bf16"),
    (4, 12, 8, 40, "fp16"),
    (3, 9, 6, 5, "bf16"),       # 10-byte rows: 2-byte accesses
    (1, 7, 3, 16, "bf16"),
]


@pytest.mark.parametrize("sd", [1, 0])
@pytest.mark.parametrize("case", PACK, ids=lambda c: "P{}T{}H{}Dv{}{}".format(*c))
def test_pack_bit_exact(cam, orc, case, sd):
    P, T, H, Dv, dt = case
    if sd == 0 and T % P:
        pytest.skip("T not divisible by P")
    announce(f"pack {case} scatter_dim={sd}")
    o, m, s, _ = synth.dcp_partials(P, T, H, Dv, seed=synth.FP16_SEED if dt == "fp16" else synth.BASE_SEED,
                                    dtype=dt, corrupt_frac=0.05)
    _pack_and_check(cam, orc, o, m, s, sd, f"pack {case}")


def test_pack_noncontiguous_and_specials(cam, orc):
    """Non-contiguous out / max / sum strides; every invalid-statistics kind;
    positive denormal sums stay valid."""
    P, T, H, Dv = 4, 16, 8, 64
    announce("pack strided + specials")
    o, m, s, _ = synth.dcp_partials(P, T, H, Dv, seed=99, corrupt_frac=0.25)
    s.view(-1)[:5] = torch.tensor([1e-45, 1e-40, 1.17e-38, 2e-44, 3e-39])
    m.view(-1)[:5] = torch.tensor([0.5, -3.0, 2.0, 0.0, 7.0])
    o_store = o.permute(0, 2, 1, 3).contiguous()          # [P][H][T][Dv]
    o_view = o_store.permute(0, 2, 1, 3)
    m_store = m.permute(2, 0, 1).contiguous()             # [H][P][T]
    s_store = s.permute(1, 2, 0).contiguous()             # [T][H][P]
    m_view = m_store.permute(1, 2, 0)
    s_view = s_store.permute(2, 0, 1)
    for sd in (0, 1):
        ref = orc.lse_pack(synth.bits(o), m.numpy(), s.numpy(), sd)
        od, md, sdv = o_store.cuda().permute(0, 2, 1, 3), m_store.cuda().permute(1, 2, 0), s_store.cuda().permute(2, 0, 1)
        assert not od.is_contiguous() and not md.is_contiguous()
        packed = cam.lse_pack(od, md, sdv, sd)
        torch.cuda.synchronize()
        O1, L1 = orc.packed_regions(ref, P, T, H, Dv, sd)
        O2, L2 = orc.packed_regions(to_host_bits(packed), P, T, H, Dv, sd)
        assert_bits_equal(O2, O1, "strided O-region")
        assert_lse_close(L2, L1, "strided L-region")
        assert np.isfinite(L2).sum() == np.isfinite(L1).sum()
    del o_view, m_view, s_view


def test_mla_pack_full_size(cam, orc):
    """MLA-style DCP decode: P = 8, T = 128, H = 128, Dv = 512, 1% corrupted
    statistics, scatter over heads."""
    P, T, H, Dv = 8, 128, 128, 512
    announce("MLA pack full size")
    o, m, s, idx = synth.dcp_partials(P, T, H, Dv, seed=synth.BASE_SEED + 3)
    assert idx.size == math.ceil(0.01 * P * T * H) == 1311
    _, _, err = _pack_and_check(cam, orc, o, m, s, 1, "MLA pack")
    print(f"MLA pack max LSE abs error {err:.3e}", flush=True)


def _combine_check(cam, orc, packed_ref, P, T, H, Dv, sd, dtype, tag):
    out_ref, lse_ref = orc.lse_combine_packed(packed_ref, P, T, H, Dv, sd, dtype=dtype)
    pk = torch.from_numpy(packed_ref).cuda()
    out, lse = cam.lse_combine_packed(pk, P, T, H, Dv, sd, dtype=torch.bfloat16 if dtype == "bf16" else torch.float16)
    torch.cuda.synchronize()
    got = orc.half_bits_to_double(to_host_bits(out), dtype)
    want = orc.half_bits_to_double(out_ref, dtype)
    worst = assert_rows_close(got, want, f"{tag}: combined payload")
    err = assert_lse_close(lse.cpu().numpy(), lse_ref, f"{tag}: lse_out")
    return worst, err


@pytest.mark.parametrize("sd", [1, 0])
@pytest.mark.parametrize("case", PACK, ids=lambda c: "P{}T{}H{}Dv{}{}".format(*c))
def test_combine_packed(cam, orc, case, sd):
    P, T, H, Dv, dt = case
    if sd == 0 and T % P:
        pytest.skip("T not divisible by P")
    announce(f"combine packed {case} scatter_dim={sd}")
    o, m, s, _ = synth.dcp_partials(P, T, H, Dv, seed=1234 + P, dtype=dt, corrupt_frac=0.1)
    packed_ref = orc.lse_pack(synth.bits(o), m.numpy(), s.numpy(), sd)
    _combine_check(cam, orc, packed_ref, P, T, H, Dv, sd, dt, f"combine {case}")


def test_mla_combine_full_size_poisoned(cam, orc):
    """MLA decode combine at full size; the O rows of invalid partials are
    overwritten with NaN in the packed buffer and must not leak."""
    P, T, H, Dv = 8, 128, 128, 512
    announce("MLA combine full size, poisoned invalid rows")
    o, m, s, _ = synth.dcp_partials(P, T, H, Dv, seed=synth.BASE_SEED + 3)
    ob = synth.bits(o).copy()
    mn, sn = m.numpy(), s.numpy()
    with np.errstate(invalid="ignore"):
        invalid = ~(np.isfinite(mn) & np.isfinite(sn) & (sn > 0))
    ob[invalid] = 0x7FC1  # NaN payload in every invalid partial row
    packed_ref = orc.lse_pack(ob, mn, sn, 1)
    worst, err = _combine_check(cam, orc, packed_ref, P, T, H, Dv, 1, "bf16", "MLA combine")
    print(f"MLA combine worst row rel err {worst:.3e}, lse err {err:.3e}", flush=True)


def test_pack_and_combine_beyond_4gib(cam, orc):
    """The MLA shape at T = 4096: the packed exchange buffer and the partials
    each exceed 2^32 bytes, so chunk, row and byte offsets pass 32 bits.  The
    whole O-region is compared bit for bit and every LSE with the oracle's;
    every combined row against the oracle's combine of its own packed buffer."""
    P, T, H, Dv = 8, 4096, 128, 512
    announce("pack and combine with buffers over 4 GiB")
    o, m, s, _ = synth.dcp_partials(P, T, H, Dv, seed=synth.BASE_SEED + 7, device="cuda")
    packed = cam.lse_pack(o, m, s, 1)
    out, lse = cam.lse_combine_packed(packed, P, T, H, Dv, 1)
    torch.cuda.synchronize()
    assert packed.numel() > 2**32 and o.numel() * 2 >= 2**32
    ob = to_host_bits(o)
    del o
    mh, sh = m.cpu().numpy(), s.cpu().numpy()
    ref = orc.lse_pack(ob, mh, sh, 1)
    got = to_host_bits(packed)
    del packed
    rows = orc.pack_rows(P, T, H, 1)
    chunk = orc.pack_chunk_bytes(P, T, H, Dv, 1)
    o_bytes = (rows * Dv * 2 + 15) // 16 * 16
    rc, gc = ref.reshape(P, P, chunk), got.reshape(P, P, chunk)
    for p in range(P):  # chunk by chunk, to keep the host temporaries small
        for r in range(P):
            assert np.array_equal(gc[p, r, :rows * Dv * 2], rc[p, r, :rows * Dv * 2]), f"O-region ({p}, {r})"
            assert_lse_close(gc[p, r, o_bytes:o_bytes + 4 * rows].view(np.float32),
                             rc[p, r, o_bytes:o_bytes + 4 * rows].view(np.float32), f"L-region ({p}, {r})")
    del got, gc
    out_ref, lse_ref = orc.lse_combine_packed(ref, P, T, H, Dv, 1)
    outh, lseh = to_host_bits(out), lse.cpu().numpy()
    worst = 0.0
    for r in range(P):
        sl = slice(r * rows, (r + 1) * rows)
        worst = max(worst, assert_rows_close(orc.half_bits_to_double(outh[sl]), orc.half_bits_to_double(out_ref[sl]),
                                             f"combine beyond 4 GiB, rank {r}"))
    err = assert_lse_close(lseh, lse_ref, "combine beyond 4 GiB: lse_out")
    print(f"beyond 4 GiB: worst row {worst:.3e}, lse err {err:.3e}", flush=True)


def test_combine_all_invalid_rows_and_p1(cam, orc):
    announce("combine all-invalid rows and P=1 identity")
    T, H, D = 33, 4, 64
    # P = 1: exact identity for valid rows, +0 / -inf for invalid ones
    o = synth.normal((1, T, H, D), seed=8)
    l = synth.partial_lse((1, T, H), seed=9)
    l[0, 3, 1] = -math.inf
    l[0, 5, 2] = math.nan
    out, lse = cam.lse_combine(o.cuda(), l.cuda())
    torch.cuda.synchronize()
    ob, lh = synth.bits(o)[0], l.numpy()[0]
    gb, gl = to_host_bits(out), lse.cpu().numpy()
    for t in range(T):
        for h in range(H):
            if np.isfinite(lh[t, h]):
                assert np.array_equal(gb[t, h], ob[t, h]) and gl[t, h] == lh[t, h]
            else:
                assert np.all(gb[t, h] == 0) and gl[t, h] == -np.inf
    # P = 4 with whole rows invalid (poisoned payload everywhere invalid)
    P = 4
    o = synth.normal((P, T, H, D), seed=10)
    l = synth.partial_lse((P, T, H), seed=11)
    l[:, 7, 0] = -math.inf
    l[:, 9, 3] = math.nan
    l[1:, 12, 2] = math.inf
    ob = synth.bits(o).copy()
    ob[~np.isfinite(l.numpy())] = 0xFFC0
    od = from_host_bits(ob, torch.bfloat16)
    out, lse = cam.lse_combine(od, l.cuda())
    torch.cuda.synchronize()
    ro, rl = orc.lse_combine(ob, l.numpy())
    assert_rows_close(orc.half_bits_to_double(to_host_bits(out)).reshape(-1, D),
                      orc.half_bits_to_double(ro).reshape(-1, D), "all-invalid rows")
    assert_lse_close(lse.cpu().numpy(), rl, "all-invalid lse")
    assert np.all(to_host_bits(out)[7, 0] == 0) and np.all(to_host_bits(out)[9, 3] == 0)


@pytest.mark.parametrize("P,T,H,D,dt", [(2, 100, 3, 8, "bf16"), (5, 64, 4, 128, "bf16"), (8, 37, 2, 24, "fp16"),
                                        (16, 20, 4, 64, "bf16"), (64, 9, 2, 16, "bf16"), (3, 50, 2, 5, "bf16"),
                                        (3, 21, 2, 300, "bf16"), (2, 10, 3, 1000, "fp16"), (8, 13, 5, 512, "bf16"),
                                        (33, 7, 3, 256, "bf16"), (64, 5, 3, 512, "bf16"), (64, 6, 2, 1024, "fp16")])
def test_combine_generic_strided(cam, orc, P, T, H, D, dt):
    announce(f"combine strided P={P} T={T} H={H} D={D} {dt}")
    o = synth.normal((P, H, T, D), seed=P * 100 + D, dtype=dt)          # stored [P][H][T][D]
    l = synth.partial_lse((T, P, H), seed=P * 100 + D + 1)              # stored [T][P][H]
    l[2, :, 0] = -math.inf
    l[4, 0, :] = math.nan
    ov = o.permute(0, 2, 1, 3)
    lv = l.permute(1, 0, 2)
    ro, rl = orc.lse_combine(synth.bits(ov.contiguous()), np.ascontiguousarray(lv.numpy()), dtype=dt)
    # output in a padded row pitch and a transposed LSE layout
    out_store = torch.zeros((T, H, D + 8), dtype=o.dtype, device="cuda")
    lse_store = torch.zeros((H, T), dtype=torch.float32, device="cuda")
    cam.lse_combine(o.cuda().permute(0, 2, 1, 3), l.cuda().permute(1, 0, 2), out=out_store[:, :, :D],
                    lse_out=lse_store.t())
    torch.cuda.synchronize()
    got = orc.half_bits_to_double(to_host_bits(out_store[:, :, :D]), dt)
    assert_rows_close(got.reshape(-1, D), orc.half_bits_to_double(ro, dt).reshape(-1, D), "strided combine")
    assert_lse_close(lse_store.t().cpu().numpy(), rl, "strided lse")
    assert torch.all(out_store[:, :, D:] == 0)


def test_combine_varlen_masked_partials_not_read(cam, orc):
    announce("varlen combine, causal masking")
    lengths, P, H, D = [5, 11, 2, 0, 7, 300, 64], 8, 4, 64
    cu = synth.cu_seqlens(lengths)
    T = int(cu[-1])
    o = synth.bits(synth.normal((P, T, H, D), seed=31)).copy()
    l = synth.partial_lse((P, T, H), seed=32).numpy().copy()
    mask = orc.causal_mask(cu, P)
    o[~mask] = 0x7FC0
    l[~mask] = np.nan
    l[0, 10, 1] = -np.inf   # an explicitly invalid admitted partial
    ro, rl = orc.lse_combine(o, l, cu=cu)
    out, lse = cam.lse_combine_varlen(from_host_bits(o, torch.bfloat16), torch.from_numpy(l).cuda(),
                                      torch.from_numpy(cu).cuda())
    torch.cuda.synchronize()
    assert_rows_close(orc.half_bits_to_double(to_host_bits(out)).reshape(-1, D),
                      orc.half_bits_to_double(ro).reshape(-1, D), "varlen combine")
    assert_lse_close(lse.cpu().numpy(), rl, "varlen lse")


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
def test_thd_combine_full_size(cam, orc, dt):
    """Packed THD at full size (131072 tokens, H = 32, D = 128, 8 KV-piece
    partials; bf16 is the launch the benchmark times): every row of the
    combined output and every LSE against the oracle, computed over token
    windows on the host's cores."""
    P, H, D = 8, 32, 128
    lens = synth.thd_lengths(20, 131072, seed=synth.BASE_SEED + 4)
    cu = synth.cu_seqlens(lens)
    T = int(cu[-1])
    announce(f"THD combine full size, every row, {dt}")
    g = synth._gen((synth.BASE_SEED if dt == "bf16" else synth.FP16_SEED) + 77, "cuda")
    tdt = torch.bfloat16 if dt == "bf16" else torch.float16
    po = torch.randn((P, T, H, D), generator=g, device="cuda", dtype=torch.float32).to(tdt)
    pl = torch.randn((P, T, H), generator=g, device="cuda", dtype=torch.float32).mul_(2.0)
    cu_d = torch.from_numpy(cu).cuda()
    out, lse = cam.lse_combine_varlen(po, pl, cu_d)
    torch.cuda.synchronize()
    po_h, pl_h = to_host_bits(po), pl.cpu().numpy()
    out_h, lse_h = to_host_bits(out), lse.cpu().numpy()
    del po

    def check(a, e):
        ro, rl = orc.lse_combine(po_h[:, a:e], pl_h[:, a:e], dtype=dt, cu=cu, t_begin=a)
        w = assert_rows_close(orc.half_bits_to_double(out_h[a:e], dt).reshape(-1, D),
                              orc.half_bits_to_double(ro, dt).reshape(-1, D), f"THD rows [{a}, {e})")
        return w, assert_lse_close(lse_h[a:e], rl, f"THD lse [{a}, {e})")

    res = window_pool(T, check)
    print(f"THD combine ({dt}), all {T * H} rows: worst row {max(r[0] for r in res):.3e}, "
          f"lse err {max(r[1] for r in res):.3e}", flush=True)


def test_mla_pack_and_combine_full_size_fp16(cam, orc):
    """The MLA decode shape with an fp16 producer (P = 8, T = 128, H = 128,
    Dv = 512, 1% corrupted statistics, the fp16 seed): the packed buffer bit
    for bit and its L-region within 1e-5, then the combine over the exchange
    within the payload bar, invalid rows NaN-poisoned."""
    P, T, H, Dv = 8, 128, 128, 512
    announce("MLA pack + combine full size, fp16")
    o, m, s, _ = synth.dcp_partials(P, T, H, Dv, seed=synth.FP16_SEED, dtype="fp16")
    packed_ref, _, err = _pack_and_check(cam, orc, o, m, s, 1, "MLA pack fp16")
    ob = synth.bits(o).copy()
    mn, sn = m.numpy(), s.numpy()
    with np.errstate(invalid="ignore"):
        invalid = ~(np.isfinite(mn) & np.isfinite(sn) & (sn > 0))
    ob[invalid] = 0x7E01  # fp16 NaN payload in every invalid partial row
    poisoned = orc.lse_pack(ob, mn, sn, 1)
    worst, lerr = _combine_check(cam, orc, poisoned, P, T, H, Dv, 1, "fp16", "MLA combine fp16")
    print(f"MLA fp16: pack LSE err {err:.3e}, combine worst row {worst:.3e}, lse err {lerr:.3e}", flush=True)
