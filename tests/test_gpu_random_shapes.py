"""Seeded random shapes against the oracle, to reach tile tails, access
widths and rank counts the hand-picked cases do not: dense relayouts (both
directions, every element, bf16/fp16/fp32 bits), varlen relayouts over
ragged batches with empty sequences, the generic strided combine with
invalid partials, the causal varlen combine, merges, the pack and the
combine over the exchange, the combine over random THD plans, and the
combine's gradient under each admission rule.  Each case is printed before
it runs."""

import numpy as np
import pytest
import torch

import synth
from helpers import announce, assert_bits_equal, assert_lse_close, assert_rows_close, from_host_bits, to_host_bits

pytestmark = pytest.mark.gpu

N_CASES = 24


@pytest.fixture(scope="module")
def cam():
    import context_attention_movement_amd as m
    m.library()
    assert torch.cuda.is_available()
    return m


def _bits(rng, shape, itemsize):
    if itemsize == 2:
        return rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
    return rng.integers(0, 1 << 32, size=shape, dtype=np.uint32)


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_dense_relayout(cam, orc, case):
    rng = np.random.default_rng(9000 + case)
    P = int(rng.integers(1, 9))
    B = int(rng.integers(1, 4))
    Sp = int(rng.integers(1, 40))
    H = P * int(rng.integers(1, 5))
    D = int(rng.choice([1, 3, 8, 24, 64, 100, 128, 136]))
    itemsize = int(rng.choice([2, 4]))
    S = Sp * P
    announce(f"random dense relayout #{case}: P={P} B={B} S={S} H={H} D={D} bytes/elem={itemsize}")
    x = _bits(rng, (P, B, Sp, H, D), itemsize)
    tdt = torch.bfloat16 if itemsize == 2 else torch.float32   # bits only: the relayout does no arithmetic
    xd = torch.from_numpy(x.view(np.int16 if itemsize == 2 else np.float32)).cuda().view(tdt)
    y = cam.ulysses_seq_to_head(xd, P)
    back = cam.ulysses_head_to_seq(y, P)
    torch.cuda.synchronize()
    want = orc.seq_to_head(x, P, B, S, H, D)
    ibits = torch.int16 if itemsize == 2 else torch.int32
    got = y.view(ibits).cpu().numpy().view(x.dtype)
    assert_bits_equal(got, want, "seq->head")
    assert_bits_equal(back.view(ibits).cpu().numpy().view(x.dtype), x, "head->seq round trip")


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_varlen_relayout(cam, orc, case):
    rng = np.random.default_rng(9100 + case)
    P = int(rng.integers(1, 9))
    B = int(rng.integers(1, 4))
    H = P * int(rng.integers(1, 4))
    D = int(rng.choice([2, 8, 40, 64, 128]))
    nseq = int(rng.integers(1, 12))
    lens = [int(v) for v in rng.integers(0, 60, size=nseq)]
    if sum(lens) == 0:
        lens[0] = 1
    cu = synth.cu_seqlens(lens)
    T = int(cu[-1])
    announce(f"random varlen relayout #{case}: P={P} B={B} H={H} D={D} lens={lens}")
    x = _bits(rng, (B * T, H, D), 2)
    plan = cam.ulysses_varlen_plan(cu, P)
    xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    y = cam.ulysses_seq_to_head_varlen(xd, plan, B)
    back = cam.ulysses_head_to_seq_varlen(y, plan)
    torch.cuda.synchronize()
    assert_bits_equal(y.view(torch.int16).cpu().numpy().view(np.uint16),
                      orc.varlen_seq_to_head(x, cu, P, B, H, D), "varlen seq->head")
    assert_bits_equal(back.view(torch.int16).cpu().numpy().view(np.uint16), x, "varlen round trip")


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_combine(cam, orc, case):
    rng = np.random.default_rng(9200 + case)
    P = int(rng.integers(1, 17))
    T = int(rng.integers(1, 40))
    H = int(rng.integers(1, 6))
    D = int(rng.choice([1, 5, 8, 64, 128, 200, 512, 600]))
    dt = str(rng.choice(["bf16", "fp16"]))
    varlen = bool(rng.integers(0, 2))
    announce(f"random combine #{case}: P={P} T={T} H={H} D={D} {dt} varlen={varlen}")
    o = synth.normal((P, T, H, D), seed=9300 + case, dtype=dt)
    l = synth.partial_lse((P, T, H), seed=9400 + case).numpy().copy()
    bad = rng.random((P, T, H)) < 0.15
    l[bad] = rng.choice([-np.inf, np.inf, np.nan], size=int(bad.sum()))
    ob = synth.bits(o).copy()
    cu = None
    if varlen:
        cuts = np.sort(rng.choice(np.arange(1, T), size=min(3, T - 1), replace=False)) if T > 1 else np.array([], int)
        cu = np.concatenate([[0], cuts, [T]]).astype(np.int32)
        mask = orc.causal_mask(cu, P)
        ob[~mask] = 0x7FC0 if dt == "bf16" else 0x7E00
        l[~mask] = np.nan
    ob[~np.isfinite(l)] = 0x7FC0 if dt == "bf16" else 0x7E00   # invalid partials' rows are never read
    ro, rl = orc.lse_combine(ob, l, dtype=dt, cu=cu)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float16
    od, ld = from_host_bits(ob, tdt), torch.from_numpy(l).cuda()
    if varlen:
        out, lse = cam.lse_combine_varlen(od, ld, torch.from_numpy(cu).cuda())
    else:
        out, lse = cam.lse_combine(od, ld)
    torch.cuda.synchronize()
    assert_rows_close(orc.half_bits_to_double(to_host_bits(out), dt).reshape(-1, D),
                      orc.half_bits_to_double(ro, dt).reshape(-1, D), "random combine")
    assert_lse_close(lse.cpu().numpy(), rl, "random combine lse")


@pytest.mark.parametrize("case", range(8))
def test_random_merge(cam, orc, case):
    rng = np.random.default_rng(9500 + case)
    T = int(rng.integers(1, 30))
    H = int(rng.integers(1, 5))
    D = int(rng.choice([4, 8, 64, 128, 256, 516]))
    announce(f"random merge #{case}: T={T} H={H} D={D}")
    acc = rng.standard_normal((T, H, D)).astype(np.float32)
    acc_l = (rng.standard_normal((T, H)) * 2).astype(np.float32)
    acc_l[rng.random((T, H)) < 0.2] = -np.inf
    part = synth.normal((T, H, D), seed=9600 + case)
    part_l = synth.partial_lse((T, H), seed=9700 + case).numpy().copy()
    part_l[rng.random((T, H)) < 0.2] = np.nan
    pb = synth.bits(part).copy()
    pb[~np.isfinite(part_l)] = 0x7FC1
    acc_in = acc.copy()
    acc_in[~np.isfinite(acc_l)] = np.nan   # an empty accumulator's payload is ignored
    ref_o, ref_l = orc.combine_f64(np.stack([acc.astype(np.float64), orc.half_bits_to_double(pb)]).reshape(2, T * H, D),
                                   np.stack([acc_l.astype(np.float64), part_l.astype(np.float64)]).reshape(2, T * H))
    a_d, al_d = torch.from_numpy(acc_in).cuda(), torch.from_numpy(acc_l).cuda()
    cam.lse_merge(a_d, al_d, from_host_bits(pb, torch.bfloat16), torch.from_numpy(part_l).cuda())
    torch.cuda.synchronize()
    got = a_d.cpu().double().numpy().reshape(T * H, D)
    assert not np.isnan(got).any()
    num = np.max(np.abs(got - ref_o), axis=1)
    den = np.max(np.abs(ref_o), axis=1)
    assert np.all(num[den == 0] == 0) and (np.max(num[den > 0] / den[den > 0]) if (den > 0).any() else 0) <= 1e-5
    assert_lse_close(al_d.cpu().numpy(), ref_l, "random merge lse")


@pytest.mark.parametrize("case", range(16))
def test_random_pack_and_packed_combine(cam, orc, case):
    rng = np.random.default_rng(9800 + case)
    P = int(rng.integers(1, 9))
    sd = int(rng.integers(0, 2))
    T = P * int(rng.integers(1, 9)) if sd == 0 else int(rng.integers(1, 30))
    H = P * int(rng.integers(1, 4)) if sd == 1 else int(rng.integers(1, 6))
    Dv = int(rng.choice([1, 4, 8, 40, 64, 128, 512]))
    dt = str(rng.choice(["bf16", "fp16"]))
    announce(f"random pack + combine #{case}: P={P} T={T} H={H} Dv={Dv} scatter_dim={sd} {dt}")
    o, m, s, _ = synth.dcp_partials(P, T, H, Dv, seed=9900 + case, dtype=dt, corrupt_frac=0.2)
    ref = orc.lse_pack(synth.bits(o), m.numpy(), s.numpy(), sd)
    packed = cam.lse_pack(o.cuda(), m.cuda(), s.cuda(), sd)
    torch.cuda.synchronize()
    O1, L1 = orc.packed_regions(ref, P, T, H, Dv, sd)
    O2, L2 = orc.packed_regions(to_host_bits(packed), P, T, H, Dv, sd)
    assert_bits_equal(O2, O1, "packed O-region")
    assert_lse_close(L2, L1, "packed L-region")
    ro, rl = orc.lse_combine_packed(ref, P, T, H, Dv, sd, dtype=dt)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float16
    out, lse = cam.lse_combine_packed(torch.from_numpy(ref).cuda(), P, T, H, Dv, sd, dtype=tdt)
    torch.cuda.synchronize()
    assert_rows_close(orc.half_bits_to_double(to_host_bits(out), dt).reshape(-1, Dv),
                      orc.half_bits_to_double(ro, dt).reshape(-1, Dv), "packed combine")
    assert_lse_close(lse.cpu().numpy(), rl, "packed combine lse")


@pytest.mark.parametrize("case", range(16))
def test_random_planned_combine(cam, orc, case):
    rng = np.random.default_rng(10000 + case)
    W = int(rng.integers(1, 9))
    b = int(rng.choice([1, 2, 4]))
    nseq = int(rng.integers(1, 8))
    blocks = [int(v) for v in rng.integers(0, 40, size=nseq)]
    while sum(blocks) < W:              # the planner needs at least one block per rank
        blocks[int(rng.integers(0, nseq))] += 1
    H = int(rng.integers(1, 5))
    D = int(rng.choice([8, 64, 128, 512]))
    cu = synth.cu_seqlens([x * b for x in blocks])
    T = int(cu[-1])
    announce(f"random planned combine #{case}: W={W} block={b} blocks={blocks} H={H} D={D}")
    q = orc.thd_plan(cu, W, block_size=b, min_split_tokens=8 * b)
    plan = cam.ThdPlan(W, T, cu, q["span_start"], q["span_rank"], q["span_local"], q["rank_off"],
                       q["rank_cost"], q["grid"]).to("cuda")
    first = orc.plan_first_positions(cu, q, W)
    mask = orc.plan_mask(cu, first, W)
    o = synth.bits(synth.normal((W, T, H, D), seed=10100 + case)).copy()
    l = synth.partial_lse((W, T, H), seed=10200 + case).numpy().copy()
    l[rng.random((W, T, H)) < 0.1] = -np.inf
    o[~mask] = 0x7FC0
    l[~mask] = np.nan
    o[~np.isfinite(l)] = 0x7FC0
    ro, rl = orc.lse_combine_planned(o, l, cu, first)
    out, lse = cam.lse_combine_planned(from_host_bits(o, torch.bfloat16), torch.from_numpy(l).cuda(), plan)
    torch.cuda.synchronize()
    assert_rows_close(orc.half_bits_to_double(to_host_bits(out)).reshape(-1, D),
                      orc.half_bits_to_double(ro).reshape(-1, D), "planned combine")
    assert_lse_close(lse.cpu().numpy(), rl, "planned combine lse")


@pytest.mark.parametrize("case", range(16))
def test_random_backward(cam, orc, case):
    """The combine's gradient on seeded random shapes, under each admission
    rule (every partial, the causal piece rule, a THD plan's rule): rank
    counts up to 64, row lengths reaching every access width and both the
    compacted and the wide-row forms, invalid and masked partials
    NaN-poisoned (never read)."""
    from helpers import assert_grad_lse_close, grad_lse_scale
    rng = np.random.default_rng(11000 + case)
    rule = ["all", "pieces", "plan"][case % 3]
    dt = str(rng.choice(["bf16", "fp16"]))
    H = int(rng.integers(1, 5))
    D = int(rng.choice([2, 5, 8, 24, 64, 128, 200, 512]))
    first = plan = cu = None
    if rule == "plan":
        P = int(rng.integers(1, 9))
        b = int(rng.choice([1, 2, 4]))
        blocks = [int(v) for v in rng.integers(0, 20, size=int(rng.integers(1, 6)))]
        while sum(blocks) < P:
            blocks[int(rng.integers(0, len(blocks)))] += 1
        cu = synth.cu_seqlens([x * b for x in blocks])
        T = int(cu[-1])
        q = orc.thd_plan(cu, P, block_size=b, min_split_tokens=8 * b)
        plan = cam.ThdPlan(P, T, cu, q["span_start"], q["span_rank"], q["span_local"], q["rank_off"],
                           q["rank_cost"], q["grid"]).to("cuda")
        first = orc.plan_first_positions(cu, q, P)
        mask = orc.plan_mask(cu, first, P)
    else:
        P = int(rng.choice([1, 2, 3, 8, 16, 33, 64]))
        T = int(rng.integers(1, 30))
        if rule == "pieces":
            cuts = np.sort(rng.choice(np.arange(1, T), size=min(3, T - 1), replace=False)) if T > 1 else []
            cu = np.concatenate([[0], cuts, [T]]).astype(np.int32)
            mask = orc.causal_mask(cu, P)
        else:
            mask = np.ones((P, T), dtype=bool)
    announce(f"random backward #{case}: rule={rule} P={P} T={T} H={H} D={D} {dt}")
    nan_bits = 0x7FC0 if dt == "bf16" else 0x7E00
    o = synth.bits(synth.normal((P, T, H, D), seed=11100 + case, dtype=dt)).copy()
    l = synth.partial_lse((P, T, H), seed=11200 + case).numpy().copy()
    bad = rng.random((P, T, H)) < 0.1
    l[bad] = rng.choice([-np.inf, np.inf, np.nan], size=int(bad.sum()))
    o[~mask] = nan_bits
    l[~mask] = np.nan
    o[~np.isfinite(l)] = nan_bits
    g = synth.bits(synth.normal((T, H, D), seed=11300 + case, dtype=dt))
    gl = synth.normal((T, H), seed=11400 + case, dtype="fp32").numpy() if case % 2 else None
    if rule == "plan":
        ro, rl = orc.lse_combine_planned_backward(o, l, g, gl, cu, first, dtype=dt)
    else:
        ro, rl = orc.lse_combine_backward(o, l, g, gl, dtype=dt, cu=cu)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float16
    args = (from_host_bits(o, tdt), torch.from_numpy(l).cuda(), from_host_bits(g, tdt),
            None if gl is None else torch.from_numpy(gl).cuda())
    if rule == "plan":
        d_po, d_pl = cam.lse_combine_backward(*args, plan=plan)
    elif rule == "pieces":
        d_po, d_pl = cam.lse_combine_backward(*args, cu_seqlens=torch.from_numpy(cu).cuda())
    else:
        d_po, d_pl = cam.lse_combine_backward(*args)
    torch.cuda.synchronize()
    got_o = orc.half_bits_to_double(to_host_bits(d_po), dt).reshape(P, T * H, D)
    want_o = orc.half_bits_to_double(ro, dt).reshape(P, T * H, D)
    assert_rows_close(got_o.reshape(-1, D), want_o.reshape(-1, D), "random backward d_part_out")
    assert np.all(got_o[want_o == 0] == 0), "d_part_out not exactly zero outside the valid set"
    scale = grad_lse_scale(np.where(np.isfinite(l)[..., None], orc.half_bits_to_double(o, dt), 0.0).reshape(P, T * H, D),
                           orc.half_bits_to_double(g, dt).reshape(T * H, D),
                           None if gl is None else gl.reshape(-1).astype(np.float64))
    assert_grad_lse_close(d_pl.cpu().numpy().reshape(P, -1), rl.reshape(P, -1), scale, "random backward d_part_lse")
