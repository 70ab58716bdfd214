"""Buffers over 2^32 bytes: the relayouts (dense, cu_seqlens varlen and over
a THD plan's spans) and the online merge, each at a size where one operand
passes 4 GiB so that byte offsets need more than 32 bits.  Every relayout
element is compared bit for bit with the oracle and the inverse relayout
must give the input back; every merged row and LSE is compared with the
oracle's combine of the same partials.  (The combines and their gradient
already run over partial stacks of 8 GiB at the packed THD size, and the pack
and packed combine have their own test over 4 GiB.)"""

import numpy as np
import pytest
import torch

import synth
from helpers import (announce, assert_bits_equal, assert_lse_close, assert_rows_close, to_host_bits,
                     window_pool)

pytestmark = pytest.mark.gpu

FOUR_GIB = 1 << 32


@pytest.fixture(scope="module")
def cam():
    import context_attention_movement_amd as m
    m.library()
    assert torch.cuda.is_available()
    return m


def _random_bits(shape, seed):
    """Payload of random 16-bit patterns (NaNs included: the relayouts copy
    bits), made on the device without a float32 temporary."""
    g = synth._gen(seed, "cuda")
    return torch.randint(-32768, 32768, shape, generator=g, device="cuda", dtype=torch.int16).view(torch.bfloat16)


# 64-token blocks, one sequence of a single block; 180,032 tokens in all
LENGTHS = [70016, 49984, 30016, 19968, 64, 9984]


def test_dense_relayout_beyond_4gib(cam, orc):
    """P = 8, Q/K/V planes, S = 120,000, H = 48, D = 128: 4.4 GB each way."""
    P, B, S, H, D = 8, 3, 120000, 48, 128
    announce(f"dense relayout over 4 GiB P={P} B={B} S={S} H={H} D={D}")
    x = _random_bits((P, B, S // P, H, D), synth.BASE_SEED + 301)
    assert x.numel() * 2 > FOUR_GIB
    y = cam.ulysses_seq_to_head(x, P)
    z = cam.ulysses_head_to_seq(y, P)
    torch.cuda.synchronize()
    assert torch.equal(z.view(torch.int16), x.view(torch.int16)), "dense round trip over 4 GiB"
    del z
    xh = to_host_bits(x)
    del x
    want = orc.seq_to_head(xh, P, B, S, H, D)
    del xh
    assert_bits_equal(to_host_bits(y), want, "dense seq->head over 4 GiB")


def test_varlen_relayout_beyond_4gib(cam, orc):
    """Packed THD batch of 180,032 tokens in 6 sequences, P = 8, Q/K/V planes,
    H = 32, D = 128: 4.4 GB each way."""
    P, B, H, D = 8, 3, 32, 128
    cu = synth.cu_seqlens(LENGTHS)
    T = int(cu[-1])
    announce(f"varlen relayout over 4 GiB T={T} P={P} B={B}")
    plan = cam.ulysses_varlen_plan(cu, P)
    x = _random_bits((B * T, H, D), synth.BASE_SEED + 302)
    assert x.numel() * 2 > FOUR_GIB
    y = cam.ulysses_seq_to_head_varlen(x, plan, B)
    z = cam.ulysses_head_to_seq_varlen(y, plan)
    torch.cuda.synchronize()
    assert torch.equal(z.view(torch.int16), x.view(torch.int16)), "varlen round trip over 4 GiB"
    del z
    xh = to_host_bits(x)
    del x
    want = orc.varlen_seq_to_head(xh, cu, P, B, H, D)
    del xh
    assert_bits_equal(to_host_bits(y), want, "varlen seq->head over 4 GiB")


def test_span_relayout_beyond_4gib(cam, orc):
    """The same batch planned over 8 ranks in 64-token blocks (the oracle's
    planner), seq->head over the plan's spans and back."""
    P, B, H, D = 8, 3, 32, 128
    cu = synth.cu_seqlens(LENGTHS)
    T = int(cu[-1])
    announce(f"span relayout over 4 GiB T={T} P={P} B={B}")
    q = orc.thd_plan(cu, P, block_size=64, min_split_tokens=8192)
    plan = cam.ThdPlan(P, T, np.asarray(cu, dtype=np.int32), q["span_start"], q["span_rank"], q["span_local"],
                       q["rank_off"], q["rank_cost"], q["grid"]).to("cuda")
    x = _random_bits((B * T, H, D), synth.BASE_SEED + 303)
    assert x.numel() * 2 > FOUR_GIB
    y = cam.ulysses_seq_to_head_spans(x, plan, B)
    z = cam.ulysses_head_to_seq_spans(y, plan)
    torch.cuda.synchronize()
    assert torch.equal(z.view(torch.int16), x.view(torch.int16)), "span round trip over 4 GiB"
    del z
    xh = to_host_bits(x)
    del x
    want = orc.span_seq_to_head(xh, q, P, B, H, D)
    del xh
    assert_bits_equal(to_host_bits(y), want, "span seq->head over 4 GiB")


def test_merge_beyond_4gib(cam, orc):
    """Two hops into an fp32 accumulator of 270,000 tokens x 32 heads x 128
    (4.4 GB): the first hop writes it, the second reads and rewrites it and
    writes the rounded rows.  Every rounded row and LSE against the oracle's
    combine of the two partials; the accumulator itself on token windows at
    its start, around the 4 GiB byte offset and at its end."""
    T, H, D = 270000, 32, 128
    announce(f"merge over 4 GiB T={T} H={H} D={D}")
    g = synth._gen(synth.BASE_SEED + 304, "cuda")
    po = torch.randn((2, T, H, D), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    pl = torch.randn((2, T, H), generator=g, device="cuda", dtype=torch.float32).mul_(2.0)
    pl[0, 5000:5100] = float("-inf")        # the first hop brings nothing there
    pl[1, T - 300:T - 200] = float("-inf")  # nor the second, near the end
    acc = torch.empty((T, H, D), device="cuda")
    assert acc.numel() * 4 > FOUR_GIB
    acc_l = torch.full((T, H), float("-inf"), device="cuda")
    fin = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    cam.lse_merge(acc, acc_l, po[0], pl[0])
    cam.lse_merge(acc, acc_l, po[1], pl[1], out_final=fin)
    torch.cuda.synchronize()
    po_h, pl_h = to_host_bits(po), pl.cpu().numpy()
    del po
    fin_h, accl_h = to_host_bits(fin), acc_l.cpu().numpy()
    boundary = FOUR_GIB // (H * D * 4)      # first token whose accumulator row starts past 4 GiB
    windows = [(0, 1000), (boundary - 1000, boundary + 1000), (T - 1000, T)]
    acc_h = {w: acc[w[0]:w[1]].cpu().double().numpy() for w in windows}
    del acc

    def check(a, e):
        ro, rl = orc.lse_combine(po_h[:, a:e], pl_h[:, a:e])
        w = assert_rows_close(orc.half_bits_to_double(fin_h[a:e]).reshape(-1, D),
                              orc.half_bits_to_double(ro).reshape(-1, D), f"merged rows [{a}, {e})")
        return w, assert_lse_close(accl_h[a:e], rl, f"merged lse [{a}, {e})")

    res = window_pool(T, check)
    for (a, e), got in acc_h.items():
        ref_o, _ = orc.combine_f64(orc.half_bits_to_double(po_h[:, a:e]).reshape(2, -1, D),
                                   pl_h[:, a:e].astype(np.float64).reshape(2, -1))
        got = got.reshape(-1, D)
        num = np.max(np.abs(got - ref_o), axis=1)
        den = np.max(np.abs(ref_o), axis=1)
        assert np.all(num[den == 0] == 0), f"accumulator [{a}, {e}): nonzero where the oracle is zero"
        assert np.max(num[den > 0] / den[den > 0]) <= 1e-5, f"accumulator [{a}, {e})"   # fp32 accumulator
    print(f"merge over 4 GiB, all {T * H} rows: worst row {max(r[0] for r in res):.3e}, "
          f"lse err {max(r[1] for r in res):.3e}", flush=True)
