"""GPU end-to-end: the tiny check (P = 2, S = 256, H = 8, D = 64) through the
library against brute-force full attention, and HIP-graph capture of the
path replayed with changed inputs at fixed addresses."""

import numpy as np
import pytest
import torch

import synth
from helpers import announce, assert_bits_equal, assert_lse_close, assert_rows_close, from_host_bits, to_host_bits

pytestmark = pytest.mark.gpu

P, S, H, D = 2, 256, 8, 64


@pytest.fixture(scope="module")
def cam():
    import context_attention_movement_amd as m
    m.library()
    assert torch.cuda.is_available()
    return m


def _partials(orc, q, k, v):
    outs, ms, ss = [], [], []
    for p in range(P):
        o, m, s = orc.attention(q, k, v, p * S // P, (p + 1) * S // P)
        outs.append(orc.round_half(o))
        ms.append(m.astype(np.float32))
        ss.append(s.astype(np.float32))
    return np.stack(outs), np.stack(ms), np.stack(ss)


def test_tiny_chain_against_full_attention(cam, orc):
    announce("tiny end-to-end chain")
    g = [synth.bits(synth.normal((S, H, D), seed=synth.BASE_SEED + i)) for i in range(3)]
    X = np.stack(g)
    seq_side = np.ascontiguousarray(X.reshape(3, P, S // P, H, D).transpose(1, 0, 2, 3, 4))
    xs = from_host_bits(seq_side, torch.bfloat16)
    hs = cam.ulysses_seq_to_head(xs, P)
    back = cam.ulysses_head_to_seq(hs, P)
    torch.cuda.synchronize()
    assert_bits_equal(to_host_bits(hs), orc.seq_to_head(seq_side, P, 3, S, H, D), "QKV seq->head")
    assert_bits_equal(to_host_bits(back), seq_side, "QKV round trip")
    q, k, v = g
    ob, m, s = _partials(orc, q, k, v)
    packed = cam.lse_pack(from_host_bits(ob, torch.bfloat16), torch.from_numpy(m).cuda(),
                          torch.from_numpy(s).cuda(), scatter_dim=1)
    comb, lse = cam.lse_combine_packed(packed, P, S, H, D, 1)
    # combined output is head-sharded [P][S][H/P][D]; bring it back to sequence shards
    seq_out = cam.ulysses_head_to_seq(comb.view(P, 1, S, H // P, D), P)
    torch.cuda.synchronize()
    full_o, full_m, full_s = orc.attention(q, k, v, 0, S)
    got = orc.half_bits_to_double(to_host_bits(seq_out)).reshape(S * H, D)
    worst = assert_rows_close(got, full_o.reshape(S * H, D), "tiny chain vs full attention")
    lse_g = lse.cpu().numpy().reshape(P, S, H // P).transpose(1, 0, 2).reshape(-1)
    assert_lse_close(lse_g, (full_m + np.log(full_s)).reshape(-1), "tiny chain LSE vs full attention")
    print(f"tiny chain worst row rel err {worst:.3e}", flush=True)


def test_graph_capture_replay_with_changed_inputs(cam, orc):
    """Capture relayout + pack + combine once; replay after overwriting the
    outputs with sentinels, then after changing the inputs in place; every
    replay is compared with the oracle, with eager work in between."""
    announce("graph capture / replay")
    Pp, T, Hh, Dv, B = 4, 64, 16, 128, 3
    x = synth.relayout_seq_side(Pp, B, T, Hh, Dv, seed=1).cuda()
    y = torch.empty((Pp, B, T, Hh // Pp, Dv), dtype=torch.bfloat16, device="cuda")
    o, m, s, _ = synth.dcp_partials(Pp, T, Hh, Dv, seed=2, corrupt_frac=0.05)
    od, md, sd = o.cuda(), m.cuda(), s.cuda()
    n = cam.lse_pack_bytes(Pp, T, Hh, Dv, 1)
    packed = torch.empty(n, dtype=torch.uint8, device="cuda")
    rows = T * Hh // Pp
    out = torch.empty((Pp * rows, Dv), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(Pp * rows, dtype=torch.float32, device="cuda")

    def step():
        cam.ulysses_seq_to_head(x, Pp, out=y)
        cam.lse_pack(od, md, sd, 1, packed=packed)
        cam.lse_combine_packed(packed, Pp, T, Hh, Dv, 1, out=out, lse_out=lse)

    def check(tag):
        xh = to_host_bits(x)
        assert_bits_equal(to_host_bits(y), orc.seq_to_head(xh, Pp, B, T, Hh, Dv), f"{tag}: relayout")
        ref_packed = orc.lse_pack(to_host_bits(od), md.cpu().numpy(), sd.cpu().numpy(), 1)
        ro, rl = orc.lse_combine_packed(ref_packed, Pp, T, Hh, Dv, 1)
        assert_rows_close(orc.half_bits_to_double(to_host_bits(out)), orc.half_bits_to_double(ro), f"{tag}: combine")
        assert_lse_close(lse.cpu().numpy(), rl, f"{tag}: lse")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    check("eager")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for i in range(3):
        for t in (y, out):
            t.view(torch.int16).fill_(0x7FC0 - i)   # sentinels
        lse.fill_(12345.0)
        graph.replay()
        torch.cuda.synchronize()
        check(f"replay {i}")
        # change inputs in place at the same addresses, with eager work between replays
        x.copy_(synth.relayout_seq_side(Pp, B, T, Hh, Dv, seed=10 + i).cuda())
        o2, m2, s2, _ = synth.dcp_partials(Pp, T, Hh, Dv, seed=20 + i, corrupt_frac=0.1)
        od.copy_(o2.cuda())
        md.copy_(m2.cuda())
        sd.copy_(s2.cuda())
        torch.cuda.synchronize()
