"""Host-side checks of the benchmark's contract (no GPU): more than one GPU
is refused with a JSON message, the rocprofv3 counter summarizer takes the
median per dispatch of every counter of the named kernel, and the full-size
parity check against the oracle leg's outputs catches planted mistakes."""

import json
import subprocess
import sys
from pathlib import Path

ROOT = Path(__file__).resolve().parents[1]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2", "--steps", "1", "--warmup", "0"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_counter_summary_median_per_dispatch(tmp_path):
    sys.path.insert(0, str(ROOT))
    import bench
    d = tmp_path / "pmc"
    d.mkdir()
    rows = ["Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value"]
    for disp, v in ((1, 10), (2, 30), (3, 20)):
        rows.append(f'{disp},"void cam::k_proj_direct<false>(cam::Proj)",SQ_LDS_BANK_CONFLICT,{v}')
        rows.append(f'{disp},"void cam::k_proj_direct<false>(cam::Proj)",SQ_INSTS_LDS,{v * 100}')
    rows.append('4,"void cam::k_pack<16>(cam::Pack)",SQ_LDS_BANK_CONFLICT,999')
    (d / "pmc_counter_collection.csv").write_text("\n".join(rows) + "\n")
    out = tmp_path / "summary.txt"
    bench.summarize_counters(str(d), "k_proj_direct", str(out), "command: example")
    text = out.read_text()
    assert text.startswith("command: example\n")
    lines = {ln.split()[0]: ln.split() for ln in text.splitlines() if ln.startswith("  SQ_")}
    assert lines["SQ_LDS_BANK_CONFLICT"][1] == "20" and lines["SQ_LDS_BANK_CONFLICT"][2] == "dispatches=3"
    assert lines["SQ_INSTS_LDS"][1] == "2000"
    assert "k_pack" not in text


def test_ab_verdict_rule():
    """Paired A/B decision: faster or slower only beyond twice the null
    control's largest per-pair difference and with every pair agreeing."""
    sys.path.insert(0, str(ROOT))
    import bench
    null = [(100.0, 101.0), (100.0, 99.5), (100.0, 100.2)]           # floor 1%
    faster = [(100.0, 97.0), (100.0, 96.5), (100.0, 97.5)]           # -3%, all pairs
    assert bench.ab_verdict(null, faster)["verdict"] == "B faster"
    assert bench.ab_verdict(null, faster)["noise_floor_pct"] == 1.0
    assert bench.ab_verdict(null, [(100.0, 98.5), (100.0, 98.6), (100.0, 98.4)])["verdict"] == "neutral"  # < 2%
    mixed = [(100.0, 96.0), (100.0, 101.0), (100.0, 96.0)]
    assert bench.ab_verdict(null, mixed)["verdict"] == "neutral"     # a pair disagrees
    slower = [(100.0, 104.0), (100.0, 103.0), (100.0, 105.0)]
    assert bench.ab_verdict(null, slower)["verdict"] == "B slower"


def test_kernel_source_hash_covers_every_library_source():
    """Every source compiled into libcam.so takes part in the hash that keys
    the stored hardware counters, so a change to any of them retires them."""
    import bench
    from context_attention_movement_amd import build as cam_build
    headers = {p.name for p in cam_build.CSRC.glob("*.h")}
    assert set(cam_build.SOURCES) | headers <= set(bench.KERNEL_SOURCES)


class _TinyWorkload:
    """A CPU stand-in for the benchmark's workload at tiny sizes: the same
    attributes the oracle leg and the parity check read, with "GPU" outputs
    written by the oracle itself (so parity must hold) unless a mistake is
    planted afterwards."""

    def __init__(self):
        import types

        import numpy as np
        import torch

        import oracle
        import synth
        self.torch = types.SimpleNamespace(int16=torch.int16, cuda=types.SimpleNamespace(synchronize=lambda: None))
        bf = torch.bfloat16

        def from_bits(a, shape):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16).reshape(shape).copy()).view(bf)

        self.vP, self.vS, self.vH, self.vD = 2, 16, 4, 8
        P, S, H, D = self.vP, self.vS, self.vH, self.vD
        self.v_qkv = synth.relayout_seq_side(P, 3, S, H, D, seed=11)
        v_o = synth.relayout_head_side(P, 1, S, H, D, seed=12)
        self.v_qkv_out = from_bits(oracle.seq_to_head(synth.bits(self.v_qkv), P, 3, S, H, D), (P, 3, S, H // P, D))
        self.v_o = v_o
        self.v_o_sets = [(v_o, from_bits(oracle.head_to_seq(synth.bits(v_o), P, 1, S, H, D), (P, 1, S // P, H, D)))]
        self.mP, self.mT, self.mH, self.mDv = 2, 4, 4, 16
        P, T, H, Dv = self.mP, self.mT, self.mH, self.mDv
        out, mx, sm, _ = synth.dcp_partials(P, T, H, Dv, seed=13, corrupt_frac=0.1)
        packed = oracle.lse_pack(synth.bits(out), mx.numpy(), sm.numpy(), 1)
        co, cl = oracle.lse_combine_packed(packed, P, T, H, Dv, 1)
        self.m_sets = [{"out": out, "max": mx, "sum": sm, "packed_out": torch.from_numpy(packed.copy()),
                        "comb": from_bits(co, co.shape), "lse": torch.from_numpy(cl.copy())}]
        self.tP, self.tH, self.tD = 4, 4, 8
        self.t_cu = synth.cu_seqlens([5, 0, 70, 3, 50])
        T = self.tT = int(self.t_cu[-1])
        P, H, D = self.tP, self.tH, self.tD
        self.t_qkv = synth.normal((3 * T, H, D), seed=14)
        self.t_o = synth.normal((P, 1, T, H // P, D), seed=15)
        self.t_qkv_out = from_bits(oracle.varlen_seq_to_head(synth.bits(self.t_qkv), self.t_cu, P, 3, H, D),
                                   (P, 3, T, H // P, D))
        self.t_o_out = from_bits(oracle.varlen_head_to_seq(synth.bits(self.t_o), self.t_cu, P, 1, H, D), (T, H, D))
        self.t_part = synth.normal((P, T, H, D), seed=16)
        self.t_lse = synth.partial_lse((P, T, H), seed=17)
        to, tl = oracle.lse_combine(synth.bits(self.t_part), self.t_lse.numpy(), cu=self.t_cu)
        self.t_comb = from_bits(to, (T, H, D))
        self.t_comb_lse = torch.from_numpy(tl.copy())

    def op_bytes(self):
        keys = ("relayout_seq_to_head_video_p4_qkv", "relayout_head_to_seq_video_p4_o", "lse_pack_mla",
                "lse_combine_mla", "relayout_seq_to_head_varlen_thd_qkv", "relayout_head_to_seq_varlen_thd_o",
                "lse_combine_varlen_thd")
        return {k: 1000 for k in keys}

    def ops(self, k=0):
        return []  # the outputs above stand for the GPU's


def test_bench_parity_check_catches_planted_mistakes():
    """The bench's full-size parity check (GPU output against the oracle
    leg's output) passes on matching outputs and flags each planted mistake:
    one relayout element, one packed payload element, one packed LSE, one
    combined row, one combined LSE."""
    import numpy as np
    import torch

    import oracle
    sys.path.insert(0, str(ROOT))
    import bench
    w = _TinyWorkload()
    ref = {}
    bench.cpu_baseline(w, 2, keep=ref)
    res = bench.oracle_parity(w, ref)
    assert res["all_pass"], res
    assert res["ops"]["THD QKV varlen seq->head"]["elements"] == w.t_qkv_out.numel()

    def planted(fn, label):
        w2 = _TinyWorkload()
        fn(w2)
        r = bench.oracle_parity(w2, ref)
        assert not r["ops"][label]["pass"] and not r["all_pass"], label
        assert sum(not v["pass"] for v in r["ops"].values()) == 1, label

    def flip(t, i):
        t.view(-1).view(torch.int16)[i] ^= 1

    def bad_pack_payload(w2):
        w2.m_sets[0]["packed_out"][3] ^= 0x40

    def bad_pack_lse(w2):
        P, T, H, Dv = w2.mP, w2.mT, w2.mH, w2.mDv
        buf = w2.m_sets[0]["packed_out"].numpy()
        rows = oracle.pack_rows(P, T, H, 1)
        chunk = oracle.pack_chunk_bytes(P, T, H, Dv, 1, 2)
        o_bytes = (rows * Dv * 2 + 15) // 16 * 16
        _, L = oracle.packed_regions(buf, P, T, H, Dv, 1)
        c, q = divmod(int(np.flatnonzero(np.isfinite(L))[0]), rows)
        buf[c * chunk + o_bytes: c * chunk + o_bytes + 4 * rows].view(np.float32)[q] += 1e-3

    def bad_row(w2):
        w2.t_comb[3, 1] *= 1.05

    def bad_lse(w2):
        lse = w2.m_sets[0]["lse"]
        lse[int(torch.isfinite(lse).nonzero()[0])] += 1e-3

    planted(lambda w2: flip(w2.v_qkv_out, 5), "video P=4 QKV seq->head")
    planted(lambda w2: flip(w2.t_o_out, w2.t_o_out.numel() - 1), "THD O varlen head->seq")
    planted(bad_pack_payload, "MLA pack")
    planted(bad_pack_lse, "MLA pack")
    planted(bad_row, "THD causal combine")
    planted(bad_lse, "MLA combine")
