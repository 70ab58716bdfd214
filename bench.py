"""Benchmark of the per-GPU hot path of sequence/context-parallel attention
movement on one MI355X.

One step runs every operation of the path once, each on the workload the
pages give for it:
  - Ulysses relayout, video DiT at P = 4 (S = 32760, H = 24, D = 128, bf16):
    seq->head of Q, K, V (B = 3) and head->seq of the attention output (B = 1);
  - MLA-style decode context parallel, P = 8, T = 128, H = 128, Dv = 512:
    max/sum-aware LSE pack (1% invalid statistics), the exchange as a strided
    view, and the stable combine;
  - packed THD, 20 short + 2 long sequences filling 131072 tokens, H = 32,
    D = 128, P = 8: varlen seq->head of Q, K, V, head->seq of O, and the
    causal combine of 8 KV-piece partials.
Inputs are synthetic and seeded, resident in HBM before the timed region.
Each buffer an operation reads was last touched a whole step earlier (more
than 15 GB of other traffic in between), so no input is served from the
256 MB Infinity Cache.

Prints ONE JSON line.  `value` is the step's algorithmic bytes (each input
read once, each output written once, invalid or causally masked partials not
read) divided by the step time.  Per-operation figures are under "ops".
The CPU leg (skipped with --no-cpu-baseline) times the oracle over the same
step ("cpu_baseline") and then compares every element of the GPU's outputs
with the oracle's ("parity").

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --summarize-rocprof TRACE FETCH WRITE BENCH_JSON --summary-out F --command TEXT
    python bench.py --summarize-counters COUNTER_DIR KERNEL --summary-out F --command TEXT
"""

from __future__ import annotations

import argparse
import csv
import gc
import glob
import hashlib
import json
import math
import os
import platform
import statistics
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "achieved HBM GB/s (% of peak) and µs/call for relayout, LSE-pack, combine"
HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores, published
KERNEL_SOURCES = ["relayout.hip", "lse.hip", "proj.hip", "cam_device.h", "cam_internal.h", "cam_api.cpp",
                  "thd_planner.cpp"]
TRAFFIC_FILE = ROOT / "profiles" / "traffic.json"


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        h.update((ROOT / "context_attention_movement_amd" / "csrc" / name).read_bytes())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------

def thd_admitted_counts(cu, P):
    """Number of (token, partial) pairs whose KV piece is admitted by the
    causal rule (non-empty piece starting at or before the token)."""
    total = 0
    for i in range(len(cu) - 1):
        L = int(cu[i + 1]) - int(cu[i])
        for p in range(P):
            a, e = (p * L) // P, ((p + 1) * L) // P
            if a < e:
                total += L - a
    return total


class Workload:
    def __init__(self, torch, cam, synth):
        self.torch, self.cam, self.synth = torch, cam, synth
        dev = "cuda"
        g = synth._gen(synth.BASE_SEED + 1, dev)
        bf = torch.bfloat16

        def randn(shape, std=1.0):
            x = torch.randn(shape, generator=g, device=dev, dtype=torch.float32)
            if std != 1.0:
                x.mul_(std)
            return x.to(bf)

        # video DiT, P = 4
        self.vP, self.vS, self.vH, self.vD = 4, 32760, 24, 128
        P, S, H, D = self.vP, self.vS, self.vH, self.vD
        self.v_qkv = randn((P, 3, S // P, H, D))
        self.v_qkv_out = torch.empty((P, 3, S, H // P, D), dtype=bf, device=dev)
        self.v_o = randn((P, 1, S, H // P, D))
        self.v_o_out = torch.empty((P, 1, S // P, H, D), dtype=bf, device=dev)
        # the O call's input and output together are 0.4 GB, under the 256 MB
        # Infinity Cache's reach when repeated: VO_SETS buffer sets (1.2 GB)
        # so that repeated calls start cold
        self.VO_SETS = 3
        self.v_o_sets = [(self.v_o, self.v_o_out)] + [
            (randn((P, 1, S, H // P, D)), torch.empty((P, 1, S // P, H, D), dtype=bf, device=dev))
            for _ in range(self.VO_SETS - 1)]
        # video DiT, P = 8 (timed beyond the step): Q/K/V [8][3][9450][48][128]
        # and O [8][1][75600][6][128], 2.8 GB and 0.9 GB
        self.v8_qkv = randn((8, 3, 75600 // 8, 48, D))
        self.v8_qkv_out = torch.empty((8, 3, 75600, 48 // 8, D), dtype=bf, device=dev)
        self.v8_o = randn((8, 1, 75600, 48 // 8, D))
        self.v8_o_out = torch.empty((8, 1, 75600 // 8, 48, D), dtype=bf, device=dev)
        # MLA decode, P = 8; NSETS independent buffer sets (> 1 GiB together) so
        # that repeated calls never find their inputs in the 256 MB Infinity Cache
        self.mP, self.mT, self.mH, self.mDv = 8, 128, 128, 512
        P, T, H, Dv = self.mP, self.mT, self.mH, self.mDv
        self.NSETS = 8
        n = cam.lse_pack_bytes(P, T, H, Dv, 1)
        rows = T * H // P
        self.m_sets = []
        for i in range(self.NSETS):
            out, mx, sm, bad = synth.dcp_partials(P, T, H, Dv, synth.BASE_SEED + 3 + 1000 * i, device=dev)
            packed_in = torch.empty(n, dtype=torch.uint8, device=dev)
            cam.lse_pack(out, mx, sm, 1, packed=packed_in)
            self.m_sets.append({
                "out": out, "max": mx, "sum": sm, "invalid": int(bad.size),
                "packed_out": torch.empty(n, dtype=torch.uint8, device=dev),   # written by the pack
                "packed_in": packed_in,                                         # read by the combine
                "comb": torch.empty((P * rows, Dv), dtype=bf, device=dev),
                "lse": torch.empty(P * rows, dtype=torch.float32, device=dev)})
        self.m_invalid = self.m_sets[0]["invalid"]
        # packed THD, P = 8
        self.tP, self.tH, self.tD = 8, 32, 128
        P, H, D = self.tP, self.tH, self.tD
        lens = synth.thd_lengths(20, 131072, seed=synth.BASE_SEED + 4)
        self.t_cu = synth.cu_seqlens(lens)
        T = self.tT = int(self.t_cu[-1])
        self.t_plan = cam.ulysses_varlen_plan(self.t_cu, P)
        self.t_qkv = randn((3 * T, H, D))
        self.t_qkv_out = torch.empty((P, 3, T, H // P, D), dtype=bf, device=dev)
        self.t_o = randn((P, 1, T, H // P, D))
        self.t_o_out = torch.empty((T, H, D), dtype=bf, device=dev)
        self.t_part = torch.empty((P, T, H, D), dtype=bf, device=dev)
        for p in range(P):
            self.t_part[p].copy_(randn((T, H, D)))
        self.t_lse = torch.randn((P, T, H), generator=g, device=dev, dtype=torch.float32).mul_(2.0)
        self.t_cu_dev = torch.from_numpy(self.t_cu).to(dev)
        self.t_comb = torch.empty((T, H, D), dtype=bf, device=dev)
        self.t_comb_lse = torch.empty((T, H), dtype=torch.float32, device=dev)
        self.t_admitted = thd_admitted_counts(self.t_cu, P)
        # ring of online merges: fp32 accumulator (payload and LSE) per token row
        self.t_acc = torch.empty((T, H, D), dtype=torch.float32, device=dev)
        self.t_acc_lse = torch.empty((T, H), dtype=torch.float32, device=dev)
        self.t_ring_out = torch.empty((T, H, D), dtype=bf, device=dev)
        # sequence-sharded outputs of the fused combine epilogues
        self.t_comb_seq = torch.empty((T, H, D), dtype=bf, device=dev)
        self.t_comb_seq_lse = torch.empty((T, H), dtype=torch.float32, device=dev)
        Pm, Tm, Hm, Dvm = self.mP, self.mT, self.mH, self.mDv
        for i, ms in enumerate(self.m_sets):
            ms["comb_seq"] = torch.empty((Tm, Hm, Dvm), dtype=bf, device=dev)
            ms["lse_seq"] = torch.empty((Tm, Hm), dtype=torch.float32, device=dev)
            ms["comb_h2s"] = torch.empty((Pm, 1, Tm // Pm, Hm, Dvm), dtype=bf, device=dev)
            # the combine's gradient at this shape (rows of 1 KB): the partials
            # above, their LSEs and an upstream gradient
            ms["bwd_lse"] = synth.partial_lse((Pm, Tm, Hm), seed=synth.BASE_SEED + 6 + 1000 * i, device=dev)
            ms["bwd_g"] = synth.normal((Tm, Hm, Dvm), seed=synth.BASE_SEED + 7 + 1000 * i, device=dev)
            ms["bwd_dpo"] = torch.empty((Pm, Tm, Hm, Dvm), dtype=bf, device=dev)
            ms["bwd_dpl"] = torch.empty((Pm, Tm, Hm), dtype=torch.float32, device=dev)
        # THD layout plan over 8 ranks of the same 131072 tokens in 64-token
        # blocks (the planned relayout reuses the THD Q/K/V and O buffers)
        self.p_lens = synth.thd_lengths(20, 131072, seed=synth.BASE_SEED + 4, align=64)
        self.p_cu = synth.cu_seqlens(self.p_lens)
        t0 = time.perf_counter()
        self.p_plan = cam.thd_plan(self.p_cu, self.tP, cam.ThdPlannerConfig(block_size=64, min_split_tokens=8192),
                                   device=dev)
        self.p_plan_ms = (time.perf_counter() - t0) * 1e3
        self.p_contig = cam.thd_plan(self.p_cu, self.tP, cam.ThdPlannerConfig(block_size=64, min_split_tokens=8192,
                                                                                contiguous=True))
        first = self.p_plan.first_pos_host
        self.p_admitted = sum(max(0, int(L) - int(first[p, i])) for i, L in enumerate(self.p_lens)
                              for p in range(self.tP) if first[p, i] < int(L))
        # Q/K/V projection of the video shape into the head-sharded layout:
        # x [S][3072] (hidden = 24 heads x 128), w [3 * 24 * 128][3072]
        P, S, H, D = self.vP, self.vS, self.vH, self.vD
        self.j_x = randn((S, H * D))
        self.j_w = (torch.randn((3 * H * D, H * D), generator=g, device=dev, dtype=torch.float32) * 0.02).to(bf)
        self.j_flops = 2 * S * (3 * H * D) * (H * D)
        # training: gradient buffers of the relayout pair and of the THD combine
        P, S, H, D = self.vP, self.vS, self.vH, self.vD
        self.v_dqkv = torch.empty((P, 3, S // P, H, D), dtype=bf, device=dev)
        self.v_do = torch.empty((P, 1, S, H // P, D), dtype=bf, device=dev)
        P, T, H, D = self.tP, self.tT, self.tH, self.tD
        self.t_dpart = torch.empty((P, T, H, D), dtype=bf, device=dev)
        # the same gradient into the library's partial-stack layout (partials 1 MiB apart)
        self.t_dpart_gap = cam.empty_partials(P, T, H, D, dtype=bf, device=dev)
        self.t_dlse = torch.empty((P, T, H), dtype=torch.float32, device=dev)
        self.t_gout = randn((T, H, D))
        self.step_index = 0
        torch.cuda.synchronize()

    def input_digests(self):
        """SHA-256 (first 16 hex digits) of every seeded input buffer's shape,
        dtype and its first and last MiB, read back before the timed steps."""
        torch = self.torch
        bufs = {"video_qkv": self.v_qkv, "video_o": self.v_o, "video_p8_qkv": self.v8_qkv, "video_p8_o": self.v8_o,
                "thd_qkv": self.t_qkv, "thd_o": self.t_o,
                "thd_partials": self.t_part, "thd_partial_lse": self.t_lse, "thd_grad_out": self.t_gout,
                "proj_x": self.j_x, "proj_w": self.j_w}
        for i, ms in enumerate(self.m_sets):
            for key in ("out", "max", "sum", "bwd_lse", "bwd_g"):
                bufs[f"mla_{key}_set{i}"] = ms[key]
        for i, (vo, _) in enumerate(self.v_o_sets[1:], start=1):
            bufs[f"video_o_set{i}"] = vo
        out = {"thd_cu_seqlens": hashlib.sha256(self.t_cu.tobytes()).hexdigest()[:16],
               "planned_thd_cu_seqlens": hashlib.sha256(self.p_cu.tobytes()).hexdigest()[:16]}
        mib = 1 << 20
        for name, t in bufs.items():
            b = t.contiguous().view(torch.uint8).reshape(-1)
            h = hashlib.sha256(f"{tuple(t.shape)}{t.dtype}".encode())
            h.update(b[:mib].cpu().numpy().tobytes())
            h.update(b[max(0, b.numel() - mib):].cpu().numpy().tobytes())
            out[name] = h.hexdigest()[:16]
        return out

    # algorithmic bytes of each operation
    def op_bytes(self):
        vP, vS, vH, vD = self.vP, self.vS, self.vH, self.vD
        mP, mT, mH, mDv = self.mP, self.mT, self.mH, self.mDv
        tT, tH, tD = self.tT, self.tH, self.tD
        m_rows = mP * mT * mH  # (source, token, head) partial rows
        m_valid = m_rows - self.m_invalid
        return {
            "relayout_seq_to_head_video_p4_qkv": 2 * 3 * vS * vH * vD * 2,
            "relayout_head_to_seq_video_p4_o": 2 * vS * vH * vD * 2,
            "lse_pack_mla": m_rows * mDv * 2 + m_rows * 8 + m_rows * mDv * 2 + m_rows * 4,
            "lse_combine_mla": m_valid * mDv * 2 + m_rows * 4 + (m_rows // mP) * (mDv * 2 + 4),
            "relayout_seq_to_head_varlen_thd_qkv": 2 * 3 * tT * tH * tD * 2,
            "relayout_head_to_seq_varlen_thd_o": 2 * tT * tH * tD * 2,
            "lse_combine_varlen_thd": self.t_admitted * tH * (tD * 2 + 4) + tT * tH * (tD * 2 + 4),
        }

    def ops(self, k=None):
        """The step's operations as (name, kernel, callable); `k` selects the
        MLA and video-O buffer sets (defaults to the step index)."""
        cam = self.cam
        k = self.step_index if k is None else k
        ms = self.m_sets[k % self.NSETS]
        vo = self.v_o_sets[k % self.VO_SETS]

        def pack():
            cam.lse_pack(ms["out"], ms["max"], ms["sum"], 1, packed=ms["packed_out"])

        def combine():
            # the exchange is a strided view of a packed buffer; this set's
            # input was packed before the timed region and is cold here
            cam.lse_combine_packed(ms["packed_in"], self.mP, self.mT, self.mH, self.mDv, 1,
                                   out=ms["comb"], lse_out=ms["lse"])

        return [
            ("relayout_seq_to_head_video_p4_qkv", "k_dense_relayout<16, true>",
             lambda: cam.ulysses_seq_to_head(self.v_qkv, self.vP, out=self.v_qkv_out)),
            ("relayout_head_to_seq_video_p4_o", "k_dense_relayout<16, false>",
             lambda: cam.ulysses_head_to_seq(vo[0], self.vP, out=vo[1])),
            ("lse_pack_mla", "k_pack<16>", pack),
            ("lse_combine_mla", "k_combine_stream<16, false, 0, 0>", combine),
            ("relayout_seq_to_head_varlen_thd_qkv", "k_varlen_relayout<16, true, false>",
             lambda: cam.ulysses_seq_to_head_varlen(self.t_qkv, self.t_plan, 3, out=self.t_qkv_out)),
            ("relayout_head_to_seq_varlen_thd_o", "k_varlen_relayout<16, false, false>",
             lambda: cam.ulysses_head_to_seq_varlen(self.t_o, self.t_plan, out=self.t_o_out)),
            ("lse_combine_varlen_thd", "k_combine<16, false, 1, 1, false, 0>",
             lambda: cam.lse_combine_varlen(self.t_part, self.t_lse, self.t_cu_dev, out=self.t_comb,
                                            lse_out=self.t_comb_lse)),
        ]


    def extension_ops(self, k=0):
        """Operations beyond the step: the video relayouts at P = 8, the
        planned THD operations, the gradient of the combine (THD, and at the
        MLA shape), the
        relayout training pair (forward and backward), the ring of online
        merges, the combine epilogues that write the sequence-sharded layout
        directly and the unfused sequence they replace.
        (name, algorithmic bytes, callable)."""
        cam = self.cam
        ms = self.m_sets[k % self.NSETS]
        Pm, Tm, Hm, Dvm = self.mP, self.mT, self.mH, self.mDv
        comb_bytes = self.op_bytes()["lse_combine_mla"]
        out_bytes = Tm * Hm * Dvm * 2

        def fused():
            cam.lse_combine_packed_seq(ms["packed_in"], Pm, Tm, Hm, Dvm, 1, out=ms["comb_seq"], lse_out=ms["lse_seq"])

        def unfused():
            cam.lse_combine_packed(ms["packed_in"], Pm, Tm, Hm, Dvm, 1, out=ms["comb"], lse_out=ms["lse"])
            cam.ulysses_head_to_seq(ms["comb"].view(Pm, 1, Tm, Hm // Pm, Dvm), Pm, out=ms["comb_h2s"])

        def mla_backward():
            cam.lse_combine_backward(ms["out"], ms["bwd_lse"], ms["bwd_g"], None, d_part_out=ms["bwd_dpo"],
                                     d_part_lse=ms["bwd_dpl"])

        # every partial valid: each partial's row and LSE read, the upstream
        # gradient row read, each partial's two gradients written
        m_rows = Tm * Hm
        mla_bwd_bytes = 2 * Pm * m_rows * (2 * Dvm + 4) + m_rows * 2 * Dvm

        def thd_fused():
            cam.lse_combine_varlen_seq(self.t_part, self.t_lse, self.t_plan, out=self.t_comb_seq,
                                       lse_out=self.t_comb_seq_lse)

        T, H, D, P = self.tT, self.tH, self.tD, self.tP

        def ring():
            # P hops; the partial that arrives at hop h is t_part[h]; the empty
            # accumulator is marked by LSE = -inf (its payload is ignored)
            self.t_acc_lse.fill_(float("-inf"))
            for hop in range(P):
                cam.lse_merge(self.t_acc, self.t_acc_lse, self.t_part[hop], self.t_lse[hop],
                              out_final=self.t_ring_out if hop == P - 1 else None)

        rows = T * H
        # hop 0 reads no accumulator; every hop reads the partial and both LSEs
        # and writes the accumulator; the last hop also writes the rounded rows
        ring_bytes = rows * (P * (2 * D + 4 + 4 * D + 4 + 4) + (P - 1) * (4 * D) + 2 * D + 4)

        def training_pair():
            # forward scatter of Q/K/V and gather of O, then their gradients:
            # the inverse relayouts of the upstream gradients
            cam.ulysses_seq_to_head(self.v_qkv, self.vP, out=self.v_qkv_out)
            cam.ulysses_head_to_seq(self.v_o, self.vP, out=self.v_o_out)
            cam.ulysses_head_to_seq(self.v_qkv_out, self.vP, out=self.v_dqkv)
            cam.ulysses_seq_to_head(self.v_o_out, self.vP, out=self.v_do)

        pair_bytes = 2 * (self.op_bytes()["relayout_seq_to_head_video_p4_qkv"]
                          + self.op_bytes()["relayout_head_to_seq_video_p4_o"])

        def thd_backward():
            cam.lse_combine_backward(self.t_part, self.t_lse, self.t_gout, None, cu_seqlens=self.t_cu_dev,
                                     d_part_out=self.t_dpart, d_part_lse=self.t_dlse)

        def thd_backward_gap():
            cam.lse_combine_backward(self.t_part, self.t_lse, self.t_gout, None, cu_seqlens=self.t_cu_dev,
                                     d_part_out=self.t_dpart_gap, d_part_lse=self.t_dlse)

        # admitted partials: O row and LSE read; every row: upstream gradient
        # read; every partial: its two gradients written
        bwd_bytes = self.t_admitted * H * (2 * D + 4) + rows * 2 * D + P * rows * (2 * D + 4)

        def planned_s2h():
            cam.ulysses_seq_to_head_spans(self.t_qkv, self.p_plan, 3, out=self.t_qkv_out)

        def planned_h2s():
            cam.ulysses_head_to_seq_spans(self.t_o, self.p_plan, out=self.t_o_out)

        def planned_combine():
            cam.lse_combine_planned(self.t_part, self.t_lse, self.p_plan, out=self.t_comb, lse_out=self.t_comb_lse)

        planned_comb_bytes = self.p_admitted * H * (2 * D + 4) + rows * (2 * D + 4)

        def p8_s2h():
            cam.ulysses_seq_to_head(self.v8_qkv, 8, out=self.v8_qkv_out)

        def lds_s2h():
            cam.ablation_seq_to_head_lds(self.v_qkv, self.vP, LDS_ROWS_PER_TILE, out=self.v_qkv_out)

        def p8_h2s():
            cam.ulysses_head_to_seq(self.v8_o, 8, out=self.v8_o_out)

        return [
            ("relayout_seq_to_head_video_p8_qkv", 2 * self.v8_qkv.numel() * 2, p8_s2h),
            ("relayout_head_to_seq_video_p8_o", 2 * self.v8_o.numel() * 2, p8_h2s),
            ("lse_combine_planned_thd", planned_comb_bytes, planned_combine),
            ("relayout_seq_to_head_planned_thd_qkv", 2 * 3 * T * H * D * 2, planned_s2h),
            ("relayout_head_to_seq_planned_thd_o", 2 * T * H * D * 2, planned_h2s),
            ("lse_combine_varlen_backward_thd", bwd_bytes, thd_backward),
            ("lse_combine_varlen_backward_thd (gradient into empty_partials)", bwd_bytes, thd_backward_gap),
            ("lse_combine_backward_mla (rows of 1 KB)", mla_bwd_bytes, mla_backward),
            ("relayout_training_pair_video_p4 (fwd + bwd)", pair_bytes, training_pair),
            ("ring_of_8_online_merges_thd (fp32 accumulator)", ring_bytes, ring),
            ("combine_to_sequence_shards_mla (fused)", comb_bytes, fused),
            ("combine_then_head_to_seq_mla (unfused)", comb_bytes + 2 * out_bytes, unfused),
            ("combine_varlen_to_sequence_shards_thd (fused)", self.op_bytes()["lse_combine_varlen_thd"], thd_fused),
            ("relayout_seq_to_head_video_p4_qkv_lds_staged (ablation)",
             self.op_bytes()["relayout_seq_to_head_video_p4_qkv"], lds_s2h),
        ]


LDS_ROWS_PER_TILE = 4  # rows staged per workgroup by the LDS-staged relayout ablation
# µs/call of each operation alone: warm-up calls, then blocks of back-to-back
# calls between two HIP events (median and 95th percentile over the blocks)
WARM_CALLS, BLOCKS, PER_BLOCK = 10, 8, 5


def paired_ab(torch, stream, fa, fb, pairs=8, calls=10):
    """Paired A/B timing: `pairs` pairs of (calls back-to-back calls of A, the
    same of B) between HIP events, the order alternating from pair to pair.
    Returns the per-pair relative differences (B - A) / A."""
    def t(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(calls):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1000.0 / calls

    with torch.cuda.stream(stream):
        for _ in range(2):
            fa()
            fb()
        torch.cuda.synchronize()
        out = []
        for i in range(pairs):
            if i % 2 == 0:
                ta, tb = t(fa), t(fb)
            else:
                tb, ta = t(fb), t(fa)
            out.append((ta, tb))
    return out


def ab_decision(torch, stream, name, fa, fb, pairs=8, calls=10):
    """A paired comparison with a null control (A against itself, same
    protocol): the noise floor is the largest per-pair |difference| of the
    null control, the threshold twice that; B is called faster or slower only
    if its median difference exceeds the threshold and every pair agrees in
    sign, otherwise neutral."""
    null = paired_ab(torch, stream, fa, fa, pairs, calls)
    res = paired_ab(torch, stream, fa, fb, pairs, calls)
    out = ab_verdict(null, res)
    out.update({"comparison": name,
                "protocol": f"{pairs} pairs x {calls} back-to-back calls per side, order alternating; null control "
                            "A against A; noise floor = largest per-pair |difference| of the null control; threshold "
                            "= twice the floor, with every pair in the same direction"})
    return out


def ab_verdict(null, res):
    """The decision rule of ab_decision on per-pair (A, B) timings."""
    dn = [(b - a) / a for a, b in null]
    d = [(b - a) / a for a, b in res]
    floor = max(abs(x) for x in dn)
    med = statistics.median(d)
    faster = sum(1 for x in d if x < 0)
    if med < -2 * floor and faster == len(d):
        verdict = "B faster"
    elif med > 2 * floor and faster == 0:
        verdict = "B slower"
    else:
        verdict = "neutral"
    return {"A_us_median": round(statistics.median(a for a, _ in res), 2),
            "B_us_median": round(statistics.median(b for _, b in res), 2),
            "B_minus_A_median_pct": round(100 * med, 3), "B_faster_pairs": f"{faster}/{len(d)}",
            "noise_floor_pct": round(100 * floor, 3), "threshold_pct": round(200 * floor, 3), "verdict": verdict}


def plan_summary(w):
    """Balance of the THD layout plan used by the planned relayouts: maximum
    over mean rank cost for the plan, the contiguous layout and the
    per-sequence split, with the planner's host time."""
    P = w.tP
    split = [0.0] * P
    for L in (int(x) for x in w.p_lens):
        for p in range(P):
            a, e = p * L // P, (p + 1) * L // P
            split[p] += (e - a) + (e * (e + 1) // 2 - a * (a + 1) // 2)
    ratio = lambda c: round(float(max(c)) / (float(sum(c)) / len(c)), 4)
    return {"ranks": P, "block_size": 64, "grid": w.p_plan.grid, "spans": w.p_plan.n_spans,
            "max_over_mean_cost": ratio(w.p_plan.rank_cost),
            "contiguous_max_over_mean_cost": ratio(w.p_contig.rank_cost),
            "sequence_split_max_over_mean_cost": ratio(split), "host_ms": round(w.p_plan_ms, 3),
            "cost": "token_weight 1 + causal_weight 1 * (k + 1) per token at position k"}


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on a bounded sample
# ---------------------------------------------------------------------------

def _cpu_work_items(w):
    """The step's seven operations at full size as independent oracle calls
    on host copies of the same synthetic inputs: (label, algorithmic bytes,
    callable).  The THD causal combine, the costly one, is cut into token
    windows (the oracle's own window arguments); each window is one item."""
    import numpy as np
    import oracle

    torch = w.torch

    def bits(t):
        t = t.detach().contiguous().cpu()
        return t.view(torch.int16).numpy().view(np.uint16)

    nb = w.op_bytes()
    items = []
    vx, vo = bits(w.v_qkv), bits(w.v_o)
    items.append(("video P=4 QKV seq->head", nb["relayout_seq_to_head_video_p4_qkv"],
                  lambda: oracle.seq_to_head(vx, w.vP, 3, w.vS, w.vH, w.vD)))
    items.append(("video P=4 O head->seq", nb["relayout_head_to_seq_video_p4_o"],
                  lambda: oracle.head_to_seq(vo, w.vP, 1, w.vS, w.vH, w.vD)))
    ob = bits(w.m_sets[0]["out"])
    m = w.m_sets[0]["max"].cpu().numpy()
    s = w.m_sets[0]["sum"].cpu().numpy()
    packed = oracle.lse_pack(ob, m, s, 1)  # the combine's input (not timed here)
    items.append(("MLA pack", nb["lse_pack_mla"], lambda: oracle.lse_pack(ob, m, s, 1)))
    items.append(("MLA combine", nb["lse_combine_mla"],
                  lambda: oracle.lse_combine_packed(packed, w.mP, w.mT, w.mH, w.mDv, 1)))
    tx, to = bits(w.t_qkv), bits(w.t_o)
    items.append(("THD QKV varlen seq->head", nb["relayout_seq_to_head_varlen_thd_qkv"],
                  lambda: oracle.varlen_seq_to_head(tx, w.t_cu, w.tP, 3, w.tH, w.tD)))
    items.append(("THD O varlen head->seq", nb["relayout_head_to_seq_varlen_thd_o"],
                  lambda: oracle.varlen_head_to_seq(to, w.t_cu, w.tP, 1, w.tH, w.tD)))
    po, pl = bits(w.t_part), w.t_lse.cpu().numpy()
    T, n_win = w.tT, 64
    for k in range(n_win):
        a, e = k * T // n_win, (k + 1) * T // n_win
        items.append((f"THD causal combine [{a}, {e})", nb["lse_combine_varlen_thd"] * (e - a) / T,
                      lambda a=a, e=e: oracle.lse_combine(po[:, a:e], pl[:, a:e], cu=w.t_cu, t_begin=a)))
    return items


def cpu_baseline(w, max_threads: int = 16, keep: dict | None = None):
    """The oracle as it stands, timed on the host cores over the whole step's
    workload (every operation at full size): once on one core, then with the
    same independent calls spread over N threads (ctypes releases the GIL
    during each oracle call).  The median of 3 runs is taken for each leg.
    `keep`, if given, receives each call's result (label -> oracle output)
    from the last threaded run: the parity reference of this run (see
    cpu_leg)."""
    from concurrent.futures import ThreadPoolExecutor

    items = _cpu_work_items(w)
    total = sum(b for _, b, _ in items)
    n_threads = max(1, min(max_threads, len(os.sched_getaffinity(0))))

    def serial():
        t0 = time.perf_counter()
        for _, _, fn in items:
            fn()
        return time.perf_counter() - t0

    def threaded():
        t0 = time.perf_counter()
        # costliest first so that the pool's tail is short
        with ThreadPoolExecutor(max_workers=n_threads) as ex:
            futs = [(label, ex.submit(fn)) for label, _, fn in sorted(items, key=lambda x: -x[1])]
            for label, f in futs:
                r = f.result()
                if keep is not None:
                    keep[label] = r
        return time.perf_counter() - t0

    t1 = serial()
    if t1 < 10.0:  # one run of a leg over 10 s, else the median of 3
        t1 = statistics.median([t1, serial(), serial()])
    tn = statistics.median(threaded() for _ in range(3))
    sample = ("the whole step at full size: video P=4 QKV seq->head and O head->seq, MLA pack and combine, THD "
              "QKV varlen seq->head and O head->seq, THD causal combine of all 131072 tokens (64 token windows); "
              "C oracle (fp64, rounded once) on the same synthetic inputs downloaded from the GPU; GB/s = the "
              "step's algorithmic bytes / oracle wall time (median of 3 runs, or one run of a leg over 10 s)")
    return {
        "value": round(total / tn / 1e9, 4),
        "unit": "GB/s",
        "cores": n_threads,
        "kind": "oracle",
        "seconds": round(tn, 2),
        "sample": sample + f"; the same {len(items)} independent oracle calls on a pool of {n_threads} threads",
        "single_core": {"value": round(total / t1 / 1e9, 4), "unit": "GB/s", "cores": 1, "seconds": round(t1, 2),
                        "sample": sample + "; the calls one after another on one thread"},
        "cpu": _cpu_model(),
        "affinity_cores": len(os.sched_getaffinity(0)),
    }


OUT_ROW_RTOL = 8e-3   # combined payload: per row max|gpu - oracle| / max|oracle|
LSE_ATOL = 1e-5       # fp32 LSE, absolute


def _rows_rel(got_bits, want_bits, D, dt="bf16"):
    """Worst per-row relative error max|g - o| / max|o| of two payload bit
    arrays, in windows of rows; rows whose reference is all zero must be
    exactly zero.  Returns (worst, bad_zero_rows, nan_count)."""
    import numpy as np
    import oracle

    g = got_bits.reshape(-1, D)
    o = want_bits.reshape(-1, D)
    worst, bad, nan = 0.0, 0, 0
    step = max(1, (1 << 23) // D)
    for a in range(0, g.shape[0], step):
        gd = oracle.half_bits_to_double(g[a:a + step], dt)
        od = oracle.half_bits_to_double(o[a:a + step], dt)
        nan += int(np.isnan(gd).sum())
        num = np.max(np.abs(gd - od), axis=-1)
        den = np.max(np.abs(od), axis=-1)
        zero = den == 0
        bad += int(np.count_nonzero(num[zero]))
        if (~zero).any():
            worst = max(worst, float(np.max(num[~zero] / den[~zero])))
    return worst, bad, nan


def _lse_diff(got, want):
    """(max |got - want| over entries finite in the oracle, entries whose
    finiteness differs, NaN count) of two fp32 LSE arrays."""
    import numpy as np

    got = np.asarray(got, dtype=np.float64).reshape(-1)
    want = np.asarray(want, dtype=np.float64).reshape(-1)
    fin = np.isfinite(want)
    mism = int(np.count_nonzero(fin & ~np.isfinite(got))) + int(np.count_nonzero(~fin & (got != want)))
    diff = float(np.max(np.abs(got[fin] - want[fin]))) if fin.any() else 0.0
    return diff, mism, int(np.isnan(got).sum())


def cpu_leg(w, max_threads: int = 16):
    """The CPU leg of the benchmark: the oracle timed over the whole step
    (cpu_baseline), then the GPU's outputs checked against the oracle's
    outputs of those same calls (oracle_parity).  Returns (baseline, parity)."""
    ref = {}
    baseline = cpu_baseline(w, max_threads, keep=ref)
    return baseline, oracle_parity(w, ref)


def oracle_parity(w, ref):
    """Every step operation run once more on the GPU (buffer set 0) and its
    output compared, element by element at full size, with the oracle's
    output for the same inputs (`ref`, from the cpu_baseline leg): bit-exact
    for the relayouts and the packed payload; LSE within 1e-5; combined rows
    within 8e-3 relative."""
    import numpy as np
    import oracle

    torch = w.torch
    for _, _, fn in w.ops(k=0):
        fn()
    torch.cuda.synchronize()

    def bits(t):
        return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)

    res = {}

    def exact(label, gpu):
        want = ref[label]
        n = int(np.count_nonzero(bits(gpu).reshape(-1) != np.asarray(want).reshape(-1)))
        res[label] = {"check": "bit-exact", "elements": int(np.asarray(want).size), "mismatches": n, "pass": n == 0}

    exact("video P=4 QKV seq->head", w.v_qkv_out)
    exact("video P=4 O head->seq", w.v_o_sets[0][1])
    exact("THD QKV varlen seq->head", w.t_qkv_out)
    exact("THD O varlen head->seq", w.t_o_out)
    ms = w.m_sets[0]
    P, T, H, Dv = w.mP, w.mT, w.mH, w.mDv
    Og, Lg = oracle.packed_regions(ms["packed_out"].cpu().numpy(), P, T, H, Dv, 1)
    Oo, Lo = oracle.packed_regions(np.asarray(ref["MLA pack"]), P, T, H, Dv, 1)
    nO = int(np.count_nonzero(Og != Oo))
    dL, mL, nanL = _lse_diff(Lg, Lo)
    res["MLA pack"] = {"check": "O-region bit-exact, L-region within 1e-5 with the same -inf entries",
                       "o_mismatches": nO, "lse_max_abs_diff": dL, "lse_nonfinite_mismatches": mL,
                       "pass": nO == 0 and dL <= LSE_ATOL and mL == 0 and nanL == 0}

    def combined(label, out, lse, D, want_out, want_lse):
        rel, bad, nan = _rows_rel(bits(out), np.asarray(want_out), D)
        dL, mL, nanL = _lse_diff(lse.cpu().numpy(), want_lse)
        res[label] = {"check": "rows within 8e-3 relative, LSE within 1e-5", "rows": int(np.asarray(want_out).size // D),
                      "worst_row_rel": rel, "lse_max_abs_diff": dL,
                      "pass": rel <= OUT_ROW_RTOL and bad == 0 and nan == 0 and dL <= LSE_ATOL and mL == 0
                      and nanL == 0}

    mo, ml = ref["MLA combine"]
    combined("MLA combine", ms["comb"], ms["lse"], Dv, mo, ml)
    wins = sorted((k for k in ref if k.startswith("THD causal combine [")),
                  key=lambda k: int(k.split("[")[1].split(",")[0]))
    to = np.concatenate([np.asarray(ref[k][0]).reshape(-1) for k in wins])
    tl = np.concatenate([np.asarray(ref[k][1]).reshape(-1) for k in wins])
    combined("THD causal combine", w.t_comb, w.t_comb_lse, w.tD, to, tl)
    return {"reference": "the oracle's outputs from the cpu_baseline leg, on the same inputs, every element",
            "ops": res, "all_pass": all(r["pass"] for r in res.values())}


def _cpu_model():
    """Model name from /proc/cpuinfo, with the family, model and stepping
    numbers (some hosts report only a generic brand string)."""
    info = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" in line:
                k, v = (x.strip() for x in line.split(":", 1))
                info.setdefault(k, v)
            if not line.strip() and info:
                break
    except OSError:
        return "unknown"
    name = info.get("model name", "unknown")
    extra = [f"{k} {info[k]}" for k in ("cpu family", "model", "stepping") if k in info]
    return f"{name} ({', '.join(extra)})" if extra else name


# ---------------------------------------------------------------------------
# rocprofv3 summaries
# ---------------------------------------------------------------------------

def _read_csvs(root, suffix):
    rows = []
    for f in sorted(glob.glob(os.path.join(root, "**", f"*{suffix}"), recursive=True)):
        with open(f, newline="") as fh:
            rows += list(csv.DictReader(fh))
    return rows


COPY_KERNEL = "k_copy16"
COPY_BYTES = 3 * 32760 * 24 * 128 * 2  # the video Q/K/V operand copied for the ceiling (each way)


def _grid_threads(r):
    g = r.get("Grid_Size_X", r.get("Grid_Size"))
    return int(float(g)) if g not in (None, "") else -1


def summarize_rocprof(trace_dir, fetch_dir, write_dir, bench_json, out_txt, command):
    """Write a short text summary of rocprofv3 output and, when both counters
    are given, profiles/traffic.json.

    - rocprofv3's own kernel statistics (--stats), as printed;
    - per kernel and grid size, the dispatch durations from the kernel trace
      (one kernel can serve several operations at different grid sizes);
    - each operation of the step, matched to its dispatches by kernel name and
      grid size (bench.py records both per operation), with its average
      duration and its HBM bytes per launch: FETCH_SIZE and WRITE_SIZE per
      dispatch, each scaled by what the same counter reads for the plain copy
      kernel of known size."""
    while command.startswith("command: "):  # a header passed back in is not repeated
        command = command[len("command: "):]
    lines = [f"command: {command}", ""]
    stats = _read_csvs(trace_dir, "kernel_stats.csv") if trace_dir else []
    if stats:
        lines.append("kernel statistics (rocprofv3 --kernel-trace --stats), microseconds:")
        lines.append(f"{'kernel':70s} {'calls':>6s} {'avg':>10s} {'min':>10s} {'max':>10s}")
        for r in stats:
            name = r.get("Name", r.get("KernelName", ""))
            if "cam::" not in name:
                continue
            lines.append(f"{name[:70]:70s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
                         f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f}")
        lines.append("")
    durs = {}
    for r in (_read_csvs(trace_dir, "kernel_trace.csv") if trace_dir else []):
        name = r.get("Kernel_Name", "")
        if "cam::" in name:
            durs.setdefault((name, _grid_threads(r)), []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    if durs:
        lines.append("per kernel and grid size (kernel trace), microseconds:")
        lines.append(f"{'kernel':70s} {'grid':>10s} {'calls':>6s} {'avg':>10s} {'min':>10s} {'max':>10s}")
        for (name, g), v in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
            lines.append(f"{name[:70]:70s} {g:10d} {len(v):6d} {statistics.mean(v):10.2f} "
                         f"{min(v):10.2f} {max(v):10.2f}")
        lines.append("")
    med = {}
    for d, cname in ((fetch_dir, "FETCH_SIZE"), (write_dir, "WRITE_SIZE")):
        if not d:
            continue
        per = {}
        for r in _read_csvs(d, "counter_collection.csv"):
            if r.get("Counter_Name") == cname and "cam::" in r["Kernel_Name"]:
                per.setdefault((r["Kernel_Name"], _grid_threads(r)), []).append(float(r["Counter_Value"]))
        med[cname] = {k: statistics.median(v) for k, v in per.items()}
        lines.append(f"{cname} per dispatch (KiB, median over dispatches):")
        for (name, g), v in sorted(per.items()):
            lines.append(f"  {name[:80]:80s} {g:10d} n={len(v):3d} {statistics.median(v):14.1f}")
        lines.append("")

    def find(table, frag, grid=None):
        for (name, g), v in table.items():
            if frag in name and (grid is None or g == grid):
                return v
        return None

    ops = json.loads(Path(bench_json).read_text()).get("ops", {}) if bench_json else {}
    if ops and durs:
        lines.append("operations of the step, matched by kernel and grid size:")
        for op, rec in ops.items():
            la = rec.get("launch") or {}
            grid = la.get("workgroups", 0) * la.get("threads", 0)
            d = find(durs, rec["kernel"] + "(", grid)
            if d:
                lines.append(f"  {op:40s} {rec['kernel']:42s} grid {grid:9d}  avg {statistics.mean(d):9.2f} us "
                             f"over {len(d)} dispatches")
        lines.append("")
    if "FETCH_SIZE" in med and "WRITE_SIZE" in med:
        cf, cw = find(med["FETCH_SIZE"], COPY_KERNEL), find(med["WRITE_SIZE"], COPY_KERNEL)
        ff = COPY_BYTES / (cf * 1024.0)
        fw = COPY_BYTES / (cw * 1024.0)
        lines.append(f"copy calibration: {COPY_BYTES} bytes each way; FETCH_SIZE {cf:.1f} KiB (factor {ff:.4f}), "
                     f"WRITE_SIZE {cw:.1f} KiB (factor {fw:.4f})")
        traffic = {}
        for op, rec in ops.items():
            la = rec.get("launch") or {}
            grid = la.get("workgroups", 0) * la.get("threads", 0)
            f = find(med["FETCH_SIZE"], rec["kernel"] + "(", grid)
            wv = find(med["WRITE_SIZE"], rec["kernel"] + "(", grid)
            if f is None or wv is None:
                continue
            fb, wb = f * 1024.0 * ff, wv * 1024.0 * fw
            traffic[op] = {"kernel": rec["kernel"], "grid_threads": grid, "fetch_bytes": round(fb),
                           "write_bytes": round(wb), "hbm_bytes_per_launch": round(fb + wb),
                           "algorithmic_bytes": rec.get("algorithmic_bytes")}
            lines.append(f"  {op:40s} fetch {fb / 1e6:10.2f} MB  write {wb / 1e6:10.2f} MB  "
                         f"algorithmic {rec.get('algorithmic_bytes', 0) / 1e6:10.2f} MB")
        TRAFFIC_FILE.write_text(json.dumps({
            "kernel_source_hash": kernel_source_hash(), "command": command,
            "copy_calibration": {"bytes_each_way": COPY_BYTES, "fetch_kib": cf, "write_kib": cw,
                                 "fetch_factor": ff, "write_factor": fw},
            "ops": traffic}, indent=1) + "\n")
    Path(out_txt).write_text("\n".join(lines) + "\n")


def summarize_counters(counter_dir, kernel, out_txt, command):
    """Write the median per dispatch of every counter rocprofv3 --pmc collected
    for the kernels whose name contains `kernel`, one line per counter."""
    while command.startswith("command: "):
        command = command[len("command: "):]
    vals = {}
    names = set()
    for r in _read_csvs(counter_dir, "counter_collection.csv"):
        name = r.get("Kernel_Name", "")
        if kernel not in name:
            continue
        names.add(name)
        key = (r.get("Dispatch_Id", ""), r["Counter_Name"])
        vals.setdefault(r["Counter_Name"], {}).setdefault(key, 0.0)
        vals[r["Counter_Name"]][key] += float(r["Counter_Value"])  # summed over the dispatch's instances
    lines = [f"command: {command}", "", f"kernel: {', '.join(sorted(names))}",
             "counter (median per dispatch over the run):"]
    for c in sorted(vals):
        v = sorted(vals[c].values())
        lines.append(f"  {c:32s} {v[len(v) // 2]:>18.0f}   dispatches={len(v)}")
    text = "\n".join(lines) + "\n"
    if out_txt:
        Path(out_txt).write_text(text)
    print(text, end="")


def profile_op(w, torch, name, calls):
    """Run one operation of the step or beyond it `calls` times after 3
    warmup calls (each on its own rotating buffer set where it has them),
    printing its launch geometry and µs per call; for rocprofv3 runs."""
    copy_ref = "copy_video_qkv"  # the plain copy of the video Q/K/V operand (the ceiling reference)
    table = [n for n, _, _ in w.ops()] + [n for n, _, _ in w.extension_ops()] + [copy_ref]
    if name not in table:
        raise SystemExit(f"unknown operation {name!r}; one of: {', '.join(table)}")
    is_step = name in [n for n, _, _ in w.ops()]

    def call(k):
        if name == copy_ref:
            return w.cam.copy(w.v_qkv, w.v_qkv_out)
        if is_step:
            return [fn for n, _, fn in w.ops(k=k) if n == name][0]()
        return [fn for n, _, fn in w.extension_ops(k=k) if n == name][0]()

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for k in range(3):
            call(k)
        torch.cuda.synchronize()
        print(f"[profile-op] {name}: {calls} calls, launch {w.cam.last_launch()}", flush=True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for k in range(calls):
            call(k)
        e1.record(stream)
        torch.cuda.synchronize()
    print(f"[profile-op] {name}: {e0.elapsed_time(e1) * 1000.0 / max(1, calls):.2f} us/call", flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--calls", type=int, default=20, help="calls of the operation under --profile-op")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=16, help="most threads of the N-core CPU baseline leg")
    ap.add_argument("--profile-op", default=None,
                    help="run only this operation (a step or extension name) --calls times and exit (for rocprofv3)")
    ap.add_argument("--digests-out", default=None, help="write the per-buffer input digests to this JSON file")
    ap.add_argument("--summarize-rocprof", nargs=4, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR", "BENCH_JSON"))
    ap.add_argument("--summarize-counters", nargs=2, metavar=("COUNTER_DIR", "KERNEL"))
    ap.add_argument("--summary-out", default=None)
    ap.add_argument("--command", default="")
    args = ap.parse_args()

    if args.summarize_rocprof:
        tr, fe, wr, bj = [None if x in ("-", "") else x for x in args.summarize_rocprof]
        summarize_rocprof(tr, fe, wr, bj, args.summary_out, args.command)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters[0], args.summarize_counters[1], args.summary_out, args.command)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark measures one GPU: the relayout, pack and combine of P "
                                   "logical ranks run in one GPU's HBM; --gpus must be 1"}), flush=True)
        sys.exit(2)

    import torch
    import context_attention_movement_amd as cam
    import synth

    cam.library()  # fails loudly without the HIP library
    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)
    w = Workload(torch, cam, synth)
    if args.profile_op:
        profile_op(w, torch, args.profile_op, args.calls)
        return
    digests = w.input_digests()
    if args.digests_out:
        Path(args.digests_out).write_text(json.dumps(digests, indent=1) + "\n")
    nbytes = w.op_bytes()
    names = [n for n, _, _ in w.ops()]
    kern = {n: k for n, k, _ in w.ops()}
    stream = torch.cuda.Stream()

    # ---- timed region: K steps, every operation once per step, events around each.
    # The steps' callables are built beforehand and Python's cyclic garbage
    # collector is paused (here and in every GPU timing after it), so that the
    # host keeps ahead of the GPU: a host pause while the queue is empty would
    # show up as GPU time between events.
    # The host work comes before the warm-up steps, so that the GPU does not
    # sit idle (and clock down) between the warm-up and the timed steps.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    step_fns = [[fn for _, _, fn in w.ops(k=w.step_index + args.warmup + k)] for k in range(args.steps)]
    gc.collect()
    gc.disable()  # until every GPU timing below is taken
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            for _, _, fn in w.ops():
                fn()
            w.step_index += 1
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            ev = evs[k]
            ev[0].record(stream)
            for i, fn in enumerate(step_fns[k]):
                fn()
                ev[i + 1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        w.step_index += args.steps
    in_step = {n: [evs[k][i].elapsed_time(evs[k][i + 1]) * 1000.0 for k in range(args.steps)]
               for i, n in enumerate(names)}
    step_ms = wall * 1000.0 / args.steps
    step_bytes = sum(nbytes.values())

    # ---- µs per call, each operation alone: after WARM_CALLS warm-up calls,
    # BLOCKS blocks of PER_BLOCK back-to-back calls, each block between two
    # events on the launch stream; the median block gives µs/call, beside its
    # 95th percentile (the MLA and video-O calls rotate over their buffer sets)
    def blocks_us(get_fn):
        for j in range(WARM_CALLS):
            get_fn(j)()
        fns = [get_fn(WARM_CALLS + j) for j in range(BLOCKS * PER_BLOCK)]
        evb = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(BLOCKS)]
        torch.cuda.synchronize()
        for b, (e0, e1) in enumerate(evb):
            e0.record(stream)
            for fn in fns[b * PER_BLOCK:(b + 1) * PER_BLOCK]:
                fn()
            e1.record(stream)
        torch.cuda.synchronize()
        per = sorted(e0.elapsed_time(e1) * 1000.0 / PER_BLOCK for e0, e1 in evb)
        return statistics.median(per), per[int(0.95 * (len(per) - 1))]

    iso_us, iso_p95, launches = {}, {}, {}
    with torch.cuda.stream(stream):
        for i, n in enumerate(names):
            iso_us[n], iso_p95[n] = blocks_us(lambda j, i=i: w.ops(k=j)[i][2])
            launches[n] = cam.last_launch()

    # ---- operations beyond the step (same µs/call method)
    ext = {}
    with torch.cuda.stream(stream):
        for i, (n, nb_ext, _) in enumerate(w.extension_ops()):
            us, p95 = blocks_us(lambda j, i=i: w.extension_ops(k=j)[i][2])
            ext[n] = {"us_per_call": round(us, 2), "us_per_call_p95": round(p95, 2), "algorithmic_bytes": int(nb_ext),
                      "last_launch": cam.last_launch(), "GBps": round(nb_ext / us / 1e3, 1),
                      "frac_of_hbm_peak": round(nb_ext / us / 1e3 / HBM_PEAK_GBPS, 4)}

    # ---- Q/K/V projection written into the head-sharded layout (MFMA); the
    # library GEMM (torch.mm) of the same product is timed beside it as a
    # reference, to be read with the seq->head relayout it would need
    with torch.cuda.stream(stream):
        P, S, H, D = w.vP, w.vS, w.vH, w.vD
        j_out = w.v_qkv_out  # [P][3][S][H/P][D]
        j_tmp = torch.empty((S, 3 * H * D), dtype=torch.bfloat16, device="cuda")

        def timed(fn, n=10):
            for _ in range(3):
                fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(n):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1000.0 / n

        j_us = timed(lambda: cam.qkv_projection_head_sharded(w.j_x, w.j_w, P, 3, H, D, out=j_out))
        j_launch = cam.last_launch()
        lib_us = timed(lambda: torch.mm(w.j_x, w.j_w.t(), out=j_tmp))
        del j_tmp
    projection = {
        "op": "qkv_projection_head_sharded_video_p4 (S=32760, K=3072, N=3x24x128)",
        "kernel": "k_proj_direct<false>", "bound": "mfma", "us_per_call": round(j_us, 2),
        "TFLOPs": round(w.j_flops / j_us / 1e6, 1), "peak_TFLOPs": MFMA_BF16_PEAK_TFLOPS,
        "frac_of_mfma_peak": round(w.j_flops / j_us / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4), "launch": j_launch,
        "reference_library_gemm_us": round(lib_us, 2),
        "reference_library_gemm_TFLOPs": round(w.j_flops / lib_us / 1e6, 1),
        "reference_note": "torch.mm (the platform's GEMM library) of the same product into [S][N]; it still "
                          "needs the seq->head relayout (relayout_seq_to_head_video_p4_qkv) to reach this layout",
    }

    # ---- plain-copy ceiling on the video Q/K/V operand size
    with torch.cuda.stream(stream):
        src, dst = w.v_qkv, w.v_qkv_out
        for _ in range(3):
            cam.copy(src, dst)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            cam.copy(src, dst)
        e1.record(stream)
        torch.cuda.synchronize()
    copy_bytes = 2 * src.numel() * src.element_size()
    copy_gbps = copy_bytes / (e0.elapsed_time(e1) * 100.0) / 1e3

    # ---- kernel-choice evidence: the direct seq->head kernel (A) against the
    # LDS-staged one (B) on the video P = 4 Q/K/V operand, paired A/B with a
    # null control
    ablations = [ab_decision(torch, stream, "relayout seq->head video P=4 QKV: direct 16-byte moves (A) vs "
                             f"LDS-staged, {LDS_ROWS_PER_TILE} rows per tile (B)",
                             lambda: cam.ulysses_seq_to_head(w.v_qkv, w.vP, out=w.v_qkv_out),
                             lambda: cam.ablation_seq_to_head_lds(w.v_qkv, w.vP, LDS_ROWS_PER_TILE,
                                                                  out=w.v_qkv_out))]

    # ---- plain-copy ceiling at each operation's own size: half its
    # algorithmic bytes each way; small sizes rotate over up to 8 disjoint
    # regions of one large pair so that repeated copies start cold, as the
    # operations' own timings do
    half_max = (max(nbytes.values()) // 2 + 15) // 16 * 16
    c_src = torch.empty(half_max, dtype=torch.uint8, device="cuda")
    c_dst = torch.empty(half_max, dtype=torch.uint8, device="cuda")
    copy_same = {}
    with torch.cuda.stream(stream):
        for n in names:
            half = max(16, nbytes[n] // 2 // 16 * 16)
            regions = max(1, min(8, half_max // half))
            fns = [lambda k=k: cam.copy(c_src[k * half:(k + 1) * half], c_dst[k * half:(k + 1) * half])
                   for k in range(regions)]
            for f in fns[:2]:
                f()
            calls = 10 if nbytes[n] > 2**30 else 40
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(calls):
                fns[i % regions]()
            e1.record(stream)
            torch.cuda.synchronize()
            copy_same[n] = 2 * half / (e0.elapsed_time(e1) * 1000.0 / calls) / 1e3
    del c_src, c_dst
    gc.enable()

    op_table = {}
    for n in names:
        us = iso_us[n]
        gbps = nbytes[n] / us / 1e3
        mean_step = statistics.mean(in_step[n])
        op_table[n] = {
            "kernel": kern[n],
            "algorithmic_bytes": int(nbytes[n]),
            "us_per_call": round(us, 2),
            "us_per_call_p95": round(iso_p95[n], 2),
            "GBps": round(gbps, 1),
            "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
            "copy_same_bytes_GBps": round(copy_same[n], 1),
            "frac_of_copy_ceiling": round(gbps / copy_same[n], 4),
            "in_step_us_mean": round(mean_step, 2),
            "in_step_us_median": round(statistics.median(in_step[n]), 2),
            "in_step_us_p95": round(sorted(in_step[n])[int(0.95 * (len(in_step[n]) - 1))], 2),
            "in_step_us_max": round(max(in_step[n]), 2),
            "in_step_GBps": round(nbytes[n] / mean_step / 1e3, 1),
            "launch": launches[n],
        }
    # the dominant kernel: the largest typical (median) share of the step; its
    # achieved rate uses the mean launch duration over the timed region
    dom = max(names, key=lambda n: statistics.median(in_step[n]))
    dom_us = statistics.mean(in_step[dom])
    for n in names:
        if max(in_step[n]) > 3.0 * statistics.median(in_step[n]):
            print(f"warning: {n} took {max(in_step[n]):.1f} us in one step (median {statistics.median(in_step[n]):.1f} us)",
                  file=sys.stderr, flush=True)
    dom_gbps = nbytes[dom] / dom_us / 1e3
    traffic = None
    if TRAFFIC_FILE.exists():
        try:
            tf = json.loads(TRAFFIC_FILE.read_text())
            if tf.get("kernel_source_hash") == kernel_source_hash() and dom in tf.get("ops", {}):
                traffic = tf["ops"][dom]["hbm_bytes_per_launch"]
        except (ValueError, KeyError):
            traffic = None
    result = {
        "metric": METRIC,
        "value": round(step_bytes / (step_ms * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "payload_dtype": "bf16",
        "data": "synthetic (seeded torch generator on the device; shapes and distributions of the pages' workloads)",
        "config": {
            "workload": "one pass of every hot-path operation: video-DiT Ulysses relayout P=4 (S=32760, H=24, "
                        "D=128; QKV seq->head B=3, O head->seq B=1) + MLA decode DCP P=8 (T=128, H=128, Dv=512; "
                        "LSE pack with 1% invalid statistics, strided-view exchange, stable combine) + packed THD "
                        "P=8 (20 short + 2 long sequences, 131072 tokens, H=32, D=128; varlen QKV seq->head, O "
                        "head->seq, causal combine of 8 KV-piece partials)",
            "step_algorithmic_bytes": int(step_bytes),
            "ops": names,
        },
        "roofline": {
            "kernel": kern[dom],
            "op": dom,
            "bound": "hbm",
            "achieved": round(dom_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(dom_gbps / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "avg_launch_us": round(dom_us, 2),
            "median_launch_us": round(statistics.median(in_step[dom]), 2),
            "algorithmic_bytes_per_launch": int(nbytes[dom]),
        },
        "extensions": ext,
        "projection": projection,
        "thd_plan": plan_summary(w),
        "ablations": ablations,
        "copy_ceiling": {"GBps": round(copy_gbps, 1), "frac_of_hbm_peak": round(copy_gbps / HBM_PEAK_GBPS, 4),
                         "bytes": int(copy_bytes), "kernel": "k_copy16"},
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                   "compute_units": props.multi_processor_count,
                   "hbm_GiB": round(props.total_memory / 2**30, 1)},
        "kernel_source_hash": kernel_source_hash(),
        "inputs_sha256": hashlib.sha256(json.dumps(digests, sort_keys=True).encode()).hexdigest()[:16],
        "inputs_sha256_note": "SHA-256 over the per-buffer digests (shape, dtype, first and last MiB of every "
                              "seeded input buffer); --digests-out writes them one by one",
        "timing": "value and ms_per_step: host clock around the K synchronized steps; ops[*].us_per_call: "
                  f"after {WARM_CALLS} warm-up calls, {BLOCKS} blocks of {PER_BLOCK} back-to-back calls of that "
                  "operation alone, each block between two HIP events: the median block (us_per_call_p95: its "
                  "95th percentile); ops[*].in_step_*: HIP events around the operation inside the steps",
    }
    result["cpu_baseline"], result["parity"] = (None, None) if args.no_cpu_baseline else cpu_leg(w, args.cpu_threads)
    # the gated figures and the per-operation table last, so that the end of
    # the line carries them
    result["gates"] = {n: {"us_per_call": op_table[n]["us_per_call"],
                           "frac_of_hbm_peak": op_table[n]["frac_of_hbm_peak"],
                           "in_step_us_mean": op_table[n]["in_step_us_mean"]}
                       for n in ("relayout_seq_to_head_video_p4_qkv", "relayout_head_to_seq_video_p4_o",
                                 "lse_combine_mla")}
    result["ops"] = op_table
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
