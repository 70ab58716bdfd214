"""GPU parity of the Q/K/V projection written into the head-sharded layout
(MFMA) against the oracle's double-precision product: every element within
one unit in the last place of the payload type plus the fp32 accumulation
bound 2e-5 * sum_k |x_k w_k|; small shapes with a ragged row tile, fp16, and
the video DiT P = 4 shape on 632 sampled rows (the first and the tail tile
whole)."""

import numpy as np
import pytest
import torch

import synth
from helpers import announce, to_host_bits, window_pool

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cam():
    import context_attention_movement_amd as m
    m.library()
    assert torch.cuda.is_available()
    return m


def _check(orc, got_bits, x_bits, w_bits, P, B, H, D, dt, what):
    want = orc.qkv_projection(x_bits, w_bits, P, B, H, D, dt)
    g = orc.half_bits_to_double(got_bits, dt)
    o = orc.half_bits_to_double(want, dt)
    xa = np.abs(orc.half_bits_to_double(x_bits, dt))
    wa = np.abs(orc.half_bits_to_double(w_bits, dt))
    S = x_bits.shape[0]
    sabs = (xa @ wa.T).reshape(S, B, P, H // P, D).transpose(2, 1, 0, 3, 4)
    ulp = np.abs(o) * (2.0 ** -7 if dt == "bf16" else 2.0 ** -10)
    err = np.abs(g - o)
    bad = err > ulp + 2e-5 * sabs
    assert not np.isnan(g).any(), f"{what}: NaN"
    assert not bad.any(), f"{what}: {int(bad.sum())} elements out of tolerance, worst {float(err.max())}"


CASES = [  # (S, K, P, B, H, D, dtype)
    (300, 128, 2, 3, 4, 64, "bf16"),
    (257, 64, 4, 1, 8, 32, "bf16"),      # ragged last row tile
    (64, 192, 2, 2, 2, 64, "fp16"),
    (512, 256, 8, 1, 16, 16, "bf16"),    # Hp*D = 32: a 256-column tile spans 8 head blocks
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "S{}K{}P{}B{}H{}D{}{}".format(*c))
def test_projection(cam, orc, case):
    S, K, P, B, H, D, dt = case
    announce(f"projection {case}")
    x = synth.normal((S, K), seed=S + K, dtype=dt)
    w = synth.normal((B * H * D, K), seed=S + K + 1, std=0.05, dtype=dt)
    out = cam.qkv_projection_head_sharded(x.cuda(), w.cuda(), P, B, H, D)
    torch.cuda.synchronize()
    _check(orc, to_host_bits(out), synth.bits(x), synth.bits(w), P, B, H, D, dt, str(case))


def _random_cases(n, seed):
    """Seeded shapes inside the ABI's limits: K a multiple of 64, B*H*D a
    multiple of 256, H divisible by P; S ragged against the 256-row tile."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        P = int(rng.choice([1, 2, 4, 8]))
        B = int(rng.integers(1, 4))
        H = P * int(rng.integers(1, 5))
        D = int(rng.choice([8, 16, 32, 64, 128]))
        if (B * H * D) % 256:
            continue
        S = P * int(rng.integers(1, 160))
        K = 64 * int(rng.integers(1, 7))
        out.append((S, K, P, B, H, D, "bf16" if len(out) % 3 else "fp16"))
    return out


@pytest.mark.parametrize("case", _random_cases(10, 20260913), ids=lambda c: "S{}K{}P{}B{}H{}D{}{}".format(*c))
def test_projection_random_shapes(cam, orc, case):
    S, K, P, B, H, D, dt = case
    announce(f"projection random shape {case}")
    x = synth.normal((S, K), seed=S * 7 + K, dtype=dt)
    w = synth.normal((B * H * D, K), seed=S * 7 + K + 1, std=0.05, dtype=dt)
    out = cam.qkv_projection_head_sharded(x.cuda(), w.cuda(), P, B, H, D)
    torch.cuda.synchronize()
    _check(orc, to_host_bits(out), synth.bits(x), synth.bits(w), P, B, H, D, dt, str(case))


def test_projection_video_shape_sampled_rows(cam, orc):
    """Video DiT P = 4: S = 32760 (127 full row tiles and a ragged one),
    K = 3072, Q/K/V of 24 heads x 128.  Every output column of 632 token rows:
    the whole first row tile, the whole ragged last one, and 128 seeded
    random rows between them (the oracle over row chunks on host threads)."""
    S, K, P, B, H, D = 32760, 3072, 4, 3, 24, 128
    announce("projection video shape")
    g = synth._gen(synth.BASE_SEED + 92, "cuda")
    x = torch.randn((S, K), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    w = (torch.randn((B * H * D, K), generator=g, device="cuda", dtype=torch.float32) * 0.02).to(torch.bfloat16)
    out = cam.qkv_projection_head_sharded(x, w, P, B, H, D)
    torch.cuda.synchronize()
    rng = np.random.default_rng(synth.BASE_SEED + 93)
    rows = np.unique(np.concatenate([np.arange(0, 256), np.arange(32512, S),
                                     rng.choice(np.arange(256, 32512), size=128, replace=False)]))
    assert rows.size == 632
    xh, wh, oh = to_host_bits(x), to_host_bits(w), to_host_bits(out)
    chunks = np.array_split(rows, 16)

    def check(a, e):
        for c in chunks[a:e]:
            _check(orc, np.ascontiguousarray(oh[:, :, c]), np.ascontiguousarray(xh[c]), wh, P, B, H, D, "bf16",
                   f"video rows {int(c[0])}..{int(c[-1])}")

    window_pool(len(chunks), check, n_windows=len(chunks))


_CAPTURE_FIRST = r"""
import sys, torch
sys.path.insert(0, sys.argv[1])
import context_attention_movement_amd as cam
torch.cuda.set_device(0)
S, K, P, B, H, D = 300, 128, 2, 3, 4, 64
g = torch.Generator(device="cuda").manual_seed(5)
x = torch.randn(S, K, device="cuda", generator=g).to(torch.bfloat16)
w = (torch.randn(B * H * D, K, device="cuda", generator=g) * 0.1).to(torch.bfloat16)
out = torch.empty((P, B, S, H // P, D), device="cuda", dtype=torch.bfloat16)
graph = torch.cuda.CUDAGraph()
with torch.cuda.graph(graph):   # the process's first call of the projection
    cam.qkv_projection_head_sharded(x, w, P, B, H, D, out=out)
torch.cuda.synchronize()
out.zero_()
graph.replay()
ref = cam.qkv_projection_head_sharded(x, w, P, B, H, D)
torch.cuda.synchronize()
sys.exit(0 if torch.equal(out, ref) else 3)
"""


def test_projection_first_call_inside_graph_capture():
    """A caller may capture the projection before ever calling it eagerly (the
    kernel's large-LDS attribute is then set during the capture): in a fresh
    process, the replay equals an eager call bit for bit."""
    import subprocess
    import sys
    from pathlib import Path
    announce("projection: first call inside a graph capture (child process)")
    root = str(Path(__file__).resolve().parents[1])
    r = subprocess.run([sys.executable, "-c", _CAPTURE_FIRST, root], capture_output=True, text=True, timeout=180)
    assert r.returncode == 0, f"child exited {r.returncode}: {r.stderr[-2000:]}"
