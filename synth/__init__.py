"""Seeded synthetic inputs shared by the oracle-side and the GPU-side of the
tests and the benchmark.

This module holds none of the method's arithmetic: it only draws random
values with the distributions and shapes of the pages' workloads and lays out
the packed-THD length mix.  Everything is deterministic in the seed.

Host tensors come from a seeded CPU ``torch.Generator``; large benchmark
tensors can be drawn on the GPU from a seeded CUDA generator instead (the
values then differ from the host draw for the same seed but are just as
deterministic).  bf16/fp16 values are float32 draws rounded by torch's own
dtype conversion (round to nearest even).
"""

from __future__ import annotations

import math

import numpy as np
import torch

BASE_SEED = 20260913  # BF16 producer seed of the Ascend DCP pack measurement
FP16_SEED = 20260914  # FP16 correctness seed of the same protocol

_TORCH_DT = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


def _gen(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & 0xFFFF_FFFF_FFFF)
    return g


def normal(shape, seed: int, std: float = 1.0, mean: float = 0.0, dtype: str = "bf16",
           device="cpu") -> torch.Tensor:
    """~N(mean, std^2) drawn in float32, stored as `dtype`."""
    g = _gen(seed, device)
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32, device=device)
    if std != 1.0:
        x.mul_(std)
    if mean != 0.0:
        x.add_(mean)
    return x.to(_TORCH_DT[dtype])


def uniform(shape, seed: int, lo: float, hi: float, device="cpu") -> torch.Tensor:
    """~U(lo, hi) float32."""
    g = _gen(seed, device)
    x = torch.rand(tuple(shape), generator=g, dtype=torch.float32, device=device)
    return x.mul_(hi - lo).add_(lo)


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw storage bits of a CPU tensor as a numpy array (uint16 for 2-byte
    dtypes, uint32 for 4-byte ones)."""
    t = t.detach().cpu().contiguous()
    if t.element_size() == 2:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.element_size() == 4:
        return t.view(torch.int32).numpy().view(np.uint32)
    raise TypeError(f"unsupported element size {t.element_size()}")


def iota16(n: int) -> np.ndarray:
    """Distinct 16-bit words 0, 1, ... (wrapping) -- an index payload."""
    return (np.arange(n, dtype=np.int64) & 0xFFFF).astype(np.uint16)


def iota32(n: int) -> np.ndarray:
    """Distinct 32-bit words: a payload that names its own source index."""
    return np.arange(n, dtype=np.uint32)


# -- relayout operands (video DiT Ulysses shapes) -----------------------------

def relayout_seq_side(P, B, S, H, D, seed, dtype="bf16", device="cpu") -> torch.Tensor:
    """Sequence-sharded operand [P][B][S/P][H][D], ~N(0,1)."""
    return normal((P, B, S // P, H, D), seed, dtype=dtype, device=device)


def relayout_head_side(P, B, S, H, D, seed, dtype="bf16", device="cpu") -> torch.Tensor:
    """Head-sharded operand [P][B][S][H/P][D], ~N(0,1)."""
    return normal((P, B, S, H // P, D), seed, dtype=dtype, device=device)


# -- MLA-style DCP decode statistics ------------------------------------------

CORRUPTION_KINDS = ("max=+inf", "max=-inf", "max=nan", "sum=nan", "sum=+inf", "sum=+0",
                    "sum=-0", "sum<0")


def dcp_partials(P, T, H, Dv, seed, dtype="bf16", corrupt_frac=0.01, device="cpu"):
    """Per-rank partial outputs and softmax statistics of a DCP decode step.

    out ~N(0,1) [P][T][H][Dv]; softmax_max ~N(0, 4) (sigma 2) and
    softmax_sum ~U(0.5, 64), both fp32 [P][T][H].  Exactly
    ceil(corrupt_frac * P*T*H) distinct (p, t, h) entries, chosen by a seeded
    permutation, are corrupted, cycling through CORRUPTION_KINDS.
    Returns (out, smax, ssum, corrupted_flat_indices)."""
    out = normal((P, T, H, Dv), seed, dtype=dtype, device=device)
    smax = normal((P, T, H), seed + 101, std=2.0, dtype="fp32", device=device)
    ssum = uniform((P, T, H), seed + 202, 0.5, 64.0, device=device)
    n = P * T * H
    k = math.ceil(corrupt_frac * n) if corrupt_frac > 0 else 0
    idx = torch.randperm(n, generator=_gen(seed + 303))[:k]
    if k:
        neg = uniform((k,), seed + 404, 0.5, 64.0)
        mf = smax.view(-1)
        sf = ssum.view(-1)
        kinds = torch.arange(k) % len(CORRUPTION_KINDS)
        idx_d = idx.to(device)
        vals_m = mf[idx_d].cpu()
        vals_s = sf[idx_d].cpu()
        for j, kind in enumerate(CORRUPTION_KINDS):
            sel = kinds == j
            if kind == "max=+inf":
                vals_m[sel] = math.inf
            elif kind == "max=-inf":
                vals_m[sel] = -math.inf
            elif kind == "max=nan":
                vals_m[sel] = math.nan
            elif kind == "sum=nan":
                vals_s[sel] = math.nan
            elif kind == "sum=+inf":
                vals_s[sel] = math.inf
            elif kind == "sum=+0":
                vals_s[sel] = 0.0
            elif kind == "sum=-0":
                vals_s[sel] = -0.0
            elif kind == "sum<0":
                vals_s[sel] = -neg[sel]
        mf[idx_d] = vals_m.to(device)
        sf[idx_d] = vals_s.to(device)
    return out, smax, ssum, idx.numpy()


# -- packed THD (varlen) workload ---------------------------------------------

def thd_lengths(n_short: int, total: int, seed: int, lo: int = 512, hi: int = 4096,
                n_long: int = 2, align: int = 1) -> np.ndarray:
    """n_short lengths ~U{lo..hi} plus n_long long sequences that fill `total`
    tokens (the remainder split as evenly as integers allow), in a seeded
    random order.  With align > 1 every length is a multiple of it (short
    lengths rounded down, at least align; total must be a multiple)."""
    rng = np.random.default_rng(seed)
    short = rng.integers(lo, hi + 1, size=n_short).astype(np.int64)
    if align > 1:
        assert total % align == 0
        short = np.maximum(short // align * align, align)
    rem = (total - int(short.sum())) // align
    assert rem >= n_long, "total too small for the short sequences"
    longs = [align * (rem // n_long + (1 if i < rem % n_long else 0)) for i in range(n_long)]
    lens = np.concatenate([short, np.array(sorted(longs), dtype=np.int64)])
    rng.shuffle(lens)
    return lens


def cu_seqlens(lengths) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(lengths.size + 1, dtype=np.int64)
    np.cumsum(lengths, out=cu[1:])
    assert cu[-1] < 2**31
    return cu.astype(np.int32)


def random_lengths(nseq: int, seed: int, lo: int = 0, hi: int = 40) -> np.ndarray:
    """Ragged lengths ~U{lo..hi} (zero-length sequences allowed when lo = 0)."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=nseq).astype(np.int64)


def partial_lse(shape, seed, device="cpu") -> torch.Tensor:
    """Partial log-sum-exp values for combine inputs: ~N(0, 4) (sigma 2), fp32."""
    return normal(shape, seed, std=2.0, dtype="fp32", device=device)
