"""Shared comparison helpers for the GPU parity tests (test code only)."""

from __future__ import annotations

import numpy as np
import torch

LSE_ATOL = 1e-5          # fp32 LSE: max abs error
OUT_ROW_RTOL = 8e-3      # combined payload: per-row max|g - o| / max|o|


def announce(msg: str) -> None:
    print(f"[case] {msg}", flush=True)


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous().cpu()
    if t.element_size() == 2:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.element_size() == 4:
        return t.view(torch.int32).numpy().view(np.uint32)
    if t.element_size() == 1:
        return t.view(torch.uint8).numpy()
    raise TypeError(t.dtype)


def from_host_bits(a: np.ndarray, dtype: torch.dtype, device="cuda") -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(dtype).to(device)
    if a.dtype == np.uint32:
        return torch.from_numpy(a.view(np.int32)).view(dtype).to(device)
    raise TypeError(a.dtype)


def assert_bits_equal(got: np.ndarray, want: np.ndarray, what: str) -> None:
    got = got.reshape(-1)
    want = want.reshape(-1)
    assert got.shape == want.shape, what
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{what}: {bad.size} mismatching elements, first at {bad[:5].tolist()}"


def assert_lse_close(got: np.ndarray, want: np.ndarray, what: str) -> float:
    got = got.reshape(-1).astype(np.float64)
    want = want.reshape(-1).astype(np.float64)
    assert not np.isnan(got).any(), f"{what}: NaN in LSE"
    gi, wi = np.isneginf(got), np.isneginf(want)
    assert np.array_equal(gi, wi), f"{what}: -inf pattern differs at {np.nonzero(gi != wi)[0][:5].tolist()}"
    assert not np.isposinf(got).any()
    f = ~wi
    err = float(np.max(np.abs(got[f] - want[f]))) if f.any() else 0.0
    assert err <= LSE_ATOL, f"{what}: max abs LSE error {err}"
    return err


def assert_rows_close(got: np.ndarray, want: np.ndarray, what: str) -> float:
    """got, want: float64 [rows][D].  Per row max|g-o| / max|o| <= 8e-3; rows
    whose reference is all zero must be exactly zero; no NaN."""
    assert not np.isnan(got).any(), f"{what}: NaN in output"
    num = np.max(np.abs(got - want), axis=-1)
    den = np.max(np.abs(want), axis=-1)
    zero = den == 0
    assert np.all(num[zero] == 0), f"{what}: nonzero output where the oracle is zero"
    rel = num[~zero] / den[~zero] if (~zero).any() else np.zeros(1)
    worst = float(np.max(rel))
    assert worst <= OUT_ROW_RTOL, f"{what}: worst row relative error {worst}"
    return worst


GRAD_LSE_RTOL = 1e-5     # gradient of the partial LSEs, relative to the row scale


def grad_lse_scale(po: np.ndarray, go: np.ndarray, gl: np.ndarray | None) -> np.ndarray:
    """Row scale of dL_p = w_p (<g, O_p> - sum_q w_q <g, O_q> + g_lse): with
    the weights in [0, 1] summing to one, |dL_p| <= 2 sum_d |g_d| max_p |O_pd|
    + |g_lse|, and fp32 rounding of the dot products is relative to that sum.
    po float64 [P][R][D] (non-finite entries of invalid partials ignored),
    go float64 [R][D], gl float64 [R] or None -> [R]."""
    amax = np.max(np.where(np.isfinite(po), np.abs(po), 0.0), axis=0)
    s = np.sum(np.abs(go) * amax, axis=-1)
    return s + (np.abs(gl) if gl is not None else 0.0)


def assert_grad_lse_close(got: np.ndarray, want: np.ndarray, scale: np.ndarray, what: str) -> float:
    """got, want: [P][R] fp32; scale [R].  |got - want| <= 1e-5 * scale (plus
    the fp32 spacing of the value), exact zeros where the oracle is exactly
    zero (partials outside the valid set), no NaN."""
    got = got.astype(np.float64)
    want = want.astype(np.float64)
    assert not np.isnan(got).any(), f"{what}: NaN in the LSE gradient"
    zero = want == 0
    assert np.all(got[zero] == 0), f"{what}: nonzero gradient where the oracle is exactly zero"
    err = np.abs(got - want)
    tol = GRAD_LSE_RTOL * scale[None, :] + np.spacing(np.abs(want).astype(np.float32)).astype(np.float64)
    bad = err > tol
    assert not bad.any(), f"{what}: {int(bad.sum())} LSE-gradient entries out of tolerance, worst " \
                          f"{float(np.max(err / np.maximum(tol, 1e-300)))} x tol"
    return float(np.max(err / np.maximum(scale[None, :], 1e-30)))


def window_pool(T: int, fn, n_windows: int = 64, threads: int | None = None) -> list:
    """Call fn(a, e) on token windows [a, e) that cover [0, T), from a pool of
    threads (the oracle's C calls and numpy's large array operations release
    the GIL); returns the results in window order.  Used to compare a whole
    full-size result with the oracle in seconds."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    threads = threads or max(1, min(16, len(os.sched_getaffinity(0))))
    n = max(1, min(n_windows, T))
    bounds = [(k * T // n, (k + 1) * T // n) for k in range(n)]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(lambda ae: fn(*ae), bounds))
