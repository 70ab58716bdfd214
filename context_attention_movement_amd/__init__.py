"""context_attention_movement_amd -- MI355X-native per-GPU hot path of
sequence/context-parallel attention movement.

A thin ctypes binding over ``libcam.so`` (C ABI in ``include/cam.h``): the
Ulysses all-to-all relayout between sequence-sharded and head-sharded slabs of
P logical ranks held in one GPU's HBM (dense and cu_seqlens varlen), the
max/sum-aware LSE pack into the packed exchange layout, and the stable
LSE-weighted combine.  Every step runs in the library's HIP kernels; this
module only checks tensor metadata, allocates outputs with torch, and passes
pointers, sizes and the current HIP stream.  There is no fallback: if the
library is missing, every call raises.
"""

from __future__ import annotations

import ctypes as C
from dataclasses import dataclass
from pathlib import Path

import numpy as np
import torch

__all__ = [
    "CamError", "library", "abi_version",
    "ulysses_seq_to_head", "ulysses_head_to_seq",
    "VarlenPlan", "ulysses_varlen_plan", "ulysses_seq_to_head_varlen", "ulysses_head_to_seq_varlen",
    "ThdPlannerConfig", "ThdPlan", "thd_plan", "ulysses_seq_to_head_spans", "ulysses_head_to_seq_spans",
    "lse_combine_planned",
    "lse_pack_bytes", "lse_pack", "lse_combine_packed", "lse_combine", "lse_combine_varlen",
    "lse_combine_packed_seq", "lse_combine_varlen_seq", "lse_merge", "lse_combine_backward",
    "empty_partials", "qkv_projection_head_sharded", "ablation_seq_to_head_lds", "copy", "last_launch",
]

LIB_PATH = Path(__file__).resolve().parent / "libcam.so"

CAM_BF16, CAM_FP16, CAM_FP32 = 0, 1, 2
STATUS = ["CAM_OK", "CAM_ERR_NULL", "CAM_ERR_SHAPE", "CAM_ERR_DIVISIBILITY", "CAM_ERR_ALIGNMENT",
          "CAM_ERR_OVERLAP", "CAM_ERR_UNSUPPORTED", "CAM_ERR_HIP"]


class CamError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        self.status_name = STATUS[status] if 0 <= status < len(STATUS) else str(status)
        super().__init__(f"{self.status_name}: {message}")


_lib = None
_i64, _vp, _int = C.c_int64, C.c_void_p, C.c_int

_SIGNATURES = {
    "cam_status_string": (C.c_char_p, [_int]),
    "cam_last_error": (C.c_char_p, []),
    "cam_abi_version": (_int, []),
    "cam_last_launch": (_int, [_vp, _vp, _vp]),
    "ulysses_seq_to_head": (_int, [_vp, _vp, _i64, _i64, _i64, _i64, _i64, _int, _vp]),
    "ulysses_head_to_seq": (_int, [_vp, _vp, _i64, _i64, _i64, _i64, _i64, _int, _vp]),
    "ulysses_varlen_plan": (_int, [_vp, _i64, _i64, _vp, _vp]),
    "ulysses_seq_to_head_varlen": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64,
                                          _int, _vp]),
    "ulysses_head_to_seq_varlen": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64,
                                          _int, _vp]),
    "lse_pack_bytes": (_i64, [_i64, _i64, _i64, _i64, _int, _int]),
    "lse_pack": (_int, [_vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64,
                        _i64, _i64, _i64, _i64, _int, _int, _vp, _vp]),
    "lse_combine_packed": (_int, [_vp, _i64, _i64, _i64, _i64, _int, _int, _vp, _vp, _vp]),
    "lse_combine": (_int, [_vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _int,
                           _vp, _i64, _i64, _vp, _i64, _i64, _vp]),
    "lse_combine_varlen": (_int, [_vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                  _int, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _vp]),
    "cam_copy": (_int, [_vp, _vp, _i64, _vp]),
    "cam_ablation_seq_to_head_lds": (_int, [_vp, _vp, _i64, _i64, _i64, _i64, _i64, _int, _i64, _vp]),
    "qkv_projection_head_sharded": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _int, _vp]),
    "thd_plan": (_int, [_vp, _i64, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "thd_plan_first_positions": (_int, [_vp, _i64, _i64, _vp, _vp, _i64, _vp]),
    "lse_combine_planned": (_int, [_vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                   _int, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _vp, _i64, _vp]),
    "lse_combine_planned_backward": (_int, [_vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64, _i64, _i64, _i64,
                                            _i64, _int, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64,
                                            _i64, _vp, _i64, _i64, _i64, _vp, _vp, _i64, _vp]),
    "ulysses_seq_to_head_spans": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64,
                                         _int, _vp]),
    "ulysses_head_to_seq_spans": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64,
                                         _int, _vp]),
    "lse_combine_backward": (_int, [_vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                    _int, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _i64,
                                    _vp, _i64, _i64, _i64, _vp]),
    "lse_combine_varlen_backward": (_int, [_vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64, _i64, _i64, _i64,
                                           _i64, _int, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64,
                                           _i64, _vp, _i64, _i64, _i64, _vp, _i64, _vp]),
    "lse_combine_packed_seq": (_int, [_vp, _i64, _i64, _i64, _i64, _int, _int, _vp, _vp, _vp]),
    "lse_combine_varlen_seq": (_int, [_vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                      _int, _vp, _vp, _vp, _vp, _vp, _i64, _vp]),
    "lse_merge": (_int, [_vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _i64, _i64, _i64,
                         _int, _vp, _i64, _i64, _vp]),
}


def library() -> C.CDLL:
    """Load libcam.so (built by ``python -m context_attention_movement_amd.build``)."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m context_attention_movement_amd.build` (no fallback exists)")
        lib = C.CDLL(str(LIB_PATH))
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def abi_version() -> int:
    return library().cam_abi_version()


def _check(status: int) -> None:
    if status != 0:
        raise CamError(status, library().cam_last_error().decode())


def _dt(t: torch.Tensor, relayout: bool = False) -> int:
    if t.dtype == torch.bfloat16:
        return CAM_BF16
    if t.dtype == torch.float16:
        return CAM_FP16
    if relayout and t.element_size() == 4:
        return CAM_FP32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _contig(t: torch.Tensor, name: str) -> None:
    _dev(t, name)
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _tables_on(ref: torch.Tensor, *tables: torch.Tensor) -> None:
    """A plan's device tables must live on the device of the data they index
    (a host table's address handed to a kernel would be read as device memory)."""
    for t in tables:
        if t.device != ref.device:
            raise ValueError(f"the plan's tables are on {t.device}, the data on {ref.device}: "
                             "build the plan for that device (device=...) or move it there")


def _check_buffer(t: torch.Tensor, name: str, shape, dtype: torch.dtype, contiguous: bool = True,
                  inner_contiguous: bool = False) -> None:
    """A caller-supplied output or input buffer: its shape and dtype must be
    exactly what the call writes or reads, checked before any device check
    or launch (the C ABI derives every extent from the sizes it is given, so
    a short buffer would be written out of bounds)."""
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} must have shape {tuple(int(x) for x in shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if inner_contiguous and t.dim() and t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError(f"{name} must have its last dimension contiguous")


def _check_packed(packed: torch.Tensor, P: int, T: int, H: int, Dv: int, scatter_dim: int,
                  dtype: torch.dtype) -> None:
    """The packed exchange buffer must be contiguous and hold at least
    lse_pack_bytes(P, T, H, Dv, scatter_dim) bytes."""
    if dtype not in (torch.bfloat16, torch.float16):
        raise TypeError(f"payload dtype must be bfloat16 or float16, got {dtype}")
    n = lse_pack_bytes(P, T, H, Dv, scatter_dim, dtype)
    if not packed.is_contiguous():
        raise ValueError("packed must be contiguous")
    if packed.numel() * packed.element_size() < n:
        raise ValueError(f"packed needs {n} bytes, got {packed.numel() * packed.element_size()}")


# ---------------------------------------------------------------------------
# Dense relayout
# ---------------------------------------------------------------------------

def ulysses_seq_to_head(x: torch.Tensor, P: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """[P][B][S/P][H][D] (rank j's sequence shard) -> [P][B][S][H/P][D]
    (rank r's head shard), bits copied."""
    _contig(x, "x")
    if x.dim() != 5 or x.shape[0] != P:
        raise ValueError("x must be [P][B][S/P][H][D]")
    _, B, Sp, H, D = x.shape
    S = Sp * P
    if H % P:
        raise ValueError("H must be a multiple of P")
    if out is None:
        out = torch.empty((P, B, S, H // P, D), dtype=x.dtype, device=x.device)
    _contig(out, "out")
    if out.numel() != x.numel() or out.dtype != x.dtype:
        raise ValueError("out must match x in size and dtype")
    _check(library().ulysses_seq_to_head(x.data_ptr(), out.data_ptr(), P, B, S, H, D, _dt(x, True),
                                         _stream(x)))
    return out


def ulysses_head_to_seq(x: torch.Tensor, P: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """[P][B][S][H/P][D] -> [P][B][S/P][H][D] (inverse of ulysses_seq_to_head)."""
    _contig(x, "x")
    if x.dim() != 5 or x.shape[0] != P:
        raise ValueError("x must be [P][B][S][H/P][D]")
    _, B, S, Hp, D = x.shape
    H = Hp * P
    if S % P:
        raise ValueError("S must be a multiple of P")
    if out is None:
        out = torch.empty((P, B, S // P, H, D), dtype=x.dtype, device=x.device)
    _contig(out, "out")
    if out.numel() != x.numel() or out.dtype != x.dtype:
        raise ValueError("out must match x in size and dtype")
    _check(library().ulysses_head_to_seq(x.data_ptr(), out.data_ptr(), P, B, S, H, D, _dt(x, True),
                                         _stream(x)))
    return out


# ---------------------------------------------------------------------------
# Varlen relayout
# ---------------------------------------------------------------------------

@dataclass
class VarlenPlan:
    """Host plan and its device copies for a packed THD batch over P ranks."""
    P: int
    nseq: int
    total_tokens: int
    cu_host: np.ndarray        # int32 [nseq+1]
    rank_cu_host: np.ndarray   # int32 [P][nseq+1]
    rank_off_host: np.ndarray  # int64 [P+1]
    cu: torch.Tensor           # device copies
    rank_cu: torch.Tensor
    rank_off: torch.Tensor

    def tokens_on_rank(self, p: int) -> int:
        return int(self.rank_off_host[p + 1] - self.rank_off_host[p])


def ulysses_varlen_plan(cu_seqlens, P: int, device="cuda") -> VarlenPlan:
    """Build the per-rank piece tables on the host (libcam) and upload them."""
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    nseq = cu.size - 1
    if nseq < 0:
        raise ValueError("cu_seqlens must have at least one entry")
    rank_cu = np.empty((P, nseq + 1), dtype=np.int32)
    rank_off = np.empty(P + 1, dtype=np.int64)
    _check(library().ulysses_varlen_plan(cu.ctypes.data, nseq, P, rank_cu.ctypes.data, rank_off.ctypes.data))
    dev = torch.device(device)
    return VarlenPlan(P, nseq, int(cu[-1]), cu, rank_cu, rank_off,
                      torch.from_numpy(cu).to(dev), torch.from_numpy(rank_cu).to(dev),
                      torch.from_numpy(rank_off).to(dev))


def ulysses_seq_to_head_varlen(x: torch.Tensor, plan: VarlenPlan, B: int = 1,
                               out: torch.Tensor | None = None) -> torch.Tensor:
    """Rank-major ragged [B*T][H][D] -> [P][B][T][H/P][D]."""
    _contig(x, "x")
    T, P = plan.total_tokens, plan.P
    if x.dim() != 3 or x.shape[0] != B * T:
        raise ValueError("x must be [B*T][H][D]")
    H, D = x.shape[1], x.shape[2]
    if out is None:
        out = torch.empty((P, B, T, H // P, D), dtype=x.dtype, device=x.device)
    _contig(out, "out")
    if out.numel() != x.numel() or out.dtype != x.dtype:
        raise ValueError("out must match x in size and dtype")
    _tables_on(x, plan.cu, plan.rank_cu, plan.rank_off)
    _check(library().ulysses_seq_to_head_varlen(
        x.data_ptr(), out.data_ptr(), plan.cu.data_ptr(), plan.rank_cu.data_ptr(), plan.rank_off.data_ptr(),
        plan.nseq, T, P, B, H, D, _dt(x, True), _stream(x)))
    return out


def ulysses_head_to_seq_varlen(x: torch.Tensor, plan: VarlenPlan, out: torch.Tensor | None = None) -> torch.Tensor:
    """[P][B][T][H/P][D] -> rank-major ragged [B*T][H][D]."""
    _contig(x, "x")
    T, P = plan.total_tokens, plan.P
    if x.dim() != 5 or x.shape[0] != P or x.shape[2] != T:
        raise ValueError("x must be [P][B][T][H/P][D]")
    B, D = x.shape[1], x.shape[4]
    H = x.shape[3] * P
    if out is None:
        out = torch.empty((B * T, H, D), dtype=x.dtype, device=x.device)
    _contig(out, "out")
    if out.numel() != x.numel() or out.dtype != x.dtype:
        raise ValueError("out must match x in size and dtype")
    _tables_on(x, plan.cu, plan.rank_cu, plan.rank_off)
    _check(library().ulysses_head_to_seq_varlen(
        x.data_ptr(), out.data_ptr(), plan.cu.data_ptr(), plan.rank_cu.data_ptr(), plan.rank_off.data_ptr(),
        plan.nseq, T, P, B, H, D, _dt(x, True), _stream(x)))
    return out


# ---------------------------------------------------------------------------
# THD layout planner and planned relayout
# ---------------------------------------------------------------------------

class _PlannerConfig(C.Structure):
    _fields_ = [("block_size", C.c_int64), ("min_split_tokens", C.c_int64), ("max_chunks_per_rank", C.c_int64),
                ("token_weight", C.c_double), ("causal_weight", C.c_double), ("mode", C.c_int64)]


@dataclass
class ThdPlannerConfig:
    """Planner inputs (cuLA THD planner): block size, the length below which a
    sample is short (kept whole), the span limit per rank, the cost weights of
    a token at position k (token_weight + causal_weight * (k + 1)), and
    contiguous=True for the contiguous block-balanced layout only."""
    block_size: int = 64
    min_split_tokens: int = 8192
    max_chunks_per_rank: int = 64
    token_weight: float = 1.0
    causal_weight: float = 1.0
    contiguous: bool = False

    def _c(self) -> _PlannerConfig:
        for name in ("block_size", "min_split_tokens", "max_chunks_per_rank"):
            v = getattr(self, name)
            if isinstance(v, bool) or not isinstance(v, (int, np.integer)):
                raise TypeError(f"{name} must be an integer")
        for name in ("token_weight", "causal_weight"):
            v = getattr(self, name)
            if isinstance(v, bool) or not isinstance(v, (int, float, np.floating, np.integer)):
                raise TypeError(f"{name} must be a number")
        return _PlannerConfig(int(self.block_size), int(self.min_split_tokens), int(self.max_chunks_per_rank),
                              float(self.token_weight), float(self.causal_weight), 1 if self.contiguous else 0)


@dataclass
class ThdPlan:
    """A THD layout plan: host tables, their device copies, per-rank costs and
    the chosen candidate (0 = contiguous layout, g >= 1 = grid g)."""
    world_size: int
    total_tokens: int
    cu_host: np.ndarray
    span_start_host: np.ndarray  # int32 [n+1]
    span_rank_host: np.ndarray   # int32 [n]
    span_local_host: np.ndarray  # int32 [n]
    rank_off_host: np.ndarray    # int64 [W+1]
    rank_cost: np.ndarray        # float64 [W]
    grid: int
    span_start: torch.Tensor | None = None
    span_rank: torch.Tensor | None = None
    span_local: torch.Tensor | None = None
    rank_off: torch.Tensor | None = None
    cu: torch.Tensor | None = None
    first_pos: torch.Tensor | None = None

    @property
    def first_pos_host(self) -> np.ndarray:
        """[W][nseq] int32: smallest position of sequence i held by rank p
        (INT32_MAX if none) -- the admission table of the planned combine."""
        if getattr(self, "_first", None) is None:
            nseq = self.cu_host.size - 1
            first = np.empty((self.world_size, nseq), dtype=np.int32)
            _check(library().thd_plan_first_positions(
                self.cu_host.ctypes.data, nseq, self.world_size, self.span_start_host.ctypes.data,
                self.span_rank_host.ctypes.data, self.n_spans, first.ctypes.data))
            self._first = first
        return self._first

    @property
    def n_spans(self) -> int:
        return int(self.span_rank_host.size)

    def tokens_on_rank(self, r: int) -> int:
        return int(self.rank_off_host[r + 1] - self.rank_off_host[r])

    def for_rank(self, r: int) -> list[tuple[int, int, int]]:
        """Rank r's spans in slab order as (sequence, start in the sequence, length)."""
        if not 0 <= r < self.world_size:
            raise ValueError(f"rank must be in [0, {self.world_size})")
        out = []
        for s in np.nonzero(self.span_rank_host == r)[0]:
            a, e = int(self.span_start_host[s]), int(self.span_start_host[s + 1])
            i = int(np.searchsorted(self.cu_host, a, side="right")) - 1
            out.append((i, a - int(self.cu_host[i]), e - a))
        return out

    def to(self, device) -> "ThdPlan":
        dev = torch.device(device)
        self.span_start = torch.from_numpy(self.span_start_host).to(dev)
        self.span_rank = torch.from_numpy(self.span_rank_host).to(dev)
        self.span_local = torch.from_numpy(self.span_local_host).to(dev)
        self.rank_off = torch.from_numpy(self.rank_off_host).to(dev)
        self.cu = torch.from_numpy(np.ascontiguousarray(self.cu_host, dtype=np.int32)).to(dev)
        self.first_pos = torch.from_numpy(self.first_pos_host).to(dev)
        return self


def thd_plan(cu_seqlens, world_size: int, config: ThdPlannerConfig | None = None, device=None) -> ThdPlan:
    """Plan a packed THD batch over world_size ranks on the host (libcam);
    with device given, the tables are also uploaded there."""
    if isinstance(world_size, bool) or not isinstance(world_size, (int, np.integer)):
        raise TypeError("world_size must be an integer")
    cfg = (config or ThdPlannerConfig())._c()
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    nseq = cu.size - 1
    if nseq < 0:
        raise ValueError("cu_seqlens must have at least one entry")
    W = int(world_size)
    n = C.c_int64(0)
    grid = C.c_int32(0)
    lib = library()
    cap = 4 * (nseq + max(W, 1)) + 16
    for _ in range(2):
        ss = np.empty(cap + 1, dtype=np.int32)
        sr = np.empty(cap, dtype=np.int32)
        sl = np.empty(cap, dtype=np.int32)
        ro = np.empty(max(W, 0) + 1, dtype=np.int64)
        rc = np.empty(max(W, 1), dtype=np.float64)
        st = lib.thd_plan(cu.ctypes.data, nseq, W, C.addressof(cfg), cap, ss.ctypes.data, sr.ctypes.data,
                          sl.ctypes.data, ro.ctypes.data, rc.ctypes.data, C.addressof(n), C.addressof(grid))
        if st != 0 and n.value > cap:
            cap = n.value
            continue
        _check(st)
        break
    k = n.value
    plan = ThdPlan(W, int(cu[-1]), cu, ss[:k + 1].copy(), sr[:k].copy(), sl[:k].copy(), ro.copy(), rc[:W].copy(),
                   int(grid.value))
    return plan.to(device) if device is not None else plan


def _spans_common(x: torch.Tensor, plan: ThdPlan):
    _contig(x, "x")
    if plan.span_start is None:
        raise ValueError("the plan's tables are not on the device (thd_plan(..., device=...) or plan.to(device))")
    return plan.total_tokens, plan.world_size


def ulysses_seq_to_head_spans(x: torch.Tensor, plan: ThdPlan, B: int = 1,
                              out: torch.Tensor | None = None) -> torch.Tensor:
    """Planned rank-major slabs [B*T][H][D] -> [P][B][T][H/P][D]."""
    T, P = _spans_common(x, plan)
    if x.dim() != 3 or x.shape[0] != B * T:
        raise ValueError("x must be [B*T][H][D]")
    H, D = x.shape[1], x.shape[2]
    if out is None:
        out = torch.empty((P, B, T, H // P, D), dtype=x.dtype, device=x.device)
    _contig(out, "out")
    if out.numel() != x.numel() or out.dtype != x.dtype:
        raise ValueError("out must match x in size and dtype")
    _tables_on(x, plan.span_start, plan.span_rank, plan.span_local, plan.rank_off)
    _check(library().ulysses_seq_to_head_spans(
        x.data_ptr(), out.data_ptr(), plan.span_start.data_ptr(), plan.span_rank.data_ptr(),
        plan.span_local.data_ptr(), plan.rank_off.data_ptr(), plan.n_spans, T, P, B, H, D, _dt(x, True),
        _stream(x)))
    return out


def ulysses_head_to_seq_spans(x: torch.Tensor, plan: ThdPlan, out: torch.Tensor | None = None) -> torch.Tensor:
    """[P][B][T][H/P][D] -> planned rank-major slabs [B*T][H][D]."""
    T, P = _spans_common(x, plan)
    if x.dim() != 5 or x.shape[0] != P or x.shape[2] != T:
        raise ValueError("x must be [P][B][T][H/P][D]")
    B, D = x.shape[1], x.shape[4]
    H = x.shape[3] * P
    if out is None:
        out = torch.empty((B * T, H, D), dtype=x.dtype, device=x.device)
    _contig(out, "out")
    if out.numel() != x.numel() or out.dtype != x.dtype:
        raise ValueError("out must match x in size and dtype")
    _tables_on(x, plan.span_start, plan.span_rank, plan.span_local, plan.rank_off)
    _check(library().ulysses_head_to_seq_spans(
        x.data_ptr(), out.data_ptr(), plan.span_start.data_ptr(), plan.span_rank.data_ptr(),
        plan.span_local.data_ptr(), plan.rank_off.data_ptr(), plan.n_spans, T, P, B, H, D, _dt(x, True),
        _stream(x)))
    return out


# ---------------------------------------------------------------------------
# LSE pack and combine
# ---------------------------------------------------------------------------

def lse_pack_bytes(P: int, T: int, H: int, Dv: int, scatter_dim: int, dtype=torch.bfloat16) -> int:
    code = CAM_BF16 if dtype == torch.bfloat16 else CAM_FP16
    n = library().lse_pack_bytes(P, T, H, Dv, scatter_dim, code)
    if n < 0:
        raise CamError(2, library().cam_last_error().decode())
    return n


def lse_pack(out: torch.Tensor, smax: torch.Tensor, ssum: torch.Tensor, scatter_dim: int,
             packed: torch.Tensor | None = None) -> torch.Tensor:
    """Pack per-rank partial outputs [P][T][H][Dv] (any strides, Dv contiguous)
    and fp32 softmax max/sum [P][T][H] (any strides) into the packed exchange
    buffer (uint8, [P_src][P_dst][chunk]), forming the LSE on the way."""
    for t, n in ((out, "out"), (smax, "smax"), (ssum, "ssum")):
        _dev(t, n)
    if out.dim() != 4 or out.stride(3) != 1:
        raise ValueError("out must be [P][T][H][Dv] with Dv contiguous")
    if smax.dtype != torch.float32 or ssum.dtype != torch.float32:
        raise TypeError("softmax statistics must be float32")
    P, T, H, Dv = out.shape
    if tuple(smax.shape) != (P, T, H) or tuple(ssum.shape) != (P, T, H):
        raise ValueError("statistics must be [P][T][H]")
    n = lse_pack_bytes(P, T, H, Dv, scatter_dim, out.dtype)
    if packed is None:
        packed = torch.empty(n, dtype=torch.uint8, device=out.device)
    _contig(packed, "packed")
    if packed.numel() < n:
        raise ValueError(f"packed needs {n} bytes")
    _check(library().lse_pack(out.data_ptr(), *out.stride()[:3], smax.data_ptr(), *smax.stride(),
                              ssum.data_ptr(), *ssum.stride(), P, T, H, Dv, scatter_dim, _dt(out),
                              packed.data_ptr(), _stream(out)))
    return packed


def lse_combine_packed(packed: torch.Tensor, P: int, T: int, H: int, Dv: int, scatter_dim: int,
                       dtype=torch.bfloat16, out: torch.Tensor | None = None,
                       lse_out: torch.Tensor | None | bool = True):
    """Combine, for every destination rank r, the chunks (p, r) of all sources
    (the exchange is a strided view of the packed buffer).  Returns
    (out [P*rows][Dv], lse_out [P*rows] or None)."""
    _check_packed(packed, P, T, H, Dv, scatter_dim, dtype)
    rows = T * (H // P) if scatter_dim == 1 else (T // P) * H
    if out is not None:
        _check_buffer(out, "out", (P * rows, Dv), dtype)
    if lse_out is not None and not isinstance(lse_out, bool):
        _check_buffer(lse_out, "lse_out", (P * rows,), torch.float32)
    _contig(packed, "packed")
    if out is None:
        out = torch.empty((P * rows, Dv), dtype=dtype, device=packed.device)
    _contig(out, "out")
    if lse_out is True:
        lse_out = torch.empty(P * rows, dtype=torch.float32, device=packed.device)
    elif lse_out is False:
        lse_out = None
    if lse_out is not None:
        _contig(lse_out, "lse_out")
    code = CAM_BF16 if dtype == torch.bfloat16 else CAM_FP16
    _check(library().lse_combine_packed(packed.data_ptr(), P, T, H, Dv, scatter_dim, code, out.data_ptr(),
                                        _ptr(lse_out), _stream(packed)))
    return out, lse_out


def _combine_common(part_out, part_lse, out, lse_out, out_name="out"):
    if part_out.dim() != 4 or part_out.stride(3) != 1:
        raise ValueError("part_out must be [P][T][H][D] with D contiguous")
    _dt(part_out)
    if part_lse.dtype != torch.float32:
        raise TypeError("part_lse must be float32")
    P, T, H, D = part_out.shape
    if tuple(part_lse.shape) != (P, T, H):
        raise ValueError("part_lse must be [P][T][H]")
    if out is not None:
        _check_buffer(out, out_name, (T, H, D), part_out.dtype, contiguous=False, inner_contiguous=True)
    if lse_out is not None and not isinstance(lse_out, bool):
        _check_buffer(lse_out, "lse_out", (T, H), torch.float32, contiguous=False)
    _dev(part_out, "part_out")
    _dev(part_lse, "part_lse")
    if out is None:
        out = torch.empty((T, H, D), dtype=part_out.dtype, device=part_out.device)
    _dev(out, out_name)
    if out.dim() != 3 or out.stride(2) != 1:
        raise ValueError(f"{out_name} must be [T][H][D] with D contiguous")
    if lse_out is True:
        lse_out = torch.empty((T, H), dtype=torch.float32, device=part_out.device)
    elif lse_out is False:
        lse_out = None
    if lse_out is not None:
        _dev(lse_out, "lse_out")
    lo = lse_out.stride() if lse_out is not None else (0, 0)
    return P, T, H, D, out, lse_out, lo


def lse_combine(part_out: torch.Tensor, part_lse: torch.Tensor, out: torch.Tensor | None = None,
                lse_out: torch.Tensor | None | bool = True):
    """Stable combine of P partials: part_out [P][T][H][D], part_lse [P][T][H]
    (any strides, D contiguous) -> (out [T][H][D], lse_out [T][H] or None)."""
    P, T, H, D, out, lse_out, lo = _combine_common(part_out, part_lse, out, lse_out)
    _check(library().lse_combine(part_out.data_ptr(), *part_out.stride()[:3], part_lse.data_ptr(),
                                 *part_lse.stride(), P, T, H, D, _dt(part_out), out.data_ptr(),
                                 *out.stride()[:2], _ptr(lse_out), *lo, _stream(part_out)))
    return out, lse_out


def lse_combine_varlen(part_out: torch.Tensor, part_lse: torch.Tensor, cu_seqlens: torch.Tensor,
                       out: torch.Tensor | None = None, lse_out: torch.Tensor | None | bool = True):
    """lse_combine for a packed THD batch whose P partials are the causal
    attention over the P KV pieces of each token's own sequence; cu_seqlens is
    a device int32 tensor [nseq+1]."""
    P, T, H, D, out, lse_out, lo = _combine_common(part_out, part_lse, out, lse_out)
    _contig(cu_seqlens, "cu_seqlens")
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    _check(library().lse_combine_varlen(part_out.data_ptr(), *part_out.stride()[:3], part_lse.data_ptr(),
                                        *part_lse.stride(), P, T, H, D, _dt(part_out), out.data_ptr(),
                                        *out.stride()[:2], _ptr(lse_out), *lo, cu_seqlens.data_ptr(),
                                        cu_seqlens.numel() - 1, _stream(part_out)))
    return out, lse_out


def lse_combine_planned(part_out: torch.Tensor, part_lse: torch.Tensor, plan: ThdPlan,
                        out: torch.Tensor | None = None, lse_out: torch.Tensor | None | bool = True):
    """Causal combine of a batch laid out by a THD layout plan: partial p of
    a token is admitted iff rank p holds a position of the token's sequence at
    or before it (the plan's device tables are used)."""
    P, T, H, D, out, lse_out, lo = _combine_common(part_out, part_lse, out, lse_out)
    if plan.first_pos is None:
        raise ValueError("the plan's tables are not on the device (thd_plan(..., device=...) or plan.to(device))")
    if P != plan.world_size or T != plan.total_tokens:
        raise ValueError("part_out must be [world_size][total_tokens][H][D] for this plan")
    _tables_on(part_out, plan.cu, plan.first_pos)
    _check(library().lse_combine_planned(part_out.data_ptr(), *part_out.stride()[:3], part_lse.data_ptr(),
                                         *part_lse.stride(), P, T, H, D, _dt(part_out), out.data_ptr(),
                                         *out.stride()[:2], _ptr(lse_out), *lo, plan.cu.data_ptr(),
                                         plan.first_pos.data_ptr(), plan.cu_host.size - 1, _stream(part_out)))
    return out, lse_out


def lse_combine_backward(part_out: torch.Tensor, part_lse: torch.Tensor, g_out: torch.Tensor,
                         g_lse: torch.Tensor | None = None, cu_seqlens: torch.Tensor | None = None,
                         d_part_out: torch.Tensor | None = None, d_part_lse: torch.Tensor | None = None,
                         plan: ThdPlan | None = None):
    """Gradient of lse_combine (with cu_seqlens, of lse_combine_varlen; with
    plan, of lse_combine_planned):
    part_out [P][T][H][D], part_lse [P][T][H], g_out [T][H][D] (the upstream
    gradient of out, payload dtype), g_lse [T][H] fp32 or None (zero) ->
    (d_part_out [P][T][H][D], d_part_lse [P][T][H] fp32).  Any strides with D
    contiguous."""
    P, T, H, D, _, _, _ = _combine_common(part_out, part_lse, g_out, None, out_name="g_out")
    if g_lse is not None:
        _dev(g_lse, "g_lse")
        if g_lse.dtype != torch.float32 or tuple(g_lse.shape) != (T, H):
            raise ValueError("g_lse must be float32 [T][H]")
    if d_part_out is None:
        d_part_out = torch.empty_like(part_out, memory_format=torch.contiguous_format)
    if d_part_lse is None:
        d_part_lse = torch.empty((P, T, H), dtype=torch.float32, device=part_out.device)
    _dev(d_part_out, "d_part_out")
    _dev(d_part_lse, "d_part_lse")
    if tuple(d_part_out.shape) != (P, T, H, D) or d_part_out.stride(3) != 1 or d_part_out.dtype != part_out.dtype:
        raise ValueError("d_part_out must be [P][T][H][D] of the payload dtype with D contiguous")
    if tuple(d_part_lse.shape) != (P, T, H) or d_part_lse.dtype != torch.float32:
        raise ValueError("d_part_lse must be float32 [P][T][H]")
    gl = g_lse.stride() if g_lse is not None else (0, 0)
    args = [part_out.data_ptr(), *part_out.stride()[:3], part_lse.data_ptr(), *part_lse.stride(), P, T, H, D,
            _dt(part_out), g_out.data_ptr(), *g_out.stride()[:2], _ptr(g_lse), *gl, d_part_out.data_ptr(),
            *d_part_out.stride()[:3], d_part_lse.data_ptr(), *d_part_lse.stride()]
    if plan is not None:
        if plan.first_pos is None:
            raise ValueError("the plan's tables are not on the device")
        if P != plan.world_size or T != plan.total_tokens:
            raise ValueError("part_out must be [world_size][total_tokens][H][D] for this plan")
        _tables_on(part_out, plan.cu, plan.first_pos)
        _check(library().lse_combine_planned_backward(*args, plan.cu.data_ptr(), plan.first_pos.data_ptr(),
                                                      plan.cu_host.size - 1, _stream(part_out)))
    elif cu_seqlens is None:
        _check(library().lse_combine_backward(*args, _stream(part_out)))
    else:
        _contig(cu_seqlens, "cu_seqlens")
        if cu_seqlens.dtype != torch.int32:
            raise TypeError("cu_seqlens must be int32")
        _check(library().lse_combine_varlen_backward(*args, cu_seqlens.data_ptr(), cu_seqlens.numel() - 1,
                                                     _stream(part_out)))
    return d_part_out, d_part_lse


# A stack of partials at least this large per partial is laid out with a gap
# of this many bytes between consecutive partials.
PARTIAL_GAP_BYTES = 1 << 20
PARTIAL_GAP_MIN_BYTES = 64 << 20


def empty_partials(P: int, T: int, H: int, D: int, dtype=torch.bfloat16, device="cuda") -> torch.Tensor:
    """An uninitialised [P][T][H][D] stack of partials, or of their gradients,
    each partial contiguous.  When one partial holds at least 64 MiB, the
    next one starts 1 MiB after its end, so that the P streams a kernel
    reads or writes side by side are not a multiple of a large power of two
    apart.  Measured on MI355X: the combine's gradient writing eight 1 GiB
    partials runs 3-8% faster into this layout than into a contiguous stack
    (the forward combine's reads gain nothing from it).  The gap size was
    chosen by measurement: the response is not monotonic (a 4 MiB gap is
    slower than none).  Every entry point takes the view like any other
    strided stack."""
    es = torch.empty((), dtype=dtype).element_size()
    n = T * H * D
    gap = PARTIAL_GAP_BYTES // es if n * es >= PARTIAL_GAP_MIN_BYTES else 0
    buf = torch.empty(P * (n + gap), dtype=dtype, device=device)
    return buf.as_strided((P, T, H, D), (n + gap, H * D, D, 1))


def lse_combine_packed_seq(packed: torch.Tensor, P: int, T: int, H: int, Dv: int, scatter_dim: int,
                           dtype=torch.bfloat16, out: torch.Tensor | None = None,
                           lse_out: torch.Tensor | None | bool = True):
    """lse_combine_packed with token-major output: (out [T][H][Dv], lse_out [T][H])."""
    _check_packed(packed, P, T, H, Dv, scatter_dim, dtype)
    if out is not None:
        _check_buffer(out, "out", (T, H, Dv), dtype)
    if lse_out is not None and not isinstance(lse_out, bool):
        _check_buffer(lse_out, "lse_out", (T, H), torch.float32)
    _contig(packed, "packed")
    if out is None:
        out = torch.empty((T, H, Dv), dtype=dtype, device=packed.device)
    _contig(out, "out")
    if lse_out is True:
        lse_out = torch.empty((T, H), dtype=torch.float32, device=packed.device)
    elif lse_out is False:
        lse_out = None
    if lse_out is not None:
        _contig(lse_out, "lse_out")
    code = CAM_BF16 if dtype == torch.bfloat16 else CAM_FP16
    _check(library().lse_combine_packed_seq(packed.data_ptr(), P, T, H, Dv, scatter_dim, code, out.data_ptr(),
                                            _ptr(lse_out), _stream(packed)))
    return out, lse_out


def lse_combine_varlen_seq(part_out: torch.Tensor, part_lse: torch.Tensor, plan: "VarlenPlan",
                           out: torch.Tensor | None = None, lse_out: torch.Tensor | None | bool = True):
    """lse_combine_varlen whose token rows go to the rank-major (sequence-
    sharded) order of the varlen relayout: (out [T][H][D], lse_out [T][H])."""
    if part_out.dim() != 4 or part_out.stride(3) != 1 or part_lse.dtype != torch.float32:
        raise ValueError("part_out must be [P][T][H][D] (D contiguous), part_lse float32 [P][T][H]")
    _dt(part_out)
    P, T, H, D = part_out.shape
    if tuple(part_lse.shape) != (P, T, H):
        raise ValueError("part_lse must be [P][T][H]")
    if P != plan.P or T != plan.total_tokens:
        raise ValueError("the plan must match the partials' P and T")
    if out is not None:
        _check_buffer(out, "out", (T, H, D), part_out.dtype)
    if lse_out is not None and not isinstance(lse_out, bool):
        _check_buffer(lse_out, "lse_out", (T, H), torch.float32)
    _dev(part_out, "part_out")
    _dev(part_lse, "part_lse")
    if out is None:
        out = torch.empty((T, H, D), dtype=part_out.dtype, device=part_out.device)
    _contig(out, "out")
    if lse_out is True:
        lse_out = torch.empty((T, H), dtype=torch.float32, device=part_out.device)
    elif lse_out is False:
        lse_out = None
    if lse_out is not None:
        _contig(lse_out, "lse_out")
    _tables_on(part_out, plan.cu, plan.rank_cu, plan.rank_off)
    _check(library().lse_combine_varlen_seq(part_out.data_ptr(), *part_out.stride()[:3], part_lse.data_ptr(),
                                            *part_lse.stride(), P, T, H, D, _dt(part_out), out.data_ptr(),
                                            _ptr(lse_out), plan.cu.data_ptr(), plan.rank_cu.data_ptr(),
                                            plan.rank_off.data_ptr(), plan.nseq, _stream(part_out)))
    return out, lse_out


def lse_merge(acc_out: torch.Tensor, acc_lse: torch.Tensor, part_out: torch.Tensor, part_lse: torch.Tensor,
              out_final: torch.Tensor | None = None):
    """In place: (acc_out fp32 [T][H][D], acc_lse fp32 [T][H]) <- stable combine of
    the accumulator and one partial (part_out [T][H][D] bf16/fp16, part_lse
    [T][H]); optionally also writes the rounded result to out_final."""
    if acc_out.dtype != torch.float32 or acc_lse.dtype != torch.float32 or part_lse.dtype != torch.float32:
        raise TypeError("accumulator and LSEs must be float32")
    if acc_out.dim() != 3 or part_out.dim() != 3 or acc_out.stride(2) != 1 or part_out.stride(2) != 1:
        raise ValueError("payloads must be [T][H][D] with D contiguous")
    T, H, D = part_out.shape
    if tuple(acc_out.shape) != (T, H, D) or tuple(acc_lse.shape) != (T, H) or tuple(part_lse.shape) != (T, H):
        raise ValueError("shape mismatch")
    fs = (0, 0)
    if out_final is not None:
        _check_buffer(out_final, "out_final", (T, H, D), part_out.dtype, contiguous=False, inner_contiguous=True)
        fs = out_final.stride()[:2]
    for t_, n in ((acc_out, "acc_out"), (acc_lse, "acc_lse"), (part_out, "part_out"), (part_lse, "part_lse")):
        _dev(t_, n)
    if out_final is not None:
        _dev(out_final, "out_final")
    _check(library().lse_merge(acc_out.data_ptr(), *acc_out.stride()[:2], acc_lse.data_ptr(), *acc_lse.stride(),
                               part_out.data_ptr(), *part_out.stride()[:2], part_lse.data_ptr(), *part_lse.stride(),
                               T, H, D, _dt(part_out), _ptr(out_final), *fs, _stream(part_out)))
    return acc_out, acc_lse


def qkv_projection_head_sharded(x: torch.Tensor, w: torch.Tensor, P: int, B: int, H: int, D: int,
                                out: torch.Tensor | None = None) -> torch.Tensor:
    """x [S][K] (stacked sequence shards) times w [B*H*D][K] (linear-layer
    layout), written as the head-sharded [P][B][S][H/P][D] (MFMA)."""
    _contig(x, "x")
    _contig(w, "w")
    if x.dim() != 2 or w.dim() != 2 or w.shape[1] != x.shape[1] or w.shape[0] != B * H * D:
        raise ValueError("x must be [S][K] and w [B*H*D][K]")
    if x.dtype != w.dtype or x.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("x and w must share a bf16 or fp16 dtype")
    S, K = x.shape
    if out is None:
        out = torch.empty((P, B, S, H // P, D), dtype=x.dtype, device=x.device)
    _contig(out, "out")
    if out.numel() != S * B * H * D or out.dtype != x.dtype:
        raise ValueError("out must be [P][B][S][H/P][D] of the operands' dtype")
    _check(library().qkv_projection_head_sharded(x.data_ptr(), w.data_ptr(), out.data_ptr(), S, K, P, B, H, D,
                                                 _dt(x), _stream(x)))
    return out


def ablation_seq_to_head_lds(x: torch.Tensor, P: int, rows_per_tile: int = 4,
                             out: torch.Tensor | None = None) -> torch.Tensor:
    """ulysses_seq_to_head by the LDS-staged kernel (kept to measure that
    choice against the direct kernel; the API does not use it)."""
    _contig(x, "x")
    if x.dim() != 5 or x.shape[0] != P:
        raise ValueError("x must be [P][B][S/P][H][D]")
    _, B, Sp, H, D = x.shape
    if H % P:
        raise ValueError("H must be a multiple of P")
    if out is None:
        out = torch.empty((P, B, Sp * P, H // P, D), dtype=x.dtype, device=x.device)
    _contig(out, "out")
    if out.numel() != x.numel() or out.dtype != x.dtype:
        raise ValueError("out must match x in size and dtype")
    _check(library().cam_ablation_seq_to_head_lds(x.data_ptr(), out.data_ptr(), P, B, Sp * P, H, D, _dt(x, True),
                                                  rows_per_tile, _stream(x)))
    return out


def copy(src: torch.Tensor, dst: torch.Tensor) -> torch.Tensor:
    """Plain 16-byte-vector device copy (the copy ceiling of the relayouts)."""
    _contig(src, "src")
    _contig(dst, "dst")
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n:
        raise ValueError("src and dst sizes differ")
    _check(library().cam_copy(src.data_ptr(), dst.data_ptr(), n, _stream(src)))
    return dst


def last_launch() -> dict:
    """Geometry of this thread's latest kernel launch: workgroups, threads per
    workgroup, dynamic LDS bytes (profilers match calls to dispatches by it)."""
    wg, th, lds = C.c_uint64(0), C.c_uint32(0), C.c_uint64(0)
    _check(library().cam_last_launch(C.addressof(wg), C.addressof(th), C.addressof(lds)))
    return {"workgroups": wg.value, "threads": th.value, "lds_bytes": lds.value}
