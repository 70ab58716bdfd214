"""CPU oracle for the per-GPU hot path of sequence/context-parallel attention
movement: Ulysses relayouts (dense and cu_seqlens varlen), the max/sum-aware
LSE pack and the stable LSE-weighted combine, plus brute-force attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this package.  It shares no code with
the HIP path: the arithmetic lives in ``cam_oracle.c`` (plain C, fp64, rounded
once), and this module only marshals numpy arrays into it.

Every function cites the page passage it follows in ``cam_oracle.c``.
"""

from __future__ import annotations

import ctypes as C
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "cam_oracle.c"
_LIB_PATH = _HERE / "liboracle.so"
_lib = None

i64 = C.c_int64
vp = C.c_void_p


def build(verbose: bool = False) -> Path:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", str(_LIB_PATH) + ".tmp", str(_SRC), "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(str(_LIB_PATH) + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not _LIB_PATH.exists() or _LIB_PATH.stat().st_mtime < _SRC.stat().st_mtime:
        build()
    lib = C.CDLL(str(_LIB_PATH))
    sig = {
        "orc_double_to_bf16": (C.c_uint16, [C.c_double]),
        "orc_bf16_to_double": (C.c_double, [C.c_uint16]),
        "orc_double_to_fp16": (C.c_uint16, [C.c_double]),
        "orc_fp16_to_double": (C.c_double, [C.c_uint16]),
        "orc_round_bf16_array": (None, [vp, vp, i64]),
        "orc_round_fp16_array": (None, [vp, vp, i64]),
        "orc_bf16_to_double_array": (None, [vp, vp, i64]),
        "orc_fp16_to_double_array": (None, [vp, vp, i64]),
        "orc_seq_to_head": (None, [vp, vp, i64, i64, i64, i64, i64, i64]),
        "orc_head_to_seq": (None, [vp, vp, i64, i64, i64, i64, i64, i64]),
        "orc_varlen_plan": (None, [vp, i64, i64, vp, vp]),
        "orc_varlen_seq_to_head": (None, [vp, vp, vp, i64, i64, i64, i64, i64, i64]),
        "orc_varlen_head_to_seq": (None, [vp, vp, vp, i64, i64, i64, i64, i64, i64]),
        "orc_lse_from_stats": (C.c_double, [C.c_float, C.c_float]),
        "orc_pack_rows": (i64, [i64, i64, i64, C.c_int]),
        "orc_pack_chunk_bytes": (i64, [i64, i64, i64, i64, C.c_int, i64]),
        "orc_lse_pack": (None, [vp, i64, i64, i64, vp, i64, i64, i64, vp, i64, i64, i64,
                                i64, i64, i64, i64, C.c_int, i64, vp]),
        "orc_combine_row_f64": (None, [vp, vp, vp, i64, i64, vp, vp]),
        "orc_combine_f64": (None, [vp, vp, i64, i64, i64, vp, vp]),
        "orc_causal_piece_valid": (C.c_int, [vp, i64, i64, i64, i64]),
        "orc_lse_combine": (None, [vp, i64, i64, i64, vp, i64, i64, i64, i64, i64, i64, i64, i64,
                                   C.c_int, vp, i64, i64, vp, i64, i64, vp, i64]),
        "orc_lse_combine_packed": (None, [vp, i64, i64, i64, i64, C.c_int, C.c_int, vp, vp]),
        "orc_attention": (None, [vp, vp, vp, i64, i64, i64, C.c_int, i64, i64, C.c_int,
                                 vp, vp, vp]),
        "orc_varlen_token_rows": (None, [vp, i64, i64, vp]),
        "orc_lse_combine_packed_seq": (None, [vp, i64, i64, i64, i64, C.c_int, C.c_int, vp, vp]),
        "orc_thd_plan": (C.c_int, [vp, i64, i64, i64, i64, i64, C.c_double, C.c_double, i64, vp, vp, vp, vp,
                                   vp, vp, vp]),
        "orc_thd_plan_candidate_trace": (C.c_int, [vp, i64, i64, i64, i64, C.c_double, C.c_double, C.c_int,
                                                   vp, i64, vp, vp, i64, vp]),
        "orc_span_seq_to_head": (None, [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64]),
        "orc_span_head_to_seq": (None, [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64]),
        "orc_plan_first_positions": (None, [vp, i64, i64, vp, vp, i64, vp]),
        "orc_plan_piece_valid": (C.c_int, [vp, i64, vp, i64, i64]),
        "orc_lse_combine_planned": (None, [vp, i64, i64, i64, vp, i64, i64, i64, i64, i64, i64, i64, i64,
                                           C.c_int, vp, i64, i64, vp, i64, i64, vp, vp, i64]),
        "orc_lse_combine_planned_backward": (None, [vp, i64, i64, i64, vp, i64, i64, i64, i64, i64, i64, i64,
                                                    i64, C.c_int, vp, i64, i64, vp, i64, i64, vp, i64, i64, i64,
                                                    vp, i64, i64, i64, vp, vp, i64]),
        "orc_qkv_projection": (None, [vp, vp, vp, i64, i64, i64, i64, i64, i64, C.c_int]),
        "orc_combine_row_backward_f64": (None, [vp, vp, vp, i64, i64, vp, C.c_double, vp, vp]),
        "orc_lse_combine_backward": (None, [vp, i64, i64, i64, vp, i64, i64, i64, i64, i64, i64, i64, i64,
                                            C.c_int, vp, i64, i64, vp, i64, i64, vp, i64, i64, i64,
                                            vp, i64, i64, i64, vp, i64]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _dt(dtype: str) -> int:
    return {"bf16": 0, "fp16": 1}[dtype]


# -- number formats ---------------------------------------------------------

def double_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty(x.shape, dtype=np.uint16)
    _load().orc_round_bf16_array(_p(x), _p(y), x.size)
    return y


def double_to_fp16_bits(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty(x.shape, dtype=np.uint16)
    _load().orc_round_fp16_array(_p(x), _p(y), x.size)
    return y


def half_bits_to_double(bits: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    y = np.empty(bits.shape, dtype=np.float64)
    fn = _load().orc_bf16_to_double_array if dtype == "bf16" else _load().orc_fp16_to_double_array
    fn(_p(bits), _p(y), bits.size)
    return y


def round_half(x: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    return double_to_bf16_bits(x) if dtype == "bf16" else double_to_fp16_bits(x)


# -- relayouts --------------------------------------------------------------

def seq_to_head(x: np.ndarray, P: int, B: int, S: int, H: int, D: int) -> np.ndarray:
    """[P][B][S/P][H][D] -> [P][B][S][H/P][D] (bits of any element size)."""
    x = np.ascontiguousarray(x)
    assert x.size == B * S * H * D
    out = np.empty(P * B * S * (H // P) * D, dtype=x.dtype)
    _load().orc_seq_to_head(_p(x), _p(out), P, B, S, H, D, x.dtype.itemsize)
    return out.reshape(P, B, S, H // P, D)


def head_to_seq(x: np.ndarray, P: int, B: int, S: int, H: int, D: int) -> np.ndarray:
    """[P][B][S][H/P][D] -> [P][B][S/P][H][D]."""
    x = np.ascontiguousarray(x)
    assert x.size == B * S * H * D
    out = np.empty(P * B * (S // P) * H * D, dtype=x.dtype)
    _load().orc_head_to_seq(_p(x), _p(out), P, B, S, H, D, x.dtype.itemsize)
    return out.reshape(P, B, S // P, H, D)


def varlen_plan(cu: np.ndarray, P: int):
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    nseq = cu.size - 1
    rank_cu = np.empty((P, nseq + 1), dtype=np.int32)
    rank_off = np.empty(P + 1, dtype=np.int64)
    _load().orc_varlen_plan(_p(cu), nseq, P, _p(rank_cu), _p(rank_off))
    return rank_cu, rank_off


def varlen_seq_to_head(x: np.ndarray, cu: np.ndarray, P: int, B: int, H: int, D: int) -> np.ndarray:
    """Rank-major ragged [B*T][H][D] (rank p's [B][T_p] slab at token B*R_p)
    -> [P][B][T][H/P][D]."""
    x = np.ascontiguousarray(x)
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    T = int(cu[-1])
    assert x.size == B * T * H * D
    out = np.empty(P * B * T * (H // P) * D, dtype=x.dtype)
    _load().orc_varlen_seq_to_head(_p(x), _p(out), _p(cu), cu.size - 1, P, B, H, D, x.dtype.itemsize)
    return out.reshape(P, B, T, H // P, D)


def varlen_head_to_seq(x: np.ndarray, cu: np.ndarray, P: int, B: int, H: int, D: int) -> np.ndarray:
    x = np.ascontiguousarray(x)
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    T = int(cu[-1])
    assert x.size == B * T * H * D
    out = np.empty(B * T * H * D, dtype=x.dtype)
    _load().orc_varlen_head_to_seq(_p(x), _p(out), _p(cu), cu.size - 1, P, B, H, D, x.dtype.itemsize)
    return out.reshape(B * T, H, D)


# -- LSE pack ---------------------------------------------------------------

def lse_from_stats(m: float, s: float) -> float:
    return _load().orc_lse_from_stats(float(m), float(s))


def pack_rows(P, T, H, scatter_dim) -> int:
    return int(_load().orc_pack_rows(P, T, H, scatter_dim))


def pack_chunk_bytes(P, T, H, Dv, scatter_dim, esize=2) -> int:
    return int(_load().orc_pack_chunk_bytes(P, T, H, Dv, scatter_dim, esize))


def _strides_el(a: np.ndarray):
    return tuple(s // a.itemsize for s in a.strides)


def lse_pack(out_bits: np.ndarray, smax: np.ndarray, ssum: np.ndarray, scatter_dim: int,
             base_out=None, base_m=None, base_s=None) -> np.ndarray:
    """out_bits: uint16 [P][T][H][Dv] (any strides with Dv contiguous, given
    as a view into a contiguous base array); smax/ssum float32 [P][T][H] views.
    Returns the packed byte buffer [P][P][chunk]."""
    P, T, H, Dv = out_bits.shape
    assert out_bits.strides[3] == out_bits.itemsize

    def ptr(view):
        return view.__array_interface__["data"][0]

    o_sp, o_st, o_sh, _ = _strides_el(out_bits)
    m_sp, m_st, m_sh = _strides_el(smax)
    s_sp, s_st, s_sh = _strides_el(ssum)
    chunk = pack_chunk_bytes(P, T, H, Dv, scatter_dim, out_bits.itemsize)
    packed = np.zeros(P * P * chunk, dtype=np.uint8)
    _load().orc_lse_pack(ptr(out_bits), o_sp, o_st, o_sh, ptr(smax), m_sp, m_st, m_sh,
                         ptr(ssum), s_sp, s_st, s_sh, P, T, H, Dv, scatter_dim,
                         out_bits.itemsize, _p(packed))
    return packed


def packed_regions(packed: np.ndarray, P, T, H, Dv, scatter_dim, esize=2):
    """Split a packed byte buffer into its O-regions [P][P][rows][Dv] (uint16
    bits) and L-regions [P][P][rows] (float32); padding excluded."""
    rows = pack_rows(P, T, H, scatter_dim)
    chunk = pack_chunk_bytes(P, T, H, Dv, scatter_dim, esize)
    o_bytes = (rows * Dv * esize + 15) // 16 * 16
    c = packed.reshape(P, P, chunk)
    O = np.ascontiguousarray(c[:, :, : rows * Dv * esize]).view(np.uint16).reshape(P, P, rows, Dv)
    L = np.ascontiguousarray(c[:, :, o_bytes: o_bytes + 4 * rows]).view(np.float32).reshape(P, P, rows)
    return O, L


# -- combine ----------------------------------------------------------------

def combine_f64(part_o: np.ndarray, part_l: np.ndarray):
    """part_o [P][R][D] float64, part_l [P][R] float64 -> (out [R][D], lse [R])."""
    part_o = np.ascontiguousarray(part_o, dtype=np.float64)
    part_l = np.ascontiguousarray(part_l, dtype=np.float64)
    P, R, D = part_o.shape
    out = np.empty((R, D))
    lse = np.empty(R)
    _load().orc_combine_f64(_p(part_o), _p(part_l), P, R, D, _p(out), _p(lse))
    return out, lse


def causal_piece_valid(cu: np.ndarray, P: int, p: int, t: int) -> bool:
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    return bool(_load().orc_causal_piece_valid(_p(cu), cu.size - 1, P, p, t))


def causal_mask(cu: np.ndarray, P: int) -> np.ndarray:
    """[P][T] bool: partial p valid for token t under the causal piece rule."""
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    T = int(cu[-1])
    lib = _load()
    m = np.zeros((P, T), dtype=bool)
    for p in range(P):
        for t in range(T):
            m[p, t] = bool(lib.orc_causal_piece_valid(_p(cu), cu.size - 1, P, p, t))
    return m


def lse_combine(part_out: np.ndarray, part_lse: np.ndarray, dtype: str = "bf16",
                cu: np.ndarray | None = None, t_begin: int = 0, with_lse: bool = True):
    """part_out uint16 view [P][T'][H][D] (D contiguous), part_lse float32 view
    [P][T'][H] -- T' rows starting at global token t_begin.  Returns
    (out uint16 [T'][H][D], lse float32 [T'][H])."""
    P, Tw, H, D = part_out.shape
    assert part_out.strides[3] == part_out.itemsize

    def ptr(view):
        return view.__array_interface__["data"][0]

    po = _strides_el(part_out)
    pl = _strides_el(part_lse)
    out = np.empty((Tw, H, D), dtype=np.uint16)
    lse = np.empty((Tw, H), dtype=np.float32) if with_lse else None
    cu_arr = None if cu is None else np.ascontiguousarray(cu, dtype=np.int32)
    _load().orc_lse_combine(ptr(part_out), po[0], po[1], po[2], ptr(part_lse), pl[0], pl[1], pl[2],
                            P, t_begin, t_begin + Tw, H, D, _dt(dtype), _p(out), H * D, D,
                            _p(lse) if lse is not None else None, H, 1,
                            _p(cu_arr) if cu_arr is not None else None,
                            0 if cu_arr is None else cu_arr.size - 1)
    return out, lse


def lse_combine_packed(packed: np.ndarray, P, T, H, Dv, scatter_dim, dtype="bf16"):
    rows = pack_rows(P, T, H, scatter_dim)
    out = np.empty((P * rows, Dv), dtype=np.uint16)
    lse = np.empty(P * rows, dtype=np.float32)
    _load().orc_lse_combine_packed(_p(np.ascontiguousarray(packed)), P, T, H, Dv, scatter_dim,
                                   _dt(dtype), _p(out), _p(lse))
    return out, lse


def varlen_token_rows(cu: np.ndarray, P: int) -> np.ndarray:
    """Rank-major (sequence-sharded) row of every global token."""
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    rows = np.empty(int(cu[-1]), dtype=np.int64)
    _load().orc_varlen_token_rows(_p(cu), cu.size - 1, P, _p(rows))
    return rows


def lse_combine_packed_seq(packed: np.ndarray, P, T, H, Dv, scatter_dim, dtype="bf16"):
    """Packed combine with token-major output: (out [T][H][Dv], lse [T][H])."""
    out = np.empty((T, H, Dv), dtype=np.uint16)
    lse = np.empty((T, H), dtype=np.float32)
    _load().orc_lse_combine_packed_seq(_p(np.ascontiguousarray(packed)), P, T, H, Dv, scatter_dim,
                                       _dt(dtype), _p(out), _p(lse))
    return out, lse


def lse_combine_varlen_seq(part_out: np.ndarray, part_lse: np.ndarray, cu: np.ndarray, dtype="bf16"):
    """Causal varlen combine whose token rows land in the rank-major
    (sequence-sharded) order of the varlen relayout: (out [T][H][D], lse [T][H])."""
    P = part_out.shape[0]
    out, lse = lse_combine(part_out, part_lse, dtype=dtype, cu=cu)
    rows = varlen_token_rows(cu, P)
    o2 = np.empty_like(out)
    l2 = np.empty_like(lse)
    o2[rows] = out
    l2[rows] = lse
    return o2, l2


# -- attention --------------------------------------------------------------

def attention(q_bits, k_bits, v_bits, kv_begin: int, kv_end: int, causal: bool = False,
              dtype: str = "bf16"):
    """q/k/v uint16 [T][H][D]; returns double (out [T][H][D], max [T][H], sum [T][H])."""
    q_bits = np.ascontiguousarray(q_bits)
    k_bits = np.ascontiguousarray(k_bits)
    v_bits = np.ascontiguousarray(v_bits)
    T, H, D = q_bits.shape
    out = np.empty((T, H, D))
    m = np.empty((T, H))
    s = np.empty((T, H))
    _load().orc_attention(_p(q_bits), _p(k_bits), _p(v_bits), T, H, D, _dt(dtype), kv_begin,
                          kv_end, int(causal), _p(out), _p(m), _p(s))
    return out, m, s


# -- gradient of the combine --------------------------------------------------

def combine_row_backward_f64(part_o: np.ndarray, part_l: np.ndarray, g: np.ndarray, g_lse: float = 0.0,
                             valid: np.ndarray | None = None):
    """One row in double: part_o [P][D], part_l [P], g [D] -> (dO [P][D], dL [P])."""
    part_o = np.ascontiguousarray(part_o, dtype=np.float64)
    part_l = np.ascontiguousarray(part_l, dtype=np.float64)
    g = np.ascontiguousarray(g, dtype=np.float64)
    P, D = part_o.shape
    v = np.ones(P, dtype=np.int32) if valid is None else np.ascontiguousarray(valid, dtype=np.int32)
    d_o = np.empty((P, D))
    d_l = np.empty(P)
    _load().orc_combine_row_backward_f64(_p(part_o), _p(part_l), _p(v), P, D, _p(g), float(g_lse),
                                         _p(d_o), _p(d_l))
    return d_o, d_l


def lse_combine_backward(part_out: np.ndarray, part_lse: np.ndarray, g_out: np.ndarray,
                         g_lse: np.ndarray | None = None, dtype: str = "bf16",
                         cu: np.ndarray | None = None, t_begin: int = 0):
    """Gradient of lse_combine.  part_out uint16 view [P][T'][H][D], part_lse
    float32 view [P][T'][H], g_out uint16 view [T'][H][D], g_lse float32 view
    [T'][H] or None -- T' rows starting at global token t_begin.  Returns
    (d_part_out uint16 [P][T'][H][D], d_part_lse float32 [P][T'][H])."""
    P, Tw, H, D = part_out.shape
    assert part_out.strides[3] == part_out.itemsize and g_out.strides[2] == g_out.itemsize

    def ptr(view):
        return view.__array_interface__["data"][0]

    po = _strides_el(part_out)
    pl = _strides_el(part_lse)
    go = _strides_el(g_out)
    gl = _strides_el(g_lse) if g_lse is not None else (0, 0)
    d_po = np.empty((P, Tw, H, D), dtype=np.uint16)
    d_pl = np.empty((P, Tw, H), dtype=np.float32)
    cu_arr = None if cu is None else np.ascontiguousarray(cu, dtype=np.int32)
    _load().orc_lse_combine_backward(
        ptr(part_out), po[0], po[1], po[2], ptr(part_lse), pl[0], pl[1], pl[2],
        P, t_begin, t_begin + Tw, H, D, _dt(dtype), ptr(g_out), go[0], go[1],
        ptr(g_lse) if g_lse is not None else None, gl[0], gl[1],
        _p(d_po), Tw * H * D, H * D, D, _p(d_pl), Tw * H, H, 1,
        _p(cu_arr) if cu_arr is not None else None, 0 if cu_arr is None else cu_arr.size - 1)
    return d_po, d_pl


# -- THD layout planner and planned-span relayout ------------------------------

PLAN_ERRORS = {-1: "config", -2: "lengths", -3: "blocks", -4: "capacity"}


def thd_plan(cu, world_size: int, block_size: int = 64, min_split_tokens: int = 8192,
             max_chunks_per_rank: int = 64, token_weight: float = 1.0, causal_weight: float = 1.0):
    """Plan a packed THD batch over world_size ranks.  Returns a dict with
    span_start [n+1], span_rank [n], span_local [n] (int32), rank_off [W+1]
    (int64), rank_cost [W] (float64) and grid (0 = contiguous); raises
    ValueError(kind) on a rejected input."""
    cu = np.ascontiguousarray(np.asarray(cu, dtype=np.int32))
    nseq = cu.size - 1
    cap = max(16, 4 * (nseq + world_size))
    while True:
        ss = np.empty(cap + 1, dtype=np.int32)
        sr = np.empty(cap, dtype=np.int32)
        sl = np.empty(cap, dtype=np.int32)
        ro = np.empty(max(world_size, 0) + 1, dtype=np.int64)
        rc = np.empty(max(world_size, 1), dtype=np.float64)
        n = np.zeros(1, dtype=np.int64)
        g = np.zeros(1, dtype=np.int32)
        code = _load().orc_thd_plan(_p(cu), nseq, world_size, block_size, min_split_tokens, max_chunks_per_rank,
                                    token_weight, causal_weight, cap, _p(ss), _p(sr), _p(sl), _p(ro), _p(rc),
                                    _p(n), _p(g))
        if code == -4:
            cap = int(n[0])
            continue
        if code != 0:
            raise ValueError(PLAN_ERRORS.get(code, str(code)))
        k = int(n[0])
        return {"span_start": ss[:k + 1].copy(), "span_rank": sr[:k].copy(), "span_local": sl[:k].copy(),
                "rank_off": ro.copy(), "rank_cost": rc[:world_size].copy(), "grid": int(g[0])}


TRACE_MAX_W = 16


class _PlanTrace(C.Structure):
    _fields_ = [(n, C.c_int64) for n in ("step", "over", "to", "amount", "top_seq", "top_a", "top_e",
                                        "bot_seq", "bot_a", "bot_e", "chose_bottom", "moved_seq", "moved_a",
                                        "moved_e")] + [("blk", C.c_int64 * TRACE_MAX_W),
                                                       ("caus", C.c_int64 * TRACE_MAX_W)]


def thd_plan_candidate_trace(cu, world_size: int, g: int, block_size: int = 64, min_split_tokens: int = 8192,
                             token_weight: float = 1.0, causal_weight: float = 1.0):
    """One planner candidate (g = 0 contiguous, g >= 1 a grid) with the record
    of its rebalancing steps: (spans [(seq, first block, end block, rank)],
    records [dict per C1 move (step 1) and C2 piece (step 2)], each with the
    ranks' blocks and causal work just before).  world_size <= 16."""
    cu = np.ascontiguousarray(np.asarray(cu, dtype=np.int32))
    nseq = cu.size - 1
    assert 1 <= world_size <= TRACE_MAX_W
    cap_t, cap_s = 256, 4 * (nseq + 8 * world_size) + 64
    while True:
        rec = (_PlanTrace * cap_t)()
        spans = np.empty((cap_s, 4), dtype=np.int64)
        nt = np.zeros(1, dtype=np.int64)
        ns = np.zeros(1, dtype=np.int64)
        code = _load().orc_thd_plan_candidate_trace(_p(cu), nseq, world_size, block_size, min_split_tokens,
                                                    token_weight, causal_weight, g, C.addressof(rec), cap_t,
                                                    _p(nt), _p(spans), cap_s, _p(ns))
        if code != 0:
            raise ValueError(PLAN_ERRORS.get(code, str(code)))
        if nt[0] <= cap_t and ns[0] <= cap_s:
            break
        cap_t, cap_s = int(max(cap_t, nt[0])), int(max(cap_s, ns[0]))
    out = []
    for k in range(int(nt[0])):
        r = rec[k]
        d = {n: int(getattr(r, n)) for n, _ in _PlanTrace._fields_[:14]}
        d["blk"] = [int(r.blk[i]) for i in range(world_size)]
        d["caus"] = [int(r.caus[i]) for i in range(world_size)]
        out.append(d)
    return [tuple(int(v) for v in spans[k]) for k in range(int(ns[0]))], out


def span_seq_to_head(x: np.ndarray, plan: dict, P: int, B: int, H: int, D: int) -> np.ndarray:
    """Rank-major planned slabs [B*T][H][D] -> [P][B][T][H/P][D]."""
    x = np.ascontiguousarray(x)
    T = int(plan["span_start"][-1])
    assert x.size == B * T * H * D
    out = np.empty(P * B * T * (H // P) * D, dtype=x.dtype)
    _load().orc_span_seq_to_head(_p(x), _p(out), _p(plan["span_start"]), _p(plan["span_rank"]),
                                 _p(plan["span_local"]), _p(plan["rank_off"]), plan["span_rank"].size,
                                 P, B, H, D, x.dtype.itemsize)
    return out.reshape(P, B, T, H // P, D)


def span_head_to_seq(x: np.ndarray, plan: dict, P: int, B: int, H: int, D: int) -> np.ndarray:
    """[P][B][T][H/P][D] -> rank-major planned slabs [B*T][H][D]."""
    x = np.ascontiguousarray(x)
    T = int(plan["span_start"][-1])
    assert x.size == B * T * H * D
    out = np.empty(B * T * H * D, dtype=x.dtype)
    _load().orc_span_head_to_seq(_p(x), _p(out), _p(plan["span_start"]), _p(plan["span_rank"]),
                                 _p(plan["span_local"]), _p(plan["rank_off"]), plan["span_rank"].size,
                                 P, B, H, D, x.dtype.itemsize)
    return out.reshape(B * T, H, D)


# -- causal combine over a THD layout plan ---------------------------------------

def plan_first_positions(cu, plan: dict, W: int) -> np.ndarray:
    """[W][nseq] int32: smallest position of sequence i held by rank p (INT32_MAX if none)."""
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    nseq = cu.size - 1
    first = np.empty((W, nseq), dtype=np.int32)
    _load().orc_plan_first_positions(_p(cu), nseq, W, _p(plan["span_start"]), _p(plan["span_rank"]),
                                     plan["span_rank"].size, _p(first))
    return first


def plan_piece_valid(cu, first: np.ndarray, p: int, t: int) -> bool:
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    return bool(_load().orc_plan_piece_valid(_p(cu), cu.size - 1, _p(np.ascontiguousarray(first)), p, t))


def plan_mask(cu, first: np.ndarray, P: int) -> np.ndarray:
    """[P][T] bool: partial p valid for token t under the planned rule."""
    T = int(cu[-1])
    m = np.zeros((P, T), dtype=bool)
    for p in range(P):
        for t in range(T):
            m[p, t] = plan_piece_valid(cu, first, p, t)
    return m


def lse_combine_planned(part_out: np.ndarray, part_lse: np.ndarray, cu, first: np.ndarray, dtype: str = "bf16",
                        t_begin: int = 0):
    """lse_combine with the planned validity rule; views as in lse_combine."""
    P, Tw, H, D = part_out.shape

    def ptr(view):
        return view.__array_interface__["data"][0]

    po = _strides_el(part_out)
    pl = _strides_el(part_lse)
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    first = np.ascontiguousarray(first, dtype=np.int32)
    out = np.empty((Tw, H, D), dtype=np.uint16)
    lse = np.empty((Tw, H), dtype=np.float32)
    _load().orc_lse_combine_planned(ptr(part_out), po[0], po[1], po[2], ptr(part_lse), pl[0], pl[1], pl[2],
                                    P, t_begin, t_begin + Tw, H, D, _dt(dtype), _p(out), H * D, D, _p(lse), H, 1,
                                    _p(cu), _p(first), cu.size - 1)
    return out, lse


def lse_combine_planned_backward(part_out: np.ndarray, part_lse: np.ndarray, g_out: np.ndarray,
                                 g_lse: np.ndarray | None, cu, first: np.ndarray, dtype: str = "bf16",
                                 t_begin: int = 0):
    P, Tw, H, D = part_out.shape

    def ptr(view):
        return view.__array_interface__["data"][0]

    po = _strides_el(part_out)
    pl = _strides_el(part_lse)
    go = _strides_el(g_out)
    gl = _strides_el(g_lse) if g_lse is not None else (0, 0)
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    first = np.ascontiguousarray(first, dtype=np.int32)
    d_po = np.empty((P, Tw, H, D), dtype=np.uint16)
    d_pl = np.empty((P, Tw, H), dtype=np.float32)
    _load().orc_lse_combine_planned_backward(
        ptr(part_out), po[0], po[1], po[2], ptr(part_lse), pl[0], pl[1], pl[2], P, t_begin, t_begin + Tw, H, D,
        _dt(dtype), ptr(g_out), go[0], go[1], ptr(g_lse) if g_lse is not None else None, gl[0], gl[1],
        _p(d_po), Tw * H * D, H * D, D, _p(d_pl), Tw * H, H, 1, _p(cu), _p(first), cu.size - 1)
    return d_po, d_pl


# -- Q/K/V projection into the head-sharded layout --------------------------------

def qkv_projection(x_bits: np.ndarray, w_bits: np.ndarray, P: int, B: int, H: int, D: int, dtype: str = "bf16"):
    """x [S][K], w [B*H*D][K] (payload bits) -> head-sharded [P][B][S][H/P][D] bits."""
    x_bits = np.ascontiguousarray(x_bits)
    w_bits = np.ascontiguousarray(w_bits)
    S, K = x_bits.shape
    out = np.empty((P, B, S, H // P, D), dtype=np.uint16)
    _load().orc_qkv_projection(_p(x_bits), _p(w_bits), _p(out), S, K, P, B, H, D, _dt(dtype))
    return out

