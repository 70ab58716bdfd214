"""Host-side checks of the C ABI (no GPU): the library loads and exports every
function include/cam.h declares; every rejection path returns its status
before anything is launched; the host varlen plan equals the oracle's; the
packed-buffer geometry equals the oracle's; the fast-division constants are
exact."""

import ctypes as C
import re
from pathlib import Path

import numpy as np
import pytest

import synth

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "cam.h"

OK, NULL, SHAPE, DIV, ALIGN, OVERLAP, UNSUP = 0, 1, 2, 3, 4, 5, 6
BF16, FP16, FP32 = 0, 1, 2
A = 0x7F0000000000  # fake, 256-byte aligned "device" addresses: never dereferenced
Bp = 0x7F0100000000


@pytest.fixture(scope="module")
def cam():
    import context_attention_movement_amd as m
    return m


@pytest.fixture(scope="module")
def lib(cam):
    return cam.library()


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s+([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["ulysses_seq_to_head", "ulysses_head_to_seq", "ulysses_varlen_plan", "ulysses_seq_to_head_varlen",
              "lse_combine_packed_seq", "lse_combine_varlen_seq", "lse_merge",
              "ulysses_head_to_seq_varlen", "lse_pack_bytes", "lse_pack", "lse_combine_packed", "lse_combine",
              "lse_combine_varlen", "cam_status_string", "cam_last_error", "cam_abi_version", "cam_copy"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    raw = C.CDLL(str(ROOT / "context_attention_movement_amd" / "libcam.so"))
    for n in declared_functions():
        assert hasattr(raw, n), n
    assert lib.cam_abi_version() == 1


def test_status_strings(lib):
    assert lib.cam_status_string(0) == b"CAM_OK"
    assert lib.cam_status_string(5) == b"CAM_ERR_OVERLAP"


def _s2h(lib, *a):
    return lib.ulysses_seq_to_head(*a)


def test_dense_relayout_rejections(lib):
    f = lib.ulysses_seq_to_head
    assert f(A, Bp, 0, 1, 8, 4, 8, BF16, None) == SHAPE
    assert f(A, Bp, 2, -1, 8, 4, 8, BF16, None) == SHAPE
    assert f(A, Bp, 3, 1, 8, 6, 8, BF16, None) == DIV          # S % P
    assert f(A, Bp, 2, 1, 8, 3, 8, BF16, None) == DIV          # H % P
    assert b"multiples of P" in lib.cam_last_error()
    assert f(None, Bp, 2, 1, 8, 4, 8, BF16, None) == NULL
    assert f(A + 1, Bp, 2, 1, 8, 4, 8, BF16, None) == ALIGN
    assert f(A + 2, Bp, 2, 1, 8, 4, 8, FP32, None) == ALIGN
    assert f(A, A + 64, 2, 1, 8, 4, 8, BF16, None) == OVERLAP
    assert f(A, Bp, 2, 1, 8, 4, 8, 9, None) == UNSUP
    assert f(A, Bp, 2, 1 << 40, 1 << 40, 2, 2, BF16, None) == SHAPE  # size overflow
    # empty work is accepted without touching the (null) pointers
    assert f(None, None, 2, 0, 8, 4, 8, BF16, None) == OK
    assert f(None, None, 2, 1, 0, 4, 8, BF16, None) == OK
    assert lib.cam_last_error() == b""
    g = lib.ulysses_head_to_seq
    assert g(A, Bp, 2, 1, 7, 4, 8, BF16, None) == DIV
    assert g(A, A, 2, 1, 8, 4, 8, BF16, None) == OVERLAP


def test_varlen_relayout_rejections(lib):
    f = lib.ulysses_seq_to_head_varlen
    cu, rc, ro = A + 0x1000_0000, A + 0x2000_0000, A + 0x3000_0000
    assert f(A, Bp, cu, rc, ro, 3, 100, 3, 1, 4, 8, BF16, None) == DIV   # H % P
    assert f(A, Bp, cu, rc, ro, 0, 100, 2, 1, 4, 8, BF16, None) == SHAPE  # tokens without sequences
    assert f(A, Bp, None, rc, ro, 3, 100, 2, 1, 4, 8, BF16, None) == NULL
    assert f(A, Bp, cu + 2, rc, ro, 3, 100, 2, 1, 4, 8, BF16, None) == ALIGN
    assert f(A, Bp, cu, rc, ro + 4, 3, 100, 2, 1, 4, 8, BF16, None) == ALIGN
    assert f(A, A + 16, cu, rc, ro, 3, 100, 2, 1, 4, 8, BF16, None) == OVERLAP
    assert f(A, Bp, cu, rc, ro, 3, 1 << 33, 2, 1, 4, 8, BF16, None) == SHAPE
    assert f(None, None, None, None, None, 0, 0, 2, 1, 4, 8, BF16, None) == OK


def _plan(lib, cu, P):
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    nseq = cu.size - 1
    rank_cu = np.full((P, nseq + 1), -7, dtype=np.int32)
    rank_off = np.full(P + 1, -7, dtype=np.int64)
    st = lib.ulysses_varlen_plan(cu.ctypes.data, nseq, P, rank_cu.ctypes.data, rank_off.ctypes.data)
    return st, rank_cu, rank_off


@pytest.mark.parametrize("seed,nseq,P", [(1, 1, 1), (2, 5, 3), (3, 22, 8), (4, 40, 7), (5, 3, 16)])
def test_varlen_plan_equals_oracle(lib, orc, seed, nseq, P):
    cu = synth.cu_seqlens(synth.random_lengths(nseq, seed, lo=0, hi=50))
    st, rank_cu, rank_off = _plan(lib, cu, P)
    assert st == OK
    o_cu, o_off = orc.varlen_plan(cu, P)
    assert np.array_equal(rank_cu, o_cu) and np.array_equal(rank_off, o_off)


def test_varlen_plan_thd_workload(lib, orc):
    lens = synth.thd_lengths(20, 131072, seed=synth.BASE_SEED + 4)
    assert lens.size == 22 and lens.sum() == 131072 and np.all(lens[lens < 4097] >= 512)
    cu = synth.cu_seqlens(lens)
    st, rank_cu, rank_off = _plan(lib, cu, 8)
    assert st == OK and rank_off[-1] == 131072
    o_cu, o_off = orc.varlen_plan(cu, 8)
    assert np.array_equal(rank_cu, o_cu) and np.array_equal(rank_off, o_off)


def test_varlen_plan_rejections(lib):
    assert _plan(lib, [1, 4, 9], 2)[0] == SHAPE      # not zero-based
    assert _plan(lib, [0, 4, 3], 2)[0] == SHAPE      # decreasing
    assert _plan(lib, [0, 4], 0)[0] == SHAPE         # P < 1
    assert lib.ulysses_varlen_plan(None, 1, 2, None, None) == NULL


def test_pack_geometry_equals_oracle(lib, orc):
    for P, T, H, Dv, sd in [(8, 128, 128, 512, 1), (8, 128, 128, 512, 0), (2, 256, 8, 64, 1), (3, 6, 6, 5, 0),
                            (2, 3, 2, 3, 1), (1, 1, 1, 1, 1)]:
        want = P * P * orc.pack_chunk_bytes(P, T, H, Dv, sd)
        assert lib.lse_pack_bytes(P, T, H, Dv, sd, BF16) == want
    assert lib.lse_pack_bytes(8, 128, 128, 512, 1, BF16) == 64 * 2_105_344
    assert lib.lse_pack_bytes(3, 4, 4, 8, 1, BF16) == -1      # H % P
    assert lib.lse_pack_bytes(3, 4, 6, 8, 0, BF16) == -1      # T % P
    assert lib.lse_pack_bytes(2, 4, 4, 8, 2, BF16) == -1      # scatter_dim
    assert lib.lse_pack_bytes(2, 4, 4, 8, 1, FP32) == -1      # payload dtype


def test_pack_rejections(lib):
    f = lib.lse_pack
    M, S, PK = A + 0x1000_0000, A + 0x2000_0000, A + 0x4000_0000
    args = lambda out=A, m=M, s=S, pk=PK, sd=1, dt=BF16, st=(512 * 128 * 128, 512 * 128, 512): \
        (out, *st, m, 128 * 128, 128, 1, s, 128 * 128, 128, 1, 8, 128, 128, 512, sd, dt, pk, None)
    assert f(*args(out=None)) == NULL
    assert f(*args(out=A + 1)) == ALIGN
    assert f(*args(m=M + 2)) == ALIGN
    assert f(*args(pk=PK + 8)) == ALIGN
    assert f(*args(pk=A + 64)) == OVERLAP
    assert f(*args(sd=3)) == UNSUP
    assert f(*args(dt=FP32)) == UNSUP
    assert f(*args(st=(-1, 512, 1))) == UNSUP


def test_combine_rejections(lib):
    f = lib.lse_combine
    L, O, LO = A + 0x1000_0000, A + 0x2000_0000, A + 0x3000_0000
    ok = lambda **k: (k.get("po", A), 64 * 8 * 16, 8 * 16, 16, k.get("pl", L), 64 * 8, 8, 1, k.get("P", 4), 64, 8, 16,
                      k.get("dt", BF16), k.get("out", O), 8 * 16, 16, k.get("lo", LO), 8, 1, None)
    assert f(*ok(P=65)) == UNSUP
    assert f(*ok(P=0)) == SHAPE
    assert f(*ok(dt=FP32)) == UNSUP
    assert f(*ok(po=None)) == NULL
    assert f(*ok(pl=L + 2)) == ALIGN
    assert f(*ok(out=A + 32)) == OVERLAP
    assert f(*ok(lo=L)) == OVERLAP
    assert f(*ok(lo=O + 64)) == OVERLAP
    g = lib.lse_combine_varlen
    assert g(A, 64 * 8 * 16, 8 * 16, 16, L, 64 * 8, 8, 1, 4, 64, 8, 16, BF16, O, 8 * 16, 16, LO, 8, 1,
             None, 3, None) == NULL
    assert g(A, 64 * 8 * 16, 8 * 16, 16, L, 64 * 8, 8, 1, 4, 64, 8, 16, BF16, O, 8 * 16, 16, LO, 8, 1,
             A + 0x5000_0000, 0, None) == SHAPE
    h = lib.lse_combine_packed
    assert h(A + 8, 8, 128, 128, 512, 1, BF16, O, LO, None) == ALIGN
    assert h(A, 8, 128, 128, 512, 1, BF16, A + 4096, LO, None) == OVERLAP
    assert h(A, 3, 128, 128, 512, 1, BF16, O, LO, None) == DIV


def test_copy_rejections(lib):
    assert lib.cam_copy(A, Bp, 100, None) == ALIGN
    assert lib.cam_copy(A, A + 16, 64, None) == OVERLAP
    assert lib.cam_copy(None, Bp, 64, None) == NULL
    assert lib.cam_copy(None, None, 0, None) == OK


def _fastdiv(d):
    l = 0
    while (1 << l) < d:
        l += 1
    m = ((1 << 32) * ((1 << l) - d)) // d + 1
    return m, l


def test_fast_division_constants_are_exact():
    rng = np.random.default_rng(0)
    divisors = list(range(1, 300)) + [1023, 1024, 1025, 8190, 9450, 65535, 65536, 2**31 - 1, 2**31, 2**31 + 1,
                                      2**32 - 1] + rng.integers(1, 2**32, size=200).tolist()
    ns = [0, 1, 2, 3, 2**31 - 1, 2**31, 2**32 - 1, 2**32 - 2] + rng.integers(0, 2**32, size=300).tolist()
    for d in divisors:
        m, l = _fastdiv(d)
        assert 0 <= m < 2**32
        for n in ns + [d - 1, d, d + 1, 2 * d - 1, 2 * d, (2**32 - 1) // d * d, (2**32 - 1) // d * d - 1]:
            if 0 <= n < 2**32:
                assert ((n * m >> 32) + n) >> l == n // d, (d, n)


def test_fused_epilogue_rejections(lib):
    O, LO, PK = A + 0x3000_0000, A + 0x4000_0000, A
    f = lib.lse_combine_packed_seq
    assert f(PK + 8, 8, 128, 128, 512, 1, BF16, O, LO, None) == ALIGN
    assert f(PK, 8, 128, 128, 512, 1, BF16, PK + 64, LO, None) == OVERLAP
    assert f(PK, 3, 128, 128, 512, 1, BF16, O, LO, None) == DIV
    assert f(None, 8, 128, 128, 512, 1, BF16, O, LO, None) == NULL
    g = lib.lse_combine_varlen_seq
    cu, rc, ro = A + 0x5000_0000, A + 0x6000_0000, A + 0x7000_0000
    args = lambda out=O, rc=rc, ro=ro: (A, 64 * 8 * 16, 8 * 16, 16, A + 0x1000_0000, 64 * 8, 8, 1, 4, 64, 8, 16, BF16,
                                        out, LO, cu, rc, ro, 3, None)
    assert g(*args(rc=None)) == NULL
    assert g(*args(ro=ro + 4)) == ALIGN
    assert g(*args(out=rc)) == OVERLAP


def test_merge_rejections(lib):
    f = lib.lse_merge
    AL, PP, PL, F = A + 0x1000_0000, A + 0x2000_0000, A + 0x3000_0000, A + 0x4000_0000
    args = lambda acc=A, D=64, part=PP, fin=F, dt=BF16: (acc, 8 * D, D, AL, 8, 1, part, 8 * D, D, PL, 8, 1, 16, 8, D,
                                                         dt, fin, 8 * D, D, None)
    assert f(*args(D=6)) == ALIGN
    assert f(*args(acc=A + 8)) == ALIGN
    assert f(*args(part=A + 64)) == OVERLAP
    assert f(*args(fin=PP)) == OVERLAP
    assert f(*args(dt=FP32)) == UNSUP
    assert f(*args(acc=None)) == NULL


def test_last_launch_record(cam):
    import ctypes as C
    lib = cam.library()
    wg, th, lds = C.c_uint64(7), C.c_uint32(7), C.c_uint64(7)
    assert lib.cam_last_launch(C.addressof(wg), C.addressof(th), C.addressof(lds)) == 0
    assert lib.cam_last_launch(None, C.addressof(th), C.addressof(lds)) != 0


def test_combine_backward_rejections(lib):
    f = lib.lse_combine_backward
    L, G, GL, DO, DL = (A + 0x1000_0000, A + 0x2000_0000, A + 0x3000_0000, A + 0x4000_0000,
                        A + 0x5000_0000)
    P, T, H, D = 4, 64, 8, 16

    def args(po=A, pl=L, go=G, gl=GL, do=DO, dl=DL, P=P, dt=BF16):
        return (po, T * H * D, H * D, D, pl, T * H, H, 1, P, T, H, D, dt, go, H * D, D, gl, H, 1,
                do, T * H * D, H * D, D, dl, T * H, H, 1, None)

    assert f(*args(P=65)) == UNSUP
    assert f(*args(P=0)) == SHAPE
    assert f(*args(dt=FP32)) == UNSUP
    assert f(*args(go=None)) == NULL
    assert f(*args(do=None)) == NULL
    assert f(*args(dl=DL + 2)) == ALIGN
    assert f(*args(do=A + 64)) == OVERLAP        # gradient over the partials
    assert f(*args(dl=G + 4)) == OVERLAP         # gradient over the upstream gradient
    assert f(*args(dl=DO + 8)) == OVERLAP        # the two gradients overlap
    g = lib.lse_combine_varlen_backward
    assert g(*args()[:-1], None, 3, None) == NULL
    assert g(*args()[:-1], A + 0x6000_0000, 0, None) == SHAPE
    assert g(*args(dl=A + 0x6000_0000)[:-1], A + 0x6000_0000, 3, None) == OVERLAP


def test_planned_combine_rejections(lib):
    f = lib.lse_combine_planned
    L, O, LO, CU, FP = A + 0x1000_0000, A + 0x2000_0000, A + 0x3000_0000, A + 0x5000_0000, A + 0x6000_0000
    args = lambda cu=CU, fp=FP, out=O: (A, 64 * 8 * 16, 8 * 16, 16, L, 64 * 8, 8, 1, 4, 64, 8, 16, BF16,
                                        out, 8 * 16, 16, LO, 8, 1, cu, fp, 3, None)
    assert f(*args(fp=None)) == NULL
    assert f(*args(cu=None)) == NULL
    assert f(*args(fp=FP + 2)) == ALIGN
    assert f(*args(out=FP)) == OVERLAP


def test_projection_rejections(lib):
    f = lib.qkv_projection_head_sharded
    X, W, O = A, A + 0x1000_0000, A + 0x2000_0000
    assert f(X, W, O, 100, 96, 2, 1, 4, 64, BF16, None) == UNSUP       # K not a multiple of 64
    assert f(X, W, O, 100, 64, 2, 1, 3, 32, BF16, None) == DIV          # H % P
    assert f(X, W, O, 100, 64, 2, 1, 2, 64, BF16, None) == UNSUP        # N = 128 not a multiple of 256
    assert f(X, W, O, 100, 64, 2, 1, 4, 64, FP32, None) == UNSUP
    assert f(X + 8, W, O, 100, 64, 2, 1, 4, 64, BF16, None) == ALIGN
    assert f(None, W, O, 100, 64, 2, 1, 4, 64, BF16, None) == NULL
    assert f(X, W, X + 64, 100, 64, 2, 1, 4, 64, BF16, None) == OVERLAP
    assert f(X, W, O, 0, 64, 2, 1, 4, 64, BF16, None) == OK              # nothing to do


# --- the binding rejects caller buffers that do not fit the call, before any
# device check or launch (host tensors reach the shape check first) ----------

def test_binding_rejects_wrong_combine_buffers(cam):
    import torch
    P, T, H, D = 2, 5, 4, 8
    po = torch.zeros((P, T, H, D), dtype=torch.bfloat16)
    pl = torch.zeros((P, T, H), dtype=torch.float32)
    with pytest.raises(ValueError, match="out must have shape"):
        cam.lse_combine(po, pl, out=torch.zeros((T, H, D - 1), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="out must have shape"):
        cam.lse_combine(po, pl, out=torch.zeros((T - 1, H, D), dtype=torch.bfloat16))
    with pytest.raises(TypeError, match="out must be torch.bfloat16"):
        cam.lse_combine(po, pl, out=torch.zeros((T, H, D), dtype=torch.float16))
    with pytest.raises(ValueError, match="lse_out must have shape"):
        cam.lse_combine(po, pl, lse_out=torch.zeros((T, H - 1), dtype=torch.float32))
    with pytest.raises(TypeError, match="lse_out must be torch.float32"):
        cam.lse_combine(po, pl, lse_out=torch.zeros((T, H), dtype=torch.float16))
    with pytest.raises(ValueError, match="g_out must have shape"):
        cam.lse_combine_backward(po, pl, torch.zeros((T, H, D + 1), dtype=torch.bfloat16))
    with pytest.raises(TypeError, match="g_out must be torch.bfloat16"):
        cam.lse_combine_backward(po, pl, torch.zeros((T, H, D), dtype=torch.float16))
    cu = torch.tensor([0, T], dtype=torch.int32)
    with pytest.raises(ValueError, match="out must have shape"):
        cam.lse_combine_varlen(po, pl, cu, out=torch.zeros((T, H, 2 * D), dtype=torch.bfloat16))
    # a correctly shaped host buffer passes the shape check and then fails the device check
    with pytest.raises(ValueError, match="device tensor"):
        cam.lse_combine(po, pl, out=torch.zeros((T, H, D), dtype=torch.bfloat16))


def test_binding_rejects_short_packed_and_wrong_outputs(cam):
    import torch
    P, T, H, Dv = 2, 4, 4, 8
    n = cam.lse_pack_bytes(P, T, H, Dv, 1)
    rows = T * (H // P)
    with pytest.raises(ValueError, match=f"packed needs {n} bytes"):
        cam.lse_combine_packed(torch.zeros(n - 16, dtype=torch.uint8), P, T, H, Dv, 1)
    with pytest.raises(ValueError, match=f"packed needs {n} bytes"):
        cam.lse_combine_packed_seq(torch.zeros(n - 1, dtype=torch.uint8), P, T, H, Dv, 1)
    packed = torch.zeros(n, dtype=torch.uint8)
    with pytest.raises(ValueError, match="out must have shape"):
        cam.lse_combine_packed(packed, P, T, H, Dv, 1, out=torch.zeros((P * rows - 1, Dv), dtype=torch.bfloat16))
    with pytest.raises(TypeError, match="out must be torch.bfloat16"):
        cam.lse_combine_packed(packed, P, T, H, Dv, 1, out=torch.zeros((P * rows, Dv), dtype=torch.float32))
    with pytest.raises(ValueError, match="lse_out must have shape"):
        cam.lse_combine_packed(packed, P, T, H, Dv, 1, lse_out=torch.zeros(P * rows - 1, dtype=torch.float32))
    with pytest.raises(ValueError, match="out must have shape"):
        cam.lse_combine_packed_seq(packed, P, T, H, Dv, 1, out=torch.zeros((T, H, Dv - 8), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="lse_out must have shape"):
        cam.lse_combine_packed_seq(packed, P, T, H, Dv, 1, lse_out=torch.zeros((T, H + 1), dtype=torch.float32))
    with pytest.raises(TypeError, match="payload dtype"):
        cam.lse_combine_packed(packed, P, T, H, Dv, 1, dtype=torch.float32)
    with pytest.raises(ValueError, match="device tensor"):
        cam.lse_combine_packed(packed, P, T, H, Dv, 1)


def test_binding_rejects_wrong_varlen_seq_outputs(cam):
    import torch
    P, H, D = 2, 4, 8
    lens = [3, 6]
    cu = synth.cu_seqlens(lens)
    T = int(cu[-1])
    rank_cu = np.empty((P, len(lens) + 1), dtype=np.int32)
    rank_off = np.empty(P + 1, dtype=np.int64)
    plan = cam.VarlenPlan(P, len(lens), T, cu, rank_cu, rank_off, None, None, None)
    po = torch.zeros((P, T, H, D), dtype=torch.bfloat16)
    pl = torch.zeros((P, T, H), dtype=torch.float32)
    with pytest.raises(ValueError, match="out must have shape"):
        cam.lse_combine_varlen_seq(po, pl, plan, out=torch.zeros((T, H, D - 1), dtype=torch.bfloat16))
    with pytest.raises(TypeError, match="out must be torch.bfloat16"):
        cam.lse_combine_varlen_seq(po, pl, plan, out=torch.zeros((T, H, D), dtype=torch.float16))
    with pytest.raises(ValueError, match="lse_out must have shape"):
        cam.lse_combine_varlen_seq(po, pl, plan, lse_out=torch.zeros((T + 1, H), dtype=torch.float32))
    with pytest.raises(ValueError, match="part_lse must be"):
        cam.lse_combine_varlen_seq(po, pl[:, :-1], plan)


def test_binding_rejects_wrong_merge_outputs(cam):
    """A caller's out_final must be exactly [T][H][D] of the payload dtype with
    D contiguous: a short one would be written out of bounds."""
    import torch
    T, H, D = 5, 3, 8
    acc = torch.zeros((T, H, D), dtype=torch.float32)
    acc_l = torch.zeros((T, H), dtype=torch.float32)
    po = torch.zeros((T, H, D), dtype=torch.bfloat16)
    pl = torch.zeros((T, H), dtype=torch.float32)
    with pytest.raises(ValueError, match="out_final must have shape"):
        cam.lse_merge(acc, acc_l, po, pl, out_final=torch.zeros((T - 1, H, D), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="out_final must have shape"):
        cam.lse_merge(acc, acc_l, po, pl, out_final=torch.zeros((T, H, D + 1), dtype=torch.bfloat16))
    with pytest.raises(TypeError, match="out_final must be torch.bfloat16"):
        cam.lse_merge(acc, acc_l, po, pl, out_final=torch.zeros((T, H, D), dtype=torch.float16))
    with pytest.raises(ValueError, match="last dimension contiguous"):
        cam.lse_merge(acc, acc_l, po, pl, out_final=torch.zeros((T, H, 2 * D), dtype=torch.bfloat16)[:, :, ::2])
    with pytest.raises(ValueError, match="shape mismatch"):
        cam.lse_merge(acc, acc_l[:-1], po, pl)
    # shapes right: the device check comes next
    with pytest.raises(ValueError, match="must be a device tensor"):
        cam.lse_merge(acc, acc_l, po, pl, out_final=torch.zeros((T, H, D), dtype=torch.bfloat16))


def test_binding_rejects_plan_tables_on_another_device(cam):
    # a plan whose tables sit on the host must not reach a kernel that runs
    # on the device (its host addresses would be read as device memory);
    # meta tensors stand in for device data on a machine without a GPU
    import torch
    data = torch.empty((2, 3), device="meta")
    with pytest.raises(ValueError, match="the plan's tables are on cpu"):
        cam._tables_on(data, torch.zeros(3, dtype=torch.int32))
    cam._tables_on(data, torch.empty(3, dtype=torch.int32, device="meta"))  # same device: accepted


def test_rows_beyond_32bit_vector_counts_rejected(lib):
    # one row (or one head block of a row) of 2^31 or more 16-byte vectors
    # would not fit the kernels' 32-bit vector counters: refused before any
    # launch (the fake addresses are far enough apart that nothing overlaps)
    G = 1 << 40
    f = lib.ulysses_seq_to_head
    assert f(A, A + G, 1, 1, 1, 1, 1 << 35, BF16, None) == UNSUP
    assert b"2^31 vectors" in lib.cam_last_error()
    assert lib.ulysses_head_to_seq(A, A + G, 1, 1, 1, 1, 1 << 35, BF16, None) == UNSUP
    v = lib.ulysses_seq_to_head_varlen
    assert v(A, A + G, A + 2 * G, A + 3 * G, A + 4 * G, 1, 1, 1, 1, 1, 1 << 35, BF16, None) == UNSUP
    D = 1 << 34                                   # 2^35-byte bf16 rows: 2^31 vectors
    c = lib.lse_combine
    assert c(A, D, D, D, A + 2 * G, 1, 1, 1, 1, 1, 1, D, BF16, A + G, D, D, A + 3 * G, 1, 1, None) == UNSUP
    assert b"one row exceeds" in lib.cam_last_error()
    b = lib.lse_combine_backward
    assert b(A, D, D, D, A + 2 * G, 1, 1, 1, 1, 1, 1, D, BF16, A + G, D, D, None, 1, 1,
             A + 3 * G, D, D, D, A + 4 * G, 1, 1, 1, None) == UNSUP
    assert b"one row exceeds" in lib.cam_last_error()
    p = lib.lse_pack
    assert p(A, D, D, D, A + 2 * G, 1, 1, 1, A + 3 * G, 1, 1, 1, 1, 1, 1, D, 1, BF16, A + G, None) == UNSUP
    assert b"one row exceeds" in lib.cam_last_error()
    m = lib.lse_merge
    Dm = 1 << 33                                  # 2^33 fp32 accumulator elements: 2^31 four-element vectors
    assert m(A, Dm, Dm, A + G, 1, 1, A + 2 * G, Dm, Dm, A + 3 * G, 1, 1, 1, 1, Dm, BF16, None, 0, 0, None) == UNSUP
    assert b"one row exceeds" in lib.cam_last_error()


def test_empty_partials_layout(cam):
    # the partial-stack layout: each partial contiguous, a 1 MiB gap after
    # each one from 64 MiB per partial on, none below (meta tensors: no memory)
    import torch
    x = cam.empty_partials(8, 131072, 32, 128, device="meta")
    assert tuple(x.shape) == (8, 131072, 32, 128)
    assert x.stride() == (131072 * 32 * 128 + (1 << 19), 32 * 128, 128, 1)   # 2^19 bf16 elements = 1 MiB
    assert x[0].is_contiguous() and not x.is_contiguous()
    y = cam.empty_partials(8, 8191, 32, 128, device="meta")                  # just under 64 MiB per partial
    assert y.is_contiguous()
    z = cam.empty_partials(4, 8192, 32, 128, dtype=torch.float16, device="meta")
    assert z.stride(0) == 8192 * 32 * 128 + (1 << 19)
    f = cam.empty_partials(2, 1 << 20, 8, 4, dtype=torch.float32, device="meta")  # 128 MiB fp32 partials
    assert f.stride(0) == (1 << 20) * 32 + (1 << 18)
