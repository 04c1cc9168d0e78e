"""Host-only checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments before enqueuing anything.  No call
here reaches a kernel launch, so these run without a GPU."""

import ctypes
import os
import re
import subprocess

import pytest

import sequence_parallelism_amd as usp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "usp.h")

OK, NULLP, SHAPE, NOTDIV, DTYPE, MISAL, WS, UNSUP = 0, 1, 2, 3, 4, 5, 6, 7
A = 1 << 20   # a fake, well-aligned non-null address: validation never dereferences it


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:usp_status|int32_t|const char\*)\s+(\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    return usp.load()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("usp_seq_to_head_permute", "usp_head_to_seq_permute", "blockattn_fwd",
              "blockattn_bwd", "lse_merge", "usp_ulysses_attn_fwd", "usp_ulysses_attn_bwd",
              "usp_seq_to_stripe_permute", "usp_stripe_to_seq_permute", "usp_striped_attn_fwd",
              "usp_striped_attn_bwd"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    out = subprocess.run(["nm", "-D", "--defined-only", usp.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if l.strip())
    for n in names:
        assert n in exported, n
        assert getattr(lib, n) is not None
    assert set(names) == set(usp.SIGNATURES)


def test_version_and_status_strings(lib):
    assert lib.usp_abi_version() == 3
    for code in range(9):
        s = lib.usp_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.usp_status_string(99).decode() == "unknown status"


def _perm(lib, fn, dst=A, src=A, P=8, S_l=16, H=32, D=128, dt=0, group=-1):
    return getattr(lib, fn)(dst, src, P, S_l, H, D, dt, group, None)


@pytest.mark.parametrize("fn", ["usp_seq_to_head_permute", "usp_head_to_seq_permute"])
def test_permute_validation(lib, fn):
    assert _perm(lib, fn, dst=None) == NULLP
    assert _perm(lib, fn, src=None) == NULLP
    assert _perm(lib, fn, H=30) == NOTDIV           # heads must split evenly over ranks
    assert _perm(lib, fn, P=0) == SHAPE
    assert _perm(lib, fn, S_l=-1) == SHAPE
    assert _perm(lib, fn, D=0) == SHAPE
    assert _perm(lib, fn, group=8) == SHAPE
    assert _perm(lib, fn, dt=7) == DTYPE


def _fwd(lib, q=A, k=A, v=A, Sq=256, Sk=256, Hq=4, Hkv=1, D=128, pos=A, qs=0, ks=0, causal=1,
         dt=0, o=A, odt=0, lse=A, ld=256, ws=A, ws_bytes=1 << 30):
    return lib.blockattn_fwd(q, k, v, Sq, Sk, Hq, Hkv, D, pos, qs, ks, causal, 0.1, dt, o, odt,
                             lse, ld, ws, ws_bytes, None)


def test_fwd_validation(lib):
    assert _fwd(lib, q=None) == NULLP
    assert _fwd(lib, lse=None) == NULLP
    assert _fwd(lib, pos=None) == NULLP                 # causal needs position_ids
    assert _fwd(lib, Hq=6, Hkv=4) == NOTDIV
    assert _fwd(lib, Sq=-1) == SHAPE
    assert _fwd(lib, ld=100) == SHAPE                   # lse leading dim < Sq
    assert _fwd(lib, qs=-5) == SHAPE
    assert _fwd(lib, D=64) == UNSUP                     # bf16 path is head dim 128
    assert _fwd(lib, dt=1, D=256, odt=1) == UNSUP
    assert _fwd(lib, dt=3) == DTYPE
    assert _fwd(lib, dt=1, odt=0, D=16) == DTYPE        # f32 input needs f32 output
    assert _fwd(lib, q=A + 2) == MISAL
    assert _fwd(lib, qs=(1 << 31) - 10) == UNSUP        # global index past int32
    n = ctypes.c_size_t(0)
    assert lib.blockattn_fwd_workspace_size(256, 256, 4, 1, 128, 0, ctypes.byref(n)) == OK and n.value > 0
    assert _fwd(lib, ws_bytes=n.value - 1) == WS
    assert _fwd(lib, ws=None) == NULLP
    assert _fwd(lib, ws=A + 8) == MISAL
    assert lib.blockattn_fwd_workspace_size(256, 256, 4, 1, 16, 1, ctypes.byref(n)) == OK and n.value == 0


def test_bwd_validation(lib):
    n = ctypes.c_size_t(0)
    assert lib.blockattn_bwd_workspace_size(256, 256, 4, 1, 128, ctypes.byref(n)) == OK
    assert n.value >= 256 * 4 * 4                       # at least D, fp32 per (row, head)
    assert lib.blockattn_bwd_workspace_size(256, 256, 4, 1, 128, None) == NULLP
    assert lib.blockattn_bwd_workspace_size(-1, 256, 4, 1, 128, ctypes.byref(n)) == SHAPE

    def bwd(ws_bytes=n.value, ws=A, dq=A, dt=0, Hq=4, Hkv=1, D=128):
        return lib.blockattn_bwd(A, A, A, A, A, 256, A, 256, 256, Hq, Hkv, D, A, 0, 0, 1, 0.1, dt,
                                 dq, A, A, ws, ws_bytes, None)
    assert bwd(ws_bytes=n.value - 1) == WS
    assert bwd(ws=None) == NULLP
    assert bwd(dq=None) == NULLP
    assert bwd(dt=1, D=16) == UNSUP
    assert bwd(Hq=3, Hkv=2) == NOTDIV
    assert bwd(ws=A + 16) == MISAL


def test_merge_validation(lib):
    m = lambda **kw: lib.lse_merge(kw.get("oa", A), kw.get("adt", 1), kw.get("la", A),
                                   kw.get("lda", 16), kw.get("ob", A), kw.get("pdt", 1),
                                   kw.get("lb", A), kw.get("ldb", 16), kw.get("S", 16),
                                   kw.get("H", 2), kw.get("D", 128), None)
    assert m(oa=None) == NULLP
    assert m(lb=None) == NULLP
    assert m(adt=5) == DTYPE
    assert m(lda=8) == SHAPE
    assert m(H=0) == SHAPE
    assert m(oa=A + 2) == MISAL


def test_ulysses_fused_validation(lib):
    """Sequence-sharded entry points: the same argument checks, plus the shard-size
    and head-divisibility rules of the fused layout."""
    n = ctypes.c_size_t(1 << 30)

    def fwd(xq=A, P=8, S_l=256, Hq=32, Hkv=8, D=128, g=0, pos=A, dt=0, o=A, lse=A, ld=2048,
            ws=A, wsb=n.value):
        return lib.usp_ulysses_attn_fwd(xq, A, A, P, S_l, Hq, Hkv, D, g, pos, 1, 0.1, dt, o, lse, ld,
                                        ws, wsb, None)
    assert fwd(xq=None) == NULLP
    assert fwd(pos=None) == NULLP
    assert fwd(ws=None) == NULLP
    assert fwd(dt=1) == UNSUP
    assert fwd(D=64) == UNSUP
    assert fwd(S_l=200) == UNSUP          # tiles must stay inside one shard
    assert fwd(g=8) == SHAPE
    assert fwd(P=0) == SHAPE
    assert fwd(Hq=30) == NOTDIV
    assert fwd(Hq=8, Hkv=16) == NOTDIV    # 1 query head per rank, 2 key/value heads
    assert fwd(ld=2047) == SHAPE
    assert fwd(xq=A + 8) == MISAL
    assert fwd(wsb=16) == WS

    def bwd(xdo=A, dxq=A, ws=A, wsb=n.value, S_l=256):
        return lib.usp_ulysses_attn_bwd(A, A, A, A, A, 2048, xdo, 8, S_l, 32, 8, 128, 0, A, 1, 0.1, 0,
                                        dxq, A, A, ws, wsb, None)
    assert bwd(xdo=None) == NULLP
    assert bwd(dxq=None) == NULLP
    assert bwd(ws=A + 16) == MISAL
    assert bwd(wsb=16) == WS
    assert bwd(S_l=128) == UNSUP


def test_striped_validation(lib):
    """Stripe permutes and stripe-pair attention: layout and rank checks on top of the
    blockattn checks."""
    for fn in ("usp_seq_to_stripe_permute", "usp_stripe_to_seq_permute"):
        f = getattr(lib, fn)
        assert f(None, A, 4, 64, 2, 128, 0, None) == NULLP
        assert f(A, A, 4, 66, 2, 128, 0, None) == NOTDIV       # S not a multiple of P
        assert f(A, A, 0, 64, 2, 128, 0, None) == SHAPE
        assert f(A, A, 4, 64, 2, 128, 5, None) == DTYPE
        assert f(A + 1, A, 4, 64, 2, 128, 0, None) == MISAL
        assert f(A, A, 4, 1 << 24, 16, 128, 0, None) == UNSUP  # S H D >= 2^31
        assert f(None, None, 4, 0, 2, 128, 0, None) == OK      # empty: nothing to do

    n = ctypes.c_size_t(1 << 30)

    def fwd(P=4, qr=1, kr=2, S=256, pos=A, ws=A):
        return lib.usp_striped_attn_fwd(A, A, A, S, 4, 1, 128, P, qr, kr, pos, 1, 0.1, 0, A, 0, A, S,
                                        ws, n.value, None)
    assert fwd(P=0) == SHAPE
    assert fwd(qr=4) == SHAPE
    assert fwd(kr=-1) == SHAPE
    assert fwd(pos=None) == NULLP
    assert fwd(ws=None) == NULLP
    assert fwd(S=(1 << 29)) == UNSUP                            # P S_stripe >= 2^31

    def bwd(P=4, qr=0, kr=3, dq=A):
        return lib.usp_striped_attn_bwd(A, A, A, A, A, 256, A, 256, 4, 1, 128, P, qr, kr, A, 1, 0.1, 0,
                                        dq, A, A, A, n.value, None)
    assert bwd(qr=-1) == SHAPE
    assert bwd(kr=4) == SHAPE
    assert bwd(dq=None) == NULLP


def test_noalloc_rejects_before_touching_the_device(lib):
    """blockattn_fwd_noalloc validates its arguments, then the size of the workspace the
    call needs against the library's scratch array, before anything else: a call whose
    launch order alone exceeds USP_NOALLOC_SCRATCH_BYTES is refused."""
    def call(q=A, Sq=256, Sk=256, Hq=4, Hkv=1, ld=None):
        return lib.blockattn_fwd_noalloc(q, A, A, Sq, Sk, Hq, Hkv, 128, A, 0, 0, 1, 0.1, 0, A, 0, A,
                                         Sq if ld is None else ld, None)
    assert call(q=None) == NULLP
    assert call(Hkv=3) == NOTDIV
    assert call(ld=100) == SHAPE
    assert call(Sq=600_000_000, Sk=16, Hq=1) == WS      # 4.7M query tiles: 18.75 MB of launch order
