"""Python binding of libusp.so, the MI355X (gfx950) attention share of a
sequence-parallel layer.

Argument marshalling only: every call forwards device pointers, sizes and the
current HIP stream to the C ABI declared in include/usp.h; all arithmetic runs in
the library's HIP kernels.  PyTorch provides device memory and streams.  There
is no fallback: if the built library is missing, every entry point raises.
"""

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libusp.so")

BF16, F32 = 0, 1

STATUS = {
    0: "USP_OK", 1: "USP_ERR_NULL_POINTER", 2: "USP_ERR_BAD_SHAPE", 3: "USP_ERR_NOT_DIVISIBLE",
    4: "USP_ERR_BAD_DTYPE", 5: "USP_ERR_MISALIGNED", 6: "USP_ERR_WORKSPACE_TOO_SMALL",
    7: "USP_ERR_UNSUPPORTED", 8: "USP_ERR_HIP",
}

# name -> (restype, argtypes) exactly as declared in include/usp.h
_c_int32, _c_int64, _c_float, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
SIGNATURES = {
    "usp_abi_version": (_c_int32, []),
    "usp_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "usp_seq_to_head_permute": (ctypes.c_int, [_vp, _vp, _c_int32, _c_int64, _c_int32, _c_int32,
                                               ctypes.c_int, _c_int32, _vp]),
    "usp_head_to_seq_permute": (ctypes.c_int, [_vp, _vp, _c_int32, _c_int64, _c_int32, _c_int32,
                                               ctypes.c_int, _c_int32, _vp]),
    "blockattn_fwd": (ctypes.c_int, [_vp, _vp, _vp, _c_int64, _c_int64, _c_int32, _c_int32,
                                     _c_int32, _vp, _c_int64, _c_int64, _c_int32, _c_float,
                                     ctypes.c_int, _vp, ctypes.c_int, _vp, _c_int64, _vp,
                                     ctypes.c_size_t, _vp]),
    "blockattn_fwd_workspace_size": (ctypes.c_int, [_c_int64, _c_int64, _c_int32, _c_int32, _c_int32,
                                                    ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]),
    "blockattn_bwd_workspace_size": (ctypes.c_int, [_c_int64, _c_int64, _c_int32, _c_int32,
                                                    _c_int32, ctypes.POINTER(ctypes.c_size_t)]),
    "blockattn_bwd": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _c_int64, _vp, _c_int64, _c_int64,
                                     _c_int32, _c_int32, _c_int32, _vp, _c_int64, _c_int64,
                                     _c_int32, _c_float, ctypes.c_int, _vp, _vp, _vp, _vp,
                                     ctypes.c_size_t, _vp]),
    "lse_merge": (ctypes.c_int, [_vp, ctypes.c_int, _vp, _c_int64, _vp, ctypes.c_int, _vp,
                                 _c_int64, _c_int64, _c_int32, _c_int32, _vp]),
    "usp_seq_to_stripe_permute": (ctypes.c_int, [_vp, _vp, _c_int32, _c_int64, _c_int32, _c_int32,
                                                 ctypes.c_int, _vp]),
    "usp_stripe_to_seq_permute": (ctypes.c_int, [_vp, _vp, _c_int32, _c_int64, _c_int32, _c_int32,
                                                 ctypes.c_int, _vp]),
    "usp_striped_attn_fwd": (ctypes.c_int, [_vp, _vp, _vp, _c_int64, _c_int32, _c_int32, _c_int32,
                                            _c_int32, _c_int32, _c_int32, _vp, _c_int32, _c_float,
                                            ctypes.c_int, _vp, ctypes.c_int, _vp, _c_int64, _vp,
                                            ctypes.c_size_t, _vp]),
    "usp_striped_attn_bwd": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _c_int64, _vp, _c_int64, _c_int32,
                                            _c_int32, _c_int32, _c_int32, _c_int32, _c_int32, _vp,
                                            _c_int32, _c_float, ctypes.c_int, _vp, _vp, _vp, _vp,
                                            ctypes.c_size_t, _vp]),
    "usp_ulysses_attn_fwd": (ctypes.c_int, [_vp, _vp, _vp, _c_int32, _c_int64, _c_int32, _c_int32,
                                            _c_int32, _c_int32, _vp, _c_int32, _c_float, ctypes.c_int,
                                            _vp, _vp, _c_int64, _vp, ctypes.c_size_t, _vp]),
    "usp_ulysses_attn_bwd": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _c_int64, _vp, _c_int32,
                                            _c_int64, _c_int32, _c_int32, _c_int32, _c_int32, _vp,
                                            _c_int32, _c_float, ctypes.c_int, _vp, _vp, _vp, _vp,
                                            ctypes.c_size_t, _vp]),
}

_lib = None


class UspError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        msg = _lib.usp_status_string(status).decode() if _lib is not None else ""
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({msg})")


def load():
    """Load libusp.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                           "(run python -m sequence_parallelism_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(fn, status):
    if status != 0:
        raise UspError(fn, status)


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need(t, name):
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")


# ---- Ulysses re-layout ----------------------------------------------------------

def seq_to_head(src, P, group=-1, out=None, stream=None):
    """[P][S_l][H][D] -> [P][P*S_l][H/P][D] (group < 0) or [P*S_l][H/P][D] (group g)."""
    import torch
    lib = load()
    _need(src, "src")
    P_, S_l, H, D = src.shape
    if P_ != P:
        raise ValueError("src leading dim must equal P")
    shape = (P, P * S_l, H // P, D) if group < 0 else (P * S_l, H // P, D)
    if out is None:
        out = torch.empty(shape, dtype=src.dtype, device=src.device)
    _need(out, "out")
    _check("usp_seq_to_head_permute",
           lib.usp_seq_to_head_permute(_ptr(out), _ptr(src), P, S_l, H, D, _dtype_code(src),
                                       group, _stream(stream)))
    return out


def head_to_seq(src, P, H, out=None, group=-1, stream=None):
    """Inverse of seq_to_head.  group g writes only heads [g*H/P, (g+1)*H/P) of out."""
    import torch
    lib = load()
    _need(src, "src")
    if group < 0:
        _, S, Hp, D = src.shape
    else:
        S, Hp, D = src.shape
    S_l = S // P
    if out is None:
        if group >= 0:
            raise ValueError("group form writes into an existing [P][S_l][H][D] tensor")
        out = torch.empty((P, S_l, H, D), dtype=src.dtype, device=src.device)
    _need(out, "out")
    _check("usp_head_to_seq_permute",
           lib.usp_head_to_seq_permute(_ptr(out), _ptr(src), P, S_l, H, D, _dtype_code(src),
                                       group, _stream(stream)))
    return out


# ---- attention --------------------------------------------------------------------

def fwd_workspace_bytes(Sq, Sk, Hq, Hkv, D, dtype_code=BF16):
    lib = load()
    n = ctypes.c_size_t(0)
    _check("blockattn_fwd_workspace_size",
           lib.blockattn_fwd_workspace_size(Sq, Sk, Hq, Hkv, D, dtype_code, ctypes.byref(n)))
    return n.value


def blockattn_fwd(q, k, v, position_ids=None, q_start=0, k_start=0, causal=True, scale=None,
                  o=None, lse=None, o_dtype=None, workspace=None, stream=None):
    """q [Sq][Hq][D], k, v [Sk][Hkv][D] -> (o [Sq][Hq][D], lse [Hq][Sq] float32)."""
    import torch
    lib = load()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n)
    Sq, Hq, D = q.shape
    Sk, Hkv, _ = k.shape
    scale = D ** -0.5 if scale is None else float(scale)
    if o is None:
        o = torch.empty((Sq, Hq, D), dtype=o_dtype or q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((Hq, Sq), dtype=torch.float32, device=q.device)
    _need(o, "o")
    if position_ids is not None:
        _need(position_ids, "position_ids")
        if position_ids.dtype != torch.int32:
            raise TypeError("position_ids must be int32")
    need = fwd_workspace_bytes(Sq, Sk, Hq, Hkv, D, _dtype_code(q))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("blockattn_fwd",
           lib.blockattn_fwd(_ptr(q), _ptr(k), _ptr(v), Sq, Sk, Hq, Hkv, D, _ptr(position_ids),
                             q_start, k_start, int(bool(causal)), scale, _dtype_code(q),
                             _ptr(o), _dtype_code(o), _ptr(lse), lse.stride(0),
                             _ptr(workspace), ws_bytes, _stream(stream)))
    return o, lse


def bwd_workspace_bytes(Sq, Sk, Hq, Hkv, D):
    lib = load()
    n = ctypes.c_size_t(0)
    _check("blockattn_bwd_workspace_size",
           lib.blockattn_bwd_workspace_size(Sq, Sk, Hq, Hkv, D, ctypes.byref(n)))
    return n.value


def blockattn_bwd(q, k, v, o, lse, dout, position_ids=None, q_start=0, k_start=0, causal=True,
                  scale=None, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Gradients (dq, dk, dv) of blockattn_fwd for upstream gradient dout."""
    import torch
    lib = load()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _need(t, n)
    Sq, Hq, D = q.shape
    Sk, Hkv, _ = k.shape
    scale = D ** -0.5 if scale is None else float(scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = bwd_workspace_bytes(Sq, Sk, Hq, Hkv, D)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check("blockattn_bwd",
           lib.blockattn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), lse.stride(0),
                             _ptr(dout), Sq, Sk, Hq, Hkv, D, _ptr(position_ids), q_start, k_start,
                             int(bool(causal)), scale, _dtype_code(q), _ptr(dq), _ptr(dk), _ptr(dv),
                             _ptr(workspace), workspace.numel() * workspace.element_size(),
                             _stream(stream)))
    return dq, dk, dv


# ---- Ulysses attention on the sequence-sharded layout (re-layout fused) -----------

def ulysses_attn_fwd(xq, xk, xv, group, position_ids=None, causal=True, scale=None, o_seq=None,
                     lse=None, workspace=None, stream=None):
    """xq [P][S_l][Hq][D], xk, xv [P][S_l][Hkv][D]: rank `group`'s share of the attention,
    read in place.  Writes rank `group`'s heads of o_seq (laid out like xq; allocated
    zero-filled if None) and returns (o_seq, lse [Hq/P][P*S_l])."""
    import torch
    lib = load()
    for t, n in ((xq, "xq"), (xk, "xk"), (xv, "xv")):
        _need(t, n)
    P, S_l, Hq, D = xq.shape
    Hkv = xk.shape[2]
    S = P * S_l
    scale = D ** -0.5 if scale is None else float(scale)
    if o_seq is None:
        o_seq = torch.zeros_like(xq)
    if lse is None:
        lse = torch.empty((Hq // P, S), dtype=torch.float32, device=xq.device)
    _need(o_seq, "o_seq")
    if workspace is None:
        n = fwd_workspace_bytes(S, S, Hq // P, Hkv // P, D, _dtype_code(xq))
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=xq.device)
    _check("usp_ulysses_attn_fwd",
           lib.usp_ulysses_attn_fwd(_ptr(xq), _ptr(xk), _ptr(xv), P, S_l, Hq, Hkv, D, group,
                                    _ptr(position_ids), int(bool(causal)), scale, _dtype_code(xq),
                                    _ptr(o_seq), _ptr(lse), lse.stride(0), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(stream)))
    return o_seq, lse


def ulysses_attn_bwd(xq, xk, xv, o_seq, lse, xdo, group, position_ids=None, causal=True, scale=None,
                     dxq=None, dxk=None, dxv=None, workspace=None, stream=None):
    """Gradients of ulysses_attn_fwd for rank `group`'s heads, written into that head
    slice of dxq, dxk, dxv (sequence-sharded layouts; allocated zero-filled if None)."""
    import torch
    lib = load()
    for t, n in ((xq, "xq"), (xk, "xk"), (xv, "xv"), (o_seq, "o_seq"), (xdo, "xdo")):
        _need(t, n)
    P, S_l, Hq, D = xq.shape
    Hkv = xk.shape[2]
    S = P * S_l
    scale = D ** -0.5 if scale is None else float(scale)
    dxq = torch.zeros_like(xq) if dxq is None else dxq
    dxk = torch.zeros_like(xk) if dxk is None else dxk
    dxv = torch.zeros_like(xv) if dxv is None else dxv
    if workspace is None:
        n = bwd_workspace_bytes(S, S, Hq // P, Hkv // P, D)
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=xq.device)
    _check("usp_ulysses_attn_bwd",
           lib.usp_ulysses_attn_bwd(_ptr(xq), _ptr(xk), _ptr(xv), _ptr(o_seq), _ptr(lse),
                                    lse.stride(0), _ptr(xdo), P, S_l, Hq, Hkv, D, group,
                                    _ptr(position_ids), int(bool(causal)), scale, _dtype_code(xq),
                                    _ptr(dxq), _ptr(dxk), _ptr(dxv), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(stream)))
    return dxq, dxk, dxv


# ---- striped layout: rank r holds tokens r, r + P, r + 2P, ... ----------------------

def seq_to_stripe(x, P, out=None, stream=None):
    """[S][H][D] -> [P][S/P][H][D] with out[r][j] = x[r + P j]."""
    import torch
    lib = load()
    _need(x, "x")
    S, H, D = x.shape
    out = torch.empty((P, S // P, H, D), dtype=x.dtype, device=x.device) if out is None else out
    _need(out, "out")
    _check("usp_seq_to_stripe_permute",
           lib.usp_seq_to_stripe_permute(_ptr(out), _ptr(x), P, S, H, D, _dtype_code(x), _stream(stream)))
    return out


def stripe_to_seq(y, out=None, stream=None):
    """[P][S/P][H][D] -> [S][H][D], the inverse of seq_to_stripe."""
    import torch
    lib = load()
    _need(y, "y")
    P, n, H, D = y.shape
    out = torch.empty((P * n, H, D), dtype=y.dtype, device=y.device) if out is None else out
    _need(out, "out")
    _check("usp_stripe_to_seq_permute",
           lib.usp_stripe_to_seq_permute(_ptr(out), _ptr(y), P, P * n, H, D, _dtype_code(y), _stream(stream)))
    return out


def striped_attn_fwd(q, k, v, P, q_rank, k_rank, position_ids=None, causal=True, scale=None, o=None,
                     lse=None, o_dtype=None, workspace=None, stream=None):
    """Stripe q_rank's queries q [n][Hq][D] against stripe k_rank's keys and values
    k, v [n][Hkv][D] -> (o [n][Hq][D], lse [Hq][n] float32)."""
    import torch
    lib = load()
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm)
    n, Hq, D = q.shape
    Hkv = k.shape[1]
    scale = D ** -0.5 if scale is None else float(scale)
    if o is None:
        o = torch.empty((n, Hq, D), dtype=o_dtype or q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((Hq, n), dtype=torch.float32, device=q.device)
    _need(o, "o")
    need = fwd_workspace_bytes(n, n, Hq, Hkv, D, _dtype_code(q))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("usp_striped_attn_fwd",
           lib.usp_striped_attn_fwd(_ptr(q), _ptr(k), _ptr(v), n, Hq, Hkv, D, P, q_rank, k_rank,
                                    _ptr(position_ids), int(bool(causal)), scale, _dtype_code(q),
                                    _ptr(o), _dtype_code(o), _ptr(lse), lse.stride(0), _ptr(workspace),
                                    ws_bytes, _stream(stream)))
    return o, lse


def striped_attn_bwd(q, k, v, o, lse, dout, P, q_rank, k_rank, position_ids=None, causal=True,
                     scale=None, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Gradients (dq, dk, dv) of striped_attn_fwd for this stripe pair, with o and lse
    the query stripe's final (merged) output and log-sum-exp."""
    import torch
    lib = load()
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _need(t, nm)
    n, Hq, D = q.shape
    Hkv = k.shape[1]
    scale = D ** -0.5 if scale is None else float(scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = bwd_workspace_bytes(n, n, Hq, Hkv, D)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check("usp_striped_attn_bwd",
           lib.usp_striped_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), lse.stride(0),
                                    _ptr(dout), n, Hq, Hkv, D, P, q_rank, k_rank, _ptr(position_ids),
                                    int(bool(causal)), scale, _dtype_code(q), _ptr(dq), _ptr(dk), _ptr(dv),
                                    _ptr(workspace), workspace.numel() * workspace.element_size(),
                                    _stream(stream)))
    return dq, dk, dv


def lse_merge(o_acc, lse_acc, o_part, lse_part, stream=None):
    """In place: (o_acc, lse_acc) <- merge((o_acc, lse_acc), (o_part, lse_part))."""
    lib = load()
    for t, n in ((o_acc, "o_acc"), (o_part, "o_part")):
        _need(t, n)
    S, H, D = o_acc.shape
    _check("lse_merge",
           lib.lse_merge(_ptr(o_acc), _dtype_code(o_acc), _ptr(lse_acc), lse_acc.stride(0),
                         _ptr(o_part), _dtype_code(o_part), _ptr(lse_part), lse_part.stride(0),
                         S, H, D, _stream(stream)))
    return o_acc, lse_acc


__all__ = ["load", "seq_to_head", "head_to_seq", "blockattn_fwd", "blockattn_bwd",
           "ulysses_attn_fwd", "ulysses_attn_bwd", "seq_to_stripe", "stripe_to_seq",
           "striped_attn_fwd", "striped_attn_bwd",
           "fwd_workspace_bytes", "bwd_workspace_bytes", "lse_merge", "UspError", "BF16", "F32", "SIGNATURES"]
