"""Python binding of libusp.so, the MI355X (gfx950) attention share of a
sequence-parallel layer.

Argument marshalling only: every call checks its tensors' shapes, dtypes and
devices on the host, then forwards device pointers, sizes and a HIP stream to the
C ABI declared in include/usp.h; all arithmetic runs in the library's HIP kernels.
PyTorch provides device memory and streams.  There is no fallback: if the built
library is missing, every entry point raises.

Streams: every call enqueues on ``stream`` (default: the current stream).  The
temporaries a call allocates (workspace, and outputs the caller did not pass) are
allocated while that stream is current, so torch's caching allocator does not hand
their memory to other work before the call's kernels are done with it.

position_ids: int32, one entry per global token.  Every call checks that the tensor
covers each global token index it touches.  With ``debug=True`` (or the environment
variable USP_DEBUG=1) it also copies the tensor to the host and checks that it is well
formed: 0 at token 0, and at every later token either 0 (a new packed document) or
one more than at the token before.  The kernels rely on both and check neither.
"""

import contextlib
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
    "blockattn_fwd_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _c_int64, _c_int64, _c_int32, _c_int32,
                                             _c_int32, _vp, _c_int64, _c_int64, _c_int32, _c_float,
                                             ctypes.c_int, _vp, ctypes.c_int, _vp, _c_int64, _vp]),
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


# ---- host-side argument checks -------------------------------------------------------

def debug_enabled(debug=None):
    """The per-call debug flag, else USP_DEBUG=1 from the environment."""
    if debug is not None:
        return bool(debug)
    return os.environ.get("USP_DEBUG", "0") not in ("", "0")


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need(t, name, shape=None, dtype=None, dim=None):
    """A contiguous tensor of the given shape / dtype / rank (checked in that order,
    before the device, so that argument errors surface on any device)."""
    if t is None:
        raise ValueError(f"{name} is required")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dimensions, got shape {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _need_lse(t, name, rows, cols):
    """An fp32 [rows][ld >= cols] view with unit stride along the tokens."""
    import torch
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32, got {t.dtype}")
    if t.dim() != 2 or t.shape[0] != rows or t.shape[1] < cols:
        raise ValueError(f"{name} must have shape ({rows}, >= {cols}), got {tuple(t.shape)}")
    if t.stride(1) != 1 or (rows > 1 and t.stride(0) < cols):
        raise ValueError(f"{name} must be unit-stride along the tokens with a leading "
                         f"dimension of at least {cols}")


def _on_device(tensors, dev=None):
    """Every tensor on one GPU (the first one's unless dev is given)."""
    for name, t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")
    return dev


def position_ids_problem(pos, n):
    """None if the int32 array pos (host, numpy) is well formed over its first n tokens,
    else a description of the first problem: a packed document starts at token 0
    (pos 0) and wherever pos is 0; inside a document pos grows by exactly 1."""
    import numpy as np
    p = np.asarray(pos)[:n].astype(np.int64)
    if n == 0:
        return None
    if p[0] != 0:
        return f"position_ids[0] = {int(p[0])}, expected 0"
    ok = (p[1:] == 0) | (p[1:] == p[:-1] + 1)
    if not ok.all():
        t = int(np.argmin(ok)) + 1
        return (f"position_ids[{t}] = {int(p[t])} after position_ids[{t - 1}] = {int(p[t - 1])}: "
                "expected 0 (a new document) or one more")
    return None


def _check_pos(pos, needed, causal, debug):
    """position_ids: required when causal; int32, 1-D, contiguous, at least `needed`
    entries (every global token index the call touches); well formed when debugging."""
    import torch
    if not causal:
        if pos is not None:
            _need(pos, "position_ids", dtype=torch.int32, dim=1)
        return
    if pos is None:
        raise ValueError("position_ids are required for causal attention")
    _need(pos, "position_ids", dtype=torch.int32, dim=1)
    if pos.numel() < needed:
        raise ValueError(f"position_ids has {pos.numel()} entries; the call touches global "
                         f"tokens up to {needed - 1}")
    if debug_enabled(debug):
        bad = position_ids_problem(pos.cpu().numpy(), needed)
        if bad:
            raise ValueError(bad)


def _attn_inputs(q, k, v, names=("q", "k", "v")):
    """Shapes of q [Sq][Hq][D], k, v [Sk][Hkv][D] (same dtype, bf16 or float32)."""
    for t, n in zip((q, k, v), names):
        _need(t, n, dim=3)
    Sq, Hq, D = q.shape
    Sk, Hkv, Dk = k.shape
    if Dk != D or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"{names[1]}, {names[2]} must both have shape ({Sk}, {Hkv}, {D}), got "
                         f"{tuple(k.shape)} and {tuple(v.shape)}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError(f"{names[0]}, {names[1]}, {names[2]} must share one dtype")
    _dtype_code(q)
    if Hkv < 1 or Hq % Hkv:
        raise ValueError(f"query heads ({Hq}) must be a multiple of key/value heads ({Hkv})")
    return Sq, Hq, Sk, Hkv, D


def _stream_ctx(stream):
    """Makes `stream` current for the temporaries of a call (nothing if None)."""
    import torch
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _stream_handle(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _workspace(need, workspace, dev, align):
    """A caller workspace of at least `need` bytes, or a fresh one (on the current
    stream, which the caller has made the call's stream)."""
    import torch
    if workspace is None:
        return torch.empty(max(need, 1), dtype=torch.uint8, device=dev) if need > 0 else None
    if not workspace.is_contiguous() or _nbytes(workspace) < need:
        raise ValueError(f"workspace must be contiguous with at least {need} bytes")
    if workspace.data_ptr() % align:
        raise ValueError(f"workspace must be {align}-byte aligned")
    return workspace


# ---- Ulysses re-layout ----------------------------------------------------------

def seq_to_head(src, P, group=-1, out=None, stream=None):
    """[P][S_l][H][D] -> [P][P*S_l][H/P][D] (group < 0) or [P*S_l][H/P][D] (group g)."""
    import torch
    lib = load()
    _need(src, "src", dim=4)
    P_, S_l, H, D = src.shape
    if P_ != P:
        raise ValueError("src leading dim must equal P")
    if H % P:
        raise ValueError(f"heads ({H}) must be divisible by ranks ({P})")
    shape = (P, P * S_l, H // P, D) if group < 0 else (P * S_l, H // P, D)
    if out is not None:
        _need(out, "out", shape=shape, dtype=src.dtype)
    _dtype_code(src)
    _on_device((("src", src), ("out", out)))
    with _stream_ctx(stream):
        if out is None:
            out = torch.empty(shape, dtype=src.dtype, device=src.device)
        _check("usp_seq_to_head_permute",
               lib.usp_seq_to_head_permute(_ptr(out), _ptr(src), P, S_l, H, D, _dtype_code(src),
                                           group, _stream_handle(stream)))
    return out


def head_to_seq(src, P, H, out=None, group=-1, stream=None):
    """Inverse of seq_to_head.  group g writes only heads [g*H/P, (g+1)*H/P) of out."""
    import torch
    lib = load()
    if group < 0:
        _need(src, "src", dim=4)
        _, S, Hp, D = src.shape
    else:
        _need(src, "src", dim=3)
        S, Hp, D = src.shape
    if H % P or Hp != H // P or S % P:
        raise ValueError(f"src shape {tuple(src.shape)} is not a head share of {P} ranks, {H} heads")
    S_l = S // P
    if group >= 0 and out is None:
        raise ValueError("group form writes into an existing [P][S_l][H][D] tensor")
    if out is not None:
        _need(out, "out", shape=(P, S_l, H, D), dtype=src.dtype)
    _dtype_code(src)
    _on_device((("src", src), ("out", out)))
    with _stream_ctx(stream):
        if out is None:
            out = torch.empty((P, S_l, H, D), dtype=src.dtype, device=src.device)
        _check("usp_head_to_seq_permute",
               lib.usp_head_to_seq_permute(_ptr(out), _ptr(src), P, S_l, H, D, _dtype_code(src),
                                           group, _stream_handle(stream)))
    return out


# ---- attention --------------------------------------------------------------------

def fwd_workspace_bytes(Sq, Sk, Hq, Hkv, D, dtype_code=BF16):
    lib = load()
    n = ctypes.c_size_t(0)
    _check("blockattn_fwd_workspace_size",
           lib.blockattn_fwd_workspace_size(Sq, Sk, Hq, Hkv, D, dtype_code, ctypes.byref(n)))
    return n.value


def bwd_workspace_bytes(Sq, Sk, Hq, Hkv, D):
    lib = load()
    n = ctypes.c_size_t(0)
    _check("blockattn_bwd_workspace_size",
           lib.blockattn_bwd_workspace_size(Sq, Sk, Hq, Hkv, D, ctypes.byref(n)))
    return n.value


def blockattn_fwd(q, k, v, position_ids=None, q_start=0, k_start=0, causal=True, scale=None,
                  o=None, lse=None, o_dtype=None, workspace=None, stream=None, debug=None):
    """q [Sq][Hq][D], k, v [Sk][Hkv][D] -> (o [Sq][Hq][D], lse [Hq][Sq] float32)."""
    import torch
    lib = load()
    Sq, Hq, Sk, Hkv, D = _attn_inputs(q, k, v)
    if q_start < 0 or k_start < 0:
        raise ValueError("q_start and k_start must be >= 0")
    o_dtype = o_dtype or (o.dtype if o is not None else q.dtype)
    if o is not None:
        _need(o, "o", shape=(Sq, Hq, D), dtype=o_dtype)
    if lse is not None:
        _need_lse(lse, "lse", Hq, Sq)
    _check_pos(position_ids, max(q_start + Sq, k_start + Sk), causal, debug)
    dev = _on_device((("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse),
                      ("position_ids", position_ids), ("workspace", workspace)))
    scale = D ** -0.5 if scale is None else float(scale)
    with _stream_ctx(stream):
        if o is None:
            o = torch.empty((Sq, Hq, D), dtype=o_dtype, device=dev)
        if lse is None:
            lse = torch.empty((Hq, Sq), dtype=torch.float32, device=dev)
        ws = _workspace(fwd_workspace_bytes(Sq, Sk, Hq, Hkv, D, _dtype_code(q)), workspace, dev, 16)
        _check("blockattn_fwd",
               lib.blockattn_fwd(_ptr(q), _ptr(k), _ptr(v), Sq, Sk, Hq, Hkv, D, _ptr(position_ids),
                                 q_start, k_start, int(bool(causal)), scale, _dtype_code(q),
                                 _ptr(o), _dtype_code(o), _ptr(lse), lse.stride(0),
                                 _ptr(ws), _nbytes(ws), _stream_handle(stream)))
    return o, lse


NOALLOC_SCRATCH_BYTES = 16 << 20    # USP_NOALLOC_SCRATCH_BYTES of include/usp.h


def blockattn_fwd_noalloc(q, k, v, o, lse, position_ids=None, q_start=0, k_start=0, causal=True,
                          scale=None, stream=None, debug=None):
    """blockattn_fwd for callers that cannot allocate: the library's scratch array is the
    workspace and the caller passes the outputs o [Sq][Hq][D] (bf16 or float32) and
    lse [Hq][>= Sq] (float32).  Allocates nothing; returns (o, lse)."""
    lib = load()
    Sq, Hq, Sk, Hkv, D = _attn_inputs(q, k, v)
    if q_start < 0 or k_start < 0:
        raise ValueError("q_start and k_start must be >= 0")
    _need(o, "o", shape=(Sq, Hq, D))
    _dtype_code(o)
    _need_lse(lse, "lse", Hq, Sq)
    _check_pos(position_ids, max(q_start + Sq, k_start + Sk), causal, debug)
    _on_device((("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse), ("position_ids", position_ids)))
    scale = D ** -0.5 if scale is None else float(scale)
    _check("blockattn_fwd_noalloc",
           lib.blockattn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), Sq, Sk, Hq, Hkv, D, _ptr(position_ids),
                                     q_start, k_start, int(bool(causal)), scale, _dtype_code(q),
                                     _ptr(o), _dtype_code(o), _ptr(lse), lse.stride(0),
                                     _stream_handle(stream)))
    return o, lse


def blockattn_bwd(q, k, v, o, lse, dout, position_ids=None, q_start=0, k_start=0, causal=True,
                  scale=None, dq=None, dk=None, dv=None, workspace=None, stream=None, debug=None):
    """Gradients (dq, dk, dv) of blockattn_fwd for upstream gradient dout."""
    import torch
    lib = load()
    Sq, Hq, Sk, Hkv, D = _attn_inputs(q, k, v)
    if q_start < 0 or k_start < 0:
        raise ValueError("q_start and k_start must be >= 0")
    if q.dtype != torch.bfloat16:
        raise TypeError("the backward supports bfloat16 inputs only")
    _need(o, "o", shape=(Sq, Hq, D), dtype=q.dtype)
    _need(dout, "dout", shape=(Sq, Hq, D), dtype=q.dtype)
    _need_lse(lse, "lse", Hq, Sq)
    for t, n, shp in ((dq, "dq", q.shape), (dk, "dk", k.shape), (dv, "dv", v.shape)):
        if t is not None:
            _need(t, n, shape=shp, dtype=q.dtype)
    _check_pos(position_ids, max(q_start + Sq, k_start + Sk), causal, debug)
    dev = _on_device((("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse), ("dout", dout),
                      ("dq", dq), ("dk", dk), ("dv", dv), ("position_ids", position_ids),
                      ("workspace", workspace)))
    scale = D ** -0.5 if scale is None else float(scale)
    with _stream_ctx(stream):
        dq = torch.empty_like(q) if dq is None else dq
        dk = torch.empty_like(k) if dk is None else dk
        dv = torch.empty_like(v) if dv is None else dv
        ws = _workspace(bwd_workspace_bytes(Sq, Sk, Hq, Hkv, D), workspace, dev, 256)
        _check("blockattn_bwd",
               lib.blockattn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), lse.stride(0),
                                 _ptr(dout), Sq, Sk, Hq, Hkv, D, _ptr(position_ids), q_start, k_start,
                                 int(bool(causal)), scale, _dtype_code(q), _ptr(dq), _ptr(dk), _ptr(dv),
                                 _ptr(ws), _nbytes(ws), _stream_handle(stream)))
    return dq, dk, dv


# ---- Ulysses attention on the sequence-sharded layout (re-layout fused) -----------

def _ulysses_shapes(xq, xk, xv, group):
    for t, n in ((xq, "xq"), (xk, "xk"), (xv, "xv")):
        _need(t, n, dim=4)
    P, S_l, Hq, D = xq.shape
    if xk.shape[:2] != xq.shape[:2] or xk.shape[3] != D or tuple(xv.shape) != tuple(xk.shape):
        raise ValueError(f"xk, xv must have shape ({P}, {S_l}, Hkv, {D}), got {tuple(xk.shape)} "
                         f"and {tuple(xv.shape)}")
    if xq.dtype != torch_bf16() or xk.dtype != xq.dtype or xv.dtype != xq.dtype:
        raise TypeError("xq, xk, xv must be bfloat16")
    Hkv = xk.shape[2]
    if Hq % P or Hkv % P or (Hq // P) % max(Hkv // P, 1):
        raise ValueError(f"heads ({Hq} query, {Hkv} key/value) must split evenly over {P} ranks")
    if not 0 <= group < P:
        raise ValueError(f"group must be in [0, {P})")
    return P, S_l, Hq, Hkv, D


def torch_bf16():
    import torch
    return torch.bfloat16


def ulysses_attn_fwd(xq, xk, xv, group, position_ids=None, causal=True, scale=None, o_seq=None,
                     lse=None, workspace=None, stream=None, debug=None):
    """xq [P][S_l][Hq][D], xk, xv [P][S_l][Hkv][D]: rank `group`'s share of the attention,
    read in place.  Writes rank `group`'s heads of o_seq (laid out like xq; allocated
    zero-filled if None) and returns (o_seq, lse [Hq/P][P*S_l])."""
    import torch
    lib = load()
    P, S_l, Hq, Hkv, D = _ulysses_shapes(xq, xk, xv, group)
    S = P * S_l
    if o_seq is not None:
        _need(o_seq, "o_seq", shape=xq.shape, dtype=xq.dtype)
    if lse is not None:
        _need_lse(lse, "lse", Hq // P, S)
    _check_pos(position_ids, S, causal, debug)
    dev = _on_device((("xq", xq), ("xk", xk), ("xv", xv), ("o_seq", o_seq), ("lse", lse),
                      ("position_ids", position_ids), ("workspace", workspace)))
    scale = D ** -0.5 if scale is None else float(scale)
    with _stream_ctx(stream):
        if o_seq is None:
            o_seq = torch.zeros_like(xq)
        if lse is None:
            lse = torch.empty((Hq // P, S), dtype=torch.float32, device=dev)
        ws = _workspace(fwd_workspace_bytes(S, S, Hq // P, Hkv // P, D, BF16), workspace, dev, 16)
        _check("usp_ulysses_attn_fwd",
               lib.usp_ulysses_attn_fwd(_ptr(xq), _ptr(xk), _ptr(xv), P, S_l, Hq, Hkv, D, group,
                                        _ptr(position_ids), int(bool(causal)), scale, BF16,
                                        _ptr(o_seq), _ptr(lse), lse.stride(0), _ptr(ws), _nbytes(ws),
                                        _stream_handle(stream)))
    return o_seq, lse


def ulysses_attn_bwd(xq, xk, xv, o_seq, lse, xdo, group, position_ids=None, causal=True, scale=None,
                     dxq=None, dxk=None, dxv=None, workspace=None, stream=None, debug=None):
    """Gradients of ulysses_attn_fwd for rank `group`'s heads, written into that head
    slice of dxq, dxk, dxv (sequence-sharded layouts; allocated zero-filled if None)."""
    import torch
    lib = load()
    P, S_l, Hq, Hkv, D = _ulysses_shapes(xq, xk, xv, group)
    S = P * S_l
    _need(o_seq, "o_seq", shape=xq.shape, dtype=xq.dtype)
    _need(xdo, "xdo", shape=xq.shape, dtype=xq.dtype)
    _need_lse(lse, "lse", Hq // P, S)
    for t, n, shp in ((dxq, "dxq", xq.shape), (dxk, "dxk", xk.shape), (dxv, "dxv", xv.shape)):
        if t is not None:
            _need(t, n, shape=shp, dtype=xq.dtype)
    _check_pos(position_ids, S, causal, debug)
    dev = _on_device((("xq", xq), ("xk", xk), ("xv", xv), ("o_seq", o_seq), ("lse", lse),
                      ("xdo", xdo), ("dxq", dxq), ("dxk", dxk), ("dxv", dxv),
                      ("position_ids", position_ids), ("workspace", workspace)))
    scale = D ** -0.5 if scale is None else float(scale)
    with _stream_ctx(stream):
        dxq = torch.zeros_like(xq) if dxq is None else dxq
        dxk = torch.zeros_like(xk) if dxk is None else dxk
        dxv = torch.zeros_like(xv) if dxv is None else dxv
        ws = _workspace(bwd_workspace_bytes(S, S, Hq // P, Hkv // P, D), workspace, dev, 256)
        _check("usp_ulysses_attn_bwd",
               lib.usp_ulysses_attn_bwd(_ptr(xq), _ptr(xk), _ptr(xv), _ptr(o_seq), _ptr(lse),
                                        lse.stride(0), _ptr(xdo), P, S_l, Hq, Hkv, D, group,
                                        _ptr(position_ids), int(bool(causal)), scale, BF16,
                                        _ptr(dxq), _ptr(dxk), _ptr(dxv), _ptr(ws), _nbytes(ws),
                                        _stream_handle(stream)))
    return dxq, dxk, dxv


# ---- striped layout: rank r holds tokens r, r + P, r + 2P, ... ----------------------

def seq_to_stripe(x, P, out=None, stream=None):
    """[S][H][D] -> [P][S/P][H][D] with out[r][j] = x[r + P j]."""
    import torch
    lib = load()
    _need(x, "x", dim=3)
    S, H, D = x.shape
    if S % P:
        raise ValueError(f"tokens ({S}) must be a multiple of ranks ({P})")
    if out is not None:
        _need(out, "out", shape=(P, S // P, H, D), dtype=x.dtype)
    _dtype_code(x)
    _on_device((("x", x), ("out", out)))
    with _stream_ctx(stream):
        out = torch.empty((P, S // P, H, D), dtype=x.dtype, device=x.device) if out is None else out
        _check("usp_seq_to_stripe_permute",
               lib.usp_seq_to_stripe_permute(_ptr(out), _ptr(x), P, S, H, D, _dtype_code(x),
                                             _stream_handle(stream)))
    return out


def stripe_to_seq(y, out=None, stream=None):
    """[P][S/P][H][D] -> [S][H][D], the inverse of seq_to_stripe."""
    import torch
    lib = load()
    _need(y, "y", dim=4)
    P, n, H, D = y.shape
    if out is not None:
        _need(out, "out", shape=(P * n, H, D), dtype=y.dtype)
    _dtype_code(y)
    _on_device((("y", y), ("out", out)))
    with _stream_ctx(stream):
        out = torch.empty((P * n, H, D), dtype=y.dtype, device=y.device) if out is None else out
        _check("usp_stripe_to_seq_permute",
               lib.usp_stripe_to_seq_permute(_ptr(out), _ptr(y), P, P * n, H, D, _dtype_code(y),
                                             _stream_handle(stream)))
    return out


def _stripe_ranks(P, q_rank, k_rank):
    if P < 1 or not (0 <= q_rank < P and 0 <= k_rank < P):
        raise ValueError(f"ranks must be in [0, {P})")


def striped_attn_fwd(q, k, v, P, q_rank, k_rank, position_ids=None, causal=True, scale=None, o=None,
                     lse=None, o_dtype=None, workspace=None, stream=None, debug=None):
    """Stripe q_rank's queries q [n][Hq][D] against stripe k_rank's keys and values
    k, v [n][Hkv][D] -> (o [n][Hq][D], lse [Hq][n] float32)."""
    import torch
    lib = load()
    n, Hq, Sk, Hkv, D = _attn_inputs(q, k, v)
    if Sk != n:
        raise ValueError("query and key stripes must have the same length")
    _stripe_ranks(P, q_rank, k_rank)
    o_dtype = o_dtype or (o.dtype if o is not None else q.dtype)
    if o is not None:
        _need(o, "o", shape=(n, Hq, D), dtype=o_dtype)
    if lse is not None:
        _need_lse(lse, "lse", Hq, n)
    _check_pos(position_ids, P * n, causal, debug)
    dev = _on_device((("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse),
                      ("position_ids", position_ids), ("workspace", workspace)))
    scale = D ** -0.5 if scale is None else float(scale)
    with _stream_ctx(stream):
        if o is None:
            o = torch.empty((n, Hq, D), dtype=o_dtype, device=dev)
        if lse is None:
            lse = torch.empty((Hq, n), dtype=torch.float32, device=dev)
        ws = _workspace(fwd_workspace_bytes(n, n, Hq, Hkv, D, _dtype_code(q)), workspace, dev, 16)
        _check("usp_striped_attn_fwd",
               lib.usp_striped_attn_fwd(_ptr(q), _ptr(k), _ptr(v), n, Hq, Hkv, D, P, q_rank, k_rank,
                                        _ptr(position_ids), int(bool(causal)), scale, _dtype_code(q),
                                        _ptr(o), _dtype_code(o), _ptr(lse), lse.stride(0), _ptr(ws),
                                        _nbytes(ws), _stream_handle(stream)))
    return o, lse


def striped_attn_bwd(q, k, v, o, lse, dout, P, q_rank, k_rank, position_ids=None, causal=True,
                     scale=None, dq=None, dk=None, dv=None, workspace=None, stream=None, debug=None):
    """Gradients (dq, dk, dv) of striped_attn_fwd for this stripe pair, with o and lse
    the query stripe's final (merged) output and log-sum-exp."""
    import torch
    lib = load()
    n, Hq, Sk, Hkv, D = _attn_inputs(q, k, v)
    if Sk != n:
        raise ValueError("query and key stripes must have the same length")
    if q.dtype != torch.bfloat16:
        raise TypeError("the backward supports bfloat16 inputs only")
    _stripe_ranks(P, q_rank, k_rank)
    _need(o, "o", shape=(n, Hq, D), dtype=q.dtype)
    _need(dout, "dout", shape=(n, Hq, D), dtype=q.dtype)
    _need_lse(lse, "lse", Hq, n)
    for t, nm, shp in ((dq, "dq", q.shape), (dk, "dk", k.shape), (dv, "dv", v.shape)):
        if t is not None:
            _need(t, nm, shape=shp, dtype=q.dtype)
    _check_pos(position_ids, P * n, causal, debug)
    dev = _on_device((("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse), ("dout", dout),
                      ("dq", dq), ("dk", dk), ("dv", dv), ("position_ids", position_ids),
                      ("workspace", workspace)))
    scale = D ** -0.5 if scale is None else float(scale)
    with _stream_ctx(stream):
        dq = torch.empty_like(q) if dq is None else dq
        dk = torch.empty_like(k) if dk is None else dk
        dv = torch.empty_like(v) if dv is None else dv
        ws = _workspace(bwd_workspace_bytes(n, n, Hq, Hkv, D), workspace, dev, 256)
        _check("usp_striped_attn_bwd",
               lib.usp_striped_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), lse.stride(0),
                                        _ptr(dout), n, Hq, Hkv, D, P, q_rank, k_rank, _ptr(position_ids),
                                        int(bool(causal)), scale, _dtype_code(q), _ptr(dq), _ptr(dk),
                                        _ptr(dv), _ptr(ws), _nbytes(ws), _stream_handle(stream)))
    return dq, dk, dv


def lse_merge(o_acc, lse_acc, o_part, lse_part, stream=None):
    """In place: (o_acc, lse_acc) <- merge((o_acc, lse_acc), (o_part, lse_part))."""
    lib = load()
    _need(o_acc, "o_acc", dim=3)
    S, H, D = o_acc.shape
    _need(o_part, "o_part", shape=(S, H, D))
    _dtype_code(o_acc)
    _dtype_code(o_part)
    _need_lse(lse_acc, "lse_acc", H, S)
    _need_lse(lse_part, "lse_part", H, S)
    _on_device((("o_acc", o_acc), ("lse_acc", lse_acc), ("o_part", o_part), ("lse_part", lse_part)))
    _check("lse_merge",
           lib.lse_merge(_ptr(o_acc), _dtype_code(o_acc), _ptr(lse_acc), lse_acc.stride(0),
                         _ptr(o_part), _dtype_code(o_part), _ptr(lse_part), lse_part.stride(0),
                         S, H, D, _stream_handle(stream)))
    return o_acc, lse_acc


__all__ = ["load", "seq_to_head", "head_to_seq", "blockattn_fwd", "blockattn_fwd_noalloc", "blockattn_bwd",
           "ulysses_attn_fwd", "ulysses_attn_bwd", "seq_to_stripe", "stripe_to_seq",
           "striped_attn_fwd", "striped_attn_bwd", "fwd_workspace_bytes", "bwd_workspace_bytes",
           "lse_merge", "position_ids_problem", "debug_enabled", "UspError", "BF16", "F32",
           "SIGNATURES"]
