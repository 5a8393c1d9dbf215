"""ctypes binding of libulysses.so: argument marshalling only.

Every step of the hot path runs in the HIP library; this module turns torch
tensors into device pointers and sizes, passes the current HIP stream, and
turns non-OK statuses into exceptions. There is no fallback: if the library
is not built, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os
from typing import Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libulysses.so"

ULY_OK, ULY_ERR_INVALID_ARG, ULY_ERR_UNSUPPORTED, ULY_ERR_HIP = 0, 1, 2, 3
ULY_F32, ULY_BF16 = 0, 1
ULY_MAX_P = 64
ULY_NOALLOC_SCRATCH_BYTES = 128 << 20

# name -> (restype, argtypes); mirrors include/ulysses.h
_vp = ctypes.c_void_p
_i32 = ctypes.c_int
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
SIGNATURES = {
    "ulysses_pack": (_i32, [ctypes.POINTER(_vp), _i32, _i64, _i32, _i32, _i32, _i32, _vp, _vp]),
    "ulysses_unpack": (_i32, [_vp, _i32, _i64, _i32, _i32, _i32, _i32, ctypes.POINTER(_vp), _vp]),
    "ulysses_pack_heads": (_i32, [ctypes.POINTER(_vp), _i32, _i64, _i32, _i32, _i32, _i32, _i32, _vp, _vp]),
    "ulysses_unpack_heads": (_i32, [_vp, _i32, _i64, _i32, _i32, _i32, _i32, _i32, ctypes.POINTER(_vp), _vp]),
    "ulysses_pack_multi": (_i32, [_i32, ctypes.POINTER(_vp), ctypes.POINTER(_i32), _i32, _i64, _i32, _i32, _i32,
                                   ctypes.POINTER(_vp), _vp]),
    "ulysses_unpack_multi": (_i32, [_i32, ctypes.POINTER(_vp), ctypes.POINTER(_i32), _i32, _i64, _i32, _i32, _i32,
                                     ctypes.POINTER(_vp), _vp]),
    "ulysses_pack_qkv": (_i32, [ctypes.POINTER(_vp), _i32, _i64, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp,
                                 _vp]),
    "ulysses_unpack_qkv": (_i32, [_vp, _vp, _vp, _i32, _i64, _i32, _i32, _i32, _i32, _i32,
                                   ctypes.POINTER(_vp), _vp]),
    "attn_fwd": (_i32, [_vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _vp, _i32, _f32, _i32, _vp]),
    "attn_fwd_from_shards": (_i32, [ctypes.POINTER(_vp), ctypes.POINTER(_vp), ctypes.POINTER(_vp), _i32, _i64, _i32,
                                     _i32, _i32, _i32, _i32, _vp, _vp, _vp, _i32, _f32, _i32, _vp]),
    "attn_merge": (_i32, [ctypes.POINTER(_vp), ctypes.POINTER(_vp), _i32, _i64, _i32, _i32, _i32, _vp, _vp, _vp]),
    "attn_bwd_workspace_size": (_i32, [_i64, _i32, _i32, _i32, _i32, ctypes.POINTER(ctypes.c_size_t)]),
    "attn_bwd": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _vp, _i32,
                        _f32, _i32, _vp, ctypes.c_size_t, _vp]),
    "attn_bwd_ex": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _vp, _i32,
                           _f32, _i32, _vp, ctypes.c_size_t, _vp, _i32]),
    "attn_bwd_accumulate": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _vp,
                                   _i32, _f32, _i32, _vp, ctypes.c_size_t, _vp]),
    "attn_bwd_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _vp,
                                _i32, _f32, _i32, _vp]),
    "uly_last_error": (ctypes.c_char_p, []),
    "uly_check_cu_seqlens": (_i32, [ctypes.POINTER(ctypes.c_int32), _i32, _i64]),
}

_lib = None


class UlyssesError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"status {status}: {message}")
        self.status = status
        self.message = message


def lib_path() -> str:
    return os.path.join(_HERE, LIB_NAME)


def lib() -> ctypes.CDLL:
    """Load the HIP library (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: the HIP library must be built (python -c "
                "'import __graft_entry__ as g; g.build()'); there is no fallback path")
        # torch ships its own HIP runtime with the same soname as ROCm's. Load
        # torch first so this library binds to that already-loaded runtime;
        # loading ours first would put two HIP runtimes in the process.
        import torch  # noqa: F401
        cdll = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(cdll, name)
            fn.restype = res
            fn.argtypes = args
        _lib = cdll
    return _lib


def last_error() -> str:
    return lib().uly_last_error().decode()


def _raise(status: int) -> None:
    if status != ULY_OK:
        raise UlyssesError(status, last_error())


# ----------------------------------------------------------------- marshalling
def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return ULY_F32
    if t.dtype == torch.bfloat16:
        return ULY_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t, shape, dtype, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _cu(cu_seqlens, N):
    import torch
    if cu_seqlens is None:
        return None, 0
    if not cu_seqlens.is_cuda or cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 \
            or not cu_seqlens.is_contiguous() or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be a contiguous 1-D int32 device tensor with >= 2 entries")
    return ctypes.c_void_p(cu_seqlens.data_ptr()), cu_seqlens.numel() - 1


# ------------------------------------------------------------------ entry points
def ulysses_pack(shards: Sequence, group: int, out, stream=None) -> None:
    """out[j*T + t, h] = shards[j][t, group*hh + h] (see include/ulysses.h)."""
    P = len(shards)
    T, H, D = shards[0].shape
    dt = shards[0].dtype
    ptrs = (ctypes.c_void_p * P)(*[_dev(s, (T, H, D), dt, f"shards[{j}]").value for j, s in enumerate(shards)])
    if H % P == 0:
        _dev(out, (P * T, H // P, D), dt, "out")
    _raise(lib().ulysses_pack(ptrs, P, T, H, D, _dtype_code(shards[0]), group,
                              ctypes.c_void_p(out.data_ptr()), _stream(stream)))


def ulysses_unpack(inp, group: int, shards: Sequence, stream=None) -> None:
    """shards[j][t, group*hh + h] = inp[j*T + t, h]; other heads untouched."""
    P = len(shards)
    T, H, D = shards[0].shape
    dt = shards[0].dtype
    ptrs = (ctypes.c_void_p * P)(*[_dev(s, (T, H, D), dt, f"shards[{j}]").value for j, s in enumerate(shards)])
    if H % P == 0:
        _dev(inp, (P * T, H // P, D), dt, "inp")
    _raise(lib().ulysses_unpack(ctypes.c_void_p(inp.data_ptr()), P, T, H, D, _dtype_code(shards[0]), group,
                                ptrs, _stream(stream)))


def ulysses_pack_heads(shards: Sequence, head0: int, nheads: int, out, stream=None) -> None:
    """out[j*T + t, h] = shards[j][t, head0 + h] (see include/ulysses.h)."""
    P = len(shards)
    T, H, D = shards[0].shape
    dt = shards[0].dtype
    ptrs = (ctypes.c_void_p * P)(*[_dev(s, (T, H, D), dt, f"shards[{j}]").value for j, s in enumerate(shards)])
    if nheads >= 1:
        _dev(out, (P * T, nheads, D), dt, "out")
    _raise(lib().ulysses_pack_heads(ptrs, P, T, H, D, _dtype_code(shards[0]), head0, nheads,
                                    ctypes.c_void_p(out.data_ptr()), _stream(stream)))


def ulysses_unpack_heads(inp, head0: int, nheads: int, shards: Sequence, stream=None) -> None:
    """shards[j][t, head0 + h] = inp[j*T + t, h]; other heads untouched."""
    P = len(shards)
    T, H, D = shards[0].shape
    dt = shards[0].dtype
    ptrs = (ctypes.c_void_p * P)(*[_dev(s, (T, H, D), dt, f"shards[{j}]").value for j, s in enumerate(shards)])
    if nheads >= 1:
        _dev(inp, (P * T, nheads, D), dt, "inp")
    _raise(lib().ulysses_unpack_heads(ctypes.c_void_p(inp.data_ptr()), P, T, H, D, _dtype_code(shards[0]), head0,
                                      nheads, ptrs, _stream(stream)))


def _multi(tensors, packed, name):
    n = len(tensors)
    if n < 1 or n != len(packed):
        raise ValueError("need one packed tensor per shard list, at least one")
    P = len(tensors[0])
    T, _, D = tensors[0][0].shape
    dt = tensors[0][0].dtype
    ptrs, heads = [], []
    for i, sh in enumerate(tensors):
        if len(sh) != P:
            raise ValueError("every tensor needs the same number of shards")
        H = sh[0].shape[1]
        heads.append(H)
        ptrs += [_dev(s, (T, H, D), dt, f"{name}[{i}][{j}]").value for j, s in enumerate(sh)]
        if H % P == 0:
            _dev(packed[i], (P * T, H // P, D), dt, f"packed[{i}]")
    return (n, (ctypes.c_void_p * len(ptrs))(*ptrs), (ctypes.c_int * n)(*heads), P, T, D, _dtype_code(tensors[0][0]),
            (ctypes.c_void_p * n)(*[t.data_ptr() for t in packed]))


def ulysses_pack_multi(tensors: Sequence, group: int, outs: Sequence, stream=None) -> None:
    """ulysses_pack of up to three tensors in one launch: tensors[i] is the
    list of P shards of tensor i (see include/ulysses.h)."""
    n, ptrs, heads, P, T, D, dt, packed = _multi(tensors, outs, "tensors")
    _raise(lib().ulysses_pack_multi(n, ptrs, heads, P, T, D, dt, group, packed, _stream(stream)))


def ulysses_unpack_multi(ins: Sequence, group: int, tensors: Sequence, stream=None) -> None:
    """ulysses_unpack of up to three tensors in one launch; heads outside the
    group are untouched."""
    n, ptrs, heads, P, T, D, dt, packed = _multi(tensors, ins, "tensors")
    _raise(lib().ulysses_unpack_multi(n, packed, heads, P, T, D, dt, group, ptrs, _stream(stream)))


def _qkv_shards(shards, Hq: int, Hkv: int):
    P = len(shards)
    T, H, D = shards[0].shape
    if H != Hq + 2 * Hkv:
        raise ValueError(f"fused shards have {H} heads, expected Hq + 2*Hkv = {Hq + 2 * Hkv}")
    dt = shards[0].dtype
    ptrs = (ctypes.c_void_p * P)(*[_dev(s, (T, H, D), dt, f"shards[{j}]").value for j, s in enumerate(shards)])
    return P, T, D, dt, ptrs


def ulysses_pack_qkv(shards: Sequence, Hq: int, Hkv: int, group: int, q_out, k_out, v_out, stream=None) -> None:
    """Fused-QKV pack: shards[j] is [T, Hq + 2*Hkv, D] (query, then key, then
    value heads); writes the group's q/k/v heads of every token (see
    include/ulysses.h)."""
    P, T, D, dt, ptrs = _qkv_shards(shards, Hq, Hkv)
    if Hq % P == 0 and Hkv % P == 0:
        _dev(q_out, (P * T, Hq // P, D), dt, "q_out")
        _dev(k_out, (P * T, Hkv // P, D), dt, "k_out")
        _dev(v_out, (P * T, Hkv // P, D), dt, "v_out")
    _raise(lib().ulysses_pack_qkv(ptrs, P, T, Hq, Hkv, D, _dtype_code(shards[0]), group,
                                  ctypes.c_void_p(q_out.data_ptr()), ctypes.c_void_p(k_out.data_ptr()),
                                  ctypes.c_void_p(v_out.data_ptr()), _stream(stream)))


def ulysses_unpack_qkv(dq, dk, dv, Hq: int, Hkv: int, group: int, shards: Sequence, stream=None) -> None:
    """Inverse of ulysses_pack_qkv; heads outside the group are untouched."""
    P, T, D, dt, ptrs = _qkv_shards(shards, Hq, Hkv)
    if Hq % P == 0 and Hkv % P == 0:
        _dev(dq, (P * T, Hq // P, D), dt, "dq")
        _dev(dk, (P * T, Hkv // P, D), dt, "dk")
        _dev(dv, (P * T, Hkv // P, D), dt, "dv")
    _raise(lib().ulysses_unpack_qkv(ctypes.c_void_p(dq.data_ptr()), ctypes.c_void_p(dk.data_ptr()),
                                    ctypes.c_void_p(dv.data_ptr()), P, T, Hq, Hkv, D, _dtype_code(shards[0]),
                                    group, ptrs, _stream(stream)))


def attn_fwd(q, k, v, o, lse, softmax_scale: float, cu_seqlens=None, causal: int = 1, stream=None) -> None:
    """Causal GQA attention forward for one head group (see include/ulysses.h)."""
    import torch
    N, hq, D = q.shape
    hk = k.shape[1]
    dt = q.dtype
    args = [_dev(q, (N, hq, D), dt, "q"), _dev(k, (N, hk, D), dt, "k"), _dev(v, (N, hk, D), dt, "v"),
            _dev(o, (N, hq, D), dt, "o"), _dev(lse, (hq, N), torch.float32, "lse")]
    cu, nd = _cu(cu_seqlens, N)
    _raise(lib().attn_fwd(*args, N, hq, hk, D, _dtype_code(q), cu, nd, float(softmax_scale), int(causal),
                          _stream(stream)))


def attn_fwd_from_shards(q_shards: Sequence, k_shards: Sequence, v_shards: Sequence, group: int, o, lse,
                         softmax_scale: float, cu_seqlens=None, causal: int = 1, stream=None) -> None:
    """attn_fwd for head group `group`, reading the sequence-sharded Q/K/V in
    place (see include/ulysses.h)."""
    import torch
    P = len(q_shards)
    if len(k_shards) != P or len(v_shards) != P:
        raise ValueError("q, k and v need the same number of shards")
    T, Hq, D = q_shards[0].shape
    Hkv = k_shards[0].shape[1]
    dt = q_shards[0].dtype

    def arr(shards, H, name):
        return (ctypes.c_void_p * P)(*[_dev(s, (T, H, D), dt, f"{name}[{j}]").value for j, s in enumerate(shards)])
    qa, ka, va = arr(q_shards, Hq, "q_shards"), arr(k_shards, Hkv, "k_shards"), arr(v_shards, Hkv, "v_shards")
    if Hq % P == 0:
        _dev(o, (P * T, Hq // P, D), dt, "o")
        _dev(lse, (Hq // P, P * T), torch.float32, "lse")
    cu, nd = _cu(cu_seqlens, P * T)
    _raise(lib().attn_fwd_from_shards(qa, ka, va, P, T, Hq, Hkv, D, _dtype_code(q_shards[0]), group,
                                      ctypes.c_void_p(o.data_ptr()), ctypes.c_void_p(lse.data_ptr()), cu, nd,
                                      float(softmax_scale), int(causal), _stream(stream)))


def attn_merge(o_parts: Sequence, lse_parts: Sequence, o, lse, stream=None) -> None:
    """o, lse = the merge of per-key-chunk results (see include/ulysses.h)."""
    import torch
    n = len(o_parts)
    if n != len(lse_parts) or n < 1:
        raise ValueError("need as many lse parts as output parts, at least one")
    N, hq, D = o.shape
    dt = o.dtype
    op = (ctypes.c_void_p * n)(*[_dev(t, (N, hq, D), dt, f"o_parts[{c}]").value for c, t in enumerate(o_parts)])
    lp = (ctypes.c_void_p * n)(*[_dev(t, (hq, N), torch.float32, f"lse_parts[{c}]").value
                                 for c, t in enumerate(lse_parts)])
    _raise(lib().attn_merge(op, lp, n, N, hq, D, _dtype_code(o), _dev(o, (N, hq, D), dt, "o"),
                            _dev(lse, (hq, N), torch.float32, "lse"), _stream(stream)))


def attn_bwd_workspace_size(N: int, hq: int, hk: int, D: int, dtype) -> int:
    out = ctypes.c_size_t(0)
    code = ULY_BF16 if str(dtype).endswith("bfloat16") else ULY_F32
    _raise(lib().attn_bwd_workspace_size(N, hq, hk, D, code, ctypes.byref(out)))
    return out.value


def attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, softmax_scale: float, workspace, cu_seqlens=None,
             causal: int = 1, stream=None) -> None:
    """Gradients dq, dk, dv (of q's dtype) of sum(dout * o) (see include/ulysses.h)."""
    _bwd("attn_bwd", q, k, v, o, dout, lse, dq, dk, dv, softmax_scale, workspace, cu_seqlens, causal, stream,
         grad_dtype=q.dtype)


def attn_bwd_ex(q, k, v, o, dout, lse, dq, dk, dv, softmax_scale: float, workspace, cu_seqlens=None,
                causal: int = 1, stream=None) -> None:
    """attn_bwd with the gradient type taken from dq: q's dtype, or float32
    (see include/ulysses.h)."""
    _bwd("attn_bwd_ex", q, k, v, o, dout, lse, dq, dk, dv, softmax_scale, workspace, cu_seqlens, causal, stream,
         grad_dtype=dq.dtype, extra=(_dtype_code(dq),))


def attn_bwd_accumulate(q, k, v, o, dout, lse, dq, dk, dv, softmax_scale: float, workspace, cu_seqlens=None,
                        causal: int = 1, stream=None) -> None:
    """attn_bwd adding to float32 dq, dk, dv (see include/ulysses.h)."""
    import torch
    _bwd("attn_bwd_accumulate", q, k, v, o, dout, lse, dq, dk, dv, softmax_scale, workspace, cu_seqlens, causal,
         stream, grad_dtype=torch.float32)


def attn_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, softmax_scale: float, cu_seqlens=None, causal: int = 1,
                     stream=None) -> None:
    """attn_bwd with the library's static buffer as workspace: allocates
    nothing (see include/ulysses.h)."""
    import torch
    N, hq, D = q.shape
    hk = k.shape[1]
    dt = q.dtype
    args = [_dev(q, (N, hq, D), dt, "q"), _dev(k, (N, hk, D), dt, "k"), _dev(v, (N, hk, D), dt, "v"),
            _dev(o, (N, hq, D), dt, "o"), _dev(dout, (N, hq, D), dt, "dout"),
            _dev(lse, (hq, N), torch.float32, "lse"), _dev(dq, (N, hq, D), dt, "dq"),
            _dev(dk, (N, hk, D), dt, "dk"), _dev(dv, (N, hk, D), dt, "dv")]
    cu, nd = _cu(cu_seqlens, N)
    _raise(lib().attn_bwd_noalloc(*args, N, hq, hk, D, _dtype_code(q), cu, nd, float(softmax_scale), int(causal),
                                  _stream(stream)))


def _bwd(fn, q, k, v, o, dout, lse, dq, dk, dv, softmax_scale, workspace, cu_seqlens, causal, stream, grad_dtype,
         extra=()):
    import torch
    N, hq, D = q.shape
    hk = k.shape[1]
    dt = q.dtype
    args = [_dev(q, (N, hq, D), dt, "q"), _dev(k, (N, hk, D), dt, "k"), _dev(v, (N, hk, D), dt, "v"),
            _dev(o, (N, hq, D), dt, "o"), _dev(dout, (N, hq, D), dt, "dout"),
            _dev(lse, (hq, N), torch.float32, "lse"), _dev(dq, (N, hq, D), grad_dtype, "dq"),
            _dev(dk, (N, hk, D), grad_dtype, "dk"), _dev(dv, (N, hk, D), grad_dtype, "dv")]
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    ws_bytes = workspace.numel() * workspace.element_size()
    cu, nd = _cu(cu_seqlens, N)
    _raise(getattr(lib(), fn)(*args, N, hq, hk, D, _dtype_code(q), cu, nd, float(softmax_scale), int(causal),
                              ctypes.c_void_p(workspace.data_ptr()), ws_bytes, _stream(stream), *extra))


def uly_check_cu_seqlens(host_cu, N: int) -> None:
    """Host check of document offsets (a sequence of ints or an int32 array)."""
    vals = [int(x) for x in host_cu]
    arr = (ctypes.c_int32 * len(vals))(*vals)
    _raise(lib().uly_check_cu_seqlens(arr, len(vals) - 1, N))
