"""ctypes binding of liblogra.so: the C ABI declared in include/logra.h.

Argument marshalling only.  Every step of the path runs in the HIP kernels of
liblogra.so; torch is used for device memory (output and workspace tensors)
and for the current stream.  There is no fallback: if the library is not
built, or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, c_char_p, c_double, c_float, c_int, c_int64, c_size_t, \
    c_uint32, c_uint64, c_void_p

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblogra.so")

OK, ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_ALIGN, ERR_ALIAS, ERR_DOMAIN, ERR_HIP, ERR_WORKSPACE, ERR_HOST = range(10)
F32, BF16, I8 = 0, 1, 2
ROUND_NEAREST, ROUND_STOCHASTIC = 0, 1
MAX_RANK = 256
MAX_GROUP = 16

# Every symbol the header exports, with (restype, argtypes).
class Key(Structure):
    _fields_ = [("seed", c_uint64), ("matrix_id", c_uint32), ("step", c_uint32)]


class AccDesc(Structure):
    _fields_ = [("D", c_void_p), ("XAt", c_void_p), ("S", c_void_p), ("d", c_int64), ("ldd", c_int64)]


class ProjectDesc(Structure):
    _fields_ = [("key", Key), ("X", c_void_p), ("k", c_int64), ("ldx", c_int64), ("XAt", c_void_p),
                ("planes", c_void_p), ("planes_bytes", c_size_t)]


class AccPackedDesc(Structure):
    _fields_ = [("D", c_void_p), ("planes", c_void_p), ("S", c_void_p), ("d", c_int64),
                ("ldd", c_int64), ("planes_bytes", c_size_t)]


class MergeDesc(Structure):
    _fields_ = [("key", Key), ("W", c_void_p), ("d", c_int64), ("k", c_int64), ("ldw", c_int64),
                ("U", c_void_p), ("row0", c_int64)]


class MergePackedDesc(Structure):
    _fields_ = [("key", Key), ("W", c_void_p), ("d", c_int64), ("k", c_int64), ("ldw", c_int64),
                ("U_packed", c_void_p), ("row0", c_int64), ("packed_bytes", c_size_t)]


class MismatchState(Structure):
    _fields_ = [("kappa", c_double), ("valid", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class SyncHeader(Structure):
    _fields_ = [("magic", ctypes.c_uint32), ("version", ctypes.c_uint32), ("key", Key), ("d", c_int64),
                ("k", c_int64), ("r", c_int64), ("mode", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("sr_seed", c_uint64), ("row0", c_int64), ("payload_bytes", c_uint64)]


class SyncDesc(Structure):
    _fields_ = [("header", POINTER(SyncHeader)), ("payload", c_void_p), ("W", c_void_p), ("ldw", c_int64)]


class RowAdamDesc(Structure):
    _fields_ = [("S", c_void_p), ("v", c_void_p), ("U_packed", c_void_p), ("packed_bytes", c_size_t),
                ("d", c_int64)]


class MergeExplicitDesc(Structure):
    _fields_ = [("key", Key), ("W", c_void_p), ("d", c_int64), ("k", c_int64), ("ldw", c_int64),
                ("U_packed", c_void_p), ("A_packed", c_void_p), ("row0", c_int64),
                ("packed_bytes", c_size_t), ("A_packed_bytes", c_size_t)]


SIGNATURES = {
    "logra_version": (c_char_p, []),
    "logra_last_error": (c_char_p, []),
    "logra_sketch_bytes": (c_int64, [c_int64, c_int64]),
    "logra_regen_A": (c_int, [POINTER(Key), c_int64, c_int64, c_int, c_void_p, c_void_p]),
    "logra_project_input": (c_int, [POINTER(Key), c_int64, c_int64, c_int64, c_void_p, c_int,
                                    c_int64, c_void_p, c_void_p]),
    "logra_packed_input_bytes": (c_size_t, [c_int64, c_int64]),
    "logra_project_input_packed": (c_int, [POINTER(Key), c_int64, c_int64, c_int64, c_void_p, c_int,
                                           c_int64, c_void_p, c_void_p, c_size_t, c_void_p]),
    "logra_sketch_accumulate_grouped_packed": (c_int, [c_int64, c_int64, POINTER(AccPackedDesc),
                                                       c_int, c_void_p]),
    "logra_sketch_accumulate_ws_bytes": (c_size_t, [c_int64, c_int64, c_int64]),
    "logra_sketch_accumulate": (c_int, [c_int64, c_int64, c_int64, c_void_p, c_int, c_int64,
                                        c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "logra_sketch_accumulate_grouped": (c_int, [c_int64, c_int64, c_int, POINTER(AccDesc), c_int,
                                                c_void_p, c_size_t, c_void_p]),
    "logra_rowadam_ws_bytes": (c_size_t, [c_int64]),
    "logra_rowadam": (c_int, [c_int64, c_int64, c_void_p, c_void_p, c_int64, c_double, c_double,
                              c_void_p, c_void_p, c_size_t, c_void_p]),
    "logra_predicted_kl_q_ws_bytes": (c_size_t, [c_int64, c_int64]),
    "logra_predicted_kl_q": (c_int, [c_int64, c_int64, c_void_p, c_void_p, c_int, c_float,
                                     c_void_p, c_void_p, c_size_t, c_void_p]),
    "logra_step_alpha": (c_int, [c_double, c_double, c_double, POINTER(c_double)]),
    "logra_step_alpha_dev": (c_int, [c_void_p, c_float, c_float, c_void_p, c_void_p]),
    "logra_merge_grouped": (c_int, [c_int64, POINTER(MergeDesc), c_int, c_double, c_void_p, c_int,
                                    c_uint64, c_void_p]),
    "logra_packed_update_bytes": (c_size_t, [c_int64, c_int64]),
    "logra_sketch_accumulate_table_ws_bytes": (c_size_t, [c_int]),
    "logra_sketch_accumulate_table": (c_int, [c_int64, c_int64, POINTER(AccPackedDesc), c_int, c_void_p,
                                              c_size_t, c_void_p]),
    "logra_project_input_table_ws_bytes": (c_size_t, [c_int]),
    "logra_project_input_table": (c_int, [c_int64, c_int64, POINTER(ProjectDesc), c_int, c_void_p, c_size_t,
                                          c_void_p]),
    "logra_merge_projection_packed_bytes": (c_size_t, [c_int64, c_int64]),
    "logra_pack_merge_projection": (c_int, [c_int64, c_int64, c_void_p, c_void_p, c_size_t, c_void_p]),
    "logra_merge_grouped_explicit": (c_int, [c_int64, POINTER(MergeExplicitDesc), c_int, c_double, c_void_p,
                                             c_int, c_uint64, c_void_p]),
    "logra_regen_A_gaussian": (c_int, [POINTER(Key), c_int64, c_int64, c_void_p, c_void_p]),
    "logra_projection_packed_bytes": (c_size_t, [c_int64, c_int64]),
    "logra_pack_projection": (c_int, [c_int64, c_int64, c_void_p, c_void_p, c_size_t, c_void_p]),
    "logra_project_input_explicit": (c_int, [c_int64, c_int64, c_int64, c_void_p, c_int, c_int64, c_void_p,
                                             c_size_t, c_void_p, c_void_p, c_size_t, c_void_p]),
    "logra_reconstruction_cosine_explicit": (c_int, [c_int64, c_int64, c_int64, c_void_p, c_int, c_int64,
                                                     c_void_p, c_void_p, c_size_t, c_void_p, c_void_p,
                                                     c_size_t, c_void_p]),
    "logra_exact_kl_ws_bytes": (c_size_t, [c_int64]),
    "logra_exact_kl": (c_int, [c_int64, c_int64, c_void_p, c_void_p, c_int, c_double, c_double, c_void_p,
                               c_void_p, c_size_t, c_void_p]),
    "logra_sync_pack": (c_int, [POINTER(Key), c_int64, c_int64, c_int64, c_void_p, c_double, c_void_p,
                                c_int, c_uint64, c_int64, POINTER(SyncHeader), c_void_p, c_size_t,
                                c_void_p]),
    "logra_sync_apply": (c_int, [POINTER(SyncDesc), c_int, c_void_p]),
    "logra_reconstruction_cosine_ws_bytes": (c_size_t, [c_int64, c_int64, c_int64]),
    "logra_reconstruction_cosine": (c_int, [POINTER(Key), c_int64, c_int64, c_int64, c_void_p, c_int,
                                            c_int64, c_void_p, c_void_p, c_size_t, c_void_p]),
    "logra_kl_budget": (c_int, [c_int64, c_int64, c_double, c_double, POINTER(c_double)]),
    "logra_mismatch_update": (c_int, [POINTER(MismatchState), c_double, c_double]),
    "logra_effective_budget": (c_int, [c_double, POINTER(MismatchState), POINTER(c_double)]),
    "logra_pack_update": (c_int, [c_int64, c_int64, c_void_p, c_void_p, c_size_t, c_void_p]),
    "logra_rowadam_packed": (c_int, [c_int64, c_int64, c_void_p, c_void_p, c_int64, c_double,
                                     c_double, c_void_p, c_size_t, c_void_p, c_size_t, c_void_p]),
    "logra_rowadam_grouped_ws_bytes": (c_size_t, [c_int, c_int64]),
    "logra_rowadam_packed_grouped": (c_int, [c_int64, POINTER(RowAdamDesc), c_int, c_int64, c_double,
                                             c_double, c_void_p, c_size_t, c_void_p]),
    "logra_merge_grouped_packed": (c_int, [c_int64, POINTER(MergePackedDesc), c_int, c_double,
                                           c_void_p, c_int, c_uint64, c_void_p]),
    "logra_merge": (c_int, [POINTER(Key), c_int64, c_int64, c_int64, c_void_p, c_int, c_int64,
                            c_void_p, c_double, c_void_p, c_int, c_uint64, c_int64, c_void_p]),
    "logra_bandwidth_probe": (c_int, [c_int, c_void_p, c_void_p, c_size_t, c_int, c_void_p]),
    "logra_predicted_kl_q_noalloc": (c_int, [c_int64, c_int64, c_void_p, c_void_p, c_int, c_float,
                                             c_void_p, c_void_p]),
}

_lib_handle = None


class LograError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"logra status {status}: {msg}")
        self.status = status


def lib():
    """Load liblogra.so once; raise if it has not been built."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m rank_gradient_sketching_logra_amd.build` (hipcc, gfx950)")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib_handle = h
    return _lib_handle


def _check(status: int):
    if status != OK:
        raise LograError(status, lib().logra_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(t: torch.Tensor, stream=None):
    if stream is not None:
        return c_void_p(stream.cuda_stream)
    return c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return None if t is None else c_void_p(t.data_ptr())


def _ld(t: torch.Tensor) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with unit column stride")
    return t.stride(0)


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _need_dtype(name: str, t: torch.Tensor, dtype):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _need_sketch(name: str, S: torch.Tensor, d: int, r: int):
    """S (or U): fp32, contiguous, [d x r]."""
    if S.dtype != torch.float32 or not S.is_contiguous() or tuple(S.shape) != (d, r):
        raise ValueError(f"{name} must be a contiguous fp32 [{d} x {r}] tensor, got "
                         f"{S.dtype} {tuple(S.shape)}{'' if S.is_contiguous() else ' (not contiguous)'}")


def _scratch(nbytes: int, device, stream=None) -> torch.Tensor:
    """An internal workspace for one call.  It is allocated on the current stream; when the
    call runs on another stream, the allocator is told so (record_stream), so the memory is
    not handed out again before that stream has finished with it."""
    ws = workspace(nbytes, device)
    if stream is not None:
        ws.record_stream(stream)
    return ws


def key(seed: int, matrix_id: int, step: int) -> Key:
    return Key(seed, matrix_id, step)


def version() -> str:
    return lib().logra_version().decode()


def sketch_bytes(d: int, r: int) -> int:
    return lib().logra_sketch_bytes(d, r)


def regen_A(k_: Key, r: int, k: int, out_dtype=torch.int8, device="cuda", stream=None):
    """Materialise A [r x k]: int8 signs or fp32 sigma * fl32(1/sqrt(r))."""
    A = torch.empty((r, k), dtype=out_dtype, device=device)
    code = I8 if out_dtype == torch.int8 else F32 if out_dtype == torch.float32 else -1
    _check(lib().logra_regen_A(ctypes.byref(k_), r, k, code, _ptr(A), _stream(A, stream)))
    return A


def project_input(k_: Key, X: torch.Tensor, r: int, out=None, stream=None):
    """XAt = X A^T, [T x r] fp32."""
    T, k = X.shape
    XAt = out if out is not None else torch.empty((T, r), dtype=torch.float32, device=X.device)
    _check(lib().logra_project_input(ctypes.byref(k_), T, k, r, _ptr(X), _dtype_code(X), _ld(X),
                                     _ptr(XAt), _stream(X, stream)))
    return XAt


def packed_input_bytes(T: int, r: int) -> int:
    return lib().logra_packed_input_bytes(T, r)


def project_input_packed(k_: Key, X: torch.Tensor, r: int, planes=None, out=None, stream=None):
    """Packed projected input (uint8 tensor of packed_input_bytes(T, r) bytes) and, if out is
    given, also XAt = X A^T [T x r] fp32 in out.  Returns planes."""
    T, k = X.shape
    nb = packed_input_bytes(T, r)
    planes = planes if planes is not None else torch.empty((nb,), dtype=torch.uint8, device=X.device)
    _check(lib().logra_project_input_packed(ctypes.byref(k_), T, k, r, _ptr(X), _dtype_code(X), _ld(X),
                                            _ptr(out), _ptr(planes), planes.numel(), _stream(X, stream)))
    return planes


def project_input_table_ws_bytes(n: int) -> int:
    return lib().logra_project_input_table_ws_bytes(n)


def project_input_table(items, r: int, ws=None, stream=None):
    """items: sequence of (key, X bf16 [T x k], XAt fp32 [T x r] or None, planes or None) sharing
    T and r; one persistent launch writes every given output."""
    n = len(items)
    T = items[0][1].shape[0]
    descs = (ProjectDesc * n)()
    for i, (k_, X, XAt, P) in enumerate(items):
        if X.shape[0] != T:
            raise ValueError("every X must have the same number of tokens")
        _need_dtype("X", X, torch.bfloat16)
        if XAt is not None:
            _need_sketch("XAt", XAt, T, r)
        descs[i] = ProjectDesc(k_, X.data_ptr(), X.shape[1], _ld(X),
                               None if XAt is None else XAt.data_ptr(),
                               None if P is None else P.data_ptr(), 0 if P is None else _nbytes(P))
    if ws is None:
        ws = _scratch(project_input_table_ws_bytes(n), items[0][1].device, stream)
    _check(lib().logra_project_input_table(T, r, descs, n, _ptr(ws), ws.numel(), _stream(items[0][1], stream)))


def sketch_accumulate_grouped_packed(items, r: int, stream=None):
    """items: sequence of (D, planes, S) with bf16 D sharing T and r; one launch."""
    n = len(items)
    T = items[0][0].shape[0]
    descs = (AccPackedDesc * n)()
    for i, (D, planes, S) in enumerate(items):
        if D.shape[0] != T:
            raise ValueError("every D must have the same number of tokens")
        _need_dtype("D", D, torch.bfloat16)
        _need_sketch("S", S, D.shape[1], r)
        descs[i] = AccPackedDesc(D.data_ptr(), planes.data_ptr(), S.data_ptr(), D.shape[1], _ld(D),
                                 _nbytes(planes))
    _check(lib().logra_sketch_accumulate_grouped_packed(T, r, descs, n, _stream(items[0][0], stream)))


def accumulate_ws_bytes(T: int, d: int, r: int) -> int:
    return lib().logra_sketch_accumulate_ws_bytes(T, d, r)


def accumulate_grouped_ws_bytes(T: int, ds, r: int) -> int:
    """Workspace of a grouped call: the per-descriptor workspaces, in order."""
    return sum(accumulate_ws_bytes(T, d, r) for d in ds)


def workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty((max(int(nbytes), 16),), dtype=torch.uint8, device=device)


def sketch_accumulate(D: torch.Tensor, XAt: torch.Tensor, S: torch.Tensor, ws=None, stream=None):
    """S += D^T XAt (in place)."""
    T, d = D.shape
    r = S.shape[1]
    if ws is None:
        ws = _scratch(accumulate_ws_bytes(T, d, r), D.device, stream)
    _check(lib().logra_sketch_accumulate(T, d, r, _ptr(D), _dtype_code(D), _ld(D), _ptr(XAt),
                                         _ptr(S), _ptr(ws), ws.numel(), _stream(D, stream)))
    return S


def sketch_accumulate_grouped(items, ws=None, stream=None):
    """items: sequence of (D, XAt, S) sharing T, r and D's dtype; one launch."""
    n = len(items)
    T = items[0][0].shape[0]
    r = items[0][2].shape[1]
    descs = (AccDesc * n)()
    for i, (D, XAt, S) in enumerate(items):
        descs[i] = AccDesc(D.data_ptr(), XAt.data_ptr(), S.data_ptr(), D.shape[1], _ld(D))
    if ws is None:
        ws = _scratch(accumulate_grouped_ws_bytes(T, [D.shape[1] for (D, _, _) in items], r),
                      items[0][0].device, stream)
    _check(lib().logra_sketch_accumulate_grouped(T, r, _dtype_code(items[0][0]), descs, n, _ptr(ws),
                                                 ws.numel(), _stream(items[0][0], stream)))


def rowadam_ws_bytes(d: int) -> int:
    return lib().logra_rowadam_ws_bytes(d)


def rowadam(S: torch.Tensor, v: torch.Tensor, t: int, beta: float, eps: float, U=None, ws=None,
            stream=None):
    """U = RowAdam(S) with v updated in place; U may be S."""
    d, r = S.shape
    U = U if U is not None else torch.empty_like(S)
    if ws is None:
        ws = _scratch(rowadam_ws_bytes(d), S.device, stream)
    _check(lib().logra_rowadam(d, r, _ptr(S), _ptr(v), t, beta, eps, _ptr(U), _ptr(ws), ws.numel(),
                               _stream(S, stream)))
    return U


def predicted_kl_q_ws_bytes(P: int, V: int) -> int:
    return lib().logra_predicted_kl_q_ws_bytes(P, V)


def predicted_kl_q(z: torch.Tensor, zdot: torch.Tensor, tau: float, out=None, ws=None, stream=None):
    """q on the device (one-element fp32 tensor)."""
    P, V = z.shape
    q = out if out is not None else torch.empty((1,), dtype=torch.float32, device=z.device)
    if ws is None:
        ws = _scratch(predicted_kl_q_ws_bytes(P, V), z.device, stream)
    _check(lib().logra_predicted_kl_q(P, V, _ptr(z), _ptr(zdot), _dtype_code(z), tau, _ptr(q),
                                      _ptr(ws), ws.numel(), _stream(z, stream)))
    return q


NOALLOC_MAX_CONTEXTS = 4096


def predicted_kl_q_noalloc(z: torch.Tensor, zdot: torch.Tensor, tau: float, out: torch.Tensor,
                           stream=None):
    """q on the device with no workspace: the library's per-GPU scratch holds the partials (for
    callers that cannot allocate).  out is the caller's one-element fp32 tensor; nothing is
    allocated here."""
    P, V = z.shape
    _need_dtype("zdot", zdot, z.dtype)
    _check(lib().logra_predicted_kl_q_noalloc(P, V, _ptr(z), _ptr(zdot), _dtype_code(z), tau, _ptr(out),
                                              _stream(z, stream)))
    return out


def step_alpha(q: float, delta: float, alpha_max: float) -> float:
    out = c_double(0.0)
    _check(lib().logra_step_alpha(q, delta, alpha_max, ctypes.byref(out)))
    return out.value


def step_alpha_dev(q_dev: torch.Tensor, delta: float, alpha_max: float, out=None, stream=None):
    a = out if out is not None else torch.empty((1,), dtype=torch.float32, device=q_dev.device)
    _check(lib().logra_step_alpha_dev(_ptr(q_dev), delta, alpha_max, _ptr(a), _stream(q_dev, stream)))
    return a


def merge(k_: Key, W: torch.Tensor, U: torch.Tensor, scale: float, scale_dev=None,
          mode: str = "nearest", sr_seed: int = 0, row0: int = 0, stream=None):
    """W <- round(W - s U A) in place."""
    d, kk = W.shape
    r = U.shape[1]
    m = ROUND_NEAREST if mode == "nearest" else ROUND_STOCHASTIC if mode == "stochastic" else -1
    _check(lib().logra_merge(ctypes.byref(k_), d, kk, r, _ptr(W), _dtype_code(W), _ld(W), _ptr(U),
                             float(scale), _ptr(scale_dev), m, sr_seed, row0, _stream(W, stream)))
    return W


def merge_grouped(items, scale: float, scale_dev=None, mode: str = "nearest", sr_seed: int = 0,
                  stream=None):
    """items: sequence of (key, W, U) or (key, W, U, row0) with bf16 W sharing r; one launch."""
    n = len(items)
    r = items[0][2].shape[1]
    descs = (MergeDesc * n)()
    for i, it in enumerate(items):
        k_, W, U = it[0], it[1], it[2]
        row0 = it[3] if len(it) > 3 else 0
        if U.shape[1] != r:
            raise ValueError("every U must be [d x r] with the same r")
        descs[i] = MergeDesc(k_, W.data_ptr(), W.shape[0], W.shape[1], _ld(W), U.data_ptr(), row0)
    m = ROUND_NEAREST if mode == "nearest" else ROUND_STOCHASTIC if mode == "stochastic" else -1
    _check(lib().logra_merge_grouped(r, descs, n, scale, _ptr(scale_dev), m, sr_seed,
                                     _stream(items[0][1], stream)))


def packed_update_bytes(d: int, r: int) -> int:
    return lib().logra_packed_update_bytes(d, r)


def pack_update(U: torch.Tensor, out=None, stream=None):
    """The merge's packed form of fp32 U [d x r] (a uint8 tensor)."""
    d, r = U.shape
    nb = packed_update_bytes(d, r)
    P = out if out is not None else torch.empty((nb,), dtype=torch.uint8, device=U.device)
    _check(lib().logra_pack_update(d, r, _ptr(U), _ptr(P), P.numel() * P.element_size(),
                                   _stream(U, stream)))
    return P


def rowadam_packed(S: torch.Tensor, v: torch.Tensor, t: int, beta: float, eps: float, out=None,
                   ws=None, stream=None):
    """RowAdam(S) written as the merge's packed update, v updated in place."""
    d, r = S.shape
    nb = packed_update_bytes(d, r)
    P = out if out is not None else torch.empty((nb,), dtype=torch.uint8, device=S.device)
    if ws is None:
        ws = _scratch(rowadam_ws_bytes(d), S.device, stream)
    _check(lib().logra_rowadam_packed(d, r, _ptr(S), _ptr(v), t, beta, eps, _ptr(P),
                                      P.numel() * P.element_size(), _ptr(ws), ws.numel(),
                                      _stream(S, stream)))
    return P


def rowadam_grouped_ws_bytes(n: int, total_rows: int) -> int:
    return lib().logra_rowadam_grouped_ws_bytes(n, total_rows)


def rowadam_packed_grouped(items, r: int, t: int, beta: float, eps: float, ws=None, stream=None):
    """items: sequence of (S fp32 [d x r], v fp32 [d], P packed update) sharing r; RowAdam of
    every sketch in three launches, each result as its own rowadam_packed call."""
    n = len(items)
    descs = (RowAdamDesc * n)()
    rows = 0
    for i, (S, v, P) in enumerate(items):
        if S.shape[1] != r or v.shape[0] != S.shape[0]:
            raise ValueError("S must be [d x r] and v [d]")
        descs[i] = RowAdamDesc(S.data_ptr(), v.data_ptr(), P.data_ptr(), P.numel() * P.element_size(),
                               S.shape[0])
        rows += S.shape[0]
    if ws is None:
        ws = _scratch(rowadam_grouped_ws_bytes(n, rows), items[0][0].device, stream)
    _check(lib().logra_rowadam_packed_grouped(r, descs, n, t, beta, eps, _ptr(ws), ws.numel(),
                                              _stream(items[0][0], stream)))


def merge_grouped_packed(items, r: int, scale: float, scale_dev=None, mode: str = "nearest",
                         sr_seed: int = 0, stream=None):
    """items: sequence of (key, W, U_packed) or (key, W, U_packed, row0) with bf16 W; one launch."""
    n = len(items)
    descs = (MergePackedDesc * n)()
    for i, it in enumerate(items):
        k_, W, P = it[0], it[1], it[2]
        row0 = it[3] if len(it) > 3 else 0
        _need_dtype("W", W, torch.bfloat16)
        descs[i] = MergePackedDesc(k_, W.data_ptr(), W.shape[0], W.shape[1], _ld(W), P.data_ptr(), row0,
                                   _nbytes(P))
    m = ROUND_NEAREST if mode == "nearest" else ROUND_STOCHASTIC if mode == "stochastic" else -1
    _check(lib().logra_merge_grouped_packed(r, descs, n, scale, _ptr(scale_dev), m, sr_seed,
                                            _stream(items[0][1], stream)))


def kl_budget(u: int, H: int, delta_max: float, delta_min: float) -> float:
    out = c_double(0.0)
    _check(lib().logra_kl_budget(u, H, delta_max, delta_min, ctypes.byref(out)))
    return out.value


def mismatch_update(state: MismatchState, measurement, weight: float = 0.3) -> MismatchState:
    """Fold one mismatch measurement (None: no valid measurement) into state, in place."""
    m = float("nan") if measurement is None else float(measurement)
    _check(lib().logra_mismatch_update(ctypes.byref(state), m, weight))
    return state


def effective_budget(delta_u: float, state: MismatchState) -> float:
    out = c_double(0.0)
    _check(lib().logra_effective_budget(delta_u, ctypes.byref(state), ctypes.byref(out)))
    return out.value


def reconstruction_cosine_ws_bytes(d: int, k: int, r: int) -> int:
    return lib().logra_reconstruction_cosine_ws_bytes(d, k, r)


def reconstruction_cosine(k_: Key, G: torch.Tensor, r: int, out=None, ws=None, stream=None):
    """{cos(G, (G A^T) A), ||G||^2, ||G A^T||^2, ||G A^T A||^2} on the device (fp64 [4])."""
    d, kk = G.shape
    o = out if out is not None else torch.empty((4,), dtype=torch.float64, device=G.device)
    if ws is None:
        ws = _scratch(reconstruction_cosine_ws_bytes(d, kk, r), G.device, stream)
    _check(lib().logra_reconstruction_cosine(ctypes.byref(k_), d, kk, r, _ptr(G), _dtype_code(G), _ld(G),
                                             _ptr(o), _ptr(ws), ws.numel(), _stream(G, stream)))
    return o


def sync_pack(k_: Key, W_shape, U: torch.Tensor, scale: float, scale_dev=None, mode: str = "nearest",
              sr_seed: int = 0, row0: int = 0, out=None, stream=None):
    """(header, payload): what the trainer sends for one matrix -- the packed fl32(s U)."""
    d, r = U.shape
    kk = int(W_shape[1])
    nb = packed_update_bytes(d, r)
    P = out if out is not None else torch.empty((nb,), dtype=torch.uint8, device=U.device)
    h = SyncHeader()
    m = ROUND_NEAREST if mode == "nearest" else ROUND_STOCHASTIC if mode == "stochastic" else -1
    _check(lib().logra_sync_pack(ctypes.byref(k_), d, kk, r, _ptr(U), float(scale), _ptr(scale_dev), m,
                                 sr_seed, row0, ctypes.byref(h), _ptr(P), P.numel() * P.element_size(),
                                 _stream(U, stream)))
    return h, P


def sync_apply(items, stream=None):
    """items: sequence of (header, payload, W); one grouped merge with scale 1."""
    n = len(items)
    descs = (SyncDesc * n)()
    keep = []
    for i, (h, P, W) in enumerate(items):
        keep.append(h)
        descs[i] = SyncDesc(ctypes.pointer(h), P.data_ptr(), W.data_ptr(), _ld(W))
    _check(lib().logra_sync_apply(descs, n, _stream(items[0][2], stream)))


def exact_kl_ws_bytes(P: int) -> int:
    return lib().logra_exact_kl_ws_bytes(P)


def exact_kl(z: torch.Tensor, zdot: torch.Tensor, alpha: float, tau: float, out=None, ws=None,
             stream=None):
    """Mean KL of a step alpha along zdot, on the device (one fp64 element)."""
    P, V = z.shape
    o = out if out is not None else torch.empty((1,), dtype=torch.float64, device=z.device)
    if ws is None:
        ws = _scratch(exact_kl_ws_bytes(P), z.device, stream)
    _check(lib().logra_exact_kl(P, V, _ptr(z), _ptr(zdot), _dtype_code(z), float(alpha), float(tau),
                                _ptr(o), _ptr(ws), ws.numel(), _stream(z, stream)))
    return o


def regen_A_gaussian(k_: Key, r: int, k: int, device="cuda", stream=None):
    """The Gaussian projection variant A [r x k] (fp32) for key k_."""
    A = torch.empty((r, k), dtype=torch.float32, device=device)
    _check(lib().logra_regen_A_gaussian(ctypes.byref(k_), r, k, _ptr(A), _stream(A, stream)))
    return A


def projection_packed_bytes(r: int, k: int) -> int:
    return lib().logra_projection_packed_bytes(r, k)


def pack_projection(A: torch.Tensor, out=None, stream=None):
    """An explicit fp32 A [r x k] in the projection kernel's operand form (uint8 tensor)."""
    r, k = A.shape
    nb = projection_packed_bytes(r, k)
    P = out if out is not None else torch.empty((nb,), dtype=torch.uint8, device=A.device)
    _check(lib().logra_pack_projection(r, k, _ptr(A), _ptr(P), P.numel(), _stream(A, stream)))
    return P


def project_input_explicit(X: torch.Tensor, A_packed: torch.Tensor, r: int, planes=None, out=None,
                           want_xat: bool = True, stream=None):
    """X A^T with an explicit packed projection: returns (XAt or None, planes or None)."""
    T, k = X.shape
    XAt = out if out is not None else (torch.empty((T, r), dtype=torch.float32, device=X.device)
                                       if want_xat else None)
    pb = planes.numel() if planes is not None else 0
    _check(lib().logra_project_input_explicit(T, k, r, _ptr(X), _dtype_code(X), _ld(X), _ptr(A_packed),
                                              A_packed.numel(), _ptr(XAt), _ptr(planes), pb,
                                              _stream(X, stream)))
    return XAt, planes


def reconstruction_cosine_explicit(G: torch.Tensor, A: torch.Tensor, A_packed: torch.Tensor, out=None,
                                   ws=None, stream=None):
    """reconstruction_cosine with an explicit projection A (fp32) and its packed form."""
    d, kk = G.shape
    r = A.shape[0]
    o = out if out is not None else torch.empty((4,), dtype=torch.float64, device=G.device)
    if ws is None:
        ws = _scratch(reconstruction_cosine_ws_bytes(d, kk, r), G.device, stream)
    _check(lib().logra_reconstruction_cosine_explicit(d, kk, r, _ptr(G), _dtype_code(G), _ld(G), _ptr(A),
                                                      _ptr(A_packed), A_packed.numel(), _ptr(o), _ptr(ws),
                                                      ws.numel(), _stream(G, stream)))
    return o


def merge_projection_packed_bytes(r: int, k: int) -> int:
    return lib().logra_merge_projection_packed_bytes(r, k)


def pack_merge_projection(A: torch.Tensor, out=None, stream=None):
    """An explicit fp32 A [r x k] in the merge's operand order (uint8 tensor)."""
    r, k = A.shape
    nb = merge_projection_packed_bytes(r, k)
    P = out if out is not None else torch.empty((nb,), dtype=torch.uint8, device=A.device)
    _check(lib().logra_pack_merge_projection(r, k, _ptr(A), _ptr(P), P.numel(), _stream(A, stream)))
    return P


def merge_grouped_explicit(items, r: int, scale: float, scale_dev=None, mode: str = "nearest",
                           sr_seed: int = 0, stream=None):
    """items: (key, W, U_packed, A_packed) or (key, W, U_packed, A_packed, row0); one launch."""
    n = len(items)
    descs = (MergeExplicitDesc * n)()
    for i, it in enumerate(items):
        k_, W, P, Ap = it[0], it[1], it[2], it[3]
        row0 = it[4] if len(it) > 4 else 0
        _need_dtype("W", W, torch.bfloat16)
        descs[i] = MergeExplicitDesc(k_, W.data_ptr(), W.shape[0], W.shape[1], _ld(W), P.data_ptr(),
                                     Ap.data_ptr(), row0, _nbytes(P), _nbytes(Ap))
    m = ROUND_NEAREST if mode == "nearest" else ROUND_STOCHASTIC if mode == "stochastic" else -1
    _check(lib().logra_merge_grouped_explicit(r, descs, n, scale, _ptr(scale_dev), m, sr_seed,
                                              _stream(items[0][1], stream)))


def sketch_accumulate_table_ws_bytes(n: int) -> int:
    return lib().logra_sketch_accumulate_table_ws_bytes(n)


def sketch_accumulate_table(items, r: int, ws=None, stream=None):
    """items: sequence of (D bf16 [T x d], packed planes, S) sharing T and r; one persistent launch."""
    n = len(items)
    T = items[0][0].shape[0]
    descs = (AccPackedDesc * n)()
    for i, (D, P, S) in enumerate(items):
        if D.shape[0] != T:
            raise ValueError("every D must have the same number of tokens")
        _need_dtype("D", D, torch.bfloat16)
        _need_sketch("S", S, D.shape[1], r)
        descs[i] = AccPackedDesc(D.data_ptr(), P.data_ptr(), S.data_ptr(), D.shape[1], _ld(D), _nbytes(P))
    if ws is None:
        ws = _scratch(sketch_accumulate_table_ws_bytes(n), items[0][0].device, stream)
    _check(lib().logra_sketch_accumulate_table(T, r, descs, n, _ptr(ws), ws.numel(),
                                               _stream(items[0][0], stream)))


PROBE_READ, PROBE_COPY = 0, 1


def bandwidth_probe(mode: str, src: torch.Tensor, dst: torch.Tensor, blocks_per_cu: int = 4, stream=None):
    """Stream src ("read"; dst takes 4 KiB of fold values) or copy it into dst ("copy"): the
    measurement helper, not a step of the method."""
    m = PROBE_READ if mode == "read" else PROBE_COPY if mode == "copy" else -1
    nbytes = _nbytes(src)
    if mode == "read" and _nbytes(dst) < 4096:
        raise ValueError("the read probe writes 4 KiB to dst")
    if mode == "copy" and _nbytes(dst) < nbytes:
        raise ValueError("dst is smaller than src")
    _check(lib().logra_bandwidth_probe(m, _ptr(src), _ptr(dst), nbytes, blocks_per_cu, _stream(src, stream)))
