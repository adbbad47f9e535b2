"""ctypes binding of libgptq2d.so (argument marshalling only).

Every step of the computation runs in the library's HIP kernels; torch provides the
device memory (outputs, workspace, info flags) and the current stream.  The names
follow the C ABI in include/gptq2d.h.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; GPTQ2D_LIB names another build of the same library (a debug or
# sanitizer build, say)
LIB_PATH = os.environ.get("GPTQ2D_LIB") or os.path.join(_PKG, "libgptq2d.so")
F32, F64 = 0, 1
_lib = None

_SYMBOLS = {
    "gptq2d_factor": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                     ctypes.c_void_p, ctypes.c_void_p]),
    "gptq2d_factor_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int]),
    "gptq2d_quantize_factored": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                                ctypes.c_int] + [ctypes.c_void_p] * 6 +
                                 [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                  ctypes.c_void_p]),
    "gptq2d_sweep_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64,
                                                       ctypes.c_int]),
    "gptq2d_quantize": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                       ctypes.c_int] + [ctypes.c_void_p] * 6 +
                        [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]),
    "gptq2d_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int]),
    "gptq2d_quantize_noalloc": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                               ctypes.c_int] + [ctypes.c_void_p] * 6 +
                                [ctypes.c_void_p, ctypes.c_void_p]),
    "gptq2d_quantize3": (ctypes.c_int, [ctypes.c_int64] * 3 + [ctypes.c_int, ctypes.c_int] +
                         [ctypes.c_void_p] * 7 + [ctypes.c_void_p, ctypes.c_size_t,
                                                  ctypes.c_void_p, ctypes.c_void_p]),
    "gptq2d_workspace3_bytes": (ctypes.c_size_t, [ctypes.c_int64] * 3 + [ctypes.c_int]),
    "gptq2d_gram_accumulate": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                              ctypes.c_void_p, ctypes.c_double, ctypes.c_void_p,
                                              ctypes.c_void_p]),
    "gptq2d_gram_accumulate_batched": (ctypes.c_int, [ctypes.c_int, ctypes.c_void_p,
                                                      ctypes.c_void_p, ctypes.c_int,
                                                      ctypes.c_void_p, ctypes.c_void_p,
                                                      ctypes.c_void_p, ctypes.c_void_p]),
    "gptq2d_packed_row_words": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int]),
    "gptq2d_pack": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_void_p]),
    "gptq2d_unpack": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int] +
                      [ctypes.c_void_p] * 4),
    "gptq2d_packed_gemv": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p]),
    "gptq2d_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "gptq2d_profile_enable": (ctypes.c_int, [ctypes.c_int]),
    "gptq2d_profile_read": (ctypes.c_int, [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p]),
    "gptq2d_profile_class_name": (ctypes.c_char_p, [ctypes.c_int]),
    "gptq2d_profile_task_classes": (ctypes.c_int, [ctypes.c_int, ctypes.c_void_p,
                                                   ctypes.c_void_p, ctypes.c_void_p]),
}


class GPTQ2DError(RuntimeError):
    pass


def load_library(path: str = LIB_PATH):
    """Load libgptq2d.so; raise if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m "
                          "two_sided_adaptive_amd.build` (there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SYMBOLS.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.float64:
        return F64
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or float64)")


def _check_dev(name: str, t: torch.Tensor, dtype, shape) -> None:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _raise_rc(rc: int, fn: str) -> None:
    if rc != 0:
        msg = load_library().gptq2d_strerror(rc).decode()
        raise GPTQ2DError(f"{fn} returned {rc}: {msg}")


_INFO_MSG = {1: "A is not positive definite (pivot {})", 2: "B is not positive definite (pivot {})",
             3: "scale of row {} is not positive and finite",
             4: "a dependency wait inside a persistent kernel timed out (outputs undefined)",
             5: "A1 is not positive definite (pivot {})", 6: "A2 is not positive definite (pivot {})",
             7: "A3 is not positive definite (pivot {})"}


def _check_info(info: torch.Tensor) -> None:
    v = info.cpu().tolist()
    if v[0] != 0:
        raise GPTQ2DError(_INFO_MSG.get(v[0], "numerical failure {}").format(v[1]))


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def workspace_bytes(m: int, n: int, dtype: torch.dtype) -> int:
    return load_library().gptq2d_workspace_bytes(m, n, F32 if dtype == torch.float32 else F64)


def factor(A: torch.Tensor, check: bool = True) -> torch.Tensor:
    """U' (unit upper) with A^-1 = U^T U, computed on the device (gptq2d_factor)."""
    lib = load_library()
    p = A.shape[0]
    dt = _dt(A)
    _check_dev("A", A, A.dtype, (p, p))
    U = torch.empty_like(A)
    ws = torch.empty(lib.gptq2d_factor_workspace_bytes(p, dt), dtype=torch.uint8, device=A.device)
    info = torch.zeros(2, dtype=torch.int32, device=A.device)
    rc = lib.gptq2d_factor(p, dt, A.data_ptr(), U.data_ptr(), ws.data_ptr(), ws.numel(),
                           info.data_ptr(), _stream(A.device))
    _raise_rc(rc, "gptq2d_factor")
    if check:
        _check_info(info)
    return U


def quantize_factored(W: torch.Tensor, Ua: torch.Tensor, Ub: torch.Tensor, bits: int,
                      scales: torch.Tensor, check: bool = True,
                      workspace: Optional[torch.Tensor] = None,
                      out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None):
    """Sweep only, given both unit factors (gptq2d_quantize_factored) -> (codes, Q)."""
    lib = load_library()
    m, n = W.shape
    dt = _dt(W)
    _check_dev("W", W, W.dtype, (m, n))
    _check_dev("Ua", Ua, W.dtype, (m, m))
    _check_dev("Ub", Ub, W.dtype, (n, n))
    _check_dev("scales", scales, W.dtype, (m,))
    codes, Q = out if out is not None else (
        torch.empty((m, n), dtype=torch.int8, device=W.device), torch.empty_like(W))
    need = lib.gptq2d_sweep_workspace_bytes(m, n, dt)
    ws = workspace if workspace is not None else torch.empty(need, dtype=torch.uint8,
                                                             device=W.device)
    info = torch.zeros(2, dtype=torch.int32, device=W.device)
    rc = lib.gptq2d_quantize_factored(m, n, int(bits), dt, W.data_ptr(), Ua.data_ptr(),
                                      Ub.data_ptr(), scales.data_ptr(), codes.data_ptr(),
                                      Q.data_ptr(), ws.data_ptr(), ws.numel(), info.data_ptr(),
                                      _stream(W.device))
    _raise_rc(rc, "gptq2d_quantize_factored")
    if check:
        _check_info(info)
    return codes, Q


def quantize(W: torch.Tensor, A: torch.Tensor, B: torch.Tensor, bits: int, scales: torch.Tensor,
             check: bool = True, workspace: Optional[torch.Tensor] = None,
             out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None):
    """Whole call: factor A and B, then sweep (gptq2d_quantize) -> (codes int8, Q)."""
    lib = load_library()
    m, n = W.shape
    dt = _dt(W)
    _check_dev("W", W, W.dtype, (m, n))
    _check_dev("A", A, W.dtype, (m, m))
    _check_dev("B", B, W.dtype, (n, n))
    _check_dev("scales", scales, W.dtype, (m,))
    codes, Q = out if out is not None else (
        torch.empty((m, n), dtype=torch.int8, device=W.device), torch.empty_like(W))
    need = lib.gptq2d_workspace_bytes(m, n, dt)
    ws = workspace if workspace is not None else torch.empty(need, dtype=torch.uint8,
                                                             device=W.device)
    info = torch.zeros(2, dtype=torch.int32, device=W.device)
    rc = lib.gptq2d_quantize(m, n, int(bits), dt, W.data_ptr(), A.data_ptr(), B.data_ptr(),
                             scales.data_ptr(), codes.data_ptr(), Q.data_ptr(), ws.data_ptr(),
                             ws.numel(), info.data_ptr(), _stream(W.device))
    _raise_rc(rc, "gptq2d_quantize")
    if check:
        _check_info(info)
    return codes, Q


def quantize_noalloc(W: torch.Tensor, A: torch.Tensor, B: torch.Tensor, bits: int,
                     scales: torch.Tensor, out: Tuple[torch.Tensor, torch.Tensor],
                     info: Optional[torch.Tensor] = None) -> None:
    """gptq2d_quantize_noalloc: the whole call into caller-provided (codes, Q), with the
    library's static scratch buffer instead of a workspace.  Allocates nothing: `info`
    (device int32[2]) is optional and is not read back here."""
    lib = load_library()
    m, n = W.shape
    dt = _dt(W)
    _check_dev("W", W, W.dtype, (m, n))
    _check_dev("A", A, W.dtype, (m, m))
    _check_dev("B", B, W.dtype, (n, n))
    _check_dev("scales", scales, W.dtype, (m,))
    codes, Q = out
    _check_dev("codes", codes, torch.int8, (m, n))
    _check_dev("Q", Q, W.dtype, (m, n))
    rc = lib.gptq2d_quantize_noalloc(m, n, int(bits), dt, W.data_ptr(), A.data_ptr(),
                                     B.data_ptr(), scales.data_ptr(), codes.data_ptr(),
                                     Q.data_ptr(), info.data_ptr() if info is not None else None,
                                     _stream(W.device))
    _raise_rc(rc, "gptq2d_quantize_noalloc")


def quantize3(W: torch.Tensor, A1: torch.Tensor, A2: torch.Tensor, A3: torch.Tensor, bits: int,
              scales: torch.Tensor, check: bool = True, workspace: Optional[torch.Tensor] = None,
              out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None):
    """Three Kronecker factors (gptq2d_quantize3): W (m1, m2, m3), scales (m1, m2)."""
    lib = load_library()
    m1, m2, m3 = W.shape
    dt = _dt(W)
    _check_dev("W", W, W.dtype, (m1, m2, m3))
    _check_dev("A1", A1, W.dtype, (m1, m1))
    _check_dev("A2", A2, W.dtype, (m2, m2))
    _check_dev("A3", A3, W.dtype, (m3, m3))
    _check_dev("scales", scales, W.dtype, (m1, m2))
    codes, Q = out if out is not None else (
        torch.empty((m1, m2, m3), dtype=torch.int8, device=W.device), torch.empty_like(W))
    need = lib.gptq2d_workspace3_bytes(m1, m2, m3, dt)
    ws = workspace if workspace is not None else torch.empty(need, dtype=torch.uint8,
                                                             device=W.device)
    info = torch.zeros(2, dtype=torch.int32, device=W.device)
    rc = lib.gptq2d_quantize3(m1, m2, m3, int(bits), dt, W.data_ptr(), A1.data_ptr(),
                              A2.data_ptr(), A3.data_ptr(), scales.data_ptr(), codes.data_ptr(),
                              Q.data_ptr(), ws.data_ptr(), ws.numel(), info.data_ptr(),
                              _stream(W.device))
    _raise_rc(rc, "gptq2d_quantize3")
    if check:
        _check_info(info)
    return codes, Q


def pack(codes: torch.Tensor, bits: int) -> torch.Tensor:
    """int8 codes (rows, n) -> packed rows (rows, ceil(n*bits/32)) as int32 words
    (gptq2d_pack; the words are uint32 bit patterns)."""
    lib = load_library()
    rows, n = codes.shape
    _check_dev("codes", codes, torch.int8, (rows, n))
    P = torch.empty((rows, lib.gptq2d_packed_row_words(n, int(bits))), dtype=torch.int32,
                    device=codes.device)
    _raise_rc(lib.gptq2d_pack(rows, n, int(bits), codes.data_ptr(), P.data_ptr(),
                              _stream(codes.device)), "gptq2d_pack")
    return P


def unpack(P: torch.Tensor, n: int, bits: int, scales: torch.Tensor) -> torch.Tensor:
    """Q = diag(s) Z from packed rows (gptq2d_unpack), in the dtype of scales."""
    lib = load_library()
    rows = P.shape[0]
    _check_dev("packed", P, torch.int32, (rows, lib.gptq2d_packed_row_words(n, int(bits))))
    _check_dev("scales", scales, scales.dtype, (rows,))
    Q = torch.empty((rows, n), dtype=scales.dtype, device=P.device)
    _raise_rc(lib.gptq2d_unpack(rows, n, int(bits), _dt(scales), P.data_ptr(), scales.data_ptr(),
                                Q.data_ptr(), _stream(P.device)), "gptq2d_unpack")
    return Q


def packed_gemv(P: torch.Tensor, n: int, bits: int, scales: torch.Tensor, X: torch.Tensor,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = X Q^T for X (batch <= 8, n) with Q = diag(s) Z held packed (gptq2d_packed_gemv)."""
    lib = load_library()
    rows = P.shape[0]
    batch = X.shape[0]
    _check_dev("packed", P, torch.int32, (rows, lib.gptq2d_packed_row_words(n, int(bits))))
    _check_dev("scales", scales, scales.dtype, (rows,))
    _check_dev("X", X, scales.dtype, (batch, n))
    Y = out if out is not None else torch.empty((batch, rows), dtype=scales.dtype,
                                                device=P.device)
    _raise_rc(lib.gptq2d_packed_gemv(rows, n, int(bits), _dt(scales), P.data_ptr(),
                                     scales.data_ptr(), batch, X.data_ptr(), Y.data_ptr(),
                                     _stream(P.device)), "gptq2d_packed_gemv")
    return Y


def gram_accumulate(A: torch.Tensor, X: torch.Tensor, alpha: float = 1.0) -> torch.Tensor:
    """A += alpha X^T X in place (gptq2d_gram_accumulate); X (N, p), A (p, p) symmetric."""
    lib = load_library()
    N, p = X.shape
    _check_dev("X", X, X.dtype, (N, p))
    _check_dev("A", A, X.dtype, (p, p))
    _raise_rc(lib.gptq2d_gram_accumulate(p, N, _dt(X), X.data_ptr(), float(alpha), A.data_ptr(),
                                         _stream(X.device)), "gptq2d_gram_accumulate")
    return A


def gram_accumulate_batched(As, Xs, alphas) -> None:
    """Several layers in one call (gptq2d_gram_accumulate_batched), each A += alpha X^T X."""
    import numpy as np
    lib = load_library()
    cnt = len(As)
    if not (len(Xs) == len(alphas) == cnt) or cnt == 0:
        raise ValueError("As, Xs and alphas must have the same non-zero length")
    dt = _dt(Xs[0])
    for A, X in zip(As, Xs):
        _check_dev("X", X, Xs[0].dtype, tuple(X.shape))
        _check_dev("A", A, Xs[0].dtype, (X.shape[1], X.shape[1]))
    p = np.array([X.shape[1] for X in Xs], dtype=np.int64)
    n = np.array([X.shape[0] for X in Xs], dtype=np.int64)
    xp = (ctypes.c_void_p * cnt)(*[X.data_ptr() for X in Xs])
    ap = (ctypes.c_void_p * cnt)(*[A.data_ptr() for A in As])
    al = np.array(alphas, dtype=np.float64)
    _raise_rc(lib.gptq2d_gram_accumulate_batched(cnt, p.ctypes.data, n.ctypes.data, dt, xp,
                                                 al.ctypes.data, ap, _stream(Xs[0].device)),
              "gptq2d_gram_accumulate_batched")


def profile_enable(on: bool = True) -> None:
    """Turn the library's per-kernel event timing on or off (gptq2d_profile_enable)."""
    load_library().gptq2d_profile_enable(1 if on else 0)


def profile_read() -> dict:
    """Per-class totals since the last read: {name: (ms, launches, flops, bytes)}."""
    import numpy as np
    lib = load_library()
    n = 8
    ms = np.zeros(n)
    la = np.zeros(n, dtype=np.int64)
    fl = np.zeros(n)
    by = np.zeros(n)
    rc = lib.gptq2d_profile_read(n, ms.ctypes.data, la.ctypes.data, fl.ctypes.data,
                                 by.ctypes.data)
    _raise_rc(rc, "gptq2d_profile_read")
    return {lib.gptq2d_profile_class_name(c).decode(): (float(ms[c]), int(la[c]), float(fl[c]),
                                                         float(by[c])) for c in range(n)}


def profile_task_classes() -> dict:
    """Band-update tasks of the last profile_read window by task class:
    {"near"|"next"|"far": (busy CU-ms, tasks, flops)}."""
    import numpy as np
    lib = load_library()
    ms = np.zeros(3)
    n = np.zeros(3, dtype=np.int64)
    fl = np.zeros(3)
    _raise_rc(lib.gptq2d_profile_task_classes(3, ms.ctypes.data, n.ctypes.data, fl.ctypes.data),
              "gptq2d_profile_task_classes")
    return {name: (float(ms[c]), int(n[c]), float(fl[c]))
            for c, name in enumerate(("near", "next", "far"))}
