"""Thin Python binding of libq8gemv.so (include/q8_gemv.h).

Argument marshalling only: every step of the computation runs in the HIP
library.  torch supplies device memory and the stream.  If the library is not
built this module raises; there is no fallback implementation.
"""

import ctypes
import os

import torch

from .build import LIB_PATH

Q8_OK = 0
Q8_ERR_INVALID = 1
Q8_ERR_TOO_LARGE = 2
Q8_ERR_UNSUPPORTED_DEVICE = 3
Q8_ERR_HIP = 4

BLOCK = 32
MAX_SIBLINGS = 4
PLAN_STREAM = 1
PLAN_MATRIX = 2

#: Every symbol include/q8_gemv.h declares.
EXPORTED = (
    "q8_matvec",
    "q8_matvec_noalloc",
    "q8_matvec_with_plan",
    "q8_matvec_choose_plan",
    "q8_matvec_fused",
    "q8_dot_t",
    "q8_dot_f32",
    "q8_dot_t_f32",
    "q8_status_string",
    "q8_last_hip_error",
    "q8_release",
)


class Q8Plan(ctypes.Structure):
    _fields_ = [("vec", ctypes.c_int32), ("m_tile", ctypes.c_int32),
                ("workgroups", ctypes.c_int32), ("waves", ctypes.c_int32), ("kind", ctypes.c_int32)]

    def as_dict(self):
        return {"vec": self.vec, "m_tile": self.m_tile, "workgroups": self.workgroups, "waves": self.waves,
                "kind": self.kind}


class Q8Sibling(ctypes.Structure):
    _fields_ = [("W", ctypes.c_void_p), ("S", ctypes.c_void_p), ("C", ctypes.c_void_p)]


class Q8Epilogue(ctypes.Structure):
    _fields_ = [("alpha", ctypes.c_float), ("corr", ctypes.c_void_p)]


class Q8Error(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        msg = f"{what}: {q8_status_string(status)}"
        if status == Q8_ERR_HIP:
            msg += f" (hipError {q8_last_hip_error()})"
        super().__init__(msg)


_lib = None


def load():
    """The loaded library (ctypes.CDLL), loading it on first use."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m quantized_decode_gemv_q8_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    L.q8_matvec.argtypes = [p, p, p, p, i64, i64, i64, p]
    L.q8_matvec.restype = ctypes.c_int
    L.q8_matvec_noalloc.argtypes = [p, p, p, p, i64, i64, i64, p]
    L.q8_matvec_noalloc.restype = ctypes.c_int
    L.q8_matvec_with_plan.argtypes = [p, p, p, p, i64, i64, i64, ctypes.POINTER(Q8Plan), p]
    L.q8_matvec_with_plan.restype = ctypes.c_int
    L.q8_matvec_choose_plan.argtypes = [i64, i64, i64, i64, i64, i32, ctypes.POINTER(Q8Plan)]
    L.q8_matvec_choose_plan.restype = ctypes.c_int
    L.q8_matvec_fused.argtypes = [p, ctypes.POINTER(Q8Sibling), i32, i64, i64, i64,
                                  ctypes.POINTER(Q8Epilogue), ctypes.POINTER(Q8Plan), p]
    L.q8_matvec_fused.restype = ctypes.c_int
    L.q8_dot_t.argtypes = [p, p, p, i64, i64, i64, p]
    L.q8_dot_t.restype = ctypes.c_int
    for name in ("q8_dot_f32", "q8_dot_t_f32"):
        fn = getattr(L, name)
        fn.argtypes = [p, p, p, i64, i64, i64, ctypes.POINTER(Q8Epilogue), p]
        fn.restype = ctypes.c_int
    L.q8_status_string.argtypes = [ctypes.c_int]
    L.q8_status_string.restype = ctypes.c_char_p
    L.q8_last_hip_error.argtypes = []
    L.q8_last_hip_error.restype = ctypes.c_int
    L.q8_release.argtypes = []
    L.q8_release.restype = None
    _lib = L
    return L


def q8_status_string(status):
    return load().q8_status_string(int(status)).decode()


def q8_last_hip_error():
    return load().q8_last_hip_error()


def q8_release():
    load().q8_release()


def _stream_handle(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _check_tensor(name, t, dtype, shape):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (dense row-major)")


def _check_disjoint(out_name, out, others):
    """The library requires outputs that share no bytes with any other
    argument; an overlap would be a silent race, so it is refused here."""
    if out.numel() == 0:
        return
    a0 = out.data_ptr()
    a1 = a0 + out.numel() * out.element_size()
    for name, t in others:
        if t is None or t.numel() == 0:
            continue
        b0 = t.data_ptr()
        b1 = b0 + t.numel() * t.element_size()
        if a0 < b1 and b0 < a1:
            raise ValueError(f"{out_name} overlaps {name}")


def _rank2(**named):
    for name, t in named.items():
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dim() != 2:
            raise ValueError(f"{name} must be rank 2, got {t.dim()} dimensions")


def _q8_args(A, W, S, out):
    _rank2(A=A, W=W)
    M, K = A.shape
    N = W.shape[1]
    KB = (K + BLOCK - 1) // BLOCK
    _check_tensor("A", A, torch.float32, (M, K))
    _check_tensor("W", W, torch.int8, (K, N))
    _check_tensor("S", S, torch.float32, (KB, N))
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    _check_tensor("out", out, torch.float32, (M, N))
    for t in (W, S, out):
        if t.device != A.device:
            raise ValueError("all tensors must be on one device")
    _check_disjoint("out", out, (("A", A), ("W", W), ("S", S)))
    return M, K, N, out


def q8_matvec(A, W, S, out=None, stream=None):
    """C[m,n] = sum_k A[m,k] W[k,n] S[k//32,n] on the GPU; returns C (f32 [M,N])."""
    M, K, N, out = _q8_args(A, W, S, out)
    with torch.cuda.device(A.device):
        st = load().q8_matvec(A.data_ptr(), W.data_ptr(), S.data_ptr(), out.data_ptr(),
                              M, K, N, _stream_handle(stream, A.device))
    if st != Q8_OK:
        raise Q8Error(st, "q8_matvec")
    return out


def q8_matvec_noalloc(A, W, S, out=None, stream=None):
    """q8_matvec through the library's fixed scratch array instead of its
    workspace: the call allocates nothing on the device (out must be given to
    avoid torch's allocation).  Calls that overlap in time on one device race."""
    M, K, N, out = _q8_args(A, W, S, out)
    with torch.cuda.device(A.device):
        st = load().q8_matvec_noalloc(A.data_ptr(), W.data_ptr(), S.data_ptr(), out.data_ptr(),
                                      M, K, N, _stream_handle(stream, A.device))
    if st != Q8_OK:
        raise Q8Error(st, "q8_matvec_noalloc")
    return out


def q8_matvec_with_plan(A, W, S, plan, out=None, stream=None):
    """q8_matvec with an explicit launch plan (dict with vec, m_tile, workgroups, waves, kind)."""
    M, K, N, out = _q8_args(A, W, S, out)
    pl = _plan_struct(plan)
    with torch.cuda.device(A.device):
        st = load().q8_matvec_with_plan(A.data_ptr(), W.data_ptr(), S.data_ptr(), out.data_ptr(),
                                        M, K, N, ctypes.byref(pl), _stream_handle(stream, A.device))
    if st != Q8_OK:
        raise Q8Error(st, "q8_matvec_with_plan")
    return out


def _plan_struct(plan):
    return Q8Plan(int(plan.get("vec", 0)), int(plan.get("m_tile", 0)),
                  int(plan.get("workgroups", 0)), int(plan.get("waves", 0)), int(plan.get("kind", 0)))


def q8_matvec_fused(A, Ws, Ss, outs=None, alpha=1.0, corr=None, plan=None, stream=None):
    """Sibling projections sharing A, in one launch, through the epilogue
    C_g = alpha * (A x dequant(W_g, S_g)) + corr[m] * C_g (corr: f32 [M] or
    None).  With corr the existing contents of outs are read.  Returns the
    list of C_g (f32 [M,N])."""
    if not isinstance(Ws, (list, tuple)) or not isinstance(Ss, (list, tuple)) or len(Ws) != len(Ss):
        raise ValueError("Ws and Ss must be lists of equal length")
    n = len(Ws)
    if not 1 <= n <= MAX_SIBLINGS:
        raise ValueError(f"1..{MAX_SIBLINGS} siblings, got {n}")
    if outs is None:
        if corr is not None:
            raise ValueError("corr reads the existing outputs: pass outs")
        outs = [None] * n
    if len(outs) != n:
        raise ValueError("outs must have one entry per sibling")
    res = []
    M = K = N = None
    for W, S, out in zip(Ws, Ss, outs):
        M, K, N, out = _q8_args(A, W, S, out)
        res.append(out)
    if corr is not None:
        _check_tensor("corr", corr, torch.float32, (M,))
        if corr.device != A.device:
            raise ValueError("all tensors must be on one device")
    inputs = [("corr", corr)] + [(f"Ws[{j}]", W) for j, W in enumerate(Ws)] + \
        [(f"Ss[{j}]", S) for j, S in enumerate(Ss)]
    for g, C in enumerate(res):
        _check_disjoint(f"outs[{g}]", C, inputs + [(f"outs[{j}]", res[j]) for j in range(g)])
    sib = (Q8Sibling * n)(*[Q8Sibling(W.data_ptr(), S.data_ptr(), C.data_ptr()) for W, S, C in zip(Ws, Ss, res)])
    ep = Q8Epilogue(float(alpha), corr.data_ptr() if corr is not None else None)
    pl = ctypes.byref(_plan_struct(plan)) if plan is not None else None
    with torch.cuda.device(A.device):
        st = load().q8_matvec_fused(A.data_ptr(), sib, n, M, K, N, ctypes.byref(ep), pl,
                                    _stream_handle(stream, A.device))
    if st != Q8_OK:
        raise Q8Error(st, "q8_matvec_fused")
    return res


def q8_matvec_choose_plan(M, K, N, w_align=256, s_align=256, num_cus=256):
    """The plan q8_matvec would pick (host logic only; touches no device)."""
    pl = Q8Plan()
    st = load().q8_matvec_choose_plan(int(M), int(K), int(N), int(w_align), int(s_align),
                                      int(num_cus), ctypes.byref(pl))
    if st != Q8_OK:
        raise Q8Error(st, "q8_matvec_choose_plan")
    return pl.as_dict()


def q8_dot_t(A, W, out=None, stream=None):
    """C[m,n] = sum_k A[m,k] W[n,k] in exact i32 on the GPU; returns C (i32 [M,N])."""
    _rank2(A=A, W=W)
    M, K = A.shape
    N = W.shape[0]
    _check_tensor("A", A, torch.int8, (M, K))
    _check_tensor("W", W, torch.int8, (N, K))
    if out is None:
        out = torch.empty((M, N), dtype=torch.int32, device=A.device)
    _check_tensor("out", out, torch.int32, (M, N))
    if W.device != A.device or out.device != A.device:
        raise ValueError("all tensors must be on one device")
    _check_disjoint("out", out, (("A", A), ("W", W)))
    with torch.cuda.device(A.device):
        st = load().q8_dot_t(A.data_ptr(), W.data_ptr(), out.data_ptr(), M, K, N,
                             _stream_handle(stream, A.device))
    if st != Q8_OK:
        raise Q8Error(st, "q8_dot_t")
    return out


def _dense(name, A, B, transposed, out, alpha, corr, stream):
    _rank2(A=A, B=B)
    M, K = A.shape
    N = B.shape[0] if transposed else B.shape[1]
    _check_tensor("A", A, torch.float32, (M, K))
    _check_tensor("B", B, torch.float32, (N, K) if transposed else (K, N))
    if out is None:
        if corr is not None:
            raise ValueError("corr reads the existing output: pass out")
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    _check_tensor("out", out, torch.float32, (M, N))
    if corr is not None:
        _check_tensor("corr", corr, torch.float32, (M,))
    for t in (B, out) + ((corr,) if corr is not None else ()):
        if t.device != A.device:
            raise ValueError("all tensors must be on one device")
    _check_disjoint("out", out, (("A", A), ("B", B), ("corr", corr)))
    ep = Q8Epilogue(float(alpha), corr.data_ptr() if corr is not None else None)
    with torch.cuda.device(A.device):
        st = getattr(load(), name)(A.data_ptr(), B.data_ptr(), out.data_ptr(), M, K, N, ctypes.byref(ep),
                                   _stream_handle(stream, A.device))
    if st != Q8_OK:
        raise Q8Error(st, name)
    return out


def q8_dot_f32(A, B, out=None, alpha=1.0, corr=None, stream=None):
    """C = alpha * (A @ B) (+ corr[m] * C) for f32 A [M,K], B [K,N]; returns C (f32 [M,N])."""
    return _dense("q8_dot_f32", A, B, False, out, alpha, corr, stream)


def q8_dot_t_f32(A, B, out=None, alpha=1.0, corr=None, stream=None):
    """C = alpha * (A @ B^T) (+ corr[m] * C) for f32 A [M,K], B [N,K]; returns C (f32 [M,N])."""
    return _dense("q8_dot_t_f32", A, B, True, out, alpha, corr, stream)
