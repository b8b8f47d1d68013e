"""MI355X (gfx950) dense GEMM library: a thin Python binding over the C ABI.

Every step of the computation runs in the HIP kernels of ``libmi355gemm.so``;
this module only marshals torch tensors (device pointers, leading dimensions,
the current HIP stream) into the C calls declared in ``include/mi355gemm.h``
and turns a nonzero status into an exception.  There is no fallback: if the
library is missing the calls raise.

    gemm_f32(A, B, C, alpha=1.0, beta=0.0)   # C = alpha*A@B + beta*C, fp32
    gemm_f16_nt(A, B, C)                     # C = A@B.T, fp16 in/out, fp32 acc
    gemm_f16_nt_ex(A, B, C, bias=None, act="none", residual=None)
                                             # C = act(A@B.T + bias) + residual
    gemm_ex(A, B, C, op_a="n", op_b="t", ...) # any layout, fp16 or bf16
    gemm_f32_splitk / gemm_f16_nt_splitk     # K cut into ranges (split-K)
    gemm_f16_nt_splitk_static(A, B, C)       # split-K into the library's static
                                             # scratch area: allocates nothing

The library allocates no memory.  Where a call's kernels need scratch memory
(split-K partial sums, gemm_ex's transposed copies and matrix-vector partial
sums) the caller may pass a ``workspace`` tensor; if it does not, this module
takes one of the size the library reports from torch's caching allocator, on
the stream the call runs on, for the duration of the call.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmi355gemm.so")

# Status and activation codes, mirroring include/mi355gemm.h.
GEMM_OK = 0
GEMM_ERR_WORKSPACE = -7
GEMM_ERR_SCRATCH_LIMIT = -8
STATIC_SCRATCH_BYTES = 32 << 20
ACTS = {"none": 0, "relu": 1, "silu": 2}

_lock = threading.Lock()
_lib = None


def _path_name(code: int) -> str:
    """The library's name for a GEMM_PATH_* code, or "error <code>" for a status."""
    if code < 0:
        return "error %d" % code
    return load_library().gemm_path_name(code).decode()


class GemmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s (status %d)" % (message, status))
        self.status = status


def library_path() -> str:
    return LIB_PATH


def load_library() -> ctypes.CDLL:
    """Load the C-ABI library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise ImportError("%s is missing: build it with `python -m dense_gemm_sgemm_amd.build` "
                              "(or __graft_entry__.build())" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        i, f, p = ctypes.c_int, ctypes.c_float, ctypes.c_void_p
        lib.gemm_f32.argtypes = [i, i, i, f, p, i, p, i, f, p, i, p]
        lib.gemm_f32.restype = i
        lib.gemm_f16_nt.argtypes = [i, i, i, p, i, p, i, p, i, p]
        lib.gemm_f16_nt.restype = i
        lib.gemm_f32_path.argtypes = [i, i, i, f, p, i, p, i, f, p, i]
        lib.gemm_f32_path.restype = i
        lib.gemm_f16_nt_path.argtypes = [i, i, i, p, i, p, i, p, i]
        lib.gemm_f16_nt_path.restype = i
        lib.gemm_f16_nt_ex.argtypes = [i, i, i, p, i, p, i, p, i, p, i, p, i, p]
        lib.gemm_f16_nt_ex.restype = i
        lib.gemm_f16_nt_ex_path.argtypes = [i, i, i, p, i, p, i, p, i, p, i, p, i]
        lib.gemm_f16_nt_ex_path.restype = i
        u64 = ctypes.c_ulonglong
        lib.gemm_f32_splitk.argtypes = [i, i, i, f, p, i, p, i, f, p, i, i, p, u64, p]
        lib.gemm_f32_splitk.restype = i
        lib.gemm_f16_nt_splitk.argtypes = [i, i, i, p, i, p, i, p, i, i, p, u64, p]
        lib.gemm_f16_nt_splitk.restype = i
        lib.gemm_f16_nt_splitk_static.argtypes = [i, i, i, p, i, p, i, p, i, i, p]
        lib.gemm_f16_nt_splitk_static.restype = i
        lib.gemm_f32_splitk_workspace.argtypes = [i, i, i, i]
        lib.gemm_f32_splitk_workspace.restype = u64
        lib.gemm_f16_nt_splitk_workspace.argtypes = [i, i, i, i]
        lib.gemm_f16_nt_splitk_workspace.restype = u64
        lib.gemm_ex.argtypes = [i, i, i, i, i, i, p, i, p, i, p, i, p, i, p, i, p, u64, p]
        lib.gemm_ex.restype = i
        lib.gemm_ex_workspace.argtypes = [i, i, i, i, i, i, i, i]
        lib.gemm_ex_workspace.restype = u64
        lib.gemm_ex_path.argtypes = [i, i, i, i, i, i, p, i, p, i, p, i, p, i, p, i]
        lib.gemm_ex_path.restype = i
        lib.gemm_status_string.argtypes = [i]
        lib.gemm_status_string.restype = ctypes.c_char_p
        lib.gemm_path_name.argtypes = [i]
        lib.gemm_path_name.restype = ctypes.c_char_p
        _lib = lib
        return lib


def status_string(status: int) -> str:
    return load_library().gemm_status_string(status).decode()


def _check(status: int) -> None:
    if status != GEMM_OK:
        raise GemmError(status, status_string(status))


_torch = None


def _torch_module():
    global _torch
    if _torch is None:
        import torch
        _torch = torch
    return _torch


def _matrix(t, name: str, dtype):
    """(rows, cols, leading dimension, device pointer or None) of a row-major
    2-D GPU tensor; raises on anything else.  Runs on every call, so it uses
    the cheapest tensor queries."""
    torch = _torch_module()
    if not isinstance(t, torch.Tensor) or t.dim() != 2:
        raise TypeError("%s must be a 2-D torch tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_cuda:
        raise TypeError("%s must live on the GPU" % name)
    rows, cols = t.shape
    s0, s1 = t.stride()
    if cols > 1 and s1 != 1:
        raise ValueError("%s must have unit stride along its rows (row-major)" % name)
    ld = s0 if rows > 1 and cols > 0 else max(1, cols)
    return rows, cols, ld, (t.data_ptr() if rows and cols else None)


_raw_stream = None


def _current_stream_handle() -> int:
    """The HIP handle of torch's current stream on the current device.  torch's
    raw-handle query costs about 0.1 us against about 3 us for building a
    ``torch.cuda.Stream``; the public route is the fallback."""
    global _raw_stream
    torch = _torch_module()
    if _raw_stream is None:
        get_raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        get_dev = getattr(torch._C, "_cuda_getDevice", None)
        if get_raw is not None and get_dev is not None:
            _raw_stream = lambda: get_raw(get_dev())
        else:
            _raw_stream = lambda: torch.cuda.current_stream().cuda_stream
    return _raw_stream()


def _stream(stream):
    if stream is None:
        return _current_stream_handle()
    return ctypes.c_void_p(stream.cuda_stream)


def gemm_f32(A, B, C, alpha: float = 1.0, beta: float = 0.0, stream=None):
    """In place ``C = alpha * A @ B + beta * C`` for float32 A[M,K], B[K,N], C[M,N].

    Enqueued on ``stream`` (default: torch's current stream); returns C."""
    torch = _torch_module()
    M, K, lda, pa = _matrix(A, "A", torch.float32)
    K2, N, ldb, pb = _matrix(B, "B", torch.float32)
    M2, N2, ldc, pc = _matrix(C, "C", torch.float32)
    if K2 != K or M2 != M or N2 != N:
        raise ValueError("shape mismatch: A %s, B %s, C %s" % (tuple(A.shape), tuple(B.shape),
                                                               tuple(C.shape)))
    _check(load_library().gemm_f32(M, N, K, float(alpha), pa, lda, pb, ldb, float(beta), pc, ldc,
                                   _stream(stream)))
    return C


def splitk_workspace_bytes(kind: str, M: int, N: int, K: int, splits: int = 0) -> int:
    """Workspace bytes of ``gemm_f32_splitk`` (kind "f32") or ``gemm_f16_nt_splitk``
    (kind "f16") for these sizes; 0 when the call would not split."""
    lib = load_library()
    fn = {"f32": lib.gemm_f32_splitk_workspace, "f16": lib.gemm_f16_nt_splitk_workspace}[kind]
    return int(fn(int(M), int(N), int(K), int(splits)))


def _workspace(workspace, need: int, device, stream=None):
    """(pointer, bytes, tensor) of a caller's workspace tensor, or of a new one.

    A new one comes from torch's caching allocator on the stream the kernels
    will run on (``stream``, default the current one): the tensor is dropped
    when the call returns, and the allocator hands its block only to later
    allocations on that same stream, which are ordered after the kernels that
    use it."""
    torch = _torch_module()
    if workspace is None:
        if need == 0:
            return None, 0, None
        if stream is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=device)
        else:
            with torch.cuda.stream(stream):
                workspace = torch.empty(need, dtype=torch.uint8, device=device)
    if not isinstance(workspace, torch.Tensor) or workspace.device.type != "cuda" or \
            not workspace.is_contiguous():
        raise TypeError("workspace must be a contiguous GPU tensor")
    nbytes = workspace.numel() * workspace.element_size()
    return (workspace.data_ptr() if nbytes else None), nbytes, workspace


def gemm_f32_splitk(A, B, C, alpha: float = 1.0, beta: float = 0.0, splits: int = 0,
                    workspace=None, stream=None):
    """``gemm_f32`` with K cut into ``splits`` ranges (0: the library's choice) and
    the fp32 partial sums in ``workspace`` (a GPU tensor of at least
    ``splitk_workspace_bytes("f32", M, N, K, splits)`` bytes; allocated here if None)."""
    torch = _torch_module()
    M, K, lda, pa = _matrix(A, "A", torch.float32)
    K2, N, ldb, pb = _matrix(B, "B", torch.float32)
    M2, N2, ldc, pc = _matrix(C, "C", torch.float32)
    if K2 != K or M2 != M or N2 != N:
        raise ValueError("shape mismatch: A %s, B %s, C %s" % (tuple(A.shape), tuple(B.shape),
                                                               tuple(C.shape)))
    pw, nw, _ws = _workspace(workspace, splitk_workspace_bytes("f32", M, N, K, splits), C.device,
                             stream)
    _check(load_library().gemm_f32_splitk(M, N, K, float(alpha), pa, lda, pb, ldb, float(beta),
                                          pc, ldc, int(splits), pw, nw, _stream(stream)))
    return C


def gemm_f16_nt_splitk(A, B, C, splits: int = 0, workspace=None, stream=None):
    """``gemm_f16_nt`` with K cut into ``splits`` ranges (0: the library's choice)
    and the fp32 partial sums in ``workspace`` (a GPU tensor of at least
    ``splitk_workspace_bytes("f16", M, N, K, splits)`` bytes; allocated here if None)."""
    torch = _torch_module()
    M, K, lda, pa = _matrix(A, "A", torch.float16)
    N, K2, ldb, pb = _matrix(B, "B", torch.float16)
    M2, N2, ldc, pc = _matrix(C, "C", torch.float16)
    if K2 != K or M2 != M or N2 != N:
        raise ValueError("shape mismatch: A %s, B %s, C %s" % (tuple(A.shape), tuple(B.shape),
                                                               tuple(C.shape)))
    pw, nw, _ws = _workspace(workspace, splitk_workspace_bytes("f16", M, N, K, splits), C.device,
                             stream)
    _check(load_library().gemm_f16_nt_splitk(M, N, K, pa, lda, pb, ldb, pc, ldc, int(splits), pw,
                                             nw, _stream(stream)))
    return C


def gemm_f16_nt_splitk_static(A, B, C, splits: int = 0, stream=None):
    """``gemm_f16_nt_splitk`` without a workspace: the partial sums go to the
    library's static scratch area (``STATIC_SCRATCH_BYTES`` per GPU), so the
    call allocates nothing.  Calls that overlap in time on one GPU race on
    that area; order them (e.g. on one stream).  Returns C."""
    torch = _torch_module()
    M, K, lda, pa = _matrix(A, "A", torch.float16)
    N, K2, ldb, pb = _matrix(B, "B", torch.float16)
    M2, N2, ldc, pc = _matrix(C, "C", torch.float16)
    if K2 != K or M2 != M or N2 != N:
        raise ValueError("shape mismatch: A %s, B %s, C %s" % (tuple(A.shape), tuple(B.shape),
                                                               tuple(C.shape)))
    _check(load_library().gemm_f16_nt_splitk_static(M, N, K, pa, lda, pb, ldb, pc, ldc,
                                                    int(splits), _stream(stream)))
    return C


def gemm_f16_nt(A, B, C, stream=None):
    """``C = A @ B.T`` for float16 A[M,K], B[N,K]; fp32 accumulation, result in C[M,N].

    Enqueued on ``stream`` (default: torch's current stream); returns C."""
    torch = _torch_module()
    M, K, lda, pa = _matrix(A, "A", torch.float16)
    N, K2, ldb, pb = _matrix(B, "B", torch.float16)
    M2, N2, ldc, pc = _matrix(C, "C", torch.float16)
    if K2 != K or M2 != M or N2 != N:
        raise ValueError("shape mismatch: A %s, B %s, C %s" % (tuple(A.shape), tuple(B.shape),
                                                               tuple(C.shape)))
    _check(load_library().gemm_f16_nt(M, N, K, pa, lda, pb, ldb, pc, ldc, _stream(stream)))
    return C


def f32_path(A, B, C, alpha: float = 1.0, beta: float = 0.0) -> str:
    """Name of the kernel ``gemm_f32`` would launch for these tensors (host only)."""
    torch = _torch_module()
    M, K, lda, pa = _matrix(A, "A", torch.float32)
    _, N, ldb, pb = _matrix(B, "B", torch.float32)
    _, _, ldc, pc = _matrix(C, "C", torch.float32)
    code = load_library().gemm_f32_path(M, N, K, float(alpha), pa, lda, pb, ldb, float(beta), pc,
                                        ldc)
    return _path_name(code)


def f16_nt_path(A, B, C) -> str:
    """Name of the kernel ``gemm_f16_nt`` would launch for these tensors (host only)."""
    torch = _torch_module()
    M, K, lda, pa = _matrix(A, "A", torch.float16)
    N, _, ldb, pb = _matrix(B, "B", torch.float16)
    _, _, ldc, pc = _matrix(C, "C", torch.float16)
    code = load_library().gemm_f16_nt_path(M, N, K, pa, lda, pb, ldb, pc, ldc)
    return _path_name(code)


def _epilogue_args(bias, act, residual, M: int, N: int, dtype=None):
    torch = _torch_module()
    dtype = dtype or torch.float16
    if act not in ACTS:
        raise ValueError("act must be one of %s" % sorted(ACTS))
    pbias = None
    if bias is not None:
        if not isinstance(bias, torch.Tensor) or bias.dtype != dtype or \
                bias.device.type != "cuda" or bias.numel() != N or \
                (bias.dim() == 1 and N > 1 and bias.stride(0) != 1):
            raise ValueError("bias must be a contiguous %s GPU vector of length N = %d"
                             % (dtype, N))
        pbias = bias.data_ptr()
    pres, ldr = None, 0
    if residual is not None:
        Mr, Nr, ldr, pres = _matrix(residual, "residual", dtype)
        if (Mr, Nr) != (M, N):
            raise ValueError("residual must be %d x %d, got %s" % (M, N, tuple(residual.shape)))
    return pbias, ACTS[act], pres, ldr


def gemm_f16_nt_ex(A, B, C, bias=None, act: str = "none", residual=None, stream=None):
    """Fused ``C = act(A @ B.T + bias) + residual`` for float16 A[M,K], B[N,K];
    ``bias`` a float16 vector of length N or None, ``act`` "none", "relu" or
    "silu", ``residual`` a float16 [M,N] tensor or None (it may be C itself).
    fp32 accumulation and epilogue, one rounding to half.  Returns C."""
    torch = _torch_module()
    M, K, lda, pa = _matrix(A, "A", torch.float16)
    N, K2, ldb, pb = _matrix(B, "B", torch.float16)
    M2, N2, ldc, pc = _matrix(C, "C", torch.float16)
    if K2 != K or M2 != M or N2 != N:
        raise ValueError("shape mismatch: A %s, B %s, C %s" % (tuple(A.shape), tuple(B.shape),
                                                               tuple(C.shape)))
    pbias, code, pres, ldr = _epilogue_args(bias, act, residual, M, N)
    _check(load_library().gemm_f16_nt_ex(M, N, K, pa, lda, pb, ldb, pbias, code, pres, ldr, pc,
                                         ldc, _stream(stream)))
    return C


def f16_nt_ex_path(A, B, C, bias=None, act: str = "none", residual=None) -> str:
    """Name of the kernel ``gemm_f16_nt_ex`` would launch for these tensors (host only)."""
    torch = _torch_module()
    M, K, lda, pa = _matrix(A, "A", torch.float16)
    N, _, ldb, pb = _matrix(B, "B", torch.float16)
    _, _, ldc, pc = _matrix(C, "C", torch.float16)
    pbias, code, pres, ldr = _epilogue_args(bias, act, residual, M, N)
    code = load_library().gemm_f16_nt_ex_path(M, N, K, pa, lda, pb, ldb, pbias, code, pres, ldr,
                                              pc, ldc)
    return _path_name(code)


OPS = {"n": 0, "t": 1}


def _ex_args(A, B, C, op_a, op_b, bias, act, residual):
    torch = _torch_module()
    if op_a not in OPS or op_b not in OPS:
        raise ValueError("op_a and op_b must be 'n' or 't'")
    dtype = A.dtype if isinstance(A, torch.Tensor) else None
    if dtype not in (torch.float16, torch.bfloat16):
        raise TypeError("A must be a float16 or bfloat16 tensor")
    ra, ca, lda, pa = _matrix(A, "A", dtype)
    rb, cb, ldb, pb = _matrix(B, "B", dtype)
    M, N, ldc, pc = _matrix(C, "C", dtype)
    M2, K = (ra, ca) if op_a == "n" else (ca, ra)
    K2, N2 = (rb, cb) if op_b == "n" else (cb, rb)
    if M2 != M or N2 != N or K2 != K:
        raise ValueError("shape mismatch: op_a %s A %s, op_b %s B %s, C %s"
                         % (op_a, tuple(A.shape), op_b, tuple(B.shape), tuple(C.shape)))
    pbias, code, pres, ldr = _epilogue_args(bias, act, residual, M, N, dtype)
    typ = 1 if dtype == torch.bfloat16 else 0
    return (typ, OPS[op_a], OPS[op_b], M, N, K, pa, lda, pb, ldb, pbias, code, pres, ldr, pc, ldc)


def ex_workspace_bytes(A, B, C, op_a: str = "n", op_b: str = "t") -> int:
    """Workspace bytes ``gemm_ex`` uses for these tensors (0 when none)."""
    a = _ex_args(A, B, C, op_a, op_b, None, "none", None)
    return int(load_library().gemm_ex_workspace(a[0], a[1], a[2], a[3], a[4], a[5], a[7], a[9]))


def gemm_ex(A, B, C, op_a: str = "n", op_b: str = "t", bias=None, act: str = "none",
            residual=None, workspace=None, stream=None):
    """``C = act(op(A) @ op(B) + bias) + residual`` for float16 or bfloat16
    tensors (all of one dtype).  op "n": A is [M,K], B is [K,N]; op "t": A is
    [K,M], B is [N,K].  fp32 accumulation, one rounding to the dtype.
    ``workspace``: a contiguous GPU tensor of at least ``ex_workspace_bytes``
    bytes, or None (one is taken from torch's allocator only when the call
    needs one: the library checks the workspace before it enqueues any work,
    so a call that reads its operands in place runs without).  Returns C."""
    args = _ex_args(A, B, C, op_a, op_b, bias, act, residual)
    lib = load_library()
    if workspace is None:
        # split-K runs only with its workspace; other calls try without first
        if _path_name(lib.gemm_ex_path(*args)) != "f16_splitk":
            status = lib.gemm_ex(*args, None, 0, _stream(stream))
            if status != GEMM_ERR_WORKSPACE:
                _check(status)
                return C
        need = int(lib.gemm_ex_workspace(args[0], args[1], args[2], args[3], args[4], args[5],
                                         args[7], args[9]))
    else:
        need = 0
    pw, nw, _ws = _workspace(workspace, need, C.device, stream)
    _check(lib.gemm_ex(*args, pw, nw, _stream(stream)))
    return C


def ex_path(A, B, C, op_a: str = "n", op_b: str = "t", bias=None, act: str = "none",
            residual=None) -> str:
    """Name of the kernel ``gemm_ex`` would run for these tensors with a
    workspace of ``ex_workspace_bytes`` (host only)."""
    return _path_name(load_library().gemm_ex_path(*_ex_args(A, B, C, op_a, op_b, bias, act,
                                                            residual)))
