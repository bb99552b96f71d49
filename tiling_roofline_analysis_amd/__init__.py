"""MI355X-native single-precision GEMM (C = A x B, row-major) for gfx950.

A thin ctypes binding of libtra_gemm.so, whose C ABI is declared in
include/tra_gemm.h.  The functions here have the ABI's names and only
marshal arguments: every step of the GEMM runs in the library's HIP kernels.
There is no CPU fallback; if the library is missing, every call raises.

Low-level calls take raw device addresses (ints) and a hipStream_t handle:

    gemm_f32(M, N, K, A, lda, B, ldb, C, ldc, stream) -> status
    gemm_f32_variant(variant, M, N, K, A, lda, B, ldb, C, ldc, stream) -> status
    gemm_f32_variant_ws(variant, M, N, K, A, lda, B, ldb, C, ldc,
                        workspace, workspace_bytes, stream) -> status
    gemm_f32_variant_noalloc(variant, M, N, K, A, lda, B, ldb, C, ldc,
                             stream) -> status

``matmul(A, B, C=None, variant=AUTO)`` is the torch-tensor convenience
form: it checks the tensors, passes their device pointers and torch's
current stream, and raises TraError on a non-OK status.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtra_gemm.so")
POISON_LIB_PATH = os.path.join(HERE, "libtra_gemm_poison.so")

# tra_status
TRA_OK = 0
TRA_ERR_INVALID_ARG = 1
TRA_ERR_UNSUPPORTED = 2
TRA_ERR_HIP = 3

# tra_gemm_variant
AUTO = 0
NAIVE = 1
LDS_TILED = 2
REGBLOCK_DB = 3
MFMA = 4
MFMA_STREAMK = 5
VARIANTS = {"auto": AUTO, "naive": NAIVE, "lds_tiled": LDS_TILED,
            "regblock_db": REGBLOCK_DB, "mfma": MFMA, "mfma_streamk": MFMA_STREAMK}
LADDER = (NAIVE, LDS_TILED, REGBLOCK_DB, MFMA)

ABI_FUNCTIONS = ("gemm_f32", "gemm_f32_variant", "gemm_f32_variant_ws",
                 "gemm_f32_variant_noalloc",
                 "tra_gemm_workspace_size", "tra_gemm_release_workspaces",
                 "tra_gemm_describe", "tra_status_string",
                 "tra_gemm_variant_name", "tra_last_hip_error", "tra_probe_work",
                 "tra_probe_copy_f32", "tra_probe_mfma_f32", "tra_probe_fma_f32",
                 "tra_probe_launch")

# tra_probe
PROBE_COPY = 0
PROBE_MFMA = 1
PROBE_FMA = 2
PROBE_BLOCKS = 1024
PROBE_SINK_FLOATS = PROBE_BLOCKS * 256

# TRA_STATIC_SCRATCH_BYTES: the scratch of gemm_f32_variant_noalloc
STATIC_SCRATCH_BYTES = 32 << 20


class TraError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        msg = f"{what}: {tra_status_string(status)} (status {status})"
        if status == TRA_ERR_HIP:
            msg += f", hipError_t {tra_last_hip_error()}"
        super().__init__(msg)


_lib = None


def load() -> ctypes.CDLL:
    """Load libtra_gemm.so (built by __graft_entry__.build() or build.py)."""
    global _lib
    if _lib is not None:
        return _lib
    _lib = _open(LIB_PATH)
    return _lib


def load_poisoned() -> ctypes.CDLL:
    """The test build of the library (libtra_gemm_poison.so): the same
    entry points, with every kernel filling its LDS with NaN before use.
    For tests only; a separate handle from load()."""
    return _open(POISON_LIB_PATH)


def _open(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
    # PyTorch ships its own libamdhip64.so.7, with the same soname as ROCm's.
    # Whichever is loaded first is the one HIP runtime of the process, and
    # the library's launches failed when it brought in ROCm's copy ahead of
    # torch's.  So torch, which owns the device buffers and streams passed
    # in, is loaded first when it is installed.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    i64, p, c_int = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.gemm_f32.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p]
    lib.gemm_f32.restype = c_int
    lib.gemm_f32_variant.argtypes = [c_int, i64, i64, i64, p, i64, p, i64, p, i64, p]
    lib.gemm_f32_variant.restype = c_int
    lib.gemm_f32_variant_ws.argtypes = [c_int, i64, i64, i64, p, i64, p, i64, p, i64, p,
                                        ctypes.c_size_t, p]
    lib.gemm_f32_variant_ws.restype = c_int
    lib.gemm_f32_variant_noalloc.argtypes = [c_int, i64, i64, i64, p, i64, p, i64, p, i64, p]
    lib.gemm_f32_variant_noalloc.restype = c_int
    lib.tra_gemm_workspace_size.argtypes = [c_int, i64, i64, i64,
                                            ctypes.POINTER(ctypes.c_size_t)]
    lib.tra_gemm_workspace_size.restype = c_int
    lib.tra_gemm_release_workspaces.argtypes = []
    lib.tra_gemm_release_workspaces.restype = c_int
    lib.tra_gemm_describe.argtypes = [c_int, i64, i64, i64, ctypes.c_char_p, ctypes.c_size_t]
    lib.tra_gemm_describe.restype = c_int
    lib.tra_status_string.argtypes = [c_int]
    lib.tra_status_string.restype = ctypes.c_char_p
    lib.tra_gemm_variant_name.argtypes = [c_int]
    lib.tra_gemm_variant_name.restype = ctypes.c_char_p
    lib.tra_last_hip_error.argtypes = []
    lib.tra_last_hip_error.restype = c_int
    lib.tra_probe_work.argtypes = [c_int, i64]
    lib.tra_probe_work.restype = ctypes.c_double
    lib.tra_probe_copy_f32.argtypes = [i64, p, p, p]
    lib.tra_probe_copy_f32.restype = c_int
    lib.tra_probe_mfma_f32.argtypes = [i64, p, p]
    lib.tra_probe_mfma_f32.restype = c_int
    lib.tra_probe_fma_f32.argtypes = [i64, p, p]
    lib.tra_probe_fma_f32.restype = c_int
    lib.tra_probe_launch.argtypes = [i64, p]
    lib.tra_probe_launch.restype = c_int
    return lib


# --- the ABI, one Python function per C function -----------------------------

def gemm_f32(M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> int:
    return load().gemm_f32(M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_f32_variant(variant, M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> int:
    return load().gemm_f32_variant(variant, M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_f32_variant_ws(variant, M, N, K, A, lda, B, ldb, C, ldc, workspace, workspace_bytes,
                        stream=None) -> int:
    return load().gemm_f32_variant_ws(variant, M, N, K, A, lda, B, ldb, C, ldc, workspace,
                                      workspace_bytes, stream)


def gemm_f32_variant_noalloc(variant, M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> int:
    return load().gemm_f32_variant_noalloc(variant, M, N, K, A, lda, B, ldb, C, ldc, stream)


def tra_gemm_workspace_size(variant: int, M: int, N: int, K: int) -> int:
    out = ctypes.c_size_t(0)
    st = load().tra_gemm_workspace_size(variant, M, N, K, ctypes.byref(out))
    if st != TRA_OK:
        raise TraError(st, "tra_gemm_workspace_size")
    return out.value


def tra_gemm_release_workspaces() -> int:
    return load().tra_gemm_release_workspaces()


def tra_gemm_describe(variant: int, M: int, N: int, K: int) -> str:
    buf = ctypes.create_string_buffer(256)
    st = load().tra_gemm_describe(variant, M, N, K, buf, len(buf))
    if st != TRA_OK:
        raise TraError(st, "tra_gemm_describe")
    return buf.value.decode()


def tra_status_string(status: int) -> str:
    return load().tra_status_string(status).decode()


def tra_gemm_variant_name(variant: int) -> str:
    return load().tra_gemm_variant_name(variant).decode()


def tra_last_hip_error() -> int:
    return load().tra_last_hip_error()


def tra_probe_work(probe: int, amount: int) -> float:
    return load().tra_probe_work(probe, amount)


def tra_probe_copy_f32(n, src, dst, stream=None) -> int:
    return load().tra_probe_copy_f32(n, src, dst, stream)


def tra_probe_mfma_f32(iters, sink, stream=None) -> int:
    return load().tra_probe_mfma_f32(iters, sink, stream)


def tra_probe_fma_f32(iters, sink, stream=None) -> int:
    return load().tra_probe_fma_f32(iters, sink, stream)


def tra_probe_launch(workgroups, stream=None) -> int:
    return load().tra_probe_launch(workgroups, stream)


# --- torch convenience --------------------------------------------------------

def _row_major_ld(shape, strides, name) -> int:
    """Leading dimension of a 2-D row-major view with this shape and these
    strides (in elements), or ValueError if the view is not row-major:
    every row must be contiguous, whatever the row count (a one-row view
    with a column stride above 1 is not a row-major matrix either), and
    rows may not overlap."""
    rows, cols = shape
    if cols > 1 and strides[1] != 1:
        raise ValueError(f"{name} must be row-major (unit column stride)")
    if rows > 1 and strides[0] < max(1, cols):
        raise ValueError(f"{name} must be row-major (row stride at least the row length)")
    return strides[0] if rows > 1 else max(1, cols)


def _check_operand(x, name) -> int:
    """Checks a matmul operand and returns its leading dimension."""
    import torch
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if x.dtype != torch.float32 or x.dim() != 2 or not x.is_cuda:
        raise TypeError(f"{name} must be a 2-D float32 tensor on a GPU")
    return _row_major_ld(tuple(x.shape), x.stride(), name)


def matmul(A, B, C=None, variant: int = AUTO, stream=None, workspace=None):
    """C = A @ B on the GPU through libtra_gemm.so; returns C.

    A (M x K) and B (K x N) are float32 row-major tensors (row padding
    allowed) on the same device; C, if given, is an M x N float32 row-major
    tensor that is overwritten.  ``stream`` is a torch.cuda.Stream or None
    for torch's current stream.  ``workspace`` (a contiguous device tensor
    of at least tra_gemm_workspace_size() bytes) replaces the library's own
    scratch for the stream-K variant.
    """
    import torch
    lda = _check_operand(A, "A")
    ldb = _check_operand(B, "B")
    M, K = A.shape
    if B.shape[0] != K:
        raise ValueError(f"inner dimensions differ: A is {tuple(A.shape)}, B is {tuple(B.shape)}")
    N = B.shape[1]
    if C is None:
        C = torch.empty((M, N), dtype=torch.float32, device=A.device)
    ldc = _check_operand(C, "C")
    if tuple(C.shape) != (M, N):
        raise ValueError(f"C must be {M} x {N}")
    if B.device != A.device or C.device != A.device:
        raise ValueError("A, B and C must be on the same device")
    s = stream if stream is not None else torch.cuda.current_stream(A.device)
    with torch.cuda.device(A.device):
        if workspace is None:
            st = gemm_f32_variant(variant, M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb,
                                  C.data_ptr(), ldc, s.cuda_stream)
        else:
            if not workspace.is_cuda or workspace.device != A.device or not workspace.is_contiguous():
                raise ValueError("workspace must be a contiguous tensor on A's device")
            st = gemm_f32_variant_ws(variant, M, N, K, A.data_ptr(), lda, B.data_ptr(),
                                     ldb, C.data_ptr(), ldc, workspace.data_ptr(),
                                     workspace.numel() * workspace.element_size(), s.cuda_stream)
    if st != TRA_OK:
        raise TraError(st, "gemm_f32_variant")
    return C
