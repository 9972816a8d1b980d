"""Fused dense GEMM + ReLU on AMD Instinct MI355X (gfx950).

Thin Python binding of ``libgemm_relu.so`` (C-ABI in ``include/gemm_relu.h``):
argument marshalling only — every step of C = max(A·op(B), 0) runs in the HIP
kernels of that library.  There is no CPU or PyTorch fallback: if the library
is missing, importing the binding's functions raises.

Operation: page "TileLang：GPU/NPU 通用算子 DSL", §3.2 (GPU minimal example:
fp16 A (M,K), B (K,N), fp32 accumulator, ReLU, fp16 C) and §3.3 (bf16 with B
stored (N,K) and transpose_B, fp32 C).
"""
import ctypes
import os

F16 = 0
BF16 = 1
F32 = 2
F8E4M3 = 3     # OCP 8-bit E4M3 (inputs only)
F8E5M2 = 4     # OCP 8-bit E5M2 (inputs only)
MX_E4M3 = 5    # block-scaled (gemm_relu_mx): MXFP8, E4M3 elements
MX_E5M2 = 6    # MXFP8, E5M2 elements
MX_E2M1 = 7    # MXFP4, E2M1 elements packed two per byte

OK = 0
EINVAL = -1
EUNSUPPORTED = -2
EHIP = -3
ESCRATCH = -4

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgemm_relu.so")
PROBE_LIB_PATH = os.path.join(_PKG, "libgemm_relu_probe.so")

EXPORTS = ("gemm_relu", "gemm_relu_strerror", "gemm_relu_configs", "gemm_relu_plan",
           "gemm_relu_ws", "gemm_relu_workspace_size", "gemm_relu_ws_plan", "gemm_relu_noalloc",
           "gemm_relu_mx", "gemm_relu_mx_plan", "gemm_relu_sp", "gemm_relu_sp_plan")

_lib = None


class GemmReluError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("gemm_relu failed (%d): %s" % (status, msg))
        self.status = status


def library():
    """The loaded product library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("HIP library %s is not built; run __graft_entry__.build()" % LIB_PATH)
    # PyTorch (the source of device memory and streams here) brings its own HIP
    # runtime; loading it first makes the library bind to that same runtime
    # instead of pulling a second copy into the process.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    i64 = ctypes.c_int64
    vp = ctypes.c_void_p
    lib.gemm_relu.argtypes = [vp, vp, vp, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                              ctypes.c_int, vp]
    lib.gemm_relu.restype = ctypes.c_int
    lib.gemm_relu_strerror.argtypes = [ctypes.c_int]
    lib.gemm_relu_strerror.restype = ctypes.c_char_p
    lib.gemm_relu_configs.argtypes = []
    lib.gemm_relu_configs.restype = ctypes.c_char_p
    lib.gemm_relu_plan.argtypes = [vp, vp, vp, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int]
    lib.gemm_relu_plan.restype = ctypes.c_char_p
    u64 = ctypes.c_uint64
    lib.gemm_relu_ws.argtypes = [vp, vp, vp, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_int, vp, u64, vp]
    lib.gemm_relu_ws.restype = ctypes.c_int
    lib.gemm_relu_noalloc.argtypes = [vp, vp, vp, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, vp]
    lib.gemm_relu_noalloc.restype = ctypes.c_int
    lib.gemm_relu_workspace_size.argtypes = [i64, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.gemm_relu_workspace_size.restype = i64
    lib.gemm_relu_ws_plan.argtypes = [vp, vp, vp, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, vp, u64]
    lib.gemm_relu_ws_plan.restype = ctypes.c_char_p
    lib.gemm_relu_mx.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, ctypes.c_int, ctypes.c_int, vp]
    lib.gemm_relu_mx.restype = ctypes.c_int
    lib.gemm_relu_mx_plan.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, ctypes.c_int,
                                      ctypes.c_int]
    lib.gemm_relu_mx_plan.restype = ctypes.c_char_p
    lib.gemm_relu_sp.argtypes = [vp, vp, vp, vp, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_int, vp]
    lib.gemm_relu_sp.restype = ctypes.c_int
    lib.gemm_relu_sp_plan.argtypes = [vp, vp, vp, vp, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int]
    lib.gemm_relu_sp_plan.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _addr(x):
    """Device address of a tensor (data_ptr) or a raw integer address."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream_handle(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def gemm_relu_strerror(status):
    return library().gemm_relu_strerror(int(status)).decode()


def gemm_relu_status(A, B, C, M, N, K, in_dtype, out_dtype, transB, stream=None):
    """Call the C-ABI and return its status code (no exception)."""
    return library().gemm_relu(_addr(A), _addr(B), _addr(C), int(M), int(N), int(K),
                               int(in_dtype), int(out_dtype), int(transB),
                               _stream_handle(stream))


def gemm_relu(A, B, C, M, N, K, in_dtype, out_dtype, transB, stream=None):
    """C = max(A·op(B), 0) through the C-ABI; raises GemmReluError on failure.

    A, B, C are device tensors or raw device addresses; stream is a
    torch.cuda.Stream, a raw hipStream_t, or None for torch's current stream.
    """
    rc = gemm_relu_status(A, B, C, M, N, K, in_dtype, out_dtype, transB, stream)
    if rc != OK:
        raise GemmReluError(rc, gemm_relu_strerror(rc))


def gemm_relu_configs():
    """Names of the kernel configurations this build of the library holds."""
    return library().gemm_relu_configs().decode().split(",")


def gemm_relu_plan(A, B, C, M, N, K, in_dtype, out_dtype, transB):
    """Configuration name gemm_relu would launch (None if the call is invalid)."""
    r = library().gemm_relu_plan(_addr(A), _addr(B), _addr(C), int(M), int(N), int(K),
                                 int(in_dtype), int(out_dtype), int(transB))
    return None if r is None else r.decode()


def gemm_relu_ws_status(A, B, C, M, N, K, in_dtype, out_dtype, transB, workspace, workspace_bytes,
                        stream=None):
    """Call the workspace C-ABI entry and return its status code (no exception)."""
    return library().gemm_relu_ws(_addr(A), _addr(B), _addr(C), int(M), int(N), int(K),
                                  int(in_dtype), int(out_dtype), int(transB), _addr(workspace),
                                  int(workspace_bytes), _stream_handle(stream))


def gemm_relu_ws(A, B, C, M, N, K, in_dtype, out_dtype, transB, workspace, workspace_bytes,
                 stream=None):
    """gemm_relu with a caller's device workspace (a tensor or raw address and
    its size in bytes); raises GemmReluError on failure."""
    rc = gemm_relu_ws_status(A, B, C, M, N, K, in_dtype, out_dtype, transB, workspace,
                             workspace_bytes, stream)
    if rc != OK:
        raise GemmReluError(rc, gemm_relu_strerror(rc))


def gemm_relu_noalloc_status(A, B, C, M, N, K, in_dtype, out_dtype, transB, stream=None):
    """Call the no-allocation C-ABI entry and return its status code."""
    return library().gemm_relu_noalloc(_addr(A), _addr(B), _addr(C), int(M), int(N), int(K),
                                       int(in_dtype), int(out_dtype), int(transB),
                                       _stream_handle(stream))


def gemm_relu_noalloc(A, B, C, M, N, K, in_dtype, out_dtype, transB, stream=None):
    """gemm_relu_ws with the library's own per-GPU scratch array as the
    workspace (allocates nothing); raises GemmReluError on failure."""
    rc = gemm_relu_noalloc_status(A, B, C, M, N, K, in_dtype, out_dtype, transB, stream)
    if rc != OK:
        raise GemmReluError(rc, gemm_relu_strerror(rc))


def gemm_relu_workspace_size(M, N, K, in_dtype, out_dtype, transB):
    """Workspace bytes gemm_relu_ws would use (0: no K split); negative status
    for invalid arguments."""
    return int(library().gemm_relu_workspace_size(int(M), int(N), int(K), int(in_dtype),
                                                  int(out_dtype), int(transB)))


def gemm_relu_ws_plan(A, B, C, M, N, K, in_dtype, out_dtype, transB, workspace, workspace_bytes):
    """Configuration name gemm_relu_ws would launch (None if the call is invalid)."""
    r = library().gemm_relu_ws_plan(_addr(A), _addr(B), _addr(C), int(M), int(N), int(K),
                                    int(in_dtype), int(out_dtype), int(transB), _addr(workspace),
                                    int(workspace_bytes))
    return None if r is None else r.decode()


def gemm_relu_mx_status(A, SA, B, SB, C, M, N, K, fmt, out_dtype, stream=None):
    """Call the block-scaled C-ABI entry and return its status code."""
    return library().gemm_relu_mx(_addr(A), _addr(SA), _addr(B), _addr(SB), _addr(C), int(M),
                                  int(N), int(K), int(fmt), int(out_dtype), _stream_handle(stream))


def gemm_relu_mx(A, SA, B, SB, C, M, N, K, fmt, out_dtype, stream=None):
    """Block-scaled C = max(sum_b XA XB (A·Bᵀ)_b, 0) through the C-ABI (B stored
    (N, K), E8M0 scales per 32 elements along K); raises GemmReluError."""
    rc = gemm_relu_mx_status(A, SA, B, SB, C, M, N, K, fmt, out_dtype, stream)
    if rc != OK:
        raise GemmReluError(rc, gemm_relu_strerror(rc))


def gemm_relu_mx_plan(A, SA, B, SB, C, M, N, K, fmt, out_dtype):
    r = library().gemm_relu_mx_plan(_addr(A), _addr(SA), _addr(B), _addr(SB), _addr(C), int(M),
                                    int(N), int(K), int(fmt), int(out_dtype))
    return None if r is None else r.decode()


def gemm_relu_sp_status(As, E, B, C, M, N, K, in_dtype, out_dtype, transB, stream=None):
    """Call the 2:4 sparse C-ABI entry and return its status code."""
    return library().gemm_relu_sp(_addr(As), _addr(E), _addr(B), _addr(C), int(M), int(N),
                                  int(K), int(in_dtype), int(out_dtype), int(transB),
                                  _stream_handle(stream))


def gemm_relu_sp(As, E, B, C, M, N, K, in_dtype, out_dtype, transB, stream=None):
    """C = max(A·op(B), 0) for a 2:4 sparse A given compressed: As (M, K/2)
    stored values and E metadata (blocked by 64 columns of K); raises
    GemmReluError."""
    rc = gemm_relu_sp_status(As, E, B, C, M, N, K, in_dtype, out_dtype, transB, stream)
    if rc != OK:
        raise GemmReluError(rc, gemm_relu_strerror(rc))


def gemm_relu_sp_plan(As, E, B, C, M, N, K, in_dtype, out_dtype, transB):
    r = library().gemm_relu_sp_plan(_addr(As), _addr(E), _addr(B), _addr(C), int(M), int(N),
                                    int(K), int(in_dtype), int(out_dtype), int(transB))
    return None if r is None else r.decode()


def _torch_dtype_code(dt):
    import torch
    return {torch.float16: F16, torch.bfloat16: BF16, torch.float32: F32,
            torch.float8_e4m3fn: F8E4M3, torch.float8_e5m2: F8E5M2}[dt]


def matmul_relu(A, B, transB=False, out_dtype=None, out=None, stream=None):
    """Tensor front end: returns C = max(A·B, 0) (or max(A·Bᵀ, 0) with transB).

    A: (M, K) fp16/bf16/float8_e4m3fn/float8_e5m2 CUDA tensor; B: (K, N), or
    (N, K) with transB, same dtype.  C is allocated (like the page's T.empty)
    unless ``out`` is given; its dtype defaults to A's for 16-bit inputs and
    to float16 for 8-bit ones.
    """
    import torch
    if A.dim() != 2 or B.dim() != 2:
        raise ValueError("A and B must be 2-D")
    inputs = (torch.float16, torch.bfloat16, torch.float8_e4m3fn, torch.float8_e5m2)
    if A.dtype != B.dtype or A.dtype not in inputs:
        raise TypeError("A and B must share dtype float16, bfloat16, float8_e4m3fn or "
                        "float8_e5m2")
    if not (A.is_cuda and B.is_cuda) or A.device != B.device:
        raise ValueError("A and B must be on the same GPU")
    if not (A.is_contiguous() and B.is_contiguous()):
        raise ValueError("A and B must be contiguous (row-major)")
    M, K = A.shape
    if transB:
        N, Kb = B.shape
    else:
        Kb, N = B.shape
    if Kb != K:
        raise ValueError("inner dimensions differ: %d vs %d" % (K, Kb))
    if out is None:
        default = A.dtype if A.dtype in (torch.float16, torch.bfloat16) else torch.float16
        out = torch.empty((M, N), dtype=out_dtype or default, device=A.device)
    elif out.shape != (M, N) or not out.is_contiguous() or out.device != A.device:
        raise ValueError("out must be a contiguous (M, N) tensor on A's device")
    gemm_relu(A, B, out, M, N, K, _torch_dtype_code(A.dtype), _torch_dtype_code(out.dtype),
              1 if transB else 0, stream)
    return out
