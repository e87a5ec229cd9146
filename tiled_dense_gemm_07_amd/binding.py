"""Python binding of the tilegemm C ABI (``include/tilegemm.h``).

Argument marshalling only: tensors are checked (device, dtype, shape,
contiguity) and their device pointers, together with the current HIP stream,
are passed to ``libtilegemm.so``.  Every step of the computation runs in the
library's HIP kernels; there is no fallback.  If the library has not been
built, loading raises instead of computing anything another way.

PyTorch is used only for device memory and streams.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_DEFAULT_LIB = os.path.join(HERE, "libtilegemm.so")

TG_F32, TG_F16, TG_BF16 = 0, 1, 2
TG_EPI_NONE, TG_EPI_RELU = 0, 1
TG_OP_GEMM, TG_OP_DEQUANT_W4, TG_OP_MX, TG_OP_SP24 = 0, 1, 2, 3
TG_MX_E2M1, TG_MX_E4M3 = 0, 1

# exported symbols, as declared in include/tilegemm.h
EXPORTS = ("tg_gemm", "tg_gemm_ex", "tg_dequant_gemm_w4", "tg_status_str", "tg_query_config",
           "tg_query_config_ex", "tg_config_count", "tg_config_name", "tg_gemm_config",
           "tg_gemm_ex_config", "tg_dequant_gemm_w4_config", "tg_tile_map", "tg_gemm_mx",
           "tg_gemm_mx_config", "tg_gemm_sp24", "tg_gemm_sp24_config", "tg_gemm_splitk",
           "tg_gemm_splitk_workspace_size", "tg_gemm_splitk_config", "tg_gemm_splitk_noalloc",
           "tg_set_clock_stamps", "tg_set_swizzle_override", "tg_config_occupancy")
TG_SPLITK_SCRATCH_BYTES = 16 * 1024 * 1024

_lib = None


class TileGemmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def library_path() -> str:
    return os.environ.get("TILEGEMM_LIB", _DEFAULT_LIB)


def load_library():
    """Load libtilegemm.so (raises if it is missing: build it first)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise FileNotFoundError(
            "libtilegemm.so not found at %s; build it with "
            "`python -m tiled_dense_gemm_07_amd.build`" % path)
    lib = ctypes.CDLL(path)
    i64, p, c_int = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.tg_gemm.argtypes = [i64, i64, i64, c_int, p, p, p, c_int, p]
    lib.tg_gemm.restype = c_int
    lib.tg_gemm_ex.argtypes = [i64, i64, i64, c_int, p, c_int, p, c_int, p, c_int, p]
    lib.tg_gemm_ex.restype = c_int
    lib.tg_gemm_ex_config.argtypes = [c_int, i64, i64, i64, c_int, p, c_int, p, c_int, p, c_int, p]
    lib.tg_gemm_ex_config.restype = c_int
    lib.tg_query_config_ex.argtypes = [c_int, i64, i64, i64, c_int, c_int, c_int, ctypes.c_char_p,
                                       ctypes.c_size_t]
    lib.tg_query_config_ex.restype = c_int
    lib.tg_dequant_gemm_w4.argtypes = [i64, i64, i64, p, p, p, p, c_int, p]
    lib.tg_dequant_gemm_w4.restype = c_int
    lib.tg_status_str.argtypes = [c_int]
    lib.tg_status_str.restype = ctypes.c_char_p
    lib.tg_query_config.argtypes = [c_int, i64, i64, i64, c_int, ctypes.c_char_p, ctypes.c_size_t]
    lib.tg_query_config.restype = c_int
    lib.tg_config_count.argtypes = [c_int, c_int]
    lib.tg_config_count.restype = c_int
    lib.tg_config_name.argtypes = [c_int, c_int, c_int, ctypes.c_char_p, ctypes.c_size_t]
    lib.tg_config_name.restype = c_int
    lib.tg_gemm_config.argtypes = [c_int, i64, i64, i64, c_int, p, p, p, c_int, p]
    lib.tg_gemm_config.restype = c_int
    lib.tg_dequant_gemm_w4_config.argtypes = [c_int, i64, i64, i64, p, p, p, p, c_int, p]
    lib.tg_dequant_gemm_w4_config.restype = c_int
    lib.tg_tile_map.argtypes = [i64, i64, c_int, p, p]
    lib.tg_tile_map.restype = c_int
    lib.tg_gemm_mx.argtypes = [i64, i64, i64, c_int, p, p, p, p, p, c_int, p]
    lib.tg_gemm_mx.restype = c_int
    lib.tg_gemm_mx_config.argtypes = [c_int, i64, i64, i64, c_int, p, p, p, p, p, c_int, p]
    lib.tg_gemm_mx_config.restype = c_int
    lib.tg_gemm_sp24.argtypes = [i64, i64, i64, c_int, p, p, p, p, c_int, p]
    lib.tg_gemm_sp24.restype = c_int
    lib.tg_gemm_sp24_config.argtypes = [c_int, i64, i64, i64, c_int, p, p, p, p, c_int, p]
    lib.tg_gemm_sp24_config.restype = c_int
    lib.tg_gemm_splitk.argtypes = [i64, i64, i64, c_int, p, p, p, c_int, c_int, p,
                                   ctypes.c_size_t, p]
    lib.tg_gemm_splitk.restype = c_int
    lib.tg_gemm_splitk_config.argtypes = [c_int, i64, i64, i64, c_int, p, p, p, c_int, c_int, p,
                                          ctypes.c_size_t, p]
    lib.tg_gemm_splitk_config.restype = c_int
    lib.tg_gemm_splitk_workspace_size.argtypes = [i64, i64, i64, c_int, c_int,
                                                  ctypes.POINTER(ctypes.c_size_t)]
    lib.tg_gemm_splitk_workspace_size.restype = c_int
    lib.tg_gemm_splitk_noalloc.argtypes = [i64, i64, i64, c_int, p, p, p, c_int, c_int, p]
    lib.tg_gemm_splitk_noalloc.restype = c_int
    lib.tg_set_clock_stamps.argtypes = [p]
    lib.tg_set_clock_stamps.restype = None
    lib.tg_set_swizzle_override.argtypes = [c_int]
    lib.tg_set_swizzle_override.restype = None
    lib.tg_config_occupancy.argtypes = [c_int, c_int, c_int, ctypes.POINTER(c_int)]
    lib.tg_config_occupancy.restype = c_int
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load_library().tg_status_str(status).decode()


def _check(status: int):
    if status != 0:
        raise TileGemmError(status, status_str(status))


_DTYPE_CODES = None


def _dtype_code(t) -> int:
    global _DTYPE_CODES
    if _DTYPE_CODES is None:
        import torch

        _DTYPE_CODES = {torch.float32: TG_F32, torch.float16: TG_F16, torch.bfloat16: TG_BF16}
    code = _DTYPE_CODES.get(t.dtype)
    if code is None:
        raise TypeError("unsupported dtype %s (float32, float16 or bfloat16)" % t.dtype)
    return code


def _epi_code(epilogue) -> int:
    if epilogue in (None, "none", TG_EPI_NONE):
        return TG_EPI_NONE
    if epilogue in ("relu", TG_EPI_RELU):
        return TG_EPI_RELU
    raise ValueError("epilogue must be None/'none' or 'relu'")


def _stream_ptr(device, stream=None):
    if stream is None:
        import torch

        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def _require_gpu_tensor(name, t):
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous (row-major)" % name)


def _gemm_args(A, B, C):
    _require_gpu_tensor("A", A)
    _require_gpu_tensor("B", B)
    if A.dim() != 2 or B.dim() != 2:
        raise ValueError("A and B must be 2-D")
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ: A is %s, B is %s" % (tuple(A.shape), tuple(B.shape)))
    if A.dtype != B.dtype:
        raise TypeError("A and B must share a dtype")
    if C is not None:
        _require_gpu_tensor("C", C)
        if tuple(C.shape) != (M, N) or C.dtype != A.dtype:
            raise ValueError("C must be [M, N] of the operand dtype")
    return M, N, K


def gemm(A, B, C=None, epilogue=None, stream=None):
    """C = epilogue(A @ B) on the GPU (fp32 / fp16 / bf16, row-major). Returns C."""
    M, N, K = _gemm_args(A, B, C)
    if C is None:
        import torch

        C = torch.empty((M, N), dtype=A.dtype, device=A.device)
    _check(load_library().tg_gemm(M, N, K, _dtype_code(A), A.data_ptr(), B.data_ptr(),
                                  C.data_ptr(), _epi_code(epilogue), _stream_ptr(A.device, stream)))
    return C


def gemm_with_config(index: int, A, B, C=None, epilogue=None, stream=None):
    """As :func:`gemm`, launching compiled configuration `index` (for the sweep)."""
    import torch

    M, N, K = _gemm_args(A, B, C)
    if C is None:
        C = torch.empty((M, N), dtype=A.dtype, device=A.device)
    _check(load_library().tg_gemm_config(index, M, N, K, _dtype_code(A), A.data_ptr(),
                                         B.data_ptr(), C.data_ptr(), _epi_code(epilogue),
                                         _stream_ptr(A.device, stream)))
    return C


def splitk_workspace_size(M: int, N: int, K: int, dtype: int, splits: int = 0) -> int:
    """Workspace bytes :func:`gemm_splitk` needs for this shape (0: no split)."""
    out = ctypes.c_size_t(0)
    _check(load_library().tg_gemm_splitk_workspace_size(M, N, K, dtype, splits,
                                                        ctypes.byref(out)))
    return out.value


def splitk_workspace(M: int, N: int, K: int, dtype: int, splits: int = 0, device="cuda"):
    """A zero-filled uint8 device tensor large enough for :func:`gemm_splitk`
    (None when no split would be launched).  Reusable across calls on one stream."""
    import torch

    n = splitk_workspace_size(M, N, K, dtype, splits)
    return torch.zeros((n,), dtype=torch.uint8, device=device) if n else None


def gemm_splitk(A, B, C=None, epilogue=None, splits: int = 0, workspace=None, stream=None,
                config=None):
    """As :func:`gemm`, with each output tile's K range split over `splits`
    workgroups (0: chosen by the library).  workspace: a zero-filled uint8
    device tensor of at least :func:`splitk_workspace_size` bytes (allocated
    here when None).  config: force a compiled configuration by index."""
    import torch

    M, N, K = _gemm_args(A, B, C)
    if C is None:
        C = torch.empty((M, N), dtype=A.dtype, device=A.device)
    dt = _dtype_code(A)
    if workspace is None:
        workspace = splitk_workspace(M, N, K, dt, splits, device=A.device)
    if workspace is not None:
        _require_gpu_tensor("workspace", workspace)
    wp = workspace.data_ptr() if workspace is not None else None
    wn = workspace.numel() * workspace.element_size() if workspace is not None else 0
    lib = load_library()
    args = (M, N, K, dt, A.data_ptr(), B.data_ptr(), C.data_ptr(), _epi_code(epilogue), splits,
            wp, wn, _stream_ptr(A.device, stream))
    _check(lib.tg_gemm_splitk(*args) if config is None else lib.tg_gemm_splitk_config(config, *args))
    return C


def gemm_splitk_noalloc(A, B, C, epilogue=None, splits: int = 0, stream=None):
    """As :func:`gemm_splitk`, with the partial tiles in the library's fixed
    scratch array instead of a workspace (tg_gemm_splitk_noalloc): C must be
    given, and nothing is allocated.  Calls that overlap on one GPU race."""
    M, N, K = _gemm_args(A, B, C)
    _check(load_library().tg_gemm_splitk_noalloc(
        M, N, K, _dtype_code(A), A.data_ptr(), B.data_ptr(), C.data_ptr(), _epi_code(epilogue),
        splits, _stream_ptr(A.device, stream)))
    return C


def set_clock_stamps(stamps):
    """Record the shader clock of every following launch into `stamps`, an
    int64 / uint64 device tensor of 32 elements (None: stop recording)."""
    if stamps is not None:
        _require_gpu_tensor("stamps", stamps)
        if stamps.numel() * stamps.element_size() < 32 * 8:
            raise ValueError("stamps must hold 32 64-bit values")
    load_library().tg_set_clock_stamps(stamps.data_ptr() if stamps is not None else None)


def set_swizzle_override(group_m: int):
    """Force swizzle group `group_m` on every following launch (0: none)."""
    load_library().tg_set_swizzle_override(int(group_m))


def config_occupancy(op: int, dtype: int, index: int) -> int:
    """Workgroups of configuration `index` one compute unit holds at once."""
    n = ctypes.c_int(0)
    _check(load_library().tg_config_occupancy(op, dtype, index, ctypes.byref(n)))
    return n.value


def stamp_clock_ghz(stamps) -> list:
    """Shader clock (GHz) of each workgroup 0..7 that wrote a record into the
    host copy of `stamps` (a sequence of 32 integers)."""
    out = []
    for b in range(8):
        t0, r0, t1, r1 = (int(x) for x in stamps[4 * b:4 * b + 4])
        if r1 > r0 and t1 > t0:
            out.append((t1 - t0) / ((r1 - r0) / 100e6) / 1e9)
    return out


def _gemm_ex_args(A, B, trans_a, trans_b, C):
    _require_gpu_tensor("A", A)
    _require_gpu_tensor("B", B)
    if A.dim() != 2 or B.dim() != 2:
        raise ValueError("A and B must be 2-D")
    K, M = A.shape if trans_a else (A.shape[1], A.shape[0])
    N, K2 = B.shape if trans_b else (B.shape[1], B.shape[0])
    if K != K2:
        raise ValueError("inner dimensions differ: A is %s (trans_a=%d), B is %s (trans_b=%d)"
                         % (tuple(A.shape), trans_a, tuple(B.shape), trans_b))
    if A.dtype != B.dtype:
        raise TypeError("A and B must share a dtype")
    if C is not None:
        _require_gpu_tensor("C", C)
        if tuple(C.shape) != (M, N) or C.dtype != A.dtype:
            raise ValueError("C must be [M, N] of the operand dtype")
    return M, N, K


def gemm_ex(A, B, trans_a=False, trans_b=False, C=None, epilogue=None, stream=None, config=None):
    """C = epilogue(op(A) @ op(B)): A stored [M, K] (or [K, M] with trans_a),
    B stored [K, N] (or [N, K] with trans_b).  config: force a compiled
    configuration by index (for the sweep and tests)."""
    import torch

    ta, tb = int(bool(trans_a)), int(bool(trans_b))
    M, N, K = _gemm_ex_args(A, B, ta, tb, C)
    if C is None:
        C = torch.empty((M, N), dtype=A.dtype, device=A.device)
    lib = load_library()
    args = (M, N, K, _dtype_code(A), A.data_ptr(), ta, B.data_ptr(), tb, C.data_ptr(),
            _epi_code(epilogue), _stream_ptr(A.device, stream))
    _check(lib.tg_gemm_ex(*args) if config is None else lib.tg_gemm_ex_config(config, *args))
    return C


def _w4_args(A, Wq, Ws, C):
    import torch

    for name, t in (("A", A), ("Wq", Wq), ("Ws", Ws)):
        _require_gpu_tensor(name, t)
    if A.dtype != torch.bfloat16:
        raise TypeError("activations must be bfloat16")
    if Wq.dtype != torch.uint8 or Ws.dtype != torch.uint8:
        raise TypeError("packed weights and scales must be uint8")
    M, K = A.shape
    N = Wq.shape[0]
    if tuple(Wq.shape) != (N, K // 2) or tuple(Ws.shape) != (N, K // 32) or K % 32:
        raise ValueError("expected Wq [N, K/2] and Ws [N, K/32] with K % 32 == 0")
    if C is not None:
        _require_gpu_tensor("C", C)
        if tuple(C.shape) != (M, N) or C.dtype != torch.bfloat16:
            raise ValueError("C must be bfloat16 [M, N]")
    return M, N, K


def dequant_gemm_w4(A, Wq, Ws, C=None, epilogue=None, stream=None):
    """C = epilogue(A @ W^T) with W given as packed E2M1 codes and E8M0 scales."""
    import torch

    M, N, K = _w4_args(A, Wq, Ws, C)
    if C is None:
        C = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    _check(load_library().tg_dequant_gemm_w4(M, N, K, A.data_ptr(), Wq.data_ptr(), Ws.data_ptr(),
                                             C.data_ptr(), _epi_code(epilogue),
                                             _stream_ptr(A.device, stream)))
    return C


def dequant_gemm_w4_with_config(index: int, A, Wq, Ws, C=None, epilogue=None, stream=None):
    import torch

    M, N, K = _w4_args(A, Wq, Ws, C)
    if C is None:
        C = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    _check(load_library().tg_dequant_gemm_w4_config(index, M, N, K, A.data_ptr(), Wq.data_ptr(),
                                                    Ws.data_ptr(), C.data_ptr(),
                                                    _epi_code(epilogue),
                                                    _stream_ptr(A.device, stream)))
    return C


def _mx_args(fmt, Aq, As, Wq, Ws, C):
    import torch

    if fmt not in (TG_MX_E2M1, TG_MX_E4M3):
        raise ValueError("activation format must be TG_MX_E2M1 or TG_MX_E4M3")
    for name, t in (("Aq", Aq), ("As", As), ("Wq", Wq), ("Ws", Ws)):
        _require_gpu_tensor(name, t)
        if t.dtype != torch.uint8:
            raise TypeError("%s must be uint8" % name)
    M = Aq.shape[0]
    K = Aq.shape[1] * (2 if fmt == TG_MX_E2M1 else 1)
    N = Wq.shape[0]
    if (tuple(As.shape) != (M, K // 32) or tuple(Wq.shape) != (N, K // 2)
            or tuple(Ws.shape) != (N, K // 32) or K % 32):
        raise ValueError("expected As [M, K/32], Wq [N, K/2], Ws [N, K/32] with K % 32 == 0")
    if C is not None:
        _require_gpu_tensor("C", C)
        if tuple(C.shape) != (M, N) or C.dtype != torch.bfloat16:
            raise ValueError("C must be bfloat16 [M, N]")
    return M, N, K


def gemm_mx(fmt: int, Aq, As, Wq, Ws, C=None, epilogue=None, stream=None, config=None):
    """C = epilogue(a @ w^T) with both operands in MX blocks: activation codes Aq
    (E2M1 [M, K/2] or E4M3 [M, K]) with E8M0 scales As [M, K/32], E2M1 weights
    Wq [N, K/2] with E8M0 scales Ws [N, K/32]; bf16 output.  `config` forces a
    compiled configuration by index."""
    import torch

    M, N, K = _mx_args(fmt, Aq, As, Wq, Ws, C)
    if C is None:
        C = torch.empty((M, N), dtype=torch.bfloat16, device=Aq.device)
    args = (M, N, K, fmt, Aq.data_ptr(), As.data_ptr(), Wq.data_ptr(), Ws.data_ptr(),
            C.data_ptr(), _epi_code(epilogue), _stream_ptr(Aq.device, stream))
    lib = load_library()
    _check(lib.tg_gemm_mx(*args) if config is None else lib.tg_gemm_mx_config(config, *args))
    return C


def gemm_sp24(Ac, Ai, B, C=None, epilogue=None, stream=None, config=None):
    """C = epilogue(A @ B) with A 2:4 sparse along K, given as kept values Ac
    [M, K/2] (fp16 or bf16) and position nibbles Ai [M, K/8] (uint8); B [K, N]
    of Ac's dtype.  `config` forces a compiled configuration by index."""
    import torch

    for name, t in (("Ac", Ac), ("Ai", Ai), ("B", B)):
        _require_gpu_tensor(name, t)
    if Ac.dtype not in (torch.float16, torch.bfloat16) or B.dtype != Ac.dtype:
        raise TypeError("Ac and B must both be float16 or both bfloat16")
    if Ai.dtype != torch.uint8:
        raise TypeError("Ai must be uint8")
    M, half = Ac.shape
    K = 2 * half
    K2, N = B.shape
    if K != K2 or tuple(Ai.shape) != (M, K // 8) or K % 8:
        raise ValueError("expected Ac [M, K/2], Ai [M, K/8], B [K, N]")
    if C is None:
        C = torch.empty((M, N), dtype=Ac.dtype, device=Ac.device)
    else:
        _require_gpu_tensor("C", C)
        if tuple(C.shape) != (M, N) or C.dtype != Ac.dtype:
            raise ValueError("C must be [M, N] of Ac's dtype")
    args = (M, N, K, _dtype_code(Ac), Ac.data_ptr(), Ai.data_ptr(), B.data_ptr(),
            C.data_ptr(), _epi_code(epilogue), _stream_ptr(Ac.device, stream))
    lib = load_library()
    _check(lib.tg_gemm_sp24(*args) if config is None else lib.tg_gemm_sp24_config(config, *args))
    return C


def query_config(op: int, M: int, N: int, K: int, dtype: int = TG_BF16, trans_a: bool = False,
                 trans_b: bool = False) -> str:
    buf = ctypes.create_string_buffer(256)
    _check(load_library().tg_query_config_ex(op, M, N, K, dtype, int(trans_a), int(trans_b), buf,
                                             len(buf)))
    return buf.value.decode()


def list_configs(op: int, dtype: int = TG_BF16):
    lib = load_library()
    names = []
    for i in range(lib.tg_config_count(op, dtype)):
        buf = ctypes.create_string_buffer(128)
        _check(lib.tg_config_name(op, dtype, i, buf, len(buf)))
        names.append(buf.value.decode())
    return names


def tile_map(tiles_m: int, tiles_n: int, group_m: int):
    """The scheduler's workgroup -> (tile_m, tile_n) map, computed on the host."""
    total = tiles_m * tiles_n
    om = np.empty(total, dtype=np.int32)
    on = np.empty(total, dtype=np.int32)
    _check(load_library().tg_tile_map(tiles_m, tiles_n, group_m,
                                      om.ctypes.data_as(ctypes.c_void_p),
                                      on.ctypes.data_as(ctypes.c_void_p)))
    return om, on
