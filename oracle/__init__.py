"""CPU oracle for the tiled GEMM, the weight-only 4-bit dequant GEMM, the
MX-format GEMM and the 2:4 structured-sparse GEMM.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The library under
``tiled_dense_gemm_07_amd`` never imports, links or calls it, and this package
imports nothing from the library.

The arithmetic lives in ``oracle.c`` (plain C, fp64, OpenMP over output rows);
this module only builds it with gcc and marshals numpy arrays through ctypes.
What it computes, and the pages it follows, are stated in ``oracle.c``:
the plain product C[i, j] = sum_k A[i, k] * B[k, j] in fp64 (the gtnt.cn
page, section 2.2; the mhpq.cn page, sections 2.1 and 3.2), an optional ReLU
applied after the sum (the blog.hotdry.top page's post-processing loop), and one
round-to-nearest-even to the output type for bitwise checks.

Every function is pinned by tests/test_oracle_pins.py against closed forms,
library codecs and exact rational brute force; none is "parity unpinned".
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32, F16, BF16 = 0, 1, 2
_NP_STORAGE = {F32: np.uint32, F16: np.uint16, BF16: np.uint16}


def build(force: bool = True, src: str = SRC, out: str = LIB_PATH) -> str:
    """Compile oracle.c into a shared library (gcc, -O2, OpenMP)."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall",
               "-o", tmp, src, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


def _bind(lib):
    i64, p, d = ctypes.c_int64, ctypes.c_void_p, ctypes.c_double
    sigs = {
        "orc_decode_f32": ([ctypes.c_uint32], d),
        "orc_decode_f16": ([ctypes.c_uint16], d),
        "orc_decode_bf16": ([ctypes.c_uint16], d),
        "orc_decode_e2m1": ([ctypes.c_uint8], d),
        "orc_decode_e8m0": ([ctypes.c_uint8], d),
        "orc_decode_e4m3": ([ctypes.c_uint8], d),
        "orc_encode_f32": ([d], ctypes.c_uint32),
        "orc_encode_f16": ([d], ctypes.c_uint16),
        "orc_encode_bf16": ([d], ctypes.c_uint16),
        "orc_decode_array": ([ctypes.c_int, i64, p, p], None),
        "orc_encode_array": ([ctypes.c_int, i64, p, p], None),
        "orc_gemm_f64": ([i64, i64, i64, ctypes.c_int, p, p, ctypes.c_int, p], ctypes.c_int),
        "orc_gemm_entries_f64": ([i64, i64, i64, ctypes.c_int, p, p, ctypes.c_int, i64, p, p,
                                  p], None),
        "orc_gemm_layout_f64": ([i64, i64, i64, ctypes.c_int, p, ctypes.c_int, p, ctypes.c_int,
                                 ctypes.c_int, p], ctypes.c_int),
        "orc_gemm_layout_entries_f64": ([i64, i64, i64, ctypes.c_int, p, ctypes.c_int, p,
                                         ctypes.c_int, ctypes.c_int, i64, p, p, p], None),
        "orc_w4_decode": ([i64, i64, p, p, p], None),
        "orc_dequant_w4_f64": ([i64, i64, i64, p, p, p, ctypes.c_int, p], ctypes.c_int),
        "orc_dequant_w4_entries_f64": ([i64, i64, i64, p, p, p, ctypes.c_int, i64, p, p, p],
                                       None),
        "orc_mx_decode_a": ([i64, i64, ctypes.c_int, p, p, p], None),
        "orc_mx_gemm_f64": ([i64, i64, i64, ctypes.c_int, p, p, p, p, ctypes.c_int, p],
                            ctypes.c_int),
        "orc_mx_gemm_entries_f64": ([i64, i64, i64, ctypes.c_int, p, p, p, p, ctypes.c_int, i64,
                                     p, p, p], None),
        "orc_sp24_densify": ([i64, i64, ctypes.c_int, p, p, p], None),
        "orc_gemm_sp24_f64": ([i64, i64, i64, ctypes.c_int, p, p, p, ctypes.c_int, p],
                              ctypes.c_int),
        "orc_gemm_sp24_entries_f64": ([i64, i64, i64, ctypes.c_int, p, p, p, ctypes.c_int, i64,
                                       p, p, p], None),
        "orc_num_threads": ([], ctypes.c_int),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _bits(x, dtype: int) -> np.ndarray:
    """View an input array as the raw storage words of `dtype` (no conversion)."""
    x = np.ascontiguousarray(x)
    want = _NP_STORAGE[dtype]
    if x.dtype == want:
        return x
    if dtype == F32 and x.dtype == np.float32:
        return x.view(np.uint32)
    if dtype == F16 and x.dtype == np.float16:
        return x.view(np.uint16)
    raise TypeError("array of dtype %s is not storage for oracle dtype %d" % (x.dtype, dtype))


class Oracle:
    """The oracle functions bound to one compiled copy of oracle.c."""

    def __init__(self, lib_path: str):
        self.path = lib_path
        self.lib = _bind(ctypes.CDLL(lib_path))

    def num_threads(self) -> int:
        return int(self.lib.orc_num_threads())

    # -- codecs (field-level definitions; see oracle.c) ---------------------
    def decode(self, dtype: int, bits) -> np.ndarray:
        """Storage words of fp32 / fp16 / bf16 -> exact float64."""
        b = _bits(np.asarray(bits), dtype)
        out = np.empty(b.shape, dtype=np.float64)
        self.lib.orc_decode_array(dtype, b.size, _ptr(b), _ptr(out))
        return out

    def encode(self, dtype: int, y) -> np.ndarray:
        """float64 -> storage words of the output type, one round-to-nearest-even."""
        y = np.ascontiguousarray(y, dtype=np.float64)
        out = np.empty(y.shape, dtype=_NP_STORAGE[dtype])
        self.lib.orc_encode_array(dtype, y.size, _ptr(y), _ptr(out))
        return out

    def decode_e2m1(self, code: int) -> float:
        return float(self.lib.orc_decode_e2m1(code))

    def decode_e8m0(self, e: int) -> float:
        return float(self.lib.orc_decode_e8m0(e))

    def decode_e4m3(self, code: int) -> float:
        return float(self.lib.orc_decode_e4m3(code))

    # -- GEMM ---------------------------------------------------------------
    def gemm_f64(self, A, B, dtype: int, relu: bool = False) -> np.ndarray:
        """Y = epi(A @ B) in fp64 for row-major A [M, K], B [K, N] given as storage words."""
        a, b = _bits(A, dtype), _bits(B, dtype)
        M, K = a.shape
        K2, N = b.shape
        if K != K2:
            raise ValueError("inner dimensions differ: %d vs %d" % (K, K2))
        Y = np.empty((M, N), dtype=np.float64)
        rc = self.lib.orc_gemm_f64(M, N, K, dtype, _ptr(a), _ptr(b), int(bool(relu)), _ptr(Y))
        if rc != 0:
            raise MemoryError("oracle allocation failed")
        return Y

    def gemm_entries_f64(self, A, B, dtype: int, rows, cols, relu: bool = False) -> np.ndarray:
        """Selected entries of epi(A @ B), each summed one by one in fp64."""
        a, b = _bits(A, dtype), _bits(B, dtype)
        M, K = a.shape
        K2, N = b.shape
        if K != K2:
            raise ValueError("inner dimensions differ: %d vs %d" % (K, K2))
        r = np.ascontiguousarray(rows, dtype=np.int64)
        c = np.ascontiguousarray(cols, dtype=np.int64)
        if r.shape != c.shape:
            raise ValueError("rows and cols differ in length")
        if r.size and (r.min() < 0 or r.max() >= M or c.min() < 0 or c.max() >= N):
            raise IndexError("entry outside the output")
        out = np.empty(r.shape, dtype=np.float64)
        self.lib.orc_gemm_entries_f64(M, N, K, dtype, _ptr(a), _ptr(b), int(bool(relu)),
                                      r.size, _ptr(r), _ptr(c), _ptr(out))
        return out

    # -- operands stored transposed -------------------------------------------
    @staticmethod
    def _layout_dims(a, ta, b, tb):
        K, M = a.shape if ta else (a.shape[1], a.shape[0])
        N, K2 = b.shape if tb else (b.shape[1], b.shape[0])
        if K != K2:
            raise ValueError("inner dimensions differ: %d vs %d" % (K, K2))
        return M, N, K

    def gemm_layout_f64(self, A, trans_a, B, trans_b, dtype: int, relu: bool = False) -> np.ndarray:
        """Y = epi(op(A) @ op(B)) in fp64: A stored [M, K] or (trans_a) [K, M],
        B stored [K, N] or (trans_b) [N, K], as storage words."""
        a, b = _bits(A, dtype), _bits(B, dtype)
        M, N, K = self._layout_dims(a, trans_a, b, trans_b)
        Y = np.empty((M, N), dtype=np.float64)
        rc = self.lib.orc_gemm_layout_f64(M, N, K, dtype, _ptr(a), int(bool(trans_a)), _ptr(b),
                                          int(bool(trans_b)), int(bool(relu)), _ptr(Y))
        if rc != 0:
            raise MemoryError("oracle allocation failed")
        return Y

    def gemm_layout_entries_f64(self, A, trans_a, B, trans_b, dtype: int, rows, cols,
                                relu: bool = False) -> np.ndarray:
        """Selected entries of epi(op(A) @ op(B)), each summed one by one in fp64."""
        a, b = _bits(A, dtype), _bits(B, dtype)
        M, N, K = self._layout_dims(a, trans_a, b, trans_b)
        r = np.ascontiguousarray(rows, dtype=np.int64)
        c = np.ascontiguousarray(cols, dtype=np.int64)
        if r.shape != c.shape:
            raise ValueError("rows and cols differ in length")
        if r.size and (r.min() < 0 or r.max() >= M or c.min() < 0 or c.max() >= N):
            raise IndexError("entry outside the output")
        out = np.empty(r.shape, dtype=np.float64)
        self.lib.orc_gemm_layout_entries_f64(M, N, K, dtype, _ptr(a), int(bool(trans_a)), _ptr(b),
                                             int(bool(trans_b)), int(bool(relu)), r.size, _ptr(r),
                                             _ptr(c), _ptr(out))
        return out

    # -- weight-only 4-bit dequant GEMM ---------------------------------------
    @staticmethod
    def _w4_check(A, Wq, Ws):
        a = _bits(A, BF16)
        wq = np.ascontiguousarray(Wq, dtype=np.uint8)
        ws = np.ascontiguousarray(Ws, dtype=np.uint8)
        M, K = a.shape
        N = wq.shape[0]
        if K % 32 != 0:
            raise ValueError("K must be a multiple of 32")
        if wq.shape != (N, K // 2) or ws.shape != (N, K // 32):
            raise ValueError("packed weight / scale shapes do not match [N, K/2] / [N, K/32]")
        return a, wq, ws, M, N, K

    def w4_decode(self, Wq, Ws) -> np.ndarray:
        """Packed e2m1 codes [N, K/2] and e8m0 scales [N, K/32] -> W [N, K] fp64."""
        wq = np.ascontiguousarray(Wq, dtype=np.uint8)
        ws = np.ascontiguousarray(Ws, dtype=np.uint8)
        N, half = wq.shape
        K = 2 * half
        if ws.shape != (N, K // 32):
            raise ValueError("scale shape does not match [N, K/32]")
        W = np.empty((N, K), dtype=np.float64)
        self.lib.orc_w4_decode(N, K, _ptr(wq), _ptr(ws), _ptr(W))
        return W

    def dequant_w4_f64(self, A, Wq, Ws, relu: bool = False) -> np.ndarray:
        """Y[m, n] = epi(sum_k A[m, k] * W[n, k]) in fp64, A bf16 storage words."""
        a, wq, ws, M, N, K = self._w4_check(A, Wq, Ws)
        Y = np.empty((M, N), dtype=np.float64)
        rc = self.lib.orc_dequant_w4_f64(M, N, K, _ptr(a), _ptr(wq), _ptr(ws),
                                         int(bool(relu)), _ptr(Y))
        if rc != 0:
            raise MemoryError("oracle allocation failed")
        return Y

    def dequant_w4_entries_f64(self, A, Wq, Ws, rows, cols, relu: bool = False) -> np.ndarray:
        """Selected entries of the dequant GEMM, each summed one by one in fp64."""
        a, wq, ws, M, N, K = self._w4_check(A, Wq, Ws)
        r = np.ascontiguousarray(rows, dtype=np.int64)
        c = np.ascontiguousarray(cols, dtype=np.int64)
        if r.shape != c.shape:
            raise ValueError("rows and cols differ in length")
        if r.size and (r.min() < 0 or r.max() >= M or c.min() < 0 or c.max() >= N):
            raise IndexError("entry outside the output")
        out = np.empty(r.shape, dtype=np.float64)
        self.lib.orc_dequant_w4_entries_f64(M, N, K, _ptr(a), _ptr(wq), _ptr(ws),
                                            int(bool(relu)), r.size, _ptr(r), _ptr(c),
                                            _ptr(out))
        return out

    # -- MX-format GEMM ---------------------------------------------------------
    MX_E2M1, MX_E4M3 = 0, 1

    @staticmethod
    def _mx_check(fmt, Aq, As, Wq, Ws):
        if fmt not in (0, 1):
            raise ValueError("activation format must be 0 (E2M1) or 1 (E4M3)")
        aq = np.ascontiguousarray(Aq, dtype=np.uint8)
        a_s = np.ascontiguousarray(As, dtype=np.uint8)
        wq = np.ascontiguousarray(Wq, dtype=np.uint8)
        ws = np.ascontiguousarray(Ws, dtype=np.uint8)
        M = aq.shape[0]
        K = aq.shape[1] * (2 if fmt == 0 else 1)
        N = wq.shape[0]
        if K % 32 != 0:
            raise ValueError("K must be a multiple of 32")
        if a_s.shape != (M, K // 32):
            raise ValueError("activation scale shape does not match [M, K/32]")
        if wq.shape != (N, K // 2) or ws.shape != (N, K // 32):
            raise ValueError("packed weight / scale shapes do not match [N, K/2] / [N, K/32]")
        return aq, a_s, wq, ws, M, N, K

    def mx_decode_a(self, fmt: int, Aq, As) -> np.ndarray:
        """Activation codes ([M, K/2] E2M1 or [M, K] E4M3) and E8M0 scales [M, K/32]
        -> a [M, K] fp64."""
        aq = np.ascontiguousarray(Aq, dtype=np.uint8)
        a_s = np.ascontiguousarray(As, dtype=np.uint8)
        M = aq.shape[0]
        K = aq.shape[1] * (2 if fmt == 0 else 1)
        if a_s.shape != (M, K // 32):
            raise ValueError("activation scale shape does not match [M, K/32]")
        out = np.empty((M, K), dtype=np.float64)
        self.lib.orc_mx_decode_a(M, K, int(fmt), _ptr(aq), _ptr(a_s), _ptr(out))
        return out

    def mx_gemm_f64(self, fmt: int, Aq, As, Wq, Ws, relu: bool = False) -> np.ndarray:
        """Y[m, n] = epi(sum_k a(m, k) * w(n, k)) in fp64 (MX blocks on both operands)."""
        aq, a_s, wq, ws, M, N, K = self._mx_check(fmt, Aq, As, Wq, Ws)
        Y = np.empty((M, N), dtype=np.float64)
        rc = self.lib.orc_mx_gemm_f64(M, N, K, int(fmt), _ptr(aq), _ptr(a_s), _ptr(wq), _ptr(ws),
                                      int(bool(relu)), _ptr(Y))
        if rc != 0:
            raise MemoryError("oracle allocation failed")
        return Y

    def mx_gemm_entries_f64(self, fmt: int, Aq, As, Wq, Ws, rows, cols,
                            relu: bool = False) -> np.ndarray:
        """Selected entries of the MX-format GEMM, each summed one by one in fp64."""
        aq, a_s, wq, ws, M, N, K = self._mx_check(fmt, Aq, As, Wq, Ws)
        r = np.ascontiguousarray(rows, dtype=np.int64)
        c = np.ascontiguousarray(cols, dtype=np.int64)
        if r.shape != c.shape:
            raise ValueError("rows and cols differ in length")
        if r.size and (r.min() < 0 or r.max() >= M or c.min() < 0 or c.max() >= N):
            raise IndexError("entry outside the output")
        out = np.empty(r.shape, dtype=np.float64)
        self.lib.orc_mx_gemm_entries_f64(M, N, K, int(fmt), _ptr(aq), _ptr(a_s), _ptr(wq),
                                         _ptr(ws), int(bool(relu)), r.size, _ptr(r), _ptr(c),
                                         _ptr(out))
        return out

    # -- 2:4 structured-sparse GEMM ------------------------------------------------
    @staticmethod
    def _sp24_check(Ac, Ai, B, dtype):
        ac = _bits(Ac, dtype)
        ai = np.ascontiguousarray(Ai, dtype=np.uint8)
        b = _bits(B, dtype)
        M, half = ac.shape
        K = 2 * half
        K2, N = b.shape
        if K != K2:
            raise ValueError("inner dimensions differ: %d vs %d" % (K, K2))
        if K % 8 != 0:
            raise ValueError("K must be a multiple of 8")
        if ai.shape != (M, K // 8):
            raise ValueError("metadata shape does not match [M, K/8]")
        return ac, ai, b, M, N, K

    def sp24_densify(self, Ac, Ai, dtype: int) -> np.ndarray:
        """Compressed values [M, K/2] and metadata [M, K/8] -> dense A [M, K] fp64."""
        ac = _bits(Ac, dtype)
        ai = np.ascontiguousarray(Ai, dtype=np.uint8)
        M, half = ac.shape
        K = 2 * half
        if ai.shape != (M, K // 8):
            raise ValueError("metadata shape does not match [M, K/8]")
        out = np.empty((M, K), dtype=np.float64)
        self.lib.orc_sp24_densify(M, K, dtype, _ptr(ac), _ptr(ai), _ptr(out))
        return out

    def gemm_sp24_f64(self, Ac, Ai, B, dtype: int, relu: bool = False) -> np.ndarray:
        """Y = epi(A_sparse @ B) in fp64 with A given in compressed 2:4 form."""
        ac, ai, b, M, N, K = self._sp24_check(Ac, Ai, B, dtype)
        Y = np.empty((M, N), dtype=np.float64)
        rc = self.lib.orc_gemm_sp24_f64(M, N, K, dtype, _ptr(ac), _ptr(ai), _ptr(b),
                                        int(bool(relu)), _ptr(Y))
        if rc != 0:
            raise MemoryError("oracle allocation failed")
        return Y

    def gemm_sp24_entries_f64(self, Ac, Ai, B, dtype: int, rows, cols,
                              relu: bool = False) -> np.ndarray:
        """Selected entries, summed one by one from the compressed form."""
        ac, ai, b, M, N, K = self._sp24_check(Ac, Ai, B, dtype)
        r = np.ascontiguousarray(rows, dtype=np.int64)
        c = np.ascontiguousarray(cols, dtype=np.int64)
        if r.shape != c.shape:
            raise ValueError("rows and cols differ in length")
        if r.size and (r.min() < 0 or r.max() >= M or c.min() < 0 or c.max() >= N):
            raise IndexError("entry outside the output")
        out = np.empty(r.shape, dtype=np.float64)
        self.lib.orc_gemm_sp24_entries_f64(M, N, K, dtype, _ptr(ac), _ptr(ai), _ptr(b),
                                           int(bool(relu)), r.size, _ptr(r), _ptr(c), _ptr(out))
        return out


_default = None


def default() -> Oracle:
    """The oracle built from oracle.c in this directory (built on first use if absent)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB_PATH):
            build(force=True)
        _default = Oracle(LIB_PATH)
    return _default


def num_threads() -> int:
    return default().num_threads()


def decode(dtype, bits):
    return default().decode(dtype, bits)


def encode(dtype, y):
    return default().encode(dtype, y)


def decode_e2m1(code):
    return default().decode_e2m1(code)


def decode_e8m0(e):
    return default().decode_e8m0(e)


def gemm_f64(A, B, dtype, relu=False):
    return default().gemm_f64(A, B, dtype, relu)


def gemm_entries_f64(A, B, dtype, rows, cols, relu=False):
    return default().gemm_entries_f64(A, B, dtype, rows, cols, relu)


def gemm_layout_f64(A, trans_a, B, trans_b, dtype, relu=False):
    return default().gemm_layout_f64(A, trans_a, B, trans_b, dtype, relu)


def gemm_layout_entries_f64(A, trans_a, B, trans_b, dtype, rows, cols, relu=False):
    return default().gemm_layout_entries_f64(A, trans_a, B, trans_b, dtype, rows, cols, relu)


def w4_decode(Wq, Ws):
    return default().w4_decode(Wq, Ws)


def dequant_w4_f64(A, Wq, Ws, relu=False):
    return default().dequant_w4_f64(A, Wq, Ws, relu)


def dequant_w4_entries_f64(A, Wq, Ws, rows, cols, relu=False):
    return default().dequant_w4_entries_f64(A, Wq, Ws, rows, cols, relu)


def decode_e4m3(code):
    return default().decode_e4m3(code)


def mx_decode_a(fmt, Aq, As):
    return default().mx_decode_a(fmt, Aq, As)


def mx_gemm_f64(fmt, Aq, As, Wq, Ws, relu=False):
    return default().mx_gemm_f64(fmt, Aq, As, Wq, Ws, relu)


def mx_gemm_entries_f64(fmt, Aq, As, Wq, Ws, rows, cols, relu=False):
    return default().mx_gemm_entries_f64(fmt, Aq, As, Wq, Ws, rows, cols, relu)


def sp24_densify(Ac, Ai, dtype):
    return default().sp24_densify(Ac, Ai, dtype)


def gemm_sp24_f64(Ac, Ai, B, dtype, relu=False):
    return default().gemm_sp24_f64(Ac, Ai, B, dtype, relu)


def gemm_sp24_entries_f64(Ac, Ai, B, dtype, rows, cols, relu=False):
    return default().gemm_sp24_entries_f64(Ac, Ai, B, dtype, rows, cols, relu)
