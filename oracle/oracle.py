"""ctypes front end of the CPU oracle (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` use this module.  It loads ``oracle/liboracle.so`` (built from
``tlg_oracle.c`` by ``oracle/build_oracle.py``) and works on numpy arrays of raw
bit patterns, so it never touches the HIP library or its Python binding.

Parity unpinned: NaN/Inf propagation (no workload produces them).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

F16, BF16, F32 = 1, 2, 3
DTYPE_CODES = {"f16": F16, "bf16": BF16, "f32": F32}


class Oracle:
    """One loaded copy of the oracle library (tests may load a rebuilt copy from another path)."""

    def __init__(self, lib_path: str = LIB_PATH):
        if not os.path.exists(lib_path):
            raise RuntimeError(f"oracle library missing: {lib_path} (run oracle/build_oracle.py)")
        lib = ctypes.CDLL(lib_path)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        lib.oracle_gemm_rows.argtypes = [i64, i64, i64, i32, i32, i32, i32, i32, i32,
                                         vp, vp, vp, i64, i64, vp, i32]
        lib.oracle_gemm_rows.restype = i32
        lib.oracle_gemm_points.argtypes = [i64, i64, i64, i32, i32, i32, i32, i32, i32,
                                           vp, vp, vp, i64, vp, vp, vp]
        lib.oracle_gemm_points.restype = i32
        lib.oracle_decode.argtypes = [i32, vp, i64, vp]
        lib.oracle_decode.restype = i32
        lib.oracle_encode.argtypes = [i32, vp, i64, vp]
        lib.oracle_encode.restype = i32
        lib.oracle_mxgemm_rows.argtypes = [i64, i64, i64, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp,
                                           i64, i64, vp, i32]
        lib.oracle_mxgemm_rows.restype = i32
        lib.oracle_mxgemm_points.argtypes = [i64, i64, i64, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp,
                                             i64, vp, vp, vp]
        lib.oracle_mxgemm_points.restype = i32
        lib.oracle_mx_decode.argtypes = [i32, vp, i64, vp]
        lib.oracle_mx_decode.restype = i32
        f64 = ctypes.c_double
        lib.oracle_sp_expand.argtypes = [i64, i64, i32, vp, vp, vp]
        lib.oracle_sp_expand.restype = i32
        lib.oracle_spgemm_rows.argtypes = [i64, i64, i64, i32, i32, vp, vp, vp, i64, i64, vp]
        lib.oracle_spgemm_rows.restype = i32
        lib.oracle_spgemm_points.argtypes = [i64, i64, i64, i32, i32, vp, vp, vp, i64, vp, vp, vp]
        lib.oracle_spgemm_points.restype = i32
        lib.oracle_w4_dequant.argtypes = [i64, i64, i64, i32, vp, vp, vp, vp]
        lib.oracle_w4_dequant.restype = i32
        lib.oracle_w4gemm_rows.argtypes = [i64, i64, i64, i64, i32, i32, vp, vp, vp, vp, i64, i64, vp]
        lib.oracle_w4gemm_rows.restype = i32
        lib.oracle_w4gemm_points.argtypes = [i64, i64, i64, i64, i32, i32, vp, vp, vp, vp, i64, vp, vp, vp]
        lib.oracle_w4gemm_points.restype = i32
        lib.oracle_attn_rows.argtypes = [i64, i64, i64, i64, i32, i32, f64, vp, vp, vp, i64, i64, vp, i32]
        lib.oracle_attn_rows.restype = i32
        lib.oracle_attn_points.argtypes = [i64, i64, i64, i64, i32, i32, f64, vp, vp, vp, i64, vp, vp, vp, vp]
        lib.oracle_attn_points.restype = i32
        self.lib = lib
        self.path = lib_path

    def gemm(self, M, N, K, A_bits, B_bits, *, ab="f16", c="f16", transpose_A=0, transpose_B=0,
             clear_accum=1, relu=0, C_in_bits=None, rows=None, nthreads=None) -> np.ndarray:
        """Oracle value o(m, n) in float64 for the rows ``rows=(m0, m1)`` (default: all)."""
        A, B, C = _u16(A_bits), _u16(B_bits), _cin(C_in_bits, c)
        m0, m1 = (0, M) if rows is None else rows
        out = np.empty((m1 - m0, N), dtype=np.float64)
        nt = nthreads if nthreads is not None else min(os.cpu_count() or 1, 16)
        rc = self.lib.oracle_gemm_rows(M, N, K, _code(ab), _code(c), int(transpose_A),
                                       int(transpose_B), int(clear_accum), int(relu),
                                       _ptr(A), _ptr(B), _ptr(C), m0, m1, out.ctypes.data, int(nt))
        if rc != 0:
            raise ValueError(f"oracle_gemm_rows failed with {rc}")
        return out

    def gemm_points(self, M, N, K, A_bits, B_bits, ms, ns, *, ab="f16", c="f16", transpose_A=0,
                    transpose_B=0, clear_accum=1, relu=0, C_in_bits=None) -> np.ndarray:
        """Oracle value at the coordinates (ms[i], ns[i])."""
        A, B, C = _u16(A_bits), _u16(B_bits), _cin(C_in_bits, c)
        ms = np.ascontiguousarray(ms, dtype=np.int64)
        ns = np.ascontiguousarray(ns, dtype=np.int64)
        out = np.empty(ms.shape[0], dtype=np.float64)
        rc = self.lib.oracle_gemm_points(M, N, K, _code(ab), _code(c), int(transpose_A),
                                         int(transpose_B), int(clear_accum), int(relu),
                                         _ptr(A), _ptr(B), _ptr(C), ms.shape[0],
                                         ms.ctypes.data, ns.ctypes.data, out.ctypes.data)
        if rc != 0:
            raise ValueError(f"oracle_gemm_points failed with {rc}")
        return out

    def mxgemm(self, M, N, K, A, SA, B, SB, *, fmt_a="e4m3", fmt_b="e4m3", c="f16", clear_accum=1, relu=0,
               C_in_bits=None, rows=None, nthreads=None) -> np.ndarray:
        """Block-scaled GEMM oracle o(m, n) in float64 (A uint8 [M,K], SA uint8 [M,K/32],
        B uint8 [N,K], SB uint8 [N,K/32]) for the rows ``rows=(m0, m1)`` (default: all)."""
        A, SA, B, SB = _u8(A), _u8(SA), _u8(B), _u8(SB)
        C = _cin(C_in_bits, c)
        m0, m1 = (0, M) if rows is None else rows
        out = np.empty((m1 - m0, N), dtype=np.float64)
        nt = nthreads if nthreads is not None else min(os.cpu_count() or 1, 16)
        rc = self.lib.oracle_mxgemm_rows(M, N, K, MX_CODES[fmt_a], MX_CODES[fmt_b], _code(c), int(clear_accum),
                                         int(relu), _ptr(A), _ptr(SA), _ptr(B), _ptr(SB), _ptr(C), m0, m1,
                                         out.ctypes.data, int(nt))
        if rc != 0:
            raise ValueError(f"oracle_mxgemm_rows failed with {rc}")
        return out

    def mxgemm_points(self, M, N, K, A, SA, B, SB, ms, ns, *, fmt_a="e4m3", fmt_b="e4m3", c="f16",
                      clear_accum=1, relu=0, C_in_bits=None) -> np.ndarray:
        A, SA, B, SB = _u8(A), _u8(SA), _u8(B), _u8(SB)
        C = _cin(C_in_bits, c)
        ms = np.ascontiguousarray(ms, dtype=np.int64)
        ns = np.ascontiguousarray(ns, dtype=np.int64)
        out = np.empty(ms.shape[0], dtype=np.float64)
        rc = self.lib.oracle_mxgemm_points(M, N, K, MX_CODES[fmt_a], MX_CODES[fmt_b], _code(c),
                                           int(clear_accum), int(relu), _ptr(A), _ptr(SA), _ptr(B), _ptr(SB),
                                           _ptr(C), ms.shape[0], ms.ctypes.data, ns.ctypes.data,
                                           out.ctypes.data)
        if rc != 0:
            raise ValueError(f"oracle_mxgemm_points failed with {rc}")
        return out

    def attn(self, B, S, H, D, Q_bits, K_bits, V_bits, *, dtype="f16", causal=1, scale=None, rows=None,
             nthreads=None) -> np.ndarray:
        """Attention forward o(b, i, h, :) in float64, operands [B, S, H, D] as uint16 bits, for the
        query positions ``rows=(i0, i1)`` (default: all); the result is [B, i1-i0, H, D]."""
        Q, K, V = _u16(Q_bits), _u16(K_bits), _u16(V_bits)
        i0, i1 = (0, S) if rows is None else rows
        out = np.empty((B, i1 - i0, H, D), dtype=np.float64)
        sc = 1.0 / np.sqrt(D) if scale is None else float(scale)
        nt = nthreads if nthreads is not None else min(os.cpu_count() or 1, 16)
        rc = self.lib.oracle_attn_rows(B, S, H, D, _code(dtype), int(causal), sc, _ptr(Q), _ptr(K), _ptr(V),
                                       i0, i1, out.ctypes.data, int(nt))
        if rc != 0:
            raise ValueError(f"oracle_attn_rows failed with {rc}")
        return out

    def attn_points(self, B, S, H, D, Q_bits, K_bits, V_bits, pb, pi, ph, *, dtype="f16", causal=1,
                    scale=None) -> np.ndarray:
        """Output rows o(pb[n], pi[n], ph[n], :) as an [n, D] float64 array."""
        Q, K, V = _u16(Q_bits), _u16(K_bits), _u16(V_bits)
        pb, pi, ph = (np.ascontiguousarray(x, dtype=np.int64) for x in (pb, pi, ph))
        out = np.empty((pb.shape[0], D), dtype=np.float64)
        sc = 1.0 / np.sqrt(D) if scale is None else float(scale)
        rc = self.lib.oracle_attn_points(B, S, H, D, _code(dtype), int(causal), sc, _ptr(Q), _ptr(K), _ptr(V),
                                         pb.shape[0], pb.ctypes.data, pi.ctypes.data, ph.ctypes.data,
                                         out.ctypes.data)
        if rc != 0:
            raise ValueError(f"oracle_attn_points failed with {rc}")
        return out

    def sp_expand(self, N, K, Wv_bits, Wm, *, dtype="f16") -> np.ndarray:
        """Dense weights w(n, k) of a 2:4 compressed [N, K] operand, float64."""
        Wv, Wm = _u16(Wv_bits), _u8(Wm)
        out = np.empty((N, K), dtype=np.float64)
        if self.lib.oracle_sp_expand(N, K, _code(dtype), _ptr(Wv), _ptr(Wm), out.ctypes.data) != 0:
            raise ValueError("oracle_sp_expand failed")
        return out

    def spgemm(self, M, N, K, A_bits, Wv_bits, Wm, *, dtype="f16", relu=0, rows=None,
               nthreads=1) -> np.ndarray:
        """2:4 sparse GEMM o(m, n) = act(sum_k a(m,k) w(n,k)) in float64 for rows=(m0, m1).
        With nthreads > 1 the rows are cut into that many ranges, each computed by one
        call of the same C routine on its own thread (the calls release the GIL)."""
        A, Wv, Wm = _u16(A_bits), _u16(Wv_bits), _u8(Wm)
        m0, m1 = (0, M) if rows is None else rows
        out = np.empty((m1 - m0, N), dtype=np.float64)

        def part(r0, r1):
            return self.lib.oracle_spgemm_rows(M, N, K, _code(dtype), int(relu), _ptr(A), _ptr(Wv), _ptr(Wm),
                                               r0, r1, out.ctypes.data + (r0 - m0) * N * 8)
        for rc in _row_ranges(part, m0, m1, nthreads):
            if rc != 0:
                raise ValueError(f"oracle_spgemm_rows failed with {rc}")
        return out

    def spgemm_points(self, M, N, K, A_bits, Wv_bits, Wm, ms, ns, *, dtype="f16", relu=0) -> np.ndarray:
        A, Wv, Wm = _u16(A_bits), _u16(Wv_bits), _u8(Wm)
        ms = np.ascontiguousarray(ms, dtype=np.int64)
        ns = np.ascontiguousarray(ns, dtype=np.int64)
        out = np.empty(ms.shape[0], dtype=np.float64)
        rc = self.lib.oracle_spgemm_points(M, N, K, _code(dtype), int(relu), _ptr(A), _ptr(Wv), _ptr(Wm),
                                           ms.shape[0], ms.ctypes.data, ns.ctypes.data, out.ctypes.data)
        if rc != 0:
            raise ValueError(f"oracle_spgemm_points failed with {rc}")
        return out

    def w4_dequant(self, N, K, G, Wq, S_bits, Z, *, dtype="f16") -> np.ndarray:
        """Dequantized 4-bit weights w(n, k) as an [N, K] float64 array."""
        Wq, Z, S = _u8(Wq), _u8(Z), _u16(S_bits)
        out = np.empty((N, K), dtype=np.float64)
        rc = self.lib.oracle_w4_dequant(N, K, G, _code(dtype), _ptr(Wq), _ptr(S), _ptr(Z), out.ctypes.data)
        if rc != 0:
            raise ValueError(f"oracle_w4_dequant failed with {rc}")
        return out

    def w4gemm(self, M, N, K, G, A_bits, Wq, S_bits, Z, *, dtype="f16", relu=0, rows=None) -> np.ndarray:
        """Dequant GEMM o(m, n) = act(sum_k a(m,k) w(n,k)) in float64 for rows=(m0, m1) (default all)."""
        A, Wq, Z, S = _u16(A_bits), _u8(Wq), _u8(Z), _u16(S_bits)
        m0, m1 = (0, M) if rows is None else rows
        out = np.empty((m1 - m0, N), dtype=np.float64)
        rc = self.lib.oracle_w4gemm_rows(M, N, K, G, _code(dtype), int(relu), _ptr(A), _ptr(Wq), _ptr(S), _ptr(Z),
                                         m0, m1, out.ctypes.data)
        if rc != 0:
            raise ValueError(f"oracle_w4gemm_rows failed with {rc}")
        return out

    def w4gemm_points(self, M, N, K, G, A_bits, Wq, S_bits, Z, ms, ns, *, dtype="f16", relu=0) -> np.ndarray:
        A, Wq, Z, S = _u16(A_bits), _u8(Wq), _u8(Z), _u16(S_bits)
        ms = np.ascontiguousarray(ms, dtype=np.int64)
        ns = np.ascontiguousarray(ns, dtype=np.int64)
        out = np.empty(ms.shape[0], dtype=np.float64)
        rc = self.lib.oracle_w4gemm_points(M, N, K, G, _code(dtype), int(relu), _ptr(A), _ptr(Wq), _ptr(S), _ptr(Z),
                                           ms.shape[0], ms.ctypes.data, ns.ctypes.data, out.ctypes.data)
        if rc != 0:
            raise ValueError(f"oracle_w4gemm_points failed with {rc}")
        return out

    def mx_decode(self, bytes_, fmt) -> np.ndarray:
        b = np.ascontiguousarray(bytes_).reshape(-1).astype(np.uint8)
        out = np.empty(b.shape[0], dtype=np.float64)
        if self.lib.oracle_mx_decode(MX_CODES[fmt], b.ctypes.data, b.shape[0], out.ctypes.data) != 0:
            raise ValueError("oracle_mx_decode failed")
        return out

    def decode(self, bits, dtype) -> np.ndarray:
        b = np.ascontiguousarray(bits).reshape(-1).astype(np.uint32)
        out = np.empty(b.shape[0], dtype=np.float64)
        rc = self.lib.oracle_decode(_code(dtype), b.ctypes.data, b.shape[0], out.ctypes.data)
        if rc != 0:
            raise ValueError("oracle_decode failed")
        return out

    def encode(self, x, dtype) -> np.ndarray:
        """Round-to-nearest-even encoding of doubles; uint16 for f16/bf16, uint32 for f32."""
        xs = np.ascontiguousarray(x, dtype=np.float64).reshape(-1)
        out = np.empty(xs.shape[0], dtype=np.uint32)
        rc = self.lib.oracle_encode(_code(dtype), xs.ctypes.data, xs.shape[0], out.ctypes.data)
        if rc != 0:
            raise ValueError("oracle_encode failed")
        return out if _code(dtype) == F32 else out.astype(np.uint16)

    def rne_out(self, x, dtype) -> np.ndarray:
        """Oracle value rounded to the output dtype and decoded back to float64."""
        return self.decode(self.encode(x, dtype), dtype)


MX_CODES = {"e4m3": 10, "e5m2": 11, "e8m0": 12, "e2m1": 13}


def _row_ranges(part, m0, m1, nthreads):
    """Run part(r0, r1) over nthreads contiguous ranges of [m0, m1); returns the results."""
    n = max(1, min(int(nthreads), m1 - m0))
    if n == 1:
        return [part(m0, m1)]
    import concurrent.futures as cf
    bounds = [m0 + (m1 - m0) * i // n for i in range(n + 1)]
    with cf.ThreadPoolExecutor(max_workers=n) as ex:
        return list(ex.map(lambda i: part(bounds[i], bounds[i + 1]), range(n)))


def _u8(x):
    if x is None:
        return None
    a = np.ascontiguousarray(x)
    if a.dtype != np.uint8:
        raise TypeError(f"block-scaled operands and scales are uint8, got {a.dtype}")
    return a.reshape(-1)


def _code(d):
    return DTYPE_CODES[d] if isinstance(d, str) else int(d)


def _u16(x):
    if x is None:
        return None
    a = np.ascontiguousarray(x)
    if a.dtype != np.uint16:
        raise TypeError(f"operand bits must be uint16, got {a.dtype}")
    return a.reshape(-1)


def _cin(x, c_dtype):
    if x is None:
        return None
    a = np.ascontiguousarray(x).reshape(-1)
    want = np.uint32 if _code(c_dtype) == F32 else np.uint16
    if a.dtype != want:
        raise TypeError(f"C_in bits must be {want.__name__}, got {a.dtype}")
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle(LIB_PATH)
    return _default


def gemm(*args, **kw):
    return default().gemm(*args, **kw)


def gemm_points(*args, **kw):
    return default().gemm_points(*args, **kw)


def decode(bits, dtype):
    return default().decode(bits, dtype)


def mxgemm(*args, **kw):
    return default().mxgemm(*args, **kw)


def mxgemm_points(*args, **kw):
    return default().mxgemm_points(*args, **kw)


def attn(*args, **kw):
    return default().attn(*args, **kw)


def attn_points(*args, **kw):
    return default().attn_points(*args, **kw)


def sp_expand(*args, **kw):
    return default().sp_expand(*args, **kw)


def spgemm(*args, **kw):
    return default().spgemm(*args, **kw)


def spgemm_points(*args, **kw):
    return default().spgemm_points(*args, **kw)


def w4_dequant(*args, **kw):
    return default().w4_dequant(*args, **kw)


def w4gemm(*args, **kw):
    return default().w4gemm(*args, **kw)


def w4gemm_points(*args, **kw):
    return default().w4gemm_points(*args, **kw)


def attn_tolerance(o: np.ndarray, vmax: float, dtype="f16") -> np.ndarray:
    """Per-element bound for the attention forward:
    |gpu - o| <= 2u (|o| + max|V|) + 1e-5, u the unit roundoff of the operand type
    (2^-11 for fp16, 2^-8 for bf16).  The probabilities are rounded to the operand
    type before the second product (relative error <= u each, so <= u max|V| on
    the weighted sum of V rows), the normaliser may use unrounded or rounded
    probabilities (<= u |o|) and the output is rounded once (<= u |o|); the fp32
    scores, exponentials and sums add far less than 1e-5 for the workloads'
    magnitudes."""
    u = 2.0 ** -8 if _code(dtype) == BF16 else 2.0 ** -11
    return 2.0 * u * (np.abs(o) + vmax) + 1e-5


def encode(x, dtype):
    return default().encode(x, dtype)


def rne_out(x, dtype):
    return default().rne_out(x, dtype)


def tolerance(o: np.ndarray, K: int, c_dtype="f16") -> np.ndarray:
    """Per-element bound |gpu - o| <= 2^-10 |o| + 1e-4 sqrt(K) (inputs in [-1, 1]).

    2^-10 is twice the relative half-ulp (2^-11) of the fp16 output cast, which
    leaves room for the fp32 accumulation; fp32 output uses the same bound.
    bf16 output rounds with a relative half-ulp of 2^-9, so its relative term is
    2^-8 (a reading: the stated bound is for fp16/fp32 outputs)."""
    rel = 2.0 ** -8 if _code(c_dtype) == BF16 else 2.0 ** -10
    return rel * np.abs(o) + 1e-4 * np.sqrt(max(K, 1))
