"""tlg — tiled, software-pipelined dense GEMM C = act(A·B) on AMD MI355X (gfx950).

Thin ctypes binding over the C-ABI of ``libtlg.so`` (declared in include/tlg.h).
It only marshals arguments: PyTorch provides device buffers and the current
stream; every step of the computation runs in the library's HIP kernels.  If
the library is not built, every call raises: there is no fallback.
"""
from __future__ import annotations

import contextlib
import ctypes
import math
import os
import threading

import torch

__all__ = ["Gemm", "gemm", "gemm_mx", "gemm_noalloc", "select", "tune", "PlanInfo", "TuneResult", "TlgError", "lib_path", "load_library",
           "status_name", "VARIANTS", "F16", "BF16", "F32", "E4M3", "E5M2", "E2M1"]

_PKG = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_PKG, "libtlg.so")

F16, BF16, F32, E4M3, E5M2, E2M1 = 1, 2, 3, 4, 5, 6
_TORCH_TO_CODE = {torch.float16: F16, torch.bfloat16: BF16, torch.float32: F32,
                  torch.float8_e4m3fn: E4M3, torch.float8_e5m2: E5M2, torch.float4_e2m1fn_x2: E2M1}
VARIANTS = {"auto": 0, "tile256": 1, "tile128": 2, "skinny": 3, "empty": 4, "tile256w8": 5,
            "tile256dma": 6, "tile128dma": 7, "tile128dma_sk": 8, "mx256": 9, "tile64dma": 10, "tile32dma": 13,
            "tile256dma_streamk": 11, "tile128dma_streamk": 12}
EPILOGUES = {"none": 0, "relu": 1}

STATUS = {0: "TLG_OK", -1: "TLG_ERR_INVALID_ARG", -2: "TLG_ERR_UNSUPPORTED", -3: "TLG_ERR_NULL",
          -4: "TLG_ERR_MISALIGNED", -5: "TLG_ERR_HIP", -6: "TLG_ERR_NOMEM", -7: "TLG_ERR_TOO_LARGE"}


class TlgError(RuntimeError):
    def __init__(self, what: str, status: int):
        super().__init__(f"{what}: {STATUS.get(status, status)}")
        self.status = status


def status_name(s: int) -> str:
    return STATUS.get(s, f"unknown({s})")


class PlanInfo(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int32), ("block_m", ctypes.c_int32), ("block_n", ctypes.c_int32),
                ("block_k", ctypes.c_int32), ("stages", ctypes.c_int32), ("threads", ctypes.c_int32),
                ("vec_a", ctypes.c_int32), ("vec_b", ctypes.c_int32), ("grid", ctypes.c_int64),
                ("lds_bytes", ctypes.c_int64), ("k_tiles", ctypes.c_int32), ("splits", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_int64), ("dp_tiles", ctypes.c_int32), ("sk_tiles", ctypes.c_int32)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class TuneResult(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int32), ("splits", ctypes.c_int32), ("ms", ctypes.c_float)]


_lib = None
_lib_lock = threading.Lock()


def load_library():
    """Load libtlg.so from the package directory; raise if it has not been built."""
    global _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(lib_path):
            raise RuntimeError(f"{lib_path} is missing: build it with "
                               f"`python -m tiled_dense_gemm_02_amd.build` (hipcc, gfx950)")
        lib = ctypes.CDLL(lib_path)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        lib.tlg_gemm_create.argtypes = [ctypes.POINTER(vp), i64, i64, i64, i32, i32, i32, i32, i32, i32]
        lib.tlg_gemm_create.restype = i32
        lib.tlg_gemm_create_variant.argtypes = [ctypes.POINTER(vp), i64, i64, i64, i32, i32, i32, i32,
                                                i32, i32, i32]
        lib.tlg_gemm_create_variant.restype = i32
        lib.tlg_gemm_run.argtypes = [vp, vp, vp, vp, vp]
        lib.tlg_gemm_run.restype = i32
        lib.tlg_gemm_run_noalloc.argtypes = [i64, i64, i64, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp]
        lib.tlg_gemm_run_noalloc.restype = i32
        lib.tlg_gemm_run_mx.argtypes = [vp, vp, vp, vp, vp, vp, vp]
        lib.tlg_gemm_run_mx.restype = i32
        lib.tlg_gemm_destroy.argtypes = [vp]
        lib.tlg_gemm_destroy.restype = i32
        lib.tlg_gemm_select.argtypes = [ctypes.POINTER(PlanInfo), i64, i64, i64, i32, i32, i32, i32, i32, i32,
                                        i32]
        lib.tlg_gemm_select.restype = i32
        lib.tlg_gemm_tune.argtypes = [ctypes.POINTER(vp), i64, i64, i64, i32, i32, i32, i32, i32, i32, vp, vp, vp,
                                      vp, i32, ctypes.POINTER(TuneResult), i32, ctypes.POINTER(i32)]
        lib.tlg_gemm_tune.restype = i32
        lib.tlg_attn_fwd.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i32, i32, ctypes.c_float, vp]
        lib.tlg_attn_fwd.restype = i32
        lib.tlg_attn_fwd_block.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i32, i32, ctypes.c_float, i32, vp]
        lib.tlg_attn_fwd_block.restype = i32
        lib.tlg_attn_query_block.argtypes = [i64, i64, i64, i64, i32]
        lib.tlg_attn_query_block.restype = i32
        lib.tlg_gemm_w4.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, i32, i32, vp]
        lib.tlg_gemm_w4.restype = i32
        lib.tlg_gemm_sp.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, vp]
        lib.tlg_gemm_sp.restype = i32
        lib.tlg_gemm_query.argtypes = [vp, ctypes.POINTER(PlanInfo)]
        lib.tlg_gemm_query.restype = i32
        lib.tlg_gemm_describe.argtypes = [vp]
        lib.tlg_gemm_describe.restype = ctypes.c_char_p
        lib.tlg_status_string.argtypes = [i32]
        lib.tlg_status_string.restype = ctypes.c_char_p
        lib.tlg_version.argtypes = []
        lib.tlg_version.restype = ctypes.c_char_p
        _lib = lib
        return lib


def _code(dt) -> int:
    if isinstance(dt, int):
        return dt
    if isinstance(dt, str):
        return {"f16": F16, "bf16": BF16, "f32": F32, "e4m3": E4M3, "e5m2": E5M2, "e2m1": E2M1}[dt]
    return _TORCH_TO_CODE[dt]


def select(M: int, N: int, K: int, ab_dtype=torch.float16, out_dtype=torch.float16, *,
           transpose_A: bool = False, transpose_B: bool = False, clear_accum: bool = True,
           epilogue: str = "none", variant: str = "auto") -> PlanInfo:
    """The plan facts tlg_gemm_create would produce for these arguments (tlg_gemm_select:
    host only, nothing is allocated)."""
    lib = load_library()
    info = PlanInfo()
    st = lib.tlg_gemm_select(ctypes.byref(info), int(M), int(N), int(K), _code(ab_dtype), _code(out_dtype),
                             int(bool(transpose_A)), int(bool(transpose_B)), int(bool(clear_accum)),
                             EPILOGUES[epilogue], VARIANTS[variant])
    if st != 0:
        raise TlgError("tlg_gemm_select", st)
    return info


class Gemm:
    """A plan for C[M,N] = act(A·B) (tlg_gemm_create).  Immutable.  A plan without a
    workspace is reusable on any stream; a split-K plan (info.splits > 1) owns a device
    workspace on the device current at creation, and its runs must not overlap."""

    def __init__(self, M: int, N: int, K: int, ab_dtype=torch.float16, out_dtype=torch.float16, *,
                 transpose_A: bool = False, transpose_B: bool = False, clear_accum: bool = True,
                 epilogue: str = "none", variant: str = "auto", _handle=None):
        lib = load_library()
        self.M, self.N, self.K = int(M), int(N), int(K)
        self.ab_code, self.c_code = _code(ab_dtype), _code(out_dtype)
        self.transpose_A, self.transpose_B = bool(transpose_A), bool(transpose_B)
        self.clear_accum = bool(clear_accum)
        self.epilogue = epilogue
        self._lib = lib
        if _handle is not None:          # a plan made by tlg_gemm_tune
            self._h = _handle
            return
        self._h = ctypes.c_void_p()
        args = (self.M, self.N, self.K, self.ab_code, self.c_code, int(self.transpose_A),
                int(self.transpose_B), int(self.clear_accum), EPILOGUES[epilogue])
        if variant == "auto":
            st = lib.tlg_gemm_create(ctypes.byref(self._h), *args)
        else:
            st = lib.tlg_gemm_create_variant(ctypes.byref(self._h), *args, VARIANTS[variant])
        if st != 0:
            self._h = None
            raise TlgError("tlg_gemm_create", st)
        self._lib = lib

    @property
    def info(self) -> PlanInfo:
        info = PlanInfo()
        st = self._lib.tlg_gemm_query(self._h, ctypes.byref(info))
        if st != 0:
            raise TlgError("tlg_gemm_query", st)
        return info

    def describe(self) -> str:
        return self._lib.tlg_gemm_describe(self._h).decode()

    def _check(self, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor):
        M, N, K = self.M, self.N, self.K
        a_shape = (K, M) if self.transpose_A else (M, K)
        b_shape = (N, K) if self.transpose_B else (K, N)
        for name, t, shape, code in (("A", A, a_shape, self.ab_code), ("B", B, b_shape, self.ab_code),
                                     ("C", C, (M, N), self.c_code)):
            if not isinstance(t, torch.Tensor):
                raise TypeError(f"{name} must be a torch.Tensor")
            if t.device.type != "cuda":
                raise ValueError(f"{name} must be a device tensor, got {t.device}")
            if tuple(t.shape) != tuple(shape):
                raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
            if _TORCH_TO_CODE.get(t.dtype) != code:
                raise ValueError(f"{name} has dtype {t.dtype}, plan expects code {code}")
            if t.numel() and not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous")

    def run(self, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor, stream=None) -> torch.Tensor:
        """Enqueue the GEMM on `stream` (default: torch's current stream).  Returns C."""
        self._check(A, B, C)
        if stream is None:
            stream = torch.cuda.current_stream(C.device)
        s = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
        with torch.cuda.device(C.device):
            st = self._lib.tlg_gemm_run(self._h, A.data_ptr() or None, B.data_ptr() or None,
                                        C.data_ptr() or None, ctypes.c_void_p(s))
        if st != 0:
            raise TlgError("tlg_gemm_run", st)
        return C

    def run_mx(self, A: torch.Tensor, SA: torch.Tensor, B: torch.Tensor, SB: torch.Tensor, C: torch.Tensor,
               stream=None) -> torch.Tensor:
        """Enqueue the block-scaled GEMM (tlg_gemm_run_mx).  A [M,K] and B [N,K] hold FP8 bytes
        (uint8 or the matching float8 dtype), or for E2M1 A [M,K/2] and B [N,K/2] packed FP4
        bytes; SA [M,K/32] and SB [N,K/32] E8M0 bytes."""
        M, N, K = self.M, self.N, self.K
        KE = K // 2 if self.ab_code == E2M1 else K      # bytes per operand row
        for name, t, shape in (("A", A, (M, KE)), ("SA", SA, (M, K // 32)), ("B", B, (N, KE)),
                               ("SB", SB, (N, K // 32)), ("C", C, (M, N))):
            if not isinstance(t, torch.Tensor):
                raise TypeError(f"{name} must be a torch.Tensor")
            if t.device.type != "cuda":
                raise ValueError(f"{name} must be a device tensor, got {t.device}")
            if tuple(t.shape) != shape:
                raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")
            if t.numel() and not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous")
            if name != "C" and t.element_size() != 1:
                raise ValueError(f"{name} must hold one byte per element, got {t.dtype}")
        if _TORCH_TO_CODE.get(C.dtype) != self.c_code:
            raise ValueError(f"C has dtype {C.dtype}, plan expects code {self.c_code}")
        if stream is None:
            stream = torch.cuda.current_stream(C.device)
        s = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
        with torch.cuda.device(C.device):
            st = self._lib.tlg_gemm_run_mx(self._h, A.data_ptr() or None, SA.data_ptr() or None,
                                           B.data_ptr() or None, SB.data_ptr() or None, C.data_ptr() or None,
                                           ctypes.c_void_p(s))
        if st != 0:
            raise TlgError("tlg_gemm_run_mx", st)
        return C

    def run_mx_ptrs(self, a, sa, b, sb, c, stream_handle: int = 0) -> int:
        """Raw-pointer form of run_mx; returns the status."""
        return self._lib.tlg_gemm_run_mx(self._h, a or None, sa or None, b or None, sb or None, c or None,
                                         ctypes.c_void_p(stream_handle))

    def run_ptrs(self, a_ptr: int, b_ptr: int, c_ptr: int, stream_handle: int = 0) -> int:
        """Raw-pointer form of run (no checks beyond the library's own); returns the status."""
        return self._lib.tlg_gemm_run(self._h, a_ptr or None, b_ptr or None, c_ptr or None,
                                      ctypes.c_void_p(stream_handle))

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            self._lib.tlg_gemm_destroy(h)
            self._h = None


def tune(A: torch.Tensor, B: torch.Tensor, C: torch.Tensor, *, transpose_A: bool = False,
         transpose_B: bool = False, clear_accum: bool = True, epilogue: str = "none", iters: int = 10,
         stream=None):
    """Autotuned plan for C = act(A·B) on these device tensors (tlg_gemm_tune): every
    candidate kernel is timed on them (C is overwritten) and the fastest kept; the
    choice is cached per device and problem.  Returns (Gemm, [(variant name, splits,
    ms), ...]) with one entry per candidate timed (empty when the cache answered)."""
    lib = load_library()
    M = A.shape[1] if transpose_A else A.shape[0]
    K = A.shape[0] if transpose_A else A.shape[1]
    N = B.shape[0] if transpose_B else B.shape[1]
    probe = Gemm.__new__(Gemm)
    probe.M, probe.N, probe.K = M, N, K
    probe.ab_code, probe.c_code = _code(A.dtype), _code(C.dtype)
    probe.transpose_A, probe.transpose_B = bool(transpose_A), bool(transpose_B)
    probe._h = None
    probe._check(A, B, C)
    if stream is None:
        stream = torch.cuda.current_stream(C.device)
    s = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    res = (TuneResult * 32)()
    n = ctypes.c_int32(0)
    h = ctypes.c_void_p()
    with torch.cuda.device(C.device):
        st = lib.tlg_gemm_tune(ctypes.byref(h), M, N, K, _code(A.dtype), _code(C.dtype), int(bool(transpose_A)),
                               int(bool(transpose_B)), int(bool(clear_accum)), EPILOGUES[epilogue],
                               A.data_ptr() or None, B.data_ptr() or None, C.data_ptr() or None,
                               ctypes.c_void_p(s), int(iters), res, 32, ctypes.byref(n))
    if st != 0:
        raise TlgError("tlg_gemm_tune", st)
    names = {v: k for k, v in VARIANTS.items()}
    plan = Gemm(M, N, K, A.dtype, C.dtype, transpose_A=transpose_A, transpose_B=transpose_B,
                clear_accum=clear_accum, epilogue=epilogue, _handle=h)
    return plan, [(names.get(r.variant, str(r.variant)), r.splits, r.ms) for r in res[:n.value]]


def gemm_mx(A: torch.Tensor, SA: torch.Tensor, B: torch.Tensor, SB: torch.Tensor, C: torch.Tensor | None = None,
            *, fmt: str = "e4m3", clear_accum: bool = True, epilogue: str = "none",
            out_dtype=torch.float16) -> torch.Tensor:
    """Block-scaled GEMM C = act(A·Bᵀ) with E8M0 scales per 32 of K: FP8 (A [M,K], B [N,K]) or,
    with fmt="e2m1", FP4 packed two per byte (A [M,K/2], B [N,K/2])."""
    M, K = A.shape
    if fmt == "e2m1":
        K *= 2
    N = B.shape[0]
    if C is None:
        if not clear_accum:
            raise ValueError("clear_accum=False needs C")
        C = torch.empty((M, N), dtype=out_dtype, device=A.device)
    key = ("mx", A.device, M, N, K, fmt, C.dtype, bool(clear_accum), epilogue)
    plan = _plan_cache.get(key)
    if plan is None:
        plan = Gemm(M, N, K, fmt, C.dtype, transpose_A=False, transpose_B=True, clear_accum=clear_accum,
                    epilogue=epilogue)
        _plan_cache[key] = plan
    return plan.run_mx(A, SA, B, SB, C)


_plan_cache: dict = {}
_has_workspace: dict = {}


def gemm(A: torch.Tensor, B: torch.Tensor, C: torch.Tensor | None = None, *, transpose_A: bool = False,
         transpose_B: bool = False, clear_accum: bool = True, epilogue: str = "none",
         out_dtype=torch.float16, variant: str = "auto") -> torch.Tensor:
    """C = act(A·B) (or act(C + A·B) with clear_accum=False).  A, B, C are device tensors."""
    M = A.shape[1] if transpose_A else A.shape[0]
    K = A.shape[0] if transpose_A else A.shape[1]
    N = B.shape[0] if transpose_B else B.shape[1]
    if C is None:
        if not clear_accum:
            raise ValueError("clear_accum=False needs C")
        C = torch.empty((M, N), dtype=out_dtype, device=A.device)
    key = (A.device, M, N, K, A.dtype, C.dtype, bool(transpose_A), bool(transpose_B), bool(clear_accum),
           epilogue, variant)
    # A plan with a workspace (split-K) must not run on two streams at once, and this
    # helper hides its plans from the caller: such plans are kept one per stream, so
    # calls on different streams never share a workspace.  Plans without one are shared.
    has_ws = _has_workspace.get(key)
    if has_ws is None:
        has_ws = _has_workspace[key] = bool(select(M, N, K, A.dtype, C.dtype, transpose_A=transpose_A,
                                                   transpose_B=transpose_B, clear_accum=clear_accum,
                                                   epilogue=epilogue, variant=variant).workspace_bytes)
    if has_ws:
        key = key + (torch.cuda.current_stream(A.device).cuda_stream,)
    plan = _plan_cache.get(key)
    if plan is None:
        # a split-K plan's workspace goes to the device current at creation: A's
        with torch.cuda.device(A.device) if A.device.type == "cuda" else contextlib.nullcontext():
            plan = Gemm(M, N, K, A.dtype, C.dtype, transpose_A=transpose_A, transpose_B=transpose_B,
                        clear_accum=clear_accum, epilogue=epilogue, variant=variant)
        _plan_cache[key] = plan
    return plan.run(A, B, C)


def gemm_noalloc(A: torch.Tensor, B: torch.Tensor, C: torch.Tensor, *, transpose_A: bool = False,
                 transpose_B: bool = False, clear_accum: bool = True, epilogue: str = "none",
                 stream=None) -> torch.Tensor:
    """C = act(A·B) through tlg_gemm_run_noalloc: planned and launched in one call that
    allocates nothing (a split-K choice uses the library's static scratch, shared by
    all such calls on the GPU: calls that overlap in time race).  C must be given."""
    M = A.shape[1] if transpose_A else A.shape[0]
    K = A.shape[0] if transpose_A else A.shape[1]
    N = B.shape[0] if transpose_B else B.shape[1]
    probe = Gemm.__new__(Gemm)
    probe.M, probe.N, probe.K = M, N, K
    probe.ab_code, probe.c_code = _code(A.dtype), _code(C.dtype)
    probe.transpose_A, probe.transpose_B = bool(transpose_A), bool(transpose_B)
    probe._h = None
    probe._check(A, B, C)
    if stream is None:
        stream = torch.cuda.current_stream(C.device)
    s = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    lib = load_library()
    with torch.cuda.device(C.device):
        st = lib.tlg_gemm_run_noalloc(M, N, K, _code(A.dtype), _code(C.dtype), int(bool(transpose_A)),
                                      int(bool(transpose_B)), int(bool(clear_accum)), EPILOGUES[epilogue],
                                      A.data_ptr() or None, B.data_ptr() or None, C.data_ptr() or None,
                                      ctypes.c_void_p(s))
    if st != 0:
        raise TlgError("tlg_gemm_run_noalloc", st)
    return C


def attention(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, O: torch.Tensor | None = None, *,
              causal: bool = True, scale: float | None = None, block_q: int = 0, stream=None) -> torch.Tensor:
    """Attention forward with online softmax (tlg_attn_fwd) on [batch, seq, heads, dim]
    device tensors of fp16 or bf16 (dim 64 or 128).  scale defaults to 1/sqrt(dim).
    block_q: queries per workgroup, 64 or 128 (0: the library's choice; tlg_attn_fwd_block).
    Returns O (allocated when not given)."""
    for name, t in (("Q", Q), ("K", K), ("V", V)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a device tensor, got {t.device}")
        if t.dim() != 4 or tuple(t.shape) != tuple(Q.shape):
            raise ValueError(f"{name} must be [batch, seq, heads, dim] like Q, got {tuple(t.shape)}")
        if t.dtype != Q.dtype:
            raise ValueError(f"{name} has dtype {t.dtype}, Q has {Q.dtype}")
        if t.numel() and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if O is None:
        O = torch.empty_like(Q)
    if tuple(O.shape) != tuple(Q.shape) or O.dtype != Q.dtype or (O.numel() and not O.is_contiguous()):
        raise ValueError("O must be a contiguous tensor of Q's shape and dtype")
    B, S, H, D = Q.shape
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if stream is None:
        stream = torch.cuda.current_stream(Q.device)
    s = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    lib = load_library()
    with torch.cuda.device(Q.device):
        st = lib.tlg_attn_fwd_block(Q.data_ptr() or None, K.data_ptr() or None, V.data_ptr() or None,
                                    O.data_ptr() or None, B, S, H, D, _code(Q.dtype), int(bool(causal)), sc,
                                    int(block_q), ctypes.c_void_p(s))
    if st != 0:
        raise TlgError("tlg_attn_fwd_block", st)
    return O


def attention_query_block(batch: int, seq: int, heads: int, dim: int, causal: bool) -> int:
    """Queries per workgroup that attention would use for this shape (tlg_attn_query_block;
    host only): 128, or 64 for grids of at most 256 blocks of 128 queries (1024 when causal
    with dim 64)."""
    return int(load_library().tlg_attn_query_block(int(batch), int(seq), int(heads), int(dim), int(bool(causal))))


def attention_ptrs(q: int, k: int, v: int, o: int, batch: int, seq: int, heads: int, dim: int, dtype, causal: int,
                   scale: float, stream_handle: int = 0) -> int:
    """Raw-pointer form of attention (no checks beyond the library's own); returns the status."""
    return load_library().tlg_attn_fwd(q or None, k or None, v or None, o or None, batch, seq, heads, dim,
                                       _code(dtype), int(causal), float(scale), ctypes.c_void_p(stream_handle))


def gemm_w4(A: torch.Tensor, Wq: torch.Tensor, S: torch.Tensor, Z: torch.Tensor, C: torch.Tensor | None = None, *,
            group: int = 128, epilogue: str = "none", out_dtype=torch.float16, stream=None) -> torch.Tensor:
    """Dequant GEMM C = act(A Wᵀ) with 4-bit weights (tlg_gemm_w4).  A [M, K] fp16/bf16;
    Wq [N, K/2] uint8 packed codes; S [N, K/group] scales (A's dtype); Z [N, K/group] uint8
    zero points.  Returns C (allocated when not given)."""
    M, K = A.shape
    N = Wq.shape[0]
    for name, t, shape, dt in (("A", A, (M, K), None), ("Wq", Wq, (N, K // 2), torch.uint8),
                               ("S", S, (N, K // group), A.dtype), ("Z", Z, (N, K // group), torch.uint8)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a device tensor, got {t.device}")
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")
        if dt is not None and t.dtype != dt:
            raise ValueError(f"{name} has dtype {t.dtype}, expected {dt}")
        if t.numel() and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if C is None:
        C = torch.empty((M, N), dtype=out_dtype, device=A.device)
    if tuple(C.shape) != (M, N) or (C.numel() and not C.is_contiguous()):
        raise ValueError("C must be a contiguous [M, N] tensor")
    if stream is None:
        stream = torch.cuda.current_stream(A.device)
    s = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    lib = load_library()
    with torch.cuda.device(A.device):
        st = lib.tlg_gemm_w4(A.data_ptr() or None, Wq.data_ptr() or None, S.data_ptr() or None,
                             Z.data_ptr() or None, C.data_ptr() or None, M, N, K, int(group), _code(A.dtype),
                             _code(C.dtype), EPILOGUES[epilogue], ctypes.c_void_p(s))
    if st != 0:
        raise TlgError("tlg_gemm_w4", st)
    return C


def gemm_w4_ptrs(a: int, wq: int, s: int, z: int, c: int, M: int, N: int, K: int, group: int, ab_dtype, c_dtype,
                 relu: int = 0, stream_handle: int = 0) -> int:
    """Raw-pointer form of gemm_w4 (no checks beyond the library's own); returns the status."""
    return load_library().tlg_gemm_w4(a or None, wq or None, s or None, z or None, c or None, M, N, K, group,
                                      _code(ab_dtype), _code(c_dtype), int(relu), ctypes.c_void_p(stream_handle))


def gemm_sp(A: torch.Tensor, Wv: torch.Tensor, Wm: torch.Tensor, C: torch.Tensor | None = None, *,
            epilogue: str = "none", out_dtype=torch.float16, stream=None) -> torch.Tensor:
    """2:4 structured-sparse GEMM C = act(A Wᵀ) (tlg_gemm_sp).  A [M, K] fp16/bf16; Wv [N, K/2]
    stored values (A's dtype); Wm [N, K/8] uint8 positions.  Returns C (allocated when not given)."""
    M, K = A.shape
    N = Wv.shape[0]
    for name, t, shape, dt in (("A", A, (M, K), None), ("Wv", Wv, (N, K // 2), A.dtype),
                               ("Wm", Wm, (N, K // 8), torch.uint8)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a device tensor, got {t.device}")
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")
        if dt is not None and t.dtype != dt:
            raise ValueError(f"{name} has dtype {t.dtype}, expected {dt}")
        if t.numel() and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if C is None:
        C = torch.empty((M, N), dtype=out_dtype, device=A.device)
    if tuple(C.shape) != (M, N) or (C.numel() and not C.is_contiguous()):
        raise ValueError("C must be a contiguous [M, N] tensor")
    if stream is None:
        stream = torch.cuda.current_stream(A.device)
    s = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    lib = load_library()
    with torch.cuda.device(A.device):
        st = lib.tlg_gemm_sp(A.data_ptr() or None, Wv.data_ptr() or None, Wm.data_ptr() or None,
                             C.data_ptr() or None, M, N, K, _code(A.dtype), _code(C.dtype), EPILOGUES[epilogue],
                             ctypes.c_void_p(s))
    if st != 0:
        raise TlgError("tlg_gemm_sp", st)
    return C


def gemm_sp_ptrs(a: int, wv: int, wm: int, c: int, M: int, N: int, K: int, ab_dtype, c_dtype, relu: int = 0,
                 stream_handle: int = 0) -> int:
    """Raw-pointer form of gemm_sp (no checks beyond the library's own); returns the status."""
    return load_library().tlg_gemm_sp(a or None, wv or None, wm or None, c or None, M, N, K, _code(ab_dtype),
                                      _code(c_dtype), int(relu), ctypes.c_void_p(stream_handle))
