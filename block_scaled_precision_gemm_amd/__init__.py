"""Python binding of the block-scaled GEMM C ABI (libbsg.so, include/bsg.h).

Argument marshalling only: every step of the GEMM runs in the HIP library.  Tensors are passed as
device pointers (anything with .data_ptr(), or a plain int); streams as hipStream_t handles (an
object with .cuda_stream, an int, or None for torch's current stream).  PyTorch is only used, when
present, to find the current stream.

The library is loaded on first use and a missing build raises LibraryNotBuilt: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["Plan", "BsgError", "LibraryNotBuilt", "load_library", "bench_loop", "null_loop", "run_noalloc", "NOALLOC_SCRATCH_BYTES", "decode_nvfp4_f16",
           "FORMATS", "OUT_DTYPES", "SCALE_LAYOUTS", "abi_version", "packed_strides", "Problem", "PROBLEM_V1_SIZE", "PROBLEM_V2_SIZE",
           "pack_scales", "scales_ktile_bytes"]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbsg.so")

FORMATS = {"mxfp8": 1, "nvfp4": 2}
OUT_DTYPES = {"bf16": 1, "f16": 2}
EPI_BIAS, EPI_SILU, SCALES_KTILE = 1, 2, 4
SCALE_LAYOUTS = ("linear", "ktile")  # row-major [rows][K/block], or K-tile-major (BSG_SCALES_KTILE)
SCALE_BLOCK = {"mxfp8": 32, "nvfp4": 16}

STATUS = {0: "BSG_OK", 1: "BSG_ERR_NULL", 2: "BSG_ERR_SHAPE", 3: "BSG_ERR_UNSUPPORTED", 4: "BSG_ERR_ALIGN",
          5: "BSG_ERR_DEVICE", 6: "BSG_ERR_HIP", 7: "BSG_ERR_ALLOC", 8: "BSG_ERR_ABI"}


class LibraryNotBuilt(RuntimeError):
    pass


class BsgError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        self.status_name = STATUS.get(status, f"status {status}")
        super().__init__(f"{self.status_name}: {message}")


class Problem(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("format", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("device", ctypes.c_int32), ("batch", ctypes.c_int32), ("stride_a", ctypes.c_int64),
                ("stride_b", ctypes.c_int64), ("stride_sa", ctypes.c_int64), ("stride_sb", ctypes.c_int64),
                ("stride_bias", ctypes.c_int64), ("stride_d", ctypes.c_int64),
                ("lda", ctypes.c_int64), ("ldb", ctypes.c_int64), ("ldd", ctypes.c_int64)]


PROBLEM_V1_SIZE = 48  # sizeof(bsg_problem) of ABI 1, still accepted by bsg_plan_create
PROBLEM_V2_SIZE = 96  # ... and of ABI 2 (no leading dimensions)


def scales_ktile_bytes(rows: int, codes_per_row: int) -> int:
    """Bytes of one operand's scales in the K-tile-major layout: ceil(codes / 4) * rows * 4."""
    return 0 if rows < 1 or codes_per_row < 1 else (codes_per_row + 3) // 4 * rows * 4


def packed_strides(fmt: str, M: int, N: int, K: int, scale_layout: str = "linear", lda: int = 0, ldb: int = 0,
                   ldd: int = 0) -> dict:
    """Byte strides of back-to-back batched operands (bias shared by every problem): each problem's
    A, B and D take rows x leading dimension (0 = packed: K, K, N)."""
    elem, blk = (1.0, 32) if fmt == "mxfp8" else (0.5, 16)
    lda, ldb, ldd = lda or K, ldb or K, ldd or N
    if scale_layout == "ktile":
        sa, sb = scales_ktile_bytes(M, K // blk), scales_ktile_bytes(N, K // blk)
    else:
        sa, sb = M * K // blk, N * K // blk
    return dict(a=int(M * lda * elem), b=int(N * ldb * elem), sa=sa, sb=sb, bias=0, d=2 * M * ldd)


class PlanInfo(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("variant", ctypes.c_char * 64), ("tile_m", ctypes.c_int32),
                ("tile_n", ctypes.c_int32), ("tile_k", ctypes.c_int32), ("grid_x", ctypes.c_uint32),
                ("grid_y", ctypes.c_uint32), ("grid_z", ctypes.c_uint32), ("block_x", ctypes.c_uint32),
                ("lds_bytes", ctypes.c_uint32), ("workspace_bytes", ctypes.c_uint64)]


_lib = None

_VP = ctypes.c_void_p
_SIGNATURES = {
    "bsg_plan_create": (ctypes.c_int, [ctypes.POINTER(Problem), ctypes.POINTER(_VP)]),
    "bsg_run": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_float, _VP, _VP]),
    "bsg_run_alpha_ptr": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
    "bsg_plan_destroy": (ctypes.c_int, [_VP]),
    "bsg_plan_query": (ctypes.c_int, [_VP, ctypes.POINTER(PlanInfo)]),
    "bsg_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "bsg_last_error": (ctypes.c_char_p, []),
    "bsg_abi_version": (ctypes.c_int, []),
    "bsg_test_decode_nvfp4_f16": (ctypes.c_int, [_VP, _VP, _VP, ctypes.c_int64, _VP]),
    "bsg_pack_scales": (ctypes.c_int, [_VP, _VP, ctypes.c_int64, ctypes.c_int64, _VP]),
    "bsg_scales_ktile_bytes": (ctypes.c_int64, [ctypes.c_int64, ctypes.c_int64]),
    "bsg_bench_loop": (ctypes.c_int, [_VP, ctypes.c_int, ctypes.POINTER(_VP), ctypes.POINTER(_VP),
                                      ctypes.POINTER(_VP), ctypes.POINTER(_VP), ctypes.POINTER(_VP),
                                      ctypes.POINTER(ctypes.c_float), ctypes.POINTER(_VP), ctypes.c_int,
                                      ctypes.c_int, _VP, ctypes.POINTER(ctypes.c_double),
                                      ctypes.POINTER(ctypes.c_double)]),
    "bsg_run_noalloc": (ctypes.c_int, [ctypes.POINTER(Problem), _VP, _VP, _VP, _VP, _VP, ctypes.c_float, _VP, _VP]),
    "bsg_bench_null_loop": (ctypes.c_int, [ctypes.c_int, _VP, ctypes.POINTER(ctypes.c_double),
                                           ctypes.POINTER(ctypes.c_double)]),
}


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libbsg.so (once).  Raises LibraryNotBuilt if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise LibraryNotBuilt(f"{path} is missing: build it with `python -m block_scaled_precision_gemm_amd.build` "
                              "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def abi_version() -> int:
    return load_library().bsg_abi_version()


def _check(status: int) -> None:
    if status != 0:
        raise BsgError(status, load_library().bsg_last_error().decode(errors="replace"))


def _ptr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s) -> int | None:
    if s is None:
        try:
            import torch
            if torch.cuda.is_available():
                return torch.cuda.current_stream().cuda_stream
        except ImportError:
            pass
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


class Plan:
    """A cached GEMM plan: D = epi(alpha * A x B^T (+ bias)) for one problem shape and variant.

    batch > 1: that many problems of this shape per call; problem z uses each pointer advanced by
    strides[key] * z bytes (keys a, b, sa, sb, bias, d; default: back-to-back operands, shared bias).
    scale_layout "ktile": sA and sB in the K-tile-major layout (pack_scales converts).
    lda, ldb, ldd: leading dimensions in elements (row pitch of A, B and D; 0 = packed).
    """

    def __init__(self, fmt: str, M: int, N: int, K: int, out: str = "bf16", bias: bool = False,
                 silu: bool = False, device: int = -1, batch: int = 1, strides: dict | None = None,
                 scale_layout: str = "linear", lda: int = 0, ldb: int = 0, ldd: int = 0):
        if scale_layout not in SCALE_LAYOUTS:
            raise ValueError(f"scale_layout must be one of {SCALE_LAYOUTS}")
        lib = load_library()
        self._lib = lib
        self._h = None
        self.fmt, self.M, self.N, self.K, self.out, self.bias, self.silu = fmt, M, N, K, out, bias, silu
        self.batch, self.scale_layout = batch, scale_layout
        st = packed_strides(fmt, M, N, K, scale_layout, lda, ldb, ldd)
        st.update(strides or {})
        self.strides = st
        self.lda, self.ldb, self.ldd = lda or K, ldb or K, ldd or N
        prob = Problem(ctypes.sizeof(Problem), FORMATS[fmt], OUT_DTYPES[out],
                       (EPI_BIAS if bias else 0) | (EPI_SILU if silu else 0)
                       | (SCALES_KTILE if scale_layout == "ktile" else 0), M, N, K, device, batch,
                       st["a"], st["b"], st["sa"], st["sb"], st["bias"], st["d"], lda, ldb, ldd)
        h = _VP()
        _check(lib.bsg_plan_create(ctypes.byref(prob), ctypes.byref(h)))
        self._h = h

    @property
    def handle(self) -> int:
        return self._h.value

    def run(self, A, B, sA, sB, D, alpha: float = 1.0, bias=None, stream=None) -> None:
        _check(self._lib.bsg_run(self._h, _ptr(A), _ptr(B), _ptr(sA), _ptr(sB), _ptr(bias), float(alpha), _ptr(D),
                                 _stream(stream)))

    def run_alpha_ptr(self, A, B, sA, sB, D, alpha_dev, bias=None, stream=None) -> None:
        _check(self._lib.bsg_run_alpha_ptr(self._h, _ptr(A), _ptr(B), _ptr(sA), _ptr(sB), _ptr(bias),
                                           _ptr(alpha_dev), _ptr(D), _stream(stream)))

    def info(self) -> dict:
        inf = PlanInfo()
        inf.struct_size = ctypes.sizeof(PlanInfo)
        _check(self._lib.bsg_plan_query(self._h, ctypes.byref(inf)))
        return dict(variant=inf.variant.decode(), tile=(inf.tile_m, inf.tile_n, inf.tile_k),
                    grid=(inf.grid_x, inf.grid_y, inf.grid_z), block=inf.block_x, lds_bytes=inf.lds_bytes,
                    workspace_bytes=inf.workspace_bytes)

    def close(self) -> None:
        if self._h is not None and self._h.value:
            _check(self._lib.bsg_plan_destroy(self._h))
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


NOALLOC_SCRATCH_BYTES = 32 << 20  # BSG_NOALLOC_SCRATCH_BYTES


def run_noalloc(fmt: str, M: int, N: int, K: int, A, B, sA, sB, D, alpha: float = 1.0, bias=None, out: str = "bf16",
                silu: bool = False, device: int = -1, stream=None) -> None:
    """One GEMM call through bsg_run_noalloc (no allocation; split-K partials in the library's static
    device scratch).  Packed, single-problem, row-major scales."""
    prob = Problem(ctypes.sizeof(Problem), FORMATS[fmt], OUT_DTYPES[out],
                   (EPI_BIAS if bias is not None else 0) | (EPI_SILU if silu else 0), M, N, K, device, 1,
                   0, 0, 0, 0, 0, 0, 0, 0, 0)
    _check(load_library().bsg_run_noalloc(ctypes.byref(prob), _ptr(A), _ptr(B), _ptr(sA), _ptr(sB), _ptr(bias),
                                          float(alpha), _ptr(D), _stream(stream)))


def bench_loop(plan: Plan, sets: list[dict], calls_per_set: int, mode: int, stream, with_submit: bool = False):
    """Native loop of len(sets) * calls_per_set bsg_run calls; returns the host wall time in us
    (with_submit: the pair (wall, enqueue-only time) in us).

    Each set is a dict with A, B, sA, sB, D, alpha and optional bias.  mode 0 = direct calls,
    mode 1 = one HIP graph per set (captured outside the timed region) replayed.
    """
    lib = load_library()
    n = len(sets)
    arr = lambda key: (_VP * n)(*[_ptr(s.get(key)) for s in sets])  # noqa: E731
    alphas = (ctypes.c_float * n)(*[float(s["alpha"]) for s in sets])
    has_bias = any(s.get("bias") is not None for s in sets)
    wall, submit = ctypes.c_double(), ctypes.c_double()
    _check(lib.bsg_bench_loop(plan._h, n, arr("A"), arr("B"), arr("sA"), arr("sB"), arr("bias") if has_bias else None,
                              alphas, arr("D"), calls_per_set, mode, _stream(stream), ctypes.byref(wall),
                              ctypes.byref(submit)))
    return (wall.value, submit.value) if with_submit else wall.value


def null_loop(n: int, stream) -> tuple[float, float]:
    """n back-to-back launches of an empty kernel from C++: (wall us, enqueue-only us)."""
    wall, submit = ctypes.c_double(), ctypes.c_double()
    _check(load_library().bsg_bench_null_loop(n, _stream(stream), ctypes.byref(wall), ctypes.byref(submit)))
    return wall.value, submit.value


def decode_nvfp4_f16(packed, scale_codes, out_f16, n_elements: int, stream=None) -> None:
    """out_f16[k] = device fp16 dequantisation of NVFP4 element k times 2^-8, through the GEMM
    kernels' routine (packed[k/2] nibble, scale_codes[k/16]); n_elements a multiple of 32."""
    _check(load_library().bsg_test_decode_nvfp4_f16(_ptr(packed), _ptr(scale_codes), _ptr(out_f16), n_elements,
                                                    _stream(stream)))


def pack_scales(src, dst, rows: int, codes_per_row: int, stream=None) -> None:
    """dst (scales_ktile_bytes(rows, codes_per_row) bytes, device) = the K-tile-major layout of the
    row-major scale codes src [rows][codes_per_row] (device); enqueued on `stream`."""
    _check(load_library().bsg_pack_scales(_ptr(src), _ptr(dst), rows, codes_per_row, _stream(stream)))
