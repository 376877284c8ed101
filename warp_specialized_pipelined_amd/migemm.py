"""ctypes binding of libmigemm.so (include/migemm.h), names unchanged.

Argument marshalling only: every step of the GEMM runs in the HIP library.
Tensors may be passed as torch tensors (their ``data_ptr()`` is used) or as
raw integer addresses; streams as ``torch.cuda.Stream``, raw handles or None
(the current torch stream).  If the library has not been built this module
raises on first use; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmigemm.so")

MIGEMM_BF16 = 1
MIGEMM_FP8_E4M3 = 2

MIGEMM_OK = 0
MIGEMM_ERR_INVALID_ARG = -1
MIGEMM_ERR_UNSUPPORTED = -2
MIGEMM_ERR_MISALIGNED = -3
MIGEMM_ERR_DEVICE = -4
MIGEMM_ERR_LAUNCH = -5
MIGEMM_ERR_TIMEOUT = -6
MIGEMM_ERR_SCRATCH = -7
MIGEMM_NO_ALLOC_SCRATCH_BYTES = 64 << 20

MIGEMM_F_TILE_CONSUMER = 0x1
MIGEMM_F_STREAM_K = 0x2
MIGEMM_F_STREAM_K_FORCE = 0x4
MIGEMM_F_HANDOFF_DEBUG = 0x10
MIGEMM_F_C_IN_EPILOGUE = 0x20
MIGEMM_F_CONSUMER_OVERLAP = 0x8
MIGEMM_F_TILE_M256 = 0x40
MIGEMM_F_TILE_M192 = 0x80
MIGEMM_TILE_M = 256
MIGEMM_TILE_N = 256

EXPORTED = [
    "gemm_desc_validate", "gemm_plan_create", "gemm_plan_destroy", "gemm_plan_get_info",
    "gemm_plan_workspace_size", "gemm_workspace_init", "gemm_run", "gemm_run_with_tile_consumer",
    "gemm_run_no_alloc", "gemm_debug_read", "gemm_status_string",
]


class migemm_desc(ctypes.Structure):
    _fields_ = [
        ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
        ("a_type", ctypes.c_int32), ("b_type", ctypes.c_int32),
        ("c_type", ctypes.c_int32), ("d_type", ctypes.c_int32),
        ("a_rs", ctypes.c_int64), ("a_cs", ctypes.c_int64),
        ("b_rs", ctypes.c_int64), ("b_cs", ctypes.c_int64),
        ("c_rs", ctypes.c_int64), ("c_cs", ctypes.c_int64),
        ("d_rs", ctypes.c_int64), ("d_cs", ctypes.c_int64),
        ("device", ctypes.c_int32), ("flags", ctypes.c_uint32),
        ("max_workgroups", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("L", ctypes.c_int64),
        ("a_bs", ctypes.c_int64), ("b_bs", ctypes.c_int64),
        ("c_bs", ctypes.c_int64), ("d_bs", ctypes.c_int64),
        ("debug_wait_ticks", ctypes.c_int64), ("debug_force_wait", ctypes.c_int32),
        ("reserved2", ctypes.c_int32),
    ]


class migemm_debug_info(ctypes.Structure):
    _fields_ = [
        ("waits_given_up", ctypes.c_uint32), ("max_occupancy", ctypes.c_uint32),
        ("trace_offset", ctypes.c_int64),
        ("grid", ctypes.c_int32), ("waves", ctypes.c_int32),
        ("trace_tiles", ctypes.c_int32), ("trace_words", ctypes.c_int32),
    ]


class migemm_plan_info(ctypes.Structure):
    _fields_ = [
        ("tiles_m", ctypes.c_int64), ("tiles_n", ctypes.c_int64), ("num_tiles", ctypes.c_int64),
        ("grid", ctypes.c_int32), ("block_threads", ctypes.c_int32),
        ("lds_bytes", ctypes.c_int32), ("stages", ctypes.c_int32),
        ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32), ("tile_k", ctypes.c_int32),
        ("swapped", ctypes.c_int32), ("a_kmajor", ctypes.c_int32), ("b_kmajor", ctypes.c_int32),
        ("cu_count", ctypes.c_int32), ("handoff_slots", ctypes.c_int32),
        ("stream_k_tiles", ctypes.c_int64), ("stream_k_units_per_tile", ctypes.c_int32),
        ("c_in_k_loop", ctypes.c_int32), ("batches", ctypes.c_int64),
    ]


class MigemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {gemm_status_string(status)} ({status})")


_lib = None


def load(path: str | None = None):
    """Load libmigemm.so (once; LIB_PATH unless a path is given).  Raises if
    it is missing.

    torch ships its own HIP runtime library.  It is imported first, when it
    is installed, so that libmigemm.so binds that same runtime: with two HIP
    runtimes in one process the second cannot use the device, and torch's
    device pointers and streams would not be valid in it."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -m warp_specialized_pipelined_amd.build`"
                           " (or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    P = ctypes.POINTER
    lib.gemm_desc_validate.argtypes = [P(migemm_desc)]
    lib.gemm_desc_validate.restype = i32
    lib.gemm_plan_create.argtypes = [P(migemm_desc), P(vp)]
    lib.gemm_plan_create.restype = i32
    lib.gemm_plan_destroy.argtypes = [vp]
    lib.gemm_plan_destroy.restype = i32
    lib.gemm_plan_get_info.argtypes = [vp, P(migemm_plan_info)]
    lib.gemm_plan_get_info.restype = i32
    lib.gemm_plan_workspace_size.argtypes = [vp]
    lib.gemm_plan_workspace_size.restype = ctypes.c_size_t
    lib.gemm_workspace_init.argtypes = [vp, vp, vp]
    lib.gemm_workspace_init.restype = i32
    lib.gemm_run.argtypes = [vp, vp, vp, vp, vp, ctypes.c_float, ctypes.c_float, vp, vp]
    lib.gemm_run.restype = i32
    lib.gemm_run_with_tile_consumer.argtypes = [vp, vp, vp, vp, vp, ctypes.c_float, ctypes.c_float,
                                                vp, vp, vp, vp, vp]
    lib.gemm_run_with_tile_consumer.restype = i32
    lib.gemm_run_no_alloc.argtypes = [vp, vp, vp, vp, vp, ctypes.c_float, ctypes.c_float, vp]
    lib.gemm_run_no_alloc.restype = i32
    lib.gemm_debug_read.argtypes = [vp, vp, vp, P(migemm_debug_info)]
    lib.gemm_debug_read.restype = i32
    lib.gemm_status_string.argtypes = [i32]
    lib.gemm_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _ptr(x) -> int | None:
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return int(x.data_ptr())
    return int(x)


def _stream(s) -> int | None:
    if s is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if hasattr(s, "cuda_stream"):
        return int(s.cuda_stream)
    return int(s)


def _plan(plan):
    """A plan handle from a Plan object or a raw handle.  Passing the Plan
    object keeps it (and so the C plan) alive for the whole call; a handle
    taken from a temporary Plan, as in gemm_run(Plan(d).handle, ...), is
    already destroyed when the call starts, which the library then rejects
    with MIGEMM_ERR_INVALID_ARG."""
    return getattr(plan, "handle", plan)


def make_desc(M, N, K, a_type, b_type, a_rs, a_cs, b_rs, b_cs, c_rs, c_cs, d_rs, d_cs,
              device=0, flags=0, max_workgroups=0, c_type=MIGEMM_BF16, d_type=MIGEMM_BF16,
              L=1, a_bs=0, b_bs=0, c_bs=0, d_bs=0, debug_wait_ticks=0, debug_force_wait=0):
    return migemm_desc(M, N, K, a_type, b_type, c_type, d_type, a_rs, a_cs, b_rs, b_cs, c_rs, c_cs,
                       d_rs, d_cs, device, flags, max_workgroups, 0, L, a_bs, b_bs, c_bs, d_bs,
                       debug_wait_ticks, debug_force_wait, 0)


def gemm_status_string(status: int) -> str:
    return load().gemm_status_string(int(status)).decode()


def gemm_desc_validate(desc: migemm_desc) -> int:
    return int(load().gemm_desc_validate(ctypes.byref(desc)))


def gemm_plan_create(desc: migemm_desc) -> int:
    """Returns the plan handle; raises MigemmError on a non-OK status."""
    h = ctypes.c_void_p()
    st = load().gemm_plan_create(ctypes.byref(desc), ctypes.byref(h))
    if st != MIGEMM_OK:
        raise MigemmError(st, "gemm_plan_create")
    return h.value


def gemm_plan_destroy(plan: int) -> int:
    return int(load().gemm_plan_destroy(_plan(plan)))


def gemm_plan_get_info(plan: int) -> migemm_plan_info:
    info = migemm_plan_info()
    st = load().gemm_plan_get_info(_plan(plan), ctypes.byref(info))
    if st != MIGEMM_OK:
        raise MigemmError(st, "gemm_plan_get_info")
    return info


def gemm_plan_workspace_size(plan: int) -> int:
    return int(load().gemm_plan_workspace_size(_plan(plan)))


def gemm_workspace_init(plan, workspace, stream=None, check: bool = True) -> int:
    st = load().gemm_workspace_init(_plan(plan), _ptr(workspace), _stream(stream))
    if check and st != MIGEMM_OK:
        raise MigemmError(st, "gemm_workspace_init")
    return st


def gemm_run(plan, A, B, C, D, alpha: float, beta: float, workspace=None, stream=None,
             check: bool = True) -> int:
    st = load().gemm_run(_plan(plan), _ptr(A), _ptr(B), _ptr(C), _ptr(D), float(alpha), float(beta),
                         _ptr(workspace), _stream(stream))
    if check and st != MIGEMM_OK:
        raise MigemmError(st, "gemm_run")
    return int(st)


def gemm_run_no_alloc(plan, A, B, C, D, alpha: float, beta: float, stream=None,
                      check: bool = True) -> int:
    st = load().gemm_run_no_alloc(_plan(plan), _ptr(A), _ptr(B), _ptr(C), _ptr(D), float(alpha),
                                  float(beta), _stream(stream))
    if check and st != MIGEMM_OK:
        raise MigemmError(st, "gemm_run_no_alloc")
    return int(st)


def gemm_debug_read(plan, workspace, stream=None) -> tuple:
    """(status, migemm_debug_info): synchronizes the stream, reads the debug
    header.  status is MIGEMM_ERR_TIMEOUT when a bounded wait gave up."""
    info = migemm_debug_info()
    st = load().gemm_debug_read(_plan(plan), _ptr(workspace), _stream(stream), ctypes.byref(info))
    return int(st), info


def gemm_run_with_tile_consumer(plan, A, B, C, D, alpha: float, beta: float, row_sum, row_max,
                                D_copy, workspace=None, stream=None, check: bool = True) -> int:
    st = load().gemm_run_with_tile_consumer(_plan(plan), _ptr(A), _ptr(B), _ptr(C), _ptr(D), float(alpha),
                                            float(beta), _ptr(row_sum), _ptr(row_max),
                                            _ptr(D_copy), _ptr(workspace), _stream(stream))
    if check and st != MIGEMM_OK:
        raise MigemmError(st, "gemm_run_with_tile_consumer")
    return int(st)


class Plan:
    """Owns a plan handle; destroys it when garbage-collected."""

    def __init__(self, desc: migemm_desc):
        self.desc = desc
        self.handle = gemm_plan_create(desc)
        self.info = gemm_plan_get_info(self.handle)

    @property
    def workspace_size(self) -> int:
        return gemm_plan_workspace_size(self.handle)

    def run(self, A, B, C, D, alpha=1.0, beta=0.0, stream=None, workspace=None):
        return gemm_run(self.handle, A, B, C, D, alpha, beta, workspace, stream)

    def run_with_tile_consumer(self, A, B, C, D, alpha, beta, row_sum, row_max, D_copy,
                               stream=None):
        return gemm_run_with_tile_consumer(self.handle, A, B, C, D, alpha, beta, row_sum, row_max,
                                           D_copy, None, stream)

    def __del__(self):
        h = getattr(self, "handle", None)
        if h:
            try:
                gemm_plan_destroy(h)
            except Exception:
                pass
            self.handle = None
