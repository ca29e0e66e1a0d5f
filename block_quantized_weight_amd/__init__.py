"""Python binding of libqgemv, the block-scaled small-M decode GEMV for MI355X.

Argument marshalling only: every step of the computation runs in the HIP kernels
behind the C ABI declared in include/qgemv.h. PyTorch supplies device memory and
streams. If the shared library has not been built the first call raises; there is
no fallback path of any kind.
"""

from __future__ import annotations

import ctypes
import os
import threading
from typing import Any, Dict, Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqgemv.so")

FORMATS = {"u4": 1, "u8": 2, "fp8": 3, "nvfp4": 4}
ACT_DTYPES = {"f16": 1, "bf16": 2}
FAMILIES = {"auto": 0, "stream": 1, "mfma": 2, "generic": 3}
FAMILY_NAMES = {v: k for k, v in FAMILIES.items()}

QGEMV_OK = 0
QGEMV_E_WORKSPACE = 9
QGEMV_E_SCRATCH = 10
NOALLOC_SCRATCH_BYTES = 16 << 20  # QGEMV_NOALLOC_SCRATCH_BYTES
FLAG_FAMILY_MASK = 0x0000000F
FLAG_KPARTS_SHIFT = 4
FLAG_STREAM_META_CHUNK = 0x00000080
FLAG_KSPLIT_SHIFT = 8
FLAG_STREAM_NWG_SHIFT = 12
FLAG_NO_RESIDENCY_FIT = 0x00008000
FLAG_NO_MFMA = 0x00010000
FLAG_STAGE_A_OFF = 0x00020000
FLAG_STAGE_A_ON = 0x00040000
FLAG_RING_OFF = 0x00080000
FLAG_RING_ON = 0x00100000
FLAG_STREAM_CPW_SHIFT = 21
FLAG_STREAM_UNR_SHIFT = 23
FLAG_STREAM_WPC_SHIFT = 25
FLAG_STREAM_CLASSIC = 0x10000000
FLAG_MFMA_DEPTH_SHIFT = 29
FLAG_STREAM_WIDE_WG = 0x80000000
TUNE_MAX_CANDIDATES = 256  # QGEMV_TUNE_MAX_CANDIDATES
MAX_M = 16  # rows one plan carries
MAX_ROWS = 65536  # rows one call accepts (more than MAX_M run as chunks of MAX_M)

_lock = threading.Lock()
_lib = None


class QGemvError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: qgemv status {status} ({status_str(status)})")
        self.status = status


class Desc(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("format", ctypes.c_int32),
        ("act_dtype", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("N", ctypes.c_int64),
        ("K", ctypes.c_int64),
        ("W", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("zero_points", ctypes.c_void_p),
        ("tensor_scale", ctypes.c_float),
        ("flags", ctypes.c_uint32),
        ("bias", ctypes.c_void_p),
    ]


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("family", ctypes.c_int32),
        ("rows_per_pass", ctypes.c_int32),
        ("passes", ctypes.c_int32),
        ("cols_per_wave", ctypes.c_int32),
        ("ksplit", ctypes.c_int32),
        ("waves_per_wg", ctypes.c_int32),
        ("grid", ctypes.c_int64),
        ("lds_bytes", ctypes.c_int32),
        ("variant", ctypes.c_int32),
        ("kparts", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_int64),
    ]


class TuneInfo(ctypes.Structure):
    _fields_ = [
        ("candidates", ctypes.c_int32),
        ("rounds", ctypes.c_int32),
        ("chosen_flags", ctypes.c_uint32),
        ("reserved", ctypes.c_int32),
        ("auto_us", ctypes.c_double),
        ("chosen_us", ctypes.c_double),
    ]


def lib() -> ctypes.CDLL:
    """Load libqgemv.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(f"{LIB_PATH} is missing: build it with block_quantized_weight_amd.build.build()")
            L = ctypes.CDLL(LIB_PATH)
            vp = ctypes.c_void_p
            L.qgemv_create.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(Desc), ctypes.c_int]
            L.qgemv_create.restype = ctypes.c_int
            L.qgemv_run.argtypes = [vp, vp, vp, ctypes.c_int, vp]
            L.qgemv_run.restype = ctypes.c_int
            L.qgemv_run_ws.argtypes = [vp, vp, vp, ctypes.c_int, vp, ctypes.c_size_t, vp]
            L.qgemv_run_ws.restype = ctypes.c_int
            L.qgemv_run_noalloc.argtypes = [vp, vp, vp, ctypes.c_int, vp]
            L.qgemv_run_noalloc.restype = ctypes.c_int
            L.qgemv_workspace_size.argtypes = [vp, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
            L.qgemv_workspace_size.restype = ctypes.c_int
            L.qgemv_plan.argtypes = [vp, ctypes.c_int, ctypes.c_int, ctypes.POINTER(PlanInfo)]
            L.qgemv_plan.restype = ctypes.c_int
            L.qgemv_select.argtypes = [ctypes.POINTER(Desc), ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.POINTER(PlanInfo)]
            L.qgemv_select.restype = ctypes.c_int
            L.qgemv_tune_candidates.argtypes = [ctypes.POINTER(Desc), ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                ctypes.POINTER(ctypes.c_uint32), ctypes.c_int,
                                                ctypes.POINTER(ctypes.c_int)]
            L.qgemv_tune_candidates.restype = ctypes.c_int
            L.qgemv_tune.argtypes = [vp, vp, vp, ctypes.c_int, ctypes.c_int, vp, ctypes.c_size_t, ctypes.c_int,
                                     ctypes.c_int, vp, ctypes.POINTER(TuneInfo)]
            L.qgemv_tune.restype = ctypes.c_int
            L.qgemv_destroy.argtypes = [vp]
            L.qgemv_destroy.restype = None
            L.qgemv_status_str.argtypes = [ctypes.c_int]
            L.qgemv_status_str.restype = ctypes.c_char_p
            L.qgemv_abi_version.restype = ctypes.c_int
            _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().qgemv_status_str(int(status)).decode()


def _ptr(x: Any) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def make_desc(fmt: str, act: str, N: int, K: int, block_size: int, W: Any, scales: Any,
              zero_points: Any = None, tensor_scale: float = 1.0, flags: int = 0, bias: Any = None) -> Desc:
    return Desc(ctypes.sizeof(Desc), FORMATS.get(fmt, 0) if isinstance(fmt, str) else int(fmt),
                ACT_DTYPES.get(act, 0) if isinstance(act, str) else int(act), int(block_size), int(N), int(K),
                _ptr(W), _ptr(scales), _ptr(zero_points), float(tensor_scale), int(flags), _ptr(bias))


def _plan_dict(p: PlanInfo) -> Dict[str, Any]:
    return {"family": FAMILY_NAMES.get(p.family, p.family), "rows_per_pass": p.rows_per_pass,
            "passes": p.passes, "cols_per_wave": p.cols_per_wave, "ksplit": p.ksplit,
            "waves_per_wg": p.waves_per_wg, "grid": p.grid, "lds_bytes": p.lds_bytes, "variant": p.variant,
            "kparts": p.kparts, "workspace_bytes": p.workspace_bytes}


def select(fmt: str, act: str, N: int, K: int, block_size: int, M: int, cu_count: int = 256,
           flags: int = 0, W: Any = 0x1000, scales: Any = 0x1000, zero_points: Any = None,
           bias: Any = None, with_workspace: bool = False) -> Dict[str, Any]:
    """Pure host dispatcher query (no GPU): the launch for M rows at cu_count CUs, as
    qgemv_run makes it, or as qgemv_run_ws does with_workspace."""
    d = make_desc(fmt, act, N, K, block_size, W, scales, zero_points, 1.0, flags, bias)
    out = PlanInfo()
    rc = lib().qgemv_select(ctypes.byref(d), int(M), int(cu_count), int(bool(with_workspace)), ctypes.byref(out))
    if rc != QGEMV_OK:
        raise QGemvError(rc, "qgemv_select")
    return _plan_dict(out)


def tune_candidates(fmt: str, act: str, N: int, K: int, block_size: int, M: int, cu_count: int = 256,
                    flags: int = 0, W: Any = 0x1000, scales: Any = 0x1000, zero_points: Any = None,
                    bias: Any = None, with_workspace: bool = False) -> "list[int]":
    """Pure host query (no GPU): the flag sets qgemv_tune would time for M rows at
    cu_count CUs (the first, 0, is the automatic plan)."""
    d = make_desc(fmt, act, N, K, block_size, W, scales, zero_points, 1.0, flags, bias)
    buf = (ctypes.c_uint32 * TUNE_MAX_CANDIDATES)()
    n = ctypes.c_int()
    rc = lib().qgemv_tune_candidates(ctypes.byref(d), int(M), int(cu_count), int(bool(with_workspace)), buf,
                                     TUNE_MAX_CANDIDATES, ctypes.byref(n))
    if rc != QGEMV_OK:
        raise QGemvError(rc, "qgemv_tune_candidates")
    return [int(buf[i]) for i in range(n.value)]


def _stream_handle(stream: Any) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


class QGemv:
    """A quantized weight resident on the GPU, ready to multiply activations.

    W, scales, zero_points and the optional bias ([N], activation dtype) are device
    buffers (torch tensors or raw device pointers) in the layouts documented in
    include/qgemv.h; they must stay alive as long as this object.
    """

    def __init__(self, fmt: str, act: str, N: int, K: int, block_size: int, W: Any, scales: Any,
                 zero_points: Any = None, tensor_scale: float = 1.0, flags: int = 0, device: int = -1,
                 bias: Any = None):
        self.fmt, self.act, self.N, self.K, self.block_size = fmt, act, int(N), int(K), int(block_size)
        self._keep = (W, scales, zero_points, bias)
        self._desc = make_desc(fmt, act, N, K, block_size, W, scales, zero_points, tensor_scale, flags, bias)
        h = ctypes.c_void_p()
        rc = lib().qgemv_create(ctypes.byref(h), ctypes.byref(self._desc), int(device))
        if rc != QGEMV_OK:
            raise QGemvError(rc, "qgemv_create")
        self._h = h

    def run(self, A: Any, Y: Any, M: Optional[int] = None, stream: Any = None, workspace: Any = None,
            workspace_bytes: Optional[int] = None) -> None:
        """Enqueue Y[M, N] = A[M, K] . dequant(W)^T on `stream` (torch stream, raw
        hipStream_t int, or None for torch's current stream). With a workspace (a
        device buffer zeroed once before its first use, see workspace_size) the call
        goes through qgemv_run_ws, which may split K across workgroups."""
        if M is None:
            M = int(A.shape[0])
        if stream is None:
            import torch
            stream = torch.cuda.current_stream().cuda_stream
        elif not isinstance(stream, int):
            stream = stream.cuda_stream
        if workspace is None and workspace_bytes is None:
            rc = lib().qgemv_run(self._h, _ptr(A), _ptr(Y), int(M), ctypes.c_void_p(stream))
            where = "qgemv_run"
        else:
            if workspace_bytes is None:
                workspace_bytes = int(workspace.numel() * workspace.element_size())
            rc = lib().qgemv_run_ws(self._h, _ptr(A), _ptr(Y), int(M), _ptr(workspace), int(workspace_bytes),
                                    ctypes.c_void_p(stream))
            where = "qgemv_run_ws"
        if rc != QGEMV_OK:
            raise QGemvError(rc, where)

    def run_noalloc(self, A: Any, Y: Any, M: Optional[int] = None, stream: Any = None) -> None:
        """qgemv_run_noalloc: the qgemv_run_ws product with the library's own device
        scratch array as the workspace; allocates nothing. Calls that overlap in time
        on one device share that array and must be serialized by the caller."""
        if M is None:
            M = int(A.shape[0])
        if stream is None:
            import torch
            stream = torch.cuda.current_stream().cuda_stream
        elif not isinstance(stream, int):
            stream = stream.cuda_stream
        rc = lib().qgemv_run_noalloc(self._h, _ptr(A), _ptr(Y), int(M), ctypes.c_void_p(stream))
        if rc != QGEMV_OK:
            raise QGemvError(rc, "qgemv_run_noalloc")

    def tune(self, A: Any, Y: Any, M: Optional[int] = None, with_workspace: bool = False, workspace: Any = None,
             workspace_bytes: Optional[int] = None, rounds: int = 0, reps: int = 0,
             stream: Any = None) -> Dict[str, Any]:
        """qgemv_tune: time the launches that give the automatic plan's bits for M rows
        on these buffers, each call cold (after a read sweep over a 512 MiB buffer the
        call allocates and frees), and keep the fastest in the handle (for qgemv_run, or
        with a workspace for qgemv_run_ws / qgemv_run_noalloc). Waits for its work."""
        if M is None:
            M = int(A.shape[0])
        if workspace is not None and workspace_bytes is None:
            workspace_bytes = int(workspace.numel() * workspace.element_size())
        info = TuneInfo()
        rc = lib().qgemv_tune(self._h, _ptr(A), _ptr(Y), int(M), int(bool(with_workspace)), _ptr(workspace),
                              int(workspace_bytes or 0), int(rounds), int(reps),
                              ctypes.c_void_p(_stream_handle(stream)), ctypes.byref(info))
        if rc != QGEMV_OK:
            raise QGemvError(rc, "qgemv_tune")
        return {"candidates": info.candidates, "rounds": info.rounds, "chosen_flags": info.chosen_flags,
                "auto_us": info.auto_us, "chosen_us": info.chosen_us}

    def workspace_size(self, M: int = MAX_M) -> int:
        """Bytes of workspace qgemv_run_ws needs for M rows (0: none)."""
        out = ctypes.c_size_t()
        rc = lib().qgemv_workspace_size(self._h, int(M), ctypes.byref(out))
        if rc != QGEMV_OK:
            raise QGemvError(rc, "qgemv_workspace_size")
        return int(out.value)

    def plan(self, M: int, with_workspace: bool = False) -> Dict[str, Any]:
        out = PlanInfo()
        rc = lib().qgemv_plan(self._h, int(M), int(bool(with_workspace)), ctypes.byref(out))
        if rc != QGEMV_OK:
            raise QGemvError(rc, "qgemv_plan")
        return _plan_dict(out)

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().qgemv_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def upload(problem, device: str = "cuda:0", flags: int = 0) -> "tuple[QGemv, dict]":
    """Copy a numpy-side problem (see synth.Problem) to device tensors and build the
    handle. Returns (QGemv, tensors) where tensors holds A (as an activation tensor of
    the problem's dtype) and the weight buffers."""
    import numpy as np
    import torch

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)

    t = {"W": dev(problem.W), "scales": dev(problem.scales.view(np.uint8) if problem.scales.dtype != np.float32
                                              else problem.scales)}
    t["zp"] = None if problem.zp is None else dev(problem.zp)
    tdt = torch.float16 if problem.act == "f16" else torch.bfloat16
    t["A"] = dev(problem.A.view(np.int16)).view(tdt)
    bias = getattr(problem, "bias", None)
    t["bias"] = None if bias is None else dev(bias.view(np.int16)).view(tdt)
    q = QGemv(problem.fmt, problem.act, problem.N, problem.K, problem.bs, t["W"], t["scales"], t["zp"],
              problem.tensor_scale, flags, bias=t["bias"])
    return q, t
