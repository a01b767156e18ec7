"""ctypes binding of libwq.so: the same entry points as include/wq.h.

This layer only marshals arguments: it takes torch tensors that already
live on the GPU (or raw integer device pointers), passes their addresses,
shapes and the current HIP stream to the C ABI, and raises on a non-zero
status.  All arithmetic runs in the HIP kernels.  There is no fallback: if
libwq.so has not been built, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwq.so")

WQ_FMT_NVFP4 = 0
WQ_FMT_FP8ROW = 1
WQ_FMT_NVFP4_TILED = 2
WQ_FMT_FP8ROW_TILED = 3

STATUS_NAMES = {
    0: "WQ_SUCCESS",
    1: "WQ_ERROR_INVALID_VALUE",
    2: "WQ_ERROR_UNSUPPORTED_SHAPE",
    3: "WQ_ERROR_MISALIGNED",
    4: "WQ_ERROR_WORKSPACE",
    5: "WQ_ERROR_LAUNCH",
    6: "WQ_ERROR_DEVICE",
    7: "WQ_ERROR_SCRATCH_LIMIT",
}


class WQError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (%d)" % (where, STATUS_NAMES.get(status, "unknown"), status))


if not os.path.exists(LIB_PATH):
    raise ImportError("libwq.so is not built; run `python -m fp8_weight_streaming_amd.build` "
                      "(hipcc for gfx950) -- there is no CPU fallback")

_lib = ctypes.CDLL(LIB_PATH)


class WqMatrix(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("M", ctypes.c_int32), ("K", ctypes.c_int32),
                ("global_scale", ctypes.c_float), ("w", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("x", ctypes.c_void_p), ("y", ctypes.c_void_p)]


class WqVerifyPlan(ctypes.Structure):
    _fields_ = [("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t), ("count", ctypes.c_int32),
                ("N", ctypes.c_int32), ("mode", ctypes.c_int32), ("grid", ctypes.c_int32),
                ("ranges_offset", ctypes.c_size_t), ("reduce_offset", ctypes.c_size_t),
                ("reduce_runs", ctypes.c_int32), ("lds_extra", ctypes.c_int32)]


class WqMlpLayer(ctypes.Structure):
    _fields_ = [("gate_up", ctypes.c_void_p), ("down", ctypes.c_void_p), ("gamma", ctypes.c_void_p),
                ("gate_scale", ctypes.c_float), ("up_scale", ctypes.c_float), ("down_scale", ctypes.c_float),
                ("reserved", ctypes.c_int32)]


class WqMlpPlan(ctypes.Structure):
    _fields_ = [("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t), ("h", ctypes.c_void_p),
                ("layers", ctypes.c_int32), ("D", ctypes.c_int32), ("F", ctypes.c_int32), ("N", ctypes.c_int32),
                ("grid_gate_up", ctypes.c_int32), ("grid_down", ctypes.c_int32), ("down_chunks", ctypes.c_int32),
                ("grid_chain", ctypes.c_int32), ("ranges_gate_up_offset", ctypes.c_size_t),
                ("ranges_down_offset", ctypes.c_size_t), ("ssp_offset", ctypes.c_size_t),
                ("ctl_offset", ctypes.c_size_t)]


_P = ctypes.c_void_p
_I = ctypes.c_int
_S = ctypes.c_size_t
_lib.wq_status_string.restype = ctypes.c_char_p
_lib.wq_status_string.argtypes = [_I]
_lib.wq_gemm_workspace_bytes.restype = _S
_lib.wq_gemm_workspace_bytes.argtypes = [_I, _I, _I, _I]
_lib.wq_gemm_split.restype = _I
_lib.wq_gemm_split.argtypes = [_I, _I, _I, _I, ctypes.POINTER(_I), ctypes.POINTER(_I)]
_lib.wq_gemm_nvfp4.restype = _I
_lib.wq_gemm_nvfp4.argtypes = [_P, _P, ctypes.c_float, _P, _P, _I, _I, _I, _P, _S, _P]
_lib.wq_gemm_fp8row.restype = _I
_lib.wq_gemm_fp8row.argtypes = [_P, _P, _P, _P, _I, _I, _I, _P, _S, _P]
_lib.wq_verify_workspace_bytes.restype = _S
_lib.wq_verify_workspace_bytes.argtypes = [ctypes.POINTER(WqMatrix), _I, _I]
_lib.wq_verify_pass.restype = _I
_lib.wq_verify_pass.argtypes = [ctypes.POINTER(WqMatrix), _I, _I, _P, _S, _P]

_lib.wq_verify_prepare.restype = _I
_lib.wq_verify_prepare.argtypes = [ctypes.POINTER(WqMatrix), _I, _I, _P, _S, _P, ctypes.POINTER(WqVerifyPlan)]
_lib.wq_verify_launch.restype = _I
_lib.wq_verify_launch.argtypes = [ctypes.POINTER(WqVerifyPlan), _P]

_lib.wq_probe_sink_words.restype = _S
_lib.wq_probe_sink_words.argtypes = []
_lib.wq_probe_read.restype = _I
_lib.wq_probe_read.argtypes = [_P, _S, _P, _P]
_lib.wq_probe_copy.restype = _I
_lib.wq_probe_copy.argtypes = [_P, _P, _S, _P]
_lib.wq_probe_read_write_bytes.restype = _S
_lib.wq_probe_read_write_bytes.argtypes = [_S, _I]
_lib.wq_probe_read_write.restype = _I
_lib.wq_probe_read_write.argtypes = [_P, _S, _P, _I, _P, _P]

_lib.wq_nvfp4_tiled_bytes.restype = _S
_lib.wq_nvfp4_tiled_bytes.argtypes = [_I, _I]
_lib.wq_nvfp4_tile.restype = _I
_lib.wq_nvfp4_tile.argtypes = [_P, _P, _I, _I, _P, _P]
_lib.wq_nvfp4_untile.restype = _I
_lib.wq_nvfp4_untile.argtypes = [_P, _I, _I, _P, _P, _P]
_lib.wq_gemm_nvfp4_tiled.restype = _I
_lib.wq_gemm_nvfp4_tiled.argtypes = [_P, ctypes.c_float, _P, _P, _I, _I, _I, _P, _S, _P]
_lib.wq_gemm_nvfp4_tiled_noalloc.restype = _I
_lib.wq_gemm_nvfp4_tiled_noalloc.argtypes = [_P, ctypes.c_float, _P, _P, _I, _I, _I, _P]
_lib.wq_fp8_tiled_bytes.restype = _S
_lib.wq_fp8_tiled_bytes.argtypes = [_I, _I]
_lib.wq_fp8_tile.restype = _I
_lib.wq_fp8_tile.argtypes = [_P, _I, _I, _P, _P]
_lib.wq_fp8_untile.restype = _I
_lib.wq_fp8_untile.argtypes = [_P, _I, _I, _P, _P]
_lib.wq_head_accept_workspace_bytes.restype = _S
_lib.wq_head_accept_workspace_bytes.argtypes = [_I, _I, _I, _I]
_lib.wq_head_accept.restype = _I
_lib.wq_head_accept.argtypes = [_I, _P, _P, ctypes.c_float, _P, _I, _I, _I, _P, _P, _P, _P, _P, _S, _P]
_lib.wq_quantize_fp8row.restype = _I
_lib.wq_quantize_fp8row.argtypes = [_P, _I, _I, _P, _P, _P]
_lib.wq_quantize_nvfp4.restype = _I
_lib.wq_quantize_nvfp4.argtypes = [_P, _I, _I, ctypes.c_float, _P, _P, _P]
_lib.wq_verify_launch_valu.restype = _I
_lib.wq_verify_launch_valu.argtypes = [ctypes.POINTER(WqVerifyPlan), _P]
_lib.wq_verify_launch_n.restype = _I
_lib.wq_verify_launch_n.argtypes = [ctypes.POINTER(WqVerifyPlan), _P, _P]
_lib.wq_gemm_fp8row_tiled.restype = _I
_lib.wq_gemm_fp8row_tiled.argtypes = [_P, _P, _P, _P, _I, _I, _I, _P, _S, _P]
_lib.wq_nvfp4_tile_glu.restype = _I
_lib.wq_nvfp4_tile_glu.argtypes = [_P, _P, _P, _P, _I, _I, _P, _P]
_lib.wq_mlp_chain_workspace_bytes.restype = _S
_lib.wq_mlp_chain_workspace_bytes.argtypes = [_I, _I, _I, _I]
_lib.wq_mlp_chain_split.restype = _I
_lib.wq_mlp_chain_split.argtypes = [_I, _I, ctypes.POINTER(_I), ctypes.POINTER(_I)]
_lib.wq_mlp_chain_prepare.restype = _I
_lib.wq_mlp_chain_prepare.argtypes = [ctypes.POINTER(WqMlpLayer), _I, _I, _I, _I, ctypes.c_float, _P, _P, _P, _P,
                                      _S, _P, ctypes.POINTER(WqMlpPlan)]
_lib.wq_mlp_chain_launch.restype = _I
_lib.wq_mlp_chain_launch.argtypes = [ctypes.POINTER(WqMlpPlan), _P]
_lib.wq_mlp_chain_launch_persistent.restype = _I
_lib.wq_mlp_chain_launch_persistent.argtypes = [ctypes.POINTER(WqMlpPlan), _P]

EXPORTED = ["wq_nvfp4_tiled_bytes", "wq_nvfp4_tile", "wq_nvfp4_untile", "wq_gemm_nvfp4_tiled",
            "wq_gemm_nvfp4_tiled_noalloc", "wq_status_string", "wq_gemm_workspace_bytes", "wq_gemm_split", "wq_gemm_nvfp4", "wq_gemm_fp8row",
            "wq_fp8_tiled_bytes", "wq_fp8_tile", "wq_fp8_untile", "wq_gemm_fp8row_tiled",
            "wq_head_accept_workspace_bytes", "wq_head_accept", "wq_quantize_fp8row", "wq_quantize_nvfp4",
            "wq_verify_launch_n", "wq_verify_launch_valu", "wq_nvfp4_tile_glu", "wq_mlp_chain_workspace_bytes", "wq_mlp_chain_split",
            "wq_mlp_chain_prepare", "wq_mlp_chain_launch", "wq_mlp_chain_launch_persistent",
            "wq_verify_workspace_bytes", "wq_verify_pass", "wq_verify_prepare", "wq_verify_launch",
            "wq_probe_sink_words", "wq_probe_read", "wq_probe_copy", "wq_probe_read_write_bytes",
            "wq_probe_read_write"]


def lib() -> ctypes.CDLL:
    return _lib


def _ptr(t) -> int:
    if t is None:
        return 0
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("libwq takes device tensors only")
    if not t.is_contiguous():
        raise ValueError("libwq takes contiguous tensors only")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str):
    if status != 0:
        raise WQError(status, where)


def _nbytes(t) -> int:
    return 0 if t is None or isinstance(t, int) else t.numel() * t.element_size()


def wq_status_string(status: int) -> str:
    return _lib.wq_status_string(status).decode()


def wq_gemm_workspace_bytes(fmt: int, M: int, K: int, N: int) -> int:
    """Workspace bytes of a single-matrix call (0: none).  Allocate it zeroed
    (torch.zeros): its first 16 KiB are arrival counters that every call
    leaves at zero, so one buffer serves any later single-matrix call."""
    return int(_lib.wq_gemm_workspace_bytes(fmt, M, K, N))


def wq_gemm_split(fmt: int, M: int, K: int, in_verify_pass: int = 0):
    """(k_chunk, n_chunks) the call would use (in_verify_pass: 0 single call, 1 or True in a verify pass,
    2 computed in blocks in a verify pass)."""
    kc, nc = _I(0), _I(0)
    _check(_lib.wq_gemm_split(fmt, M, K, int(in_verify_pass), ctypes.byref(kc), ctypes.byref(nc)),
           "wq_gemm_split")
    return kc.value, nc.value


def wq_gemm_nvfp4(codes, scales, global_scale: float, x, y, workspace=None, stream=None,
                  M: Optional[int] = None, K: Optional[int] = None, N: Optional[int] = None,
                  workspace_bytes: Optional[int] = None):
    """y[N, M] = x[N, K] . W^T for NVFP4 W (codes uint8 [M, K/2], scales uint8 [M, K/16]).

    Tensors are torch device tensors (x as int16/uint16/bfloat16 bits, y float32);
    shapes are taken from them unless given explicitly (raw-pointer use)."""
    if M is None:
        M = codes.shape[0]
    if K is None:
        K = 2 * codes.shape[1]
    if N is None:
        N = x.shape[0]
    wsb = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    _check(_lib.wq_gemm_nvfp4(_ptr(codes), _ptr(scales), float(global_scale), _ptr(x), _ptr(y), M, K, N,
                              _ptr(workspace), wsb, _stream(stream)), "wq_gemm_nvfp4")


def wq_nvfp4_tiled_bytes(M: int, K: int) -> int:
    return int(_lib.wq_nvfp4_tiled_bytes(M, K))


def wq_nvfp4_tile(codes, scales, tiled, stream=None, M: Optional[int] = None, K: Optional[int] = None):
    """Permute plain NVFP4 codes/scales into the tiled layout (on the GPU)."""
    if M is None:
        M = codes.shape[0]
    if K is None:
        K = 2 * codes.shape[1]
    _check(_lib.wq_nvfp4_tile(_ptr(codes), _ptr(scales), M, K, _ptr(tiled), _stream(stream)), "wq_nvfp4_tile")


def wq_nvfp4_untile(tiled, codes, scales, stream=None, M: Optional[int] = None, K: Optional[int] = None):
    """Inverse of wq_nvfp4_tile."""
    if M is None:
        M = codes.shape[0]
    if K is None:
        K = 2 * codes.shape[1]
    _check(_lib.wq_nvfp4_untile(_ptr(tiled), M, K, _ptr(codes), _ptr(scales), _stream(stream)), "wq_nvfp4_untile")


def wq_gemm_nvfp4_tiled(tiled, global_scale: float, x, y, M: int, K: int, workspace=None, stream=None,
                        N: Optional[int] = None, workspace_bytes: Optional[int] = None):
    """y[N, M] = x[N, K] . W^T for NVFP4 W in the tiled layout."""
    if N is None:
        N = x.shape[0]
    wsb = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    _check(_lib.wq_gemm_nvfp4_tiled(_ptr(tiled), float(global_scale), _ptr(x), _ptr(y), M, K, N, _ptr(workspace),
                                    wsb, _stream(stream)), "wq_gemm_nvfp4_tiled")


def wq_gemm_nvfp4_tiled_noalloc(tiled, global_scale: float, x, y, M: int, K: int, stream=None,
                                N: Optional[int] = None):
    """wq_gemm_nvfp4_tiled with its split-K scratch in the library's static
    device buffer (no workspace argument, nothing allocated)."""
    if N is None:
        N = x.shape[0]
    _check(_lib.wq_gemm_nvfp4_tiled_noalloc(_ptr(tiled), float(global_scale), _ptr(x), _ptr(y), M, K, N,
                                            _stream(stream)), "wq_gemm_nvfp4_tiled_noalloc")


NOALLOC_SCRATCH_BYTES = 4 << 20  # WQ_NOALLOC_SCRATCH_BYTES in include/wq.h


def wq_gemm_fp8row(w, row_scale, x, y, workspace=None, stream=None, M: Optional[int] = None,
                   K: Optional[int] = None, N: Optional[int] = None, workspace_bytes: Optional[int] = None):
    """y[N, M] = x[N, K] . W^T for row-scaled FP8 W (w uint8 [M, K], row_scale float32 [M])."""
    if M is None:
        M = w.shape[0]
    if K is None:
        K = w.shape[1]
    if N is None:
        N = x.shape[0]
    wsb = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    _check(_lib.wq_gemm_fp8row(_ptr(w), _ptr(row_scale), _ptr(x), _ptr(y), M, K, N, _ptr(workspace), wsb,
                               _stream(stream)), "wq_gemm_fp8row")


@dataclass
class Matrix:
    """One matrix of a verify pass (device tensors or raw pointers)."""
    fmt: int
    M: int
    K: int
    w: object
    scales: object
    x: object
    y: object
    global_scale: float = 1.0


def _descs(mats: Sequence[Matrix]):
    arr = (WqMatrix * len(mats))()
    for i, m in enumerate(mats):
        arr[i] = WqMatrix(m.fmt, m.M, m.K, float(m.global_scale), _ptr(m.w), _ptr(m.scales), _ptr(m.x),
                          _ptr(m.y))
    return arr


def wq_verify_workspace_bytes(mats: Sequence[Matrix], N: int) -> int:
    arr = _descs(mats)
    return int(_lib.wq_verify_workspace_bytes(arr, len(mats), N))


def wq_verify_pass(mats: Sequence[Matrix], N: int, workspace, stream=None, workspace_bytes: Optional[int] = None):
    """All matrices at N columns in one persistent launch."""
    arr = _descs(mats)
    wsb = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    _check(_lib.wq_verify_pass(arr, len(mats), N, _ptr(workspace), wsb, _stream(stream)), "wq_verify_pass")


def wq_verify_prepare(mats: Sequence[Matrix], N: int, workspace, stream=None,
                      workspace_bytes: Optional[int] = None) -> WqVerifyPlan:
    """Write the pass's device table into `workspace`; returns the plan."""
    arr = _descs(mats)
    plan = WqVerifyPlan()
    wsb = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    _check(_lib.wq_verify_prepare(arr, len(mats), N, _ptr(workspace), wsb, _stream(stream), ctypes.byref(plan)),
           "wq_verify_prepare")
    return plan


def wq_probe_sink_words() -> int:
    return int(_lib.wq_probe_sink_words())


def wq_probe_read(src, sink, stream=None, nbytes: Optional[int] = None):
    """Stream `src` (device tensor) once with the weight stream's loads."""
    nb = _nbytes(src) if nbytes is None else nbytes
    _check(_lib.wq_probe_read(_ptr(src), nb, _ptr(sink), _stream(stream)), "wq_probe_read")


def wq_probe_read_write_bytes(nbytes: int, every_kb: int) -> int:
    return int(_lib.wq_probe_read_write_bytes(nbytes, every_kb))


def wq_probe_read_write(src, dst, every_kb: int, sink, stream=None, nbytes: Optional[int] = None):
    """Stream `src` once, writing 256 bytes per wave to `dst` every `every_kb` KB read."""
    nb = _nbytes(src) if nbytes is None else nbytes
    _check(_lib.wq_probe_read_write(_ptr(src), nb, _ptr(dst), every_kb, _ptr(sink), _stream(stream)),
           "wq_probe_read_write")


def wq_probe_copy(src, dst, stream=None, nbytes: Optional[int] = None):
    """Copy `src` to `dst` (device tensors of equal size)."""
    nb = _nbytes(src) if nbytes is None else nbytes
    _check(_lib.wq_probe_copy(_ptr(src), _ptr(dst), nb, _stream(stream)), "wq_probe_copy")


def wq_verify_launch(plan: WqVerifyPlan, stream=None):
    """Launch a prepared pass (kernel launch only)."""
    _check(_lib.wq_verify_launch(ctypes.byref(plan), _stream(stream)), "wq_verify_launch")


def wq_fp8_tiled_bytes(M: int, K: int) -> int:
    return int(_lib.wq_fp8_tiled_bytes(M, K))


def wq_fp8_tile(w, tiled, stream=None, M: Optional[int] = None, K: Optional[int] = None):
    """Permute plain FP8-row bytes (uint8 [M, K]) into the tiled layout (on the GPU)."""
    if M is None:
        M = w.shape[0]
    if K is None:
        K = w.shape[1]
    _check(_lib.wq_fp8_tile(_ptr(w), M, K, _ptr(tiled), _stream(stream)), "wq_fp8_tile")


def wq_fp8_untile(tiled, w, stream=None, M: Optional[int] = None, K: Optional[int] = None):
    """Inverse of wq_fp8_tile."""
    if M is None:
        M = w.shape[0]
    if K is None:
        K = w.shape[1]
    _check(_lib.wq_fp8_untile(_ptr(tiled), M, K, _ptr(w), _stream(stream)), "wq_fp8_untile")


def wq_gemm_fp8row_tiled(tiled, row_scale, x, y, M: int, K: int, workspace=None, stream=None,
                         N: Optional[int] = None, workspace_bytes: Optional[int] = None):
    """y[N, M] = x[N, K] . W^T for row-scaled FP8 W in the tiled layout."""
    if N is None:
        N = x.shape[0]
    wsb = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    _check(_lib.wq_gemm_fp8row_tiled(_ptr(tiled), _ptr(row_scale), _ptr(x), _ptr(y), M, K, N, _ptr(workspace), wsb,
                                     _stream(stream)), "wq_gemm_fp8row_tiled")


def wq_head_accept_workspace_bytes(fmt: int, M: int, K: int, N: int) -> int:
    return int(_lib.wq_head_accept_workspace_bytes(fmt, M, K, N))


def wq_head_accept(fmt: int, w, row_scale, global_scale: float, x, M: int, K: int, drafts, tokens, accepted,
                   logits=None, workspace=None, stream=None, N: Optional[int] = None,
                   workspace_bytes: Optional[int] = None):
    """Greedy acceptance on a tiled head: tokens[N] = per-column greedy rows,
    accepted[1] = leading drafts equal to the previous column's token."""
    if N is None:
        N = x.shape[0]
    wsb = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    _check(_lib.wq_head_accept(fmt, _ptr(w), _ptr(row_scale), float(global_scale), _ptr(x), M, K, N, _ptr(drafts),
                               _ptr(logits), _ptr(tokens), _ptr(accepted), _ptr(workspace), wsb, _stream(stream)),
           "wq_head_accept")


def wq_quantize_fp8row(w, q, row_scale, stream=None, M: Optional[int] = None, K: Optional[int] = None):
    """BF16 bits [M, K] -> E4M3 bytes q [M, K] and FP32 row scales [M] (round to nearest)."""
    if M is None:
        M = w.shape[0]
    if K is None:
        K = w.shape[1]
    _check(_lib.wq_quantize_fp8row(_ptr(w), M, K, _ptr(q), _ptr(row_scale), _stream(stream)), "wq_quantize_fp8row")


def wq_quantize_nvfp4(w, global_scale: float, codes, scales, stream=None, M: Optional[int] = None,
                      K: Optional[int] = None):
    """BF16 bits [M, K] -> NVFP4 codes [M, K/2] and E4M3 block scales [M, K/16] (round to nearest)."""
    if M is None:
        M = w.shape[0]
    if K is None:
        K = w.shape[1]
    _check(_lib.wq_quantize_nvfp4(_ptr(w), M, K, float(global_scale), _ptr(codes), _ptr(scales), _stream(stream)),
           "wq_quantize_nvfp4")


def wq_verify_launch_valu(plan: WqVerifyPlan, stream=None):
    """Launch a prepared tiled pass with its NVFP4 steps on the vector ALUs
    (the matrix-core comparison)."""
    _check(_lib.wq_verify_launch_valu(ctypes.byref(plan), _stream(stream)), "wq_verify_launch_valu")


def wq_verify_launch_n(plan: WqVerifyPlan, n_device, stream=None):
    """Launch a plan prepared for N = 8 with the column count read from the
    int32 device tensor n_device when the kernels run."""
    _check(_lib.wq_verify_launch_n(ctypes.byref(plan), _ptr(n_device), _stream(stream)), "wq_verify_launch_n")


def wq_nvfp4_tile_glu(gate_codes, gate_scales, up_codes, up_scales, tiled, stream=None,
                      F: Optional[int] = None, D: Optional[int] = None):
    """Interleave gate/up NVFP4 weights [F][D] into the chain's tiled layout."""
    if F is None:
        F = gate_codes.shape[0]
    if D is None:
        D = 2 * gate_codes.shape[1]
    _check(_lib.wq_nvfp4_tile_glu(_ptr(gate_codes), _ptr(gate_scales), _ptr(up_codes), _ptr(up_scales), F, D,
                                  _ptr(tiled), _stream(stream)), "wq_nvfp4_tile_glu")


class MlpLayer:
    """One chained layer's device buffers (tensors or raw pointers)."""

    def __init__(self, gate_up, down, gamma, gate_scale: float, up_scale: float, down_scale: float):
        self.gate_up, self.down, self.gamma = gate_up, down, gamma
        self.gate_scale, self.up_scale, self.down_scale = gate_scale, up_scale, down_scale


def wq_mlp_chain_workspace_bytes(layers: int, D: int, F: int, N: int) -> int:
    return int(_lib.wq_mlp_chain_workspace_bytes(layers, D, F, N))


def wq_mlp_chain_split(D: int, F: int):
    kc, nc = _I(0), _I(0)
    _check(_lib.wq_mlp_chain_split(D, F, ctypes.byref(kc), ctypes.byref(nc)), "wq_mlp_chain_split")
    return kc.value, nc.value


def wq_mlp_chain_prepare(layers: Sequence[MlpLayer], D: int, F: int, N: int, eps: float, h, a, s, workspace,
                         stream=None, workspace_bytes: Optional[int] = None) -> WqMlpPlan:
    """Write the chain's device table into `workspace`; returns the plan."""
    arr = (WqMlpLayer * max(1, len(layers)))()
    for i, y in enumerate(layers):
        arr[i] = WqMlpLayer(_ptr(y.gate_up), _ptr(y.down), _ptr(y.gamma), float(y.gate_scale), float(y.up_scale),
                            float(y.down_scale), 0)
    plan = WqMlpPlan()
    wsb = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    _check(_lib.wq_mlp_chain_prepare(arr, len(layers), D, F, N, float(eps), _ptr(h), _ptr(a), _ptr(s),
                                     _ptr(workspace), wsb, _stream(stream), ctypes.byref(plan)),
           "wq_mlp_chain_prepare")
    return plan


def wq_mlp_chain_launch(plan: WqMlpPlan, stream=None):
    """Run the prepared layers (launches only); updates h in place."""
    _check(_lib.wq_mlp_chain_launch(ctypes.byref(plan), _stream(stream)), "wq_mlp_chain_launch")


def wq_mlp_chain_launch_persistent(plan: WqMlpPlan, stream=None):
    """Run the prepared layers in one cooperative launch; updates h in place."""
    _check(_lib.wq_mlp_chain_launch_persistent(ctypes.byref(plan), _stream(stream)), "wq_mlp_chain_launch_persistent")
