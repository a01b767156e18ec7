"""Helpers for the GPU parity tests: upload seeded inputs, run libwq through
its C ABI, compare with the CPU oracle element by element."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from fp8_weight_streaming_amd import inputs

# Acceptance bound of the product: |y_gpu - y| <= TOL * sum_k |w x| per
# element.  The GPU forms every product exactly and rounds only in FP32
# sums over blocks of at most 16 (MFMA) and chunks of at most 8704 k, whose
# worst-case relative error is far below 1e-3.
TOL = 1e-3

DEV = "cuda:0"


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def dev_bf16bits(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).to(DEV)


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def workspace(nbytes: int):
    if nbytes == 0:
        return None
    return torch.zeros(nbytes, dtype=torch.uint8, device=DEV)


def run_nvfp4(wq, d: inputs.NVFP4Inputs, N=None, x=None):
    x = d.x if x is None else x
    N = x.shape[0] if N is None else N
    codes, scales, xd = dev_u8(d.codes), dev_u8(d.scales), dev_bf16bits(x[:N])
    y = torch.full((N, d.M), float("nan"), dtype=torch.float32, device=DEV)
    ws = workspace(wq.wq_gemm_workspace_bytes(wq.WQ_FMT_NVFP4, d.M, d.K, N))
    wq.wq_gemm_nvfp4(codes, scales, d.g, xd, y, ws)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def run_fp8(wq, d: inputs.FP8RowInputs, N=None, x=None):
    x = d.x if x is None else x
    N = x.shape[0] if N is None else N
    w, rs, xd = dev_u8(d.w), dev_f32(d.row_scale), dev_bf16bits(x[:N])
    y = torch.full((N, d.M), float("nan"), dtype=torch.float32, device=DEV)
    ws = workspace(wq.wq_gemm_workspace_bytes(wq.WQ_FMT_FP8ROW, d.M, d.K, N))
    wq.wq_gemm_fp8row(w, rs, xd, y, ws)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def assert_close(y_gpu, y_ref, a_ref, what=""):
    """Element-wise |y_gpu - y| <= TOL * a, NaN exactly where the oracle has NaN."""
    y_gpu = np.asarray(y_gpu, np.float64)
    nan_ref = np.isnan(y_ref)
    assert np.array_equal(np.isnan(y_gpu), nan_ref), "%s: NaN pattern differs" % what
    ok = ~nan_ref
    err = np.abs(y_gpu[ok] - y_ref[ok])
    bound = TOL * a_ref[ok]
    bad = err > bound
    if bad.any():
        i = np.flatnonzero(bad)[0]
        raise AssertionError("%s: %d of %d elements outside |dy| <= %g*a; first: gpu=%r ref=%r a=%r"
                             % (what, int(bad.sum()), bad.size, TOL, y_gpu[ok][i], y_ref[ok][i], a_ref[ok][i]))
    return float((err / np.maximum(bound, 1e-300)).max()) if err.size else 0.0


def check_nvfp4(wq, d, N=None, rows=None, what="nvfp4"):
    y = run_nvfp4(wq, d, N)
    N = y.shape[0]
    yr, ar = oracle.gemm_nvfp4(d.codes, d.scales, d.g, d.x[:N], rows=rows)
    return assert_close(y if rows is None else y[:, rows], yr, ar, what)


def check_fp8(wq, d, N=None, rows=None, what="fp8row"):
    y = run_fp8(wq, d, N)
    N = y.shape[0]
    yr, ar = oracle.gemm_fp8row(d.w, d.row_scale, d.x[:N], rows=rows)
    return assert_close(y if rows is None else y[:, rows], yr, ar, what)
