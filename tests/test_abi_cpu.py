"""The C ABI library on the host: it loads, exports every function that
include/wq.h declares, and rejects bad arguments before touching the GPU.

Nothing here launches a kernel; the validation paths return their status
without any HIP call, so these tests run on a machine with no GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wq.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(wq_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def wq():
    from fp8_weight_streaming_amd import wq as mod
    return mod


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["wq_gemm_nvfp4", "wq_gemm_fp8row", "wq_verify_pass", "wq_gemm_workspace_bytes",
              "wq_verify_workspace_bytes", "wq_status_string", "wq_gemm_split"]:
        assert n in names


def test_library_exports_every_declared_symbol(wq):
    lib = ctypes.CDLL(wq.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert sorted(wq.EXPORTED) == declared_functions()


def test_status_strings(wq):
    assert wq.wq_status_string(0) == "success"
    for s in range(1, 8):
        assert wq.wq_status_string(s) not in ("", "unknown status")
    assert wq.wq_status_string(99) == "unknown status"


FAKE = 1 << 20          # 16-byte aligned fake device address; never dereferenced
MISALIGNED = FAKE + 4


def nv(lib, codes=FAKE, scales=FAKE, x=FAKE, y=FAKE, M=64, K=128, N=4, ws=0, wsb=0):
    return lib.wq_gemm_nvfp4(codes, scales, 1.0, x, y, M, K, N, ws, wsb, 0)


def fp8(lib, w=FAKE, rs=FAKE, x=FAKE, y=FAKE, M=64, K=128, N=4, ws=0, wsb=0):
    return lib.wq_gemm_fp8row(w, rs, x, y, M, K, N, ws, wsb, 0)


def test_gemm_argument_errors(wq):
    lib = wq.lib()
    INV, SHAPE, MIS = 1, 2, 3
    assert nv(lib, codes=0) == INV
    assert nv(lib, scales=0) == INV
    assert nv(lib, x=0) == INV
    assert nv(lib, y=0) == INV
    assert nv(lib, N=0) == INV and nv(lib, N=9) == INV and nv(lib, N=-1) == INV
    assert nv(lib, M=0) == INV and nv(lib, K=0) == INV
    assert nv(lib, K=48) == SHAPE and nv(lib, K=16) == SHAPE and nv(lib, K=(1 << 24) + 32) == SHAPE
    assert nv(lib, M=1 << 30, K=1 << 12) == SHAPE
    assert nv(lib, codes=MISALIGNED) == MIS and nv(lib, y=MISALIGNED) == MIS and nv(lib, x=FAKE + 8) == MIS
    assert fp8(lib, w=0) == INV and fp8(lib, rs=0) == INV
    assert fp8(lib, K=40) == SHAPE and fp8(lib, K=8) == SHAPE
    assert fp8(lib, rs=MISALIGNED) == MIS
    assert fp8(lib, N=9) == INV


def test_verify_argument_errors(wq):
    lib = wq.lib()
    good = wq.WqMatrix(0, 64, 128, 1.0, FAKE, FAKE, FAKE, FAKE)
    arr = (wq.WqMatrix * 2)(good, good)
    assert lib.wq_verify_pass(arr, 0, 4, FAKE, 1 << 20, 0) == 1
    assert lib.wq_verify_pass(None, 2, 4, FAKE, 1 << 20, 0) == 1
    assert lib.wq_verify_pass(arr, 2, 0, FAKE, 1 << 20, 0) == 1
    assert lib.wq_verify_pass(arr, 2, 4, 0, 1 << 20, 0) == 4
    assert lib.wq_verify_pass(arr, 2, 4, MISALIGNED, 1 << 20, 0) == 3
    arr[1] = wq.WqMatrix(0, 64, 96 + 8, 1.0, FAKE, FAKE, FAKE, FAKE)
    assert lib.wq_verify_pass(arr, 2, 4, FAKE, 1 << 20, 0) == 2
    arr[1] = wq.WqMatrix(1, 64, 96, 1.0, FAKE, 0, FAKE, FAKE)
    assert lib.wq_verify_pass(arr, 2, 4, FAKE, 1 << 20, 0) == 1
    arr[1] = wq.WqMatrix(7, 64, 96, 1.0, FAKE, FAKE, FAKE, FAKE)
    assert lib.wq_verify_pass(arr, 2, 4, FAKE, 1 << 20, 0) == 1
    assert lib.wq_verify_workspace_bytes(arr, 2, 4) == 0  # invalid descriptor -> 0


def test_split_query_rejects_bad_args(wq):
    lib = wq.lib()
    kc, nc = ctypes.c_int(0), ctypes.c_int(0)
    assert lib.wq_gemm_split(0, 64, 48, 1, ctypes.byref(kc), ctypes.byref(nc)) == 2
    assert lib.wq_gemm_split(0, 64, 128, 1, None, ctypes.byref(nc)) == 1
    # inside a verify pass the split depends only on (M, K): no device needed
    assert lib.wq_gemm_split(0, 5120, 17408, 1, ctypes.byref(kc), ctypes.byref(nc)) == 0
    assert (kc.value, nc.value) == (8704, 2)
    assert lib.wq_gemm_split(0, 7168, 5120, 1, ctypes.byref(kc), ctypes.byref(nc)) == 0
    assert (kc.value, nc.value) == (5120, 1)
    assert lib.wq_gemm_split(1, 151936, 5120, 1, ctypes.byref(kc), ctypes.byref(nc)) == 0
    assert (kc.value, nc.value) == (5120, 1)
    # computed in blocks inside a verify pass (tiled formats): chunks of at
    # most 6144 k, whole 256-k steps, as even as that allows
    assert lib.wq_gemm_split(2, 5120, 17408, 2, ctypes.byref(kc), ctypes.byref(nc)) == 0
    assert (kc.value, nc.value) == (5888, 3)
    assert lib.wq_gemm_split(2, 150000, 8736, 2, ctypes.byref(kc), ctypes.byref(nc)) == 0
    assert (kc.value, nc.value) == (4608, 2)
    assert lib.wq_gemm_split(3, 64, 17424, 2, ctypes.byref(kc), ctypes.byref(nc)) == 0
    assert (kc.value, nc.value) == (5888, 3)


def fp8t(lib, w=FAKE, rs=FAKE, x=FAKE, y=FAKE, M=64, K=128, N=4, ws=0, wsb=0):
    return lib.wq_gemm_fp8row_tiled(w, rs, x, y, M, K, N, ws, wsb, 0)


def test_fp8_tiled_argument_errors(wq):
    lib = wq.lib()
    INV, SHAPE, MIS = 1, 2, 3
    assert fp8t(lib, w=0) == INV and fp8t(lib, rs=0) == INV and fp8t(lib, x=0) == INV and fp8t(lib, y=0) == INV
    assert fp8t(lib, N=0) == INV and fp8t(lib, N=9) == INV and fp8t(lib, M=0) == INV
    assert fp8t(lib, K=40) == SHAPE and fp8t(lib, K=8) == SHAPE
    assert fp8t(lib, M=1 << 30, K=1 << 12) == SHAPE  # tiled buffer past 32-bit offsets
    assert fp8t(lib, w=MISALIGNED) == MIS and fp8t(lib, rs=MISALIGNED) == MIS
    # conversions: sizes, and errors before any launch
    assert lib.wq_fp8_tiled_bytes(17, 48) == 2 * 1 * 2048
    assert lib.wq_fp8_tiled_bytes(151936, 5120) == 9496 * 40 * 2048
    assert lib.wq_fp8_tiled_bytes(16, 40) == 0 and lib.wq_fp8_tiled_bytes(0, 128) == 0
    assert lib.wq_fp8_tile(0, 16, 128, FAKE, 0) == INV and lib.wq_fp8_tile(FAKE, 16, 128, 0, 0) == INV
    assert lib.wq_fp8_tile(FAKE, 16, 40, FAKE, 0) == SHAPE and lib.wq_fp8_tile(MISALIGNED, 16, 128, FAKE, 0) == MIS
    assert lib.wq_fp8_untile(FAKE, 16, 128, 0, 0) == INV and lib.wq_fp8_untile(FAKE, 16, 40, FAKE, 0) == SHAPE
    # in a verify pass the tiled FP8 descriptor needs its row scales
    good = wq.WqMatrix(3, 64, 128, 1.0, FAKE, FAKE, FAKE, FAKE)
    arr = (wq.WqMatrix * 2)(good, good)
    arr[1] = wq.WqMatrix(3, 64, 128, 1.0, FAKE, 0, FAKE, FAKE)
    assert lib.wq_verify_pass(arr, 2, 4, FAKE, 1 << 20, 0) == INV
    kc, nc = ctypes.c_int(0), ctypes.c_int(0)
    assert lib.wq_gemm_split(3, 151936, 5120, 1, ctypes.byref(kc), ctypes.byref(nc)) == 0
    assert (kc.value, nc.value) == (5120, 1)
    assert lib.wq_gemm_split(3, 64, 17408, 1, ctypes.byref(kc), ctypes.byref(nc)) == 0
    assert (kc.value, nc.value) == (8704, 2)


def head(lib, fmt=3, w=FAKE, rs=FAKE, x=FAKE, M=1000, K=1024, N=4, drafts=FAKE, logits=FAKE, tokens=FAKE,
         accepted=FAKE, ws=FAKE, wsb=1 << 20):
    return lib.wq_head_accept(fmt, w, rs, 1.0, x, M, K, N, drafts, logits, tokens, accepted, ws, wsb, 0)


def test_head_accept_argument_errors(wq):
    lib = wq.lib()
    INV, SHAPE, MIS = 1, 2, 3
    assert head(lib, fmt=1) == INV and head(lib, fmt=0) == INV          # tiled heads only
    assert head(lib, w=0) == INV and head(lib, x=0) == INV
    assert head(lib, tokens=0) == INV and head(lib, accepted=0) == INV
    assert head(lib, rs=0) == INV                                        # FP8 head needs its row scales
    assert head(lib, drafts=0) == INV and head(lib, N=9) == INV and head(lib, N=0) == INV
    assert head(lib, K=40) == SHAPE
    assert head(lib, K=17408) == SHAPE                                   # more than one K chunk
    assert head(lib, tokens=FAKE + 2) == MIS and head(lib, logits=FAKE + 4) == MIS and head(lib, w=FAKE + 8) == MIS
    assert lib.wq_head_accept_workspace_bytes(1, 1000, 1024, 4) == 0
    assert lib.wq_head_accept_workspace_bytes(3, 1000, 17408, 4) == 0


def test_quantizer_argument_errors(wq):
    lib = wq.lib()
    INV, SHAPE, MIS = 1, 2, 3
    q8 = lib.wq_quantize_fp8row
    assert q8(0, 16, 64, FAKE, FAKE, 0) == INV and q8(FAKE, 16, 64, 0, FAKE, 0) == INV
    assert q8(FAKE, 16, 64, FAKE, 0, 0) == INV and q8(FAKE, 0, 64, FAKE, FAKE, 0) == INV
    assert q8(FAKE, 16, 40, FAKE, FAKE, 0) == SHAPE and q8(MISALIGNED, 16, 64, FAKE, FAKE, 0) == MIS
    q4 = lib.wq_quantize_nvfp4
    assert q4(FAKE, 16, 64, 0.0, FAKE, FAKE, 0) == INV and q4(FAKE, 16, 64, -1.0, FAKE, FAKE, 0) == INV
    assert q4(FAKE, 16, 64, float("inf"), FAKE, FAKE, 0) == INV and q4(FAKE, 16, 64, float("nan"), FAKE, FAKE, 0) == INV
    assert q4(0, 16, 64, 1.0, FAKE, FAKE, 0) == INV and q4(FAKE, 16, 48, 1.0, FAKE, FAKE, 0) == SHAPE
    assert q4(FAKE, 16, 64, 1.0, FAKE + 8, FAKE, 0) == MIS


def test_device_n_launch_argument_errors(wq):
    lib = wq.lib()
    plan = wq.WqVerifyPlan()
    plan.workspace, plan.workspace_bytes, plan.count, plan.N, plan.mode, plan.grid = FAKE, 1 << 20, 2, 8, 4, 1
    plan.ranges_offset = 256
    import ctypes as C
    assert lib.wq_verify_launch_n(None, FAKE, 0) == 1
    assert lib.wq_verify_launch_n(C.byref(plan), 0, 0) == 1           # no device count
    assert lib.wq_verify_launch_n(C.byref(plan), FAKE + 2, 0) == 1     # misaligned count
    plan.N = 4
    assert lib.wq_verify_launch_n(C.byref(plan), FAKE, 0) == 1         # plan not prepared for N = 8
    plan.N, plan.mode = 8, 3
    assert lib.wq_verify_launch_n(C.byref(plan), FAKE, 0) == 1         # not an all-tiled plan


def test_verify_launch_rejects_bad_lds_extra(wq):
    # a blocked plan's workgroups have all the LDS: lds_extra is either 0 or
    # exactly what brings the launch to the limit, and only for the tiled kernel
    import ctypes as C
    lib = wq.lib()
    plan = wq.WqVerifyPlan()
    plan.workspace, plan.workspace_bytes, plan.count, plan.N, plan.mode, plan.grid = FAKE, 1 << 20, 2, 8, 4, 1
    plan.ranges_offset = 256
    for extra in (512, 123, -512, 1 << 20):
        plan.lds_extra = extra
        assert lib.wq_verify_launch(C.byref(plan), 0) == 1
        assert lib.wq_verify_launch_n(C.byref(plan), FAKE, 0) == 1
    plan.mode, plan.N, plan.lds_extra = 0, 2, 512
    assert lib.wq_verify_launch(C.byref(plan), 0) == 1                 # blocked LDS on a plain-layout plan


def test_chain_argument_errors(wq):
    import ctypes as C
    lib = wq.lib()
    INV, SHAPE, MIS, WS, DEVERR = 1, 2, 3, 4, 6
    layer = wq.WqMlpLayer(FAKE, FAKE, FAKE, 1.0, 1.0, 1.0, 0)
    arr = (wq.WqMlpLayer * 2)(layer, layer)
    plan = wq.WqMlpPlan()

    def prep(count=2, D=256, F=512, N=4, eps=1e-6, h=FAKE, a=FAKE, s=FAKE, ws=FAKE, wsb=1 << 30, layers=arr,
             p=C.byref(plan)):
        return lib.wq_mlp_chain_prepare(layers, count, D, F, N, eps, h, a, s, ws, wsb, 0, p)

    assert prep(p=None) == INV and prep(layers=None) == INV
    assert prep(count=0) == INV and prep(N=0) == INV and prep(N=9) == INV
    assert prep(D=48) == SHAPE and prep(F=40) == SHAPE and prep(D=8736) == SHAPE      # D past one LDS chunk
    assert prep(eps=-1.0) == INV and prep(eps=float("inf")) == INV and prep(eps=float("nan")) == INV
    assert prep(h=0) == INV and prep(a=0) == INV and prep(s=0) == INV
    assert prep(h=MISALIGNED) == MIS and prep(s=FAKE + 2) == MIS
    bad = (wq.WqMlpLayer * 2)(layer, wq.WqMlpLayer(FAKE, 0, FAKE, 1.0, 1.0, 1.0, 0))
    assert prep(layers=bad) == INV
    bad = (wq.WqMlpLayer * 2)(layer, wq.WqMlpLayer(FAKE, FAKE, FAKE + 2, 1.0, 1.0, 1.0, 0))
    assert prep(layers=bad) == MIS
    assert prep(ws=0) == WS and prep(ws=MISALIGNED) == MIS
    assert prep() == DEVERR if not _has_gpu() else True                 # valid arguments reach the device query
    assert lib.wq_mlp_chain_workspace_bytes(0, 256, 512, 4) == 0 and lib.wq_mlp_chain_workspace_bytes(1, 40, 512, 4) == 0
    kc, nc = C.c_int(0), C.c_int(0)
    assert lib.wq_mlp_chain_split(256, 40, C.byref(kc), C.byref(nc)) == SHAPE
    assert lib.wq_mlp_chain_split(256, 512, None, C.byref(nc)) == INV
    assert lib.wq_mlp_chain_launch(None, 0) == INV
    assert lib.wq_mlp_chain_launch(C.byref(wq.WqMlpPlan()), 0) == INV                    # never prepared
    tg = lib.wq_nvfp4_tile_glu
    assert tg(0, FAKE, FAKE, FAKE, 64, 256, FAKE, 0) == INV and tg(FAKE, FAKE, FAKE, FAKE, 0, 256, FAKE, 0) == INV
    assert tg(FAKE, FAKE, FAKE, FAKE, 60, 256, FAKE, 0) == SHAPE and tg(FAKE, FAKE, FAKE, FAKE, 64, 48, FAKE, 0) == SHAPE
    assert tg(FAKE, FAKE, FAKE + 4, FAKE, 64, 256, FAKE, 0) == MIS


def _has_gpu():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


def test_noalloc_gemm_argument_errors(wq):
    # validated like wq_gemm_nvfp4_tiled, before any HIP call
    lib = wq.lib()
    INV, SHAPE, MIS = 1, 2, 3

    def na(t=FAKE, x=FAKE, y=FAKE, M=64, K=256, N=4):
        return lib.wq_gemm_nvfp4_tiled_noalloc(t, 1.0, x, y, M, K, N, 0)

    assert na(t=0) == INV and na(x=0) == INV and na(y=0) == INV
    assert na(N=0) == INV and na(N=9) == INV and na(M=0) == INV
    assert na(K=48) == SHAPE and na(M=1 << 30, K=1 << 12) == SHAPE
    assert na(t=MISALIGNED) == MIS and na(y=MISALIGNED) == MIS
    assert wq.wq_status_string(7) != "unknown status"
