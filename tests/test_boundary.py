"""The C-ABI boundary, on the CPU: the library loads, exports every function that
include/*.h declares, and refuses bad arguments before touching a device.

No call here reaches a kernel: each either fails host-side validation (fake but
aligned addresses are never dereferenced) or stops at the device check, which on a
machine without a gfx950 GPU must say FP4_ERR_DEVICE.  Every call that passes
validation runs only where NO_GPU holds: on a machine with a GPU it would launch a
kernel on the fake addresses.  Error conventions follow the
pages' failure modes: "GLM-5.3-Flash on vLLM, on GB10" (a zero activation scale
must be refused, not computed with) and "vLLM on the NVIDIA DGX Spark (GB10 /
sm_121): A Complete Technical Guide", §6.3 (unsupported device fails loudly).
"""
import ctypes
import os
import re

import numpy as np
import pytest

import block_scaled_fp4_quantize_amd as F

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include")
A = 0x10000          # fake, 16-byte aligned device addresses (never dereferenced)
B = 0x20000
C = 0x30000
D = 0x40000


def _has_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


NO_GPU = not _has_gpu()


def header_functions():
    names = set()
    for h in sorted(os.listdir(INCLUDE)):
        if h.endswith(".h"):
            text = re.sub(r"/\*.*?\*/", "", open(os.path.join(INCLUDE, h)).read(), flags=re.S)
            names |= set(re.findall(r"\b((?:fp[48]|mx)_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def test_every_declared_function_is_exported():
    names = header_functions()
    assert len(names) >= 18 and {"fp8_gemm", "mx_gemm"} <= set(names)
    lib = ctypes.CDLL(F.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(F.EXPORTED)


def test_arch_predicate():
    assert F.fp4_arch_supported("gfx950")
    assert F.fp4_arch_supported("gfx950:sramecc+:xnack-")
    for bad in ("gfx942", "gfx9500", "gfx90a", "", "sm_121"):
        assert not F.fp4_arch_supported(bad)


def test_status_strings():
    for code in range(-9, 2):
        assert F.status_str(code).startswith("FP4_")
    assert F.status_str(F.FP4_ERR_INPUT_SCALE) == "FP4_ERR_INPUT_SCALE"


def q(fmt, x, M, K, ldx, s, codes, scales):
    return F.fp4_quantize_act(fmt, x, M, K, ldx, s, codes, scales, check=False)


def test_quantize_validation():
    assert q(7, A, 4, 32, 32, 1.0, B, C) == F.FP4_ERR_FORMAT
    assert q(F.FP4_NVFP4, A, -1, 32, 32, 1.0, B, C) == F.FP4_ERR_SHAPE
    assert q(F.FP4_NVFP4, A, 4, 24, 24, 1.0, B, C) == F.FP4_ERR_SHAPE       # K % 16
    assert q(F.FP4_MXFP4, A, 4, 48, 48, 1.0, B, C) == F.FP4_ERR_SHAPE       # K % 32
    assert q(F.FP4_NVFP4, A, 4, 32, 16, 1.0, B, C) == F.FP4_ERR_SHAPE       # ldx < K
    assert q(F.FP4_NVFP4, None, 4, 32, 32, 1.0, B, C) == F.FP4_ERR_NULL
    assert q(F.FP4_NVFP4, A, 4, 32, 32, 1.0, None, C) == F.FP4_ERR_NULL
    assert q(F.FP4_NVFP4, A + 2, 4, 32, 32, 1.0, B, C) == F.FP4_ERR_ALIGN
    assert q(F.FP4_NVFP4, A, 4, 32, 36, 1.0, B, C) == F.FP4_ERR_ALIGN       # ldx % 8
    for bad in (0.0, -1.0, float("inf"), float("nan"), 2.0 ** -101):
        assert q(F.FP4_NVFP4, A, 4, 32, 32, bad, B, C) == F.FP4_ERR_INPUT_SCALE
    assert q(F.FP4_MXFP4, A, 4, 32, 32, 0.5, B, C) == F.FP4_ERR_FORMAT
    # empty problems are a no-op, even with NULL pointers
    assert q(F.FP4_NVFP4, None, 0, 32, 32, 1.0, None, None) == F.FP4_OK
    assert q(F.FP4_NVFP4, None, 4, 0, 0, 1.0, None, None) == F.FP4_OK
    w = F.fp4_quantize_weight(F.FP4_NVFP4, A, 4, 32, 32, 0.0, B, C, check=False)
    assert w == F.FP4_ERR_WEIGHT_SCALE


@pytest.mark.skipif(not NO_GPU, reason="device check only observable without a GPU")
def test_valid_calls_stop_at_device_check_without_gpu():
    assert q(F.FP4_NVFP4, A, 4, 32, 32, 1.0, B, C) == F.FP4_ERR_DEVICE
    st = F.fp4_moe_topk_softmax(A, 4, 8, 2, 1, B, C, check=False)
    assert st == F.FP4_ERR_DEVICE
    assert g(F.FP4_MXFP4, F.FP4_W4A4, a_codes=A, a_scales=B) == F.FP4_ERR_DEVICE


def g(fmt, mode, M=4, N=8, K=64, a_bf16=None, lda=64, a_codes=None, a_scales=None,
      w_codes=C, w_scales=D, ws2=1.0, s=1.0, out=0x50000, ldo=8, od=0, flags=0, ws=None,
      wsb=0):
    return F.fp4_gemm(fmt, mode, M, N, K, a_bf16, lda, a_codes, a_scales, w_codes, w_scales,
                      ws2, s, out, ldo, od, flags, ws, wsb, check=False)


def test_gemm_validation():
    NV, MX, W44, W416 = F.FP4_NVFP4, F.FP4_MXFP4, F.FP4_W4A4, F.FP4_W4A16
    assert g(NV, 5, a_bf16=A) == F.FP4_ERR_FORMAT
    assert g(NV, W44, a_bf16=A, od=3) == F.FP4_ERR_FORMAT
    assert g(NV, W44, a_bf16=A, flags=8) == F.FP4_ERR_FORMAT
    assert g(NV, W44, K=40, a_bf16=A) == F.FP4_ERR_SHAPE
    assert g(NV, W44, K=0, a_bf16=A) == F.FP4_ERR_SHAPE
    assert g(NV, W44, M=0, a_bf16=None, w_codes=None) == F.FP4_OK   # empty: no-op
    assert g(NV, W44, ldo=4, a_bf16=A) == F.FP4_ERR_SHAPE
    assert g(NV, W44, a_bf16=A, lda=32) == F.FP4_ERR_SHAPE
    assert g(NV, W416) == F.FP4_ERR_NULL                            # W4A16 needs a_bf16
    assert g(NV, W44, a_codes=A) == F.FP4_ERR_NULL                  # scales missing
    assert g(NV, W44, a_bf16=A, w_codes=None) == F.FP4_ERR_NULL
    assert g(NV, W44, a_bf16=A + 8) == F.FP4_ERR_ALIGN
    assert g(NV, W44, a_bf16=A, lda=68) == F.FP4_ERR_ALIGN
    assert g(NV, W44, a_bf16=A, ws2=0.0) == F.FP4_ERR_WEIGHT_SCALE
    assert g(MX, W44, a_codes=A, a_scales=B, ws2=2.0) == F.FP4_ERR_FORMAT
    assert g(MX, W44, a_codes=A, a_scales=B, s=0.5) == F.FP4_ERR_FORMAT
    # the zeroed-activation-scale case is refused ...
    assert g(NV, W44, a_bf16=A, s=0.0) == F.FP4_ERR_INPUT_SCALE
    assert g(NV, W44, a_codes=A, a_scales=B, s=0.0) == F.FP4_ERR_INPUT_SCALE
    # ... unless weight-only execution is explicitly allowed (needs the bf16 input)
    st = g(NV, W44, a_codes=A, a_scales=B, s=0.0, flags=F.FP4_FLAG_ALLOW_W4A16_FALLBACK)
    assert st == F.FP4_ERR_INPUT_SCALE
    if NO_GPU:  # these pass validation; with a GPU they would launch on fake addresses
        st = g(NV, W44, a_bf16=A, s=0.0, flags=F.FP4_FLAG_ALLOW_W4A16_FALLBACK)
        assert st == F.FP4_ERR_DEVICE
        # weight-only ignores input_scale, so 0 is legitimate there
        assert g(NV, W416, a_bf16=A, s=0.0) == F.FP4_ERR_DEVICE
    # fused W4A4 needs a workspace of the reported size
    need = F.fp4_gemm_workspace_size(NV, W44, 4, 64, 1)
    assert need >= 4 * 32 + 4 * 4
    assert F.fp4_gemm_workspace_size(NV, W416, 4, 64, 1) == 0
    assert F.fp4_gemm_workspace_size(NV, W44, 4, 64, 0) == 0
    assert g(NV, W44, a_bf16=A) == F.FP4_ERR_WORKSPACE
    assert g(NV, W44, a_bf16=A, ws=0x60000, wsb=need - 1) == F.FP4_ERR_WORKSPACE


def test_gemm_workspace_size_mnk():
    # the fused quantization's bytes, plus the stage-ordered block scales of both
    # operands when the problem runs on the 256 x 256 tile (M > 64, >= 256 tiles)
    NV, W44, W416 = F.FP4_NVFP4, F.FP4_W4A4, F.FP4_W4A16
    assert F.fp4_gemm_workspace_size_mnk(NV, W44, 4, 256, 64, 1) == \
        F.fp4_gemm_workspace_size(NV, W44, 4, 64, 1)
    assert F.fp4_gemm_workspace_size_mnk(NV, W44, 4, 256, 64, 0) == 0
    assert F.fp4_gemm_workspace_size_mnk(NV, W416, 8192, 4096, 4096, 1) == 0
    for fmt, G in ((NV, 16), (F.FP4_MXFP4, 32)):
        M, N, K = 8192, 4096, 4096
        fused = F.fp4_gemm_workspace_size(fmt, W44, M, K, 1)
        relayout = M * K // G + N * K // G
        assert F.fp4_gemm_workspace_size_mnk(fmt, W44, M, N, K, 1) == fused + relayout
        assert F.fp4_gemm_workspace_size_mnk(fmt, W44, M, N, K, 0) == relayout
        # rows padded to whole 256-row tiles
        assert F.fp4_gemm_workspace_size_mnk(fmt, W44, 8200, 4100, 1024, 0) == \
            8448 * 1024 // G + 4352 * 1024 // G
        # too few 256 x 256 tiles, or K not a multiple of 128: no relayout
        assert F.fp4_gemm_workspace_size_mnk(fmt, W44, 1024, 1024, 1024, 0) == 0
        assert F.fp4_gemm_workspace_size_mnk(fmt, W44, 8192, 4096, 4064, 0) == 0

def test_topk_validation():
    t = lambda T, E, k: F.fp4_moe_topk_softmax(A, T, E, k, 1, B, C, check=False)
    assert t(4, 8, 0) == F.FP4_ERR_SHAPE
    assert t(4, 8, 9) == F.FP4_ERR_SHAPE
    assert t(4, 2048, 8) == F.FP4_ERR_SHAPE
    assert t(4, 64, 33) == F.FP4_ERR_SHAPE
    assert t(0, 8, 2) == F.FP4_OK
    assert F.fp4_moe_topk_softmax(None, 4, 8, 2, 1, B, C, check=False) == F.FP4_ERR_NULL


def moe_args(fmt=F.FP4_NVFP4, mode=F.FP4_W4A4, T=4, H=64, I=32, E=4, k=2, a13=None, a2=None,
             flags=0, shared=None, ws13=None, ws2=None):
    nv = fmt == F.FP4_NVFP4
    if nv:
        ws13 = np.full(E, 0.01, np.float32) if ws13 is None else ws13
        ws2 = np.full(E, 0.01, np.float32) if ws2 is None else ws2
        if mode == F.FP4_W4A4:
            a13 = np.full(E, 0.02, np.float32) if a13 is None else a13
            a2 = np.full(E, 0.03, np.float32) if a2 is None else a2
    args, keep = F.make_moe_args(fmt, mode, T, H, I, E, k, A, B, C, 0x50000, 0x60000, 0x70000,
                                 0x80000, 0x90000, ws13, ws2, a13, a2, shared=shared,
                                 flags=flags)
    return args, keep


def test_moe_validation_and_layout():
    NV, MX = F.FP4_NVFP4, F.FP4_MXFP4
    args, keep = moe_args()
    size = F.fp4_moe_workspace_size(args)
    lay = F.fp4_moe_workspace_layout(args)
    assert size == lay.total_bytes > 0
    offs = [lay.expert_offsets, lay.sorted_rows, lay.inverse, lay.x_codes, lay.x_scales, lay.gu,
            lay.h_codes, lay.h_scales, lay.y]
    assert all(o % 256 == 0 for o in offs) and len(set(offs)) == len(offs)
    assert lay.x_rows == 4 * 2                      # NVFP4: one row per routed pair
    st = F.fp4_moe_grouped_gemm(args, 0x100000, size - 1, check=False)
    assert st == F.FP4_ERR_WORKSPACE
    # zero activation scale for one expert: refused (the zeroed-MoE failure) ...
    a13 = np.array([0.02, 0.0, 0.02, 0.02], np.float32)
    args, keep = moe_args(a13=a13)
    assert F.fp4_moe_grouped_gemm(args, 0x100000, 1 << 30, check=False) == F.FP4_ERR_INPUT_SCALE
    assert F.fp4_moe_workspace_size(args) == 0
    # ... and a missing scale array is the same failure
    args, keep = moe_args()
    args.a2_scale = ctypes.POINTER(ctypes.c_float)()
    assert F.fp4_moe_grouped_gemm(args, 0x100000, 1 << 30, check=False) == F.FP4_ERR_INPUT_SCALE
    # with the opt-in flag the layer may run weight-only; the layout reserves bf16 space
    args, keep = moe_args(a13=a13, flags=F.FP4_FLAG_ALLOW_W4A16_FALLBACK)
    lay = F.fp4_moe_workspace_layout(args)
    assert lay.h_bf16 > 0
    # shapes and formats
    assert F.fp4_moe_grouped_gemm(moe_args(k=5)[0], A, 1 << 30, check=False) == F.FP4_ERR_SHAPE
    assert F.fp4_moe_grouped_gemm(moe_args(H=40)[0], A, 1 << 30, check=False) == F.FP4_ERR_SHAPE
    mx, keep = moe_args(fmt=MX)
    assert F.fp4_moe_workspace_layout(mx).x_rows == 4   # MXFP4: one row per token
    bad, keep2 = moe_args(fmt=MX, ws13=np.ones(4, np.float32), ws2=np.ones(4, np.float32))
    assert F.fp4_moe_grouped_gemm(bad, 0x100000, 1 << 30, check=False) == F.FP4_ERR_FORMAT
    ws_bad, keep3 = moe_args(ws13=np.array([0.01, -1, 0.01, 0.01], np.float32))
    assert F.fp4_moe_grouped_gemm(ws_bad, 0x100000, 1 << 30, check=False) == F.FP4_ERR_WEIGHT_SCALE
    half = {"w13_codes": 0x110000}
    assert F.fp4_moe_grouped_gemm(moe_args(shared=half)[0], 0x100000, 1 << 30,
                                  check=False) == F.FP4_ERR_NULL


def test_single_hip_runtime_in_process():
    # libfp4 must bind to the HIP runtime torch uses; two runtimes in one process
    # would race each other's queues and synchronization
    import subprocess
    import sys
    code = ("import block_scaled_fp4_quantize_amd as F, torch; "
            "print(len(F._hip_runtimes()))")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                         cwd=os.path.dirname(os.path.dirname(__file__)))
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip() == "1"


def test_row_block_capacity_bound_exhaustive():
    # The MoE row-block table reserves ceil(P / bm) + min(E, P) blocks for P routed rows
    # over E experts at bm rows per block.  Every routing must fit: over all ways of
    # splitting P rows among at most E experts, sum_e ceil(c_e / bm) never exceeds it.
    def partitions(n, parts, cap):
        # non-increasing splits of n into at most `parts` positive parts <= cap
        if n == 0:
            yield []
            return
        if parts == 0:
            return
        for first in range(min(n, cap), 0, -1):
            for rest in partitions(n - first, parts - 1, first):
                yield [first] + rest

    for bm in (1, 2, 3, 16):
        for E in range(1, 7):
            for P in range(0, 19):
                cap = -(-P // bm) + min(E, P)
                worst = max(sum(-(-c // bm) for c in split) for split in partitions(P, E, P))
                assert worst <= cap, (bm, E, P, worst, cap)


def test_noalloc_gemm_validation():
    # the allocation-free variant validates like fp4_gemm, and refuses a fused call
    # larger than its 32 MiB scratch array before touching a device
    NV, W44 = F.FP4_NVFP4, F.FP4_W4A4

    def gn(M=8192, K=8192, **kw):
        return F.fp4_gemm_noalloc(NV, W44, M, 64, K, kw.get("a", A), K, None, None, B, C,
                                  1.0, kw.get("s", 1.0), D, 64, check=False)
    assert gn() == F.FP4_ERR_WORKSPACE                    # 37.7 MB > 32 MiB
    assert gn(s=0.0) == F.FP4_ERR_INPUT_SCALE
    assert gn(a=A + 8) == F.FP4_ERR_ALIGN
    if NO_GPU:
        assert gn(M=8192, K=4096) == F.FP4_ERR_DEVICE    # fits: stops at the device check


# ---- FP8 family ("vLLM per-format kernel capability matrix derived from source": MXFP8,
# FP8 THREE SCALING MODES) ---------------------------------------------------------------


def q8(mode, x=A, M=4, K=128, ldx=128, s=1.0, codes=B, scales=C, weight=False):
    f = F.fp8_quantize_weight if weight else F.fp8_quantize_act
    return f(mode, x, M, K, ldx, s, codes, scales, check=False)


def g8(mode, M=4, N=8, K=128, ac=A, asc=B, ats=1.0, wc=C, wsc=D, wts=1.0, out=0x50000, ldo=8,
       od=0):
    return F.fp8_gemm(mode, M, N, K, ac, asc, ats, wc, wsc, wts, out, ldo, od, check=False)


def test_fp8_quantize_validation():
    assert q8(9) == F.FP4_ERR_FORMAT
    assert q8(F.FP8_MX, K=48, ldx=48) == F.FP4_ERR_SHAPE                   # K % 32
    assert q8(F.FP8_BLOCK, K=96, ldx=96) == F.FP4_ERR_SHAPE                # K % 128
    assert q8(F.FP8_ROWWISE, K=12, ldx=16) == F.FP4_ERR_SHAPE              # K % 8
    assert q8(F.FP8_ROWWISE, M=-1) == F.FP4_ERR_SHAPE
    assert q8(F.FP8_MX, ldx=64) == F.FP4_ERR_SHAPE                         # ldx < K
    assert q8(F.FP8_MX, x=None) == F.FP4_ERR_NULL
    assert q8(F.FP8_ROWWISE, scales=None) == F.FP4_ERR_NULL                # dynamic modes need scales
    assert q8(F.FP8_MX, codes=A + 8) == F.FP4_ERR_ALIGN
    assert q8(F.FP8_MX, ldx=132) == F.FP4_ERR_ALIGN                        # bf16 stride % 8
    if NO_GPU:  # (passes validation: with a GPU it would launch on fake addresses)
        assert q8(F.FP8_MX, ldx=132, weight=True) == F.FP4_ERR_DEVICE      # fp32 stride % 4
    for bad in (0.0, -2.0, float("inf"), float("nan"), 2.0 ** 101):
        assert q8(F.FP8_PER_TENSOR, s=bad, scales=None) == F.FP4_ERR_INPUT_SCALE
        assert q8(F.FP8_PER_TENSOR, s=bad, scales=None, weight=True) == F.FP4_ERR_WEIGHT_SCALE
    assert q8(F.FP8_PER_TENSOR, s=0.5) == F.FP4_ERR_FORMAT                 # per-tensor: no scale array
    for m in (F.FP8_MX, F.FP8_ROWWISE, F.FP8_BLOCK):
        assert q8(m, s=0.5) == F.FP4_ERR_FORMAT                            # dynamic: tensor scale 1
    assert q8(F.FP8_BLOCK, x=None, M=0, codes=None, scales=None) == F.FP4_OK


def test_fp8_gemm_validation():
    assert g8(4) == F.FP4_ERR_FORMAT
    assert g8(F.FP8_MX, od=3) == F.FP4_ERR_FORMAT
    assert g8(F.FP8_MX, K=96) == F.FP4_ERR_SHAPE                           # K % 128
    assert g8(F.FP8_MX, K=0) == F.FP4_ERR_SHAPE
    assert g8(F.FP8_MX, ldo=4) == F.FP4_ERR_SHAPE
    assert g8(F.FP8_MX, M=0, ac=None, asc=None) == F.FP4_OK
    assert g8(F.FP8_BLOCK, wsc=None) == F.FP4_ERR_NULL
    assert g8(F.FP8_ROWWISE, out=None) == F.FP4_ERR_NULL
    assert g8(F.FP8_MX, ac=A + 4) == F.FP4_ERR_ALIGN
    assert g8(F.FP8_PER_TENSOR, asc=None, wsc=None, ats=0.0) == F.FP4_ERR_INPUT_SCALE
    assert g8(F.FP8_PER_TENSOR, asc=None, wsc=None, wts=float("nan")) == F.FP4_ERR_WEIGHT_SCALE
    # the product of the two tensor scales must stay a finite normal fp32
    assert g8(F.FP8_PER_TENSOR, asc=None, wsc=None, ats=2.0 ** 90, wts=2.0 ** 90) == F.FP4_ERR_INPUT_SCALE
    assert g8(F.FP8_PER_TENSOR, asc=None, wsc=None, ats=2.0 ** -90, wts=2.0 ** -90) == F.FP4_ERR_INPUT_SCALE
    assert g8(F.FP8_PER_TENSOR, ats=0.5, wts=0.5) == F.FP4_ERR_FORMAT      # scale arrays given
    assert g8(F.FP8_ROWWISE, ats=0.5) == F.FP4_ERR_FORMAT


@pytest.mark.skipif(not NO_GPU, reason="device check only observable without a GPU")
def test_fp8_valid_calls_stop_at_device_check_without_gpu():
    assert q8(F.FP8_MX) == F.FP4_ERR_DEVICE
    assert q8(F.FP8_BLOCK, weight=True) == F.FP4_ERR_DEVICE
    assert g8(F.FP8_PER_TENSOR, asc=None, wsc=None, ats=0.5, wts=0.25) == F.FP4_ERR_DEVICE
    assert g8(F.FP8_MX) == F.FP4_ERR_DEVICE


# ---- MX formats of any element type (same page: group size 32, MXFP6, MXFP8) ----------


def test_mx_validation():
    qa = lambda t, **kw: F.mx_quantize_act(t, kw.get("x", A), kw.get("M", 4), kw.get("K", 64),
                                           kw.get("ldx", 64), kw.get("c", B), kw.get("s", C),
                                           check=False)
    assert qa(7) == F.FP4_ERR_FORMAT
    assert qa(F.MX_E2M3, K=48, ldx=48) == F.FP4_ERR_SHAPE                 # K % 32
    assert qa(F.MX_E3M2, ldx=32) == F.FP4_ERR_SHAPE                       # ldx < K
    assert qa(F.MX_E2M3, s=None) == F.FP4_ERR_NULL
    assert qa(F.MX_E2M3, x=A + 4) == F.FP4_ERR_ALIGN
    assert qa(F.MX_E2M3, ldx=68) == F.FP4_ERR_ALIGN                       # bf16 stride % 8
    assert qa(F.MX_E2M3, M=0, x=None, c=None, s=None) == F.FP4_OK
    if NO_GPU:  # (passes validation: with a GPU it would launch on fake addresses)
        wq = F.mx_quantize_weight(F.MX_E3M2, A, 4, 64, 68, B, C, check=False)
        assert wq == F.FP4_ERR_DEVICE                                     # fp32 stride % 4
    gm = lambda at, wt, **kw: F.mx_gemm(at, wt, kw.get("M", 4), kw.get("N", 8), kw.get("K", 128),
                                        kw.get("ac", A), kw.get("asc", B), C, D,
                                        kw.get("out", 0x50000), kw.get("ldo", 8), kw.get("od", 0),
                                        check=False)
    assert gm(F.MX_E2M1, 9) == F.FP4_ERR_FORMAT
    assert gm(F.MX_E2M1, F.MX_E4M3, od=2) == F.FP4_ERR_FORMAT
    assert gm(F.MX_E2M1, F.MX_E4M3, K=96) == F.FP4_ERR_SHAPE                # K % 128
    assert gm(F.MX_E2M1, F.MX_E4M3, ldo=7) == F.FP4_ERR_SHAPE
    assert gm(F.MX_E2M1, F.MX_E4M3, asc=None) == F.FP4_ERR_NULL
    assert gm(F.MX_E2M1, F.MX_E4M3, out=0x50008) == F.FP4_ERR_ALIGN
    assert gm(F.MX_E2M1, F.MX_E4M3, M=0, ac=None) == F.FP4_OK
    if NO_GPU:
        assert qa(F.MX_E2M3) == F.FP4_ERR_DEVICE
        assert gm(F.MX_E3M2, F.MX_E2M1) == F.FP4_ERR_DEVICE


# ---- one-time weight preparation ("vLLM on the NVIDIA DGX Spark (GB10 / sm_121): A
# Complete Technical Guide", §4.3 / §5.3: scales converted once at load) -------------


def test_prepare_validation():
    assert F.fp4_prepared_weight_bytes(32, 256) == 32 * 128
    assert F.fp4_prepared_weight_bytes(30, 256) == 0           # N % 16
    assert F.fp4_prepared_weight_bytes(32, 192) == 0           # K % 128
    pw = lambda fmt=F.FP4_MXFP4, N=32, K=256, c=A, s=B, o=C, chk=D: F.fp4_prepare_weights(
        fmt, c, s, N, K, o, chk, check=False)
    assert pw(fmt=5) == F.FP4_ERR_FORMAT
    assert pw(N=24) == F.FP4_ERR_SHAPE
    assert pw(K=320) == F.FP4_ERR_SHAPE
    assert pw(chk=None) == F.FP4_ERR_NULL
    assert pw(o=C + 8) == F.FP4_ERR_ALIGN
    assert pw(chk=D + 2) == F.FP4_ERR_ALIGN
    if NO_GPU:
        assert pw() == F.FP4_ERR_DEVICE
    P = F.FP4_FLAG_PREPARED_WEIGHTS
    # prepared weights serve W4A4 calls of at most 64 rows with whole 16-row blocks
    assert g(F.FP4_MXFP4, F.FP4_W4A16, a_bf16=A, K=128, lda=128, flags=P) == F.FP4_ERR_FORMAT
    assert g(F.FP4_NVFP4, F.FP4_W4A4, a_codes=A, a_scales=B, K=128,
             flags=P | F.FP4_FLAG_ALLOW_W4A16_FALLBACK) == F.FP4_ERR_FORMAT
    assert g(F.FP4_MXFP4, F.FP4_W4A4, a_codes=A, a_scales=B, M=65, K=128, flags=P) == F.FP4_ERR_SHAPE
    assert g(F.FP4_MXFP4, F.FP4_W4A4, a_codes=A, a_scales=B, N=24, ldo=24, K=128, flags=P) == \
        F.FP4_ERR_SHAPE
    assert g(F.FP4_MXFP4, F.FP4_W4A4, a_codes=A, a_scales=B, N=16, ldo=16, K=96, flags=P) == \
        F.FP4_ERR_SHAPE
    assert g(F.FP4_MXFP4, F.FP4_W4A4, a_codes=A, a_scales=B, flags=8) == F.FP4_ERR_FORMAT
    if NO_GPU:
        assert g(F.FP4_MXFP4, F.FP4_W4A4, a_codes=A, a_scales=B, N=16, ldo=16, K=128, flags=P) == \
            F.FP4_ERR_DEVICE
