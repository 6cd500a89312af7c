"""Python binding of libfp4, the gfx950 block-scaled FP4 (NVFP4 / MXFP4) library and its
8-bit members (MXFP8, FP8 W8A8).

The functions carry the C names of include/fp4.h and include/fp8.h and only marshal
arguments:
torch tensors (or raw integer device addresses) become pointers, the current
torch stream becomes the hipStream_t, and negative status codes raise
``Fp4Error``.  Every computation runs in the HIP kernels of libfp4.so; there is
no Python or CPU fallback -- importing fails loudly when the library is missing.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp4.so")

FP4_NVFP4, FP4_MXFP4 = 0, 1
FP4_W4A4, FP4_W4A16 = 0, 1
FP4_OUT_BF16, FP4_OUT_F32 = 0, 1
FP4_FLAG_ALLOW_W4A16_FALLBACK = 1
FP4_FLAG_PREPARED_WEIGHTS = 2

FP4_OK = 0
FP4_OK_FELL_BACK_W4A16 = 1
FP4_ERR_NULL = -1
FP4_ERR_SHAPE = -2
FP4_ERR_ALIGN = -3
FP4_ERR_INPUT_SCALE = -4
FP4_ERR_WEIGHT_SCALE = -5
FP4_ERR_FORMAT = -6
FP4_ERR_WORKSPACE = -7
FP4_ERR_DEVICE = -8
FP4_ERR_LAUNCH = -9

FP8_MX, FP8_PER_TENSOR, FP8_ROWWISE, FP8_BLOCK = 0, 1, 2, 3
MX_E2M1, MX_E2M3, MX_E3M2, MX_E4M3 = 0, 1, 2, 3

FORMATS = {"nvfp4": FP4_NVFP4, "mxfp4": FP4_MXFP4}
MX_ELEMS = {"e2m1": MX_E2M1, "e2m3": MX_E2M3, "e3m2": MX_E3M2, "e4m3": MX_E4M3}
MX_BITS = {MX_E2M1: 4, MX_E2M3: 6, MX_E3M2: 6, MX_E4M3: 8}
FP8_MODES = {"mx": FP8_MX, "per_tensor": FP8_PER_TENSOR, "rowwise": FP8_ROWWISE,
             "block": FP8_BLOCK}
MODES = {"w4a4": FP4_W4A4, "w4a16": FP4_W4A16}
GROUP = {FP4_NVFP4: 16, FP4_MXFP4: 32}

EXPORTED = [
    "fp4_quantize_act", "fp4_quantize_weight", "fp4_gemm", "fp4_gemm_workspace_size",
    "fp4_gemm_workspace_size_mnk",
    "fp4_gemm_noalloc", "fp4_prepared_weight_bytes", "fp4_prepare_weights",
    "fp4_moe_topk_softmax", "fp4_moe_workspace_size", "fp4_moe_workspace_layout",
    "fp4_moe_grouped_gemm", "fp4_arch_supported", "fp4_status_str", "fp4_last_kernel",
    "fp8_quantize_act", "fp8_quantize_weight", "fp8_gemm",
    "mx_quantize_act", "mx_quantize_weight", "mx_gemm",
]

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python block_scaled_fp4_quantize_amd/build.py` "
        "(there is no fallback implementation)")

# torch (the device-memory and stream plumbing) ships its own HIP runtime under
# the same soname as the system one.  Load it first so that libfp4 binds to that
# same runtime: two HIP/HSA runtimes in one process do not share queues, memory
# bookkeeping or synchronization, and kernels launched through one race copies
# and syncs made through the other.
import torch  # noqa: E402,F401


def _hip_runtimes():
    try:
        with open("/proc/self/maps") as f:
            return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})
    except OSError:
        return []


_lib = ctypes.CDLL(LIB_PATH)
if len(_hip_runtimes()) > 1:
    raise ImportError("more than one HIP runtime is mapped into this process: "
                      + ", ".join(_hip_runtimes()))

_i64, _u32, _f32, _vp, _sz = ctypes.c_int64, ctypes.c_uint32, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
_int = ctypes.c_int


class Fp4Error(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} ({status})")


class MoeArgs(ctypes.Structure):
    _fields_ = [
        ("fmt", _int), ("mode", _int), ("T", _i64), ("H", _i64), ("I", _i64), ("E", _i64),
        ("k", _int), ("flags", _u32),
        ("hidden_bf16", _vp), ("topk_ids", _vp), ("topk_w", _vp),
        ("w13_codes", _vp), ("w13_scales", _vp), ("w2_codes", _vp), ("w2_scales", _vp),
        ("w13_scale_2", ctypes.POINTER(_f32)), ("w2_scale_2", ctypes.POINTER(_f32)),
        ("a13_scale", ctypes.POINTER(_f32)), ("a2_scale", ctypes.POINTER(_f32)),
        ("sh_w13_codes", _vp), ("sh_w13_scales", _vp), ("sh_w2_codes", _vp), ("sh_w2_scales", _vp),
        ("sh_w13_scale_2", _f32), ("sh_w2_scale_2", _f32), ("sh_a13_scale", _f32),
        ("sh_a2_scale", _f32),
        ("out_bf16", _vp),
    ]


class MoeLayout(ctypes.Structure):
    _fields_ = [(n, _sz) for n in ("total_bytes", "expert_offsets", "sorted_rows", "inverse",
                                   "x_codes", "x_scales", "gu", "h_codes", "h_scales", "h_bf16",
                                   "y")] + [("x_rows", _i64), ("gu_rows", _i64),
                                            ("swiglu_fused", ctypes.c_int32)]


def _proto(name, res, args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = args
    return f


_c = {
    "fp4_quantize_act": _proto("fp4_quantize_act", _int, [_int, _vp, _i64, _i64, _i64, _f32, _vp, _vp, _vp]),
    "fp4_quantize_weight": _proto("fp4_quantize_weight", _int, [_int, _vp, _i64, _i64, _i64, _f32, _vp, _vp, _vp]),
    "fp4_gemm": _proto("fp4_gemm", _int, [_int, _int, _i64, _i64, _i64, _vp, _i64, _vp, _vp, _vp, _vp,
                                          _f32, _f32, _vp, _i64, _int, _u32, _vp, _sz, _vp]),
    "fp4_gemm_noalloc": _proto("fp4_gemm_noalloc", _int, [_int, _int, _i64, _i64, _i64, _vp, _i64, _vp,
                                                          _vp, _vp, _vp, _f32, _f32, _vp, _i64, _int,
                                                          _u32, _vp]),
    "fp4_prepared_weight_bytes": _proto("fp4_prepared_weight_bytes", _sz, [_i64, _i64]),
    "fp4_prepare_weights": _proto("fp4_prepare_weights", _int, [_int, _vp, _vp, _i64, _i64, _vp, _vp, _vp]),
    "fp4_gemm_workspace_size": _proto("fp4_gemm_workspace_size", _sz, [_int, _int, _i64, _i64, _int]),
    "fp4_gemm_workspace_size_mnk": _proto("fp4_gemm_workspace_size_mnk", _sz,
                                          [_int, _int, _i64, _i64, _i64, _int]),
    "fp4_moe_topk_softmax": _proto("fp4_moe_topk_softmax", _int, [_vp, _i64, _i64, _int, _int, _vp, _vp, _vp]),
    "fp4_moe_workspace_size": _proto("fp4_moe_workspace_size", _sz, [ctypes.POINTER(MoeArgs)]),
    "fp4_moe_workspace_layout": _proto("fp4_moe_workspace_layout", _int,
                                       [ctypes.POINTER(MoeArgs), ctypes.POINTER(MoeLayout)]),
    "fp4_moe_grouped_gemm": _proto("fp4_moe_grouped_gemm", _int, [ctypes.POINTER(MoeArgs), _vp, _sz, _vp]),
    "fp4_arch_supported": _proto("fp4_arch_supported", _int, [ctypes.c_char_p]),
    "fp4_status_str": _proto("fp4_status_str", ctypes.c_char_p, [_int]),
    "fp4_last_kernel": _proto("fp4_last_kernel", ctypes.c_char_p, []),
    "fp8_quantize_act": _proto("fp8_quantize_act", _int, [_int, _vp, _i64, _i64, _i64, _f32, _vp, _vp, _vp]),
    "fp8_quantize_weight": _proto("fp8_quantize_weight", _int, [_int, _vp, _i64, _i64, _i64, _f32, _vp, _vp,
                                                                _vp]),
    "mx_quantize_act": _proto("mx_quantize_act", _int, [_int, _vp, _i64, _i64, _i64, _vp, _vp, _vp]),
    "mx_quantize_weight": _proto("mx_quantize_weight", _int, [_int, _vp, _i64, _i64, _i64, _vp, _vp, _vp]),
    "mx_gemm": _proto("mx_gemm", _int, [_int, _int, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _i64,
                                        _int, _vp]),
    "fp8_gemm": _proto("fp8_gemm", _int, [_int, _i64, _i64, _i64, _vp, _vp, _f32, _vp, _vp, _f32, _vp,
                                          _i64, _int, _vp]),
}


# ---------------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------------


def _ptr(x):
    """Tensor -> device address; int -> itself; None -> NULL."""
    if x is None:
        return None
    if isinstance(x, int):
        return x or None
    return x.data_ptr() or None


def _stream(stream, *tensors):
    if stream is not None:
        return stream
    for t in tensors:
        if t is not None and not isinstance(t, int) and getattr(t, "is_cuda", False):
            import torch
            return torch.cuda.current_stream(t.device).cuda_stream
    return None


def _fmt(f):
    return FORMATS.get(f, f) if isinstance(f, str) else int(f)


def _mode(m):
    return MODES.get(m, m) if isinstance(m, str) else int(m)


def _f8mode(m):
    return FP8_MODES.get(m, m) if isinstance(m, str) else int(m)


def _mxelem(t):
    return MX_ELEMS.get(t, t) if isinstance(t, str) else int(t)


def _check(st, where, raise_on_error):
    if raise_on_error and st < 0:
        raise Fp4Error(st, where)
    return st


def status_str(st):
    return _c["fp4_status_str"](int(st)).decode()


# ---------------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------------


def fp4_quantize_act(fmt, x, M, K, ldx, input_scale, codes, scales, stream=None, check=True):
    st = _c["fp4_quantize_act"](_fmt(fmt), _ptr(x), M, K, ldx, input_scale, _ptr(codes),
                                _ptr(scales), _stream(stream, x, codes))
    return _check(st, "fp4_quantize_act", check)


def fp4_quantize_weight(fmt, w, N, K, ldw, weight_scale_2, codes, scales, stream=None, check=True):
    st = _c["fp4_quantize_weight"](_fmt(fmt), _ptr(w), N, K, ldw, weight_scale_2, _ptr(codes),
                                   _ptr(scales), _stream(stream, w, codes))
    return _check(st, "fp4_quantize_weight", check)


def fp4_gemm_workspace_size(fmt, mode, M, K, has_a_bf16):
    return _c["fp4_gemm_workspace_size"](_fmt(fmt), _mode(mode), M, K, int(bool(has_a_bf16)))


def fp4_gemm_workspace_size_mnk(fmt, mode, M, N, K, has_a_bf16):
    return _c["fp4_gemm_workspace_size_mnk"](_fmt(fmt), _mode(mode), M, N, K,
                                             int(bool(has_a_bf16)))


def fp4_gemm(fmt, mode, M, N, K, a_bf16, lda, a_codes, a_scales, w_codes, w_scales,
             weight_scale_2, input_scale, out, ldo, out_dtype=FP4_OUT_BF16, flags=0,
             workspace=None, workspace_bytes=0, stream=None, check=True):
    st = _c["fp4_gemm"](_fmt(fmt), _mode(mode), M, N, K, _ptr(a_bf16), lda, _ptr(a_codes),
                        _ptr(a_scales), _ptr(w_codes), _ptr(w_scales), weight_scale_2,
                        input_scale, _ptr(out), ldo, out_dtype, flags, _ptr(workspace),
                        workspace_bytes, _stream(stream, out, w_codes))
    return _check(st, "fp4_gemm", check)


def fp4_gemm_noalloc(fmt, mode, M, N, K, a_bf16, lda, a_codes, a_scales, w_codes, w_scales,
                     weight_scale_2, input_scale, out, ldo, out_dtype=FP4_OUT_BF16, flags=0,
                     stream=None, check=True):
    st = _c["fp4_gemm_noalloc"](_fmt(fmt), _mode(mode), M, N, K, _ptr(a_bf16), lda, _ptr(a_codes),
                                _ptr(a_scales), _ptr(w_codes), _ptr(w_scales), weight_scale_2,
                                input_scale, _ptr(out), ldo, out_dtype, flags,
                                _stream(stream, out, w_codes))
    return _check(st, "fp4_gemm_noalloc", check)


def fp4_prepared_weight_bytes(N, K):
    return _c["fp4_prepared_weight_bytes"](N, K)


def fp4_prepare_weights(fmt, w_codes, w_scales, N, K, prepared_codes, check_i32, stream=None,
                        check=True):
    st = _c["fp4_prepare_weights"](_fmt(fmt), _ptr(w_codes), _ptr(w_scales), N, K,
                                   _ptr(prepared_codes), _ptr(check_i32),
                                   _stream(stream, w_codes, prepared_codes))
    return _check(st, "fp4_prepare_weights", check)


def fp4_moe_topk_softmax(logits, T, E, k, renormalize, topk_ids, topk_w, stream=None, check=True):
    st = _c["fp4_moe_topk_softmax"](_ptr(logits), T, E, k, int(renormalize), _ptr(topk_ids),
                                    _ptr(topk_w), _stream(stream, logits))
    return _check(st, "fp4_moe_topk_softmax", check)


def _host_f32(arr):
    if arr is None:
        return None, None
    a = np.ascontiguousarray(np.asarray(arr, dtype=np.float32))
    return a, a.ctypes.data_as(ctypes.POINTER(_f32))


def make_moe_args(fmt, mode, T, H, I, E, k, hidden, topk_ids, topk_w, w13_codes, w13_scales,
                  w2_codes, w2_scales, out, w13_scale_2=None, w2_scale_2=None, a13_scale=None,
                  a2_scale=None, shared=None, flags=0):
    """Fill an fp4_moe_args struct.  ``shared`` is None or a dict with keys
    w13_codes, w13_scales, w2_codes, w2_scales and (NVFP4) w13_scale_2, w2_scale_2,
    a13_scale, a2_scale.  Returns (struct, keepalive)."""
    keep = []
    a = MoeArgs()
    a.fmt, a.mode = _fmt(fmt), _mode(mode)
    a.T, a.H, a.I, a.E, a.k, a.flags = T, H, I, E, k, flags
    a.hidden_bf16, a.topk_ids, a.topk_w = _ptr(hidden), _ptr(topk_ids), _ptr(topk_w)
    a.w13_codes, a.w13_scales = _ptr(w13_codes), _ptr(w13_scales)
    a.w2_codes, a.w2_scales = _ptr(w2_codes), _ptr(w2_scales)
    for name, arr in (("w13_scale_2", w13_scale_2), ("w2_scale_2", w2_scale_2),
                      ("a13_scale", a13_scale), ("a2_scale", a2_scale)):
        h, p = _host_f32(arr)
        keep.append(h)
        setattr(a, name, p)
    a.sh_w13_scale_2 = a.sh_w2_scale_2 = a.sh_a13_scale = a.sh_a2_scale = 1.0
    if shared is not None:
        a.sh_w13_codes, a.sh_w13_scales = _ptr(shared.get("w13_codes")), _ptr(shared.get("w13_scales"))
        a.sh_w2_codes, a.sh_w2_scales = _ptr(shared.get("w2_codes")), _ptr(shared.get("w2_scales"))
        for n in ("w13_scale_2", "w2_scale_2", "a13_scale", "a2_scale"):
            if n in shared:
                setattr(a, "sh_" + n, float(shared[n]))
    a.out_bf16 = _ptr(out)
    keep.extend([hidden, topk_ids, topk_w, out])
    return a, keep


def fp4_moe_workspace_size(args):
    return _c["fp4_moe_workspace_size"](ctypes.byref(args))


def fp4_moe_workspace_layout(args, check=True):
    lay = MoeLayout()
    st = _c["fp4_moe_workspace_layout"](ctypes.byref(args), ctypes.byref(lay))
    _check(st, "fp4_moe_workspace_layout", check)
    return lay


def fp4_moe_grouped_gemm(args, workspace, workspace_bytes, stream=None, check=True,
                         device_tensor=None):
    st = _c["fp4_moe_grouped_gemm"](ctypes.byref(args), _ptr(workspace), workspace_bytes,
                                    _stream(stream, workspace, device_tensor))
    return _check(st, "fp4_moe_grouped_gemm", check)


def fp4_arch_supported(name):
    return _c["fp4_arch_supported"](name.encode() if isinstance(name, str) else name)


def fp4_status_str(st):
    return status_str(st)


def fp4_last_kernel():
    return _c["fp4_last_kernel"]().decode()


def fp8_quantize_act(mode, x, M, K, ldx, tensor_scale, codes, scales, stream=None, check=True):
    st = _c["fp8_quantize_act"](_f8mode(mode), _ptr(x), M, K, ldx, tensor_scale, _ptr(codes),
                                _ptr(scales), _stream(stream, x, codes))
    return _check(st, "fp8_quantize_act", check)


def fp8_quantize_weight(mode, w, N, K, ldw, tensor_scale, codes, scales, stream=None, check=True):
    st = _c["fp8_quantize_weight"](_f8mode(mode), _ptr(w), N, K, ldw, tensor_scale, _ptr(codes),
                                   _ptr(scales), _stream(stream, w, codes))
    return _check(st, "fp8_quantize_weight", check)


def fp8_gemm(mode, M, N, K, a_codes, a_scales, a_tensor_scale, w_codes, w_scales, w_tensor_scale,
             out, ldo, out_dtype=FP4_OUT_BF16, stream=None, check=True):
    st = _c["fp8_gemm"](_f8mode(mode), M, N, K, _ptr(a_codes), _ptr(a_scales), a_tensor_scale,
                        _ptr(w_codes), _ptr(w_scales), w_tensor_scale, _ptr(out), ldo, out_dtype,
                        _stream(stream, out, w_codes))
    return _check(st, "fp8_gemm", check)


def mx_quantize_act(t, x, M, K, ldx, codes, scales, stream=None, check=True):
    st = _c["mx_quantize_act"](_mxelem(t), _ptr(x), M, K, ldx, _ptr(codes), _ptr(scales),
                               _stream(stream, x, codes))
    return _check(st, "mx_quantize_act", check)


def mx_quantize_weight(t, w, N, K, ldw, codes, scales, stream=None, check=True):
    st = _c["mx_quantize_weight"](_mxelem(t), _ptr(w), N, K, ldw, _ptr(codes), _ptr(scales),
                                  _stream(stream, w, codes))
    return _check(st, "mx_quantize_weight", check)


def mx_gemm(a_t, w_t, M, N, K, a_codes, a_scales, w_codes, w_scales, out, ldo,
            out_dtype=FP4_OUT_BF16, stream=None, check=True):
    st = _c["mx_gemm"](_mxelem(a_t), _mxelem(w_t), M, N, K, _ptr(a_codes), _ptr(a_scales),
                       _ptr(w_codes), _ptr(w_scales), _ptr(out), ldo, out_dtype,
                       _stream(stream, out, w_codes))
    return _check(st, "mx_gemm", check)
