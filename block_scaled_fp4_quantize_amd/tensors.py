"""Tensor-level wrappers over the C ABI: allocate outputs with torch on the input's
device and call the library.  Plumbing only; no arithmetic happens here."""
import torch

from . import (FP4_MXFP4, FP4_NVFP4, FP4_OUT_BF16, FP4_OUT_F32, FP4_W4A4, FP4_W4A16,
               FP8_BLOCK, FP8_MX, FP8_ROWWISE, GROUP, _f8mode, _fmt, _mode,
               fp4_gemm, fp4_gemm_workspace_size_mnk, fp4_moe_grouped_gemm, fp4_moe_topk_softmax,
               fp4_moe_workspace_layout, fp4_moe_workspace_size, fp4_quantize_act,
               fp4_quantize_weight, fp8_gemm, fp8_quantize_act, fp8_quantize_weight,
               make_moe_args, MX_BITS, _mxelem, mx_gemm, mx_quantize_act, mx_quantize_weight)


def _alloc_u8(rows, cols, device):
    return torch.empty((rows, cols), dtype=torch.uint8, device=device)


def quantize_act(fmt, x, input_scale=1.0):
    """x: bf16 [M, K] (row stride may exceed K) -> (codes [M, K/2], scales [M, K/G])."""
    f = _fmt(fmt)
    M, K = x.shape
    codes = _alloc_u8(M, K // 2, x.device)
    scales = _alloc_u8(M, K // GROUP[f], x.device)
    fp4_quantize_act(f, x, M, K, x.stride(0), float(input_scale), codes, scales)
    return codes, scales


def quantize_weight(fmt, w, weight_scale_2=1.0):
    """w: fp32 [N, K] -> (codes [N, K/2], scales [N, K/G])."""
    f = _fmt(fmt)
    N, K = w.shape
    codes = _alloc_u8(N, K // 2, w.device)
    scales = _alloc_u8(N, K // GROUP[f], w.device)
    fp4_quantize_weight(f, w, N, K, w.stride(0), float(weight_scale_2), codes, scales)
    return codes, scales


def gemm(fmt, mode, w_codes, w_scales, a_bf16=None, a_codes=None, a_scales=None,
         weight_scale_2=1.0, input_scale=1.0, out_dtype=torch.bfloat16, flags=0, out=None,
         workspace=None):
    """out [M, N] = alpha * a_hat @ w_hat^T.  Returns (out, status)."""
    f, m = _fmt(fmt), _mode(mode)
    N, Kh = w_codes.shape
    K = Kh * 2
    M = a_bf16.shape[0] if a_bf16 is not None else a_codes.shape[0]
    dev = w_codes.device
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=dev)
    od = FP4_OUT_F32 if out.dtype == torch.float32 else FP4_OUT_BF16
    wsz = fp4_gemm_workspace_size_mnk(f, m, M, N, K, a_bf16 is not None)
    if workspace is None and wsz:
        workspace = torch.empty(wsz, dtype=torch.uint8, device=dev)
    elif workspace is not None:
        wsz = workspace.numel() * workspace.element_size()
    lda = a_bf16.stride(0) if a_bf16 is not None else 0
    st = fp4_gemm(f, m, M, N, K, a_bf16, lda, a_codes, a_scales, w_codes, w_scales,
                  float(weight_scale_2), float(input_scale), out, out.stride(0), od, flags,
                  workspace, wsz if workspace is not None else 0)
    return out, st


def _fp8_scales(mode, rows, K, device, weight):
    """Scale tensor of an FP8 operand (None for per-tensor scaling)."""
    if mode == FP8_MX:
        return torch.empty((rows, K // 32), dtype=torch.uint8, device=device)
    if mode == FP8_ROWWISE:
        return torch.empty((rows,), dtype=torch.float32, device=device)
    if mode == FP8_BLOCK:
        r = (rows + 127) // 128 if weight else rows
        return torch.empty((r, K // 128), dtype=torch.float32, device=device)
    return None


def fp8_quantize_act_t(mode, x, tensor_scale=1.0):
    """x: bf16 [M, K] -> (codes uint8 [M, K], scales by mode or None)."""
    m = _f8mode(mode)
    M, K = x.shape
    codes = _alloc_u8(M, K, x.device)
    scales = _fp8_scales(m, M, K, x.device, False)
    fp8_quantize_act(m, x, M, K, x.stride(0), float(tensor_scale), codes, scales)
    return codes, scales


def fp8_quantize_weight_t(mode, w, tensor_scale=1.0):
    """w: fp32 [N, K] -> (codes uint8 [N, K], scales by mode or None)."""
    m = _f8mode(mode)
    N, K = w.shape
    codes = _alloc_u8(N, K, w.device)
    scales = _fp8_scales(m, N, K, w.device, True)
    fp8_quantize_weight(m, w, N, K, w.stride(0), float(tensor_scale), codes, scales)
    return codes, scales


def fp8_gemm_t(mode, a_codes, a_scales, w_codes, w_scales, a_tensor_scale=1.0,
               w_tensor_scale=1.0, out_dtype=torch.bfloat16, out=None):
    """out [M, N] = a_hat @ w_hat^T for FP8 operands of one scaling mode."""
    m = _f8mode(mode)
    M, K = a_codes.shape
    N = w_codes.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=w_codes.device)
    od = FP4_OUT_F32 if out.dtype == torch.float32 else FP4_OUT_BF16
    fp8_gemm(m, M, N, K, a_codes, a_scales, float(a_tensor_scale), w_codes, w_scales,
             float(w_tensor_scale), out, out.stride(0), od)
    return out


def mx_quantize_t(t, x):
    """bf16 activations or fp32 weights [R, K] -> (packed codes [R, K*bits/8], e8m0 [R, K/32])."""
    e = _mxelem(t)
    R, K = x.shape
    codes = _alloc_u8(R, K * MX_BITS[e] // 8, x.device)
    scales = _alloc_u8(R, K // 32, x.device)
    f = mx_quantize_weight if x.dtype == torch.float32 else mx_quantize_act
    f(e, x, R, K, x.stride(0), codes, scales)
    return codes, scales


def mx_gemm_t(a_t, w_t, a_codes, a_scales, w_codes, w_scales, out_dtype=torch.bfloat16, out=None):
    """out [M, N] = a_hat @ w_hat^T for MX operands of element types a_t and w_t."""
    ea, ew = _mxelem(a_t), _mxelem(w_t)
    M = a_codes.shape[0]
    K = a_scales.shape[1] * 32
    N = w_codes.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=w_codes.device)
    od = FP4_OUT_F32 if out.dtype == torch.float32 else FP4_OUT_BF16
    mx_gemm(ea, ew, M, N, K, a_codes, a_scales, w_codes, w_scales, out, out.stride(0), od)
    return out


def topk_softmax(logits, k, renormalize=True):
    T, E = logits.shape
    ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    fp4_moe_topk_softmax(logits, T, E, k, renormalize, ids, w)
    return ids, w


class Moe:
    """Holds the device weights of a MoE layer and runs fp4_moe_grouped_gemm."""

    def __init__(self, fmt, mode, H, I, E, w13_codes, w13_scales, w2_codes, w2_scales,
                 w13_scale_2=None, w2_scale_2=None, a13_scale=None, a2_scale=None,
                 shared=None, flags=0):
        self.fmt, self.mode = _fmt(fmt), _mode(mode)
        self.H, self.I, self.E = H, I, E
        self.w = (w13_codes, w13_scales, w2_codes, w2_scales)
        self.scales = (w13_scale_2, w2_scale_2, a13_scale, a2_scale)
        self.shared = shared
        self.flags = flags
        self._ws = None

    def args(self, hidden, ids, w, out):
        T = hidden.shape[0]
        k = ids.shape[1]
        return make_moe_args(self.fmt, self.mode, T, self.H, self.I, self.E, k, hidden, ids, w,
                             *self.w, out, *self.scales, shared=self.shared, flags=self.flags)

    def workspace_for(self, args):
        need = fp4_moe_workspace_size(args)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.w[0].device)
        return self._ws, need

    def __call__(self, hidden, ids, w, out=None, check=True):
        if out is None:
            out = torch.empty((hidden.shape[0], self.H), dtype=torch.bfloat16, device=hidden.device)
        args, keep = self.args(hidden, ids, w, out)
        ws, need = self.workspace_for(args)
        st = fp4_moe_grouped_gemm(args, ws, ws.numel(), check=check, device_tensor=hidden)
        self.last_args, self._keep = args, keep
        return out, st

    def layout(self, hidden, ids, w, out):
        args, keep = self.args(hidden, ids, w, out)
        return fp4_moe_workspace_layout(args)
