"""Python binding of libskiparse (Skiparse-2D sparse attention forward on
MI355X).  Argument marshalling only: every step of the computation runs in the
library's HIP kernels.  PyTorch supplies device memory and the current stream.

The names mirror the C ABI in include/skiparse.h:

    skiparse_abi_version()
    skiparse_plan_init(B, T, H, W, heads, d, k, mode) -> SkiparsePlan
    skiparse_plan_index_map(plan) -> numpy int32 (n_sub, sub_len_padded)
    skiparse_index_map_device(plan, out, stream=None)
    skiparse_attn_fwd(plan, dtype, q, k, v, o, softmax_scale=0.0,
                      descale_qkv=None, sub_begin=0, sub_count=0, stream=None)
    skiparse_attn_fwd_lse(plan, dtype, q, k, v, o, lse, softmax_scale=0.0,
                          sub_begin=0, sub_count=0, stream=None)
    skiparse_attn_bwd_workspace_bytes(plan)
    skiparse_attn_bwd(plan, dtype, q, k, v, o, dout, lse, dq, dk, dv,
                      softmax_scale=0.0, workspace=None, sub_begin=0,
                      sub_count=0, stream=None)
    skiparse_attn_fwd_lse_fp8(plan, q8, k8, v8, descale_qkv, o, lse,
                              softmax_scale=0.0, sub_begin=0, sub_count=0,
                              stream=None)
    skiparse_attn_bwd_fp8(plan, q8, k8, v8, descale_qkv, o, dout8,
                          descale_dout, lse, dq, dk, dv, softmax_scale=0.0,
                          workspace=None, sub_begin=0, sub_count=0,
                          stream=None)
    skiparse_quant_fp8_workspace_bytes(numel)
    skiparse_quant_fp8(x, y, scale, fp8_max=448.0, eps=1e-12,
                       workspace=None, stream=None)
    skiparse_block_workspace_bytes(plan)
    skiparse_block_fwd_fp8(plan, x, w_qkvo, w_scales, y, rope_theta=10000.0,
                           rope_dims=None, workspace=None, stream=None)
    skiparse_gemm_fp8(x, w, sx, sw, y, stream=None)
    skiparse_rope_fp8_workspace_bytes(plan)
    skiparse_rope_fp8(plan, x, y, scale, rope_theta=10000.0, rope_dims=None,
                      workspace=None, stream=None)
    skiparse_last_error()

plus conveniences that allocate their outputs with torch:
``attention``, ``attention_fp8``, ``quantize_fp8``, ``attention_train``
(output and log-sum-exp), ``attention_bwd`` (dq, dk, dv),
``SkiparseAttention`` (a torch.autograd.Function over the last two),
``quantize_weights`` and ``BlockFP8`` (the fp8 attention block).

There is no fallback: if libskiparse.so is missing the calls raise.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libskiparse.so")

OK = 0
EINVAL = -1
EUNSUPPORTED = -2
EHIP = -3
EWORKSPACE = -4

MODE_TOKEN = 0
MODE_GROUP = 1
MODE_TOKEN_1D = 2
MODE_GROUP_1D = 3

F32 = 0
BF16 = 1
FP8_E4M3 = 2

MAX_K = 8
ABI_VERSION = 1

EXPORTED = (
    "skiparse_abi_version",
    "skiparse_plan_init",
    "skiparse_plan_index_map",
    "skiparse_index_map_device",
    "skiparse_attn_fwd",
    "skiparse_attn_fwd_lse",
    "skiparse_attn_bwd_workspace_bytes",
    "skiparse_attn_bwd",
    "skiparse_attn_fwd_lse_fp8",
    "skiparse_attn_bwd_fp8",
    "skiparse_quant_fp8_workspace_bytes",
    "skiparse_quant_fp8_noalloc",
    "skiparse_quant_fp8",
    "skiparse_block_workspace_bytes",
    "skiparse_block_fwd_fp8",
    "skiparse_gemm_fp8",
    "skiparse_rope_fp8_workspace_bytes",
    "skiparse_rope_fp8",
    "skiparse_last_error",
)


class SkiparsePlan(ctypes.Structure):
    """Mirror of ``skiparse_plan`` (plain data)."""
    _fields_ = [
        ("abi", ctypes.c_int32),
        ("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32), ("W", ctypes.c_int32),
        ("heads", ctypes.c_int32), ("d", ctypes.c_int32), ("k", ctypes.c_int32), ("mode", ctypes.c_int32),
        ("Hp", ctypes.c_int32), ("Wp", ctypes.c_int32),
        ("sub_h", ctypes.c_int32), ("sub_w", ctypes.c_int32),
        ("n_sub", ctypes.c_int32), ("reserved0", ctypes.c_int32),
        ("sub_len_padded", ctypes.c_int64),
        ("pairs", ctypes.c_int64),
        ("real_h", ctypes.c_int32 * MAX_K),
        ("real_w", ctypes.c_int32 * MAX_K),
    ]

    @property
    def flops(self) -> int:
        """Algorithmic FLOPs of one call over all subsequences: 4 * d * pairs."""
        return 4 * self.d * self.pairs

    def sub_lengths(self):
        """Real tokens per subsequence, in subsequence order."""
        if self.mode in (MODE_TOKEN_1D, MODE_GROUP_1D):
            return [self.T * self.real_w[q] for q in range(self.n_sub)]
        k = self.k
        return [self.T * self.real_h[p] * self.real_w[q] for p in range(k) for q in range(k)]


class SkiparseError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"skiparse error {code}: {msg}")
        self.code = code


_lib = None


def lib():
    """Load libskiparse.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m fixed_pattern_sparse_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(SkiparsePlan)
    vp = ctypes.c_void_p
    L.skiparse_abi_version.restype = ctypes.c_int
    L.skiparse_abi_version.argtypes = []
    L.skiparse_plan_init.restype = ctypes.c_int
    L.skiparse_plan_init.argtypes = [P] + [ctypes.c_int32] * 8
    L.skiparse_plan_index_map.restype = ctypes.c_int
    L.skiparse_plan_index_map.argtypes = [P, vp]
    L.skiparse_index_map_device.restype = ctypes.c_int
    L.skiparse_index_map_device.argtypes = [P, vp, vp]
    L.skiparse_attn_fwd.restype = ctypes.c_int
    L.skiparse_attn_fwd.argtypes = [P, ctypes.c_int, vp, vp, vp, vp, ctypes.c_float, vp,
                                    ctypes.c_int32, ctypes.c_int32, vp]
    L.skiparse_attn_fwd_lse.restype = ctypes.c_int
    L.skiparse_attn_fwd_lse.argtypes = [P, ctypes.c_int, vp, vp, vp, vp, vp, ctypes.c_float,
                                        ctypes.c_int32, ctypes.c_int32, vp]
    L.skiparse_attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.skiparse_attn_bwd_workspace_bytes.argtypes = [P]
    L.skiparse_attn_bwd.restype = ctypes.c_int
    L.skiparse_attn_bwd.argtypes = [P, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float,
                                    vp, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int32, vp]
    L.skiparse_attn_fwd_lse_fp8.restype = ctypes.c_int
    L.skiparse_attn_fwd_lse_fp8.argtypes = [P, vp, vp, vp, vp, vp, vp, ctypes.c_float, ctypes.c_int32,
                                            ctypes.c_int32, vp]
    L.skiparse_attn_bwd_fp8.restype = ctypes.c_int
    L.skiparse_attn_bwd_fp8.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp,
                                        ctypes.c_size_t, ctypes.c_int32, ctypes.c_int32, vp]
    L.skiparse_quant_fp8_workspace_bytes.restype = ctypes.c_size_t
    L.skiparse_quant_fp8_workspace_bytes.argtypes = [ctypes.c_int64]
    L.skiparse_quant_fp8.restype = ctypes.c_int
    L.skiparse_quant_fp8.argtypes = [vp, ctypes.c_int, ctypes.c_int64, vp, vp, ctypes.c_float, ctypes.c_float,
                                     vp, ctypes.c_size_t, vp]
    L.skiparse_quant_fp8_noalloc.restype = ctypes.c_int
    L.skiparse_quant_fp8_noalloc.argtypes = [vp, ctypes.c_int, ctypes.c_int64, vp, vp, ctypes.c_float, ctypes.c_float,
                                             vp]
    L.skiparse_block_workspace_bytes.restype = ctypes.c_size_t
    L.skiparse_block_workspace_bytes.argtypes = [P]
    L.skiparse_block_fwd_fp8.restype = ctypes.c_int
    L.skiparse_block_fwd_fp8.argtypes = [P, vp, vp, vp, ctypes.c_float, vp, vp, vp, ctypes.c_size_t, vp]
    L.skiparse_gemm_fp8.restype = ctypes.c_int
    L.skiparse_gemm_fp8.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, vp]
    L.skiparse_rope_fp8_workspace_bytes.restype = ctypes.c_size_t
    L.skiparse_rope_fp8_workspace_bytes.argtypes = [P]
    L.skiparse_rope_fp8.restype = ctypes.c_int
    L.skiparse_rope_fp8.argtypes = [P, vp, ctypes.c_float, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.skiparse_last_error.restype = ctypes.c_char_p
    L.skiparse_last_error.argtypes = []
    if L.skiparse_abi_version() != ABI_VERSION:
        raise RuntimeError("libskiparse ABI version mismatch")
    _lib = L
    return L


def _check(code):
    if code != OK:
        raise SkiparseError(code, skiparse_last_error())


def _ptr(x):
    """Device/host address of a torch tensor, or an int address, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_contiguous():
        # every entry point reads and writes dense row-major buffers
        raise ValueError("tensors passed to libskiparse must be contiguous")
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def skiparse_abi_version() -> int:
    return lib().skiparse_abi_version()


def skiparse_last_error() -> str:
    return lib().skiparse_last_error().decode()


def skiparse_plan_init(B, T, H, W, heads, d, k, mode) -> SkiparsePlan:
    plan = SkiparsePlan()
    _check(lib().skiparse_plan_init(ctypes.byref(plan), B, T, H, W, heads, d, k, mode))
    return plan


def skiparse_plan_index_map(plan: SkiparsePlan) -> np.ndarray:
    out = np.empty((plan.n_sub, plan.sub_len_padded), np.int32)
    _check(lib().skiparse_plan_index_map(ctypes.byref(plan), out.ctypes.data))
    return out


def skiparse_index_map_device(plan: SkiparsePlan, out, stream=None):
    """Write the device index map into ``out`` (int32 device tensor with
    n_sub * sub_len_padded elements)."""
    if out.numel() != plan.n_sub * plan.sub_len_padded:
        raise ValueError("out has the wrong number of elements")
    _check(lib().skiparse_index_map_device(ctypes.byref(plan), _ptr(out), _stream(stream)))
    return out


def skiparse_attn_fwd(plan: SkiparsePlan, dtype: int, q, k, v, o, softmax_scale: float = 0.0,
                      descale_qkv=None, sub_begin: int = 0, sub_count: int = 0, stream=None):
    _check(lib().skiparse_attn_fwd(ctypes.byref(plan), dtype, _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                   float(softmax_scale), _ptr(descale_qkv), sub_begin, sub_count,
                                   _stream(stream)))
    return o


def skiparse_attn_fwd_lse(plan: SkiparsePlan, dtype: int, q, k, v, o, lse, softmax_scale: float = 0.0,
                          sub_begin: int = 0, sub_count: int = 0, stream=None):
    _check(lib().skiparse_attn_fwd_lse(ctypes.byref(plan), dtype, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                       float(softmax_scale), sub_begin, sub_count, _stream(stream)))
    return o, lse


def skiparse_attn_bwd_workspace_bytes(plan: SkiparsePlan) -> int:
    return int(lib().skiparse_attn_bwd_workspace_bytes(ctypes.byref(plan)))


def skiparse_attn_bwd(plan: SkiparsePlan, dtype: int, q, k, v, o, dout, lse, dq, dk, dv,
                      softmax_scale: float = 0.0, workspace=None, sub_begin: int = 0, sub_count: int = 0,
                      stream=None):
    """Backward pass; ``workspace`` (device, >= skiparse_attn_bwd_workspace_bytes)
    is allocated with torch when None."""
    if workspace is None:
        import torch
        workspace = torch.empty(skiparse_attn_bwd_workspace_bytes(plan), dtype=torch.uint8, device=q.device)
    wb = workspace.numel() * workspace.element_size() if hasattr(workspace, "numel") else 0
    _check(lib().skiparse_attn_bwd(ctypes.byref(plan), dtype, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout),
                                   _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), float(softmax_scale), _ptr(workspace),
                                   wb, sub_begin, sub_count, _stream(stream)))
    return dq, dk, dv


def skiparse_attn_fwd_lse_fp8(plan: SkiparsePlan, q8, k8, v8, descale_qkv, o, lse, softmax_scale: float = 0.0,
                              sub_begin: int = 0, sub_count: int = 0, stream=None):
    _check(lib().skiparse_attn_fwd_lse_fp8(ctypes.byref(plan), _ptr(q8), _ptr(k8), _ptr(v8), _ptr(descale_qkv),
                                           _ptr(o), _ptr(lse), float(softmax_scale), sub_begin, sub_count,
                                           _stream(stream)))
    return o, lse


def skiparse_attn_bwd_fp8(plan: SkiparsePlan, q8, k8, v8, descale_qkv, o, dout8, descale_dout, lse, dq, dk, dv,
                          softmax_scale: float = 0.0, workspace=None, sub_begin: int = 0, sub_count: int = 0,
                          stream=None):
    """Backward pass on e4m3 inputs; ``workspace`` as in skiparse_attn_bwd."""
    if workspace is None:
        import torch
        workspace = torch.empty(skiparse_attn_bwd_workspace_bytes(plan), dtype=torch.uint8, device=o.device)
    wb = workspace.numel() * workspace.element_size() if hasattr(workspace, "numel") else 0
    _check(lib().skiparse_attn_bwd_fp8(ctypes.byref(plan), _ptr(q8), _ptr(k8), _ptr(v8), _ptr(descale_qkv),
                                       _ptr(o), _ptr(dout8), _ptr(descale_dout), _ptr(lse), _ptr(dq), _ptr(dk),
                                       _ptr(dv), float(softmax_scale), _ptr(workspace), wb, sub_begin, sub_count,
                                       _stream(stream)))
    return dq, dk, dv


def skiparse_quant_fp8_workspace_bytes(numel: int) -> int:
    return int(lib().skiparse_quant_fp8_workspace_bytes(numel))


def skiparse_quant_fp8(x, y, scale, fp8_max: float = 448.0, eps: float = 1e-12, workspace=None,
                       stream=None, x_dtype=None):
    """Quantize the whole tensor ``x`` (bf16 or fp32, device) into ``y`` (uint8,
    same numel); ``scale`` receives {scale, 1/scale} (2 fp32, device)."""
    import torch
    if x_dtype is None:
        x_dtype = _float_code(x)
    numel = x.numel()
    if workspace is None:
        nb = skiparse_quant_fp8_workspace_bytes(numel)
        workspace = torch.empty(nb, dtype=torch.uint8, device=x.device)
    wb = workspace.numel() * workspace.element_size() if hasattr(workspace, "numel") else 0
    _check(lib().skiparse_quant_fp8(_ptr(x), x_dtype, numel, _ptr(y), _ptr(scale), float(fp8_max), float(eps),
                                    _ptr(workspace), wb, _stream(stream)))
    return y


def skiparse_quant_fp8_noalloc(x, y, scale, fp8_max: float = 448.0, eps: float = 1e-12, stream=None, x_dtype=None):
    """skiparse_quant_fp8 with the library's own scratch: allocates nothing.
    Calls that overlap in time on one GPU race (one shared scratch per GPU)."""
    import torch
    if x_dtype is None:
        x_dtype = _float_code(x)
    _check(lib().skiparse_quant_fp8_noalloc(_ptr(x), x_dtype, x.numel(), _ptr(y), _ptr(scale), float(fp8_max),
                                            float(eps), _stream(stream)))
    return y


def skiparse_block_workspace_bytes(plan: SkiparsePlan) -> int:
    return int(lib().skiparse_block_workspace_bytes(ctypes.byref(plan)))


def skiparse_block_fwd_fp8(plan: SkiparsePlan, x, w_qkvo, w_scales, y, rope_theta: float = 10000.0,
                           rope_dims=None, workspace=None, stream=None):
    """fp8 attention block; ``workspace`` (device, >= skiparse_block_workspace_bytes,
    256-byte aligned) is allocated with torch when None."""
    if workspace is None:
        import torch
        workspace = torch.empty(skiparse_block_workspace_bytes(plan), dtype=torch.uint8, device=x.device)
    wb = workspace.numel() * workspace.element_size() if hasattr(workspace, "numel") else 0
    dims = None if rope_dims is None else (ctypes.c_int32 * 3)(*rope_dims)
    _check(lib().skiparse_block_fwd_fp8(ctypes.byref(plan), _ptr(x), _ptr(w_qkvo), _ptr(w_scales),
                                        float(rope_theta), dims, _ptr(y), _ptr(workspace), wb, _stream(stream)))
    return y


def skiparse_gemm_fp8(x, w, sx, sw, y, stream=None):
    """y (M, N) bf16 = sx * sw * x (M, K) . w (N, K)^T on e4m3 codes (uint8
    device tensors); sx, sw: device fp32 dequantization factors (1/scale)."""
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K or tuple(y.shape) != (M, N):
        raise ValueError("shapes must be x (M, K), w (N, K), y (M, N)")
    _check(lib().skiparse_gemm_fp8(_ptr(x), _ptr(w), _ptr(sx), _ptr(sw), _ptr(y), M, N, K, _stream(stream)))
    return y


def skiparse_rope_fp8_workspace_bytes(plan: SkiparsePlan) -> int:
    return int(lib().skiparse_rope_fp8_workspace_bytes(ctypes.byref(plan)))


def skiparse_rope_fp8(plan: SkiparsePlan, x, y, scale, rope_theta: float = 10000.0, rope_dims=None,
                      workspace=None, stream=None):
    """y = e4m3 codes of the rotated x, scale = {scale, 1/scale}; ``workspace``
    is allocated with torch when None."""
    if workspace is None:
        import torch
        workspace = torch.empty(skiparse_rope_fp8_workspace_bytes(plan), dtype=torch.uint8, device=x.device)
    wb = workspace.numel() * workspace.element_size() if hasattr(workspace, "numel") else 0
    dims = None if rope_dims is None else (ctypes.c_int32 * 3)(*rope_dims)
    _check(lib().skiparse_rope_fp8(ctypes.byref(plan), _ptr(x), float(rope_theta), dims, _ptr(y), _ptr(scale),
                                   _ptr(workspace), wb, _stream(stream)))
    return y


# ---------------------------------------------------------------------------
# conveniences (torch allocates, the library computes)
# ---------------------------------------------------------------------------

def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.uint8 or t.dtype == getattr(torch, "float8_e4m3fn", None):
        return FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _float_code(x):
    """BF16 or F32 for a tensor the quantizer reads; anything else would be
    read at the wrong element size."""
    import torch
    if x.dtype == torch.bfloat16:
        return BF16
    if x.dtype == torch.float32:
        return F32
    raise TypeError(f"the quantizer reads bfloat16 or float32, not {x.dtype}")


def _check_like(names, tensors, shape, dtype, device):
    """Inputs a kernel reads at a fixed size: each must have the given shape
    and dtype and sit on the given device (layout is made contiguous by the
    caller where it copies)."""
    for name, t in zip(names, tensors):
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
        if t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, not {t.dtype}")
        if t.device != device:
            raise ValueError(f"{name} must be on {device}, not {t.device}")


def _check_lse(lse, B, N, nh, device):
    import torch
    _check_like(("lse",), (lse,), (B, N, nh), torch.float32, device)
    if not lse.is_contiguous():
        raise ValueError("lse must be contiguous")


def _check_out(out, shape, dtype, device):
    """A caller's output tensor must be exactly what the kernels write:
    contiguous, of the given shape and dtype, on the inputs' device."""
    if (tuple(out.shape) != tuple(shape) or out.dtype != dtype or not out.is_contiguous()
            or out.device != device):
        raise ValueError(f"out must be a contiguous {dtype} tensor of shape {tuple(shape)} on {device}")


def attention(q, k, v, kf: int, mode: int, softmax_scale: float = 0.0, descale_qkv=None, out=None,
              sub_begin: int = 0, sub_count: int = 0, plan: SkiparsePlan | None = None):
    """Skiparse-2D attention forward on (B, T, H, W, heads, d) device tensors."""
    import torch
    if q.dim() != 6 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one (B, T, H, W, heads, d) shape")
    for t in (q, k, v):
        if not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous")
    _check_like(("k", "v"), (k, v), q.shape, q.dtype, q.device)
    B, T, H, W, nh, d = q.shape
    code = _dtype_code(q)
    if code == FP8_E4M3:
        if descale_qkv is None:
            raise ValueError("e4m3 inputs need descale_qkv (3 x {scale, 1/scale}, fp32)")
        _check_like(("descale_qkv",), (descale_qkv,), (3, 2), torch.float32, q.device)
        if not descale_qkv.is_contiguous():
            raise ValueError("descale_qkv must be contiguous")
    if plan is None:
        plan = skiparse_plan_init(B, T, H, W, nh, d, kf, mode)
    odt = torch.float32 if code == F32 else torch.bfloat16
    if out is None:
        out = torch.empty(q.shape, dtype=odt, device=q.device)
    else:
        _check_out(out, q.shape, odt, q.device)
    skiparse_attn_fwd(plan, code, q, k, v, out, softmax_scale, descale_qkv, sub_begin, sub_count)
    return out


def quantize_fp8(x, fp8_max: float = 448.0, eps: float = 1e-12, scale_out=None):
    """Per-tensor e4m3 quantization: returns (codes uint8, scale pair fp32[2]).
    ``scale_out`` (2 fp32 on the device) receives {scale, 1/scale} if given."""
    import torch
    y = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scale_out is None:
        sc = torch.empty(2, dtype=torch.float32, device=x.device)
    else:
        _check_out(scale_out, (2,), torch.float32, x.device)
        sc = scale_out
    skiparse_quant_fp8(x.contiguous(), y, sc, fp8_max, eps)
    return y, sc


def attention_fp8(q, k, v, kf: int, mode: int, softmax_scale: float = 0.0, fp8_max: float = 448.0,
                  eps: float = 1e-12):
    """The fp8 path end to end: quantize Q, K, V per tensor on the device, then
    run the e4m3 attention kernel.  Returns (out bf16, codes (q, k, v),
    scales fp32 (3, 2) = {scale, 1/scale} per tensor)."""
    import torch
    scales = torch.empty((3, 2), dtype=torch.float32, device=q.device)
    codes = [quantize_fp8(t, fp8_max, eps, scale_out=scales[i])[0] for i, t in enumerate((q, k, v))]
    out = attention(codes[0], codes[1], codes[2], kf, mode, softmax_scale, descale_qkv=scales)
    return out, codes, scales


def attention_train(q, k, v, kf: int, mode: int, softmax_scale: float = 0.0, plan: SkiparsePlan | None = None):
    """Training forward on bf16 (B, T, H, W, heads, d) device tensors: returns
    (out, lse) with lse fp32 (B, T*H*W, heads)."""
    import torch
    if q.dim() != 6:
        raise ValueError("q must be (B, T, H, W, heads, d)")
    _check_like(("q", "k", "v"), (q, k, v), q.shape, torch.bfloat16, q.device)
    B, T, H, W, nh, d = q.shape
    if plan is None:
        plan = skiparse_plan_init(B, T, H, W, nh, d, kf, mode)
    # the kernel writes rows in contiguous order, whatever q's strides are
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, T * H * W, nh), dtype=torch.float32, device=q.device)
    skiparse_attn_fwd_lse(plan, _dtype_code(q), q.contiguous(), k.contiguous(), v.contiguous(), out, lse,
                          softmax_scale)
    return out, lse


def attention_bwd(q, k, v, o, dout, lse, kf: int, mode: int, softmax_scale: float = 0.0,
                  plan: SkiparsePlan | None = None):
    """Backward pass on bf16 device tensors: returns (dq, dk, dv)."""
    import torch
    if q.dim() != 6:
        raise ValueError("q must be (B, T, H, W, heads, d)")
    _check_like(("q", "k", "v", "o", "dout"), (q, k, v, o, dout), q.shape, torch.bfloat16, q.device)
    B, T, H, W, nh, d = q.shape
    _check_lse(lse, B, T * H * W, nh, q.device)
    if plan is None:
        plan = skiparse_plan_init(B, T, H, W, nh, d, kf, mode)
    # the kernels write rows in contiguous order, whatever q's strides are
    dq, dk, dv = (torch.empty(q.shape, dtype=torch.bfloat16, device=q.device) for _ in range(3))
    skiparse_attn_bwd(plan, _dtype_code(q), q.contiguous(), k.contiguous(), v.contiguous(), o.contiguous(),
                      dout.contiguous(), lse, dq, dk, dv, softmax_scale)
    return dq, dk, dv


def attention_train_fp8(q, k, v, kf: int, mode: int, softmax_scale: float = 0.0, fp8_max: float = 448.0,
                        eps: float = 1e-12, plan: SkiparsePlan | None = None):
    """8-bit training forward on (B, T, H, W, heads, d) device tensors:
    quantize Q, K, V per tensor, then run the e4m3 attention keeping the
    log-sum-exp.  Returns (out bf16, lse fp32 (B, T*H*W, heads), codes
    (q8, k8, v8), scales fp32 (3, 2))."""
    import torch
    if q.dim() != 6:
        raise ValueError("q must be (B, T, H, W, heads, d)")
    _check_like(("k", "v"), (k, v), q.shape, q.dtype, q.device)
    B, T, H, W, nh, d = q.shape
    if plan is None:
        plan = skiparse_plan_init(B, T, H, W, nh, d, kf, mode)
    scales = torch.empty((3, 2), dtype=torch.float32, device=q.device)
    codes = [quantize_fp8(t, fp8_max, eps, scale_out=scales[i])[0] for i, t in enumerate((q, k, v))]
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, T * H * W, nh), dtype=torch.float32, device=q.device)
    skiparse_attn_fwd_lse_fp8(plan, codes[0], codes[1], codes[2], scales, out, lse, softmax_scale)
    return out, lse, codes, scales


def attention_bwd_fp8(codes, scales, o, dout, lse, kf: int, mode: int, softmax_scale: float = 0.0,
                      fp8_max_grad: float = 448.0, eps: float = 1e-12, plan: SkiparsePlan | None = None):
    """8-bit backward: quantize dout per tensor with the gradient maximum
    fp8_max_grad, then run the backward on the e4m3 codes of Q, K, V (from
    attention_train_fp8) and of dO.  Returns (dq, dk, dv) bf16."""
    import torch
    q8, k8, v8 = codes
    if q8.dim() != 6:
        raise ValueError("the codes must be (B, T, H, W, heads, d)")
    _check_like(("q8", "k8", "v8"), (q8, k8, v8), q8.shape, torch.uint8, q8.device)
    for t in (q8, k8, v8):
        if not t.is_contiguous():
            raise ValueError("the codes must be contiguous")
    _check_like(("scales",), (scales,), (3, 2), torch.float32, q8.device)
    if not scales.is_contiguous():
        raise ValueError("scales must be contiguous")
    _check_like(("o",), (o,), q8.shape, torch.bfloat16, q8.device)
    _check_like(("dout",), (dout,), q8.shape, dout.dtype, q8.device)
    B, T, H, W, nh, d = q8.shape
    _check_lse(lse, B, T * H * W, nh, q8.device)
    if plan is None:
        plan = skiparse_plan_init(B, T, H, W, nh, d, kf, mode)
    dscale = torch.empty(2, dtype=torch.float32, device=o.device)
    dout8 = quantize_fp8(dout, fp8_max_grad, eps, scale_out=dscale)[0]
    dq, dk, dv = (torch.empty(q8.shape, dtype=torch.bfloat16, device=o.device) for _ in range(3))
    skiparse_attn_bwd_fp8(plan, q8, k8, v8, scales, o.contiguous(), dout8, dscale, lse, dq, dk, dv, softmax_scale)
    return dq, dk, dv


def quantize_weights(wq, wk, wv, wo):
    """Per-tensor e4m3 codes of four (C, C) weights (fp32 or bf16, device) in
    one (4, C, C) uint8 tensor, and their {scale, 1/scale} as fp32 (4, 2)."""
    import torch
    ws = (wq, wk, wv, wo)
    C = wq.shape[0]
    for w in ws:
        if tuple(w.shape) != (C, C):
            raise ValueError("weights must all be (C, C)")
    codes = torch.empty((4, C, C), dtype=torch.uint8, device=wq.device)
    scales = torch.empty((4, 2), dtype=torch.float32, device=wq.device)
    for i, w in enumerate(ws):
        skiparse_quant_fp8(w.contiguous(), codes[i], scales[i])
    return codes, scales


class BlockFP8:
    """The fp8 attention block on one device: e4m3 projections, rotary
    embedding, Skiparse attention.  Holds a workspace sized for the largest
    shape seen."""

    def __init__(self, w_codes, w_scales, heads: int, kf: int, mode: int, rope_theta: float = 10000.0,
                 rope_dims=None):
        self.w_codes, self.w_scales = w_codes, w_scales
        self.heads, self.kf, self.mode = heads, kf, mode
        self.rope_theta, self.rope_dims = rope_theta, rope_dims
        self._ws = None

    def __call__(self, x, out=None):
        import torch
        if x.dim() != 5 or x.dtype != torch.bfloat16 or not x.is_contiguous():
            raise ValueError("x must be contiguous bf16 (B, T, H, W, C)")
        B, T, H, W, C = x.shape
        if C % self.heads:
            raise ValueError("C must be a multiple of heads")
        plan = skiparse_plan_init(B, T, H, W, self.heads, C // self.heads, self.kf, self.mode)
        need = skiparse_block_workspace_bytes(plan)
        if self._ws is None or self._ws.numel() < need:
            self._ws = None
            self._ws = torch.empty(need, dtype=torch.uint8, device=x.device)
        if out is None:
            y = torch.empty(x.shape, dtype=torch.bfloat16, device=x.device)
        else:
            _check_out(out, x.shape, torch.bfloat16, x.device)
            y = out
        skiparse_block_fwd_fp8(plan, x, self.w_codes, self.w_scales, y, self.rope_theta, self.rope_dims, self._ws)
        return y


def _autograd_function():
    import torch

    class SkiparseAttention(torch.autograd.Function):
        """Skiparse-2D attention as a torch autograd op (bf16, device):
        ``SkiparseAttention.apply(q, k, v, kf, mode)``."""

        @staticmethod
        def forward(ctx, q, k, v, kf, mode):
            out, lse = attention_train(q, k, v, kf, mode)
            ctx.save_for_backward(q, k, v, out, lse)
            ctx.kf, ctx.mode = kf, mode
            return out

        @staticmethod
        def backward(ctx, dout):
            q, k, v, out, lse = ctx.saved_tensors
            dq, dk, dv = attention_bwd(q, k, v, out, dout, lse, ctx.kf, ctx.mode)
            return dq, dk, dv, None, None

    class SkiparseAttentionFP8(torch.autograd.Function):
        """8-bit training op: ``SkiparseAttentionFP8.apply(q, k, v, kf, mode)``
        on bf16 device tensors.  The forward quantizes Q, K, V per tensor and
        keeps only their e4m3 codes (half the bytes of bf16) with the output
        and log-sum-exp; the backward quantizes dO per tensor and returns the
        bf16 gradients of the dequantized tensors."""

        @staticmethod
        def forward(ctx, q, k, v, kf, mode):
            out, lse, codes, scales = attention_train_fp8(q, k, v, kf, mode)
            ctx.save_for_backward(*codes, scales, out, lse)
            ctx.kf, ctx.mode = kf, mode
            return out

        @staticmethod
        def backward(ctx, dout):
            q8, k8, v8, scales, out, lse = ctx.saved_tensors
            dq, dk, dv = attention_bwd_fp8((q8, k8, v8), scales, out, dout, lse, ctx.kf, ctx.mode)
            return dq, dk, dv, None, None

    return SkiparseAttention, SkiparseAttentionFP8


def __getattr__(name):
    if name in ("SkiparseAttention", "SkiparseAttentionFP8"):
        a, b = _autograd_function()
        globals()["SkiparseAttention"] = a
        globals()["SkiparseAttentionFP8"] = b
        return globals()[name]
    raise AttributeError(name)
