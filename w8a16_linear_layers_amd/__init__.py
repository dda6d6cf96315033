"""Python binding of libfp8lin (static per-tensor FP8 linear layers, MI355X).

Argument marshalling only: every function below forwards to the C entry
point of the same name in ``libfp8lin.so`` (declared in ``include/fp8lin.h``),
passing device pointers, sizes, host scales and the current HIP stream.
torch provides device memory and streams; no arithmetic of the layer runs
here. If the library is not built, loading fails loudly -- there is no
fallback path.
"""

import ctypes
import json
import os

import torch

__all__ = [
    "Fp8LinError",
    "load_library",
    "library_path",
    "MODE_W8A8",
    "MODE_W8A16",
    "DT_BF16",
    "DT_E4M3",
    "DT_F16",
    "DT_F32",
    "TOWER_GENERATION",
    "TOWER_REASONER",
    "Policy",
    "policy_from_json",
    "fp8lin_quantize_static",
    "fp8lin_gemm_w8a8",
    "fp8lin_gemm_w8a16",
    "fp8lin_gemm_w8a16_f32",
    "fp8lin_w8a16_f32_workspace_bytes",
    "fp8lin_gemm_w8a8_group",
    "fp8lin_gemm_w8a8_splitk",
    "fp8lin_gemm_w8a8_splitk_choice",
    "fp8lin_gemm_w8a8_splitk_noalloc",
    "fp8lin_gemm_w8a16_splitk",
    "fp8lin_gemm_w8a16_splitk_choice",
    "fp8lin_qkv_shared",
    "fp8lin_swiglu_2in_quant",
    "fp8lin_swiglu_2in",
    "fp8lin_gate_up_swiglu_w8a8",
    "fp8lin_gate_up_swiglu_w8a16",
    "fp8lin_quantize_dynamic",
    "fp8lin_gemm_w8a8_dev_scale",
    "fp8lin_qk_norm_rope",
    "fp8lin_qkv_w8a8_norm_rope",
    "fp8lin_policy_validate",
    "fp8lin_step_policy",
    "fp8lin_strerror",
    "fp8lin_launch_count",
    "KERNEL_QUANTIZE",
    "KERNEL_GEMM_W8A8",
    "KERNEL_GEMM_W8A16",
    "KERNEL_SWIGLU",
    "KERNEL_GATE_UP_SWIGLU",
    "KERNEL_AMAX",
    "KERNEL_SPLIT",
    "KERNEL_QK_NORM_ROPE",
    "KERNEL_SPLITK_REDUCE",
]

MODE_W8A8, MODE_W8A16 = 0, 1
DT_BF16, DT_E4M3, DT_F16, DT_F32 = 0, 1, 2, 3
TOWER_GENERATION, TOWER_REASONER = 0, 1
(
    KERNEL_QUANTIZE,
    KERNEL_GEMM_W8A8,
    KERNEL_GEMM_W8A16,
    KERNEL_SWIGLU,
    KERNEL_GATE_UP_SWIGLU,
    KERNEL_AMAX,
    KERNEL_SPLIT,
    KERNEL_QK_NORM_ROPE,
    KERNEL_SPLITK_REDUCE,
) = range(9)

# torch dtype -> fp8lin_dtype (E4M3 codes travel as uint8 or float8_e4m3fn)
_DT_OF = {
    torch.bfloat16: DT_BF16,
    torch.float16: DT_F16,
    torch.float32: DT_F32,
    torch.uint8: DT_E4M3,
    torch.float8_e4m3fn: DT_E4M3,
}
_TORCH_OF = {DT_BF16: torch.bfloat16, DT_F16: torch.float16, DT_F32: torch.float32, DT_E4M3: torch.uint8}

OK, EINVAL, ELAYOUT, EDTYPE, ESCALE, EPOLICY, EUNSUPPORTED, EHIP = 0, -1, -2, -3, -4, -5, -6, -7

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

EXPORTS = (
    "fp8lin_quantize_static",
    "fp8lin_gemm_w8a8",
    "fp8lin_gemm_w8a16",
    "fp8lin_gemm_w8a16_f32",
    "fp8lin_w8a16_f32_workspace_bytes",
    "fp8lin_gemm_w8a8_group",
    "fp8lin_gemm_w8a8_splitk",
    "fp8lin_gemm_w8a8_splitk_choice",
    "fp8lin_gemm_w8a8_splitk_noalloc",
    "fp8lin_gemm_w8a16_splitk",
    "fp8lin_gemm_w8a16_splitk_choice",
    "fp8lin_qkv_shared",
    "fp8lin_swiglu_2in_quant",
    "fp8lin_swiglu_2in",
    "fp8lin_gate_up_swiglu_w8a8",
    "fp8lin_gate_up_swiglu_w8a16",
    "fp8lin_quantize_dynamic",
    "fp8lin_gemm_w8a8_dev_scale",
    "fp8lin_qk_norm_rope",
    "fp8lin_qkv_w8a8_norm_rope",
    "fp8lin_policy_validate",
    "fp8lin_step_policy",
    "fp8lin_strerror",
    "fp8lin_launch_count",
)


class Fp8LinError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (what, fp8lin_strerror(status), status))


class Policy(ctypes.Structure):
    """fp8lin_policy (see include/fp8lin.h)."""

    _fields_ = [
        ("schema_version", ctypes.c_int32),
        ("type", ctypes.c_int32),
        ("index_space", ctypes.c_int32),
        ("default_mode", ctypes.c_int32),
        ("overlap", ctypes.c_int32),
        ("first_steps", ctypes.c_int32),
        ("last_steps", ctypes.c_int32),
        ("reasoner_mode", ctypes.c_int32),
        ("present_mask", ctypes.c_uint32),
    ]


def library_path():
    return os.path.join(_HERE, "libfp8lin.so")


def load_library():
    """Load libfp8lin.so (once). Raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            "libfp8lin.so is not built (%s); run `python -m w8a16_linear_layers_amd.build` "
            "or __graft_entry__.build()" % path
        )
    lib = ctypes.CDLL(path)
    i32, i64, f32, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
    lib.fp8lin_quantize_static.argtypes = [vp, vp, i64, i64, f32, vp]
    lib.fp8lin_gemm_w8a8.argtypes = [vp, vp, vp, i64, i64, i64, i64, f32, f32, vp]
    lib.fp8lin_gemm_w8a16.argtypes = [vp, i32, vp, vp, i64, i64, i64, i64, f32, vp]
    lib.fp8lin_gemm_w8a16_f32.argtypes = [vp, vp, vp, i64, i64, i64, i64, f32, vp, i64, vp]
    lib.fp8lin_w8a16_f32_workspace_bytes.argtypes = [i64, i64]
    lib.fp8lin_w8a16_f32_workspace_bytes.restype = i64
    lib.fp8lin_swiglu_2in.argtypes = [vp, vp, i32, vp, i32, i64, i64, f32, vp]
    lib.fp8lin_gemm_w8a8_group.argtypes = [
        vp, i64, i64, i32, ctypes.POINTER(vp), ctypes.POINTER(i64), ctypes.POINTER(f32), f32, ctypes.POINTER(vp), vp,
    ]
    lib.fp8lin_qkv_shared.argtypes = [
        vp, i64, i64, i32, ctypes.POINTER(vp), ctypes.POINTER(i64), ctypes.POINTER(f32),
        ctypes.POINTER(f32), ctypes.POINTER(vp), vp, i32, vp,
    ]
    lib.fp8lin_swiglu_2in_quant.argtypes = [vp, vp, vp, i32, i64, i64, f32, vp]
    lib.fp8lin_gate_up_swiglu_w8a8.argtypes = [vp, i64, i64, vp, vp, i64, f32, f32, f32, f32, vp, vp]
    lib.fp8lin_gate_up_swiglu_w8a16.argtypes = [vp, i32, i64, i64, vp, vp, i64, f32, f32, vp, vp]
    lib.fp8lin_quantize_dynamic.argtypes = [vp, vp, i64, i64, vp, vp, vp]
    lib.fp8lin_gemm_w8a8_dev_scale.argtypes = [vp, vp, vp, i64, i64, i64, i64, vp, f32, vp]
    lib.fp8lin_gemm_w8a8_splitk.argtypes = [vp, vp, vp, i64, i64, i64, i64, f32, f32, i32, vp, i64, vp]
    lib.fp8lin_gemm_w8a8_splitk_choice.argtypes = [i64, i64, i64]
    lib.fp8lin_gemm_w8a8_splitk_noalloc.argtypes = [vp, vp, vp, i64, i64, i64, i64, f32, f32, i32, vp]
    lib.fp8lin_gemm_w8a16_splitk.argtypes = [vp, i32, vp, vp, i64, i64, i64, i64, f32, i32, vp, i64, vp]
    lib.fp8lin_gemm_w8a16_splitk_choice.argtypes = [i64, i64, i64]
    lib.fp8lin_qk_norm_rope.argtypes = [vp, vp, vp, vp, i64, i32, i32, i32, vp, vp, vp, vp, f32, vp]
    lib.fp8lin_qkv_w8a8_norm_rope.argtypes = [
        vp, i64, i64, i32, ctypes.POINTER(vp), ctypes.POINTER(i64), ctypes.POINTER(f32), f32, ctypes.POINTER(vp),
        vp, vp, vp, vp, f32, vp,
    ]
    lib.fp8lin_policy_validate.argtypes = [ctypes.POINTER(Policy)]
    lib.fp8lin_step_policy.argtypes = [ctypes.POINTER(Policy), i32, i32, i32, ctypes.POINTER(i32)]
    lib.fp8lin_strerror.argtypes = [i32]
    lib.fp8lin_strerror.restype = ctypes.c_char_p
    lib.fp8lin_launch_count.argtypes = [i32]
    lib.fp8lin_launch_count.restype = i64
    for name in EXPORTS:
        if name not in ("fp8lin_strerror", "fp8lin_launch_count", "fp8lin_w8a16_f32_workspace_bytes"):
            getattr(lib, name).restype = i32
    _LIB = lib
    return lib


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _check(status, what):
    if status != OK:
        raise Fp8LinError(status, what)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _rows(t):
    """Flatten the leading dimensions of a rank-N tensor: [..., K] -> (rows, K)."""
    k = t.shape[-1] if t.dim() > 0 else 1
    return (t.numel() // k if k else 0), k


def fp8lin_quantize_static(x, input_scale, out=None, stream=None):
    """E4M3 codes (torch.uint8, same shape as x) of a bf16 tensor x."""
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    rows, cols = _rows(x)
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _check(
        load_library().fp8lin_quantize_static(_ptr(x), _ptr(out), rows, cols, float(input_scale), _stream(stream)),
        "fp8lin_quantize_static",
    )
    return out


def _gemm_out(m_shape, n, device, out, ldy, dtype=torch.bfloat16):
    if out is None:
        out = torch.empty(tuple(m_shape) + (n,), dtype=dtype, device=device)
        ldy = n
    elif ldy is None:
        ldy = out.stride(-2) if out.dim() >= 2 else n
    return out, ldy


def fp8lin_gemm_w8a8(qx, qw, input_scale, weight_scale, out=None, ldy=None, stream=None):
    """y = (dec(qx) dec(qw)^T) * s_in * s_w in bf16; qx [..., K] uint8, qw [N, K] uint8."""
    if qx.dtype != torch.uint8 or qw.dtype != torch.uint8:
        raise TypeError("qx and qw must hold E4M3 codes as torch.uint8")
    m, k = _rows(qx)
    n = qw.shape[0]
    out, ldy = _gemm_out(qx.shape[:-1], n, qx.device, out, ldy)
    _check(
        load_library().fp8lin_gemm_w8a8(
            _ptr(qx), _ptr(qw), _ptr(out), m, n, k, ldy, float(input_scale), float(weight_scale), _stream(stream)
        ),
        "fp8lin_gemm_w8a8",
    )
    return out


def fp8lin_gemm_w8a16(x, qw, weight_scale, out=None, ldy=None, stream=None):
    """y = (x dec(qw)^T) * s_w in x's 16-bit dtype; x [..., K] bf16 or fp16.

    FP8 and float32 activations are passed on as such and refused by the
    library (float32 takes fp8lin_gemm_w8a16_f32)."""
    if x.dtype not in _DT_OF:
        raise TypeError("x must be bfloat16 or float16")
    dtype = _DT_OF[x.dtype]
    m, k = _rows(x)
    n = qw.shape[0]
    out, ldy = _gemm_out(x.shape[:-1], n, x.device, out, ldy, x.dtype if dtype in (DT_BF16, DT_F16) else torch.bfloat16)
    _check(
        load_library().fp8lin_gemm_w8a16(
            _ptr(x), dtype, _ptr(qw), _ptr(out), m, n, k, ldy, float(weight_scale), _stream(stream)
        ),
        "fp8lin_gemm_w8a16",
    )
    return out


def fp8lin_gemm_w8a8_splitk_choice(m, n, k):
    """The split count fp8lin_gemm_w8a8_splitk does best with on this device (1 = no split)."""
    return int(load_library().fp8lin_gemm_w8a8_splitk_choice(int(m), int(n), int(k)))


def fp8lin_gemm_w8a8_splitk(qx, qw, input_scale, weight_scale, splits=None, out=None, ldy=None, workspace=None,
                            stream=None):
    """fp8lin_gemm_w8a8 with K split into `splits` float32 partial products (default: the device's choice)."""
    if qx.dtype != torch.uint8 or qw.dtype != torch.uint8:
        raise TypeError("qx and qw must hold E4M3 codes as torch.uint8")
    m, k = _rows(qx)
    n = qw.shape[0]
    if splits is None:
        splits = fp8lin_gemm_w8a8_splitk_choice(m, n, k)
    out, ldy = _gemm_out(qx.shape[:-1], n, qx.device, out, ldy)
    need = int(splits) * m * n * 4 if splits > 1 else 16
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=qx.device)
    _check(
        load_library().fp8lin_gemm_w8a8_splitk(
            _ptr(qx), _ptr(qw), _ptr(out), m, n, k, ldy, float(input_scale), float(weight_scale), int(splits),
            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)
        ),
        "fp8lin_gemm_w8a8_splitk",
    )
    return out


SCRATCH_BYTES = 32 * 1024 * 1024  # FP8LIN_SCRATCH_BYTES: the library's static scratch array per GPU


def fp8lin_gemm_w8a8_splitk_noalloc(qx, qw, input_scale, weight_scale, splits=None, out=None, ldy=None, stream=None):
    """fp8lin_gemm_w8a8_splitk with the float32 partials in the library's static scratch array: the C call
    allocates nothing (the output is allocated here only when `out` is not given). splits * M * N * 4 must fit
    SCRATCH_BYTES; calls that overlap on one GPU race (one scratch array per GPU)."""
    if qx.dtype != torch.uint8 or qw.dtype != torch.uint8:
        raise TypeError("qx and qw must hold E4M3 codes as torch.uint8")
    m, k = _rows(qx)
    n = qw.shape[0]
    if splits is None:
        splits = fp8lin_gemm_w8a8_splitk_choice(m, n, k)
    out, ldy = _gemm_out(qx.shape[:-1], n, qx.device, out, ldy)
    _check(
        load_library().fp8lin_gemm_w8a8_splitk_noalloc(
            _ptr(qx), _ptr(qw), _ptr(out), m, n, k, ldy, float(input_scale), float(weight_scale), int(splits),
            _stream(stream)
        ),
        "fp8lin_gemm_w8a8_splitk_noalloc",
    )
    return out


def fp8lin_gemm_w8a16_splitk_choice(m, n, k):
    """The split count for fp8lin_gemm_w8a16_splitk on this device (1 = no split)."""
    return int(load_library().fp8lin_gemm_w8a16_splitk_choice(int(m), int(n), int(k)))


def fp8lin_gemm_w8a16_splitk(x, qw, weight_scale, splits=None, out=None, ldy=None, workspace=None, stream=None):
    """fp8lin_gemm_w8a16 with K split into `splits` float32 partial products (default: the device's choice);
    bf16 activations (binary16 ones only with splits = 1)."""
    if x.dtype not in _DT_OF:
        raise TypeError("x must be bfloat16 or float16")
    dtype = _DT_OF[x.dtype]
    m, k = _rows(x)
    n = qw.shape[0]
    if splits is None:
        splits = fp8lin_gemm_w8a16_splitk_choice(m, n, k) if dtype == DT_BF16 else 1
    out, ldy = _gemm_out(x.shape[:-1], n, x.device, out, ldy, x.dtype)
    need = int(splits) * m * n * 4 if splits > 1 else 16
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    _check(
        load_library().fp8lin_gemm_w8a16_splitk(
            _ptr(x), dtype, _ptr(qw), _ptr(out), m, n, k, ldy, float(weight_scale), int(splits),
            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)
        ),
        "fp8lin_gemm_w8a16_splitk",
    )
    return out


def fp8lin_w8a16_f32_workspace_bytes(m, k):
    """Bytes of the workspace fp8lin_gemm_w8a16_f32 needs for an [m, k] activation."""
    return int(load_library().fp8lin_w8a16_f32_workspace_bytes(int(m), int(k)))


def fp8lin_gemm_w8a16_f32(x, qw, weight_scale, out=None, ldy=None, workspace=None, stream=None):
    """y = (x dec(qw)^T) * s_w in float32 from a float32 x [..., K] (exact products, float32 sums)."""
    if x.dtype != torch.float32:
        raise TypeError("x must be float32")
    m, k = _rows(x)
    n = qw.shape[0]
    out, ldy = _gemm_out(x.shape[:-1], n, x.device, out, ldy, torch.float32)
    need = fp8lin_w8a16_f32_workspace_bytes(m, k)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    _check(
        load_library().fp8lin_gemm_w8a16_f32(
            _ptr(x), _ptr(qw), _ptr(out), m, n, k, ldy, float(weight_scale), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream)
        ),
        "fp8lin_gemm_w8a16_f32",
    )
    return out


def fp8lin_gemm_w8a8_group(qx, qws, input_scale, weight_scales, outs=None, stream=None):
    """The projections of a group on one quantized activation, in one launch; returns the bf16 outputs."""
    if qx.dtype != torch.uint8 or any(w.dtype != torch.uint8 for w in qws):
        raise TypeError("qx and the weights must hold E4M3 codes as torch.uint8")
    m, k = _rows(qx)
    n = len(qws)
    if outs is None:
        outs = [torch.empty(tuple(qx.shape[:-1]) + (w.shape[0],), dtype=torch.bfloat16, device=qx.device) for w in qws]
    vp, i64, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float
    c_w = (vp * n)(*[w.data_ptr() for w in qws])
    c_n = (i64 * n)(*[w.shape[0] for w in qws])
    c_sw = (f32 * n)(*[float(s) for s in weight_scales])
    c_y = (vp * n)(*[o.data_ptr() for o in outs])
    _check(
        load_library().fp8lin_gemm_w8a8_group(
            _ptr(qx), m, k, n, c_w, c_n, c_sw, float(input_scale), c_y, _stream(stream)
        ),
        "fp8lin_gemm_w8a8_group",
    )
    return outs


def fp8lin_qkv_shared(x, qws, weight_scales, input_scales, mode, outs=None, workspace=None, stream=None):
    """Shared-input projections; returns (list of bf16 outputs, workspace codes or None)."""
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    m, k = _rows(x)
    n = len(qws)
    if outs is None:
        outs = [torch.empty(tuple(x.shape[:-1]) + (w.shape[0],), dtype=torch.bfloat16, device=x.device) for w in qws]
    if mode == MODE_W8A8 and workspace is None:
        workspace = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    vp, i64, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float
    c_w = (vp * n)(*[w.data_ptr() for w in qws])
    c_n = (i64 * n)(*[w.shape[0] for w in qws])
    c_sw = (f32 * n)(*[float(s) for s in weight_scales])
    c_si = (f32 * n)(*[float(s) for s in input_scales])
    c_y = (vp * n)(*[o.data_ptr() for o in outs])
    _check(
        load_library().fp8lin_qkv_shared(
            _ptr(x), m, k, n, c_w, c_n, c_sw, c_si, c_y, _ptr(workspace), int(mode), _stream(stream)
        ),
        "fp8lin_qkv_shared",
    )
    return outs, (workspace if mode == MODE_W8A8 else None)


def fp8lin_swiglu_2in_quant(gate, up, out_scale=1.0, out_dtype=DT_E4M3, out=None, stream=None):
    """silu(gate) * up as E4M3 codes (uint8) or bf16; gate/up contiguous bf16 of one shape."""
    if gate.dtype != torch.bfloat16 or up.dtype != torch.bfloat16:
        raise TypeError("gate and up must be bfloat16")
    if gate.shape != up.shape:
        raise ValueError("gate and up must have the same shape")
    if not (gate.is_contiguous() and up.is_contiguous()):
        raise ValueError("gate and up must be contiguous")
    rows, cols = _rows(gate)
    if out is None:
        dt = torch.uint8 if out_dtype == DT_E4M3 else torch.bfloat16
        out = torch.empty(gate.shape, dtype=dt, device=gate.device)
    _check(
        load_library().fp8lin_swiglu_2in_quant(
            _ptr(gate), _ptr(up), _ptr(out), int(out_dtype), rows, cols, float(out_scale), _stream(stream)
        ),
        "fp8lin_swiglu_2in_quant",
    )
    return out


def fp8lin_swiglu_2in(gate, up, out_scale=1.0, out_dtype=DT_E4M3, out=None, stream=None):
    """silu(gate) * up from bf16 or fp16 inputs, as E4M3 codes (uint8) or in the input's dtype."""
    if gate.dtype != up.dtype or gate.dtype not in _DT_OF:
        raise TypeError("gate and up must share a supported dtype")
    if gate.shape != up.shape:
        raise ValueError("gate and up must have the same shape")
    if not (gate.is_contiguous() and up.is_contiguous()):
        raise ValueError("gate and up must be contiguous")
    rows, cols = _rows(gate)
    if out is None:
        out = torch.empty(gate.shape, dtype=_TORCH_OF.get(int(out_dtype), torch.uint8), device=gate.device)
    _check(
        load_library().fp8lin_swiglu_2in(
            _ptr(gate), _ptr(up), _DT_OF[gate.dtype], _ptr(out), int(out_dtype), rows, cols, float(out_scale),
            _stream(stream)
        ),
        "fp8lin_swiglu_2in",
    )
    return out


def fp8lin_gate_up_swiglu_w8a8(qx, qw_gate, qw_up, input_scale, gate_scale, up_scale, out_scale, out=None,
                               stream=None):
    """h = E4M3(silu(g) * u / out_scale) with g, u the bf16 W8A8 gate/up outputs, in one launch (uint8 codes)."""
    if qx.dtype != torch.uint8 or qw_gate.dtype != torch.uint8 or qw_up.dtype != torch.uint8:
        raise TypeError("qx and the weights must hold E4M3 codes as torch.uint8")
    if qw_gate.shape != qw_up.shape:
        raise ValueError("gate and up weights must have the same shape")
    m, k = _rows(qx)
    inter = qw_gate.shape[0]
    if out is None:
        out = torch.empty(tuple(qx.shape[:-1]) + (inter,), dtype=torch.uint8, device=qx.device)
    _check(
        load_library().fp8lin_gate_up_swiglu_w8a8(
            _ptr(qx), m, k, _ptr(qw_gate), _ptr(qw_up), inter, float(input_scale), float(gate_scale),
            float(up_scale), float(out_scale), _ptr(out), _stream(stream)
        ),
        "fp8lin_gate_up_swiglu_w8a8",
    )
    return out


def fp8lin_gate_up_swiglu_w8a16(x, qw_gate, qw_up, gate_scale, up_scale, out=None, stream=None):
    """h = silu(g) * u with g, u the W8A16 gate/up outputs, in one launch, in x's 16-bit dtype (FP8 refused)."""
    if x.dtype not in _DT_OF:
        raise TypeError("x must be bfloat16 or float16")
    dtype = _DT_OF[x.dtype]
    if qw_gate.dtype != torch.uint8 or qw_up.dtype != torch.uint8:
        raise TypeError("the weights must hold E4M3 codes as torch.uint8")
    if qw_gate.shape != qw_up.shape:
        raise ValueError("gate and up weights must have the same shape")
    m, k = _rows(x)
    inter = qw_gate.shape[0]
    if out is None:
        odt = x.dtype if dtype in (DT_BF16, DT_F16) else torch.bfloat16
        out = torch.empty(tuple(x.shape[:-1]) + (inter,), dtype=odt, device=x.device)
    _check(
        load_library().fp8lin_gate_up_swiglu_w8a16(
            _ptr(x), dtype, m, k, _ptr(qw_gate), _ptr(qw_up), inter, float(gate_scale), float(up_scale), _ptr(out),
            _stream(stream)
        ),
        "fp8lin_gate_up_swiglu_w8a16",
    )
    return out


def fp8lin_qk_norm_rope(q, k, q_weight, k_weight, cos, sin, head_dim, eps=1e-6, q_out=None, k_out=None,
                        stream=None):
    """Per-head RMSNorm + rotate-half RoPE of bf16 q [tokens, Hq * D] and k [tokens, Hk * D].

    cos, sin: float32 [tokens, D / 2]; weights bf16 [D] or None. Pass
    q_out=q / k_out=k to work in place. Returns (q_out, k_out)."""
    if q.dtype != torch.bfloat16 or (k is not None and k.dtype != torch.bfloat16):
        raise TypeError("q and k must be bfloat16")
    if cos.dtype != torch.float32 or sin.dtype != torch.float32:
        raise TypeError("cos and sin must be float32")
    tokens = q.shape[0] if q.dim() > 0 else 0
    qh = q.shape[-1] // head_dim
    kh = k.shape[-1] // head_dim if k is not None else 0
    if q_out is None:
        q_out = torch.empty_like(q)
    if k is not None and k_out is None:
        k_out = torch.empty_like(k)
    _check(
        load_library().fp8lin_qk_norm_rope(
            _ptr(q), _ptr(k), _ptr(q_out), _ptr(k_out), tokens, qh, kh, int(head_dim), _ptr(q_weight),
            _ptr(k_weight), _ptr(cos), _ptr(sin), float(eps), _stream(stream)
        ),
        "fp8lin_qk_norm_rope",
    )
    return q_out, k_out


def fp8lin_qkv_w8a8_norm_rope(qx, qws, input_scale, weight_scales, q_weight, k_weight, cos, sin, eps=1e-6,
                              outs=None, stream=None):
    """Grouped W8A8 Q, K (, V) projections with the per-head (128) RMSNorm + RoPE on Q and K in the epilogue."""
    m, k = _rows(qx)
    n = len(qws)
    if outs is None:
        outs = [torch.empty(tuple(qx.shape[:-1]) + (w.shape[0],), dtype=torch.bfloat16, device=qx.device) for w in qws]
    vp, i64, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float
    _check(
        load_library().fp8lin_qkv_w8a8_norm_rope(
            _ptr(qx), m, k, n, (vp * n)(*[w.data_ptr() for w in qws]), (i64 * n)(*[w.shape[0] for w in qws]),
            (f32 * n)(*[float(s) for s in weight_scales]), float(input_scale), (vp * n)(*[o.data_ptr() for o in outs]),
            _ptr(q_weight), _ptr(k_weight), _ptr(cos), _ptr(sin), float(eps), _stream(stream)
        ),
        "fp8lin_qkv_w8a8_norm_rope",
    )
    return outs


def fp8lin_quantize_dynamic(x, out=None, scale=None, workspace=None, stream=None):
    """(codes, scale): E4M3 codes of bf16 x with its own runtime scale; `scale` is a 1-element float32 device tensor."""
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    rows, cols = _rows(x)
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = torch.empty(1, dtype=torch.int32, device=x.device)
    _check(
        load_library().fp8lin_quantize_dynamic(_ptr(x), _ptr(out), rows, cols, _ptr(scale), _ptr(workspace),
                                               _stream(stream)),
        "fp8lin_quantize_dynamic",
    )
    return out, scale


def fp8lin_gemm_w8a8_dev_scale(qx, qw, input_scale_dev, weight_scale, out=None, ldy=None, stream=None):
    """fp8lin_gemm_w8a8 with the input scale taken from a 1-element float32 device tensor."""
    if qx.dtype != torch.uint8 or qw.dtype != torch.uint8:
        raise TypeError("qx and qw must hold E4M3 codes as torch.uint8")
    if input_scale_dev.dtype != torch.float32 or input_scale_dev.numel() < 1:
        raise TypeError("input_scale_dev must be a float32 device tensor")
    m, k = _rows(qx)
    n = qw.shape[0]
    out, ldy = _gemm_out(qx.shape[:-1], n, qx.device, out, ldy)
    _check(
        load_library().fp8lin_gemm_w8a8_dev_scale(
            _ptr(qx), _ptr(qw), _ptr(out), m, n, k, ldy, _ptr(input_scale_dev), float(weight_scale), _stream(stream)
        ),
        "fp8lin_gemm_w8a8_dev_scale",
    )
    return out


# ---------------------------------------------------------------- policy

_POLICY_FIELDS = (
    "schema_version",
    "type",
    "index_space",
    "default_mode",
    "overlap",
    "first_steps",
    "last_steps",
    "reasoner",
)
_ENUMS = {
    "type": {"first_last_steps": 1},
    "index_space": {"scheduler_step": 1},
    "default_mode": {"w8a8": MODE_W8A8, "w8a16": MODE_W8A16},
    "overlap": {"a16": 1},
    "reasoner": {"a8": MODE_W8A8, "a16": MODE_W8A16},
}
_UNKNOWN = -1


def _int_field(v):
    return v if isinstance(v, int) and not isinstance(v, bool) and -(2**31) <= v < 2**31 else None


def policy_from_json(doc):
    """Parse a diffusion_step_policy (dict or JSON text) into a Policy.

    Returns None for a null policy (runtime: null). Field values are mapped
    without judging them; fp8lin_policy_validate decides. Unknown fields set
    the unknown-field bit; a non-integer count becomes -1 (refused).
    """
    if isinstance(doc, (str, bytes)):
        doc = json.loads(doc)
    if doc is None:
        return None
    p = Policy()
    if not isinstance(doc, dict):
        p.present_mask = 1 << 31
        return p
    mask = 0
    for i, f in enumerate(_POLICY_FIELDS):
        if f in doc:
            mask |= 1 << i
    if set(doc) - set(_POLICY_FIELDS):
        mask |= 1 << 31
    p.present_mask = mask
    sv = _int_field(doc.get("schema_version"))
    p.schema_version = sv if sv is not None else _UNKNOWN
    for f, attr in (("type", "type"), ("index_space", "index_space"), ("default_mode", "default_mode"),
                    ("overlap", "overlap"), ("reasoner", "reasoner_mode")):
        v = doc.get(f)
        setattr(p, attr, _ENUMS[f].get(v, _UNKNOWN) if isinstance(v, str) else _UNKNOWN)
    for f in ("first_steps", "last_steps"):
        v = _int_field(doc.get(f))
        setattr(p, f, v if v is not None else _UNKNOWN)
    return p


def fp8lin_policy_validate(policy):
    return load_library().fp8lin_policy_validate(ctypes.byref(policy) if policy is not None else None)


def fp8lin_step_policy(policy, tower, step, num_steps):
    """Mode (MODE_W8A8 / MODE_W8A16) of one call; raises Fp8LinError on a bad policy."""
    out = ctypes.c_int32(-1)
    st = load_library().fp8lin_step_policy(
        ctypes.byref(policy) if policy is not None else None, int(tower), int(step), int(num_steps), ctypes.byref(out)
    )
    _check(st, "fp8lin_step_policy")
    return out.value


def fp8lin_strerror(status):
    return load_library().fp8lin_strerror(int(status)).decode()


def fp8lin_launch_count(kind):
    return load_library().fp8lin_launch_count(int(kind))
