"""Python binding of libmt.so, the MI355X tensor-parallel GPT layer-shard library.

Argument marshalling only: every step of the layer runs in the HIP kernels behind the
C ABI of include/mt.h. torch tensors provide device memory and the stream; nothing
here computes. If the library has not been built, loading fails loudly (build it with
``python -m tensor_layer_gemms_amd.build``).

Names follow include/mt.h: layer_fwd / layer_bwd / mlp_fwd / mlp_bwd, adamw_step and
the *_bytes queries; Shape, LayerWeights and LayerGrads mirror the C structs.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmt.so")

MT_OK, MT_ERR_INVALID_ARG, MT_ERR_UNSUPPORTED, MT_ERR_HIP, MT_ERR_WORKSPACE, MT_ERR_NOALLOC_LIMIT = range(6)
NOALLOC_SCRATCH_BYTES = 64 << 20  # MT_NOALLOC_SCRATCH_BYTES of include/mt.h
MT_BF16, MT_FP32, MT_BF16_QK = 0, 1, 2
_DTYPES = {"bf16": MT_BF16, "fp32": MT_FP32, "bf16qk": MT_BF16_QK}

WEIGHT_NAMES = ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_o", "b_o",
                "ln2_g", "ln2_b", "w_fc1", "b_fc1", "w_fc2", "b_fc2")

# C function name -> (restype, argtypes)
_VP, _SZ, _I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int


class Shape(ctypes.Structure):
    _fields_ = [("h", ctypes.c_int32), ("heads", ctypes.c_int32), ("seq", ctypes.c_int32),
                ("micro_batch", ctypes.c_int32), ("tp", ctypes.c_int32), ("shard", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in WEIGHT_NAMES]


class LayerGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in WEIGHT_NAMES]


_SIGS = {
    "mt_layer_saved_bytes": (_SZ, [ctypes.POINTER(Shape)]),
    "mt_layer_workspace_bytes": (_SZ, [ctypes.POINTER(Shape)]),
    "mt_layer_fwd": (_I, [ctypes.POINTER(Shape), ctypes.POINTER(LayerWeights), _VP, _VP, _VP, _SZ, _VP, _SZ, _VP]),
    "mt_layer_bwd": (_I, [ctypes.POINTER(Shape), ctypes.POINTER(LayerWeights), _VP, _VP, _SZ, _VP, _VP,
                          ctypes.POINTER(LayerGrads), _VP, _SZ, _VP]),
    "mt_mlp_saved_bytes": (_SZ, [ctypes.POINTER(Shape)]),
    "mt_mlp_workspace_bytes": (_SZ, [ctypes.POINTER(Shape)]),
    "mt_mlp_fwd": (_I, [ctypes.POINTER(Shape), _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP, _SZ, _VP]),
    "mt_mlp_bwd": (_I, [ctypes.POINTER(Shape), _VP, _VP, _VP, _VP, _SZ, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "mt_mlp_bwd_noalloc": (_I, [ctypes.POINTER(Shape), _VP, _VP, _VP, _VP, _SZ, _VP, _VP, _VP, _VP, _VP, _VP]),
    "mt_attn_saved_bytes": (_SZ, [ctypes.POINTER(Shape)]),
    "mt_attn_workspace_bytes": (_SZ, [ctypes.POINTER(Shape)]),
    "mt_attn_fwd": (_I, [ctypes.POINTER(Shape), _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP, _SZ, _VP]),
    "mt_attn_bwd": (_I, [ctypes.POINTER(Shape), _VP, _VP, _VP, _VP, _SZ, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "mt_sp_ln_fwd": (_I, [ctypes.POINTER(Shape), _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
    "mt_sp_add_fwd": (_I, [ctypes.POINTER(Shape), _VP, _VP, _VP, _VP, _VP]),
    "mt_sp_ln_workspace_bytes": (_SZ, [ctypes.POINTER(Shape)]),
    "mt_sp_ln_bwd": (_I, [ctypes.POINTER(Shape), _VP, _VP, _I, _VP, _VP, _VP, _VP, _I, _VP, _VP, _VP, _VP, _VP,
                          _VP, _VP, _SZ, _VP]),
    "mt_adamw_step": (_I, [ctypes.c_int64, _VP, _VP, _VP, _VP, _VP, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                           ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_int32, _VP]),
    "mt_status_string": (ctypes.c_char_p, [_I]),
    "mt_timing_enable": (_I, [_I, ctypes.c_char_p]),
    "mt_timing_reset": (_I, []),
    "mt_timing_count": (_I, []),
    "mt_timing_get": (_I, [_I, ctypes.c_char_p, _SZ, ctypes.POINTER(ctypes.c_float),
                           ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]),
}
EXPORTED = tuple(_SIGS)

_lib: Optional[ctypes.CDLL] = None


class MTError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: status {status} ({status_string(status)})")


def lib() -> ctypes.CDLL:
    """Load libmt.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build the HIP library first "
                               "(python -m tensor_layer_gemms_amd.build)")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(l, name)
            fn.restype, fn.argtypes = res, args
        _lib = l
    return _lib


def status_string(status: int) -> str:
    return lib().mt_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != MT_OK:
        raise MTError(fn, status)


def make_shape(h: int, heads: int, seq: int, micro_batch: int, tp: int = 1, shard: int = 0,
               dtype: str = "bf16") -> Shape:
    """dtype: "bf16" (MT_BF16), "fp32" (MT_FP32) or "bf16qk" (MT_BF16_QK: bf16 with the
    attention logits formed from hi + lo pairs of Q and K)."""
    if dtype not in _DTYPES:
        raise ValueError(f"dtype {dtype!r}: expected one of {sorted(_DTYPES)}")
    return Shape(h, heads, seq, micro_batch, tp, shard, _DTYPES[dtype])


def _ptr(t) -> int:
    """Device address of a tensor (or a raw integer address / None)."""
    if t is None:
        return 0
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _nbytes(t) -> int:
    if t is None or isinstance(t, int):
        return 0
    return t.numel() * t.element_size()


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def layer_saved_bytes(shape: Shape) -> int:
    return lib().mt_layer_saved_bytes(ctypes.byref(shape))


def layer_workspace_bytes(shape: Shape) -> int:
    return lib().mt_layer_workspace_bytes(ctypes.byref(shape))


def mlp_saved_bytes(shape: Shape) -> int:
    return lib().mt_mlp_saved_bytes(ctypes.byref(shape))


def mlp_workspace_bytes(shape: Shape) -> int:
    return lib().mt_mlp_workspace_bytes(ctypes.byref(shape))


def layer_weights(w: Dict[str, object]) -> LayerWeights:
    return LayerWeights(*[_ptr(w.get(n)) for n in WEIGHT_NAMES])


def layer_grads(g: Dict[str, object]) -> LayerGrads:
    return LayerGrads(*[_ptr(g.get(n)) for n in WEIGHT_NAMES])


def weight_shapes(shape: Shape) -> Dict[str, Tuple[int, ...]]:
    """Shard-local weight shapes of mt_layer_weights for `shape`."""
    h, t = shape.h, shape.tp
    ht, ft = h // t, 4 * h // t
    return dict(ln1_g=(h,), ln1_b=(h,), w_qkv=(3 * ht, h), b_qkv=(3 * ht,), w_o=(h, ht), b_o=(h,),
                ln2_g=(h,), ln2_b=(h,), w_fc1=(ft, h), b_fc1=(ft,), w_fc2=(h, ft), b_fc2=(h,))


def _expect(name: str, t, numel: int, dtype=None) -> None:
    """Host-side check that a tensor is a contiguous device buffer of the size the
    kernels will index (the C side cannot see tensor sizes)."""
    if t is None:
        raise ValueError(f"{name}: missing tensor")
    if isinstance(t, int):
        return
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name}: must be a contiguous device tensor")
    if t.numel() != numel:
        raise ValueError(f"{name}: has {t.numel()} elements, the shape needs {numel}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")


def _act_dtype(shape: Shape):
    import torch
    return torch.float32 if shape.dtype == MT_FP32 else torch.bfloat16


def check_layer_tensors(shape: Shape, weights: Dict[str, object], grads: Optional[Dict[str, object]] = None,
                        **acts) -> None:
    """Raise unless every tensor matches `shape` (call before launching)."""
    import torch
    import math
    M = shape.micro_batch * shape.seq
    for n, shp in weight_shapes(shape).items():
        _expect(n, weights.get(n), math.prod(shp), _act_dtype(shape))
        if grads is not None:
            _expect("grad " + n, grads.get(n), math.prod(shp), torch.float32)
    for n, t in acts.items():
        _expect(n, t, M * shape.h, _act_dtype(shape))


def layer_fwd(shape: Shape, weights: Dict[str, object], x, out, saved, workspace, stream=None) -> None:
    """mt_layer_fwd: x [M, h] -> out [M, h]; saved / workspace are byte buffers."""
    w = layer_weights(weights)
    _check("mt_layer_fwd", lib().mt_layer_fwd(ctypes.byref(shape), ctypes.byref(w), _ptr(x), _ptr(out), _ptr(saved),
                                              _nbytes(saved), _ptr(workspace), _nbytes(workspace), _stream(stream)))


def layer_bwd(shape: Shape, weights: Dict[str, object], x, saved, dout, dx, grads: Dict[str, object], workspace,
              stream=None) -> None:
    """mt_layer_bwd: dout [M, h] -> dx [M, h] and the fp32 parameter gradients."""
    w, g = layer_weights(weights), layer_grads(grads)
    _check("mt_layer_bwd", lib().mt_layer_bwd(ctypes.byref(shape), ctypes.byref(w), _ptr(x), _ptr(saved),
                                              _nbytes(saved), _ptr(dout), _ptr(dx), ctypes.byref(g), _ptr(workspace),
                                              _nbytes(workspace), _stream(stream)))


def mlp_fwd(shape: Shape, x, w_fc1, b_fc1, w_fc2, y_partial, saved, workspace=None, stream=None) -> None:
    """mt_mlp_fwd: y_partial = GeLU(x W1^T + b1) W2^T."""
    _check("mt_mlp_fwd", lib().mt_mlp_fwd(ctypes.byref(shape), _ptr(x), _ptr(w_fc1), _ptr(b_fc1), _ptr(w_fc2),
                                          _ptr(y_partial), _ptr(saved), _nbytes(saved), _ptr(workspace),
                                          _nbytes(workspace), _stream(stream)))


def mlp_bwd(shape: Shape, x, w_fc1, w_fc2, saved, dy, dx_partial, dw_fc1, db_fc1, dw_fc2, workspace,
            stream=None) -> None:
    """mt_mlp_bwd: dx_partial and fp32 dW1, db1, dW2 of the MLP block."""
    _check("mt_mlp_bwd", lib().mt_mlp_bwd(ctypes.byref(shape), _ptr(x), _ptr(w_fc1), _ptr(w_fc2), _ptr(saved),
                                          _nbytes(saved), _ptr(dy), _ptr(dx_partial), _ptr(dw_fc1), _ptr(db_fc1),
                                          _ptr(dw_fc2), _ptr(workspace), _nbytes(workspace), _stream(stream)))


def mlp_bwd_noalloc(shape: Shape, x, w_fc1, w_fc2, saved, dy, dx_partial, dw_fc1, db_fc1, dw_fc2,
                    stream=None) -> None:
    """mt_mlp_bwd_noalloc: mt_mlp_bwd with its scratch in the library's static device
    array (no workspace argument; the call allocates nothing)."""
    _check("mt_mlp_bwd_noalloc", lib().mt_mlp_bwd_noalloc(ctypes.byref(shape), _ptr(x), _ptr(w_fc1), _ptr(w_fc2),
                                                          _ptr(saved), _nbytes(saved), _ptr(dy), _ptr(dx_partial),
                                                          _ptr(dw_fc1), _ptr(db_fc1), _ptr(dw_fc2),
                                                          _stream(stream)))


def attn_saved_bytes(shape: Shape) -> int:
    return lib().mt_attn_saved_bytes(ctypes.byref(shape))


def attn_workspace_bytes(shape: Shape) -> int:
    return lib().mt_attn_workspace_bytes(ctypes.byref(shape))


def attn_fwd(shape: Shape, u, w_qkv, b_qkv, w_o, o_partial, saved, workspace, stream=None) -> None:
    """mt_attn_fwd: o_partial = Attn(u W_qkv^T + b_qkv) W_o^T over the shard's heads."""
    _check("mt_attn_fwd", lib().mt_attn_fwd(ctypes.byref(shape), _ptr(u), _ptr(w_qkv), _ptr(b_qkv), _ptr(w_o),
                                            _ptr(o_partial), _ptr(saved), _nbytes(saved), _ptr(workspace),
                                            _nbytes(workspace), _stream(stream)))


def attn_bwd(shape: Shape, u, w_qkv, w_o, saved, d_o, du_partial, dw_qkv, db_qkv, dw_o, workspace,
             stream=None) -> None:
    """mt_attn_bwd: du_partial and fp32 dW_qkv, db_qkv, dW_o of the attention block."""
    _check("mt_attn_bwd", lib().mt_attn_bwd(ctypes.byref(shape), _ptr(u), _ptr(w_qkv), _ptr(w_o), _ptr(saved),
                                            _nbytes(saved), _ptr(d_o), _ptr(du_partial), _ptr(dw_qkv),
                                            _ptr(db_qkv), _ptr(dw_o), _ptr(workspace), _nbytes(workspace),
                                            _stream(stream)))


def sp_ln_fwd(shape: Shape, x, gamma, beta, y, mean, rstd, resid=None, bias=None, x2=None, stream=None) -> None:
    """mt_sp_ln_fwd over the rank's seq/tp share of the tokens: y = LN(x), or with resid,
    x2 = x + resid + bias (fp32) and y = LN(x2)."""
    _check("mt_sp_ln_fwd", lib().mt_sp_ln_fwd(ctypes.byref(shape), _ptr(x), _ptr(resid), _ptr(bias), _ptr(gamma),
                                              _ptr(beta), _ptr(x2), _ptr(y), _ptr(mean), _ptr(rstd),
                                              _stream(stream)))


def sp_add_fwd(shape: Shape, x2, y, bias, out, stream=None) -> None:
    """mt_sp_add_fwd: out = x2 + y + bias over the rank's rows."""
    _check("mt_sp_add_fwd", lib().mt_sp_add_fwd(ctypes.byref(shape), _ptr(x2), _ptr(y), _ptr(bias), _ptr(out),
                                                _stream(stream)))


def sp_ln_workspace_bytes(shape: Shape) -> int:
    return lib().mt_sp_ln_workspace_bytes(ctypes.byref(shape))


def sp_ln_bwd(shape: Shape, dy, xin, gamma, mean, rstd, dres, dx, dgamma, dbeta, workspace, *, xin_f32: bool,
              dres_f32: bool, dx_f32=None, dsum=None, dres_sum=None, stream=None) -> None:
    """mt_sp_ln_bwd: dx = dres + LN-backward(dy) over the rank's rows, with the rank's
    partial column sums dgamma, dbeta and optionally sum(dx) and sum(dres)."""
    _check("mt_sp_ln_bwd", lib().mt_sp_ln_bwd(ctypes.byref(shape), _ptr(dy), _ptr(xin), 1 if xin_f32 else 0,
                                              _ptr(gamma), _ptr(mean), _ptr(rstd), _ptr(dres), 1 if dres_f32 else 0,
                                              _ptr(dx), _ptr(dx_f32), _ptr(dgamma), _ptr(dbeta), _ptr(dsum),
                                              _ptr(dres_sum), _ptr(workspace), _nbytes(workspace),
                                              _stream(stream)))


def timing_enable(enable: bool = True, label_filter: Optional[str] = None) -> None:
    _check("mt_timing_enable", lib().mt_timing_enable(1 if enable else 0,
                                                      label_filter.encode() if label_filter else None))


def timing_reset() -> None:
    _check("mt_timing_reset", lib().mt_timing_reset())


def timing_records() -> List[Tuple[str, float, float, float]]:
    """(label, ms, algorithmic flops, algorithmic bytes) of every recorded launch."""
    out = []
    buf = ctypes.create_string_buffer(64)
    ms, fl, by = ctypes.c_float(), ctypes.c_double(), ctypes.c_double()
    for i in range(lib().mt_timing_count()):
        _check("mt_timing_get", lib().mt_timing_get(i, buf, 64, ctypes.byref(ms), ctypes.byref(fl), ctypes.byref(by)))
        out.append((buf.value.decode(), ms.value, fl.value, by.value))
    return out


def adamw_step(param, grad, exp_avg, exp_avg_sq, param_bf16=None, *, lr: float, beta1: float, beta2: float,
               eps: float, weight_decay: float, step: int, grad_scale: float = 1.0, stream=None) -> None:
    """mt_adamw_step: one fused AdamW step over flat fp32 tensors of equal size
    (param, exp_avg, exp_avg_sq updated in place; param_bf16 optional bf16 output)."""
    import torch
    n = param.numel() if not isinstance(param, int) else None
    if n is None:
        raise ValueError("param: a device tensor is required (its size is the step's length)")
    for name, t in (("param", param), ("grad", grad), ("exp_avg", exp_avg), ("exp_avg_sq", exp_avg_sq)):
        _expect(name, t, n, torch.float32)
    if param_bf16 is not None:
        _expect("param_bf16", param_bf16, n, torch.bfloat16)
    _check("mt_adamw_step", lib().mt_adamw_step(n, _ptr(param), _ptr(grad), _ptr(exp_avg), _ptr(exp_avg_sq),
                                                _ptr(param_bf16), lr, beta1, beta2, eps, weight_decay, grad_scale,
                                                int(step), _stream(stream)))
