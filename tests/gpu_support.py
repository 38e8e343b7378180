"""Helpers for the GPU parity tests: seeded inputs to device tensors, one call of the
HIP path through the C ABI, and the per-tensor comparison against the fp64 oracle.

Bar per output tensor T (Out, dX and every parameter gradient):
  * fp32 path: max |T_gpu - T_oracle| <= 1e-4 * RMS(T_oracle) (the literal bar);
  * bf16 path: RMS(T_gpu - T_oracle) <= 2e-2 * RMS(T_oracle) and
               max |T_gpu - T_oracle| <= c_T * RMS(T_oracle),
    c_T = 2e-2 (the literal bar) unless the bf16 rounding model predicts a larger
    max|err| / RMS for T on the same inputs, then 1.5 x that prediction (2 x for
    one-dimensional tensors; scaled by the GPU's RMS error over the model's where that
    is larger; tests/ceilings.py). Every
    comparison prints all three ratios and, with MT_PARITY_LOG set, appends them to that
    file as a JSON line.
"""
from __future__ import annotations

import json
import os
import sys
from typing import Dict, List, Tuple

import numpy as np

import oracle
import seeded_inputs as si

TOL = {"bf16": 2e-2, "fp32": 1e-4}


def torch_mod():
    import torch
    return torch


def mt_mod():
    import tensor_layer_gemms_amd as mt
    return mt


def to_dev(a: np.ndarray, dtype: str):
    torch = torch_mod()
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def to_np(t) -> np.ndarray:
    return t.detach().to(torch_mod().float32).cpu().numpy().astype(np.float64)


def mt_shape(shape: si.LayerShape):
    dtype = "bf16qk" if shape.qk_pairs else shape.dtype
    return mt_mod().make_shape(shape.h, shape.heads, shape.seq, shape.micro_batch, shape.tp, shape.shard, dtype)


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def run_layer_gpu(shape: si.LayerShape, x: np.ndarray, dout: np.ndarray, params: Dict[str, np.ndarray],
                  repeat: int = 1):
    """One mt_layer_fwd + mt_layer_bwd; returns (out, dx, grads) as float64 arrays."""
    torch, mt = torch_mod(), mt_mod()
    sh = mt_shape(shape)
    saved = torch.empty(mt.layer_saved_bytes(sh), dtype=torch.uint8, device="cuda")
    ws = torch.empty(mt.layer_workspace_bytes(sh), dtype=torch.uint8, device="cuda")
    w = {k: to_dev(v, shape.dtype) for k, v in params.items()}
    xd, dd = to_dev(x, shape.dtype), to_dev(dout, shape.dtype)
    out, dx = torch.empty_like(xd), torch.empty_like(xd)
    grads = {k: torch.empty(v.shape, dtype=torch.float32, device="cuda") for k, v in params.items()}
    mt.check_layer_tensors(sh, w, grads, x=xd, out=out, dout=dd, dx=dx)
    results = []
    for _ in range(repeat):
        mt.layer_fwd(sh, w, xd, out, saved, ws)
        mt.layer_bwd(sh, w, xd, saved, dd, dx, grads, ws)
        torch.cuda.synchronize()
        results.append((to_np(out), to_np(dx), {k: to_np(g) for k, g in grads.items()}))
    return results[0] if repeat == 1 else results


def run_stage_gpu(shape: si.LayerShape, x: np.ndarray, dout: np.ndarray, layers: List[Dict[str, np.ndarray]]):
    """Consecutive layers as one stage: forward l0..lL-1, then backward lL-1..l0."""
    torch, mt = torch_mod(), mt_mod()
    sh = mt_shape(shape)
    L = len(layers)
    saved = [torch.empty(mt.layer_saved_bytes(sh), dtype=torch.uint8, device="cuda") for _ in range(L)]
    ws = torch.empty(mt.layer_workspace_bytes(sh), dtype=torch.uint8, device="cuda")
    ws_ = [{k: to_dev(v, shape.dtype) for k, v in p.items()} for p in layers]
    acts = [to_dev(x, shape.dtype)] + [torch.empty_like(to_dev(x, shape.dtype)) for _ in range(L)]
    grads = [{k: torch.empty(v.shape, dtype=torch.float32, device="cuda") for k, v in p.items()} for p in layers]
    for l in range(L):
        mt.check_layer_tensors(sh, ws_[l], grads[l], x=acts[l], out=acts[l + 1])
        mt.layer_fwd(sh, ws_[l], acts[l], acts[l + 1], saved[l], ws)
    g = to_dev(dout, shape.dtype)
    for l in reversed(range(L)):
        dx = torch.empty_like(g)
        mt.layer_bwd(sh, ws_[l], acts[l], saved[l], g, dx, grads[l], ws)
        g = dx
    torch.cuda.synchronize()
    return to_np(acts[L]), to_np(g), [{k: to_np(v) for k, v in gr.items()} for gr in grads]


def run_mlp_gpu(shape: si.LayerShape, x: np.ndarray, dy: np.ndarray, p: Dict[str, np.ndarray]):
    """mt_mlp_fwd + mt_mlp_bwd of one shard; returns (y_partial, dx_partial, grads)."""
    torch, mt = torch_mod(), mt_mod()
    sh = mt_shape(shape)
    dt = shape.dtype
    xd, dyd = to_dev(x, dt), to_dev(dy, dt)
    w1, b1, w2 = to_dev(p["w_fc1"], dt), to_dev(p["b_fc1"], dt), to_dev(p["w_fc2"], dt)
    saved = torch.empty(mt.mlp_saved_bytes(sh), dtype=torch.uint8, device="cuda")
    ws = torch.empty(mt.mlp_workspace_bytes(sh), dtype=torch.uint8, device="cuda")
    y, dx = torch.empty_like(xd), torch.empty_like(xd)
    dw1 = torch.empty(p["w_fc1"].shape, dtype=torch.float32, device="cuda")
    db1 = torch.empty(p["b_fc1"].shape, dtype=torch.float32, device="cuda")
    dw2 = torch.empty(p["w_fc2"].shape, dtype=torch.float32, device="cuda")
    ft = 4 * shape.h // shape.tp
    assert w1.numel() == ft * shape.h and w2.numel() == ft * shape.h and b1.numel() == ft
    assert xd.numel() == shape.tokens * shape.h and dyd.numel() == xd.numel()
    mt.mlp_fwd(sh, xd, w1, b1, w2, y, saved, ws)
    mt.mlp_bwd(sh, xd, w1, w2, saved, dyd, dx, dw1, db1, dw2, ws)
    torch.cuda.synchronize()
    return to_np(y), to_np(dx), dict(w_fc1=to_np(dw1), b_fc1=to_np(db1), w_fc2=to_np(dw2))


def rel_rms(gpu: np.ndarray, ref: np.ndarray) -> float:
    """RMS(gpu - ref) / RMS(ref)."""
    return float(np.sqrt(np.mean((gpu - ref) ** 2)) / max(np.sqrt(np.mean(ref * ref)), 1e-30))


def compare(name: str, gpu: np.ndarray, ref: np.ndarray, tol: float, normwise: bool = False,
            pred=None) -> Tuple[bool, float, float]:
    """normwise=False (fp32 path): max|err| <= tol * RMS(ref). normwise=True (bf16 path):
    RMS(err) <= tol * RMS(ref) and max|err| <= ceiling(pred) * RMS(ref), pred the rounding
    model's (max|err| / RMS, RMS(err) / RMS) for the tensor; the ceiling is tol itself
    when there is no prediction or it is small (tests/ceilings.py)."""
    from ceilings import ceiling
    diff = np.abs(gpu - ref)
    err = float(np.max(diff)) if ref.size else 0.0
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    finite = bool(np.all(np.isfinite(gpu)))
    if normwise:
        rms_err = float(np.sqrt(np.mean(diff * diff))) if ref.size else 0.0
        amax = float(np.max(np.abs(ref))) if ref.size else 0.0
        cap = ceiling(pred, tol, rms_err / max(rms, 1e-300), one_d=np.ndim(gpu) == 1)
        ok = finite and rms_err <= tol * rms and err <= cap * rms
        extra = (f"  rms-err/rms {rms_err / max(rms, 1e-30):.2e}  max/max {err / max(amax, 1e-30):.2e}"
                 f"  ceiling {cap:.2e}" + (f" (model {pred[0]:.2e} / {pred[1]:.2e})" if pred is not None else ""))
    else:
        cap = tol
        ok = finite and err <= tol * rms
        extra = ""
    log(f"  {name:10s} max|err| {err:.3e}  rms {rms:.3e}  max/rms {err / max(rms, 1e-30):.2e}{extra}  "
        f"{'ok' if ok else 'FAIL'}")
    record(name, gpu, ref, ok, cap, list(pred) if pred is not None else None)
    return ok, err, rms


def record(name: str, gpu: np.ndarray, ref: np.ndarray, ok: bool, cap: float = None, pred=None) -> None:
    """With MT_PARITY_LOG set, append one JSON line per compared tensor to that file:
    the test, the tensor, its three error ratios (max|err| / RMS, RMS(err) / RMS,
    max|err| / max|T|), the max|err| / RMS ceiling applied and the model's prediction."""
    path = os.environ.get("MT_PARITY_LOG")
    if not path or not ref.size:
        return
    d = np.abs(gpu - ref)
    rms = max(float(np.sqrt(np.mean(ref * ref))), 1e-300)
    rec = {"test": os.environ.get("PYTEST_CURRENT_TEST", os.environ.get("MT_PARITY_CASE", "")).split(" (")[0],
           "tensor": name, "max_rms": float(d.max()) / rms, "rms_rel": float(np.sqrt(np.mean(d * d))) / rms,
           "max_max": float(d.max()) / max(float(np.abs(ref).max()), 1e-300), "ok": bool(ok),
           "ceiling": cap, "model": pred}
    with open(path, "a") as f:
        f.write(json.dumps(rec) + "\n")


def check_all(gpu_out, gpu_dx, gpu_grads, ref_out, ref_dx, ref_grads, tol: float, keys=None,
              preds: Dict[str, Tuple[float, float]] = None, prefix: str = "") -> List[str]:
    """Every tensor: the literal bar on the fp32 path; on the bf16 path the normwise bar
    and the per-tensor max ceiling from `preds` (tensor name -> the model's (max|err| /
    RMS, RMS(err) / RMS); names of the layer: out, dx and the parameter names, each
    after `prefix`)."""
    bad = []
    normwise = tol > TOL["fp32"]
    preds = preds or {}
    names = [("out", gpu_out, ref_out), ("dx", gpu_dx, ref_dx)]
    names += [(k, gpu_grads[k], ref_grads[k]) for k in (keys or sorted(ref_grads))]
    for k, g, r in names:
        name = prefix + k
        if not compare(name, g, r, tol, normwise, preds.get(name))[0]:
            bad.append(name)
    return bad


def oracle_layer(shape: si.LayerShape, x, dout, params):
    out, c = oracle.layer_fwd(x, [params], shape.micro_batch, shape.seq, shape.head_dim)
    dx, g = oracle.layer_bwd(dout, c, [params])
    return out, dx, g[0]
