"""CPU model of the bf16 path's rounding points (test-side analysis tool).

The layer is computed with the oracle's formulas in fp64, except that every tensor the
HIP path stores in bf16 between kernels is rounded to bf16 at the same point. With no
rounding enabled the model IS the oracle; with the rounding set of one of the HIP
path's bf16 modes (BF16 for MT_BF16, BF16_QK for MT_BF16_QK) it predicts that mode's
error against the oracle (the BF16_QK set reproduced the measured GPU errors of the
175B shard to three digits). Switching single rounding points on or off
shows which of them drive which error, and which tolerance readings a bf16 path can
meet at all.

    python tests/precision_model.py gpt175b_tp8
prints, per output tensor, the RMS error / RMS, max error / RMS and max error / max|T|
for the HIP path's rounding set and for variants.
"""
from __future__ import annotations

import math
import sys
from typing import Dict, Iterable, Tuple

import numpy as np

import seeded_inputs as si
from oracle.layer import gelu, gelu_grad, layernorm_bwd, layernorm_fwd

# Rounding points of the HIP path's MT_BF16_QK mode. The residual stream X2 and its
# gradient dX2 are fp32. U enters the QKV GEMM as U_hi + U_lo and Q, K enter the score
# products as hi + lo pairs, so neither is rounded there ("u_qkv", "qk_fwd" absent); the
# backward uses the single bf16 U, Q, K ("u", "qk") and V is bf16 throughout ("v").
BF16_QK = frozenset({"u", "qk", "v", "p", "ctx", "o", "v2", "a", "z", "y", "out",
                     "da", "dv2", "dx2_operand", "dctx", "ds", "dqkv", "du", "dx"})
# MT_BF16: U rounded before the QKV GEMM and Q, K rounded before the scores.
BF16 = BF16_QK | {"u_qkv", "qk_fwd"}


def _rb(a) -> np.ndarray:
    return si.bf16_round(np.asarray(a, np.float32)).astype(np.float64)


def layer(case: si.Case, rounded: Iterable[str]):
    """Forward + backward of shard case.layers[0] with bf16 rounding at `rounded`."""
    R = frozenset(rounded)
    r = lambda name, a: _rb(a) if name in R else a  # noqa: E731
    sh = case.shape
    B, s, d = sh.micro_batch, sh.seq, sh.head_dim
    p = {k: v.astype(np.float64) for k, v in case.layers[0].items()}
    x = case.x.astype(np.float64)
    u_exact, mu1, rs1 = layernorm_fwd(x, p["ln1_g"], p["ln1_b"])
    u = r("u", u_exact)
    qkv_exact = (u if "u_qkv" in R else u_exact) @ p["w_qkv"].T + p["b_qkv"]
    at = qkv_exact.shape[1] // (3 * d)
    cols = lambda w, k: slice(w * at * d + k * d, w * at * d + (k + 1) * d)  # noqa: E731
    qk_cols = slice(0, 2 * at * d)
    v_cols = slice(2 * at * d, 3 * at * d)
    qkv = qkv_exact.copy()                      # as used by the backward
    qkv[:, qk_cols] = r("qk", qkv_exact[:, qk_cols])
    qkv[:, v_cols] = r("v", qkv_exact[:, v_cols])
    qkv_s = qkv_exact.copy()                    # as used by the score product
    qkv_s[:, qk_cols] = r("qk_fwd", qkv_exact[:, qk_cols])
    ctx = np.zeros((B * s, at * d))
    P = np.zeros((B, at, s, s))
    vis = np.tril(np.ones((s, s), bool))
    for b in range(B):
        rows = slice(b * s, (b + 1) * s)
        for k in range(at):
            S = np.where(vis, qkv_s[rows, cols(0, k)] @ qkv_s[rows, cols(1, k)].T / math.sqrt(d), -np.inf)
            e = np.exp(S - S.max(1, keepdims=True))
            P[b, k] = r("p", e / e.sum(1, keepdims=True))
            ctx[rows, k * d:(k + 1) * d] = P[b, k] @ qkv[rows, cols(2, k)]
    ctx = r("ctx", ctx)
    x2 = x + r("o", ctx @ p["w_o"].T) + p["b_o"]
    v2, mu2, rs2 = layernorm_fwd(x2, p["ln2_g"], p["ln2_b"])
    v2 = r("v2", v2)
    a = r("a", v2 @ p["w_fc1"].T + p["b_fc1"])
    z = r("z", gelu(a))
    out = r("out", x2 + r("y", z @ p["w_fc2"].T) + p["b_fc2"])

    dout = case.dout.astype(np.float64)
    g: Dict[str, np.ndarray] = {"b_fc2": dout.sum(0), "w_fc2": dout.T @ z}
    da = r("da", (dout @ p["w_fc2"]) * gelu_grad(a))
    g["b_fc1"], g["w_fc1"] = da.sum(0), da.T @ v2
    dv2 = r("dv2", da @ p["w_fc1"])
    dxl, g["ln2_g"], g["ln2_b"] = layernorm_bwd(dv2, x2, p["ln2_g"], mu2, rs2)
    dx2 = dout + dxl
    dx2_op = r("dx2_operand", dx2)
    g["b_o"], g["w_o"] = dx2.sum(0), dx2_op.T @ ctx
    dctx = r("dctx", dx2_op @ p["w_o"])
    dqkv = np.zeros_like(qkv)
    for b in range(B):
        rows = slice(b * s, (b + 1) * s)
        for k in range(at):
            q, kk, v = (qkv[rows, cols(w, k)] for w in range(3))
            pp, dc = P[b, k], dctx[rows, k * d:(k + 1) * d]
            dp = dc @ v.T
            D = (dc * ctx[rows, k * d:(k + 1) * d]).sum(1, keepdims=True)  # rowsum(P dP) from ctx, as the HIP path
            ds = r("ds", pp * (dp - D))
            dqkv[rows, cols(2, k)] = pp.T @ dc
            dqkv[rows, cols(0, k)] = ds @ kk / math.sqrt(d)
            dqkv[rows, cols(1, k)] = ds.T @ q / math.sqrt(d)
    dqkv = r("dqkv", dqkv)
    g["b_qkv"], g["w_qkv"] = dqkv.sum(0), dqkv.T @ u
    du = r("du", dqkv @ p["w_qkv"])
    dxl, g["ln1_g"], g["ln1_b"] = layernorm_bwd(du, x, p["ln1_g"], mu1, rs1)
    dx = r("dx", dx2 + dxl)
    return out, dx, g


def metrics(res, ref) -> Dict[str, Tuple[float, float, float]]:
    """Per tensor: (RMS error / RMS, max error / RMS, max error / max |T|)."""
    out, dx, g = res
    rout, rdx, rg = ref
    pairs = [("out", out, rout), ("dx", dx, rdx)] + [(k, g[k], rg[k]) for k in sorted(rg)]
    m = {}
    for k, a, b in pairs:
        d = np.abs(a - b)
        rms = max(np.sqrt(np.mean(b * b)), 1e-300)
        m[k] = (float(np.sqrt(np.mean(d * d)) / rms), float(d.max() / rms), float(d.max() / max(np.abs(b).max(), 1e-300)))
    return m


def _print(tag, m):
    print(tag)
    for k, (a, b, c) in m.items():
        print(f"   {k:7s} rms-err/rms {a * 100:6.3f}%   max/rms {b * 100:6.2f}%   max/max {c * 100:6.3f}%")


if __name__ == "__main__":
    name = sys.argv[1] if len(sys.argv) > 1 else "gpt_h1024"
    case = si.workload_case(name)
    ref = layer(case, ())
    _print("MT_BF16 (U and Q, K rounded before their products)", metrics(layer(case, BF16), ref))
    _print("MT_BF16_QK (hi + lo U and Q, K in the logits)", metrics(layer(case, BF16_QK), ref))
    _print("only the QKV-GEMM operand U rounded", metrics(layer(case, {"u_qkv"}), ref))
