"""Rounding model of a bf16-storage layer path (test infrastructure).

TEST INFRASTRUCTURE ONLY: it sets the per-tensor error ceilings of the GPU parity tests
and is never imported by the product.

The layer is evaluated with the oracle's own formulas in float64, except that every
tensor the bf16 path stores in bf16 between its kernels is rounded to bf16 at that
point (float64 -> float32 -> bf16, each to nearest even). Which tensors those are is
the documented storage precision of the C ABI (include/mt.h): GEMM operands,
intermediates and the residual gradient dX2 in bf16; accumulation, LayerNorm / softmax /
GeLU math and the residual stream X2 in fp32 (not rounded here). The sequence-parallel
share takes dX2 in fp32 from its caller, so its model leaves out the "dx2" point. With
no rounding point enabled the model is exactly the oracle (pinned in
tests/test_rounding_model.py).

A rounding point is a name; ``BF16`` is the set of the default MT_BF16 mode and
``BF16_QK`` that of the MT_BF16_QK mode, which carries U into the Q and K columns of the
QKV product and Q, K into the logits as hi + lo bf16 pairs ("u_pair", "qk_pair": hi =
bf16(x), lo = bf16(x - hi), about 16 significant bits; the V columns take the bf16 U,
and the logits are Q_hi K_hi + Q_hi K_lo + Q_lo K_hi, without Q_lo K_lo).

Attention with head dim 64, 128 or 160 is fused on the bf16 path: the forward rounds the
unnormalised exponentials exp(S - max) to bf16 as the P V operand and divides by their
fp32 sum afterwards, and the backward recomputes P in fp32, rounds it to bf16 as the dV
operand and forms dS from the fp32 P. Other head dims store the normalised P in bf16 and
use it everywhere. The one-shard layer adds the FC2 product to the residual stream from
its fp32 accumulators (the partial is never stored), while a tensor-parallel group and
the sequence-parallel share store every partial in bf16 ("y").

The model is not bit-exact against any GPU run (fp32
accumulation order, the fused attention's rounding of the unnormalised probabilities
and fp32 element-wise math differ in the last bits); it predicts the size of the errors
a bf16 path with these storage points makes against the fp64 oracle.
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, List, Tuple

import numpy as np

from .layer import gelu, gelu_grad, layernorm_bwd, layernorm_fwd

# Storage points of the MT_BF16_QK mode (see the module docstring).
BF16_QK = frozenset({
    "u",            # LayerNorm-1 output as read by the backward (and the attention block input)
    "qk", "v",      # Q, K as read by the backward; V everywhere
    "p",            # probabilities as multiplied with V (and with dctx for dV)
    "ctx", "o",     # context, out-projection partial
    "v2", "a", "z", "y", "out",
    "da", "dv2", "dx2_operand", "dctx", "ds", "dqkv", "du", "dx",
    "dx2",          # its gradient as the LayerNorm-1 backward's residual input
    "ar",           # a reduce-scatter's output (sequence-parallel share), rounded once after the sum
    "u_pair",       # U as hi + lo into the Q and K columns of the projection (bf16 U into the V columns)
    "qk_pair",      # Q, K as hi + lo pairs in the logits
})
# MT_BF16: U rounded before the QKV product and Q, K before the logits.
BF16 = (BF16_QK - {"u_pair", "qk_pair"}) | {"u_qkv", "qk_fwd"}
MODES = {"bf16": BF16, "bf16qk": BF16_QK}


def pair(a) -> Tuple[np.ndarray, np.ndarray]:
    """hi + lo bf16 pair of a value: hi = bf16(a), lo = bf16(a - hi)."""
    hi = bf16(a)
    return hi, bf16(np.asarray(a, dtype=np.float64) - hi)


def bf16(a) -> np.ndarray:
    """Round to bfloat16 through float32 (nearest even at both steps), as float64."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32)
    u = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return u.view(np.float32).astype(np.float64)


class _R:
    def __init__(self, rounded: Iterable[str]):
        self.names = frozenset(rounded)

    def __call__(self, name: str, a):
        return bf16(a) if name in self.names else np.asarray(a, dtype=np.float64)

    def __contains__(self, name: str) -> bool:
        return name in self.names


def _f64(p: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
    return {k: np.asarray(v, dtype=np.float64) for k, v in p.items()}


# --------------------------------------------------------------------------- blocks
def fused_attention(d: int, r: _R) -> bool:
    """Whether the bf16 path runs this head dim's attention fused (see the module docstring)."""
    return "p" in r and d in (64, 128, 160)


def attn_fwd(u: np.ndarray, u_exact: np.ndarray, p, B: int, s: int, d: int, r: _R):
    """Attention block of one shard: QKV projection, causal attention, out-projection
    partial (rounded "o"). u is the stored LayerNorm output, u_exact its unrounded value
    (the MT_BF16_QK projection sees it to ~16 bits)."""
    fused = fused_attention(d, r)
    at = p["w_qkv"].shape[0] // (3 * d)
    cols = lambda w, k: slice(w * at * d + k * d, w * at * d + (k + 1) * d)  # noqa: E731
    qk, vv = slice(0, 2 * at * d), slice(2 * at * d, 3 * at * d)
    if "u_qkv" in r:    # bf16 U into every column
        u_qk = u_v = u
    elif "u_pair" in r:  # hi + lo U into the Q, K columns, bf16 U into the V columns
        u_qk, u_v = sum(pair(u_exact)), u
    else:
        u_qk = u_v = u_exact
    qkv_exact = np.empty((u.shape[0], 3 * at * d))
    qkv_exact[:, qk] = u_qk @ p["w_qkv"][qk].T + p["b_qkv"][qk]
    qkv_exact[:, vv] = u_v @ p["w_qkv"][vv].T + p["b_qkv"][vv]
    qkv = qkv_exact.copy()              # as read by the backward
    qkv[:, qk] = r("qk", qkv_exact[:, qk])
    qkv[:, vv] = r("v", qkv_exact[:, vv])
    if "qk_pair" in r:                   # as read by the logits: hi and lo parts
        q_hi, q_lo = pair(qkv_exact[:, qk])
    else:
        q_hi, q_lo = r("qk_fwd", qkv_exact[:, qk]), None
    ctx = np.zeros((B * s, at * d))
    P = np.zeros((B, at, s, s))    # as the backward multiplies it with dctx (dV)
    Pe = np.zeros((B, at, s, s))   # unrounded, as the backward forms dS from it
    vis = np.tril(np.ones((s, s), bool))
    for b in range(B):
        rows = slice(b * s, (b + 1) * s)
        for k in range(at):
            qc, kc = slice(k * d, (k + 1) * d), slice(at * d + k * d, at * d + (k + 1) * d)
            L = q_hi[rows, qc] @ q_hi[rows, kc].T
            if q_lo is not None:
                L = L + q_hi[rows, qc] @ q_lo[rows, kc].T + q_lo[rows, qc] @ q_hi[rows, kc].T
            S = np.where(vis, L / math.sqrt(d), -np.inf)
            e = np.exp(S - S.max(1, keepdims=True))
            tot = e.sum(1, keepdims=True)
            Pe[b, k] = e / tot
            P[b, k] = r("p", Pe[b, k])
            pv = r("p", e) / tot if fused else P[b, k]  # the P V operand
            ctx[rows, k * d:(k + 1) * d] = pv @ qkv[rows, cols(2, k)]
    ctx = r("ctx", ctx)
    o = r("o", ctx @ p["w_o"].T)
    return o, dict(u=u, qkv=qkv, P=P, Pe=Pe if fused else P, ctx=ctx, at=at, d=d, B=B, s=s, p=p)


def attn_bwd(do_op: np.ndarray, c, r: _R):
    """Backward of attn_fwd given the stored output gradient: du partial (rounded
    "du") and the shard's w_qkv, b_qkv, w_o gradients."""
    p, at, d, B, s = c["p"], c["at"], c["d"], c["B"], c["s"]
    qkv, ctx, P, Pe = c["qkv"], c["ctx"], c["P"], c["Pe"]
    cols = lambda w, k: slice(w * at * d + k * d, w * at * d + (k + 1) * d)  # noqa: E731
    g = {"w_o": do_op.T @ ctx}
    dctx = r("dctx", do_op @ p["w_o"])
    dqkv = np.zeros_like(qkv)
    for b in range(B):
        rows = slice(b * s, (b + 1) * s)
        for k in range(at):
            q, kk, v = (qkv[rows, cols(w, k)] for w in range(3))
            pp, dc = P[b, k], dctx[rows, k * d:(k + 1) * d]
            dp = dc @ v.T
            D = (dc * ctx[rows, k * d:(k + 1) * d]).sum(1, keepdims=True)  # rowsum(P dP) from the stored ctx
            ds = r("ds", Pe[b, k] * (dp - D))
            dqkv[rows, cols(2, k)] = pp.T @ dc
            dqkv[rows, cols(0, k)] = ds @ kk / math.sqrt(d)
            dqkv[rows, cols(1, k)] = ds.T @ q / math.sqrt(d)
    dqkv = r("dqkv", dqkv)
    g["b_qkv"], g["w_qkv"] = dqkv.sum(0), dqkv.T @ c["u"]
    return r("du", dqkv @ p["w_qkv"]), g


def mlp_fwd(v2: np.ndarray, p, r: _R):
    """MLP block of one shard: y partial (rounded "y") = GeLU(v2 W1^T + b1) W2^T."""
    a = r("a", v2 @ p["w_fc1"].T + p["b_fc1"])
    z = r("z", gelu(a))
    return r("y", z @ p["w_fc2"].T), dict(v2=v2, a=a, z=z, p=p)


def mlp_bwd(dy: np.ndarray, c, r: _R):
    """Backward of mlp_fwd: dv2 partial (rounded "dv2") and w_fc1, b_fc1, w_fc2 grads."""
    p = c["p"]
    g = {"w_fc2": dy.T @ c["z"]}
    da = r("da", (dy @ p["w_fc2"]) * gelu_grad(c["a"]))
    g["b_fc1"], g["w_fc1"] = da.sum(0), da.T @ c["v2"]
    return r("dv2", da @ p["w_fc1"]), g


# --------------------------------------------------------------------------- layer
def layer(x, dout, ranks: List[Dict[str, np.ndarray]], B: int, s: int, d: int, rounded: Iterable[str],
          ar_round: bool = False):
    """Forward + backward of the tensor-parallel layer over `ranks` (per-rank shard
    weights; one dict = the one-GPU shard with the all-reduce as the identity). The
    all-reduce sums the ranks' stored (rounded) partials; with ar_round its output is
    rounded once more ("ar": the sequence-parallel reduce-scatter's bf16 output).

    Returns out, dx, the per-rank gradients (shard tensors and the replicated ones) and
    the per-row contributions of the replicated gradients (row r of rows[k] summed over
    rows gives gradient k), from which a subset of rows' partial sums can be formed.
    """
    r = _R(rounded)
    ar = lambda parts: r("ar", sum(parts)) if (ar_round and "ar" in r) else sum(parts)  # noqa: E731
    ps = [_f64(p) for p in ranks]
    p0 = ps[0]
    x = np.asarray(x, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    u_exact, mu1, rs1 = layernorm_fwd(x, p0["ln1_g"], p0["ln1_b"])
    u = r("u", u_exact)
    fa = [attn_fwd(u, u_exact, p, B, s, d, r) for p in ps]
    x2 = x + ar([o for o, _ in fa]) + p0["b_o"]
    v2e, mu2, rs2 = layernorm_fwd(x2, p0["ln2_g"], p0["ln2_b"])
    v2 = r("v2", v2e)
    # one shard with the all-reduce as the identity: the FC2 product goes to the residual
    # add unrounded; otherwise each rank's partial is stored in bf16
    rm = _R(r.names - {"y"}) if len(ps) == 1 and not ar_round else r
    fm = [mlp_fwd(v2, p, rm) for p in ps]
    out = r("out", x2 + ar([y for y, _ in fm]) + p0["b_fc2"])

    grads = [dict() for _ in ps]
    bm = [mlp_bwd(dout, c, r) for _, c in fm]
    for g, (_, gm) in zip(grads, bm):
        g.update(gm)
    dv2 = ar([dv for dv, _ in bm])
    xh2 = (x2 - mu2[:, None]) * rs2[:, None]
    dxl, _, _ = layernorm_bwd(dv2, x2, p0["ln2_g"], mu2, rs2)
    dx2 = dout + dxl
    dx2_op = r("dx2_operand", dx2)
    ba = [attn_bwd(dx2_op, c, r) for _, c in fa]
    for g, (_, gb) in zip(grads, ba):
        g.update(gb)
    du = ar([du_ for du_, _ in ba])
    xh1 = (x - mu1[:, None]) * rs1[:, None]
    dxl1, _, _ = layernorm_bwd(du, x, p0["ln1_g"], mu1, rs1)
    dx = r("dx", r("dx2", dx2) + dxl1)
    # db_o: summed from the unrounded dX2 where the LayerNorm-2 backward carries the column
    # sums in its row pass (h <= 16384), else from the stored dX2
    db_o_rows = dx2 if x.shape[1] <= 16384 else r("dx2", dx2)
    rows = {"ln1_g": du * xh1, "ln1_b": du, "b_o": db_o_rows, "ln2_g": dv2 * xh2, "ln2_b": dv2, "b_fc2": dout}
    for g in grads:
        g.update({k: v.sum(0) for k, v in rows.items()})
    return out, dx, grads, rows


def stage(x, dout, layers: List[Dict[str, np.ndarray]], B: int, s: int, d: int, rounded: Iterable[str]):
    """Consecutive one-shard layers: forward l0 .. lL-1, backward lL-1 .. l0, each
    layer's stored output feeding the next layer and each stored dx the previous one
    (both rounded to bf16 by the "out" / "dx" points). Returns out, dx and the per-layer
    gradients."""
    r = _R(rounded)
    acts = [np.asarray(x, dtype=np.float64)]
    for p in layers:  # forward only, to get each layer's input
        out, _, _, _ = _layer_fwd_only(acts[-1], p, B, s, d, r)
        acts.append(out)
    g = np.asarray(dout, dtype=np.float64)
    grads: List[Dict[str, np.ndarray]] = [None] * len(layers)  # type: ignore[list-item]
    for l in reversed(range(len(layers))):
        _, g, gl, _ = layer(acts[l], g, [layers[l]], B, s, d, r.names)
        grads[l] = gl[0]
    return acts[-1], g, grads


def _layer_fwd_only(x, p, B, s, d, r: _R):
    p = _f64(p)
    u_exact, _, _ = layernorm_fwd(x, p["ln1_g"], p["ln1_b"])
    o, _ = attn_fwd(r("u", u_exact), u_exact, p, B, s, d, r)
    x2 = x + o + p["b_o"]
    v2e, _, _ = layernorm_fwd(x2, p["ln2_g"], p["ln2_b"])
    y, _ = mlp_fwd(r("v2", v2e), p, _R(r.names - {"y"}))  # one shard: the FC2 product unrounded
    return r("out", x2 + y + p["b_fc2"]), None, None, None


# --------------------------------------------------------------------------- error ratios
def ratios(got, ref) -> Tuple[float, float, float]:
    """(max|err| / RMS(ref), RMS(err) / RMS(ref), max|err| / max|ref|) of one tensor."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    e = np.abs(got - ref)
    rms = max(float(np.sqrt(np.mean(ref * ref))), 1e-300)
    return float(e.max()) / rms, float(np.sqrt(np.mean(e * e))) / rms, float(e.max()) / max(float(np.abs(ref).max()),
                                                                                              1e-300)
