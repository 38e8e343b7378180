"""Plain fp64 definition of a tensor-parallel GPT layer shard, forward and backward.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the product.

Sources and readings
--------------------
* Tensor-parallel block Y = f(X A) B: A split by columns, B split by rows, each rank
  computes f(X A_i) B_i and an all-reduce sums the partials; attention heads are split
  across ranks -- "Megatron-LM" concept report (compassingai.com), section 4.1.
* Communication (hence the summed partials) happens in the forward AND the backward
  pass, each message O(B*S*H) -- same report, section 4.2. In the backward the
  input-gradient of a column-parallel GEMM is the partial that gets summed.
* The QKV projection is split into per-rank chunks -- "In-Depth Analysis of
  Distributed Training Frameworks for Large Models ... Megatron-LM" (oreateai.com),
  section 2.1. LayerNorm and GeLU are the element-wise operations that get fused --
  same blog, section 2.2.
* Readings where the pages are silent (each restated where it is used):
  pre-LN GPT layer (x + Attn(LN1 x), then x2 + MLP(LN2 x2)); LayerNorm with biased
  variance and eps = 1e-5; exact GeLU x*Phi(x) with the erf form; softmax scale
  1/sqrt(d); causal mask keeps key j iff j <= query q; no dropout; biases on QKV,
  out-projection, FC1 and FC2 with the row-parallel biases (b_o, b_fc2) added once,
  after the all-reduce point.

Tensor-parallel modes
---------------------
Every function takes ``shards``: a list of per-rank weight dicts (keys as in
seeded_inputs.PARAM_NAMES). The all-reduce point sums over that list. With a single
dict this is the one-GPU shard with the all-reduce replaced by the identity (exactly
what one rank computes before communicating); with all t dicts of a split it is the
true tensor-parallel layer, which equals the unsharded layer.
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence, Tuple

import numpy as np
from scipy.special import erf

EPS = 1e-5  # LayerNorm epsilon (silent on the pages; common default)

Params = Dict[str, np.ndarray]


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------- LayerNorm
def layernorm_fwd(x, gamma, beta, eps: float = EPS) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Row-wise LayerNorm (LayerNorm is one of the fused element-wise ops of the
    "In-Depth Analysis ... Megatron-LM" blog, section 2.2).

    mu = mean_c x; var = mean_c (x - mu)^2 (biased); rstd = 1/sqrt(var + eps);
    y = (x - mu) * rstd * gamma + beta. Returns y, mu [rows], rstd [rows].
    """
    x = _f64(x)
    mu = x.mean(axis=1)
    xc = x - mu[:, None]
    var = (xc * xc).mean(axis=1)
    rstd = 1.0 / np.sqrt(var + eps)
    y = xc * rstd[:, None] * _f64(gamma)[None, :] + _f64(beta)[None, :]
    return y, mu, rstd


def layernorm_bwd(dy, x, gamma, mu, rstd) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradient of layernorm_fwd.

    With xhat = (x - mu) * rstd and g = dy * gamma:
      dx = rstd * (g - mean_c g - xhat * mean_c(g * xhat)),
      dgamma = sum_rows dy * xhat,  dbeta = sum_rows dy.
    """
    dy, x = _f64(dy), _f64(x)
    xhat = (x - _f64(mu)[:, None]) * _f64(rstd)[:, None]
    g = dy * _f64(gamma)[None, :]
    dx = _f64(rstd)[:, None] * (g - g.mean(axis=1, keepdims=True)
                                - xhat * (g * xhat).mean(axis=1, keepdims=True))
    return dx, (dy * xhat).sum(axis=0), dy.sum(axis=0)


# --------------------------------------------------------------------------- GeLU
_SQRT2 = math.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


def gelu(a) -> np.ndarray:
    """Exact GeLU, the f of f(X A) B ("Megatron-LM" concept report, section 4.1):
    GeLU(a) = a * Phi(a) = a/2 * (1 + erf(a / sqrt 2)). The erf form is the definition;
    no tanh approximation."""
    a = _f64(a)
    return 0.5 * a * (1.0 + erf(a / _SQRT2))


def gelu_grad(a) -> np.ndarray:
    """d GeLU / da = Phi(a) + a * phi(a), phi the standard normal density."""
    a = _f64(a)
    return 0.5 * (1.0 + erf(a / _SQRT2)) + a * _INV_SQRT_2PI * np.exp(-0.5 * a * a)


# --------------------------------------------------------------------------- attention
def _head_cols(heads: int, d: int, which: int, k: int) -> slice:
    """Columns of head k's Q (which=0), K (1) or V (2) in a shard's QKV activation.

    Layout reading: the shard's QKV columns are [Q heads | K heads | V heads], each block
    a_t*d wide with head k at columns k*d ... k*d+d-1 (the per-rank QKV chunk of the
    "In-Depth Analysis ... Megatron-LM" blog, section 2.1; heads per rank from the
    "Megatron-LM" concept report, section 4.1)."""
    base = which * heads * d + k * d
    return slice(base, base + d)


def attention_fwd(qkv, micro_batch: int, seq: int, heads: int, d: int) -> Tuple[np.ndarray, np.ndarray]:
    """Causal softmax attention over one shard's heads.

    For each sequence b and head k: S = Q K^T / sqrt(d); S[q, j] = -inf for j > q
    (causal reading: key j is visible to query q iff j <= q); P = softmax over j
    (subtract the row max, exponentiate, normalise); C = P V. The heads' C are
    concatenated in columns. Returns ctx [B*s, heads*d] and P [B, heads, s, s].
    """
    qkv = _f64(qkv)
    ctx = np.zeros((micro_batch * seq, heads * d))
    probs = np.zeros((micro_batch, heads, seq, seq))
    visible = np.tril(np.ones((seq, seq), dtype=bool))
    scale = 1.0 / math.sqrt(d)
    for b in range(micro_batch):
        rows = slice(b * seq, (b + 1) * seq)
        for k in range(heads):
            q = qkv[rows, _head_cols(heads, d, 0, k)]
            kt = qkv[rows, _head_cols(heads, d, 1, k)]
            v = qkv[rows, _head_cols(heads, d, 2, k)]
            s = (q @ kt.T) * scale
            s = np.where(visible, s, -np.inf)
            e = np.exp(s - s.max(axis=1, keepdims=True))
            p = e / e.sum(axis=1, keepdims=True)
            probs[b, k] = p
            ctx[rows, k * d:(k + 1) * d] = p @ v
    return ctx, probs


def attention_bwd(dctx, qkv, probs, micro_batch: int, seq: int, heads: int, d: int) -> np.ndarray:
    """Gradient of attention_fwd with respect to the QKV activation.

    Per (b, k): dV = P^T dC; dP = dC V^T; dS = P * (dP - rowsum(P * dP));
    dQ = dS K / sqrt(d); dK = dS^T Q / sqrt(d). (Masked entries have P = 0, so dS = 0.)
    """
    dctx, qkv, probs = _f64(dctx), _f64(qkv), _f64(probs)
    dqkv = np.zeros_like(qkv)
    scale = 1.0 / math.sqrt(d)
    for b in range(micro_batch):
        rows = slice(b * seq, (b + 1) * seq)
        for k in range(heads):
            cq, ck, cv = (_head_cols(heads, d, w, k) for w in range(3))
            q, kt, v = qkv[rows, cq], qkv[rows, ck], qkv[rows, cv]
            p = probs[b, k]
            dc = dctx[rows, k * d:(k + 1) * d]
            dp = dc @ v.T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dqkv[rows, cv] = p.T @ dc
            dqkv[rows, cq] = (ds @ kt) * scale
            dqkv[rows, ck] = (ds.T @ q) * scale
    return dqkv


# --------------------------------------------------------------------------- MLP block
def mlp_fwd(x, shards: Sequence[Params]) -> Tuple[np.ndarray, dict]:
    """The pages' tensor-parallel MLP block ("Megatron-LM" concept report, section 4.1):
    rank i computes Y_i = GeLU(X W1_i^T + b1_i) W2_i^T (W1_i: the rank's output rows of
    FC1, W2_i: its input columns of FC2); the all-reduce point returns sum_i Y_i.
    No LayerNorm, no b_fc2 and no residual here: this is the bare f(X A_i) B_i partial.
    """
    x = _f64(x)
    cache = dict(x=x, a=[], z=[])
    y = np.zeros((x.shape[0], _f64(shards[0]["w_fc2"]).shape[0]))
    for p in shards:
        a = x @ _f64(p["w_fc1"]).T + _f64(p["b_fc1"])[None, :]
        z = gelu(a)
        y += z @ _f64(p["w_fc2"]).T
        cache["a"].append(a)
        cache["z"].append(z)
    return y, cache


def mlp_bwd(dy, cache: dict, shards: Sequence[Params]) -> Tuple[np.ndarray, List[Params]]:
    """Backward of mlp_fwd. Per rank: dW2_i = dY^T Z_i; dA_i = (dY W2_i) * GeLU'(A_i);
    db1_i = sum_rows dA_i; dW1_i = dA_i^T X; dX_i = dA_i W1_i is the backward partial
    whose sum over ranks (the backward all-reduce of the concept report, section 4.2)
    is returned as dX."""
    dy = _f64(dy)
    dx = np.zeros_like(cache["x"])
    grads = []
    for p, a, z in zip(shards, cache["a"], cache["z"]):
        da = (dy @ _f64(p["w_fc2"])) * gelu_grad(a)
        grads.append(dict(w_fc2=dy.T @ z, b_fc1=da.sum(axis=0), w_fc1=da.T @ cache["x"]))
        dx += da @ _f64(p["w_fc1"])
    return dx, grads


# --------------------------------------------------------------------------- layer
def layer_fwd(x, shards: Sequence[Params], micro_batch: int, seq: int, head_dim: int
              ) -> Tuple[np.ndarray, dict]:
    """Pre-LN GPT layer with tensor-parallel attention and MLP blocks.

      U = LN1(X);  per rank: QKV_i = U W_qkv_i^T + b_qkv_i, ctx_i = Attn(QKV_i),
      O_i = ctx_i W_o_i^T (row-parallel partial);  X2 = X + AR(O_i) + b_o;
      V2 = LN2(X2);  per rank: A_i = V2 W1_i^T + b1_i, Z_i = GeLU(A_i), Y_i = Z_i W2_i^T;
      Out = X2 + AR(Y_i) + b_fc2.
    AR sums over ``shards``. Replicated parameters (LayerNorm, b_o, b_fc2) come from
    shards[0]; all ranks hold the same copies.
    """
    x = _f64(x)
    p0 = shards[0]
    d = head_dim
    u, mu1, rstd1 = layernorm_fwd(x, p0["ln1_g"], p0["ln1_b"])
    c = dict(x=x, u=u, mu1=mu1, rstd1=rstd1, qkv=[], probs=[], ctx=[], a=[], z=[])
    o_sum = np.zeros_like(x)
    for p in shards:
        qkv = u @ _f64(p["w_qkv"]).T + _f64(p["b_qkv"])[None, :]
        heads = qkv.shape[1] // (3 * d)
        ctx, probs = attention_fwd(qkv, micro_batch, seq, heads, d)
        o_sum += ctx @ _f64(p["w_o"]).T
        c["qkv"].append(qkv)
        c["probs"].append(probs)
        c["ctx"].append(ctx)
    x2 = x + o_sum + _f64(p0["b_o"])[None, :]
    v2, mu2, rstd2 = layernorm_fwd(x2, p0["ln2_g"], p0["ln2_b"])
    y_sum = np.zeros_like(x)
    for p in shards:
        a = v2 @ _f64(p["w_fc1"]).T + _f64(p["b_fc1"])[None, :]
        z = gelu(a)
        y_sum += z @ _f64(p["w_fc2"]).T
        c["a"].append(a)
        c["z"].append(z)
    out = x2 + y_sum + _f64(p0["b_fc2"])[None, :]
    c.update(x2=x2, v2=v2, mu2=mu2, rstd2=rstd2, micro_batch=micro_batch, seq=seq, head_dim=d)
    return out, c


def layer_bwd(dout, c: dict, shards: Sequence[Params]) -> Tuple[np.ndarray, List[Params]]:
    """Backward of layer_fwd given dOut. Returns dX and one grad dict per rank.

    MLP block: db_fc2 = sum_rows dOut; dW2_i = dOut^T Z_i; dA_i = (dOut W2_i) * GeLU'(A_i);
      db1_i = sum_rows dA_i; dW1_i = dA_i^T V2; dV2 = AR(dA_i W1_i);
      dX2 = dOut + LN2-backward(dV2), with dgamma2, dbeta2.
    Attention block: db_o = sum_rows dX2; dW_o_i = dX2^T ctx_i; dctx_i = dX2 W_o_i;
      dQKV_i = attention_bwd(dctx_i); db_qkv_i = sum_rows dQKV_i; dW_qkv_i = dQKV_i^T U;
      dU = AR(dQKV_i W_qkv_i); dX = dX2 + LN1-backward(dU), with dgamma1, dbeta1.
    Replicated grads (LayerNorm, b_o, b_fc2) are identical on every rank and are put in
    each rank's dict, as each rank computes them redundantly.
    """
    dout = _f64(dout)
    p0 = shards[0]
    B, s, d = c["micro_batch"], c["seq"], c["head_dim"]
    grads: List[Params] = [dict() for _ in shards]
    dv2 = np.zeros_like(dout)
    for i, p in enumerate(shards):
        da = (dout @ _f64(p["w_fc2"])) * gelu_grad(c["a"][i])
        grads[i].update(w_fc2=dout.T @ c["z"][i], b_fc1=da.sum(axis=0), w_fc1=da.T @ c["v2"])
        dv2 += da @ _f64(p["w_fc1"])
    dx2_ln, dg2, db2ln = layernorm_bwd(dv2, c["x2"], p0["ln2_g"], c["mu2"], c["rstd2"])
    dx2 = dout + dx2_ln
    db_o = dx2.sum(axis=0)
    du = np.zeros_like(dout)
    for i, p in enumerate(shards):
        dctx = dx2 @ _f64(p["w_o"])
        heads = c["qkv"][i].shape[1] // (3 * d)
        dqkv = attention_bwd(dctx, c["qkv"][i], c["probs"][i], B, s, heads, d)
        grads[i].update(w_o=dx2.T @ c["ctx"][i], b_qkv=dqkv.sum(axis=0), w_qkv=dqkv.T @ c["u"])
        du += dqkv @ _f64(p["w_qkv"])
    dx1_ln, dg1, db1ln = layernorm_bwd(du, c["x"], p0["ln1_g"], c["mu1"], c["rstd1"])
    dx = dx2 + dx1_ln
    db_fc2 = dout.sum(axis=0)
    for g in grads:
        g.update(ln1_g=dg1, ln1_b=db1ln, b_o=db_o, ln2_g=dg2, ln2_b=db2ln, b_fc2=db_fc2)
    return dx, grads


# --------------------------------------------------------------------------- stage
def stage_fwd(x, layers: Sequence[Sequence[Params]], micro_batch: int, seq: int, head_dim: int
              ) -> Tuple[np.ndarray, List[dict]]:
    """Consecutive layers run as one pipeline stage (each entry of ``layers`` is the
    shards list of one layer); the output of layer l is the input of layer l+1."""
    caches = []
    for shards in layers:
        x, c = layer_fwd(x, shards, micro_batch, seq, head_dim)
        caches.append(c)
    return x, caches


def stage_bwd(dout, caches: List[dict], layers: Sequence[Sequence[Params]]
              ) -> Tuple[np.ndarray, List[List[Params]]]:
    """Backward through the stage, last layer first; returns dX and per-layer grads."""
    all_grads: List[List[Params]] = [None] * len(layers)  # type: ignore[list-item]
    for l in reversed(range(len(layers))):
        dout, all_grads[l] = layer_bwd(dout, caches[l], layers[l])
    return dout, all_grads
