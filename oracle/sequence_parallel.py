"""fp64 definition of the sequence-parallel share of the tensor-parallel layer.

TEST INFRASTRUCTURE (see the package docstring): only tests/ may use it.

The "Megatron-LM" concept report (compassingai.com), section 4.3, adds sequence
parallelism to the tensor-parallel split: the sequence dimension is split over the
same group of devices, each device handles one segment of the sequence and runs
LayerNorm locally, and devices communicate only where the attention (and the
tensor-parallel blocks) need the whole sequence. Section 6.4: each device then holds
S/tp of the sequence, so its activations shrink to 1/tp. Section 8(1): the
tensor-parallel all-reduce is carried out as a reduce-scatter and an all-gather.

Readings where the pages leave the step open:
  - Rank i owns positions [i s/t, (i+1) s/t) of every sequence of the micro-batch; its
    rows are kept in (sequence, position) order.
  - All-gather before each tensor-parallel block (of the LayerNorm output, and in the
    backward of the block's output gradient); reduce-scatter after each row-parallel
    product (the forward partials O_i, Y_i and the backward input-gradient partials).
    That is the all-reduce of section 4.1 split in its two halves (section 8(1)).
  - The bias + residual adds and both LayerNorms run on the rank's rows. Gradients of
    the replicated parameters (LayerNorm gains and shifts, b_o, b_fc2) are each rank's
    sum over its own rows; the group's all-reduce adds them.

Everything else is the layer of oracle/layer.py, reused block by block; the
collectives are index arithmetic on NumPy arrays.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np

from .layer import Params, _f64, attention_bwd, attention_fwd, layernorm_bwd, layernorm_fwd, mlp_bwd, mlp_fwd


def seq_rows(rank: int, tp: int, micro_batch: int, seq: int) -> np.ndarray:
    """Row indices (of the [B s, h] token-major activation) that rank `rank` owns."""
    assert seq % tp == 0, "the sequence must split evenly over the group"
    n = seq // tp
    return (np.arange(micro_batch)[:, None] * seq + rank * n + np.arange(n)[None, :]).reshape(-1)


def all_gather_seq(parts: Sequence[np.ndarray], micro_batch: int, seq: int) -> np.ndarray:
    """Each rank's rows put back in their places: the full [B s, ...] tensor."""
    tp = len(parts)
    full = np.zeros((micro_batch * seq,) + parts[0].shape[1:])
    for i, p in enumerate(parts):
        full[seq_rows(i, tp, micro_batch, seq)] = p
    return full


def reduce_scatter_seq(partials: Sequence[np.ndarray], micro_batch: int, seq: int) -> List[np.ndarray]:
    """Sum of the ranks' partials, each rank keeping its own rows."""
    total = np.zeros_like(_f64(partials[0]))
    for p in partials:
        total += _f64(p)
    return [total[seq_rows(i, len(partials), micro_batch, seq)] for i in range(len(partials))]


def attn_block_fwd(u, p: Params, micro_batch: int, seq: int, head_dim: int) -> Tuple[np.ndarray, dict]:
    """Rank's attention block (concept report, section 4.1: heads split over ranks,
    output projection split by rows): O_i = Attn(U W_qkv_i^T + b_qkv_i) W_o_i^T."""
    u = _f64(u)
    qkv = u @ _f64(p["w_qkv"]).T + _f64(p["b_qkv"])[None, :]
    heads = qkv.shape[1] // (3 * head_dim)
    ctx, probs = attention_fwd(qkv, micro_batch, seq, heads, head_dim)
    o = ctx @ _f64(p["w_o"]).T
    return o, dict(u=u, qkv=qkv, probs=probs, ctx=ctx, micro_batch=micro_batch, seq=seq, head_dim=head_dim)


def attn_block_bwd(do, c: dict, p: Params) -> Tuple[np.ndarray, Params]:
    """Backward of attn_block_fwd given dO: dW_o = dO^T ctx, dctx = dO W_o, the
    attention backward, db_qkv, dW_qkv = dQKV^T U and the input-gradient partial
    dU_i = dQKV W_qkv_i (summed over ranks by the backward all-reduce, section 4.2)."""
    do = _f64(do)
    d = c["head_dim"]
    dctx = do @ _f64(p["w_o"])
    heads = c["qkv"].shape[1] // (3 * d)
    dqkv = attention_bwd(dctx, c["qkv"], c["probs"], c["micro_batch"], c["seq"], heads, d)
    grads = dict(w_o=do.T @ c["ctx"], b_qkv=dqkv.sum(axis=0), w_qkv=dqkv.T @ c["u"])
    return dqkv @ _f64(p["w_qkv"]), grads


def sp_layer_fwd(x_parts: Sequence[np.ndarray], shards: Sequence[Params], micro_batch: int, seq: int,
                 head_dim: int) -> Tuple[List[np.ndarray], dict]:
    """One layer under tensor + sequence parallelism, every rank of the group.

    x_parts[i]: rank i's rows of X. Per rank: u_i = LN1(x_i); all-gather U; O_i = the
    rank's attention block on U; reduce-scatter O; x2_i = x_i + O_rs_i + b_o,
    v2_i = LN2(x2_i); all-gather V2; Y_i = the rank's MLP block on V2; reduce-scatter Y;
    out_i = x2_i + Y_rs_i + b_fc2. Returns each rank's out rows."""
    t = len(shards)
    p0 = shards[0]
    ln1 = [layernorm_fwd(_f64(x), p0["ln1_g"], p0["ln1_b"]) for x in x_parts]
    U = all_gather_seq([l[0] for l in ln1], micro_batch, seq)
    blocks = [attn_block_fwd(U, p, micro_batch, seq, head_dim) for p in shards]
    o_rs = reduce_scatter_seq([b[0] for b in blocks], micro_batch, seq)
    x2 = [_f64(x_parts[i]) + o_rs[i] + _f64(p0["b_o"])[None, :] for i in range(t)]
    ln2 = [layernorm_fwd(x2[i], p0["ln2_g"], p0["ln2_b"]) for i in range(t)]
    V2 = all_gather_seq([l[0] for l in ln2], micro_batch, seq)
    mlps = [mlp_fwd(V2, [p]) for p in shards]
    y_rs = reduce_scatter_seq([m[0] for m in mlps], micro_batch, seq)
    outs = [x2[i] + y_rs[i] + _f64(p0["b_fc2"])[None, :] for i in range(t)]
    cache = dict(x=[_f64(x) for x in x_parts], ln1=ln1, blocks=blocks, x2=x2, ln2=ln2, mlps=mlps,
                 micro_batch=micro_batch, seq=seq)
    return outs, cache


def sp_layer_bwd(dout_parts: Sequence[np.ndarray], c: dict, shards: Sequence[Params]
                 ) -> Tuple[List[np.ndarray], List[Params]]:
    """Backward of sp_layer_fwd, the collectives swapped: all-gather dOut; per rank the
    MLP block backward (dV2 partial, dW1, db1, dW2); reduce-scatter dV2; per rank
    dX2_i = dout_i + LN2-backward(dV2_rs_i) with its row sums (dgamma2, dbeta2, db_o =
    sum dX2_i, db_fc2 = sum dout_i); all-gather dX2; per rank the attention block
    backward (dU partial, dW_qkv, db_qkv, dW_o); reduce-scatter dU; per rank
    dX_i = dX2_i + LN1-backward(dU_rs_i) with dgamma1, dbeta1.
    Returns each rank's dX rows and grads (replicated ones: the rank's row sums)."""
    B, s = c["micro_batch"], c["seq"]
    t = len(shards)
    p0 = shards[0]
    dout_parts = [_f64(d) for d in dout_parts]
    dOut = all_gather_seq(dout_parts, B, s)
    grads: List[Params] = [dict() for _ in shards]
    dv2_partials = []
    for i, p in enumerate(shards):
        dv2_i, g = mlp_bwd(dOut, c["mlps"][i][1], [p])
        grads[i].update(g[0])
        dv2_partials.append(dv2_i)
    dv2_rs = reduce_scatter_seq(dv2_partials, B, s)
    dx2 = []
    for i in range(t):
        _, mu2, rstd2 = c["ln2"][i]
        dln, dg2, db2ln = layernorm_bwd(dv2_rs[i], c["x2"][i], p0["ln2_g"], mu2, rstd2)
        dx2.append(dout_parts[i] + dln)
        grads[i].update(ln2_g=dg2, ln2_b=db2ln, b_o=dx2[i].sum(axis=0), b_fc2=dout_parts[i].sum(axis=0))
    dX2 = all_gather_seq(dx2, B, s)
    du_partials = []
    for i, p in enumerate(shards):
        du_i, g = attn_block_bwd(dX2, c["blocks"][i][1], p)
        grads[i].update(g)
        du_partials.append(du_i)
    du_rs = reduce_scatter_seq(du_partials, B, s)
    dx = []
    for i in range(t):
        _, mu1, rstd1 = c["ln1"][i]
        dln, dg1, db1ln = layernorm_bwd(du_rs[i], c["x"][i], p0["ln1_g"], mu1, rstd1)
        dx.append(dx2[i] + dln)
        grads[i].update(ln1_g=dg1, ln1_b=db1ln)
    return dx, grads
