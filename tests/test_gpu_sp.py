"""GPU parity of the sequence-parallel share ("Megatron-LM" concept report, section 4.3;
the all-reduce as reduce-scatter + all-gather, section 8(1)).

Every rank of the group runs its phases one after the other on one device, through the
C ABI: mt_sp_ln_fwd on its rows, mt_attn_fwd and mt_mlp_fwd on the gathered rows,
mt_sp_add_fwd, and the backward in reverse. The all-gathers and reduce-scatters between
the calls are plain torch indexing and sums (the collectives are the caller's; a
reduce-scatter's output is rounded to the activation dtype once, after an fp32 sum).
Each rank's out rows, dx rows, shard weight gradients and replicated-parameter partial
gradients are compared with oracle.sp_layer_fwd / sp_layer_bwd (pinned against the
tensor-parallel layer in tests/test_oracle_sp.py) at the bar of the layer tests, the
bf16 ceilings from the rounding model of the tensor-parallel layer with the
reduce-scatter outputs rounded once (tests/ceilings.py).
"""
from __future__ import annotations

import numpy as np
import pytest

import ceilings
import oracle
import seeded_inputs as si
from gpu_support import TOL, check_all, log, mt_mod, mt_shape, to_dev, to_np, torch_mod

pytestmark = pytest.mark.gpu

SHARD_KEYS = ("w_qkv", "b_qkv", "w_o", "w_fc1", "b_fc1", "w_fc2")
REPLICATED = ("ln1_g", "ln1_b", "b_o", "ln2_g", "ln2_b", "b_fc2")


def _rows(rank: int, tp: int, micro_batch: int, seq: int) -> np.ndarray:
    """Token rows of rank `rank`: positions [rank s/t, (rank+1) s/t) of every sequence."""
    n = seq // tp
    return np.concatenate([b * seq + rank * n + np.arange(n) for b in range(micro_batch)])


def run_sp_layer_gpu(shape: si.LayerShape, x: np.ndarray, dout: np.ndarray, shards):
    torch, mt = torch_mod(), mt_mod()
    dt = shape.dtype
    t, B, s, h = shape.tp, shape.micro_batch, shape.seq, shape.h
    M = B * s
    n = M // t
    idx = [torch.from_numpy(_rows(i, t, B, s)).cuda() for i in range(t)]
    xd, dd = to_dev(x, dt), to_dev(dout, dt)
    act = xd.dtype
    W = [{k: to_dev(v, dt) for k, v in p.items()} for p in shards]
    sh = [mt_shape(shape.replace(shard=i)) for i in range(t)]
    f32 = dict(dtype=torch.float32, device="cuda")

    def gather(parts):  # all-gather along the sequence
        full = torch.empty((M,) + tuple(parts[0].shape[1:]), dtype=parts[0].dtype, device="cuda")
        for i, p in enumerate(parts):
            full[idx[i]] = p
        return full

    def scatter(partials):  # reduce-scatter along the sequence
        total = sum(p.float() for p in partials)
        return [total[idx[i]].to(act).contiguous() for i in range(t)]

    def rows_of(full, i):
        return full[idx[i]].contiguous()

    assert xd.shape == (M, h) and all(W[i]["w_qkv"].shape == (3 * h // t, h) for i in range(t))
    x_i = [rows_of(xd, i) for i in range(t)]
    asaved = [torch.empty(mt.attn_saved_bytes(sh[i]), dtype=torch.uint8, device="cuda") for i in range(t)]
    msaved = [torch.empty(mt.mlp_saved_bytes(sh[i]), dtype=torch.uint8, device="cuda") for i in range(t)]
    aws = torch.empty(mt.attn_workspace_bytes(sh[0]), dtype=torch.uint8, device="cuda")
    mws = torch.empty(mt.mlp_workspace_bytes(sh[0]), dtype=torch.uint8, device="cuda")
    lws = torch.empty(mt.sp_ln_workspace_bytes(sh[0]), dtype=torch.uint8, device="cuda")
    assert min(t.numel() for t in asaved + msaved) > 0 and aws.numel() > 0 and lws.numel() > 0

    # ---- forward
    u = [torch.empty(n, h, dtype=act, device="cuda") for _ in range(t)]
    mean1 = [torch.empty(n, **f32) for _ in range(t)]
    rstd1 = [torch.empty(n, **f32) for _ in range(t)]
    for i in range(t):
        mt.sp_ln_fwd(sh[i], x_i[i], W[i]["ln1_g"], W[i]["ln1_b"], u[i], mean1[i], rstd1[i])
    U = gather(u)
    o = [torch.empty(M, h, dtype=act, device="cuda") for _ in range(t)]
    for i in range(t):
        mt.attn_fwd(sh[i], U, W[i]["w_qkv"], W[i]["b_qkv"], W[i]["w_o"], o[i], asaved[i], aws)
    o_rs = scatter(o)
    x2 = [torch.empty(n, h, **f32) for _ in range(t)]
    v2 = [torch.empty(n, h, dtype=act, device="cuda") for _ in range(t)]
    mean2 = [torch.empty(n, **f32) for _ in range(t)]
    rstd2 = [torch.empty(n, **f32) for _ in range(t)]
    for i in range(t):
        mt.sp_ln_fwd(sh[i], x_i[i], W[i]["ln2_g"], W[i]["ln2_b"], v2[i], mean2[i], rstd2[i], resid=o_rs[i],
                     bias=W[i]["b_o"], x2=x2[i])
    V2 = gather(v2)
    y = [torch.empty(M, h, dtype=act, device="cuda") for _ in range(t)]
    for i in range(t):
        mt.mlp_fwd(sh[i], V2, W[i]["w_fc1"], W[i]["b_fc1"], W[i]["w_fc2"], y[i], msaved[i], mws)
    y_rs = scatter(y)
    out = [torch.empty(n, h, dtype=act, device="cuda") for _ in range(t)]
    for i in range(t):
        mt.sp_add_fwd(sh[i], x2[i], y_rs[i], W[i]["b_fc2"], out[i])

    # ---- backward
    dout_i = [rows_of(dd, i) for i in range(t)]
    dOut = gather(dout_i)
    grads = [{k: torch.empty(v.shape, **f32) for k, v in shards[i].items()} for i in range(t)]
    dv2 = [torch.empty(M, h, dtype=act, device="cuda") for _ in range(t)]
    for i in range(t):
        g = grads[i]
        mt.mlp_bwd(sh[i], V2, W[i]["w_fc1"], W[i]["w_fc2"], msaved[i], dOut, dv2[i], g["w_fc1"], g["b_fc1"],
                   g["w_fc2"], mws)
    dv2_rs = scatter(dv2)
    dx2 = [torch.empty(n, h, dtype=act, device="cuda") for _ in range(t)]
    dx2f = [torch.empty(n, h, **f32) for _ in range(t)]
    for i in range(t):
        g = grads[i]
        mt.sp_ln_bwd(sh[i], dv2_rs[i], x2[i], W[i]["ln2_g"], mean2[i], rstd2[i], dout_i[i], dx2[i], g["ln2_g"],
                     g["ln2_b"], lws, xin_f32=True, dres_f32=False, dx_f32=dx2f[i], dsum=g["b_o"],
                     dres_sum=g["b_fc2"])
    dX2 = gather(dx2)
    du = [torch.empty(M, h, dtype=act, device="cuda") for _ in range(t)]
    for i in range(t):
        g = grads[i]
        mt.attn_bwd(sh[i], U, W[i]["w_qkv"], W[i]["w_o"], asaved[i], dX2, du[i], g["w_qkv"], g["b_qkv"], g["w_o"],
                    aws)
    du_rs = scatter(du)
    dx = [torch.empty(n, h, dtype=act, device="cuda") for _ in range(t)]
    for i in range(t):
        g = grads[i]
        mt.sp_ln_bwd(sh[i], du_rs[i], x_i[i], W[i]["ln1_g"], mean1[i], rstd1[i], dx2f[i], dx[i], g["ln1_g"],
                     g["ln1_b"], lws, xin_f32=False, dres_f32=True)
    torch.cuda.synchronize()
    return ([to_np(a) for a in out], [to_np(a) for a in dx],
            [{k: to_np(v) for k, v in g.items()} for g in grads])


@pytest.mark.parametrize("h,heads,seq,mb,tp,dtype", [
    (64, 4, 32, 2, 2, "fp32"),     # the tiny fp32 layer (unfused attention), literal 1e-4 bar
    (512, 4, 136, 2, 2, "bf16"),   # head dim 128: fused attention; 68-token segments
    (640, 4, 264, 1, 2, "bf16"),   # head dim 160: materialised attention, ragged tiles
    (512, 8, 64, 3, 4, "bf16"),    # tp=4, head dim 64, three sequences of 16-token segments
    (256, 2, 64, 2, 1, "bf16"),    # tp=1: the share is the whole layer
    (384, 6, 72, 1, 3, "bf16"),    # 24-token segments: the rank's row count is not a tile multiple
])
def test_sequence_parallel_share_matches_oracle(h, heads, seq, mb, tp, dtype):
    shape = si.LayerShape(h=h, heads=heads, seq=seq, micro_batch=mb, tp=tp, dtype=dtype)
    log(f"[sp] h={h} heads={heads} seq={seq} micro_batch={mb} tp={tp} {dtype}")
    case = si.make_case(shape.replace(tp=1), seed=h + seq + tp, global_weights=True, random_affine=True)
    g = case.global_layers[0]
    shards = [si.shard_slice(g, shape, i) for i in range(tp)]
    outs, dxs, grads = run_sp_layer_gpu(shape, case.x, case.dout, shards)
    rows = [_rows(i, tp, mb, seq) for i in range(tp)]
    r_out, c = oracle.sp_layer_fwd([case.x[r] for r in rows], shards, mb, seq, shape.head_dim)
    r_dx, r_g = oracle.sp_layer_bwd([case.dout[r] for r in rows], c, shards)
    preds = ceilings.sp_ranks(shape, case.x, case.dout, shards, rows) if dtype == "bf16" else [None] * tp
    bad = []
    for i in range(tp):
        log(f"[sp] rank {i}")
        bad += [f"rank {i}: {k}" for k in check_all(outs[i], dxs[i], grads[i], r_out[i], r_dx[i], r_g[i],
                                                        TOL[dtype], keys=SHARD_KEYS + REPLICATED, preds=preds[i])]
    assert not bad, bad
