"""Pins of the oracle's sequence-parallel share (CPU, fp64).

Sequence parallelism ("Megatron-LM" concept report, section 4.3) only moves where the
tensor-parallel layer's work happens: LayerNorm and the residual adds on each rank's
segment of the sequence, the all-reduce split into reduce-scatter and all-gather
(section 8(1)). So every rank's outputs must be its rows of the tensor-parallel
layer's outputs (oracle.layer_fwd / layer_bwd with the all-reduce as a sum, itself
pinned by finite differences and the pages' sum-of-partials invariant), its shard
weight gradients must equal the tensor-parallel ones, and the replicated parameters'
gradients must sum over ranks to the tensor-parallel ones.
"""
import numpy as np
import pytest

import oracle
import seeded_inputs as si

TINY = si.WORKLOADS["tiny_fp32"].shape  # h=64, 4 heads, seq 32, micro-batch 2
REPLICATED = ("ln1_g", "ln1_b", "b_o", "ln2_g", "ln2_b", "b_fc2")


def _rel(a, b):
    return np.max(np.abs(np.asarray(a) - np.asarray(b))) / max(np.sqrt(np.mean(np.asarray(b) ** 2)), 1e-300)


@pytest.mark.parametrize("tp,B,s", [(1, 2, 32), (2, 2, 32), (4, 3, 16), (8, 1, 64)])
def test_rows_partition_the_tokens(tp, B, s):
    """Every token belongs to exactly one rank; rank i holds positions [i s/t, (i+1) s/t)
    of every sequence, in (sequence, position) order."""
    rows = [oracle.seq_rows(i, tp, B, s) for i in range(tp)]
    allr = np.concatenate(rows)
    assert len(allr) == B * s and len(np.unique(allr)) == B * s
    n = s // tp
    for i, r in enumerate(rows):
        b, j = r // s, r % s
        assert np.array_equal(b, np.repeat(np.arange(B), n))
        assert np.array_equal(j, np.tile(np.arange(i * n, (i + 1) * n), B))


def test_gather_and_scatter_compose_to_the_sum():
    """all-gather(reduce-scatter(partials)) is the sum of the partials, and all-gather
    of a tensor's row chunks is the tensor."""
    rng = np.random.default_rng(5)
    B, s, tp = 2, 16, 4
    parts = [rng.standard_normal((B * s, 3)) for _ in range(tp)]
    total = parts[0] + parts[1] + parts[2] + parts[3]
    rs = oracle.reduce_scatter_seq(parts, B, s)
    assert np.allclose(oracle.all_gather_seq(rs, B, s), total, rtol=0, atol=1e-15)
    full = rng.standard_normal((B * s, 5))
    chunks = [full[oracle.seq_rows(i, tp, B, s)] for i in range(tp)]
    assert np.array_equal(oracle.all_gather_seq(chunks, B, s), full)


def test_attention_block_partials_sum_to_the_unsharded_block():
    """Heads split over ranks: sum_i Attn_i(U) W_o_i^T equals the unsharded block, and
    the input-gradient partials sum to the unsharded input gradient (sections 4.1, 4.2)."""
    case = si.make_case(TINY, seed=2, global_weights=True, random_affine=True)
    g = case.global_layers[0]
    u = case.x
    B, s, d = TINY.micro_batch, TINY.seq, TINY.head_dim
    o1, c1 = oracle.attn_block_fwd(u, g, B, s, d)
    du1, g1 = oracle.attn_block_bwd(case.dout, c1, g)
    for tp in (2, 4):
        shards = [si.shard_slice(g, TINY.replace(tp=tp), i) for i in range(tp)]
        outs = [oracle.attn_block_fwd(u, p, B, s, d) for p in shards]
        assert _rel(sum(o for o, _ in outs), o1) < 1e-12
        bw = [oracle.attn_block_bwd(case.dout, c, p) for (_, c), p in zip(outs, shards)]
        assert _rel(sum(du for du, _ in bw), du1) < 1e-12
        for i, (_, gi) in enumerate(bw):
            want = si.shard_slice(dict(g1, **{k: g[k] for k in g if k not in g1}), TINY.replace(tp=tp), i)
            for k in ("w_qkv", "b_qkv", "w_o"):
                assert _rel(gi[k], want[k]) < 1e-12, k


@pytest.mark.parametrize("tp,affine", [(1, True), (2, True), (4, True), (2, False)])
def test_sequence_parallel_layer_equals_tensor_parallel_layer(tp, affine):
    case = si.make_case(TINY, seed=3, global_weights=True, random_affine=affine)
    g = case.global_layers[0]
    shards = [si.shard_slice(g, TINY.replace(tp=tp), i) for i in range(tp)]
    B, s, d = TINY.micro_batch, TINY.seq, TINY.head_dim
    out, c = oracle.layer_fwd(case.x, shards, B, s, d)
    dx, grads = oracle.layer_bwd(case.dout, c, shards)
    rows = [oracle.seq_rows(i, tp, B, s) for i in range(tp)]
    outs, sc = oracle.sp_layer_fwd([case.x[r] for r in rows], shards, B, s, d)
    dxs, sg = oracle.sp_layer_bwd([case.dout[r] for r in rows], sc, shards)
    for i, r in enumerate(rows):
        assert _rel(outs[i], out[r]) < 1e-12
        assert _rel(dxs[i], dx[r]) < 1e-12
        for k in ("w_qkv", "b_qkv", "w_o", "w_fc1", "b_fc1", "w_fc2"):
            assert _rel(sg[i][k], grads[i][k]) < 1e-12, k
    for k in REPLICATED:
        assert _rel(sum(gr[k] for gr in sg), grads[0][k]) < 1e-12, k
    if tp > 1:  # and a rank's replicated gradient is a partial, not the whole
        assert _rel(sg[0]["ln1_g"], grads[0]["ln1_g"]) > 1e-3
