"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on seeded inputs.

Every output of the layer is compared: Out, dX and all twelve parameter gradients,
to the bar stated in gpu_support (fp32: max-abs <= 1e-4 RMS; bf16: RMS error <= 2e-2
RMS and max error <= c_T RMS, c_T the literal 2e-2 unless the bf16 rounding model
predicts more for that tensor, then 1.5 x the prediction, 2 x for one-dimensional
tensors: tests/ceilings.py).
Shapes go from the tiny fp32 layer through multi-tile shapes with ragged tails and
odd head dims to the workloads' full sizes, in both bf16 modes wherever bench.py can
report the workload in that mode.
"""
import numpy as np
import pytest

import ceilings
import oracle
import seeded_inputs as si
from gpu_support import (TOL, check_all, compare, log, oracle_layer, run_layer_gpu, run_mlp_gpu, run_stage_gpu)

pytestmark = pytest.mark.gpu


def _layer_case(shape, seed=0, random_affine=False, global_weights=True):
    return si.make_case(shape, seed=seed, global_weights=global_weights, random_affine=random_affine)


def _check_layer(shape, case, params=None, stored_key=None):
    """One layer shard against the oracle; bf16 ceilings from the rounding model (run
    here, or stored for the full-size workloads)."""
    params = params if params is not None else case.layers[0]
    log(f"layer {shape}")
    g_out, g_dx, g_gr = run_layer_gpu(shape, case.x, case.dout, params)
    r_out, r_dx, r_gr = oracle_layer(shape, case.x, case.dout, params)
    preds = None
    if shape.dtype == "bf16":
        preds = ceilings.stored(stored_key) if stored_key else ceilings.layer(shape, case.x, case.dout, params)
    bad = check_all(g_out, g_dx, g_gr, r_out, r_dx, r_gr, TOL[shape.dtype], preds=preds)
    assert not bad, f"tensors over the bar: {bad}"


TINY = si.WORKLOADS["tiny_fp32"].shape


@pytest.mark.parametrize("random_affine", [False, True])
def test_tiny_fp32_layer(random_affine):
    _check_layer(TINY, _layer_case(TINY, random_affine=random_affine))


@pytest.mark.parametrize("shard", [0, 1])
def test_tiny_fp32_tp2_shard(shard):
    """One rank of a tp=2 split: the shard's weights, all-reduce as the identity."""
    shape = TINY.replace(tp=2, shard=shard)
    case = _layer_case(shape, random_affine=True)
    _check_layer(shape, case)


@pytest.mark.parametrize("qk_pairs", [False, True])
def test_tiny_bf16_layer(qk_pairs):
    shape = TINY.replace(dtype="bf16", qk_pairs=qk_pairs)
    _check_layer(shape, _layer_case(shape, random_affine=True))


@pytest.mark.parametrize("dtype,tp", [("fp32", 2), ("bf16", 2), ("bf16", 4)])
def test_mlp_shards_sum_to_unsharded_block(dtype, tp):
    """The pages' invariant on the GPU: run every shard of the MLP block sequentially on
    one device and sum the partials; compare with the unsharded oracle block."""
    shape = si.LayerShape(h=256, heads=4, seq=72, micro_batch=3, tp=tp, dtype=dtype)
    case = si.mlp_case(shape.replace(tp=1), seed=5, random_bias=True)
    g = case.global_layers[0]
    y_sum = dx_sum = 0.0
    grads = []
    for i in range(tp):
        p = si.shard_slice(g, shape, i)
        y, dx, gr = run_mlp_gpu(shape.replace(shard=i), case.x, case.dout, p)
        y_sum, dx_sum = y_sum + y, dx_sum + dx
        grads.append(gr)
    y_ref, c = oracle.mlp_fwd(case.x, [g])
    dx_ref, g_ref = oracle.mlp_bwd(case.dout, c, [g])
    tol = TOL[dtype]
    nw = dtype == "bf16"
    pr = ceilings.mlp_shards(shape, case.x, case.dout, [si.shard_slice(g, shape, i) for i in range(tp)]) if nw else {}
    ok = compare("sum y", y_sum, y_ref, tol, nw, pr.get("sum y"))[0]
    ok &= compare("sum dx", dx_sum, dx_ref, tol, nw, pr.get("sum dx"))[0]
    fs = 4 * shape.h // tp
    for i, gr in enumerate(grads):
        ok &= compare(f"dW1[{i}]", gr["w_fc1"], g_ref[0]["w_fc1"][i * fs:(i + 1) * fs], tol, nw, pr.get(f"dW1[{i}]"))[0]
        ok &= compare(f"db1[{i}]", gr["b_fc1"], g_ref[0]["b_fc1"][i * fs:(i + 1) * fs], tol, nw, pr.get(f"db1[{i}]"))[0]
        ok &= compare(f"dW2[{i}]", gr["w_fc2"], g_ref[0]["w_fc2"][:, i * fs:(i + 1) * fs], tol, nw,
                      pr.get(f"dW2[{i}]"))[0]
    assert ok


def _run_attn_gpu(shape, u, d_o, p):
    """mt_attn_fwd + mt_attn_bwd of one shard; returns (o_partial, du_partial, grads)."""
    import torch
    import tensor_layer_gemms_amd as mt
    from gpu_support import mt_shape, to_dev, to_np
    sh = mt_shape(shape)
    dt = shape.dtype
    ud, dod = to_dev(u, dt), to_dev(d_o, dt)
    wq, bq, wo = to_dev(p["w_qkv"], dt), to_dev(p["b_qkv"], dt), to_dev(p["w_o"], dt)
    ht = shape.h // shape.tp
    assert wq.shape == (3 * ht, shape.h) and wo.shape == (shape.h, ht) and ud.shape == (shape.tokens, shape.h)
    saved = torch.empty(mt.attn_saved_bytes(sh), dtype=torch.uint8, device="cuda")
    ws = torch.empty(mt.attn_workspace_bytes(sh), dtype=torch.uint8, device="cuda")
    o, du = torch.empty_like(ud), torch.empty_like(ud)
    g = {k: torch.empty(p[k].shape, dtype=torch.float32, device="cuda") for k in ("w_qkv", "b_qkv", "w_o")}
    mt.attn_fwd(sh, ud, wq, bq, wo, o, saved, ws)
    mt.attn_bwd(sh, ud, wq, wo, saved, dod, du, g["w_qkv"], g["b_qkv"], g["w_o"], ws)
    torch.cuda.synchronize()
    return to_np(o), to_np(du), {k: to_np(v) for k, v in g.items()}


@pytest.mark.parametrize("dtype,tp,h,heads,seq,mb", [
    ("fp32", 2, 64, 4, 32, 2),       # unfused attention, literal 1e-4 bar
    ("bf16", 2, 512, 4, 136, 2),     # head dim 128: fused attention
    ("bf16", 4, 512, 8, 72, 3),      # head dim 64, three sequences
    ("bf16", 2, 640, 4, 104, 1),     # head dim 160: fused attention, ragged blocks
    ("bf16", 2, 384, 4, 104, 1),     # head dim 96: materialised attention
    ("bf16", 2, 512, 8, 512, 4),     # 2048 tokens: out-projection and QKV weight gradients in 4 token slices
])
def test_attn_shards_sum_to_unsharded_block(dtype, tp, h, heads, seq, mb):
    """The pages' head-parallel split on the GPU: every shard of the attention block
    (mt_attn_*) run in turn on one device; the sum of the output partials and of the
    input-gradient partials against the unsharded oracle block, and each shard's weight
    gradients against the matching slice of the unsharded ones."""
    shape = si.LayerShape(h=h, heads=heads, seq=seq, micro_batch=mb, tp=tp, dtype=dtype)
    log(f"[attn block] {dtype} tp={tp} h={h} heads={heads} seq={seq} micro_batch={mb}")
    case = si.make_case(shape.replace(tp=1), seed=h + tp, global_weights=True, random_affine=True)
    g = case.global_layers[0]
    o_ref, c = oracle.attn_block_fwd(case.x, g, mb, seq, shape.head_dim)
    du_ref, g_ref = oracle.attn_block_bwd(case.dout, c, g)
    o_sum = du_sum = 0.0
    tol, nw = TOL[dtype], dtype == "bf16"
    pr = ceilings.attn_shards(shape, case.x, case.dout, [si.shard_slice(g, shape, i) for i in range(tp)]) if nw else {}
    ok = True
    for i in range(tp):
        p = si.shard_slice(g, shape, i)
        o, du, gr = _run_attn_gpu(shape.replace(shard=i), case.x, case.dout, p)
        o_sum, du_sum = o_sum + o, du_sum + du
        want = si.shard_slice(dict(g, **g_ref), shape, i)
        for k in ("w_qkv", "b_qkv", "w_o"):
            ok &= compare(f"{k}[{i}]", gr[k], want[k], tol, nw, pr.get(f"{k}[{i}]"))[0]
    ok &= compare("sum o", o_sum, o_ref, tol, nw, pr.get("sum o"))[0]
    ok &= compare("sum du", du_sum, du_ref, tol, nw, pr.get("sum du"))[0]
    assert ok


@pytest.mark.parametrize("h,heads,seq,mb,tp,shard", [
    (320, 5, 136, 3, 1, 0),    # several tiles, ragged token and feature tails
    (640, 4, 264, 1, 2, 1),    # head dim 160 (fused attention), shard 1 of 2, ragged seq
    (1280, 8, 200, 2, 2, 0),   # head dim 160, 4 heads per shard, ragged query and key blocks
    (384, 4, 136, 2, 2, 1),    # head dim 96: materialised attention
    (512, 8, 520, 2, 2, 0),    # seq spanning three causal chunks
    (512, 4, 200, 2, 2, 1),    # head dim 128 (fused attention): ragged query and key blocks
    (1024, 8, 72, 3, 1, 0),    # head dim 128, short sequences, 3 sequences per micro-batch
    (512, 8, 512, 4, 2, 1),    # 2048 tokens over a narrow shard: FC1, out-projection and QKV
                               # weight gradients in token slices (2, 4, 4)
])
@pytest.mark.parametrize("qk_pairs", [False, True], ids=["bf16", "bf16qk"])
def test_layer_bf16_multi_tile(h, heads, seq, mb, tp, shard, qk_pairs):
    shape = si.LayerShape(h=h, heads=heads, seq=seq, micro_batch=mb, tp=tp, shard=shard, qk_pairs=qk_pairs)
    case = _layer_case(shape, seed=h + seq, random_affine=True)
    _check_layer(shape, case)


def test_qk_pairs_lower_the_logit_error():
    """MT_BF16_QK against MT_BF16 on the same inputs. At h=8192 the logits are large
    enough that the plain bf16 logits leave RMS errors of about 1% for dW_qkv and dX (the
    GPU measures 0.98% and 0.90%, against 0.58% and 0.56% with the hi + lo logits): the
    compensated mode must bring both at least 20% closer to the oracle."""
    from gpu_support import rel_rms
    shape = si.LayerShape(h=8192, heads=64, seq=256, micro_batch=1, tp=8, shard=3)  # head dim 128, fused
    case = si.make_case(shape, seed=31, global_weights=False, random_affine=True)
    plain = run_layer_gpu(shape, case.x, case.dout, case.layers[0])
    pairs = run_layer_gpu(shape.replace(qk_pairs=True), case.x, case.dout, case.layers[0])
    r_out, r_dx, r_gr = oracle_layer(shape, case.x, case.dout, case.layers[0])
    e_plain = (rel_rms(plain[2]["w_qkv"], r_gr["w_qkv"]), rel_rms(plain[1], r_dx))
    e_pairs = (rel_rms(pairs[2]["w_qkv"], r_gr["w_qkv"]), rel_rms(pairs[1], r_dx))
    log(f"  rms error dW_qkv, dX: bf16 {e_plain}, bf16qk {e_pairs}")
    assert e_pairs[0] < 0.8 * e_plain[0] and e_pairs[1] < 0.8 * e_plain[1]
    qk = shape.replace(qk_pairs=True)
    bad = check_all(*pairs, r_out, r_dx, r_gr, TOL["bf16"], preds=ceilings.layer(qk, case.x, case.dout, case.layers[0]))
    assert not bad, bad


@pytest.mark.parametrize("h,heads,seq,mb,tp,shard,dtype", [
    (64, 4, 8, 1, 4, 3, "fp32"),     # 8 tokens, one head (of 16) per shard, last shard
    (128, 2, 8, 1, 2, 1, "bf16"),    # one head of 64 per shard: fused attention on an 8-row block
    (256, 2, 8, 3, 2, 0, "bf16"),    # head dim 128, three 8-token sequences in one row block each
    (512, 4, 16, 2, 1, 0, "bf16"),   # tp = 1, two 16-token sequences
])
def test_layer_degenerate_shapes(h, heads, seq, mb, tp, shard, dtype):
    """The smallest sequences the ABI accepts (a fraction of one attention block), one head
    per shard, and tp = 1: every output and gradient against the oracle."""
    shape = si.LayerShape(h=h, heads=heads, seq=seq, micro_batch=mb, tp=tp, shard=shard, dtype=dtype)
    case = _layer_case(shape, seed=seq + h, random_affine=True)
    _check_layer(shape, case)


def test_layer_fp32_multi_tile():
    shape = si.LayerShape(h=192, heads=3, seq=200, micro_batch=2, tp=1, dtype="fp32")
    _check_layer(shape, _layer_case(shape, seed=3, random_affine=True))


@pytest.mark.parametrize("mode", ["bf16", "bf16qk"])
def test_gpt_h1024_full(mode):
    w = si.WORKLOADS["gpt_h1024"]
    case = si.workload_case("gpt_h1024")
    _check_layer(w.shape.replace(qk_pairs=mode == "bf16qk"), case, stored_key=f"gpt_h1024:{mode}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("mode", ["bf16", "bf16qk"])
def test_gpt175b_tp8_shard_full(mode):
    """The 175B-shaped shard at full size, every output against the full oracle."""
    w = si.WORKLOADS["gpt175b_tp8"]
    case = si.workload_case("gpt175b_tp8")
    _check_layer(w.shape.replace(qk_pairs=mode == "bf16qk"), case, stored_key=f"gpt175b_tp8:{mode}")


def test_bitwise_deterministic():
    """Two runs give identical bits: no float atomics, fixed reduction orders."""
    shape = si.LayerShape(h=512, heads=8, seq=256, micro_batch=2, tp=2)
    case = _layer_case(shape, seed=9, random_affine=True)
    (o1, d1, g1), (o2, d2, g2) = run_layer_gpu(shape, case.x, case.dout, case.layers[0], repeat=2)
    assert np.array_equal(o1, o2) and np.array_equal(d1, d2)
    for k in g1:
        assert np.array_equal(g1[k], g2[k]), k


def test_stage_two_layers_small():
    """Consecutive layers as one pipeline stage (forward l0, l1; backward l1, l0)."""
    shape = si.LayerShape(h=256, heads=4, seq=128, micro_batch=2, tp=2)
    case = si.make_case(shape, seed=12, layers=2, random_affine=True)
    out, dx, grads = run_stage_gpu(shape, case.x, case.dout, case.layers)
    layers = [[p] for p in case.layers]
    r_out, caches = oracle.stage_fwd(case.x, layers, shape.micro_batch, shape.seq, shape.head_dim)
    r_dx, r_grads = oracle.stage_bwd(case.dout, caches, layers)
    preds = ceilings.stage(shape, case.x, case.dout, case.layers)
    bad = _check_stage(out, dx, grads, r_out, r_dx, [g[0] for g in r_grads], preds)
    assert not bad, bad


def _check_stage(out, dx, grads, r_out, r_dx, r_grads, preds):
    """Every output of a stage: out, dx, and each layer's gradients as "l<l>.<tensor>"."""
    bad = []
    for name, g, r in [("out", out, r_out), ("dx", dx, r_dx)]:
        if not compare(name, g, r, TOL["bf16"], True, preds.get(name))[0]:
            bad.append(name)
    for l, rg in enumerate(r_grads):
        for k in sorted(rg):
            name = f"l{l}.{k}"
            if not compare(name, grads[l][k], rg[k], TOL["bf16"], True, preds.get(name))[0]:
                bad.append(name)
    return bad


# ------------------------------------------------------------------ full-size workloads
@pytest.mark.timeout(1800)
def test_gpt1t_tp8_shard_full():
    """The 1T-shaped shard (head dim 160) at full size against the full oracle, in the
    MT_BF16_QK mode, the mode bench.py runs it in: with bf16 Q and K alone its large
    logits put the normwise error of Out, dX and the attention gradients at ~3%
    (measured and predicted by the rounding model), over the 2e-2 bar."""
    w = si.WORKLOADS["gpt1t_tp8"]
    case = si.workload_case("gpt1t_tp8")
    _check_layer(w.shape.replace(qk_pairs=True), case, stored_key="gpt1t_tp8:bf16qk")


# The h=8192 stage runs in the MT_BF16_QK mode (as bench.py runs it): in MT_BF16 the
# rounding of the large logits compounds over the four layers and puts the RMS error of
# the first layers' dW_qkv, dW_o and d(ln1 gain) at 2.1-2.3%, over the bar.
STAGE_SHAPE = dict(qk_pairs=True)


def _stage_oracle(mb):
    w = si.WORKLOADS[f"gpt_h8192_stage_mb{mb}"]
    case = si.workload_case(f"gpt_h8192_stage_mb{mb}")
    layers = [[p] for p in case.layers]
    sh = w.shape
    out, caches = oracle.stage_fwd(case.x, layers, sh.micro_batch, sh.seq, sh.head_dim)
    dx, grads = oracle.stage_bwd(case.dout, caches, layers)
    del caches
    return w, case, (out, dx, [g[0] for g in grads])


@pytest.mark.timeout(1800)
@pytest.mark.parametrize("mb", [1, 2, 4])
def test_stage_h8192_full(mb):
    """4 consecutive h=8192 tp=8 layers as one stage at micro-batch mb: every output and
    every layer's gradients against the full oracle of the stage."""
    w, case, (r_out, r_dx, r_grads) = _stage_oracle(mb)
    shape = w.shape.replace(**STAGE_SHAPE)
    log(f"stage {shape} x{w.layers}")
    out, dx, grads = run_stage_gpu(shape, case.x, case.dout, case.layers)
    bad = _check_stage(out, dx, grads, r_out, r_dx, r_grads, ceilings.stored(f"gpt_h8192_stage_mb{mb}:bf16qk"))
    assert not bad, bad


@pytest.mark.timeout(1800)
def test_stage_h8192_micro_batch8_sampled():
    """Micro-batch 8 of the same stage. Sequences are independent in the layer and
    sequence 0's inputs are the same seeded rows at every micro-batch size, so sequence
    0's rows of Out and dX must equal those of the micro-batch-1 run bit for bit (no
    kernel's per-element arithmetic depends on the number of tokens) and meet the
    micro-batch-1 oracle. Weight gradients are sums over sequences: they must equal the
    sum of the eight per-sequence runs (each of which is a micro-batch-1 run, checked
    against the oracle by test_stage_h8192_full) to the fp32 bar, the runs differing
    only in the fp32 summation order over tokens."""
    mb = 8
    w = si.WORKLOADS[f"gpt_h8192_stage_mb{mb}"]
    case = si.workload_case(f"gpt_h8192_stage_mb{mb}")
    s = w.shape.seq
    shape = w.shape.replace(**STAGE_SHAPE)
    log(f"stage {shape} x{w.layers}")
    out, dx, grads = run_stage_gpu(shape, case.x, case.dout, case.layers)
    _, _, (r_out, r_dx, _) = _stage_oracle(1)
    preds = ceilings.stored("gpt_h8192_stage_mb1:bf16qk")
    assert compare("out[seq0]", out[:s], r_out, TOL["bf16"], True, preds["out"])[0]
    assert compare("dx[seq0]", dx[:s], r_dx, TOL["bf16"], True, preds["dx"])[0]
    one = shape.replace(micro_batch=1)
    total = None
    for b in range(mb):
        ob, db, gb = run_stage_gpu(one, case.x[b * s:(b + 1) * s], case.dout[b * s:(b + 1) * s], case.layers)
        if b == 0:
            same = bool(np.array_equal(out[:s], ob)) and bool(np.array_equal(dx[:s], db))
            log(f"  seq0 rows bitwise equal to the micro-batch-1 run: {same}")
            assert same
        total = gb if total is None else [{k: t[k] + g[k] for k in t} for t, g in zip(total, gb)]
    for l in range(w.layers):
        for k in ("w_qkv", "w_fc1", "b_o", "ln1_g"):
            assert compare(f"l{l}.{k} sum", grads[l][k], total[l][k], TOL["fp32"], False)[0]
