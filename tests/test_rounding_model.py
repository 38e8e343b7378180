"""CPU pins of the bf16 rounding model (oracle/rounding.py), which sets the per-tensor
max-error ceilings of the bf16 parity tests."""
import json
import os

import numpy as np
import pytest

import oracle
import seeded_inputs as si
from oracle import rounding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _case(tp=2, shard=0, layers=1, seed=2):
    shape = si.LayerShape(h=256, heads=4, seq=128, micro_batch=2, tp=tp, shard=shard)
    return si.make_case(shape, seed=seed, layers=layers, global_weights=True, random_affine=True)


def test_bf16_rounding_matches_the_input_generator():
    """The model's bf16 rounding (via float32, nearest even) is the generators' rounding on
    float32 values, including ties and values that round up across a binade."""
    rng = np.random.default_rng(0)
    a = (rng.standard_normal(100000) * 10.0 ** rng.integers(-8, 8, 100000)).astype(np.float32)
    ties = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 255.5, -(2.0 - 2.0 ** -9)], np.float32)
    for v in (a, ties):
        assert np.array_equal(rounding.bf16(v), si.bf16_round(v).astype(np.float64))


def test_model_without_rounding_is_the_oracle_one_shard():
    case = _case()
    sh = case.shape
    out, dx, g, _ = rounding.layer(case.x, case.dout, case.layers, sh.micro_batch, sh.seq, sh.head_dim, ())
    r_out, c = oracle.layer_fwd(case.x, case.layers, sh.micro_batch, sh.seq, sh.head_dim)
    r_dx, r_g = oracle.layer_bwd(case.dout, c, case.layers)
    assert np.allclose(out, r_out, rtol=0, atol=1e-12) and np.allclose(dx, r_dx, rtol=0, atol=1e-11)
    for k in r_g[0]:
        assert np.allclose(g[0][k], r_g[0][k], rtol=1e-10, atol=1e-10), k


def test_model_without_rounding_is_the_tensor_parallel_oracle():
    """All ranks of a tp=2 split with the all-reduce as the sum: the oracle's sharded
    layer; the per-row contributions of the replicated gradients sum to them."""
    case = _case()
    sh = case.shape
    shards = [si.shard_slice(case.global_layers[0], sh, i) for i in range(2)]
    out, dx, g, rows = rounding.layer(case.x, case.dout, shards, sh.micro_batch, sh.seq, sh.head_dim, ())
    r_out, c = oracle.layer_fwd(case.x, shards, sh.micro_batch, sh.seq, sh.head_dim)
    r_dx, r_g = oracle.layer_bwd(case.dout, c, shards)
    assert np.allclose(out, r_out, atol=1e-11) and np.allclose(dx, r_dx, atol=1e-11)
    for i in range(2):
        for k in r_g[i]:
            assert np.allclose(g[i][k], r_g[i][k], rtol=1e-10, atol=1e-10), (i, k)
    for k, v in rows.items():
        assert np.allclose(v.sum(0), r_g[0][k], rtol=1e-10, atol=1e-10), k


def test_stage_model_without_rounding_is_the_oracle_stage():
    case = _case(tp=1, layers=2)
    sh = case.shape
    out, dx, g = rounding.stage(case.x, case.dout, case.layers, sh.micro_batch, sh.seq, sh.head_dim, ())
    layers = [[p] for p in case.layers]
    r_out, caches = oracle.stage_fwd(case.x, layers, sh.micro_batch, sh.seq, sh.head_dim)
    r_dx, r_g = oracle.stage_bwd(case.dout, caches, layers)
    assert np.allclose(out, r_out, atol=1e-11) and np.allclose(dx, r_dx, atol=1e-10)
    for l in range(2):
        for k in r_g[l][0]:
            assert np.allclose(g[l][k], r_g[l][0][k], rtol=1e-9, atol=1e-10), (l, k)


@pytest.mark.parametrize("mode", ["bf16", "bf16qk"])
def test_rounding_is_applied_and_stays_within_the_normwise_bar(mode):
    case = _case()
    sh = case.shape
    args = (case.x, case.dout, case.layers, sh.micro_batch, sh.seq, sh.head_dim)
    ref, mod = rounding.layer(*args, ()), rounding.layer(*args, rounding.MODES[mode])
    r = [rounding.ratios(mod[0], ref[0]), rounding.ratios(mod[1], ref[1])]
    r += [rounding.ratios(mod[2][0][k], ref[2][0][k]) for k in ref[2][0]]
    assert all(x[1] < 2e-2 for x in r)
    assert max(x[1] for x in r) > 1e-4  # the roundings are really applied
    # the modes differ only in how U reaches the QKV product and Q, K reach the logits
    assert rounding.BF16 - rounding.BF16_QK == {"u_qkv", "qk_fwd"}
    assert rounding.BF16_QK - rounding.BF16 == {"u_pair", "qk_pair"}


def test_compensated_qk_is_more_accurate_than_plain_bf16():
    """The hi/lo treatment of U and Q, K lowers the error of the attention gradients once
    the logits are large (W_qkv x 4, exact in bf16: logits x 16)."""
    case = _case()
    case.layers[0]["w_qkv"] = case.layers[0]["w_qkv"] * 4
    sh = case.shape
    args = (case.x, case.dout, case.layers, sh.micro_batch, sh.seq, sh.head_dim)
    ref = rounding.layer(*args, ())
    qk, plain = rounding.layer(*args, rounding.BF16_QK), rounding.layer(*args, rounding.BF16)
    for k in ("w_qkv",):
        assert rounding.ratios(qk[2][0][k], ref[2][0][k])[1] < rounding.ratios(plain[2][0][k], ref[2][0][k])[1]
    assert rounding.ratios(qk[1], ref[1])[1] < rounding.ratios(plain[1], ref[1])[1]


def test_stored_predictions_are_the_models():
    """An entry of tests/golden/precision_ceilings.json recomputed from the model."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "make_precision_ceilings", os.path.join(ROOT, "tests", "golden", "make_precision_ceilings.py"))
    gen = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(gen)
    with open(gen.OUT) as f:
        stored = json.load(f)
    for key in gen.KEYS:
        assert key in stored, f"{key} missing: run tests/golden/make_precision_ceilings.py {key}"
    fresh = gen.predict("gpt_h1024:bf16")
    for k, v in stored["gpt_h1024:bf16"].items():
        assert np.allclose(fresh[k], v, rtol=1e-4, atol=1e-6), k
