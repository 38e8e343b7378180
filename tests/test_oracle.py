"""Pins of the fp64 oracle against things other than itself (CPU only).

* calculus: central finite differences of L = <Out, dOut> for every gradient;
* the pages' invariant ("Megatron-LM" concept report, section 4.1): the sum over
  ranks of f(X A_i) B_i equals the unsharded f(X A) B, and (section 4.2) the backward
  partials sum to the unsharded input gradient;
* brute force: per-element attention loops on the tiny shape;
* closed forms and special cases: LayerNorm of a constant row, GeLU values, the first
  causal query, a zero query projection, a zeroed residual branch;
* library: torch's fp64 CPU functional ops with autograd (an implementation that
  shares nothing with the oracle).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si

TINY = si.WORKLOADS["tiny_fp32"].shape  # h=64, 4 heads, seq 32, micro-batch 2


def _case(tp=1, random_affine=True, seed=0, **kw):
    shape = TINY.replace(tp=tp, **kw)
    return si.make_case(shape, seed=seed, global_weights=True, random_affine=random_affine)


def _shards(case, tp):
    g = case.global_layers[0]
    return [si.shard_slice(g, case.shape.replace(tp=tp), i) for i in range(tp)]


def _fwd(x, shards, shape):
    return oracle.layer_fwd(x, shards, shape.micro_batch, shape.seq, shape.head_dim)


def _rel(a, b):
    return np.max(np.abs(np.asarray(a) - np.asarray(b))) / max(np.sqrt(np.mean(np.asarray(b) ** 2)), 1e-300)


# ------------------------------------------------------------------- input generator
def test_bf16_round_matches_torch():
    rng = np.random.default_rng(3)
    a = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    a[:4] = [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 0.0]  # ties to even
    ours = si.bf16_round(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_shard_slices_partition_global_weights():
    case = _case(tp=1)
    g = case.global_layers[0]
    for tp in (2, 4):
        sh = _shards(case, tp)
        assert np.array_equal(np.concatenate([s["w_fc1"] for s in sh], 0), g["w_fc1"])
        assert np.array_equal(np.concatenate([s["w_fc2"] for s in sh], 1), g["w_fc2"])
        assert np.array_equal(np.concatenate([s["w_o"] for s in sh], 1), g["w_o"])
        assert sum(s["w_qkv"].shape[0] for s in sh) == g["w_qkv"].shape[0]


# ------------------------------------------------------------------- closed forms
def test_gelu_closed_forms_and_library():
    assert oracle.gelu(0.0) == 0.0
    assert oracle.gelu_grad(0.0) == 0.5
    x = np.linspace(-8, 8, 2001)
    assert np.allclose(oracle.gelu(-x), oracle.gelu(x) - x, rtol=0, atol=1e-15)
    assert abs(oracle.gelu(40.0) - 40.0) < 1e-12 and abs(oracle.gelu(-40.0)) < 1e-12
    assert abs(oracle.gelu(1.0) - 0.5 * (1 + math.erf(1 / math.sqrt(2)))) < 1e-16
    t = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    y = torch.nn.functional.gelu(t, approximate="none")
    y.sum().backward()
    assert np.allclose(oracle.gelu(x), y.detach().numpy(), rtol=1e-14, atol=1e-15)
    assert np.allclose(oracle.gelu_grad(x), t.grad.numpy(), rtol=1e-13, atol=1e-15)


def test_layernorm_closed_forms_and_library():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((16, 48)) * 3 + 1
    x[0] = 2.5  # constant row: xhat = 0, output = beta exactly
    g, b = 1 + 0.1 * rng.standard_normal(48), 0.1 * rng.standard_normal(48)
    y, mu, rstd = oracle.layernorm_fwd(x, g, b)
    assert np.allclose(y[0], b, rtol=0, atol=1e-12)
    assert abs(rstd[0] - 1 / math.sqrt(1e-5)) < 1e-6
    y1, _, _ = oracle.layernorm_fwd(x, np.ones(48), np.zeros(48))
    var = x.var(axis=1)
    assert np.allclose(y1.mean(axis=1), 0, atol=1e-12)
    assert np.allclose((y1 ** 2).mean(axis=1), var / (var + 1e-5), rtol=1e-12, atol=1e-12)
    ref = torch.nn.functional.layer_norm(torch.tensor(x), (48,), torch.tensor(g), torch.tensor(b), eps=1e-5)
    assert np.allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_attention_matches_brute_force_loops():
    case = _case()
    sh = case.layers[0]
    B, s, d = TINY.micro_batch, TINY.seq, TINY.head_dim
    heads = TINY.heads
    rng = np.random.default_rng(5)
    qkv = rng.standard_normal((B * s, 3 * heads * d))
    ctx, probs = oracle.attention_fwd(qkv, B, s, heads, d)
    for b in range(B):
        for k in range(heads):
            for q in range(0, s, 3):
                r = b * s + q
                logits = []
                for j in range(q + 1):
                    rj = b * s + j
                    acc = 0.0
                    for c in range(d):
                        acc += qkv[r, k * d + c] * qkv[rj, heads * d + k * d + c]
                    logits.append(acc / math.sqrt(d))
                mx = max(logits)
                w = [math.exp(v - mx) for v in logits]
                tot = sum(w)
                for j in range(s):
                    pj = w[j] / tot if j <= q else 0.0
                    assert abs(probs[b, k, q, j] - pj) < 1e-14
                for c in range(d):
                    ref = sum(w[j] / tot * qkv[b * s + j, 2 * heads * d + k * d + c] for j in range(q + 1))
                    assert abs(ctx[r, k * d + c] - ref) < 1e-13
    del sh


def test_attention_causal_first_query_and_prefix_mean():
    B, s, d, heads = 2, 32, 16, 4
    rng = np.random.default_rng(6)
    qkv = rng.standard_normal((B * s, 3 * heads * d))
    ctx, _ = oracle.attention_fwd(qkv, B, s, heads, d)
    for b in range(B):  # query 0 sees only key 0: ctx row = V row 0, exactly
        assert np.array_equal(ctx[b * s], qkv[b * s, 2 * heads * d:])
    qkv[:, :heads * d] = 0.0  # Q = 0: uniform weights over the visible prefix
    ctx, probs = oracle.attention_fwd(qkv, B, s, heads, d)
    v = qkv[:, 2 * heads * d:].reshape(B, s, heads * d)
    prefix_mean = np.cumsum(v, axis=1) / np.arange(1, s + 1)[None, :, None]
    assert np.allclose(ctx.reshape(B, s, -1), prefix_mean, rtol=1e-13, atol=1e-13)


def test_residual_wiring_zero_branches():
    case = _case()
    p = dict(case.layers[0])
    p["w_o"] = np.zeros_like(p["w_o"])
    p["w_fc2"] = np.zeros_like(p["w_fc2"])
    out, c = _fwd(case.x, [p], TINY)
    want = case.x.astype(np.float64) + p["b_o"].astype(np.float64) + p["b_fc2"].astype(np.float64)
    assert np.allclose(out, want, rtol=0, atol=1e-14)
    dx, g = oracle.layer_bwd(case.dout, c, [p])
    # No path from X to Out except the residual: dX = dOut; db_o = db_fc2 = colsum(dOut).
    assert np.allclose(dx, case.dout, rtol=0, atol=1e-13)
    assert np.allclose(g[0]["b_o"], case.dout.sum(0), atol=1e-12)
    assert np.allclose(g[0]["w_fc1"], 0) and np.allclose(g[0]["w_qkv"], 0)


# ------------------------------------------------------------------- the pages' invariant
@pytest.mark.parametrize("tp", [2, 4])
def test_mlp_tensor_parallel_invariant(tp):
    """sum_i GeLU(X W1_i^T + b1_i) W2_i^T = GeLU(X W1^T + b1) W2^T, and backward partials."""
    case = _case(tp=1)
    full = [case.global_layers[0]]
    shards = _shards(case, tp)
    y1, c1 = oracle.mlp_fwd(case.x, full)
    yt, ct = oracle.mlp_fwd(case.x, shards)
    assert _rel(yt, y1) < 1e-12
    partials = [oracle.mlp_fwd(case.x, [s])[0] for s in shards]
    assert _rel(sum(partials), y1) < 1e-12
    dx1, g1 = oracle.mlp_bwd(case.dout, c1, full)
    dxt, gt = oracle.mlp_bwd(case.dout, ct, shards)
    assert _rel(dxt, dx1) < 1e-12
    fs = TINY.ffn // tp
    for i, g in enumerate(gt):
        assert _rel(g["w_fc1"], g1[0]["w_fc1"][i * fs:(i + 1) * fs]) < 1e-12
        assert _rel(g["b_fc1"], g1[0]["b_fc1"][i * fs:(i + 1) * fs]) < 1e-12
        assert _rel(g["w_fc2"], g1[0]["w_fc2"][:, i * fs:(i + 1) * fs]) < 1e-12


@pytest.mark.parametrize("tp", [2, 4])
def test_layer_tensor_parallel_invariant(tp):
    """Heads split across ranks plus the summed partials reproduce the unsharded layer."""
    case = _case(tp=1)
    full = [case.global_layers[0]]
    shards = _shards(case, tp)
    out1, c1 = _fwd(case.x, full, TINY)
    outt, ct = _fwd(case.x, shards, TINY)
    assert _rel(outt, out1) < 1e-12
    dx1, g1 = oracle.layer_bwd(case.dout, c1, full)
    dxt, gt = oracle.layer_bwd(case.dout, ct, shards)
    assert _rel(dxt, dx1) < 1e-12
    ref = si.shard_slice  # slicing the unsharded grads like weights gives each rank's grads
    for i, g in enumerate(gt):
        want = ref(g1[0], TINY.replace(tp=tp), i)
        for k in si.PARAM_NAMES:
            assert _rel(g[k], want[k]) < 1e-11, k


# ------------------------------------------------------------------- finite differences
def _fd_check(case, shards, shape, n_entries=32, every_dx=False, seed=0, h=1e-5):
    """Central differences of L = <Out, dOut> against the analytic gradients."""
    rng = np.random.default_rng(seed)
    dout = case.dout.astype(np.float64)
    x = case.x.astype(np.float64)
    shards = [{k: v.astype(np.float64) for k, v in p.items()} for p in shards]
    out, c = _fwd(x, shards, shape)
    dx, grads = oracle.layer_bwd(dout, c, shards)

    def loss(xx, ss):
        return float(np.sum(_fwd(xx, ss, shape)[0] * dout))

    def fd_dir(which, key, direction):
        if which == "x":
            return (loss(x + h * direction, shards) - loss(x - h * direction, shards)) / (2 * h)
        plus = [dict(p) for p in shards]
        minus = [dict(p) for p in shards]
        plus[which][key] = shards[which][key] + h * direction
        minus[which][key] = shards[which][key] - h * direction
        return (loss(x, plus) - loss(x, minus)) / (2 * h)

    def check(an, fd, scale):
        assert abs(an - fd) <= 1e-6 * (abs(an) + scale), (an, fd)

    # X: every entry (or a sample) and a random direction
    rms = np.sqrt(np.mean(dx ** 2))
    idx = list(np.ndindex(*x.shape)) if every_dx else [tuple(rng.integers(0, n) for n in x.shape) for _ in range(n_entries)]
    for ij in idx:
        e = np.zeros_like(x)
        e[ij] = 1.0
        check(dx[ij], fd_dir("x", None, e), rms)
    u = rng.standard_normal(x.shape)
    check(float(np.sum(dx * u)), fd_dir("x", None, u), rms * math.sqrt(u.size))
    # every parameter tensor of every rank: random direction + sampled entries.
    # Replicated parameters: a rank's copy is shared, so perturb all ranks' copies together.
    replicated = {"ln1_g", "ln1_b", "b_o", "ln2_g", "ln2_b", "b_fc2"}
    for r in range(len(shards)):
        for key in si.PARAM_NAMES:
            if key in replicated and r > 0:
                continue
            g = grads[r][key]
            grms = np.sqrt(np.mean(g ** 2)) + 1e-12
            if key in replicated:
                def fdr(direction, key=key):
                    plus = [dict(p, **{key: p[key] + h * direction}) for p in shards]
                    minus = [dict(p, **{key: p[key] - h * direction}) for p in shards]
                    return (loss(x, plus) - loss(x, minus)) / (2 * h)
            else:
                def fdr(direction, key=key, r=r):
                    return fd_dir(r, key, direction)
            u = rng.standard_normal(g.shape)
            check(float(np.sum(g * u)), fdr(u), grms * math.sqrt(u.size))
            for _ in range(n_entries):
                ij = tuple(rng.integers(0, n) for n in g.shape)
                e = np.zeros_like(g)
                e[ij] = 1.0
                check(g[ij], fdr(e), grms)


def test_finite_differences_every_dx_tp1():
    case = _case(tp=1, random_affine=False)
    _fd_check(case, case.layers, TINY, n_entries=8, every_dx=True)


@pytest.mark.parametrize("tp,sharded,affine", [(1, False, True), (2, False, True), (2, True, True), (4, True, False)])
def test_finite_differences(tp, sharded, affine):
    """tp with sharded=False: one rank with the all-reduce as identity (what one GPU
    computes); sharded=True: all ranks with the all-reduce as the sum."""
    case = _case(tp=1, random_affine=affine)
    shards = _shards(case, tp)
    shape = TINY.replace(tp=tp)
    _fd_check(case, shards if sharded else shards[:1], shape, n_entries=16, seed=tp)


def test_finite_differences_mlp_block():
    case = _case(tp=1)
    shards = _shards(case, 2)[:1]
    x, dy = case.x.astype(np.float64), case.dout.astype(np.float64)
    y, c = oracle.mlp_fwd(x, shards)
    dx, g = oracle.mlp_bwd(dy, c, shards)
    rng = np.random.default_rng(9)
    h = 1e-5
    loss = lambda xx, ss: float(np.sum(oracle.mlp_fwd(xx, ss)[0] * dy))  # noqa: E731
    u = rng.standard_normal(x.shape)
    fd = (loss(x + h * u, shards) - loss(x - h * u, shards)) / (2 * h)
    assert abs(fd - np.sum(dx * u)) < 1e-7 * (abs(fd) + 1)
    for key in ("w_fc1", "b_fc1", "w_fc2"):
        u = rng.standard_normal(shards[0][key].shape)
        p = dict(shards[0], **{key: shards[0][key] + h * u})
        m = dict(shards[0], **{key: shards[0][key] - h * u})
        fd = (loss(x, [p]) - loss(x, [m])) / (2 * h)
        assert abs(fd - np.sum(g[0][key] * u)) < 1e-7 * (abs(fd) + 1), key


def test_finite_differences_stage():
    shape = TINY.replace(seq=16)
    case = si.make_case(shape, seed=4, layers=2, global_weights=True, random_affine=True)
    layers = [[p] for p in case.layers]
    x, dy = case.x.astype(np.float64), case.dout.astype(np.float64)
    out, caches = oracle.stage_fwd(x, layers, shape.micro_batch, shape.seq, shape.head_dim)
    dx, grads = oracle.stage_bwd(dy, caches, layers)
    loss = lambda xx, ll: float(np.sum(oracle.stage_fwd(xx, ll, shape.micro_batch, shape.seq, shape.head_dim)[0] * dy))  # noqa: E731
    rng = np.random.default_rng(2)
    h = 1e-5
    u = rng.standard_normal(x.shape)
    fd = (loss(x + h * u, layers) - loss(x - h * u, layers)) / (2 * h)
    assert abs(fd - np.sum(dx * u)) < 1e-6 * (abs(fd) + 1)
    for l in range(2):
        for key in ("w_qkv", "w_fc1", "ln2_g"):
            u = rng.standard_normal(layers[l][0][key].shape)
            lp = [[dict(s[0])] for s in layers]
            lm = [[dict(s[0])] for s in layers]
            lp[l][0][key] = layers[l][0][key] + h * u
            lm[l][0][key] = layers[l][0][key] - h * u
            fd = (loss(x, lp) - loss(x, lm)) / (2 * h)
            assert abs(fd - np.sum(grads[l][0][key] * u)) < 1e-6 * (abs(fd) + 1), (l, key)


# ------------------------------------------------------------------- torch cross-check
def _torch_layer(x, p, B, s, d):
    """The same layer written with torch's fp64 CPU functional ops (a library path)."""
    F = torch.nn.functional
    h = x.shape[1]
    u = F.layer_norm(x, (h,), p["ln1_g"], p["ln1_b"], eps=1e-5)
    qkv = F.linear(u, p["w_qkv"], p["b_qkv"])
    hd = qkv.shape[1] // 3
    nh = hd // d
    q, k, v = (qkv[:, i * hd:(i + 1) * hd].reshape(B, s, nh, d).transpose(1, 2) for i in range(3))
    ctx = F.scaled_dot_product_attention(q, k, v, is_causal=True)
    ctx = ctx.transpose(1, 2).reshape(B * s, hd)
    x2 = x + F.linear(ctx, p["w_o"]) + p["b_o"]
    v2 = F.layer_norm(x2, (h,), p["ln2_g"], p["ln2_b"], eps=1e-5)
    z = F.gelu(F.linear(v2, p["w_fc1"], p["b_fc1"]), approximate="none")
    return x2 + F.linear(z, p["w_fc2"]) + p["b_fc2"]


@pytest.mark.parametrize("tp", [1, 2])
def test_matches_torch_fp64_autograd(tp):
    case = _case(tp=1, random_affine=True, seed=11)
    shape = TINY.replace(tp=tp)
    p = _shards(case, tp)[0]
    out, c = _fwd(case.x, [p], shape)
    dx, g = oracle.layer_bwd(case.dout, c, [p])
    tx = torch.tensor(case.x, dtype=torch.float64, requires_grad=True)
    tp_ = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in p.items()}
    tout = _torch_layer(tx, tp_, shape.micro_batch, shape.seq, shape.head_dim)
    tout.backward(torch.tensor(case.dout, dtype=torch.float64))
    assert _rel(out, tout.detach().numpy()) < 1e-12
    assert _rel(dx, tx.grad.numpy()) < 1e-11
    for k in si.PARAM_NAMES:
        assert _rel(g[0][k], tp_[k].grad.numpy()) < 1e-11, k


def test_keyed_streams_are_independent():
    """Shard-local inputs come from distinct streams (NumPy pads seed words with zeros,
    so [0] and [0, 0, 0, 0] would otherwise collide and correlate X with the weights)."""
    shape = si.LayerShape(h=256, heads=4, seq=64, micro_batch=2, tp=2)
    case = si.make_case(shape, seed=0)
    w = case.layers[0]["w_qkv"] / si.WEIGHT_STD
    n = min(case.x.shape[0], w.shape[0])
    corr = np.sum(case.x[:n] * w[:n], axis=1) / shape.h
    assert np.max(np.abs(corr)) < 0.35
    assert not np.allclose(case.x[0, :8], case.dout[0, :8])
    heads = [si.keyed_rng(0, p, l, r, t).standard_normal(4).tobytes()
             for p in (1, 2, 3) for l in (0, 1) for r in (0, 1) for t in (0, 1, 2)]
    assert len(set(heads)) == len(heads)
