"""Pins of the fp64 AdamW oracle against things other than itself (CPU only).

The update is the textbook AdamW (Adam's bias-corrected moments, decoupled weight
decay) read from the oreateai.com Megatron-LM analysis, sections 2.2 and 3.1. Each pin
below derives its expected value independently of the oracle's formula:

* first step from zero moments: the bias-corrected moments are g and g^2, so the step
  is lr g / (|g| + eps) (the sign of g when |g| >> eps);
* a constant gradient: the bias correction turns every moment estimate into g and g^2
  exactly, so T steps move p by T lr g / (|g| + eps) (without decay);
* decay alone (g = 0, zero moments): p scales by (1 - lr wd) per step;
* Adam is invariant to the gradient's scale when eps = 0;
* torch.optim.AdamW (fp64, CPU, single-tensor loop): an implementation that shares
  nothing with the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si

HP = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


def _rng(seed=0):
    return np.random.default_rng([seed, 0xAD])


def test_first_step_is_sign_like():
    r = _rng()
    p, g = r.standard_normal(1000), r.standard_normal(1000) * 1e-3
    z = np.zeros_like(p)
    p1, m1, v1 = oracle.adamw_step(p, g, z, z, step=1, **HP)
    lr, wd, eps = HP["lr"], HP["weight_decay"], HP["eps"]
    np.testing.assert_allclose(p1, p * (1 - lr * wd) - lr * g / (np.abs(g) + eps), rtol=1e-13, atol=1e-17)
    np.testing.assert_allclose(m1, (1 - HP["beta1"]) * g, rtol=1e-14)
    np.testing.assert_allclose(v1, (1 - HP["beta2"]) * g * g, rtol=1e-14)


@pytest.mark.parametrize("beta2", [0.95, 0.999])
def test_constant_gradient_moves_linearly(beta2):
    r = _rng(1)
    p0, g = r.standard_normal(257), r.standard_normal(257) * 3e-2
    hp = dict(HP, weight_decay=0.0, beta2=beta2)
    p, m, v = p0.copy(), np.zeros_like(p0), np.zeros_like(p0)
    T = 50
    for t in range(1, T + 1):
        p, m, v = oracle.adamw_step(p, g, m, v, step=t, **hp)
    np.testing.assert_allclose(p, p0 - T * hp["lr"] * g / (np.abs(g) + hp["eps"]), rtol=1e-10, atol=1e-14)


def test_decay_alone_is_geometric():
    r = _rng(2)
    p0 = r.standard_normal(100)
    z = np.zeros_like(p0)
    p = p0.copy()
    T = 20
    for t in range(1, T + 1):
        p, _, _ = oracle.adamw_step(p, z, z, z, step=t, **HP)
    np.testing.assert_allclose(p, p0 * (1 - HP["lr"] * HP["weight_decay"]) ** T, rtol=1e-13)


def test_gradient_scale_invariance():
    r = _rng(3)
    p0 = r.standard_normal(300)
    grads = [r.standard_normal(300) for _ in range(5)]
    hp = dict(HP, eps=0.0)
    runs = []
    for c in (1.0, 1e-4, 37.0):
        p, m, v = p0.copy(), np.zeros_like(p0), np.zeros_like(p0)
        for t, g in enumerate(grads, 1):
            p, m, v = oracle.adamw_step(p, c * g, m, v, step=t, **hp)
        runs.append(p)
    np.testing.assert_allclose(runs[1], runs[0], rtol=1e-12)
    np.testing.assert_allclose(runs[2], runs[0], rtol=1e-12)


@pytest.mark.parametrize("grad_scale", [1.0, 0.25])
def test_matches_torch_adamw_fp64(grad_scale):
    r = _rng(4)
    n = 777
    p0 = r.standard_normal(n) * 0.02
    grads = [r.standard_normal(n) * 1e-3 for _ in range(7)]
    hp = dict(lr=6e-5, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    tp = torch.tensor(p0, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([tp], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                            weight_decay=hp["weight_decay"], foreach=False)
    p, m, v = p0.copy(), np.zeros(n), np.zeros(n)
    for t, g in enumerate(grads, 1):
        tp.grad = torch.tensor(g * grad_scale, dtype=torch.float64)
        opt.step()
        p, m, v = oracle.adamw_step(p, g, m, v, step=t, grad_scale=grad_scale, **hp)
    st = opt.state[tp]
    np.testing.assert_allclose(p, tp.detach().numpy(), rtol=1e-13, atol=1e-18)
    np.testing.assert_allclose(m, st["exp_avg"].numpy(), rtol=1e-13)
    np.testing.assert_allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-13)


def test_seeded_adam_case_and_param_count():
    p, g, m, v = si.adam_case(1000, seed=0)
    assert p.dtype == g.dtype == m.dtype == v.dtype == np.float32
    assert (v > 0).all()
    p2, *_ = si.adam_case(1000, seed=0)
    assert np.array_equal(p, p2)
    shape = si.WORKLOADS["gpt175b_tp8"].shape
    # W_qkv [4608, 12288], W_o [12288, 1536], W1 [6144, 12288], W2 [12288, 6144],
    # their biases and the two LayerNorms
    expect = 4608 * 12288 + 4608 + 12288 * 1536 + 12288 + 6144 * 12288 + 6144 + 12288 * 6144 + 12288 + 4 * 12288
    assert si.shard_param_count(shape) == expect
