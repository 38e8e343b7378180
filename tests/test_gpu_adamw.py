"""GPU parity of the fused AdamW step (mt_adamw_step, through the C ABI) against the
fp64 oracle (oracle.adamw_step), on seeded inputs.

Bound, elementwise, derived from the kernel's fp32 arithmetic (u = 2^-24, each
operation rounds once; the hyperparameters are passed to the oracle as the float32
values the kernel receives; bias corrections are computed in double on the host):
  m:  |m_gpu - m| <= 4u (|b1 m0| + |(1 - b1) g|)
  v:  |v_gpu - v| <= 4u (b2 v0 + (1 - b2) g^2)            (no cancellation: all terms >= 0)
  p:  |p_gpu - p| <= 4u (|p0| + |p|) + 2 s (tol_m + 8u |m|) / den,
      s = lr / (1 - b1^t), den = sqrt(v / (1 - b2^t)) + eps
      (the step term's relative error is at most that of m plus ~8u from sqrt, the
      scaling, eps, the division and the product; the factor 2 is margin)
  bf16 copy: within half a bf16 ulp (<= 2^-8 relative) of p_gpu, so
      |q - p| <= 2^-8 (|p| + tol_p) + tol_p.
"""
import numpy as np
import pytest

import oracle
import seeded_inputs as si
from gpu_support import log

pytestmark = pytest.mark.gpu
U = 2.0 ** -24


def _f32(x):
    return float(np.float32(x))


def _hp(**over):
    hp = dict(si.ADAM_HPARAMS)
    hp.update(over)
    for k in ("lr", "beta1", "beta2", "eps", "weight_decay", "grad_scale"):
        hp[k] = _f32(hp[k])
    return hp


def _run_gpu(p, g, m, v, hp, bf16_copy=True):
    import torch
    import tensor_layer_gemms_amd as mt
    tp, tg, tm, tv = (torch.from_numpy(a).to("cuda") for a in (p, g, m, v))
    q = torch.empty(p.size, dtype=torch.bfloat16, device="cuda") if bf16_copy else None
    mt.adamw_step(tp, tg, tm, tv, q, **hp)
    torch.cuda.synchronize()
    return tp, tm, tv, q


def _check(idx, p0, g, m0, v0, tp, tm, tv, q, hp):
    import torch
    sel = lambda a: np.asarray(a, dtype=np.float64)[idx]  # noqa: E731
    p0, g, m0, v0 = sel(p0), sel(g), sel(m0), sel(v0)
    p, m, v = oracle.adamw_step(p0, g, m0, v0, **hp)
    g = g * hp["grad_scale"]  # the gradient the moments see, for the bounds
    ti = torch.from_numpy(np.asarray(idx, dtype=np.int64)).to("cuda")
    got = lambda t: t.index_select(0, ti).to(torch.float64).cpu().numpy()  # noqa: E731
    pg, mg, vg = got(tp), got(tm), got(tv)
    b1, b2, t = hp["beta1"], hp["beta2"], hp["step"]
    tol_m = 4 * U * (np.abs(b1 * m0) + np.abs((1 - b1) * g))
    tol_v = 4 * U * (b2 * v0 + (1 - b2) * g * g)
    s = hp["lr"] / (1 - b1 ** t)
    den = np.sqrt(v / (1 - b2 ** t)) + hp["eps"]
    tol_p = 4 * U * (np.abs(p0) + np.abs(p)) + 2 * s * (tol_m + 8 * U * np.abs(m)) / den
    for name, a, b, tol in (("m", mg, m, tol_m), ("v", vg, v, tol_v), ("p", pg, p, tol_p)):
        err = np.abs(a - b)
        ratio = float(np.max(err / tol)) if err.size else 0.0
        log(f"  {name}: max err {err.max() if err.size else 0:.3e}  max err/bound {ratio:.3f}")
        assert np.all(err <= tol), f"{name}: {int(np.sum(err > tol))} of {err.size} outside the bound"
    if q is not None:
        qg = got(q)
        tol_q = 2.0 ** -8 * (np.abs(p) + tol_p) + tol_p
        assert np.all(np.abs(qg - p) <= tol_q), "bf16 copy outside half an ulp of p"


@pytest.mark.parametrize("n,step,wd,gs,copy", [
    (1, 1, 0.1, 1.0, True),
    (3, 1000, 0.1, 1.0, True),
    (8, 2, 0.0, 1.0, False),
    (13, 1000, 0.1, 0.5, True),
    (4099, 1, 0.1, 1.0, True),
    (1 << 20 | 5, 1000, 0.1, 1.0, True),
    (1 << 20 | 5, 7, 0.0, 2.0, False),
])
def test_adamw_matches_oracle(n, step, wd, gs, copy):
    log(f"[adamw] n={n} step={step} wd={wd} grad_scale={gs} bf16_copy={copy}")
    p, g, m, v = si.adam_case(n, seed=n % 97)
    hp = _hp(step=step, weight_decay=wd, grad_scale=gs)
    tp, tm, tv, q = _run_gpu(p, g, m, v, hp, copy)
    _check(np.arange(n), p, g, m, v, tp, tm, tv, q, hp)


def test_adamw_full_shard_sampled():
    """The 175B tp=8 shard's parameter count in one flat buffer (the launch bench.py
    times): 200k sampled parameters plus both ends and the ragged tail."""
    shape = si.WORKLOADS["gpt175b_tp8"].shape
    n = si.shard_param_count(shape)
    log(f"[adamw] full shard n={n}")
    p, g, m, v = si.adam_case(n, seed=0)
    hp = _hp()
    tp, tm, tv, q = _run_gpu(p, g, m, v, hp, True)
    rng = np.random.default_rng(5)
    idx = np.unique(np.concatenate([np.arange(1000), np.arange(n - 1000, n), rng.integers(0, n, 200000)]))
    _check(idx, p, g, m, v, tp, tm, tv, q, hp)


def test_adamw_rejects_bad_arguments_before_launch():
    import torch
    import tensor_layer_gemms_amd as mt
    log("[adamw] invalid arguments")
    p, g, m, v = (torch.zeros(64, device="cuda") for _ in range(4))
    hp = _hp()
    for over in (dict(step=0), dict(beta1=1.0), dict(beta2=-0.5)):
        with pytest.raises(mt.MTError) as e:
            mt.adamw_step(p, g, m, v, **dict(hp, **over))
        assert e.value.status == mt.MT_ERR_INVALID_ARG
    with pytest.raises(mt.MTError) as e:  # 4-byte offset: misaligned, rejected on the host
        mt.adamw_step(p[1:], g[1:], m[1:], v[1:], **hp)
    assert e.value.status == mt.MT_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert float(p.abs().sum()) == 0.0  # nothing ran
    e0 = torch.zeros(0, device="cuda")
    mt.adamw_step(e0, e0, e0, e0, **hp)  # n == 0: no-op
