"""CPU checks of the bf16 rounding model used to choose the bf16 tolerance reading."""
import numpy as np
import pytest

import oracle
import seeded_inputs as si
from precision_model import BF16, BF16_QK, layer, metrics


def _case():
    shape = si.LayerShape(h=256, heads=4, seq=128, micro_batch=2, tp=2)
    return si.make_case(shape, seed=2, global_weights=True, random_affine=True)


def test_model_without_rounding_is_the_oracle():
    case = _case()
    out, dx, g = layer(case, ())
    sh = case.shape
    r_out, c = oracle.layer_fwd(case.x, case.layers, sh.micro_batch, sh.seq, sh.head_dim)
    r_dx, r_g = oracle.layer_bwd(case.dout, c, case.layers)
    assert np.allclose(out, r_out, rtol=0, atol=1e-12) and np.allclose(dx, r_dx, rtol=0, atol=1e-11)
    for k in g:
        assert np.allclose(g[k], r_g[0][k], rtol=1e-10, atol=1e-10), k


@pytest.mark.parametrize("mode", ["bf16", "bf16qk"])
def test_bf16_rounding_stays_within_normwise_bar(mode):
    case = _case()
    m = metrics(layer(case, BF16 if mode == "bf16" else BF16_QK), layer(case, ()))
    for k, (rms_rel, _, max_rel) in m.items():
        assert rms_rel < 2e-2 and max_rel < 2e-2, (k, m[k])
    assert max(v[0] for v in m.values()) > 1e-4  # the roundings are really applied


def test_compensated_qk_is_more_accurate_than_plain_bf16():
    """The hi/lo treatment of U and Q, K lowers the error of the attention gradients."""
    case = _case()
    ref = layer(case, ())
    ours, plain = metrics(layer(case, BF16_QK), ref), metrics(layer(case, BF16), ref)
    assert ours["w_qkv"][0] < plain["w_qkv"][0] and ours["dx"][0] < plain["dx"][0]
