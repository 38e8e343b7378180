"""The GeLU epilogues evaluate erf by Abramowitz & Stegun's formula 7.1.26 (device code,
tensor_layer_gemms_amd/csrc/device_common.hpp). This CPU check reads the six constants
from that source and verifies, in float32 as the kernels compute, that the formula stays
within its published bound of the exact erf (1.5e-7, plus fp32 rounding near the
cancellation at small |x|), so a mistyped coefficient fails here as well as in the GPU
parity tests of the GeLU layers."""
import math
import os
import re

import numpy as np

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "tensor_layer_gemms_amd", "csrc",
                   "device_common.hpp")


def _constants():
    text = open(SRC).read()
    body = text[text.index("float erf_as("):]
    body = body[:body.index("}")]
    p = float(re.search(r"1\.0f \+ ([0-9.]+)f \* ax", body).group(1))
    poly = body[body.index("poly ="):]
    a = [float(v) for v in re.findall(r"(-?[0-9]\.[0-9]+)f", poly[:poly.index(";")])]
    return p, a


def test_erf_constants_are_the_published_ones_within_the_bound():
    p, a = _constants()
    assert p == 0.3275911 and len(a) == 5
    assert a == [0.254829592, -0.284496736, 1.421413741, -1.453152027, 1.061405429]
    x = np.linspace(-6, 6, 120001).astype(np.float32)
    ax = np.abs(x)
    f = np.float32
    t = f(1) / (f(1) + f(p) * ax)
    poly = t * (f(a[0]) + t * (f(a[1]) + t * (f(a[2]) + t * (f(a[3]) + t * f(a[4])))))
    r = np.copysign(f(1) - poly * np.exp(-ax * ax), x)
    ref = np.array([math.erf(float(v)) for v in x])
    err = np.abs(r.astype(np.float64) - ref)
    assert err.max() <= 1.5e-7 + 4 * 2.0 ** -23  # published bound + fp32 rounding of 1 - poly e
    # GeLU and GeLU' built on it: absolute errors far below bf16 rounding and the fp32 bar
    a_ = x.astype(np.float64) * math.sqrt(2)
    assert np.abs(0.5 * a_ * (1 + r) - 0.5 * a_ * (1 + ref)).max() < 1e-6
