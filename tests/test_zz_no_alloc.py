"""mt_mlp_bwd_noalloc (the MLP backward with its scratch in the library's static device
array) against mt_mlp_bwd (caller workspace) through the C ABI: the same kernels, so
every output must be bit-identical (which is stricter than any tolerance); the fp32
shapes also against the fp64 oracle at the literal 1e-4 bar. Two calls in a row, the
second on a smaller shape, so the second runs on scratch that still holds the first
call's values."""
import numpy as np
import pytest

import oracle
import seeded_inputs as si
from gpu_support import TOL, compare, log, to_dev, to_np

pytestmark = pytest.mark.gpu


def _run(shape, case, p, noalloc: bool):
    import torch
    import tensor_layer_gemms_amd as mt
    from gpu_support import mt_shape
    sh = mt_shape(shape)
    dt = shape.dtype
    xd, dyd = to_dev(case.x, dt), to_dev(case.dout, dt)
    w1, b1, w2 = to_dev(p["w_fc1"], dt), to_dev(p["b_fc1"], dt), to_dev(p["w_fc2"], dt)
    ft = 4 * shape.h // shape.tp
    assert w1.numel() == ft * shape.h and w2.numel() == ft * shape.h and b1.numel() == ft
    assert xd.numel() == shape.tokens * shape.h and dyd.numel() == xd.numel()
    saved = torch.empty(mt.mlp_saved_bytes(sh), dtype=torch.uint8, device="cuda")
    y, dx = torch.empty_like(xd), torch.empty_like(xd)
    dw1 = torch.empty(p["w_fc1"].shape, dtype=torch.float32, device="cuda")
    db1 = torch.empty(p["b_fc1"].shape, dtype=torch.float32, device="cuda")
    dw2 = torch.empty(p["w_fc2"].shape, dtype=torch.float32, device="cuda")
    mt.mlp_fwd(sh, xd, w1, b1, w2, y, saved)
    if noalloc:
        assert mt.mlp_workspace_bytes(sh) <= mt.NOALLOC_SCRATCH_BYTES
        mt.mlp_bwd_noalloc(sh, xd, w1, w2, saved, dyd, dx, dw1, db1, dw2)
    else:
        ws = torch.empty(mt.mlp_workspace_bytes(sh), dtype=torch.uint8, device="cuda")
        mt.mlp_bwd(sh, xd, w1, w2, saved, dyd, dx, dw1, db1, dw2, ws)
    torch.cuda.synchronize()
    return {"dx": to_np(dx), "w_fc1": to_np(dw1), "b_fc1": to_np(db1), "w_fc2": to_np(dw2)}


SHAPES = {
    # the 175B shard's MLP block (27 MiB of scratch), then a smaller ragged one
    "bf16": [si.LayerShape(h=12288, heads=96, seq=2048, micro_batch=1, tp=8, shard=0),
             si.LayerShape(h=528, heads=6, seq=72, micro_batch=3, tp=2, shard=1)],
    "fp32": [si.LayerShape(h=256, heads=4, seq=200, micro_batch=2, tp=2, shard=0, dtype="fp32"),
             si.LayerShape(h=64, heads=4, seq=32, micro_batch=2, tp=1, dtype="fp32")],
}


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_mlp_bwd_noalloc_matches_workspace_call(dtype):
    for i, shape in enumerate(SHAPES[dtype]):
        log(f"[noalloc] call {i}: {shape}")
        if shape.h >= 4096:
            case = si.make_case(shape, seed=11 + i)
        else:
            case = si.mlp_case(shape, seed=11 + i, random_bias=True)
        p = case.layers[0]
        got = _run(shape, case, p, noalloc=True)
        ref = _run(shape, case, p, noalloc=False)
        for k in ref:
            assert np.array_equal(got[k], ref[k]), f"call {i} {k}: differs from mt_mlp_bwd"
        if dtype == "fp32":  # also against the oracle, literal bar
            y_ref, c = oracle.mlp_fwd(case.x, [p])
            dx_ref, g_ref = oracle.mlp_bwd(case.dout, c, [p])
            assert compare("dx", got["dx"], dx_ref, TOL["fp32"])[0]
            for k in ("w_fc1", "b_fc1", "w_fc2"):
                assert compare(k, got[k], g_ref[0][k], TOL["fp32"])[0]


def test_mlp_bwd_noalloc_rejects_oversized_shape():
    """A shape whose scratch exceeds the static array is refused before any launch."""
    import torch
    import tensor_layer_gemms_amd as mt
    sh = mt.make_shape(8192, 64, 2048, 8, 8, 0, "bf16")  # 132 MiB of scratch
    assert mt.mlp_workspace_bytes(sh) > mt.NOALLOC_SCRATCH_BYTES
    buf = torch.empty(1024, dtype=torch.uint8, device="cuda")
    p = buf.data_ptr()
    st = mt.lib().mt_mlp_bwd_noalloc(sh, p, p, p, p, mt.mlp_saved_bytes(sh), p, p, p, p, p,
                                     torch.cuda.current_stream().cuda_stream)
    assert st == mt.MT_ERR_NOALLOC_LIMIT
