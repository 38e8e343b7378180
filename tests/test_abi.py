"""C-ABI checks that need no GPU: the library loads, exports every symbol include/mt.h
declares, sizes its buffers consistently and rejects bad arguments with the documented
status before launching anything (every call below fails validation on the host)."""
import ctypes
import os
import re
import subprocess

import pytest

import tensor_layer_gemms_amd as mt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mt.LIB_PATH):
        from tensor_layer_gemms_amd.build import build
        build(verbose=False)
    return mt.lib()


def _declared():
    text = open(os.path.join(ROOT, "include", "mt.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mt_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    declared = _declared()
    assert "mt_layer_fwd" in declared and "mt_mlp_bwd" in declared
    out = subprocess.run(["nm", "-D", "--defined-only", mt.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (mt_\w+)", out))
    missing = [s for s in declared if s not in exported]
    assert not missing, missing
    assert set(declared) == set(mt.EXPORTED), "binding signatures must cover the header"


def _shape(**kw):
    base = dict(h=1024, heads=16, seq=1024, micro_batch=4, tp=1, shard=0, dtype="bf16")
    base.update(kw)
    if isinstance(base["dtype"], int):  # a raw mt_dtype value, past the binding's check
        return mt.Shape(*(base[k] for k in ("h", "heads", "seq", "micro_batch", "tp", "shard", "dtype")))
    return mt.make_shape(**base)


def test_buffer_queries_consistent(lib):
    s = _shape()  # head dim 64: fused attention
    M, h, f, a, seq, B = 4096, 1024, 4096, 16, 1024, 4
    saved = mt.layer_saved_bytes(s)
    # U, QKV, ctx, V2, A, Z in bf16, the fp32 residual X2, four fp32 row statistics and
    # the fp32 row log-sum-exp (no P)
    need = 2 * (M * h + M * 3 * h + M * h + M * h + 2 * M * f) + 4 * M * h + 16 * M + 4 * B * a * seq
    assert need <= saved <= need + 64 * 256
    # MT_BF16_QK also saves the Q/K rounding remainders (QKV layout) and needs the fp32
    # partials of the two QKV products and U's remainder in the workspace
    sq = _shape(dtype="bf16qk")
    need_q = need + 2 * M * 3 * h
    assert need_q <= mt.layer_saved_bytes(sq) <= need_q + 64 * 256
    assert mt.layer_workspace_bytes(sq) >= 4 * M * (3 * h + 2 * h) + 2 * M * h
    assert mt.layer_workspace_bytes(s) <= mt.layer_workspace_bytes(sq)
    # head dim 160 is fused too (row log-sum-exp, no P)
    s160 = _shape(h=640, heads=4, seq=256, micro_batch=2)
    M1, h1, f1, a1, q1, B1 = 512, 640, 2560, 4, 256, 2
    need160 = 2 * (M1 * h1 + M1 * 3 * h1 + M1 * h1 + M1 * h1 + 2 * M1 * f1) + 4 * M1 * h1 + 16 * M1 + 4 * B1 * a1 * q1
    assert need160 <= mt.layer_saved_bytes(s160) <= need160 + 64 * 256
    # head dim 96 keeps the materialised attention: P (bf16) in the saved store, fp32
    # scores in the workspace
    s96 = _shape(h=384, heads=4, seq=256, micro_batch=2)
    M2, h2, f2, a2, q2 = 512, 384, 1536, 4, 256
    need96 = 2 * (M2 * h2 * 2 + M2 * 3 * h2 + 2 * a2 * q2 * q2 + M2 * h2 + 2 * M2 * f2) + 4 * M2 * h2 + 16 * M2
    assert need96 <= mt.layer_saved_bytes(s96) <= need96 + 64 * 256
    assert mt.layer_workspace_bytes(s96) >= 4 * 2 * a2 * q2 * q2
    assert mt.mlp_saved_bytes(s) == 2 * 2 * M * f
    s8 = _shape(h=12288, heads=96, seq=2048, micro_batch=1, tp=8)
    s8b = _shape(h=12288, heads=96, seq=2048, micro_batch=1, tp=8, shard=7)
    assert mt.layer_saved_bytes(s8) == mt.layer_saved_bytes(s8b) > 0
    assert mt.layer_saved_bytes(_shape(dtype="fp32")) > saved


@pytest.mark.parametrize("kw,status", [
    (dict(heads=12), mt.MT_ERR_INVALID_ARG),            # h % heads
    (dict(tp=3), mt.MT_ERR_INVALID_ARG),                # heads % tp
    (dict(tp=2, shard=2), mt.MT_ERR_INVALID_ARG),       # shard out of range
    (dict(shard=-1), mt.MT_ERR_INVALID_ARG),
    (dict(seq=1020), mt.MT_ERR_UNSUPPORTED),            # seq % 8
    (dict(seq=8192), mt.MT_ERR_UNSUPPORTED),            # beyond the softmax row limit
    (dict(h=1028, heads=257), mt.MT_ERR_UNSUPPORTED),   # head dim 4
    (dict(h=65536, heads=512), mt.MT_ERR_UNSUPPORTED),  # LayerNorm row limit
    (dict(micro_batch=0), mt.MT_ERR_INVALID_ARG),
    (dict(dtype=3), mt.MT_ERR_INVALID_ARG),             # no such mt_dtype
])
def test_bad_shapes_rejected(lib, kw, status):
    s = _shape(**kw)
    assert mt.layer_saved_bytes(s) == 0 and mt.layer_workspace_bytes(s) == 0
    w = mt.LayerWeights(*([0x1000] * 12))
    rc = lib.mt_layer_fwd(ctypes.byref(s), ctypes.byref(w), 0x1000, 0x1000, 0x1000, 1 << 40, 0x1000, 1 << 40, None)
    assert rc == status


def test_null_and_misaligned_pointers_rejected(lib):
    s = _shape()
    good = [0x10000] * 12
    for i in range(12):
        bad = list(good)
        bad[i] = 0
        w = mt.LayerWeights(*bad)
        assert lib.mt_layer_fwd(ctypes.byref(s), ctypes.byref(w), 0x1000, 0x1000, 0x1000, 1 << 40, 0x1000, 1 << 40,
                                None) == mt.MT_ERR_INVALID_ARG
    w = mt.LayerWeights(*good)
    assert lib.mt_layer_fwd(ctypes.byref(s), ctypes.byref(w), 0x1008, 0x1000, 0x1000, 1 << 40, 0x1000, 1 << 40,
                            None) == mt.MT_ERR_INVALID_ARG
    assert lib.mt_layer_fwd(None, ctypes.byref(w), 0x1000, 0x1000, 0x1000, 1 << 40, 0x1000, 1 << 40,
                            None) == mt.MT_ERR_INVALID_ARG
    assert lib.mt_mlp_fwd(ctypes.byref(s), 0, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 1 << 40, None, 0,
                          None) == mt.MT_ERR_INVALID_ARG
    g = mt.LayerGrads(*([0x1000] * 11 + [0]))
    assert lib.mt_layer_bwd(ctypes.byref(s), ctypes.byref(w), 0x1000, 0x1000, 1 << 40, 0x1000, 0x1000, ctypes.byref(g),
                            0x1000, 1 << 40, None) == mt.MT_ERR_INVALID_ARG


def test_small_buffers_rejected(lib):
    s = _shape()
    w = mt.LayerWeights(*([0x1000] * 12))
    g = mt.LayerGrads(*([0x1000] * 12))
    saved, ws = mt.layer_saved_bytes(s), mt.layer_workspace_bytes(s)
    assert lib.mt_layer_fwd(ctypes.byref(s), ctypes.byref(w), 0x1000, 0x1000, 0x1000, saved - 1, 0x1000, ws,
                            None) == mt.MT_ERR_WORKSPACE
    assert lib.mt_layer_fwd(ctypes.byref(s), ctypes.byref(w), 0x1000, 0x1000, 0x1000, saved, 0x1000, ws - 1,
                            None) == mt.MT_ERR_WORKSPACE
    assert lib.mt_layer_bwd(ctypes.byref(s), ctypes.byref(w), 0x1000, 0x1000, saved - 256, 0x1000, 0x1000,
                            ctypes.byref(g), 0x1000, ws, None) == mt.MT_ERR_WORKSPACE
    ms = mt.mlp_saved_bytes(s)
    assert lib.mt_mlp_fwd(ctypes.byref(s), 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, ms - 1, None, 0,
                          None) == mt.MT_ERR_WORKSPACE
    mw = mt.mlp_workspace_bytes(s)
    assert lib.mt_mlp_bwd(ctypes.byref(s), 0x1000, 0x1000, 0x1000, 0x1000, ms, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000,
                          0x1000, mw - 1, None) == mt.MT_ERR_WORKSPACE


def test_status_strings_and_timing_api(lib):
    for st in range(5):
        assert len(mt.status_string(st)) >= 2
    assert "unknown" in mt.status_string(99)
    mt.timing_enable(True, "fc1")
    mt.timing_enable(False)
    mt.timing_reset()
    assert mt.timing_records() == []
    assert lib.mt_timing_get(0, None, 0, None, None, None) == mt.MT_ERR_INVALID_ARG


def test_binding_rejects_mismatched_tensors():
    torch = pytest.importorskip("torch")
    s = _shape(h=64, heads=4, seq=32, micro_batch=2, dtype="fp32")
    w = {k: torch.zeros(v) for k, v in mt.weight_shapes(s).items()}
    with pytest.raises(ValueError):
        mt.check_layer_tensors(s, w)  # host tensors are not device buffers


def test_attention_block_and_sp_queries(lib):
    """Buffer queries of the attention block and the sequence-parallel row calls: the
    attention store holds at least the projections and the context; MT_BF16_QK and a
    sequence that does not split evenly over tp are refused (size 0)."""
    sh = _shape(h=256, heads=4, seq=64, micro_batch=2, tp=2)
    M, ht = 2 * 64, 256 // 2
    assert lib.mt_attn_saved_bytes(ctypes.byref(sh)) >= M * 3 * ht * 2 + M * ht * 2
    assert lib.mt_attn_workspace_bytes(ctypes.byref(sh)) > 0
    assert lib.mt_sp_ln_workspace_bytes(ctypes.byref(sh)) > 0
    qk = _shape(h=256, heads=4, seq=64, micro_batch=2, tp=2, dtype=mt.MT_BF16_QK)
    assert lib.mt_attn_saved_bytes(ctypes.byref(qk)) == 0
    assert lib.mt_attn_workspace_bytes(ctypes.byref(qk)) == 0
    assert lib.mt_sp_ln_workspace_bytes(ctypes.byref(qk)) == 0
    uneven = _shape(h=384, heads=6, seq=72, micro_batch=1, tp=3)  # 72 % 3 == 0: accepted
    assert lib.mt_sp_ln_workspace_bytes(ctypes.byref(uneven)) > 0
    uneven = _shape(h=256, heads=8, seq=72, micro_batch=1, tp=8)  # 72 % 8 == 0
    assert lib.mt_sp_ln_workspace_bytes(ctypes.byref(uneven)) > 0
    uneven = _shape(h=256, heads=16, seq=72, micro_batch=1, tp=16)  # 72 % 16 != 0
    assert lib.mt_sp_ln_workspace_bytes(ctypes.byref(uneven)) == 0


def test_attention_block_and_sp_reject_bad_arguments(lib):
    """Null or misaligned pointers, small buffers, MT_BF16_QK and an uneven sequence split
    are rejected with the documented status before anything is launched."""
    sh = _shape(h=256, heads=4, seq=64, micro_batch=2, tp=2)
    A = 1 << 20  # an aligned host address (never dereferenced: validation fails first)
    big = 1 << 40
    attn_fwd = lib.mt_attn_fwd
    assert attn_fwd(ctypes.byref(sh), 0, A, A, A, A, A, big, A, big, None) == mt.MT_ERR_INVALID_ARG
    assert attn_fwd(ctypes.byref(sh), A + 2, A, A, A, A, A, big, A, big, None) == mt.MT_ERR_INVALID_ARG
    assert attn_fwd(ctypes.byref(sh), A, A, A, A, A, A, 16, A, big, None) == mt.MT_ERR_WORKSPACE
    assert attn_fwd(ctypes.byref(sh), A, A, A, A, A, A, big, A, 16, None) == mt.MT_ERR_WORKSPACE
    qk = _shape(h=256, heads=4, seq=64, micro_batch=2, tp=2, dtype=mt.MT_BF16_QK)
    assert attn_fwd(ctypes.byref(qk), A, A, A, A, A, A, big, A, big, None) == mt.MT_ERR_UNSUPPORTED
    assert lib.mt_attn_bwd(ctypes.byref(qk), A, A, A, A, big, A, A, A, A, A, A, big, None) == mt.MT_ERR_UNSUPPORTED
    assert lib.mt_attn_bwd(ctypes.byref(sh), A, A, A, A, big, A, A, 0, A, A, A, big, None) == mt.MT_ERR_INVALID_ARG
    # mt_sp_ln_fwd: resid given without bias / x2
    assert lib.mt_sp_ln_fwd(ctypes.byref(sh), A, A, 0, A, A, 0, A, A, A, None) == mt.MT_ERR_INVALID_ARG
    assert lib.mt_sp_ln_fwd(ctypes.byref(sh), A, 0, 0, A, A, 0, 0, A, A, None) == mt.MT_ERR_INVALID_ARG
    uneven = _shape(h=256, heads=16, seq=72, micro_batch=1, tp=16)
    assert lib.mt_sp_ln_fwd(ctypes.byref(uneven), A, 0, 0, A, A, 0, A, A, A, None) == mt.MT_ERR_INVALID_ARG
    assert lib.mt_sp_ln_fwd(ctypes.byref(qk), A, 0, 0, A, A, 0, A, A, A, None) == mt.MT_ERR_UNSUPPORTED
    assert lib.mt_sp_add_fwd(ctypes.byref(sh), A, A, 0, A, None) == mt.MT_ERR_INVALID_ARG
    # mt_sp_ln_bwd: dsum without dx_f32; small workspace
    ln_bwd = lib.mt_sp_ln_bwd
    assert ln_bwd(ctypes.byref(sh), A, A, 1, A, A, A, A, 0, A, 0, A, A, A, 0, A, big, None) == mt.MT_ERR_INVALID_ARG
    assert ln_bwd(ctypes.byref(sh), A, A, 1, A, A, A, A, 0, A, A, A, A, A, A, A, 4, None) == mt.MT_ERR_WORKSPACE


def test_mlp_bwd_noalloc_host_checks(lib):
    """mt_mlp_bwd_noalloc refuses, before touching the device, a null pointer, a small
    saved store and a shape whose scratch exceeds the static array."""
    A, big = 1 << 20, 1 << 40
    fn = lib.mt_mlp_bwd_noalloc
    over = _shape(h=8192, heads=64, seq=2048, micro_batch=8, tp=8)  # 132 MiB of scratch
    assert mt.mlp_workspace_bytes(over) > mt.NOALLOC_SCRATCH_BYTES
    assert fn(ctypes.byref(over), A, A, A, A, big, A, A, A, A, A, None) == mt.MT_ERR_NOALLOC_LIMIT
    ok = _shape(h=12288, heads=96, seq=2048, micro_batch=1, tp=8)  # 27 MiB: fits
    assert mt.mlp_workspace_bytes(ok) <= mt.NOALLOC_SCRATCH_BYTES
    assert fn(ctypes.byref(ok), A, A, 0, A, big, A, A, A, A, A, None) == mt.MT_ERR_INVALID_ARG
    assert fn(ctypes.byref(ok), A, A, A, A, mt.mlp_saved_bytes(ok) - 1, A, A, A, A, A,
              None) == mt.MT_ERR_WORKSPACE
    assert "no-alloc" in mt.status_string(mt.MT_ERR_NOALLOC_LIMIT)
