"""Seeded synthetic inputs for the tensor-parallel GPT layer shard.

This module is the ONLY code shared between the HIP path's tests/bench and the fp64
oracle. It holds no arithmetic of the layer: it draws seeded Gaussian tensors, rounds
them to bfloat16-representable values, and slices global weights into the per-shard
pieces that one tensor-parallel rank owns.

Workloads (all synthetic; the pages measure on no dataset):
  * the tensor-parallel split follows the "Megatron-LM" concept report
    (compassingai.com), section 4.1: the first weight of a block is split by columns
    (output features), the second by rows (input features), attention heads are
    split across ranks;
  * the shapes are GPT shapes named by model size on the study-notes page
    "Efficient Large-Scale Language Model Training on GPU Clusters Using Megatron-LM"
    (knowledgebase-35y.pages.dev), section on main results (175B, 1T models).

Layouts (row-major, torch ``nn.Linear`` convention ``W[out, in]``):
  x, dout        [micro_batch * seq, h]           token rows, batch-major
  w_qkv          [3h/tp, h]  rows = [Q heads | K heads | V heads] of the shard
  b_qkv          [3h/tp]
  w_o            [h, h/tp]   (row-parallel: the shard's slice of input features)
  b_o            [h]         replicated, added after the all-reduce point
  w_fc1, b_fc1   [4h/tp, h], [4h/tp]
  w_fc2          [h, 4h/tp]
  b_fc2          [h]         replicated
  ln1_g, ln1_b, ln2_g, ln2_b  [h]
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

WEIGHT_STD = 0.02

PARAM_NAMES = (
    "ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_o", "b_o",
    "ln2_g", "ln2_b", "w_fc1", "b_fc1", "w_fc2", "b_fc2",
)


@dataclasses.dataclass(frozen=True)
class LayerShape:
    """One tensor-parallel shard of a GPT layer (global h and heads)."""

    h: int
    heads: int
    seq: int
    micro_batch: int
    tp: int = 1
    shard: int = 0
    dtype: str = "bf16"  # "bf16" or "fp32"
    # bf16 only: the attention logits from hi + lo bf16 pairs of Q and K (MT_BF16_QK)
    qk_pairs: bool = False

    @property
    def tokens(self) -> int:
        return self.micro_batch * self.seq

    @property
    def head_dim(self) -> int:
        return self.h // self.heads

    @property
    def heads_per_shard(self) -> int:
        return self.heads // self.tp

    @property
    def ffn(self) -> int:
        return 4 * self.h

    @property
    def ffn_per_shard(self) -> int:
        return self.ffn // self.tp

    @property
    def qkv_per_shard(self) -> int:
        return 3 * self.h // self.tp

    def replace(self, **kw) -> "LayerShape":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    shape: LayerShape
    layers: int = 1
    # True: draw the global (unsharded) weights and slice the shard out of them;
    # False: draw the shard-local weights directly (the global tensors of the big
    # shapes are 8x larger and never needed).
    global_weights: bool = False
    description: str = ""


WORKLOADS: Dict[str, Workload] = {
    "tiny_fp32": Workload(
        "tiny_fp32",
        LayerShape(h=64, heads=4, seq=32, micro_batch=2, tp=1, dtype="fp32"),
        global_weights=True,
        description="tiny fp32 layer, FC1 64->256, FC2 256->64; also split tp=2",
    ),
    "gpt_h1024": Workload(
        "gpt_h1024",
        LayerShape(h=1024, heads=16, seq=1024, micro_batch=4, tp=1),
        global_weights=True,
        description="GPT layer h=1024, 16 heads of 64, seq 1024, micro-batch 4, bf16",
    ),
    "gpt175b_tp8": Workload(
        "gpt175b_tp8",
        LayerShape(h=12288, heads=96, seq=2048, micro_batch=1, tp=8),
        description="GPT-175B layer shape, shard 0 of tp=8: 12 heads of 128, seq 2048",
    ),
    "gpt1t_tp8": Workload(
        "gpt1t_tp8",
        LayerShape(h=25600, heads=160, seq=2048, micro_batch=1, tp=8),
        description="1T-parameter GPT layer shape, shard 0 of tp=8: 20 heads of 160",
    ),
}
for _mb in (1, 2, 4, 8):
    WORKLOADS[f"gpt_h8192_stage_mb{_mb}"] = Workload(
        f"gpt_h8192_stage_mb{_mb}",
        LayerShape(h=8192, heads=64, seq=2048, micro_batch=_mb, tp=8),
        layers=4,
        description=f"h=8192 shard of tp=8, 4-layer stage, micro-batch {_mb}",
    )


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32.

    Uses the integer trick on the IEEE bit pattern: add 0x7FFF plus the lowest kept
    bit, then clear the 16 discarded bits. Inputs here are finite Gaussians.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _normal(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    out = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def _affine(shape: LayerShape, rng: Optional[np.random.Generator], n_out_qkv, n_ffn):
    """Biases and LayerNorm affine parameters.

    rng is None: biases 0, gamma 1, beta 0 (the baseline workloads).
    Otherwise: biases ~N(0, 0.02), gamma ~ 1 + N(0, 0.1), beta ~ N(0, 0.02), to
    exercise the bias and affine paths.
    """
    h = shape.h
    if rng is None:
        z = lambda n: np.zeros(n, np.float32)  # noqa: E731
        return dict(ln1_g=np.ones(h, np.float32), ln1_b=z(h), b_qkv=z(n_out_qkv), b_o=z(h),
                    ln2_g=np.ones(h, np.float32), ln2_b=z(h), b_fc1=z(n_ffn), b_fc2=z(h))
    return dict(
        ln1_g=1.0 + _normal(rng, h, 0.1), ln1_b=_normal(rng, h, 0.02),
        b_qkv=_normal(rng, n_out_qkv, 0.02), b_o=_normal(rng, h, 0.02),
        ln2_g=1.0 + _normal(rng, h, 0.1), ln2_b=_normal(rng, h, 0.02),
        b_fc1=_normal(rng, n_ffn, 0.02), b_fc2=_normal(rng, h, 0.02),
    )


def draw_global_layer(shape: LayerShape, rng: np.random.Generator,
                      affine_rng: Optional[np.random.Generator] = None) -> Dict[str, np.ndarray]:
    """Unsharded weights of one layer: W_qkv [3h, h], W_o [h, h], W1 [4h, h], W2 [h, 4h]."""
    h = shape.h
    p = dict(
        w_qkv=_normal(rng, (3 * h, h), WEIGHT_STD),
        w_o=_normal(rng, (h, h), WEIGHT_STD),
        w_fc1=_normal(rng, (4 * h, h), WEIGHT_STD),
        w_fc2=_normal(rng, (h, 4 * h), WEIGHT_STD),
    )
    p.update(_affine(shape, affine_rng, 3 * h, 4 * h))
    return p


def shard_slice(global_params: Dict[str, np.ndarray], shape: LayerShape, shard: int) -> Dict[str, np.ndarray]:
    """The weights tensor-parallel rank `shard` of `shape.tp` holds.

    Column split (output rows of W) for QKV and FC1, row split (input columns of W)
    for the out-projection and FC2; Q, K and V rows each keep the shard's heads.
    """
    h, t = shape.h, shape.tp
    hs = h // t            # a_t * d columns of Q (or K, or V) for this shard
    fs = shape.ffn // t
    q_rows = slice(shard * hs, (shard + 1) * hs)
    rows = np.r_[q_rows, h + shard * hs: h + (shard + 1) * hs, 2 * h + shard * hs: 2 * h + (shard + 1) * hs]
    g = global_params
    return dict(
        ln1_g=g["ln1_g"].copy(), ln1_b=g["ln1_b"].copy(),
        w_qkv=np.ascontiguousarray(g["w_qkv"][rows]), b_qkv=np.ascontiguousarray(g["b_qkv"][rows]),
        w_o=np.ascontiguousarray(g["w_o"][:, shard * hs:(shard + 1) * hs]), b_o=g["b_o"].copy(),
        ln2_g=g["ln2_g"].copy(), ln2_b=g["ln2_b"].copy(),
        w_fc1=np.ascontiguousarray(g["w_fc1"][shard * fs:(shard + 1) * fs]),
        b_fc1=np.ascontiguousarray(g["b_fc1"][shard * fs:(shard + 1) * fs]),
        w_fc2=np.ascontiguousarray(g["w_fc2"][:, shard * fs:(shard + 1) * fs]), b_fc2=g["b_fc2"].copy(),
    )


# NumPy's SeedSequence zero-pads its entropy words, so keys that differ only by trailing
# zeros (0 and [0, 0, 0, 0]) give the SAME stream. Every keyed stream therefore ends in
# this fixed nonzero word.
_KEY_TAIL = 0x6D74
PURPOSE_X, PURPOSE_DOUT, PURPOSE_WEIGHT = 1, 2, 3


def keyed_rng(seed: int, purpose: int, layer: int = 0, shard: int = 0, tensor: int = 0) -> np.random.Generator:
    """Independent stream per (seed, purpose, layer, shard, tensor)."""
    return np.random.default_rng([seed, purpose, layer, shard, tensor, _KEY_TAIL])


def draw_shard_layer(shape: LayerShape, seed: int, layer: int, shard: int,
                     random_affine: bool = False) -> Dict[str, np.ndarray]:
    """Shard-local weights drawn directly, one keyed stream per tensor."""
    h, t = shape.h, shape.tp
    key = lambda tid: keyed_rng(seed, PURPOSE_WEIGHT, layer, shard, tid)  # noqa: E731
    p = dict(
        w_qkv=_normal(key(0), (3 * h // t, h), WEIGHT_STD),
        w_o=_normal(key(1), (h, h // t), WEIGHT_STD),
        w_fc1=_normal(key(2), (4 * h // t, h), WEIGHT_STD),
        w_fc2=_normal(key(3), (h, 4 * h // t), WEIGHT_STD),
    )
    p.update(_affine(shape, key(4) if random_affine else None, 3 * h // t, 4 * h // t))
    return p


@dataclasses.dataclass
class Case:
    """One seeded input set: activations, upstream grad, per-layer shard weights."""

    shape: LayerShape
    x: np.ndarray
    dout: np.ndarray
    layers: List[Dict[str, np.ndarray]]
    # For global-weight workloads: the unsharded weights of each layer, so that
    # tests can run every shard and compare against the unsharded layer.
    global_layers: Optional[List[Dict[str, np.ndarray]]] = None


def make_case(shape: LayerShape, seed: int = 0, layers: int = 1, global_weights: bool = False,
              random_affine: bool = False) -> Case:
    """Draw X, the layer weights and dOut, in the workload's dtype.

    Order for global-weight workloads: default_rng(seed) draws X, then per layer
    W_qkv, W_o, W1, W2 (global), then dOut; biases/affine from default_rng([seed, 7])
    when random_affine. Shard-local workloads draw X, dOut and each weight tensor from
    its own keyed stream (keyed_rng).
    bf16 workloads round every tensor to bfloat16-representable float32 values, so the
    GPU (bf16) and the oracle (fp64) see the same numbers.
    """
    M, h = shape.tokens, shape.h
    rng = np.random.default_rng(seed)
    global_layers = None
    if global_weights:
        arng = np.random.default_rng([seed, 7]) if random_affine else None
        x = _normal(rng, (M, h))
        global_layers = [draw_global_layer(shape, rng, arng) for _ in range(layers)]
        dout = _normal(rng, (M, h))
        shard_layers = [shard_slice(g, shape, shape.shard) for g in global_layers]
    else:
        x = _normal(keyed_rng(seed, PURPOSE_X), (M, h))
        dout = _normal(keyed_rng(seed, PURPOSE_DOUT), (M, h))
        shard_layers = [draw_shard_layer(shape, seed, l, shape.shard, random_affine) for l in range(layers)]
    if shape.dtype == "bf16":
        x, dout = bf16_round(x), bf16_round(dout)
        shard_layers = [{k: bf16_round(v) for k, v in p.items()} for p in shard_layers]
        if global_layers is not None:
            global_layers = [{k: bf16_round(v) for k, v in p.items()} for p in global_layers]
    return Case(shape, x, dout, shard_layers, global_layers)


def workload_case(name: str, seed: int = 0, random_affine: bool = False, **shape_overrides) -> Case:
    w = WORKLOADS[name]
    shape = w.shape.replace(**shape_overrides) if shape_overrides else w.shape
    return make_case(shape, seed=seed, layers=w.layers, global_weights=w.global_weights,
                     random_affine=random_affine)


def mlp_case(shape: LayerShape, seed: int = 0, random_bias: bool = False) -> Case:
    """Inputs of the bare MLP block f(X W1^T + b1) W2^T (global weights drawn, shard sliced)."""
    return make_case(shape, seed=seed, layers=1, global_weights=True, random_affine=random_bias)


def model_flops(shape: LayerShape, causal: bool = True) -> float:
    """Model FLOPs of one shard's fwd+bwd: 3x the forward GEMM + attention FLOPs.

    Causal count: the score and context products cover s(s+1)/2 (query, key) pairs per
    head; the dense count covers s^2.
    """
    M, h, B, s = shape.tokens, shape.h, shape.micro_batch, shape.seq
    t = shape.tp
    gemm = 2 * M * (3 * h // t) * h + 2 * M * h * (h // t) + 2 * 2 * M * h * (4 * h // t)
    pairs = s * (s + 1) / 2 if causal else s * s
    attn = 2 * 2 * B * (h // t) * pairs
    return 3.0 * (gemm + attn)


# ------------------------------------------------------------------ optimizer step
PURPOSE_ADAM = 4

# Hyperparameters of the AdamW step workload. beta1, beta2 and the peak learning rate
# are the typical 175B settings listed on the oreateai.com Megatron-LM analysis
# ("In-Depth Analysis of Distributed Training Frameworks for Large Models ...
# Megatron-LM"), section 3.1; eps and the weight decay are not given there (1e-8 and
# 0.1 are the common GPT values); step 1000 is an arbitrary mid-training step.
ADAM_HPARAMS = dict(lr=6e-5, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=1000, grad_scale=1.0)


def shard_param_count(shape: LayerShape) -> int:
    """Parameters one tensor-parallel rank owns for one layer (every tensor of
    mt_layer_weights, the replicated LayerNorm and row-parallel biases included)."""
    h, t = shape.h, shape.tp
    ht, ft = h // t, 4 * h // t
    return (3 * ht * h + 3 * ht) + (h * ht + h) + (ft * h + ft) + (h * ft + h) + 4 * h


def adam_case(n: int, seed: int = 0):
    """fp32 master parameters, gradient and Adam moments for n parameters: p ~ N(0,
    0.02) like the weights, g ~ N(0, 1e-3), m ~ N(0, 3e-4) and v = (N(0, 1e-3))^2 +
    1e-10 (a second moment of gradients of that size). Each array from its own keyed
    stream."""
    key = lambda tid: keyed_rng(seed, PURPOSE_ADAM, 0, 0, tid)  # noqa: E731
    p = key(0).standard_normal(n, dtype=np.float32) * np.float32(WEIGHT_STD)
    g = key(1).standard_normal(n, dtype=np.float32) * np.float32(1e-3)
    m = key(2).standard_normal(n, dtype=np.float32) * np.float32(3e-4)
    v = np.square(key(3).standard_normal(n, dtype=np.float32) * np.float32(1e-3)) + np.float32(1e-10)
    return p, g, m, v
