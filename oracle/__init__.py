"""fp64 CPU oracle of one tensor-parallel GPT layer shard (forward and backward).

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import or run anything in this package. The HIP product path
(tensor_layer_gemms_amd) never imports it and shares no code with it.

Everything is plain NumPy in float64: matrix products use ``@`` (a library matmul);
LayerNorm, softmax, GeLU and every gradient are the textbook formulas written out.
Where the pages leave a step open the reading taken is stated at the function.

Pins (tests/test_oracle.py): central finite differences of <Out, dOut> for every
gradient; the pages' tensor-parallel invariant (sum over shards of
f(X A_i) B_i equals f(X A) B) forward and backward; brute-force per-element
attention loops; closed forms of LayerNorm, GeLU, the causal first query, a zero
query projection and a zeroed residual branch; and torch's fp64 CPU functional ops
with autograd as an independent library cross-check. adamw_step (oracle/adamw.py) is
pinned in tests/test_oracle_adamw.py. The sequence-parallel share
(oracle/sequence_parallel.py) is pinned in tests/test_oracle_sp.py against the
tensor-parallel layer, whose function it must reproduce exactly. No function is parity
unpinned.
"""
from .adamw import adamw_step  # noqa: F401
from .layer import (  # noqa: F401
    EPS,
    attention_bwd,
    attention_fwd,
    gelu,
    gelu_grad,
    layer_bwd,
    layer_fwd,
    layernorm_bwd,
    layernorm_fwd,
    mlp_bwd,
    mlp_fwd,
    stage_bwd,
    stage_fwd,
)
from .sequence_parallel import (  # noqa: F401
    all_gather_seq,
    attn_block_bwd,
    attn_block_fwd,
    reduce_scatter_seq,
    seq_rows,
    sp_layer_bwd,
    sp_layer_fwd,
)
