"""CPU oracle for the MiLo W3A16 + low-rank MoE expert GEMM.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import anything from this package; the GPU
library never calls it and shares no code with it.

Plain, slow, obviously correct NumPy in float64.  Sources (the pages):

* [talk] "MiLo: Efficient Quantized MoE Inference with Mixture of Low-Rank
  Compensators" (write-up of the MLSys 2025 talk), sections Background,
  Technical Deep Dive (MiLo Algorithm; MiLo Kernel), Experimental Setup &
  Results.
* [abs] the arXiv abstract of "MiLo: Efficient Quantized MoE Inference with
  Mixture of Low-Rank Compensators" (2504.02658).

Every function below is pinned by tests marked "not gpu" against facts other
than itself (hand-derived golden cases, closed forms, brute force, identities);
see tests/test_oracle_*.py.
"""
from .quant import (  # noqa: F401
    f16_rne,
    f16_bits,
    quantize_rtn_int3,
    dequant_int3,
)
from .layout import (  # noqa: F401
    LAYOUT_VERSION,
    packed_words,
    pack_v1,
    unpack_v1,
    pack_v1_scalar,
    unpack_v1_scalar,
    pack_sz_v1,
    unpack_sz_v1,
)
from .route import route_ref  # noqa: F401
from .compensator import (  # noqa: F401
    quantize_compensator,
    dequant_compensator,
    pack_lr_v,
    unpack_lr_v,
    pack_lr_u,
    unpack_lr_u,
    lr_v_words,
    lr_v_sz_words,
    lr_u_words,
    lr_u_sz_words,
)
from .builder import (  # noqa: F401
    residual_ref,
    exact_lowrank_ref,
    rsvd_ref,
    build_ref,
)
from .rank_policy import (  # noqa: F401
    kurtosis_ref,
    expert_frequency_ref,
    rank_scores_ref,
    apportion_ranks_ref,
    rank_policy_ref,
)
from .moe import (  # noqa: F401
    linear_ref,
    quantize_expert,
    silu,
    expert_ffn_ref,
    moe_layer_ref,
    combine_ref,
    rel_fro,
    max_abs,
)
