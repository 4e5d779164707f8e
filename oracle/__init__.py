"""CPU oracle for fine-grained tile-sparse attention (test infrastructure only).

This package is the plain, slow definition of what the GPU library computes,
written in numpy float64 from the FG-Attn abstract ("FG-Attn: Leveraging
Fine-Grained Sparse Attention in Video Diffusion Models", section Abstract):
attention whose score matrix is decided per M x N tile of query-key dot
products (M queries by N keys), skipped tiles excluded from the softmax.

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
import it.  It imports nothing from the GPU library, and the library never
routes through it.

Every function is pinned by tests/test_oracle.py (forward, compaction, mask diff,
predictor, FLOP count) and tests/test_oracle_bwd.py (backward) against brute
force or finite differences, closed
forms, a library routine for the dense special case, invariants and
hand-worked fixtures (tests/golden/).  No function here is "parity unpinned".
"""
from .sparse_attention import attention, attention_rows, unpack_mask, keep_matrix  # noqa: F401
from .compaction import compact  # noqa: F401
from .predictor import predict_mask, topk_count, pooled_scores  # noqa: F401
from .flops import kept_flops  # noqa: F401
from .backward import attention_bwd, attention_bwd_rows  # noqa: F401
from .mask_reuse import mask_diff  # noqa: F401
from . import fp8  # noqa: F401
