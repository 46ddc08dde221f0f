"""fp64 CPU oracle for exact attention. TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the package entry's ``smoke()`` check and the benchmark's
CPU-baseline leg may import it. The HIP library never does.
"""
from .attention import (attention_bwd, attention_fwd, head_bwd, head_dq_rows, head_fwd,  # noqa: F401
                        head_probs, online_softmax_attention)
