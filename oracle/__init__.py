"""fp64 CPU oracle for the Nystrom self-attention forward (test infrastructure only).

Only tests/, the package smoke check and the benchmark's CPU-baseline leg import this
package. It shares no code with the HIP library.
"""
from .nystrom import (  # noqa: F401
    depthwise_conv_seq,
    exact_attention_head,
    iterative_pinv,
    nystrom_forward,
    nystrom_head,
    pinv_scaling,
    segment_boundaries,
    segment_means,
    softmax_rows,
)
from .projections import nystrom_layer, out_project, qkv_project  # noqa: F401
from .backward import nystrom_backward  # noqa: F401
from .flash import mixed_chunk_attention  # noqa: F401
