"""fp64 CPU oracle for exact attention — test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg import this
package; the HIP library and its binding never do. See ``oracle.attention``.
"""
from .attention import (  # noqa: F401
    attention_backward,
    attention_backward_sampled,
    attention_forward,
    attention_forward_rows,
    logits,
    online_softmax_attention,
    softmax_rows,
    to_f64,
    visible,
)
from .varlen import (  # noqa: F401
    sequence_bounds,
    varlen_backward,
    varlen_backward_sampled,
    varlen_forward,
    varlen_forward_rows,
)
from .blocksparse import (  # noqa: F401
    blocksparse_backward,
    blocksparse_backward_sampled,
    blocksparse_forward,
    blocksparse_forward_rows,
)
from .dropout import (  # noqa: F401
    dropout_backward,
    dropout_backward_sampled,
    dropout_forward,
    dropout_forward_rows,
    keep_rows,
    keep_threshold,
    philox4x32,
)
