"""CPU oracle for the FlashAttention forward path -- TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously correct fp64 NumPy implementation of
what the GPU library computes.  It exists to check the GPU path.  Only the test
suite, the smoke check and the benchmark's CPU-baseline leg may import it; the
product library and its Python binding never do, and the oracle imports
nothing from them.

Definition followed (page "Intro to FlashAttention on Ascend CANN", sections
"where the traditional implementation is slow" and "the first pitfall"):
attention is softmax(Q K^T * scale) V computed with the full score matrix
materialised; the tiled method with an online softmax is stated there to reach
the same result as the standard softmax.  The causal mask (same page, the
paragraph on fusing the causal mask) lets each query see only keys at or before
its own position.

Attention over a paged KV cache (paged.py) reads each sequence's keys and
values through its page table (page "why FA is 2x on A100 but 1.5x on Ascend
910", section 5, PagedAttention) and then applies the same definition.

Attention on fp8 inputs (fp8.py) decodes OCP E4M3 bytes with per-tensor
factors and applies the same definition.

The gradients (backward.py) follow the page's statement that the backward pass
recomputes the forward (same page, the second pitfall) and are the exact
chain-rule derivative of the definition above.

Every function in this package is pinned by CPU tests against closed forms,
invariants, a brute-force per-query loop and, for the gradients, central finite
differences of the forward; none is "parity unpinned".
"""

from .attention import (  # noqa: F401
    bf16_bits_to_f64,
    visible_mask,
    softmax_probs,
    attention_one,
    attention_dense,
    attention_varlen,
    attention_query,
)
from .layout import unpad_gather, pad_scatter, mask_to_varlen  # noqa: F401
from .paged import gather_pages, attention_paged, attention_paged_fp8kv  # noqa: F401
from .fp8 import e4m3_to_f64, attention_fp8_varlen, attention_fp8_dense  # noqa: F401
from .backward import (  # noqa: F401
    attention_backward_one,
    attention_backward_varlen,
    attention_backward_dense,
)
