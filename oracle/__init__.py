"""CPU oracle for IO-aware (FlashAttention-style) attention.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH.  Only the test suite, the entry point's smoke
check and the benchmark's CPU-baseline leg may import, call or execute anything in this package.
The GPU library never routes through it, and it shares no code with the GPU library.

Everything here is plain float64 numpy written from the definitions the pages give: attention
(materialise the score matrix, mask it, take the row softmax, multiply by V, report the natural
log-sum-exp) in ``attention_ref``; its gradients in ``attention_bwd_ref``; the row softmax and
its running (max, sum) recurrence in ``softmax_ref``; GELU, the bias-GELU-dropout chain and its
Philox4x32-10 dropout stream in ``elementwise_ref``.  Each module cites its passages.
"""
from .attention_ref import (  # noqa: F401
    causal_visible,
    combine_split_partials,
    naive_attention,
    naive_attention_head,
    online_softmax_row,
    scalar_attention_loops,
    scores,
    softmax_attend,
    split_kv_decode,
    split_kv_partials,
)
