"""CPU oracle for paged FP8-KV attention -- TEST INFRASTRUCTURE ONLY.

A plain, slow, fp64 statement of what the GPU path computes.  Only the tests,
the smoke check and the bench's CPU-baseline leg may import it; the library
(`paged_fp8_kv_attn_amd`) never does, and this package imports nothing from
the library.  The two share no code; only the seeded input generator
(`synth`) feeds both.

What it follows:
  * Atlas engine article (ainews.cool), "技术深度解析": the attention section
    (a FlashAttention-2 variant with native MQA/GQA kernels), the quantisation
    section (FP8 with per-group scale factors folded into the kernels) and the
    memory section (fixed-size preallocated KV blocks).
  * "Atlas Takes On vLLM ... on a Single GB10" (ainews.surl.tw): the paged
    FP8 KV cache and MTP with K=4 draft tokens (verification attention).
Two neighbouring steps of the same serving path have their own plain
statements: kv_append.py (new tokens' K/V quantised into the paged FP8
pool, the step before the attention) and mtp_accept.py (greedy acceptance
of the K = 4 drafts from the target's logits, the step after MTP
verification; GB10 article: MTP with K = 4 under deterministic decoding).
FlashAttention-2's tiled online softmax reaches, in exact arithmetic, plain
softmax attention over the dequantised keys and values; so the oracle is that
plain definition (see attention.py).  Every function is pinned by the
`-m "not gpu"` tests (OCP table values, library decode, brute force, a
library attention routine, closed forms and invariants); none is
"parity unpinned".
"""

from .e4m3 import decode, decode_table  # noqa: F401
from .attention import gather_sequence, paged_attention  # noqa: F401
from .kv_append import encode as encode_e4m3, kv_append as paged_kv_append  # noqa: F401
from .mtp_accept import accept as greedy_accept, greedy_tokens  # noqa: F401
