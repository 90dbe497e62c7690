"""CPU oracle for paged KV-cache attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product path (``paged_kv_cache_455_amd``) never imports it and has no CPU fallback.

It is a plain numpy float64 implementation written from the pages:

* uml.org.cn vLLM article, sections "PagedAttention", "Prefix Sharing",
  "Continuous Batching";
* "3、核心概念：LLM推理原理、KV Cache、PagedAttention、连续批处理" (5688vip.com
  course chapter 3), sections 3.1-3.3;
* "从KV Cache到vLLM：大模型推理提速与显存优化实战" (xxqk.cn), sections 1-3.

It shares no code, header, table or constant generator with the HIP library.
"""
from .paged_attention import (  # noqa: F401
    kv_cache_bytes,
    slot_for_position,
    gather_sequence,
    attention_rows,
    decode,
    prefill_chunk,
    cache_write,
    quantised_cache_write,
    block_copy,
    swap_blocks,
)
from .codec import (  # noqa: F401
    e4m3fn_decode,
    e4m3fn_encode,
    int8_decode,
    int8_encode,
)
