"""Float64 CPU oracle for paged KV-cache attention.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import anything from this package.  It shares
no code, constants or helpers with the HIP library or its Python binding, and it
imports neither.  It is a plain, slow, obviously correct restatement of what
the method computes, as described on the nano-vLLM pages:

  * "nano-vllm walkthrough" = the xingyun3d.csdn.net article on nano-vllm
    (untitled in its text), sections 五 (KV Block 管理), 七 (后端执行) and
    八 (序列与上下文);
  * "paging article" = the gsyq.cn article whose first heading is
    "项目概述：为什么我们需要关注 LLM 推理引擎？", sections 4.1 and 5.3;
  * "deep dive" = "万字深度解析 Nano-vLLM" (chenxutan.com), sections 1.2 and 3.2.1;
  * "gitcode summary" = the gitcode.csdn.net nano-vLLM summary, section 三.4.

``oracle.block_manager`` restates the walkthrough's section 五 block manager (ref
counts, rolling-hash prefix reuse of full blocks, may_append, deallocate) in plain
Python; its hash step calls the xxhash library's XXH64.  It is pinned by hand-worked
traces, a published XXH64 digest and brute-force invariants over random traces
(tests/test_block_manager_oracle.py, with planted mistakes in
tests/test_block_manager_mutants.py).

``oracle.sampler`` restates the walkthrough's section 六 sampler (temperature scaling,
Gumbel noise added, argmax; temperature 0 is greedy).  It is pinned by the Gumbel-max
theorem (token frequencies over many noise draws against softmax(logits / T)), a
pure-Python brute force, the greedy limit, tie and shift rules
(tests/test_oracle_sampler.py, with planted mistakes in the same file).

Every attention function below is pinned by CPU tests against brute force, closed forms,
invariants and a library special case (torch's scaled_dot_product_attention in
float64); none is "parity unpinned".
"""
from .paged_oracle import (  # noqa: F401
    to_f64, slot_of, decode_slot_mapping, prefill_metadata, fill_slot_mapping,
    store_kvcache, gather, attend, paged_decode, paged_prefill, new_pool,
)
from .sampler import sample, first_argmax  # noqa: F401,E402
