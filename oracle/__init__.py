"""CPU oracle for paged-attention decode.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import anything from this package.  The GPU library
(``paged_kv_cache_443_amd``) never imports it, and it imports nothing from
the GPU library: the two share no code.  Inputs come from ``workloads``.

What the oracle computes (plain definitions, float64 unless a step fixes
another precision):

* ``decode``: for each sequence and query head, softmax(scale * q . k_t) over
  every cached token t of the sequence, applied to the v_t; the cached
  tokens are found by walking the sequence's block table.  Source: page
  "字节跳动 AI Infra (2)", question on KV cache principles (KV Cache原理与优化),
  the step-t equations (cache = old cache with the new K/V row appended;
  attention = softmax of the query against all cached keys, scaled by
  1/sqrt(d), times the cached values); the block-table lookup follows the
  kernel sketch in the same page's PagedAttention question; the GQA head
  map follows page "LLM推理优化", section 1.3.
* ``decode_multi``: several new query tokens per sequence, each attending
  causally to the cached tokens up to its own position (the step-t
  attention applied token by token; chunked prefill, page "vLLM框架是怎么做
  推理加速的", section 3).
* ``decode_partials`` / ``merge_partials``: the KV-split form (FlashDecoding,
  page "字节跳动 AI Infra (2)", third question, layer-2 table) -- one
  normalised partial output and log-sum-exp per token range, merged by
  weighting each range with exp(lse - max lse).
* ``quantize_int8`` / ``quantize_int4`` / ``append``: writing a new token's
  K/V into its slot, as a plain copy or as symmetric int8 (int4) with one
  fp16 scale per (token, kv head) (INT8 KV cache: page "字节跳动 AI Infra
  (2)", optimisation table; INT8/INT4: page "LLM推理优化", section 1.3).

* ``copy_blocks`` / ``BlockManager``: copying physical blocks, and the
  reference counts, on-demand allocation, fork and copy-on-write of a block
  pool (page "字节跳动 AI Infra (2)", PagedAttention question, block-pool
  figure; page "LLM推理优化", section 3.2).

* ``swap_blocks``: whole blocks moved between a GPU pool and a host pool of
  the same layout, for preemption (page "字节跳动 AI Infra (2)",
  PagedAttention question, scheduling list; page "vLLM框架是怎么做推理加速的",
  section 2 and its second follow-up).

* ``mla_decode`` / ``mla_append``: decode over an MLA latent cache -- one
  compressed vector per token, each head's K and V recovered by the
  up-projections K = c W_up_K, V = c W_up_V, then attended as in
  ``decode`` (page "字节跳动 AI Infra (2)", question on KV-cache principles,
  MLA paragraph).  Pinned by ``tests/test_oracle_mla.py``.

Parity status: every function here is pinned by tests that do not re-use
its own code path (closed forms, invariants, pure-Python brute force, the
pages' worked block counts); see ``tests/test_oracle_pins.py``.
"""
from .layout import PagedCache  # noqa: F401
from .storage import k_slot, x_per_16b  # noqa: F401
from . import storage  # noqa: F401
from .quant import quantize_int4, quantize_int8, dequantize_int8  # noqa: F401
from .paged import (  # noqa: F401
    blocks_for,
    kv_head_for,
    gather_sequence,
    decode,
    decode_multi,
    decode_partials,
    merge_partials,
    append,
    build_cache,
)
from .brute import decode_bruteforce  # noqa: F401
from .blocks import BlockManager, OutOfBlocks, copy_blocks, swap_blocks  # noqa: F401
from .mla import LatentCache, mla_append, mla_build_cache, mla_decode, mla_expand, mla_gather  # noqa: F401,E402
