"""Seeded synthetic decode batches for paged attention.

This module only draws inputs: sequence lengths, a block pool allocation
with block tables, query vectors and per-token K/V values.  It holds none
of the attention arithmetic and no knowledge of how a cache block is laid
out in memory; both the GPU library's tests/bench and the CPU oracle take
their inputs from here.

The five workloads follow the decode batches described for the method:
a tiny MHA case, a LLaMA-13B-shaped MHA layer, a 70B-shaped GQA layer with
chat-like length spread and beam pairs that share prefix blocks
(copy-on-write), a long-context GQA case for the KV-split path and an int8
KV-cache GQA case with cache append; ``workloads.mla`` draws decode batches
over an MLA latent cache.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    WorkloadSpec,
    Workload,
    make_workload,
    make_custom,
    bf16_round,
    bf16_bits,
    bf16_from_bits,
    blocks_needed,
)
from .mla import MLA_CONFIG, MlaSpec, MlaWorkload, make_mla, make_mla_custom  # noqa: F401,E402
