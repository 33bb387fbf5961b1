"""Float64 CPU oracle for one decode step of attention over a latent KV cache.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The library in
``branch_rank_amd/`` never imports it, and it imports nothing from there: the
two share no kernels, helpers, tables or pre/post-processing.

Pages cited (by title and section):

* "Multi-Head Low-Rank Attention" (summary of arXiv 2603.02188), sections
  前置知识 (RoPE), 研究动机 (motivation), 核心方法 (core method),
  方法步骤详情 (method steps), 技术新颖性 (novelty) and its results table.
* "MLA多头潜在注意力机制", section 3 (3.1 latent compression, 3.2 attention).
* "ML Revisit: Attention", section "Multi-Head Latent Attention".
* "vllbc02MLA", sections 核心思想, 苏神思路, 猛猿大佬思路.

Every function is pinned by a CPU test in ``tests/test_oracle_pins.py``
against something other than itself (closed forms, the absorption identity,
brute force, a library attention routine, the pages' byte counts, the
variance statements). See the docstring of each function for its pin.
"""

from .mlra_ref import (  # noqa: F401
    rope,
    branch_slices,
    mlra_decode_ref,
    mla_decode_ref,
    mlra_prefill_ref,
    absorb_q_ref,
    latent_attn_ref,
    out_proj_ref,
    partial_state,
    merge_partials,
    kv_elems_per_token_per_device,
    variance_scales,
    rms_norm,
    cache_append_ref,
    e4m3_decode,
    e4m3_encode,
    fp8_dequantize,
    fp8_quantize,
)
