"""Plain CPU float64 oracle for the FADE tiered KV-cache hot path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path (the libfade C-ABI
library and its Python binding) imports, links or calls this package. Only
`tests/`, `__graft_entry__.smoke()` and the `cpu_baseline` leg of `bench.py`
may use it. It shares no code, table or constant generator with the HIP
kernels.

Sources (cited by page title and section, never by line):
  * "FADE：面向LLM推理的注意力感知分层KV缓存压缩技术" (zingnex.cn forum
    thread), abbreviated "FADE post" below; its English summary page
    "FADE: Attention-Aware Hierarchical KV Cache Compression for LLM
    Inference" is "FADE summary".
  * "探秘Transformer系列之（25）--- KV Cache优化之处理长文本序列" (dg7.cn),
    abbreviated "Transformer series (25)"; sections 1.2.2 StreamingLLM and
    1.3.1 H2O.

Everything is float64 on the exact values of stored fp16/bf16 inputs, and a
value is rounded only where a step stores it. Where the pages are silent the
plainest reading is taken; each reading is named where it is used.

Modules:
  rope        rotary embedding (default, llama3, linear, ntk, yarn, dynamic,
              proportional, none; rotate-half or interleaved pairing)
  quant       symmetric INTb quantizer, bit-packing, dequantizer
  attention   joint-softmax decode attention over all tiers, side output
  h2o         H2O prefill column sums, cumulative / EMA score updates
  cache       the three-tier cache: tier layout, prefill build, append,
              demotion, eviction with un-RoPE / re-RoPE compaction; the
              optional INT2 overflow tier (int2_budget) and its two-level
              event (demote the INT4 overflow, drop the INT2 overflow)
  accounting  compressed-bytes closed form
  pq          product-quantization codebook: Lloyd training, encode, decode;
              cache.middle_pq stores the middle tier as PQ codes

Parity status: every function here is pinned by `tests/test_oracle_*.py`
against closed forms, library routines, invariants or brute force.
"""
