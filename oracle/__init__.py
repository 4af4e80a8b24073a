"""CPU oracle for quantized-KV decode/verify attention — TEST INFRASTRUCTURE.

A plain, slow, obviously correct numpy implementation of what the GPU path
computes, used only to check it.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it; the product path
(``quantized_kv_attention_quant_amd``) never does, and this package imports
nothing from the product path.  The two share no code: the oracle reads the
layout and arithmetic definitions from the C header's documentation and from
the pages, and implements them on its own.

Modules
  quant      KIVI-style asymmetric group quantizer (float32-exact emulation)
  layout     device byte layouts: pack logical codes into the buffers the
             library defines, and unpack them again
  cache      append / flush / rollback replay of the hierarchical cache
  attention  float64 softmax attention over the dequantized cache
  topk       canonical float32 speculative-token keys and exact top-k
  gather     on-demand reconstruction of a token subset (binary32-exact)

Sources (cited by page title and section):
  "QuantSpec: Self-Speculative Decoding with Hierarchical Quantized KV Cache"
      Approach (upper 4 bits = INT4 draft, upper+lower = INT8 target, double
      fp16 buffer of size 2G, no requantization on rollback); Measured-effects
      table (INT4 kernel reading the upper 4-bit cache); Experimental setup
      ("Builds on: FlashDecoding, KIVI").
  "SpeCache: Speculative Key-Value Caching for Efficient Generation of LLMs"
      Approach (1/2-bit KIVI copy on the GPU; speculative token's scores
      choose the top-k KV pairs).
  "MSpecKV" Abstract (KV traffic dominates; offloaded KV stored quantized,
      only the needed subsets reconstructed on demand).

Parity status (which function is pinned by what) is listed in each module's
docstring.  Every function is pinned against values the pages or the
mathematics fix; the two binary32 definitions that decide integers (the
quantizer's correctly rounded quotient and the top-k key's sequential,
unfused channel sum) are pinned by hand-derived goldens that a plausible
alternative (reciprocal-multiply, pairwise or fused sum) fails.
"""
