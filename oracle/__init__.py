"""CPU oracle for the routed-expert MoE step — TEST INFRASTRUCTURE ONLY.

A plain, slow, single-threaded numpy implementation, in float64 wherever the
arithmetic is floating point, of what the HIP path computes:

* ``oracle.quant`` — the affine int4/int8 group quantiser, the packed expert
  record and the fixed-stride blob addressing;
* ``oracle.moe``   — router logits, softmax + top-k with renormalisation, the
  SwiGLU expert FFN on dequantised weights, the sigmoid-gated shared expert,
  the weighted combine, prefill bucketing and the residual stack;
* ``oracle.pool``  — the LFU + recency expert-pool policy (and a brute-force
  twin used only to pin it).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product path never does, and this
package never imports the product package: the two share no code. The only
shared module is ``synth`` (seeded random inputs, no method arithmetic).

Sources. The method is described by five web pages about the Swiftlet runtime:
a paotong.dev commentary, a vance.xin blog post, a cheshm.ai news article, a
field-test write-up on alphalab.site and a we.inc marketing post (the last
contradicts the others and is not used). Each function cites the page and the
passage it follows.

Parity unpinned (no page fixes these, so only internal invariants and the
agreement of two independent implementations pin them): the exact rounding
rules of the "MLX-style" quantisation grid, the distribution of the shared
gate vector, and the Zipf strength lambda of the pooled workload.
"""
