"""Plain, slow fp64 CPU oracle for the int4 routed-expert MoE block.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
CPU-baseline leg of the benchmark may import anything from this package.
The product path (the HIP library and its Python binding) never imports,
calls or links it, and this package imports nothing from the product path:
the two share no code.  Inputs come from the seeded generators in ``synth``
(which hold none of the method's arithmetic) or from hand-written fixtures.

What is modelled (pages: "Show HN: Run an 80B Qwen in 4.3 GB of RAM on a Mac
and a 35B on an iPhone", the how-it-works list and the what-was-built list;
"Swiftlet" news rewrite, working-principle paragraph; creativeainews
explainer, "How Expert Streaming Works"):

* ``moe_oracle``  - router logits, top-k with lower-index tie-break,
  renormalised softmax weights, sigmoid shared gate, affine int4 dequant,
  SwiGLU expert FFN, weighted combine, residual/RMS stack epilogue.
* ``blob_ref``    - an independent reader (and writer) of the fixed-stride
  expert blob byte layout.
* ``pool_sim``    - the bounded slot pool with LFU-plus-recency eviction.

Every function works in float64 unless it models a rounding step the method
itself defines (bf16 round-to-nearest-even of the next layer's input).

Parity status per function (pins live in ``tests/test_oracle_*.py``):
all functions are pinned except the absolute output values of the full-size
80B/35B-shaped layers, for which the pages print no tensors: there the
oracle is checked only through the invariants and closed forms that hold at
any size ("parity unpinned" beyond those invariants).
"""
