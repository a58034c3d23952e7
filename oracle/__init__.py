"""Plain, slow CPU oracle of the routed-expert MoE step.

TEST INFRASTRUCTURE ONLY.  Only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of bench.py may import this package.  It shares no code
with the HIP library or its Python binding, and neither imports the other;
its only shared input is the seeded generator package ``workload``.

Integers are Python ints; floating point is fp64.  Every function cites the
passage it follows, by page and section:

  signalovernoise  https://signalovernoise.tech/p/freetoken-treat-the-whole-pc-as-one
                   (an essay with no section headings)
  snackonai        https://www.snackonai.com/p/freetoken-or-why-your-laptop-was-never-the-bottleneck
                   sections "What It Actually Does", "The Architecture, Unpacked",
                   "The Locality Result Nobody Is Quoting", "The Code, Annotated"
                   ("The split policy itself", "Resizing the cache without a
                   restart"), "It In Action", "Insights"
  satyajit         https://ai.thesatyajit.com/articles/freetoken
                   sections "Prefill: hide the pool behind the wire",
                   "Decode: the one equation", "Residency that follows the router",
                   "Elastic memory, because the machine is not yours",
                   "Four backends, and the one that has to be measured"
  devto            https://dev.to/khasky/freetoken-runs-frontier-scale-moe-models-by-treating-the-whole-pc-as-the-inference-platform-54pf

Modules:
  route      softmax router top-k
  plan       residency state, q split, K-victim LRU, slot rewrite, resize,
             prefill admission (all integer)
  expert     bank decoding (f32 / bf16 / MXFP4) and the SwiGLU expert in fp64
  layer      MoE-layer output (sparse sum), its dense equivalent, merge, the
             grouped prefill evaluation
  placement  routing-blind static placements and miss counting
  costmodel  the two-branch time model behind the q split

Parity unpinned: nothing here reproduces the pages' measured miss rates
(16% / 39%), decode tok/s or prefill seconds; they need routing traces,
models and hardware that are not available.
"""
