"""CPU oracle for the paged-decode path -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct numpy code that states what the path computes.
Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
it; the product library never does, and this package imports nothing from the
product package (the seeded input generators in ``synth`` serve both).

Sources (three web pages; each function names the page and section it follows):

* mlxcel issue #235, "perf(core): chunked slab storage for the paged pool to
  eliminate growth reallocation entirely" -- the slab pool, the row mapping,
  growth by appending zeroed slabs, write_block, gather_visible.
* mlx-swift-lm PR #142, "Add packed paged KV formats with bounded workspace
  admission" -- K8/V8, K8/V4, K4/V4 token-local affine groups with FP32
  scale/offset and a fixed signed Hadamard basis on Q/K.
* mlxcel issue #2171, "refactor: one KV storage abstraction with dense and
  paged backends" -- attend(q, k, v, scale, mask): the single-token, unmasked
  decode attention over a pooled sequence.

Modules:
  slab_pool  -- byte-level model of the chunked-slab pool
  attention  -- fp64 softmax attention of one query token per sequence
  packed     -- signed Hadamard rotation, affine group quantiser, packed records
"""
