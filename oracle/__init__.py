"""fp64 CPU oracle for attention through a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only the test suite, the smoke check of
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it.  It
shares no code with the HIP library (no kernels, headers, helpers, constants
or pre-/post-processing); the only thing both sides consume is the seeded
input generator in ``workloads``, which holds none of the method's
arithmetic.

Two independent implementations:

* ``oracle.ref``   - vectorised NumPy, float64, the plain definitions written
  out (write, gather through the block table, scores, max-subtracted softmax,
  weighted sum of values; window and causal masks).
* ``oracle.brute`` - scalar pure Python (``math.exp``/``math.fsum``) for tiny
  inputs, used to cross-check ``oracle.ref``.
* ``oracle.quant`` - the 8-bit (INT8 / FP8 E4M3) row encoding of KV pages and
  decode over the decoded pools (float32 encoding steps, float64 attention).
* ``oracle.compressed`` - the compressed-slot tier: mean-pooled slots of
  evicted positions ("Build a Memory-Compressed Attention Engine with KV
  Caching from Scratch", Steps 2-4), the paged compression step, decode over
  slots plus the full tier, and the page's unpaged cache to compare against.

Sources (the pages these follow, by title and section):

* "Build a Paged KV Cache in Pure Python", Step 1 (block layout
  ``(block_size, num_heads, head_dim)``), Step 3 (``append``: block index =
  position // block_size, offset = position % block_size; ``retrieve``: blocks
  concatenated in table order, the last one cut to the tokens present) and
  Step 4 (``scaled_dot_product_attention``: per-head scores over the sequence
  axis, scaled, max-subtracted softmax, weighted sum of values; an empty
  context gives zeros).
* "Build a Minimal LLM Inference Engine with Paged Attention and Adaptive KV
  Cache", Step 1 and Step 4 (block table of page ids; gather then attend;
  empty -> zeros; refcount = number of sequences referencing a page).
* "Building a Streaming Sliding-Window Attention Engine in Pure Python",
  Step 2 (contiguous cache: the reference that paged results must equal),
  Step 3 (decode window = the last ``w`` positions; prefill mask
  ``0 <= i - j < w``) and Step 4 (K/V appended before attending).

Parity-unpinned: none of the oracle's functions.  Every function is pinned by
``tests/test_oracle.py`` against closed forms, invariants, a library routine
(``torch.nn.functional.scaled_dot_product_attention`` in float64) and the
scalar brute force; the 8-bit encoding by ``tests/test_oracle_quant.py``
(torch's float8_e4m3fn conversion, round-trip bounds, exact cases); the
compressed tier by ``tests/test_oracle_compressed.py`` (numpy's casts, a
hand-traced golden of the page's append procedure, closed forms, the plain
decode it reduces to, the scalar brute force).
"""
