"""Reference oracle for the refined low-bit decode step -- TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, fp64 numpy restatement of what the decode step
computes.  It exists to check the HIP library, and nothing in the product path may
import, call or execute it: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, tables or helpers
with ``bit_decode_selective_amd`` (the HIP path) and imports nothing from it; the two
meet only in the seeded input generators (``bit_decode_selective_amd.inputs``),
which hold none of the method's arithmetic.

Sources.  The method is described on the pages gathered about StrataFlux:

* "rag-lover.com" summary of StrataFlux (Japanese), its explainer dialogue (解説):
  low-bit weights and KV stay on the GPU; the extra precision fetched from host
  memory consists of additional bits that subdivide the interval between resident
  low-bit levels ("nested refinement"), not a full FP16 replacement; weight
  refinements are chosen by input-activation magnitude and KV refinements by the
  attention weight seen through the low-bit keys; fetched precision is cached and
  reused across decode steps.
* the same page, limitations section (限界と未検証の範囲): a cache miss leaves the
  value at its resident low-bit precision.
* "StrataFlux: Memory-Hierarchy-Native Low-Bit LLM Inference" (arXiv 2611.08363,
  paperdot listing), abstract: refinement representation, selection and delivery
  are co-designed; only selected precision is streamed, delivery overlaps
  computation, and fetched precision is reused across decoding steps.

The pages fix no number format, group size, tie rule or cache policy.  The readings
this oracle takes are (each function repeats the one it relies on):

* per group of ``group`` (128) consecutive values: asymmetric uniform quantisation
  to B = b + r bits with an fp16 offset ``z = fp16(min)`` and an fp16 step
  ``s = fp16((max - min) / (2^B - 1))``, each a single round-to-nearest-even of the
  exact value; codes ``c = clip(rint((x - z) / s), 0, 2^B - 1)`` in fp64;
* resident code = top b bits ``c >> r``, dequantised as ``z + (s * 2^r) * (c >> r)``
  (the lower edge of its cell); refinement = low r bits, full value ``z + s * c``;
* packing: little-endian, LSB-first bit streams;
* selection ties go to the lower index; ``k_sel = ceil(p * n / 100)``.

Modules:

* ``nested``     -- quantisation, packing, dequantisation
* ``selection``  -- channel and token top-k
* ``gemv``       -- refined GEMV
* ``attention``  -- refined GQA decode attention
* ``cache``      -- refinement slot cache (LRU), deterministic mode
* ``decode``     -- one full decoder step around the refined ops
"""
