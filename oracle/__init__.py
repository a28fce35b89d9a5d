"""CPU oracle for the hybrid compressed attention forward pass (CSA / HCA).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or execute this package:
it is used by ``tests/``, by ``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of
``bench.py``.  It shares no code, table or constant generator with the HIP library.

Plain NumPy in float64.  Each function follows one step of the method as the source pages state
it, and cites the page and the section it follows:

* [EXPLAINER]  "DeepSeek-V4: Million-Token Context" (codexsims.com explainer): the CSA walk-through
  (compressor, lightning indexer, top-k selector, core attention plus sliding window) and the HCA
  walk-through (128-token non-overlapping windows, dense multi-query attention, sliding window).
* [DEVTO]      "How DeepSeek-V4 Achieves Million-Token Contexts Without Quadratic Attention
  Costs" (dev.to), section "Two Compression Strategies: CSA and HCA".
* [SUMMARY]    "DeepSeek-V4: Towards Highly Efficient Million-Token Context Intelligence"
  (paperlayer.ai summary of the technical report), section 2.3 "Hybrid Attention with CSA and HCA".
* [RABBIT]     "Follow the white rabbit: DeepSeek V4's architecture in 3D" (sambatista.com), the
  paragraphs on HCA, CSA, the sliding window and the lightning indexer.

Where the pages leave a step open, the reading taken is stated at the function.  Readings that no
page fixes and that no independent pin can fix are marked "parity unpinned" in the docstring:

* the RoPE frequency schedule (base 10000, interleaved pairs): pinned only against GPT-J's
  interleaved rotary implementation, i.e. a convention, not a statement of the pages;
* the indexer activation (ReLU) and head weighting: the pages describe the indexer only as a
  lightweight scoring head -- parity unpinned;
* the quantisation granularity of the indexer (per-row power-of-two fp8 scale; OCP MX blocks of
  32 for fp4) -- the pages name only low precision and FP4: parity unpinned for the
  granularity (the element encodings themselves are pinned against library casts).
"""
from . import compress, quant, indexer, attention, pipeline  # noqa: F401
