"""Plain float64 CPU oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) may import, call or link anything in this package; only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the GPU path: it receives numpy
arrays and returns numpy arrays.

Sources (web pages on FlashAttention, cited by title and section):

* "Paper Notes: FlashAttention" (bv003me.vercel.app/blog/flashattention),
  sections "What Are We Computing?", "Tiling: Block-by-Block Softmax",
  "Background", "Key Ideas", "Worked Example".
* "flash attention" (muhibwaqar.com/writing/flash-attention), section
  "build it from scratch" (the 1/sqrt(d) scale and the tiled loop).
* The aicassindra.com transformer-math page on FlashAttention, sections
  "Online softmax: the running-max, running-sum idea", "Rescale and
  accumulate", "The backward pass: recompute instead of store",
  "A tiny worked example", "Common pitfalls".

Modules:

* :mod:`oracle.attention` -- the definition (S, P, O, LSE) and its
  textbook chain-rule gradients, materialising S and P.
* :mod:`oracle.online` -- softmax attention from per-part states (m, l and
  the unnormalised output) and the two-block merge rule, kept only to pin the
  definition (block-wise == one-shot) and to replay the pages' worked
  examples step by step.
* :mod:`oracle.blocksparse` -- the same definition under a block mask (the
  block-sparse variant named in "Experiments & Results" on the Paper Notes
  page), with the conventions for rows that allow no key.
* :mod:`oracle.varlen` -- unequal query and key lengths (bottom-right causal
  alignment) and the split-K/V merge by the two-block rule of "Tiling:
  Block-by-Block Softmax".
* :mod:`oracle.dropout` -- dropout on the probabilities (an element-wise op
  that "Background" on the Paper Notes page lists among those kernel fusion
  folds in), with the mask from the Philox4x32-10 counter-based generator.
* :mod:`oracle.keypad` -- the key padding mask (the mask of that same list, as
  per-sequence key lengths), with the conventions for rows that see no key.
* :mod:`oracle.window` -- the causal sliding-window mask (each query sees its
  last ``window`` keys).

Every function here is pinned by ``tests/test_oracle*.py`` against page-printed
values, closed forms, invariants, finite differences and a library autograd.
``oracle.dropout.philox4x32_10`` is pinned to the generator's published
known-answer vectors (Salmon et al., SC 2011, as distributed with the
authors' Random123 library), besides the properties a counter-based generator
must have (bijection, uniform bits, avalanche, keep rates); GPU masks are
compared with the oracle's bit for bit.
"""

from . import attention, online  # noqa: F401
