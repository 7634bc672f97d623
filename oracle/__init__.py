"""CPU oracle for the DSA lightning-indexer hot path.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously-correct
numpy implementation of what the hot path computes.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The product path (the HIP library and its Python binding) never
imports, links or calls anything here, and this package never imports the
product path: the two share no code.  Floating point is carried in fp64 except
where the method itself fixes a precision (the FP8 codes and the fp32 scales).

Modules
-------
fp8          OCP FP8 e4m3fn codec written from the bit definition.
indexer      q quantisation, paged K dequantisation, logits, causal mask,
             exact sort-based top-k, shared-buffer write.
index_cache  IndexCache F/S layer rule and the layer loop.
k_write      indexer-K write path: slot mapping, per-token FP8 quantisation
             of new keys, scatter into 8448-byte pages.
handoff      sparse-attention hand-off: top-k rows as physical slots and as
             the additive 0 / -inf score mask.
chunking     logits budget and the forward pass over row chunks.

Pins (what each function is checked against, other than itself) are listed in
each module's docstring.  Functions with no external pin say
"parity unpinned" there.
"""

from . import fp8, indexer, index_cache, k_write, handoff, chunking  # noqa: F401
